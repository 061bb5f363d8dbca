"""The allocation-free rotate-quantize entry point against the workspace entry point, through the
C ABI: identical codes and scales on two calls in a row (the second smaller, so it reuses the
library's scratch left dirty by the first), per-token and per-step, plus the size limit."""
import numpy as np
import pytest

import oracle
from w4a4_post_quantized_zigzag_amd import binding as bd

from parity_util import dev, host

pytestmark = pytest.mark.gpu


def _case(M, K, B, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 15.0
    W = rng.normal(0.0, 0.02, (64, K))
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B)
    return dev(X.astype(np.float16)), dev(perm), rot, U, perm


def _same(a, b):
    return np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8))


@pytest.mark.parametrize("mode", ["per_token", "per_step"])
def test_noalloc_matches_workspace_entry(mode):
    # first call: 600 tokens x 4096 channels (per token: row maxima and staged zigzag rows in the
    # scratch); second call: 100 tokens x 1024 channels (few-token kernel, maxima only)
    for (M, K, B, seed) in ((600, 4096, 128, 1), (100, 1024, 128, 2)):
        X, perm, rot, U, perm_h = _case(M, K, B, seed)
        table = None
        if mode == "per_step":
            t0 = oracle.calibrate_table([[host(X)]], perm_h, U, B)[0]
            table = dev(np.array([t0, t0 / 4], np.float32))
        T = 0 if table is None else 2
        for step in range(1 if table is None else 2):
            q_ref, s_ref = bd.rotate_quant_act(X, perm, rot, B, table, T, step)
            q_na, s_na = bd.rotate_quant_act_noalloc(X, perm, rot, B, table, T, step)
            assert _same(q_na, q_ref) and _same(s_na, s_ref), (M, K, mode, step)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lim = bd.lib().w4a4_noalloc_scratch_bytes()
    M, K = 4096, 4096   # per-token workspace: row maxima + 32 MB of staged rows
    assert bd.lib().w4a4_act_workspace_bytes(M, K, 128, 1) > lim
    torch = __import__("torch")
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    perm = dev(np.arange(K, dtype=np.int32))
    U = np.broadcast_to(np.eye(128, dtype=np.float32), (K // 128, 128, 128)).copy()
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), perm, dev(U), 128)
    with pytest.raises(bd.W4A4Error) as e:
        bd.rotate_quant_act_noalloc(X, perm, rot, 128)
    assert e.value.status == bd.W4A4_ERR_UNSUPPORTED
