"""GPU parity of the Hadamard-only rotation mode (R_b = H_B, U_b = I) against the CPU oracle,
through the C ABI.

The device transform runs in fp64 butterflies and rounds each result to fp32 once, so its fp32 x'
equals the oracle's (fp64 dot products with the fp64 H entries, rounded to fp32) except where the
exact value lies within a few fp64 ulps of an fp32 rounding boundary, or where the block's signed
sum cancels to a value so small that the oracle's fp64 product roundings (about 2^-53 of the inputs)
are a visible part of it. The tests therefore ask for equality of x', the scales and the packed
codes, allowing a difference only at the rare positions where the two fp32 values differ, by one
fp32 ulp or by less than 2^-40 of the row's largest input. Cases cover both block sizes, fp16 and
fp32 inputs, the zigzag and the identity order, several rows per workgroup, rows long enough that
the per-token sweep recomputes blocks beyond the ones kept in registers, strided rows, and the
weight side packed with U == NULL.
"""
import numpy as np
import pytest

import oracle
from w4a4_post_quantized_zigzag_amd import binding as bd

from parity_util import dev, host

pytestmark = pytest.mark.gpu

CASES = {
    # tag: (M, K, B, x dtype, mode, zigzag order)
    "dit_step_b128": (50, 1024, 128, np.float16, "per_step", True),
    "prefill_token_b128": (300, 2048, 128, np.float16, "per_token", True),
    "rows_per_wg_b64": (1600, 1024, 64, np.float16, "per_token", False),
    "longk_token_kept": (97, 16384, 128, np.float16, "per_token", True),
    "longk_token_recomputed": (20, 32768, 128, np.float16, "per_token", True),
    "fp32_step_b64": (16, 256, 64, np.float32, "per_step", True),
    "fp32_token_b64": (33, 512, 64, np.float32, "per_token", False),
    "single_row": (1, 4096, 128, np.float16, "per_token", True),
}


def _inputs(M, K, B, xdt, zigzag, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20.0
    if M > 2:
        X[M // 2] = 0.0  # an all-zero row: scale 1.0, codes 0
    X = X.astype(xdt)
    W = rng.normal(0.0, 0.02, (64, K))
    perm = oracle.zigzag_perm(W, B) if zigzag else np.arange(K, dtype=np.int32)
    return X, W, perm


def _ulp_apart(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def _check(X, perm, B, mode, table=None, step=0, x_dev=None, dev_perm=True):
    torch = __import__("torch")
    M, K = X.shape
    U = np.broadcast_to(np.eye(B, dtype=np.float32), (K // B, B, B))
    ref = oracle.rotate_quant_act(X, perm, U, B, mode, table, None if table is None else len(table),
                                  step)
    xrot = torch.empty((M, K), dtype=torch.float32, device="cuda")
    xq, xs = bd.rotate_quant_act_hadamard(dev(X) if x_dev is None else x_dev,
                                          dev(perm) if dev_perm else None, B,
                                          dev(table) if table is not None else None,
                                          0 if table is None else len(table), step, xrot_dbg=xrot)
    x32 = host(xrot)
    ref32 = ref["x32"].astype(np.float32)
    # one fp32 ulp, or (where the block's +-sum cancels to a tiny x') the oracle's own fp64
    # rounding of its B products, below 2^-40 of the row's largest input
    d = _ulp_apart(x32, ref32)
    tiny = np.abs(x32.astype(np.float64) - ref32) <= 2.0 ** -40 * np.max(np.abs(
        X.astype(np.float64)), axis=1, keepdims=True)
    assert np.all((d <= 1) | tiny), d[~tiny].max()
    differ = d != 0
    assert differ.sum() <= max(2, X.size * 1e-5), differ.sum()
    s_dev = host(xs)
    if mode == "per_token":
        rows_differ = differ.any(axis=1)
        ok = s_dev == ref["scale"].astype(np.float32)
        assert np.all(ok | rows_differ)
    else:
        assert s_dev[0] == table[step]
    q_dev = oracle.unpack_int4(host(xq), K)
    code_diff = q_dev != ref["codes"]
    if mode == "per_token":
        code_diff &= ~np.repeat(rows_differ[:, None], K, axis=1)
    assert np.all(~code_diff | differ), np.argwhere(code_diff & ~differ)[:5]
    return differ.sum()


@pytest.mark.parametrize("tag", list(CASES))
def test_hadamard_rotate_quant(tag):
    M, K, B, xdt, mode, zz = CASES[tag]
    X, W, perm = _inputs(M, K, B, xdt, zz, seed=len(tag) + 100)
    if mode == "per_step":
        U = np.broadcast_to(np.eye(B, dtype=np.float32), (K // B, B, B))
        t0 = oracle.calibrate_table([[X]], perm, U, B)[0]
        table = np.array([t0, t0 / 8, 1e-3], np.float32)
        for step in range(3):
            _check(X, perm, B, mode, table, step, dev_perm=zz)
    else:
        _check(X, perm, B, mode, dev_perm=zz)


def test_hadamard_strided_rows():
    torch = __import__("torch")
    M, K, B = 70, 2048, 128
    X, W, perm = _inputs(M, K, B, np.float16, True, seed=9)
    wide = np.zeros((M, K + 4), np.float16)
    wide[:, :K] = X
    xd = torch.from_numpy(wide).cuda()[:, :K]
    _check(X, perm, B, "per_token", x_dev=xd)


def test_hadamard_linear_end_to_end():
    """Weights packed with U == NULL (R_b = H_B), activations through the Hadamard kernel, GEMM:
    packed weights bit-exact, fp16 outputs within the end-to-end tolerances."""
    from parity_util import check_y_tolerance
    M, K, N, B = 64, 2048, 512, 128
    X, W, perm = _inputs(M, K, B, np.float16, True, seed=21)
    W = W.astype(np.float32)
    W = np.concatenate([W] * (N // W.shape[0]), axis=0) * np.linspace(0.5, 2.0, N)[:, None]
    W = W.astype(np.float32)
    U = np.broadcast_to(np.eye(B, dtype=np.float32), (K // B, B, B)).copy()
    wq, sw, _ = bd.pack_weights(dev(W), dev(perm), None, B)
    ref_w = oracle.pack_weights(W, perm, U, B)
    assert np.array_equal(host(wq), ref_w["wq"])
    assert np.array_equal(host(sw), ref_w["w_scale"])
    xq, xs = bd.rotate_quant_act_hadamard(dev(X), dev(perm), B)
    Y = host(bd.gemm(xq, xs, True, wq, sw, K))
    ref = oracle.linear(X, W, B, "per_token", perm=perm, U=U)
    check_y_tolerance(Y, ref["Y"])
