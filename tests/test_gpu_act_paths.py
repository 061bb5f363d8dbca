"""GPU parity of every launch path of the activation side (rotate-quantize and calibration) against
the CPU oracle, through the C ABI.

The library picks a kernel by batch shape: a few-token kernel that gathers the zigzag order itself,
a coalesced permutation pass followed by the streaming (LDS-ring) kernel, the streaming kernel
directly when rows are already in zigzag order (identity permutation), and a register-staged
kernel that gathers per element (per-step batches of a few MB, or rows whose stride is not 16-byte
aligned). Each case below lands on one of them, with ragged tails, both block sizes, block counts
that do and do not divide into the 8 XCDs, and several row tiles per workgroup. Codes must equal
the oracle's except for certified near-tie flips (the device rotation is within the derived error
bound of the fp64 one and the oracle's value lies within that bound of a rounding boundary).
"""
import numpy as np
import pytest

import oracle
from w4a4_post_quantized_zigzag_amd import binding as bd

from parity_util import compare_codes, dev, host, rotation_error_bound

pytestmark = pytest.mark.gpu

# tag: (M, K, B, mode, permutation, path the shape selects)
PATHS = {
    "few_step_perm": (50, 1024, 128, "per_step", "zigzag", "few-token kernel"),
    "few_token_perm_b64": (33, 512, 64, "per_token", "zigzag", "few-token kernel"),
    "few_token_ident_nb3": (256, 384, 128, "per_token", "identity", "few-token kernel"),
    "ring_step_ident_multi": (600, 8192, 128, "per_step", "identity", "streaming, 2 tiles/workgroup"),
    "ring_step_permuted": (520, 8192, 128, "per_step", "zigzag", "permutation pass + streaming"),
    "ring_token_permuted_b64": (300, 2048, 64, "per_token", "zigzag", "permutation pass + streaming"),
    "ring_token_ident_nb3": (400, 384, 128, "per_token", "identity", "streaming, 3 blocks"),
    "gather_step": (300, 1024, 128, "per_step", "zigzag", "register-staged gather"),
    # K beyond the staged-row permutation pass (64 Ki halves): both per-token passes gather
    "long_k_token_gather": (260, 131072, 128, "per_token", "zigzag", "register-staged gather"),
}


def _inputs(M, K, B, perm_kind, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 15.0
    X = X.astype(np.float16)
    W = rng.normal(0.0, 0.02, (64, K))
    perm = (oracle.zigzag_perm(W, B) if perm_kind == "zigzag" else np.arange(K, dtype=np.int32))
    U = oracle.block_svd(W, perm, B)
    return X, perm, U


def _check(X, perm, U, B, mode, table=None, step=0, dev_perm=True, x_dev=None):
    torch = __import__("torch")
    K = X.shape[1]
    R = oracle.rotation(U, B)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B)
    xrot = torch.empty(X.shape, dtype=torch.float32, device="cuda")
    xd = dev(X) if x_dev is None else x_dev
    tab = dev(table) if table is not None else None
    xq, xs = bd.rotate_quant_act(xd, dev(perm) if dev_perm else None, rot, B, tab,
                                 0 if table is None else len(table), step, xrot_dbg=xrot)
    ref = oracle.rotate_quant_act(X, perm, U, B, mode, table, None, step, R=R)
    eps = rotation_error_bound(X, perm, R, B)
    xr = host(xrot).astype(np.float64)
    assert np.all(np.abs(xr - ref["x_rot"]) <= eps), np.max(np.abs(xr - ref["x_rot"]) / eps)
    s_dev = host(xs)
    if mode == "per_token":
        assert np.all(np.abs(s_dev - ref["scale"]) <= np.max(eps, axis=1) / 7 * 1.01
                      + 2 ** -23 * ref["scale"])
    else:
        assert s_dev[0] == table[step]
    q_dev = oracle.unpack_int4(host(xq), K)
    flips = compare_codes(q_dev, ref["codes"], ref["v"], ref["x_rot"], eps,
                          s_dev if mode == "per_token" else np.full(X.shape[0], s_dev[0]),
                          ref["scale"], mode == "per_token")
    assert flips <= max(3, q_dev.size * 1e-4), flips


@pytest.mark.parametrize("tag", list(PATHS))
def test_activation_path(tag):
    M, K, B, mode, perm_kind, _ = PATHS[tag]
    X, perm, U = _inputs(M, K, B, perm_kind, seed=len(tag))
    table = None
    if mode == "per_step":
        # one calibrated entry plus a coarse one that clips (codes at -8 and 7)
        t0 = oracle.calibrate_table([[X]], perm, U, B)[0]
        table = np.array([t0, t0 / 8], np.float32)
    for step in ([0, 1] if table is not None else [0]):
        _check(X, perm, U, B, mode, table, step, dev_perm=(perm_kind == "zigzag"))


@pytest.mark.parametrize("mode", ["per_step", "per_token"])
def test_activation_unaligned_row_stride(mode):
    # rows 4 halves longer than K: 16-byte tile loads do not apply, the element gather does
    torch = __import__("torch")
    M, K, B = 300, 512, 128
    X, perm, U = _inputs(M, K, B, "identity", seed=5)
    wide = np.zeros((M, K + 4), np.float16)
    wide[:, :K] = X
    xd = torch.from_numpy(wide).cuda()[:, :K]
    assert xd.stride(0) == K + 4
    table = np.array([oracle.calibrate_table([[X]], perm, U, B)[0]], np.float32)
    _check(X, perm, U, B, mode, table if mode == "per_step" else None, 0, dev_perm=False, x_dev=xd)


@pytest.mark.parametrize("M,K,B,perm_kind", [(50, 1024, 128, "zigzag"), (700, 2048, 128, "zigzag"),
                                             (600, 1024, 64, "identity")])
def test_calibration_paths(M, K, B, perm_kind):
    X, perm, U = _inputs(M, K, B, perm_kind, seed=M)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B)
    want = oracle.calibrate_table([[X]], perm, U, B)[0]
    got = host(bd.calibrate_act_scale(dev(X), dev(perm) if perm_kind == "zigzag" else None, rot,
                                      B))[0]
    eps = np.max(rotation_error_bound(X, perm, oracle.rotation(U, B), B))
    assert abs(got - want) <= eps / 7 * 1.01 + 2 ** -23 * want


def test_permute_pass_lds_grows():
    # the permutation pass stages a whole row in LDS: after a call with short rows, a call whose
    # rows take 80 KB must still launch (the kernel's LDS limit is raised when a launch needs more);
    # per-token quantization is row-local, so sampled rows are compared with the oracle
    from parity_util import compare_codes, rotation_error_bound
    B, M = 128, 260
    for K in (2048, 40960):
        X, perm, U = _inputs(M, K, B, "zigzag", seed=K)
        R = oracle.rotation(U, B)
        _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B)
        xq, xs = bd.rotate_quant_act(dev(X), dev(perm), rot, B)
        rows = np.array([0, 1, 2, 129, M - 1])
        ref = oracle.rotate_quant_act(X[rows], perm, U, B, "per_token", R=R)
        eps = rotation_error_bound(X[rows], perm, R, B)
        q_dev = oracle.unpack_int4(host(xq)[rows], K)
        s_dev = host(xs)[rows]
        assert np.all(np.abs(s_dev - ref["scale"]) <= np.max(eps, axis=1) / 7 * 1.01
                      + 2 ** -23 * ref["scale"])
        flips = compare_codes(q_dev, ref["codes"], ref["v"], ref["x_rot"], eps, s_dev,
                              ref["scale"], True)
        assert flips <= max(3, q_dev.size * 1e-4), flips
