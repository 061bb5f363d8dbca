"""GPU parity of the group-wise (per rotation block) per-step activation scales against the CPU
oracle, through the C ABI.

Activation codes must equal the oracle's except for certified near-tie flips (each position checked
with its own block's scale) and the scales written back must be the table row bit for bit. The
group-wise GEMM folds every block's exact partial into fp32 with one fused multiply-add per block
in block order on both sides, so its fp16 outputs must equal the oracle's bit for bit (GELU within
one fp16 ulp, as for the per-step GEMM). Shapes cover the few-token, register-gather, LDS-ring and
permute-pass rotate kernels, the small-M and pipelined GEMMs with ragged tails, and an end-to-end
linear against the tolerances.
"""
import numpy as np
import pytest

import oracle
from oracle.reference import EPI_GELU, EPI_NONE, EPI_RESIDUAL
from w4a4_post_quantized_zigzag_amd import binding as bd
from w4a4_post_quantized_zigzag_amd import inputs

from parity_util import check_y_tolerance, compare_codes, dev, host, rotation_error_bound

pytestmark = pytest.mark.gpu
B = 128


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _activations(M, K, seed):
    rng = _rng(seed)
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 15.0
    # blocks of different ranges, so the per-block scales differ
    X *= np.repeat(rng.uniform(0.3, 3.0, K // B), B)[None, :]
    return X.astype(np.float16)


@pytest.mark.parametrize("M,K,zz", [
    (50, 1024, True),      # few tokens (k_rq_small)
    (1, 256, True),
    (300, 1024, True),     # register-staged gather
    (600, 1024, False),    # rows already in zigzag order: LDS ring
    (520, 8192, True),     # permutation pass + ring
    (257, 2048, True),
])
def test_rotate_quant_grouped(M, K, zz):
    torch = __import__("torch")
    X = _activations(M, K, M + K)
    W = _rng(K).normal(0.0, 0.02, (64, K))
    perm = oracle.zigzag_perm(W, B) if zz else np.arange(K, dtype=np.int32)
    U = oracle.block_svd(W, perm, B)
    R = oracle.rotation(U, B)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B)
    T, step = 3, 1
    draws = [[_activations(64, K, 100 * t + M)] for t in range(T)]
    table = oracle.calibrate_table_grouped(draws, perm, U, B)
    xrot = torch.empty((M, K), dtype=torch.float32, device="cuda")
    xq, xs = bd.rotate_quant_act_grouped(dev(X), dev(perm) if zz else None, rot, B, dev(table), T,
                                         step, xrot_dbg=xrot)
    Xr = oracle.rotate_rows(X, perm, R, B)
    ref = oracle.quantize_act_grouped(Xr, B, table, T, step)
    eps = rotation_error_bound(X, perm, R, B)
    assert np.all(np.abs(host(xrot).astype(np.float64) - Xr) <= eps)
    assert np.array_equal(host(xs).view(np.uint32), table[step].view(np.uint32))
    q_dev = oracle.unpack_int4(host(xq), K)
    per_col = np.repeat(table[step], B)[None, :]
    flips = compare_codes(q_dev, ref["codes"], ref["v"], Xr, eps, per_col, per_col, False)
    assert flips <= max(3, q_dev.size * 1e-4)


def test_calibrate_grouped():
    M, K = 700, 2048
    X = _activations(M, K, 9)
    W = _rng(10).normal(0.0, 0.02, (64, K))
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B)
    want = oracle.calibrate_table_grouped([[X]], perm, U, B)[0]
    got = host(bd.calibrate_act_scale_grouped(dev(X), dev(perm), rot, B))
    eps = np.max(rotation_error_bound(X, perm, oracle.rotation(U, B), B))
    assert got.shape == want.shape
    assert np.all(np.abs(got - want) <= eps / 7 * 1.01 + 2 ** -23 * want)


def _operands(M, N, K, seed):
    rng = _rng(seed)
    xq = rng.integers(0, 256, (M, K // 2), dtype=np.int64).astype(np.uint8)
    wq = rng.integers(0, 256, (N, K // 2), dtype=np.int64).astype(np.uint8)
    sx = (rng.uniform(0.5, 2.0, K // B) * 2.0 ** rng.integers(-10, -4, K // B)).astype(np.float32)
    sw = rng.uniform(1e-3, 5e-2, N).astype(np.float32)
    res = (rng.standard_normal((M, N)) * 4).astype(np.float16)
    return xq, wq, sx, sw, res


@pytest.mark.parametrize("epi", [EPI_NONE, EPI_RESIDUAL, EPI_GELU])
@pytest.mark.parametrize("M,N,K", [(1, 64, 256), (50, 4096, 1024), (64, 100, 2048), (16, 520, 16384),
                                   (300, 1000, 2048), (257, 520, 128), (1600, 3072, 1024)])
def test_gemm_grouped(M, N, K, epi):
    xq, wq, sx, sw, res = _operands(M, N, K, M + N + K + epi)
    Y = host(bd.gemm_grouped(dev(xq), dev(sx), dev(wq), dev(sw), K, B, epilogue=epi,
                             residual=dev(res) if epi == EPI_RESIDUAL else None))
    rows = np.arange(M) if M * N * K <= 2 ** 30 else np.unique(np.r_[np.arange(0, M, 61), M - 1])
    q = oracle.unpack_int4(xq[rows], K)
    p = oracle.unpack_int4(wq, K)
    ref = oracle.gemm_grouped(q, sx, p, sw, B, epi, res[rows] if epi == EPI_RESIDUAL else None)["Y"]
    got = Y[rows].view(np.float16)
    if epi == EPI_GELU:
        d = np.abs(got.view(np.int16).astype(np.int32) - ref.view(np.int16).astype(np.int32))
        assert d.max() <= 1
    else:
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("M,K,N", [(50, 1024, 512), (300, 2048, 640)])
def test_grouped_linear_end_to_end(M, K, N):
    d = inputs.linear_inputs("dit_mlp_up", M=M, K=K, N=N, calib=2)
    W = d["W"]
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    T = 2
    table = oracle.calibrate_table_grouped([d["X_calib"][t] for t in range(T)], perm, U, B)
    X = d["X_steps"][1]
    wq, sw, rot = bd.pack_weights(dev(W), dev(perm), dev(U), B)
    xq, xs = bd.rotate_quant_act_grouped(dev(X), dev(perm), rot, B, dev(table), T, 1)
    Y = host(bd.gemm_grouped(xq, xs, wq, sw, K, B))
    ref = oracle.linear(X, W, B, "per_block", table, T, 1, perm=perm, U=U)
    check_y_tolerance(Y, ref["Y"])
