"""GPU parity of the W4A4 GEMM (int8 MFMA) against the CPU oracle, through the C ABI.

Operands are seeded random packed bytes (every byte is a valid pair of int4 codes, so the whole
code range including -8 is exercised). Accumulators must match the oracle's int64 sums bit for bit,
and the fused dequantization must match the oracle's fp32 rounding sequence bit for bit (GELU
within one fp16 ulp, since the device and the oracle evaluate erf differently).
"""
import numpy as np
import pytest

import oracle
from oracle.reference import EPI_GELU, EPI_NONE, EPI_RESIDUAL
from w4a4_post_quantized_zigzag_amd import binding as bd
from w4a4_post_quantized_zigzag_amd import inputs

from parity_util import dev, host

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed=0):
    xq = inputs.random_packed(M, K, seed=1000 + seed + M)
    wq = inputs.random_packed(N, K, seed=2000 + seed + N)
    return xq, wq


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 2), (1, 64, 64), (16, 256, 256), (50, 4096, 1024), (64, 128, 128), (65, 72, 330),
    (130, 200, 320), (300, 1000, 2048), (257, 129, 4096), (1, 3, 8),
])
def test_gemm_i32_bit_exact(M, N, K):
    xq, wq = _operands(M, N, K)
    acc = host(bd.gemm_i32(dev(xq), dev(wq), K))
    ref = oracle.int_gemm(oracle.unpack_int4(xq, K), oracle.unpack_int4(wq, K))
    assert np.array_equal(acc.astype(np.int64), ref)


# (1590, 3072, 1024): the 80-row tile plan with a ragged last row band
@pytest.mark.parametrize("M,N,K", [(1024, 16384, 2048), (1024, 2048, 16384), (1600, 3072, 1024),
                                   (1600, 1024, 4096), (50, 4096, 1024), (1590, 3072, 1024)])
def test_gemm_i32_full_size_sampled(M, N, K):
    xq, wq = _operands(M, N, K, seed=7)
    acc = host(bd.gemm_i32(dev(xq), dev(wq), K)).astype(np.int64)
    rng = np.random.Generator(np.random.PCG64(M + N + K))
    mi = np.concatenate([rng.integers(0, M, 1500), [0, M - 1, M - 1, 0]])
    ni = np.concatenate([rng.integers(0, N, 1500), [0, N - 1, 0, N - 1]])
    rows = np.unique(mi)
    cols = np.unique(ni)
    q = oracle.unpack_int4(xq[rows], K)
    p = oracle.unpack_int4(wq[cols], K)
    ref = oracle.int_gemm_sampled(q, p, np.searchsorted(rows, mi), np.searchsorted(cols, ni))
    assert np.array_equal(acc[mi, ni], ref)


# M <= 64 shapes that reach each tile of the weight-streaming kernel (16, 32 or 64 output columns
# per workgroup, 8 or 4 waves splitting K), through its short-wave loop and its two-chunk prefetch
# loop, with ragged M, ragged N (a partial last tile) and uneven K ranges per wave; the largest are
# compared on sampled outputs.
@pytest.mark.parametrize("M,N,K", [
    (37, 4100, 2048),     # 16 columns, 8 waves, one chunk per wave
    (64, 8200, 1536),     # 32 columns, 8 waves, prefetch loop
    (20, 16400, 1024),    # 64 columns, 8 waves, one chunk per wave
    (3, 16448, 4096),     # 64 columns, 8 waves, prefetch loop
    (16, 4096, 16512),    # 16 columns, 4 waves, 129 windows (uneven split)
    (50, 8192, 12288),    # 32 columns, 4 waves
    (64, 16384, 9216),    # 64 columns, 4 waves
    (1, 4097, 8320),      # one row, partial last tile
])
def test_gemm_i32_small_m_tiles(M, N, K):
    xq, wq = _operands(M, N, K, seed=11)
    acc = host(bd.gemm_i32(dev(xq), dev(wq), K)).astype(np.int64)
    if M * N * K <= 2 ** 30:
        ref = oracle.int_gemm(oracle.unpack_int4(xq, K), oracle.unpack_int4(wq, K))
        assert np.array_equal(acc, ref)
        return
    rng = np.random.Generator(np.random.PCG64(M * N + K))
    mi = np.concatenate([rng.integers(0, M, 2000), [0, M - 1, M - 1, 0]])
    ni = np.concatenate([rng.integers(0, N, 2000), [0, N - 1, 0, N - 1]])
    rows, cols = np.unique(mi), np.unique(ni)
    q = oracle.unpack_int4(xq[rows], K)
    p = oracle.unpack_int4(wq[cols], K)
    ref = oracle.int_gemm_sampled(q, p, np.searchsorted(rows, mi), np.searchsorted(cols, ni))
    assert np.array_equal(acc[mi, ni], ref)


@pytest.mark.parametrize("M,N,K", [
    (3, 40, 1 << 20),      # small M, more than 2^16 k per wave: the folding small-M kernel
    (64, 96, 1 << 18),     # small M at the wide kernel's per-wave limit (4 waves x 2^16 k)
    (130, 64, 1 << 18),    # K split into 64 Ki pieces with an exact int32 reduction
])
def test_gemm_i32_long_k(M, N, K):
    xq, wq = _operands(M, N, K, seed=13)
    acc = host(bd.gemm_i32(dev(xq), dev(wq), K)).astype(np.int64)
    ref = oracle.int_gemm(oracle.unpack_int4(xq, K), oracle.unpack_int4(wq, K))
    assert np.array_equal(acc, ref)


@pytest.mark.parametrize("M,N,K", [(130, 40, (1 << 20) + 128), (70, 24, 1 << 21)])
def test_gemm_long_k_beyond_one_split(M, N, K):
    # more than 2^16 k per tile accumulator: K is cut into pieces with exact int32 partials; every
    # row is written (rows beyond 64 were once left unwritten) -- sampled outputs plus the dequant
    xq, wq = _operands(M, N, K, seed=17)
    acc = host(bd.gemm_i32(dev(xq), dev(wq), K)).astype(np.int64)
    rows = np.array([0, 63, 64, 65, M - 1])
    q = oracle.unpack_int4(xq[rows], K)
    p = oracle.unpack_int4(wq, K)
    ref = oracle.int_gemm(q, p)
    assert np.array_equal(acc[rows], ref)
    sx = inputs.random_scales(M, seed=1)
    sw = inputs.random_scales(N, seed=2, lo=1e-5, hi=1e-4)
    Y = host(bd.gemm(dev(xq), dev(sx), True, dev(wq), dev(sw), K))
    want, _ = oracle.dequant(ref, sx[rows], True, sw)
    assert np.array_equal(Y[rows].view(np.uint16), want.view(np.uint16))
    # the all -8 closed form on every row
    neg = inputs.constant_packed(M, K, 0x88)
    a = host(bd.gemm_i32(dev(neg), dev(neg[:N]), K))
    assert np.all(a == 64 * K)


@pytest.mark.parametrize("K", [64, 2048, 16384, 1 << 20])
def test_gemm_i32_extremes(K):
    neg = inputs.constant_packed(70, K, 0x88)   # all codes -8
    pos = inputs.constant_packed(130, K, 0x77)  # all codes +7
    a = host(bd.gemm_i32(dev(neg), dev(neg[:65]), K))
    assert np.all(a == 64 * K)
    b = host(bd.gemm_i32(dev(neg), dev(pos), K))
    assert np.all(b == -56 * K)


@pytest.mark.parametrize("per_token", [True, False])
@pytest.mark.parametrize("epi", [EPI_NONE, EPI_RESIDUAL, EPI_GELU])
@pytest.mark.parametrize("M,N,K", [(50, 4096, 1024), (40, 16400, 1024), (200, 300, 512),
                                   (1024, 2048, 16384), (1590, 3072, 1024)])
def test_gemm_dequant_epilogue(per_token, epi, M, N, K):
    xq, wq = _operands(M, N, K, seed=3)
    sx = inputs.random_scales(M if per_token else 1, seed=M, lo=1e-3, hi=5e-2)
    sw = inputs.random_scales(N, seed=N, lo=1e-3, hi=5e-2)
    res = (np.random.Generator(np.random.PCG64(5)).standard_normal((M, N)) * 4).astype(np.float16)
    Y = host(bd.gemm(dev(xq), dev(sx), per_token, dev(wq), dev(sw), K, epilogue=epi,
                     residual=dev(res) if epi == EPI_RESIDUAL else None))
    if M * N * K > 2 ** 32:
        rows = np.unique(np.r_[np.arange(0, M, 97), M - 1])
        q = oracle.unpack_int4(xq[rows], K)
        acc = oracle.int_gemm(q, oracle.unpack_int4(wq, K))
        ref, _ = oracle.dequant(acc, sx[rows] if per_token else sx, per_token, sw, epi,
                                res[rows] if epi == EPI_RESIDUAL else None)
        Yc = Y[rows]
    else:
        acc = oracle.int_gemm(oracle.unpack_int4(xq, K), oracle.unpack_int4(wq, K))
        ref, _ = oracle.dequant(acc, sx, per_token, sw, epi, res)
        Yc = Y
    got = Yc.view(np.float16)
    if epi == EPI_GELU:
        gi = got.view(np.int16).astype(np.int32)
        ri = ref.view(np.int16).astype(np.int32)
        # within one fp16 ulp (the two erf evaluations differ below fp16 resolution)
        assert np.max(np.abs(gi - ri)) <= 1
    else:
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def _near_boundary_scales(n, mode, seed):
    """fp32 scales with full random mantissas just below (tiny) or just above (edge) 2^-118, or
    alternating per row (mixed): around the smallest scale whose 2^-8 multiple is still a normal
    fp32 number, so that a dequantization that folded the accumulator's 2^8 factor into the scale
    instead of shifting the accumulator would round differently below it."""
    m = inputs.random_scales(n, seed=seed, lo=1.0, hi=2.0).astype(np.float64)
    lo, hi = np.ldexp(m, -120), np.ldexp(m, -117)
    out = {"tiny": lo, "edge": hi, "mixed": np.where(np.arange(n) % 2 == 0, lo, hi)}[mode]
    return out.astype(np.float32)


@pytest.mark.parametrize("mode,per_token", [("tiny", False), ("edge", False), ("tiny", True),
                                             ("edge", True), ("mixed", True)])
@pytest.mark.parametrize("epi", [EPI_NONE, EPI_RESIDUAL, EPI_GELU])
@pytest.mark.parametrize("M,N,K", [(1600, 4096, 1024), (1590, 3072, 1024), (1024, 2048, 2048)])
def test_gemm_dequant_scales_near_the_fp32_normal_limit(mode, per_token, epi, M, N, K):
    # the activation scales sit around 2^-118 and the weight scales near 2^108, so that the
    # outputs are ordinary fp16 values and every fp32 rounding of the dequantization shows in them
    xq, wq = _operands(M, N, K, seed=9)
    sx = _near_boundary_scales(M if per_token else 1, mode, seed=M + 1)
    sw = (inputs.random_scales(N, seed=N + 2, lo=0.5, hi=1.0).astype(np.float64) * 2.0 ** 108)
    sw = sw.astype(np.float32)
    res = (np.random.Generator(np.random.PCG64(6)).standard_normal((M, N)) * 4).astype(np.float16)
    Y = host(bd.gemm(dev(xq), dev(sx), per_token, dev(wq), dev(sw), K, epilogue=epi,
                     residual=dev(res) if epi == EPI_RESIDUAL else None))
    rows = np.unique(np.r_[np.arange(0, M, 61), np.arange(M - 4, M)])
    q = oracle.unpack_int4(xq[rows], K)
    acc = oracle.int_gemm(q, oracle.unpack_int4(wq, K))
    ref, _ = oracle.dequant(acc, sx[rows] if per_token else sx, per_token, sw, epi,
                            res[rows] if epi == EPI_RESIDUAL else None)
    got = Y[rows].view(np.float16)
    assert np.all(np.isfinite(ref.astype(np.float32)))
    if epi == EPI_GELU:
        d = np.abs(got.view(np.int16).astype(np.int32) - ref.view(np.int16).astype(np.int32))
        assert np.max(d) <= 1
    else:
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def test_gemm_row_stride_and_empty():
    M, N, K = 33, 96, 256
    xq, wq = _operands(M, N, K)
    sx = inputs.random_scales(M, 1)
    sw = inputs.random_scales(N, 2)
    torch = __import__("torch")
    big = torch.zeros((M, 200), dtype=torch.float16, device="cuda")
    Yv = big[:, 50:50 + N]
    bd.gemm(dev(xq), dev(sx), True, dev(wq), dev(sw), K, Y=Yv)
    acc = oracle.int_gemm(oracle.unpack_int4(xq, K), oracle.unpack_int4(wq, K))
    ref, _ = oracle.dequant(acc, sx, True, sw)
    full = host(big)
    assert np.array_equal(full[:, 50:50 + N].view(np.uint16), ref.view(np.uint16))
    assert not full[:, :50].any() and not full[:, 50 + N:].any()
    empty = bd.gemm(dev(xq[:0]), dev(sx[:0]), True, dev(wq), dev(sw), K)
    assert tuple(empty.shape) == (0, N)
