"""CPU pins of the oracle's group-wise (per rotation block) per-step activation scales.

The pages' act_scale_table is per layer, per step and per channel; its integer-GEMM-compatible form
keeps one scale per rotation block (vnrobo.com "Y tuong paper"; gist.science "Calibracao por
Passo"). The oracle folds each block's exact int32 partial into an fp32 accumulator with one fused
multiply-add per block, in block order. These tests fix that arithmetic against things other than
the oracle itself: an exact rational evaluation with hand-written fp32 rounding, the reduction to
the per-step mode when every block has the same power-of-two scale, brute-force block sums, the
relation between the grouped and per-step calibration tables, and the error reduction the
per-block scales exist for.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.reference import EPI_GELU, EPI_NONE, EPI_RESIDUAL


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _round_f32(x: Fraction) -> float:
    """Correctly rounded (ties to even) fp32 value of an exact rational, normal or subnormal."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = max(e - 23, -149)
    scaled = a / Fraction(2) ** ulp
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * math.ldexp(n, ulp)


def _chain_exact(acc_col, scales, sw):
    y = 0.0
    for a, s in zip(acc_col, scales):
        y = _round_f32(Fraction(int(a)) * Fraction(float(s)) + Fraction(y))
    return _round_f32(Fraction(y) * Fraction(float(sw)))


def test_fma_chain_matches_exact_rational_rounding():
    rng = _rng(1)
    nb, M, N = 6, 40, 50
    acc = rng.integers(-8192, 8193, (nb, M, N)).astype(np.int64)
    sg = (rng.uniform(0.5, 2.0, nb) * 2.0 ** rng.integers(-12, 0, nb)).astype(np.float32)
    sw = (rng.uniform(0.5, 2.0, N) * 2.0 ** -8).astype(np.float32)
    _, y32 = oracle.dequant_grouped(acc, sg, sw)
    unfused = 0
    for m in range(M):
        for n in range(N):
            want = _chain_exact(acc[:, m, n], sg, sw[n])
            assert y32[m, n] == np.float32(want), (m, n)
            # the separate multiply-then-add chain differs somewhere: the pin can see the fusion
            t = np.float32(0.0)
            for g in range(nb):
                t = np.float32(t + np.float32(np.float32(acc[g, m, n]) * sg[g]))
            unfused += int(np.float32(t * sw[n]) != y32[m, n])
    assert unfused > 0


def test_equal_power_of_two_scales_reduce_to_per_step():
    rng = _rng(2)
    M, N, K, B = 24, 33, 512, 128
    q = rng.integers(-8, 8, (M, K)).astype(np.int8)
    p = rng.integers(-8, 8, (N, K)).astype(np.int8)
    s = np.float32(2.0 ** -6)
    sw = rng.uniform(1e-3, 5e-2, N).astype(np.float32)
    g = oracle.gemm_grouped(q, np.full(K // B, s, np.float32), p, sw, B)
    ref = oracle.gemm(q, np.array([s], np.float32), False, p, sw)
    assert np.array_equal(g["acc"], ref["acc"])
    assert np.array_equal(g["y32"].view(np.uint32), ref["y32"].view(np.uint32))
    assert np.array_equal(g["Y"].view(np.uint16), ref["Y"].view(np.uint16))


def test_block_sums_brute_force():
    rng = _rng(3)
    M, N, K, B = 9, 7, 256, 64
    q = rng.integers(-8, 8, (M, K)).astype(np.int8)
    p = rng.integers(-8, 8, (N, K)).astype(np.int8)
    acc = oracle.int_gemm_grouped(q, p, B)
    for g in range(K // B):
        blk = slice(g * B, (g + 1) * B)
        assert np.array_equal(acc[g], q[:, blk].astype(np.int64) @ p[:, blk].astype(np.int64).T)
    assert np.array_equal(acc.sum(axis=0), oracle.int_gemm(q, p))


def test_grouped_codes_equal_per_step_codes_for_a_constant_row():
    rng = _rng(4)
    Xr = rng.standard_normal((13, 256)) * 3
    s = np.float32(0.37)
    a = oracle.quantize_act_grouped(Xr, 64, np.full((2, 4), s, np.float32), 2, 1)
    b = oracle.quantize_act(Xr, "per_step", np.array([s, s], np.float32), 2, 1)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["v"].view(np.uint32), b["v"].view(np.uint32))
    assert np.array_equal(a["xq"], b["xq"])


def test_grouped_quantization_picks_each_blocks_scale():
    # a hand case: block 0 scale 1, block 1 scale 0.25; x = 1.4 -> 1 in block 0, 5.6 -> 6 in block 1
    Xr = np.array([[1.4, -2.6, 0.5, 9.0, 1.4, -0.6, 0.125, 9.0]])
    table = np.array([[1.0, 0.25]], np.float32)
    out = oracle.quantize_act_grouped(Xr, 4, table, 1, 0)
    assert out["codes"].tolist() == [[1, -3, 0, 7, 6, -2, 0, 7]]
    assert out["scale"].tolist() == [1.0, 0.25]


def test_step_and_table_shape_errors():
    Xr = np.zeros((2, 128))
    t = np.ones((3, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.quantize_act_grouped(Xr, 64, t, 3, 3)
    with pytest.raises(ValueError):
        oracle.quantize_act_grouped(Xr, 64, t, 4, 0)            # table shorter than num_steps
    with pytest.raises(ValueError):
        oracle.quantize_act_grouped(Xr, 64, np.ones((3, 3), np.float32), 3, 0)  # wrong width
    # a zero scale is no scale: codes 0 and a NaN scale for that block (not an exception)
    z = oracle.quantize_act_grouped(Xr + 1.0, 64, np.zeros((3, 2), np.float32), 3, 0)
    assert not z["codes"].any() and np.all(np.isnan(z["scale"]))


def test_grouped_table_relates_to_per_step_table():
    rng = _rng(5)
    K, B, T = 512, 128, 3
    W = rng.normal(0.0, 0.02, (96, K))
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    X = [[(rng.standard_normal((20, K)) * (1 + t)).astype(np.float16) for _ in range(2)]
         for t in range(T)]
    tg = oracle.calibrate_table_grouped(X, perm, U, B)
    ts = oracle.calibrate_table(X, perm, U, B)
    assert tg.shape == (T, K // B)
    assert np.array_equal(tg.max(axis=1), ts)        # the global max is some block's max
    R = oracle.rotation(U, B)
    for t in range(T):
        for Xs in X[t]:
            q = oracle.quantize_act_grouped(oracle.rotate_rows(Xs, perm, R, B), B, tg, T, t)["codes"]
            assert q.min() >= -7 and q.max() <= 7      # calibration data never clips


def test_per_block_scales_lower_the_error_on_uneven_blocks():
    # identity order and U = I (R = H): block 0 carries 20x larger activations than the others, so
    # one per-step scale leaves the other blocks with 20x coarser steps than they need
    rng = _rng(6)
    M, K, B = 32, 512, 128
    X = rng.standard_normal((M, K))
    X[:, :B] *= 20
    perm = np.arange(K, dtype=np.int32)
    U = np.stack([np.eye(B, dtype=np.float32)] * (K // B))
    Xr = oracle.rotate_rows(X, perm, oracle.rotation(U, B), B)
    tg = oracle.calibrate_table_grouped([[X]], perm, U, B)
    ts = oracle.calibrate_table([[X]], perm, U, B)
    qg = oracle.quantize_act_grouped(Xr, B, tg, 1, 0)
    qs = oracle.quantize_act(Xr, "per_step", ts, 1, 0)
    # on the blocks that do not hold the maximum the reconstruction error drops about tenfold;
    # block 0 is quantized identically in both modes
    rest = slice(B, K)
    eg = np.linalg.norm(Xr[:, rest] - qg["codes"][:, rest] * np.repeat(tg[0], B)[None, rest])
    es = np.linalg.norm(Xr[:, rest] - qs["codes"][:, rest] * ts[0])
    assert eg < 0.2 * es
    assert np.array_equal(qg["codes"][:, :B], qs["codes"][:, :B])
    # block 0 keeps the per-step scale (it holds the maximum), the others get finer ones
    assert tg[0, 0] == ts[0] and np.all(tg[0, 1:] < ts[0] / 10)
    # and the quantized linear follows: the output error of the small blocks' share drops
    W = rng.normal(0.0, 0.02, (48, K))
    Wr = oracle.rotate_rows(W, perm, oracle.rotation(U, B), B)
    s_w, p = oracle.weight_rtn(Wr)
    exact = Xr[:, rest] @ (p[:, rest] * s_w[:, None]).T
    yg = (qg["codes"][:, rest] * np.repeat(tg[0], B)[None, rest]) @ (p[:, rest] * s_w[:, None]).T
    ys = (qs["codes"][:, rest] * ts[0]) @ (p[:, rest] * s_w[:, None]).T
    assert np.linalg.norm(yg - exact) < 0.2 * np.linalg.norm(ys - exact)


@pytest.mark.parametrize("epi", [EPI_NONE, EPI_GELU, EPI_RESIDUAL])
def test_grouped_epilogues_follow_the_per_step_ones(epi):
    rng = _rng(7)
    M, N, nb = 5, 6, 3
    acc = rng.integers(-500, 500, (nb, M, N)).astype(np.int64)
    sg = np.full(nb, 2.0 ** -5, np.float32)
    sw = rng.uniform(1e-2, 5e-2, N).astype(np.float32)
    res = rng.standard_normal((M, N)).astype(np.float16)
    Yg, _ = oracle.dequant_grouped(acc, sg, sw, epi, res)
    Ys, _ = oracle.dequant(acc.sum(axis=0), sg[:1], False, sw, epi, res)
    assert np.array_equal(Yg.view(np.uint16), Ys.view(np.uint16))
