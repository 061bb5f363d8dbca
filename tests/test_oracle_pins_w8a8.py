"""Pins of the oracle's int8 grid (the W8A8 linears the FoldQuantVLA summary keeps for the
attention-output and FFN-down projections, key change 5), checked against what the mathematics
fixes rather than against the oracle's own formulas:

- round-to-nearest error bound (at most half a step) and the extreme codes +-127 at the row maximum;
- ties to even at exact half steps, and saturation at -128 / 127, on inputs built so that every
  intermediate value is exact;
- brute-force integer products on the full int8 range;
- the byte layout (two's complement, one code per byte);
- the calibration table scaling with the grid (max / 127 against max / 7 on the same statistic);
- a W8A8 linear being at least 8x closer to the exact product than the W4A4 one (the step is 16x
  finer on both operands).
"""
import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_int8_rtn_error_and_extreme_codes():
    rng = _rng(1)
    Wr = rng.standard_normal((37, 300)) * np.exp(rng.standard_normal((37, 1)))
    Wr[5] = 0.0
    s, p = oracle.weight_rtn(Wr, bits=8)
    assert p.dtype == np.int8
    assert p.min() >= -128 and p.max() <= 127
    err = np.abs(Wr - p.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-6))
    for n in range(Wr.shape[0]):
        if n == 5:
            assert s[n] == 1.0 and not p[n].any()
            continue
        k = np.argmax(np.abs(Wr[n]))
        assert abs(int(p[n, k])) == 127


def test_int8_activation_ties_to_even_and_saturation():
    # per-token: row max 127 * 2^-3 gives s = 2^-3 and r = 8 exactly, so x * r is exact
    row = np.array([127, -127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5, 0.0]) / 8.0
    out = oracle.quantize_act(row[None, :], "per_token", bits=8)
    assert out["scale"][0] == np.float32(0.125)
    assert out["codes"][0].tolist() == [127, -127, 2, 4, -2, -4, 0, 2, 126, 0]
    # per-step with a small scale saturates both ends of the grid
    out = oracle.quantize_act(row[None, :] * 64, "per_step", np.array([0.125], np.float32), 1, 0,
                              bits=8)
    assert out["codes"][0].tolist()[:2] == [127, -128]
    assert out["codes"].min() == -128 and out["codes"].max() == 127


def test_int8_gemm_brute_force_full_range():
    rng = _rng(2)
    q = rng.integers(-128, 128, (5, 67), dtype=np.int64).astype(np.int8)
    p = rng.integers(-128, 128, (7, 67), dtype=np.int64).astype(np.int8)
    q[0, :] = -128
    p[0, :] = -128
    acc = oracle.int_gemm(q, p)
    for m in range(5):
        for n in range(7):
            assert acc[m, n] == sum(int(q[m, k]) * int(p[n, k]) for k in range(67))
    assert acc[0, 0] == 128 * 128 * 67


def test_int8_byte_layout_round_trip():
    q = np.arange(-128, 128, dtype=np.int16).astype(np.int8).reshape(4, 64)
    b = oracle.pack_codes(q, 8)
    assert b.dtype == np.uint8 and b.shape == (4, 64)
    # rows hold -128..-65, -64..-1, 0..63, 64..127
    assert b[0, 0] == 0x80 and b[1, 0] == 0xC0 and b[1, 63] == 0xFF
    assert b[2, 0] == 0x00 and b[3, 63] == 0x7F
    assert np.array_equal(b.view(np.int8), q)


def test_int8_calibration_scales_with_the_grid():
    rng = _rng(3)
    K, B = 256, 64
    W = rng.normal(0, 0.02, (32, K))
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    Xs = [[rng.standard_normal((8, K)).astype(np.float16)] for _ in range(3)]
    t4 = oracle.calibrate_table(Xs, perm, U, B, bits=4)
    t8 = oracle.calibrate_table(Xs, perm, U, B, bits=8)
    # both are fp32 roundings of the same fp32 max divided by 7 or 127
    amax4 = t4.astype(np.float64) * 7.0
    amax8 = t8.astype(np.float64) * 127.0
    assert np.allclose(amax4, amax8, rtol=2 ** -22, atol=0)


def test_w8a8_linear_is_much_closer_to_the_exact_product():
    rng = _rng(4)
    M, K, N, B = 24, 512, 96, 64
    X = rng.standard_normal((M, K)).astype(np.float16)
    X[:, rng.choice(K, 5, replace=False)] *= 20
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    e4 = np.linalg.norm(oracle.linear(X, W, B, "per_token")["Y"].astype(np.float64) - exact)
    e8 = np.linalg.norm(oracle.linear(X, W, B, "per_token", bits=8)["Y"].astype(np.float64) - exact)
    assert e8 * 8 < e4, (e8, e4)
    assert e8 / np.linalg.norm(exact) < 2e-2


def test_bad_width_is_rejected():
    with pytest.raises(ValueError):
        oracle.weight_rtn(np.ones((2, 4)), bits=6)
