"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU needed).

Each test checks the oracle against something other than itself: a library routine that computes
the same quantity another way (scipy's Sylvester Hadamard, LAPACK eigenvalues, numpy's integer
matmul), a closed form, a hand-worked case of the zigzag reading, an exhaustive enumeration, an
invariant the method relies on (orthogonality, X W^T preserved, equal energy per rotated channel,
RTN error at most half a step), or a degenerate case that reduces to textbook int4 RTN.

Sources, cited by page title and section:
 gist.science (pt) "Metodologia" 1: SVD W = U Sigma V^T with R_SVD = U equalizing per-row weight
   energy; normalized Hadamard H spreading a dominant channel; R = R_SVD . H; blocks along C_in;
   zigzag permutation by weight column norms. Item 2: per-step table from calibration trajectories.
 vnrobo.com "Build DiT action head pack": 4-bit weights and activations, RTN, 8 steps, block 64.
 aiexpert.news: a step-count mismatch or truncated table is a failure mode.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from w4a4_post_quantized_zigzag_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------- Hadamard (I1)

@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_is_normalized_sylvester(B):
    H = oracle.hadamard(B)
    ref = scipy.linalg.hadamard(B).astype(np.float64) / np.sqrt(float(B))
    assert np.array_equal(H, ref)
    assert np.max(np.abs(H @ H.T - np.eye(B))) <= 1e-15 * max(1, B)


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.hadamard(96)


# --------------------------------------------------------------------------- zigzag (I8)

def _w_with_norm_order(order):
    """One-row weight whose column norms strictly decrease along `order`."""
    K = len(order)
    W = np.zeros((1, K))
    for rank, ch in enumerate(order):
        W[0, ch] = float(K - rank)
    return W


def test_zigzag_hand_example():
    # K = 8, B = 2, nb = 4. Ranks 0..3 go to blocks 0..3 (pass 0), ranks 4..7 to blocks 3..0
    # (pass 1), so block b holds {s_b, s_(7-b)} in that order.
    s = [3, 0, 7, 1, 5, 2, 6, 4]
    perm = oracle.zigzag_perm(_w_with_norm_order(s), 2)
    assert perm.tolist() == [s[0], s[7], s[1], s[6], s[2], s[5], s[3], s[4]]


def test_zigzag_ties_go_to_lower_index():
    perm = oracle.zigzag_perm(np.ones((3, 8)), 2)
    assert perm.tolist() == [0, 7, 1, 6, 2, 5, 3, 4]


def test_zigzag_three_passes():
    # K = 16, B = 4, nb = 4: even passes run forward, odd passes backward.
    s = list(range(16))
    perm = oracle.zigzag_perm(_w_with_norm_order(s), 4)
    assert perm.reshape(4, 4).tolist() == [[0, 7, 8, 15], [1, 6, 9, 14], [2, 5, 10, 13],
                                           [3, 4, 11, 12]]


@pytest.mark.parametrize("K,B", [(256, 64), (1024, 128), (2048, 128), (512, 1), (64, 64)])
def test_zigzag_one_channel_per_pass(K, B):
    W = _rng(K + B).standard_normal((37, K)) * _rng(1).uniform(0.1, 3.0, K)
    perm = oracle.zigzag_perm(W, B)
    assert sorted(perm.tolist()) == list(range(K))
    c2 = (W.astype(np.float64) ** 2).sum(axis=0)
    rank = np.empty(K, np.int64)
    rank[np.argsort(-c2, kind="stable")] = np.arange(K)
    nb = K // B
    # block b takes exactly one channel from each run of nb consecutive ranks, at position = pass
    for b in range(nb):
        for p in range(B):
            assert rank[perm[b * B + p]] // nb == p
    # spreading: the per-block norm sums are far more even than for contiguous blocks of ranks
    if nb > 1 and B > 1:
        zz = np.array([c2[perm[b * B:(b + 1) * B]].sum() for b in range(nb)])
        order = np.argsort(-c2, kind="stable")
        contig = np.array([c2[order[b * B:(b + 1) * B]].sum() for b in range(nb)])
        assert zz.max() / zz.min() < contig.max() / contig.min()


def test_colnorm2_matches_numpy():
    W = _rng(5).standard_normal((300, 40)).astype(np.float16)
    c2 = oracle.colnorm2(W)
    ref = np.einsum("nk,nk->k", W.astype(np.float64), W.astype(np.float64))
    assert np.allclose(c2, ref, rtol=1e-13, atol=0)


# --------------------------------------------------------------------------- SVD factor (I2, I4)

@pytest.mark.parametrize("N,K,B", [(256, 256, 64), (300, 256, 128), (96, 128, 64), (40, 128, 64)])
def test_block_svd_is_right_singular_basis(N, K, B):
    W = _rng(N * K).normal(0, 0.02, (N, K))
    W[:2] *= 10
    perm = oracle.zigzag_perm(W, B)
    U32, U64, sig = oracle.block_svd(W, perm, B, return_fp64=True)
    nb = K // B
    for b in range(nb):
        Wb = W[:, perm[b * B:(b + 1) * B]]
        V = U64[b]
        assert np.max(np.abs(V.T @ V - np.eye(B))) < 1e-12
        assert np.max(np.abs(U32[b].astype(np.float64).T @ U32[b] - np.eye(B))) < 2e-6
        # W_b V has mutually orthogonal columns whose squared norms are the eigenvalues of
        # W_b^T W_b in descending order (LAPACK's symmetric eigensolver, a different routine)
        G = (Wb @ V).T @ (Wb @ V)
        lam = np.sort(np.linalg.eigvalsh(Wb.T @ Wb))[::-1]
        scale = lam[0]
        assert np.max(np.abs(G - np.diag(np.diag(G)))) < 1e-10 * scale
        assert np.allclose(np.diag(G), lam, rtol=0, atol=1e-10 * scale)
        # sign convention: the largest-magnitude entry of each column is positive
        idx = np.argmax(np.abs(V), axis=0)
        assert np.all(V[idx, np.arange(B)] > 0)
        # equal energy: every column of W_b . U_b . H carries ||W_b||_F^2 / B
        # (sum_i sigma_i^2 H_ij^2 with H_ij^2 = 1/B)
        H = scipy.linalg.hadamard(B) / np.sqrt(B)
        e = ((Wb @ V @ H) ** 2).sum(axis=0)
        target = (Wb ** 2).sum() / B
        assert np.allclose(e, target, rtol=1e-10, atol=0)
        e32 = ((Wb @ U32[b].astype(np.float64) @ H) ** 2).sum(axis=0)
        assert np.allclose(e32, target, rtol=1e-5, atol=0)


def test_equal_energy_fails_for_hadamard_first():
    # the composition order matters: H . U does not equalize column energies
    W = _rng(9).normal(0, 0.02, (128, 64))
    W[:, 3] *= 30
    perm = np.arange(64, dtype=np.int32)
    _, U64, _ = oracle.block_svd(W, perm, 64, return_fp64=True)
    H = scipy.linalg.hadamard(64) / 8.0
    good = ((W @ U64[0] @ H) ** 2).sum(axis=0)
    bad = ((W @ H @ U64[0]) ** 2).sum(axis=0)
    assert np.ptp(good) / good.mean() < 1e-10
    assert np.ptp(bad) / bad.mean() > 1e-3


# --------------------------------------------------------------------------- rotation (I2, I3)

def test_rotation_matches_matmul_and_is_orthogonal():
    B, nb = 128, 3
    W = _rng(2).standard_normal((200, nb * B))
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    R = oracle.rotation(U, B)
    H = scipy.linalg.hadamard(B) / np.sqrt(B)
    for b in range(nb):
        assert np.allclose(R[b], U[b].astype(np.float64) @ H, rtol=0, atol=1e-15)
        assert np.max(np.abs(R[b] @ R[b].T - np.eye(B))) < 2e-6


def test_rotate_rows_matches_block_matmul():
    B, K = 64, 256
    A = _rng(3).standard_normal((9, K))
    perm = _rng(4).permutation(K).astype(np.int32)
    U = _rng(5).standard_normal((K // B, B, B)).astype(np.float32)
    R = oracle.rotation(U, B)
    Y = oracle.rotate_rows(A, perm, R, B)
    Ap = A[:, perm]
    for b in range(K // B):
        ref = Ap[:, b * B:(b + 1) * B] @ R[b]
        assert np.allclose(Y[:, b * B:(b + 1) * B], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("name,M,K,N", [("linear_small", 16, 256, 256), ("dit_mlp_up", 50, 1024, 256),
                                        ("prefill_proj", 64, 512, 300), ("longk_down", 32, 2048, 128)])
def test_rotation_preserves_xwt(name, M, K, N):
    d = inputs.linear_inputs(name, M=M, K=K, N=N, calib=1)
    X = d["X_steps"][0] if "X_steps" in d else d["X"]
    W, B = d["W"], d["block"]
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    R = oracle.rotation(U, B)
    Xr = oracle.rotate_rows(X, perm, R, B)
    Wr = oracle.rotate_rows(W, perm, R, B)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    rel = np.linalg.norm(Xr @ Wr.T - ref) / np.linalg.norm(ref)
    assert rel <= 1e-4
    assert rel <= 1e-6  # fp32-rounded U: expected ~1e-7
    # a mismatched permutation (inverse perm on the weight side) breaks it
    inv = np.argsort(perm).astype(np.int32)
    if not np.array_equal(inv, perm):
        bad = Xr @ oracle.rotate_rows(W, inv, R, B).T
        assert np.linalg.norm(bad - ref) / np.linalg.norm(ref) > 1e-2


# --------------------------------------------------------------------------- RTN (I5)

def test_weight_rtn_error_at_most_half_step():
    d = inputs.linear_inputs("prefill_proj", M=4, K=512, N=300)
    W, B = d["W"], d["block"]
    perm = oracle.zigzag_perm(W, B)
    pw = oracle.pack_weights(W, perm, oracle.block_svd(W, perm, B), B)
    Wr, s, p = pw["w_rot"], pw["w_scale"].astype(np.float64), pw["codes"]
    err = np.abs(Wr - s[:, None] * p)
    assert np.all(err <= s[:, None] / 2 * (1 + 1e-12))
    assert p.min() >= -7 and p.max() <= 7
    assert np.all(np.max(np.abs(p), axis=1) == 7)
    m = np.max(np.abs(Wr), axis=1)
    assert np.allclose(s * 7, m, rtol=2 ** -23, atol=0)


def test_weight_rtn_zero_row():
    s, p = oracle.weight_rtn(np.zeros((2, 8)))
    assert s.tolist() == [1.0, 1.0] and not p.any()


def test_per_token_error_at_most_half_step():
    X = _rng(11).laplace(0, 1, (40, 256))
    X[3] = 0.0
    out = oracle.quantize_act(X, "per_token")
    x32, s, q = out["x32"].astype(np.float64), out["scale"].astype(np.float64), out["codes"]
    nz = np.arange(40) != 3
    err = np.abs(x32 - s[:, None] * q)
    assert np.all(err[nz] <= s[nz, None] / 2 * (1 + 2 ** -20))
    assert q.min() >= -7 and q.max() <= 7
    assert np.all(np.max(np.abs(q[nz]), axis=1) == 7)
    assert s[3] == 1.0 and not q[3].any()


def test_per_step_selects_scale_and_rejects_bad_step():
    # table = 2^t: the reciprocal and the product are exact, so codes are clip(rint(x / 2^t))
    table = np.array([2.0 ** t for t in range(8)], np.float32)
    X = _rng(12).normal(0, 20, (16, 64))
    for t in range(8):
        out = oracle.quantize_act(X, "per_step", table, 8, t)
        x32 = X.astype(np.float32).astype(np.float64)
        assert np.array_equal(out["codes"], np.clip(np.rint(x32 / 2.0 ** t), -8, 7))
        assert np.all(out["scale"] == table[t])
    # clipping under a static scale reaches -8
    assert out["codes"].min() == -8 or np.min(X) / 128 > -7.5
    for bad in (8, -1, 100):
        with pytest.raises(ValueError):
            oracle.quantize_act(X, "per_step", table, 8, bad)
    with pytest.raises(ValueError):
        oracle.quantize_act(X, "per_step", table[:5], 8, 2)


@pytest.mark.parametrize("bad", [0.0, -1.0, np.inf, -np.inf, np.nan])
def test_per_step_unusable_entry_poisons_output(bad):
    # an entry that is not a positive finite scale produces no code (all 0) and a NaN scale, so the
    # dequantized output is NaN everywhere: a wrong or truncated table is a failure mode
    # (aiexpert.news) and must not look like a valid result; the neighbouring entries are unaffected
    table = np.array([0.25, bad, 0.5], np.float32)
    X = _rng(13).normal(0, 3, (6, 32))
    out = oracle.quantize_act(X, "per_step", table, 3, 1)
    assert not out["codes"].any() and np.all(np.isnan(out["scale"]))
    p = _rng(14).integers(-8, 8, (5, 32)).astype(np.int8)
    y = oracle.gemm(out["codes"], out["scale"][:1], False, p, np.full(5, 0.1, np.float32))["Y"]
    assert np.all(np.isnan(y.astype(np.float32)))
    ok = oracle.quantize_act(X, "per_step", table, 3, 2)
    x32 = X.astype(np.float32).astype(np.float64)
    assert np.array_equal(ok["codes"], np.clip(np.rint(x32 * 2.0), -8, 7))
    og = oracle.quantize_act_grouped(X, 16, np.array([[0.5, bad]], np.float32), 1, 0)
    assert np.isnan(og["scale"][1]) and og["scale"][0] == np.float32(0.5)
    assert not og["codes"][:, 16:].any()
    assert np.array_equal(og["codes"][:, :16], np.clip(np.rint(x32[:, :16] * 2.0), -8, 7))


def test_rne_ties_at_half_steps():
    # exact half-steps round to the even code
    X = np.array([[0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 6.5, -7.5]])
    out = oracle.quantize_act(X, "per_step", np.ones(1, np.float32), 1, 0)
    assert out["codes"].tolist() == [[0, 2, 2, 0, -2, -2, 6, -8]]


# --------------------------------------------------------------------------- packing (I7)

def test_pack_unpack_exhaustive():
    allbytes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = oracle.unpack_int4(allbytes, 512)
    assert q.min() == -8 and q.max() == 7
    assert np.array_equal(oracle.pack_int4(q), allbytes)


def test_nibble_order_and_twos_complement():
    q = np.array([[1, -2, -8, 7, 7, -8, 0, -1]], np.int8)
    assert oracle.pack_int4(q).tolist() == [[0xE1, 0x78, 0x87, 0xF0]]


# --------------------------------------------------------------------------- integer GEMM (I6)

@pytest.mark.parametrize("M,N,K", [(1, 1, 2), (3, 5, 16), (8, 8, 256), (7, 3, 130)])
def test_int_gemm_matches_numpy(M, N, K):
    q = inputs._rng(M * 100 + K).integers(-8, 8, (M, K), dtype=np.int8)
    p = inputs._rng(N * 7 + K).integers(-8, 8, (N, K), dtype=np.int8)
    assert np.array_equal(oracle.int_gemm(q, p), q.astype(np.int64) @ p.astype(np.int64).T)


def test_int_gemm_all_nibble_pairs():
    a = np.repeat(np.arange(-8, 8, dtype=np.int8), 16).reshape(1, 256)
    b = np.tile(np.arange(-8, 8, dtype=np.int8), 16).reshape(1, 256)
    expect = sum(i * j for i in range(-8, 8) for j in range(-8, 8))
    assert oracle.int_gemm(a, b)[0, 0] == expect


@pytest.mark.parametrize("K", [2, 256, 16384])
def test_int_gemm_extremes(K):
    neg = np.full((2, K), -8, np.int8)
    pos = np.full((3, K), 7, np.int8)
    assert np.all(oracle.int_gemm(neg, neg) == 64 * K)
    assert np.all(oracle.int_gemm(neg, pos) == -56 * K)
    if K == 16384:
        assert oracle.int_gemm(neg, neg)[0, 0] == 2 ** 20


def test_int_gemm_sampled_agrees():
    q = inputs._rng(1).integers(-8, 8, (20, 64), dtype=np.int8)
    p = inputs._rng(2).integers(-8, 8, (30, 64), dtype=np.int8)
    mi, ni = np.array([0, 19, 5]), np.array([29, 0, 7])
    full = q.astype(np.int64) @ p.astype(np.int64).T
    assert oracle.int_gemm_sampled(q, p, mi, ni).tolist() == full[mi, ni].tolist()


# --------------------------------------------------------------------------- dequant

def test_dequant_exact_cases():
    acc = np.array([[3, -5, 0], [1024, -2048, 7]], np.int64)
    Y, y32 = oracle.dequant(acc, np.array([0.5, 0.25], np.float32), True,
                            np.array([2.0, 4.0, 0.125], np.float32))
    assert Y.tolist() == [[3.0, -10.0, 0.0], [512.0, -2048.0, 0.21875]]
    Y2, _ = oracle.dequant(acc, np.array([2.0], np.float32), False, np.ones(3, np.float32))
    assert Y2.tolist() == (2.0 * acc).tolist()
    big, _ = oracle.dequant(np.array([[2 ** 20]]), np.array([1.0], np.float32), False,
                            np.array([1.0], np.float32))
    assert np.isinf(big[0, 0])  # fp16 overflow saturates to inf
    res = np.array([[1.0, -1.0, 0.5], [0.0, 0.0, -0.125]], np.float16)
    Y3, _ = oracle.dequant(acc, np.array([0.5, 0.25], np.float32), True,
                           np.array([2.0, 4.0, 0.125], np.float32), oracle.reference.EPI_RESIDUAL,
                           res)
    assert Y3.tolist() == [[4.0, -11.0, 0.5], [512.0, -2048.0, 0.09375]]
    with pytest.raises(OverflowError):
        oracle.dequant(np.array([[2 ** 31]]), np.ones(1, np.float32), False, np.ones(1, np.float32))


def test_gelu_epilogue():
    from scipy.special import erf
    acc = np.arange(-40, 40, dtype=np.int64).reshape(4, 20)
    sx = np.array([0.1], np.float32)
    sw = np.linspace(0.05, 2, 20).astype(np.float32)
    Y, y32 = oracle.dequant(acc, sx, False, sw, oracle.reference.EPI_GELU)
    v = y32.astype(np.float64)
    ref = (0.5 * v * (1 + erf(v / np.sqrt(2)))).astype(np.float16)
    assert np.array_equal(Y, ref)
    assert Y[acc == 0].tolist() == [0.0] * int((acc == 0).sum())


# --------------------------------------------------------------------------- closed forms (I9, I10)

@pytest.mark.parametrize("K,B,c,v", [(256, 64, 77, 3.0), (512, 128, 5, -11.0), (64, 8, 63, 0.25)])
def test_one_hot_row_codes_follow_hadamard_row(K, B, c, v):
    W = _rng(K).standard_normal((10, K))
    perm = oracle.zigzag_perm(W, B)
    U = np.broadcast_to(np.eye(B, dtype=np.float32), (K // B, B, B)).copy()
    X = np.zeros((1, K))
    X[0, c] = v
    out = oracle.rotate_quant_act(X, perm, U, B, "per_token")
    pos = int(np.argsort(perm)[c])
    b, i = divmod(pos, B)
    codes = out["codes"][0]
    H = scipy.linalg.hadamard(B)
    expect = np.zeros(K, np.int64)
    expect[b * B:(b + 1) * B] = 7 * np.sign(v) * H[i]
    assert np.array_equal(codes, expect)


def test_block_one_is_textbook_int4_rtn():
    rng = _rng(21)
    M, K, N = 12, 64, 20
    X = rng.laplace(0, 1, (M, K)).astype(np.float32)
    W = rng.normal(0, 0.05, (N, K)).astype(np.float32)
    out = oracle.linear(X, W, 1, "per_token")
    # textbook symmetric int4 RTN: per-token activation scale, per-channel weight scale
    ax = np.max(np.abs(X), axis=1).astype(np.float64)
    sx = (ax / 7.0).astype(np.float32)
    rx = (1.0 / sx.astype(np.float64)).astype(np.float32)
    q = np.clip(np.rint(X * rx[:, None]), -8, 7).astype(np.int64)
    aw = np.max(np.abs(W.astype(np.float64)), axis=1)
    sw = (aw / 7.0).astype(np.float32)
    p = np.clip(np.rint(W.astype(np.float64) / sw.astype(np.float64)[:, None]), -8, 7).astype(np.int64)
    acc = q @ p.T
    Y = ((acc.astype(np.float32) * sx[:, None]) * sw[None, :]).astype(np.float16)
    assert np.array_equal(out["acc"], acc)
    assert np.array_equal(out["Y"], Y)


# --------------------------------------------------------------------------- calibration, quality

def test_calibrated_table_covers_calibration_set():
    d = inputs.linear_inputs("dit_mlp_up", M=50, K=256, N=64, calib=3)
    W, B = d["W"], 128
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    table = oracle.calibrate_table(d["X_calib"], perm, U, B)
    assert table.shape == (8,)
    # sigma_t falls from 3.0 to 0.5, so the table falls too
    assert np.all(np.diff(table) < 0)
    for t in range(8):
        amax = 0.0
        for Xc in d["X_calib"][t]:
            out = oracle.rotate_quant_act(Xc, perm, U, B, "per_step", table, 8, t)
            assert out["codes"].min() >= -7 and out["codes"].max() <= 7
            amax = max(amax, float(np.max(np.abs(out["x32"]))))
        assert table[t] == np.float32(amax / 7.0)


@pytest.mark.parametrize("name,M,K,N", [("linear_small", 16, 256, 256), ("prefill_proj", 64, 512, 256),
                                        ("longk_down", 32, 1024, 128)])
def test_rotation_reduces_w4a4_error(name, M, K, N):
    d = inputs.linear_inputs(name, M=M, K=K, N=N, calib=1)
    X = d["X_steps"][0] if "X_steps" in d else d["X"]
    W, B = d["W"], d["block"]
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    rot = oracle.linear(X, W, B, "per_token")["Y"].astype(np.float64)
    plain = oracle.linear(X, W, 1, "per_token")["Y"].astype(np.float64)
    e_rot = np.linalg.norm(rot - ref) / np.linalg.norm(ref)
    e_plain = np.linalg.norm(plain - ref) / np.linalg.norm(ref)
    assert e_rot < e_plain


def test_stack_wiring_zero_weights_is_identity():
    # QKV = 0 -> V = 0 -> O(V) = 0 -> h2 = x; up = 0 -> GELU(0) = 0 -> down = 0 -> out = h2 = x
    h, f, B = 128, 256, 64
    W = [{"qkv": np.zeros((3 * h, h), np.float16), "o": np.zeros((h, h), np.float16),
          "up": np.zeros((f, h), np.float16), "down": np.zeros((h, f), np.float16)}
         for _ in range(2)]
    layers = oracle.stack_prepare(W, B)
    X = (_rng(4).standard_normal((9, h)) * 3).astype(np.float16)
    outs = []
    Y = oracle.stack_run(layers, X, B, "per_token", outputs=outs)
    assert np.array_equal(Y, X)
    assert len(outs) == 8 and not outs[0].any() and np.array_equal(outs[1], X)
    # calibration of the zero branches records scale 1.0 (all-zero rotated inputs)
    tables = oracle.stack_calibrate(layers, [[X]], B)
    assert tables[0]["o"][0] == 1.0 and tables[0]["down"][0] == 1.0 and tables[0]["qkv"][0] > 0


def test_stack_rows_are_independent():
    # tokens never mix: running a subset of rows gives the same rows of the full run
    h, f, B = 128, 256, 128
    W = inputs.stack_weights(layers=1, hidden=h, ffn=f, seed=3)
    layers = oracle.stack_prepare(W, B)
    X = (_rng(5).standard_normal((12, h))).astype(np.float16)
    full = oracle.stack_run(layers, X, B, "per_token")
    part = oracle.stack_run(layers, X[[2, 7, 11]], B, "per_token")
    assert np.array_equal(full[[2, 7, 11]], part)


def test_recipe_constants_from_the_pages():
    with open(os.path.join(GOLDEN, "recipe.json")) as f:
        rc = json.load(f)
    # 4-bit symmetric two's complement: codes span [-2^(b-1), 2^(b-1)-1]
    lo, hi = -(2 ** (rc["a_bits"] - 1)), 2 ** (rc["a_bits"] - 1) - 1
    X = np.array([[-1000.0, 1000.0, 0.0, 1.0]])
    out = oracle.quantize_act(X, "per_step", np.ones(rc["num_steps"], np.float32), rc["num_steps"],
                              rc["num_steps"] - 1)
    assert out["codes"].min() == lo and out["codes"].max() == hi
    with pytest.raises(ValueError):
        oracle.quantize_act(X, "per_step", np.ones(rc["num_steps"], np.float32), rc["num_steps"],
                            rc["num_steps"])
    # the recipe's block size is a supported rotation block
    B = rc["duquant_block_size"]
    W = _rng(0).standard_normal((B, 2 * B))
    assert sorted(oracle.zigzag_perm(W, B).tolist()) == list(range(2 * B))
    assert rc["svd_rank"] == 0 and rc["use_rtn"] and rc["w_bits"] == 4


def test_mixed_stack_w8a8_linears():
    # FoldQuantVLA summary: attention-output and FFN-down at W8A8, the rest W4A4. Layer 0's QKV is
    # W4A4 in both configurations, so the O projection sees the same input; its table entry is the
    # same max over 127 instead of 7, and its output lands much closer to the exact product.
    h, f, B = 128, 512, 64
    W = inputs.stack_weights(layers=1, hidden=h, ffn=f, seed=8)
    X = (_rng(9).standard_normal((24, h))).astype(np.float16)
    l4 = oracle.stack_prepare(W, B)
    l8 = oracle.stack_prepare(W, B, w8=("o", "down"))
    assert [l8[0][n]["bits"] for n in ("qkv", "o", "up", "down")] == [4, 8, 4, 8]
    assert l8[0]["o"]["pack"]["wq"].shape == (h, h) and l4[0]["o"]["pack"]["wq"].shape == (h, h // 2)
    t4 = oracle.stack_calibrate(l4, [[X]], B)
    t8 = oracle.stack_calibrate(l8, [[X]], B)
    assert t8[0]["qkv"][0] == t4[0]["qkv"][0]
    for a, b in ((t4[0]["o"][0], t8[0]["o"][0]),):
        assert abs(float(a) * 7.0 - float(b) * 127.0) <= 2 ** -22 * float(a) * 7.0
    o4, o8 = [], []
    oracle.stack_run(l4, X, B, "per_token", outputs=o4)
    oracle.stack_run(l8, X, B, "per_token", outputs=o8)
    assert np.array_equal(o4[0], o8[0])
    V = o4[0][:, 2 * h:3 * h].astype(np.float64)
    exact = V @ W[0]["o"].astype(np.float64).T + X.astype(np.float64)
    e4 = np.linalg.norm(o4[1] - exact) / np.linalg.norm(exact - X)
    e8 = np.linalg.norm(o8[1] - exact) / np.linalg.norm(exact - X)
    assert e8 < e4 / 4
