"""CPU pins of the oracle's GPTQ weight solver (the pages' "SVD-Hadamard rotation + GPTQ pack",
--gptq-damp-percent 0.05; vnrobo.com "Kien truc thuc thi", "Build LLM pack").

The solver is fixed against things other than itself: a hand-worked sweep with exact binary values
(the error of column 1 moves column 2 across a rounding boundary), the reduction to round-to-nearest
when the Hessian has no cross terms, the defining identity of the inverse-Hessian factor, the dead
channel rule, and the reconstruction error the method exists to lower.
"""
import numpy as np

import oracle


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _identity_rotation(K):
    # block size 1: every rotation block is [1], and the zigzag order is the descending norm order
    return np.ones((K, 1, 1), np.float32)


def test_hand_worked_sweep():
    # one row, block size 1 (R = 1), columns already in descending-norm order; s = 0.875 / 7 = 1/8
    W = np.array([[0.875, 0.3, 0.2, 0.0]])
    perm = oracle.zigzag_perm(W, 1)
    assert perm.tolist() == [0, 1, 2, 3]
    U = _identity_rotation(4)
    Hf = np.array([[1.0, 0.5, 0.25, 0.0],
                   [0.0, 0.5, 1.0, 0.0],
                   [0.0, 0.0, 2.0, 3.0],
                   [0.0, 0.0, 0.0, 1.0]])
    g = oracle.gptq_pack(W, perm, U, 1, Hf)
    # k=0: 0.875/s = 7 exactly, no error; k=1: 0.3/s = 2.4 -> 2, err = 0.05 / 0.5 = 0.1, so
    # w2 = 0.2 - 0.1 * 1.0 = 0.1 -> 0.8 -> 1 (round-to-nearest alone gives 2); k=2: err =
    # (0.1 - 0.125) / 2 = -0.0125, w3 = 0 + 0.0125 * 3 = 0.0375 -> 0.3 -> 0
    assert g["w_scale"].tolist() == [0.125]
    assert g["codes"].tolist() == [[7, 2, 1, 0]]
    assert oracle.pack_weights(W, perm, U, 1)["codes"].tolist() == [[7, 2, 2, 0]]


def test_no_cross_terms_reduce_to_rtn():
    rng = _rng(1)
    N, K, B = 40, 256, 64
    W = rng.normal(0.0, 0.02, (N, K))
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    H = np.diag(rng.uniform(0.5, 2.0, K))            # uncorrelated channels
    Hf, dead = oracle.gptq_factor(H)
    assert not dead.any()
    assert np.allclose(Hf, np.diag(np.diag(Hf)))        # the factor of a diagonal is diagonal
    g = oracle.gptq_pack(W, perm, U, B, Hf)
    r = oracle.pack_weights(W, perm, U, B)
    assert np.array_equal(g["codes"], r["codes"])
    assert np.array_equal(g["wq"], r["wq"])


def test_factor_identity_and_damping():
    rng = _rng(2)
    K = 96
    A = rng.standard_normal((300, K)) @ rng.standard_normal((K, K))
    H = A.T @ A
    Hf, dead = oracle.gptq_factor(H, 0.05)
    Hd = H + 0.05 * np.mean(np.diag(H)) * np.eye(K)
    assert np.allclose(np.tril(Hf, -1), 0.0)
    assert np.all(np.diag(Hf) > 0)
    assert np.allclose(Hf.T @ Hf @ Hd, np.eye(K), atol=1e-9)


def test_dead_channels():
    rng = _rng(3)
    N, K, B = 16, 128, 64
    W = rng.normal(0.0, 0.02, (N, K))
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    H = np.eye(K) * 2.0
    H[5, :] = H[:, 5] = 0.0                              # channel 5 never sees an activation
    Hf, dead = oracle.gptq_factor(H)
    assert dead.tolist() == [k == 5 for k in range(K)]
    assert np.isclose(Hf[5, 5], 1.0 / np.sqrt(1.0 + 0.05 * np.mean(np.diag(H) + (np.arange(K) == 5))))
    g = oracle.gptq_pack(W, perm, U, B, Hf, dead)
    assert not g["codes"][:, 5].any()
    r = oracle.pack_weights(W, perm, U, B)
    assert np.array_equal(g["w_scale"], r["w_scale"])  # scales come from the weights before zeroing


def test_gptq_lowers_the_calibration_error():
    rng = _rng(4)
    N, K, B = 64, 512, 128
    W = rng.normal(0.0, 0.02, (N, K))
    W[:, rng.choice(K, 5, replace=False)] *= 8
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    mix = np.eye(K) + 0.3 * rng.standard_normal((K, K)) / np.sqrt(K)
    X = [rng.standard_normal((200, K)) @ mix for _ in range(2)]
    Hf, dead = oracle.gptq_factor(oracle.gptq_hessian(X, perm, U, B))
    g = oracle.gptq_pack(W, perm, U, B, Hf, dead)
    r = oracle.pack_weights(W, perm, U, B)
    R = oracle.rotation(U, B)
    Xr = np.concatenate([oracle.rotate_rows(x, perm, R, B) for x in X])
    err = lambda p: np.linalg.norm(Xr @ (p["w_rot"] - p["codes"] * p["w_scale"][:, None]).T)  # noqa: E731
    assert err(g) < 0.8 * err(r)
    # the Hessian is the rotated activations' Gram matrix
    assert np.allclose(oracle.gptq_hessian(X, perm, U, B), Xr.T @ Xr)


def test_hessian_hand_worked():
    # three calibration rows, K = 4, block 2 with U = I (R_b = H_2 = [[1, 1], [1, -1]] / sqrt 2), so
    # X' = A / sqrt 2 with A written out by hand and H = A^T A / 2 (integers halved):
    #   row (1, 0, 2, 0) -> (1, 1, 2, 2);  row (0, 1, 0, 3) -> (1, -1, 3, -3);
    #   row (1, 1, 1, 1) -> (2, 0, 2, 0)
    X = np.array([[1, 0, 2, 0], [0, 1, 0, 3], [1, 1, 1, 1]], np.float32)
    U = np.broadcast_to(np.eye(2, dtype=np.float32), (2, 2, 2)).copy()
    want = 0.5 * np.array([[6, 0, 9, -1], [0, 2, -1, 5], [9, -1, 17, -5], [-1, 5, -5, 13]], float)
    H = oracle.gptq_hessian([X], np.arange(4, dtype=np.int32), U, 2)
    assert np.max(np.abs(H - want)) < 1e-12
    # two samples accumulate
    H2 = oracle.gptq_hessian([X[:2], X[2:]], np.arange(4, dtype=np.int32), U, 2)
    assert np.max(np.abs(H2 - want)) < 1e-12
    # the permutation is applied before the rotation: perm = [2, 0, 3, 1] gathers the columns
    # (x2, x0, x3, x1), i.e. rows (2, 1, 0, 0), (0, 0, 3, 1), (1, 1, 1, 1), so
    # A = [[3, 1, 0, 0], [0, 0, 4, 2], [2, 0, 2, 0]] and H = A^T A / 2
    perm = np.array([2, 0, 3, 1], np.int32)
    Ap = np.array([[3, 1, 0, 0], [0, 0, 4, 2], [2, 0, 2, 0]], float)
    Hp = oracle.gptq_hessian([X], perm, U, 2)
    assert np.max(np.abs(Hp - Ap.T @ Ap / 2)) < 1e-12
    # a mis-permuted Hessian is a different matrix
    assert np.max(np.abs(Hp - H)) > 1.0


def test_hessian_products_and_energy():
    # H v = X'^T (X' v) for the rotated rows of the weight pack's rotation, and the trace is the
    # Frobenius energy of X (an orthogonal rotation preserves it); an unrotated Gram matrix differs
    rng = _rng(41)
    K, B = 64, 16
    X = rng.standard_normal((50, K))
    W = rng.standard_normal((20, K))
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    H = oracle.gptq_hessian([X], perm, U, B)
    R = oracle.rotation(U, B)
    Xr = oracle.rotate_rows(X, perm, R, B)
    for _ in range(3):
        v = rng.standard_normal(K)
        assert np.allclose(H @ v, Xr.T @ (Xr @ v), rtol=1e-12, atol=1e-10)
    Xe = X.astype(np.float32).astype(np.float64)
    assert abs(np.trace(H) - np.sum(Xe ** 2)) < 1e-6 * np.sum(Xe ** 2)
    assert np.max(np.abs(H - Xe.T @ Xe)) > 1.0
