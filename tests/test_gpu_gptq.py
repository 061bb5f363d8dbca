"""GPU parity of the GPTQ weight solver against the CPU oracle, through the C ABI.

The Hessian and the inverse-Hessian factor are fp64 results reached by different summation and
factorization orders on the two sides, so they are compared within fp64-level tolerances. Given the
same factor, the device column sweep repeats the oracle's fp64 operations in the same order, so its
packed codes and weight scales must equal the oracle's bit for bit (and the rotation operand must
equal the round-to-nearest pack's). End to end, device Hessian -> factor -> pack must lower the
calibration error below round-to-nearest, and the runtime linear on those weights must meet the
output tolerances against the oracle's linear on the same codes.
"""
import numpy as np
import pytest

import oracle
from w4a4_post_quantized_zigzag_amd import binding as bd

from parity_util import check_y_tolerance, dev, host

pytestmark = pytest.mark.gpu


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _problem(N, K, B, seed, M=300):
    rng = _rng(seed)
    W = rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    W[:, rng.choice(K, max(1, K // 64), replace=False)] *= 6
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    mix = np.eye(K) + 0.3 * rng.standard_normal((K, K)) / np.sqrt(K)
    X = [(rng.standard_normal((M, K)) @ mix).astype(np.float16) for _ in range(2)]
    return W, perm, U, X


@pytest.mark.parametrize("K,B", [(512, 128), (256, 64)])
def test_hessian(K, B):
    W, perm, U, X = _problem(64, K, B, K)
    H = bd.gptq_hessian(dev(X[0]), dev(perm), dev(U), B)
    H = bd.gptq_hessian(dev(X[1]), dev(perm), dev(U), B, H=H, accumulate=True)
    ref = oracle.gptq_hessian(X, perm, U, B)
    Hd = host(H)
    assert np.array_equal(Hd, Hd.T)
    assert np.max(np.abs(Hd - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("K", [96, 512, 1024])
def test_factor(K):
    rng = _rng(K)
    A = rng.standard_normal((3 * K, K)) @ (np.eye(K) + 0.2 * rng.standard_normal((K, K)) / np.sqrt(K))
    H = A.T @ A
    H[7, :] = H[:, 7] = 0.0                       # a dead channel
    Hf, dead = bd.gptq_factor(dev(H), 0.05)
    ref, rdead = oracle.gptq_factor(H, 0.05)
    assert np.array_equal(host(dead).astype(bool), rdead)
    assert np.max(np.abs(host(Hf) - ref)) <= 1e-9 * np.max(np.abs(ref))


@pytest.mark.parametrize("N,K,B", [(256, 512, 128), (300, 1024, 64), (64, 4096, 128), (33, 256, 64),
                                   (40, 2048, 128)])
def test_pack_gptq_bit_exact(N, K, B):
    W, perm, U, X = _problem(N, K, B, N + K, M=max(64, K // 4))
    Hf, dead = oracle.gptq_factor(oracle.gptq_hessian(X, perm, U, B))
    wq, sw, rot = bd.pack_weights_gptq(dev(W), dev(perm), dev(U), B, dev(Hf),
                                       dev(dead.astype(np.uint8)))
    ref = oracle.gptq_pack(W, perm, U, B, Hf, dead)
    assert np.array_equal(host(sw).view(np.uint32), ref["w_scale"].view(np.uint32))
    assert np.array_equal(host(wq), ref["wq"])
    _, _, rot_rtn = bd.pack_weights(dev(W), dev(perm), dev(U), B)
    assert np.array_equal(host(rot), host(rot_rtn))


def test_gptq_end_to_end():
    N, K, B, M = 512, 1024, 128, 400
    W, perm, U, X = _problem(N, K, B, 5, M=M)
    H = None
    for x in X:
        H = bd.gptq_hessian(dev(x), dev(perm), dev(U), B, H=H, accumulate=H is not None)
    Hf, dead = bd.gptq_factor(H)
    wq, sw, rot = bd.pack_weights_gptq(dev(W), dev(perm), dev(U), B, Hf, dead)
    # lower calibration error than round-to-nearest, measured on the device's own codes
    R = oracle.rotation(U, B)
    Xr = np.concatenate([oracle.rotate_rows(x, perm, R, B) for x in X])
    Wr = oracle.rotate_rows(W, perm, R, B)
    q_g = oracle.unpack_int4(host(wq), K) * host(sw)[:, None].astype(np.float64)
    rtn = oracle.pack_weights(W, perm, U, B)
    q_r = rtn["codes"] * rtn["w_scale"][:, None].astype(np.float64)
    assert np.linalg.norm(Xr @ (Wr - q_g).T) < 0.8 * np.linalg.norm(Xr @ (Wr - q_r).T)
    # the runtime path is unchanged: per-token linear on the GPTQ weights
    Xt = _rng(6).standard_normal((M, K)).astype(np.float16)
    xq, xs = bd.rotate_quant_act(dev(Xt), dev(perm), rot, B)
    Y = host(bd.gemm(xq, xs, True, wq, sw, K))
    act = oracle.rotate_quant_act(Xt, perm, U, B, "per_token", R=R)
    ref = oracle.gemm(act["codes"], act["scale"], True, oracle.unpack_int4(host(wq), K), host(sw))
    check_y_tolerance(Y, ref["Y"])
