"""GPU parity of the W8A8 linears (int8 grid: the FoldQuantVLA summary keeps the attention-output
and FFN-down projections at W8A8) against the CPU oracle's bits=8 path, through the C ABI.

Integer results are compared bit for bit: packed weights and weight scales, and the int32
accumulators of the int8 GEMM on the small-M, pipelined, split-K and ragged shapes. Activation codes
must equal the oracle's except for certified near-tie flips (as for int4, with a grid 16x finer), and
fp16 outputs must meet the end-to-end tolerances.
"""
import numpy as np
import pytest

import oracle
from w4a4_post_quantized_zigzag_amd import binding as bd

from parity_util import check_y_tolerance, compare_codes, dev, host, rotation_error_bound

pytestmark = pytest.mark.gpu


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _weights(N, K, B, seed):
    rng = _rng(seed)
    W = rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    W[rng.choice(N, max(1, N // 100), replace=False)] *= 8.0
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W[: min(N, 256)], perm, B)
    return W, perm, U


@pytest.mark.parametrize("N,K,B", [(256, 1024, 128), (300, 4096, 128), (64, 256, 64)])
def test_pack_weights_int8_bit_exact(N, K, B):
    W, perm, U = _weights(N, K, B, seed=N)
    wq, sw, _ = bd.pack_weights(dev(W), dev(perm), dev(U), B, bits=8)
    ref = oracle.pack_weights(W, perm, U, B, bits=8)
    assert np.array_equal(host(wq), ref["wq"])
    assert np.array_equal(host(sw).view(np.uint32), ref["w_scale"].view(np.uint32))
    assert host(wq).view(np.int8).min() == -127 or host(wq).view(np.int8).max() == 127


@pytest.mark.parametrize("M,N,K", [(50, 512, 1024), (1, 64, 64), (64, 100, 4096), (300, 1000, 2048),
                                   (1024, 256, 16384), (257, 520, 192), (50, 16400, 2048),
                                   (33, 8200, 4096), (7, 512, 65536)])
def test_gemm_int8_i32_bit_exact(M, N, K):
    rng = _rng(M + N)
    q = rng.integers(-128, 128, (M, K), dtype=np.int64).astype(np.int8)
    p = rng.integers(-128, 128, (N, K), dtype=np.int64).astype(np.int8)
    q[0] = -128
    p[0] = -128
    acc = host(bd.gemm_i32(dev(q.view(np.uint8)), dev(p.view(np.uint8)), K, bits=8))
    if M * N * K <= 64 * 2 ** 20:
        ref = oracle.int_gemm(q, p)
        assert np.array_equal(acc, ref)
    else:
        mi = np.concatenate([rng.integers(0, M, 300), [0, M - 1]])
        ni = np.concatenate([rng.integers(0, N, 300), [0, N - 1]])
        assert np.array_equal(acc[mi, ni], oracle.int_gemm_sampled(q, p, mi, ni))
    assert acc[0, 0] == 128 * 128 * K


def test_gemm_int8_rejects_bad_shapes():
    torch = __import__("torch")
    q = torch.zeros((4, 96), dtype=torch.uint8, device="cuda")
    with pytest.raises(bd.W4A4Error) as e:
        bd.gemm_i32(q, q, 96, bits=8)
    assert e.value.status == bd.W4A4_ERR_SHAPE


@pytest.mark.parametrize("M,K,B,mode,xdt,zz", [
    (50, 1024, 128, "per_step", np.float16, True),      # few tokens
    (600, 1024, 128, "per_token", np.float16, False),   # streaming kernel, identity order
    (520, 8192, 128, "per_step", np.float16, True),     # permutation pass + streaming
    (300, 1024, 128, "per_step", np.float16, True),     # register-staged gather
    (33, 512, 64, "per_token", np.float32, True),       # VALU kernel (fp32 activations)
])
def test_rotate_quant_int8(M, K, B, mode, xdt, zz):
    torch = __import__("torch")
    rng = _rng(M + K)
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 15.0
    X = X.astype(xdt)
    W = rng.normal(0.0, 0.02, (64, K))
    perm = oracle.zigzag_perm(W, B) if zz else np.arange(K, dtype=np.int32)
    U = oracle.block_svd(W, perm, B)
    R = oracle.rotation(U, B)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B, bits=8)
    table = None
    if mode == "per_step":
        table = np.array([oracle.calibrate_table([[X]], perm, U, B, bits=8)[0]], np.float32)
    xrot = torch.empty((M, K), dtype=torch.float32, device="cuda")
    xq, xs = bd.rotate_quant_act(dev(X), dev(perm) if zz else None, rot, B,
                                 dev(table) if table is not None else None,
                                 0 if table is None else 1, 0, xrot_dbg=xrot, bits=8)
    ref = oracle.rotate_quant_act(X, perm, U, B, mode, table, None if table is None else 1, 0, R=R,
                                  bits=8)
    eps = rotation_error_bound(X, perm, R, B)
    assert np.all(np.abs(host(xrot).astype(np.float64) - ref["x_rot"]) <= eps)
    s_dev = host(xs)
    if mode == "per_token":
        assert np.all(np.abs(s_dev - ref["scale"]) <= np.max(eps, axis=1) / 127 * 1.01
                      + 2 ** -23 * ref["scale"])
    else:
        assert s_dev[0] == table[0]
    q_dev = host(xq).view(np.int8)
    assert q_dev.shape == (M, K)
    flips = compare_codes(q_dev, ref["codes"], ref["v"], ref["x_rot"], eps,
                          s_dev if mode == "per_token" else np.full(M, s_dev[0]), ref["scale"],
                          mode == "per_token")
    assert flips <= max(3, q_dev.size * 1e-4)


@pytest.mark.parametrize("M,K,N,mode", [(50, 1024, 512, "per_step"), (300, 2048, 640, "per_token")])
def test_w8a8_linear_end_to_end(M, K, N, mode):
    B = 128
    rng = _rng(M)
    X = rng.standard_normal((M, K)).astype(np.float16)
    W, perm, U = _weights(N, K, B, seed=M + 1)
    table = None
    if mode == "per_step":
        table = oracle.calibrate_table([[X]], perm, U, B, bits=8)
    wq, sw, rot = bd.pack_weights(dev(W), dev(perm), dev(U), B, bits=8)
    xq, xs = bd.rotate_quant_act(dev(X), dev(perm), rot, B, dev(table) if table is not None else None,
                                 0 if table is None else 1, 0, bits=8)
    Y = host(bd.gemm(xq, xs, mode == "per_token", wq, sw, K, bits=8))
    ref = oracle.linear(X, W, B, mode, table, None if table is None else 1, 0 if table is not None
                        else None, perm=perm, U=U, bits=8)
    check_y_tolerance(Y, ref["Y"])


def test_calibrate_int8_scale():
    M, K, B = 700, 2048, 128
    rng = _rng(5)
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = rng.normal(0.0, 0.02, (64, K))
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B, bits=8)
    want = oracle.calibrate_table([[X]], perm, U, B, bits=8)[0]
    got = host(bd.calibrate_act_scale(dev(X), dev(perm), rot, B, bits=8))[0]
    eps = np.max(rotation_error_bound(X, perm, oracle.rotation(U, B), B))
    assert abs(got - want) <= eps / 127 * 1.01 + 2 ** -23 * want
