"""GPU tests of the GEMM that also produces the next linear's per-step codes (w4a4_gemm_next_rq).

Per the pages, each linear quantizes its input with its own step scale after the zigzag order and
the block rotation (vnrobo.com "Y tuong paper"; gist.science "Metodologia" item 1). When the
input is another linear's output in that order, the rotate-quantize can run on the producer's
output tiles. Two checks:
- device consistency: Y equals w4a4_gemm's output, and the codes and scale equal
  w4a4_rotate_quant_act's on the stored Y column slice, bit for bit. This covers int4 and int8
  codes, every epilogue, ragged M, plans that fuse and plans that run the rotate-quantize
  afterwards (K split, small M, a column range the tiles do not divide);
- oracle: Y equals the oracle's GEMM output and the codes equal the oracle's rotate-quantize of
  that Y slice, up to certified near-ties.
"""
import numpy as np
import pytest

import oracle
from oracle.reference import EPI_GELU, EPI_NONE, EPI_RESIDUAL
from w4a4_post_quantized_zigzag_amd import binding as bd
from w4a4_post_quantized_zigzag_amd import inputs

from parity_util import compare_codes, dev, host, rotation_error_bound

pytestmark = pytest.mark.gpu

B = 128
T = 4


def _orthogonal_blocks(nb, seed):
    """Seeded orthogonal U blocks (QR of a Gaussian draw): a rotation input shared by both sides."""
    rng = np.random.Generator(np.random.PCG64(seed))
    U = np.empty((nb, B, B), np.float32)
    for b in range(nb):
        q, r = np.linalg.qr(rng.standard_normal((B, B)))
        U[b] = (q * np.sign(np.diag(r))).astype(np.float32)
    return U


def _setup(M, N, K, epi, kn, per_token, seed):
    xq = inputs.random_packed(M, K, seed=seed)
    wq = inputs.random_packed(N, K, seed=seed + 1)
    sx = inputs.random_scales(M if per_token else 1, seed=seed + 2, lo=2e-3, hi=8e-3)
    sw = inputs.random_scales(N, seed=seed + 3, lo=2e-3, hi=8e-3)
    res = (np.random.Generator(np.random.PCG64(seed + 4)).standard_normal((M, N)) * 0.05
           ).astype(np.float16) if epi == EPI_RESIDUAL else None
    U = _orthogonal_blocks(kn // B, seed + 5)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, kn), np.float32)), dev(np.arange(kn, dtype=np.int32)),
                                dev(U), B)
    return xq, wq, sx, sw, res, U, rot


def _table(Y, col0, kn):
    # step scales around the slice's absmax / 7, so the codes span the grid
    amax = float(np.max(np.abs(Y[:, col0:col0 + kn].astype(np.float32))))
    return np.array([amax * f / 7.0 for f in (0.6, 0.9, 1.2, 1.5)], np.float32)


@pytest.mark.parametrize("M,N,K,epi,col0,kn,bits,per_token", [
    (1600, 3072, 1024, EPI_NONE, 2048, 1024, 4, False),    # QKV-shaped: the V columns feed O
    (1600, 4096, 1024, EPI_GELU, 0, 4096, 4, False),       # up-shaped, 8-wave tiles
    (1600, 4096, 1024, EPI_GELU, 0, 4096, 8, False),       # int8 codes for a W8A8 next linear
    (300, 1024, 2048, EPI_RESIDUAL, 256, 512, 4, True),    # ragged M, per-token input scales
    (1024, 2048, 16384, EPI_NONE, 0, 2048, 4, False),      # K split: runs after the GEMM
    (40, 4096, 1024, EPI_NONE, 1024, 1024, 4, False),      # small M: runs after the GEMM
    (520, 1280, 1024, EPI_RESIDUAL, 128, 1024, 4, False),  # column range vs tile width
    (777, 2560, 1024, EPI_NONE, 512, 2048, 8, True),
])
def test_next_rq_equals_gemm_then_rotate_quant(M, N, K, epi, col0, kn, bits, per_token):
    xq, wq, sx, sw, res, U, rot = _setup(M, N, K, epi, kn, per_token, seed=M + N)
    Yref = bd.gemm(dev(xq), dev(sx), per_token, dev(wq), dev(sw), K, epilogue=epi,
                   residual=dev(res) if res is not None else None)
    table = _table(host(Yref).view(np.float16), col0, kn)
    for step in (0, T - 1):
        Y, xqn, xsn = bd.gemm_next_rq(dev(xq), dev(sx), per_token, dev(wq), dev(sw), K, col0, rot,
                                      dev(table), T, step, kn, next_bits=bits, epilogue=epi,
                                      residual=dev(res) if res is not None else None)
        assert np.array_equal(host(Y).view(np.uint16), host(Yref).view(np.uint16))
        xq_ref, xs_ref = bd.rotate_quant_act(Yref[:, col0:col0 + kn], None, rot, B, dev(table), T,
                                             step, bits=bits)
        assert np.array_equal(host(xqn), host(xq_ref))
        assert host(xsn)[0] == host(xs_ref)[0] == table[step]


@pytest.mark.parametrize("M,N,K,epi,col0,kn", [
    (520, 1024, 1024, EPI_RESIDUAL, 256, 512),
    (200, 512, 2048, EPI_NONE, 0, 512),
])
def test_next_rq_matches_oracle(M, N, K, epi, col0, kn):
    xq, wq, sx, sw, res, U, rot = _setup(M, N, K, epi, kn, False, seed=7 * M + N)
    ref = oracle.gemm(oracle.unpack_int4(xq, K), sx, False, oracle.unpack_int4(wq, K), sw, epi, res)
    Yo = ref["Y"]
    table = _table(Yo, col0, kn)
    step = 1
    Y, xqn, xsn = bd.gemm_next_rq(dev(xq), dev(sx), False, dev(wq), dev(sw), K, col0, rot,
                                  dev(table), T, step, kn, epilogue=epi,
                                  residual=dev(res) if res is not None else None)
    assert np.array_equal(host(Y).view(np.uint16), Yo.view(np.uint16))
    Xn = Yo[:, col0:col0 + kn]
    perm = np.arange(kn, dtype=np.int32)
    R = oracle.rotation(U, B)
    act = oracle.rotate_quant_act(Xn, perm, U, B, "per_step", table, T, step, R=R)
    eps = rotation_error_bound(Xn, perm, R, B)
    q_dev = oracle.unpack_int4(host(xqn), kn)
    assert host(xsn)[0] == table[step]
    flips = compare_codes(q_dev, act["codes"], act["v"], act["x_rot"], eps,
                          np.full(M, table[step]), act["scale"], False)
    assert flips <= max(3, q_dev.size * 1e-4)


def test_next_rq_empty_batch():
    K, N, kn = 256, 256, 128
    xq = inputs.random_packed(0, K, seed=1)
    wq = inputs.random_packed(N, K, seed=2)
    _, _, _, _, _, _, rot = _setup(1, N, K, EPI_NONE, kn, False, seed=3)
    Y, xqn, _ = bd.gemm_next_rq(dev(xq), dev(np.ones(1, np.float32)), False, dev(wq),
                                dev(np.ones(N, np.float32)), K, 0, rot,
                                dev(np.ones(T, np.float32)), T, 0, kn)
    assert tuple(Y.shape) == (0, N) and tuple(xqn.shape) == (0, kn // 2)
