"""GPU parity of the two large single linears at their full benchmark shapes, through the C ABI, in
the launch configuration the benchmark times:

  prefill projection  X fp16 [1024, 2048], W fp16 [16384, 2048], block 128, per-token scales;
  long-K projection   X fp16 [1024, 16384], W fp16 [2048, 16384], block 128, per-token scales.

The device runs the whole linear (weight pack, rotate-quantize, GEMM) at full size. Per-token
quantization is row-local, so the oracle runs on sampled rows:
  - packed weights and weight scales: every row, bit for bit;
  - quantize stage on every row: the oracle's quantizer on the device's rotated activations gives
    the device's codes and scales exactly;
  - sampled rows end to end: codes equal the oracle's fp64-path codes except for certified
    near-tie flips; given the device's codes and scales the oracle's integer GEMM and
    dequantization reproduce the device's fp16 output bit for bit; and the output is within the
    fp16 tolerance of the oracle's own linear.
The zigzag permutation and SVD factor are the oracle's (inputs to both sides).

Pages: gist.science (pt) "Metodologia" 1 (zigzag, blockwise composite rotation before
quantization); FoldQuantVLA summary key change 2 (dynamic per-token activation scales).
"""
import numpy as np
import pytest

import oracle
from w4a4_post_quantized_zigzag_amd import binding as bd
from w4a4_post_quantized_zigzag_amd import inputs

from parity_util import (check_y_tolerance, compare_codes, dev, host, oracle_calibration,
                         rotation_error_bound)

pytestmark = pytest.mark.gpu


def _same_f32(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("name", ["prefill_proj", "longk_down"])
def test_full_shape_linear(name):
    torch = __import__("torch")
    d = inputs.linear_inputs(name)
    W, X, B = d["W"], d["X"], d["block"]
    M, K = X.shape
    perm, U = oracle_calibration(name + "_full", W, B)
    wq, sw, rot = bd.pack_weights(dev(W), dev(perm), dev(U), B)
    xd = dev(X)
    xq, xs = bd.rotate_quant_act(xd, dev(perm), rot, B)
    Y = host(bd.gemm(xq, xs, True, wq, sw, K))
    xrot = torch.empty((M, K), dtype=torch.float32, device="cuda")
    xq_dbg, xs_dbg = bd.rotate_quant_act(xd, dev(perm), rot, B, xrot_dbg=xrot)
    q_all, s_all = host(xq), host(xs)
    assert np.array_equal(q_all, host(xq_dbg)) and _same_f32(s_all, host(xs_dbg))

    # weights: every row bit for bit
    pw = oracle.pack_weights(W, perm, U, B)
    assert np.array_equal(host(wq), pw["wq"])
    assert _same_f32(host(sw), pw["w_scale"])

    # quantize stage on every row
    st = oracle.quantize_act(host(xrot).astype(np.float64), "per_token")
    assert np.array_equal(oracle.unpack_int4(q_all, K), st["codes"])
    assert _same_f32(s_all, st["scale"])

    # sampled rows end to end
    rows = np.array([0, 1, 100, 511, 512, 777, M - 2, M - 1])
    ref = oracle.rotate_quant_act(X[rows], perm, U, B, "per_token", R=pw["R"])
    eps = rotation_error_bound(X[rows], perm, pw["R"], B)
    q_dev = oracle.unpack_int4(q_all[rows], K)
    s_dev = s_all[rows]
    assert np.all(np.abs(s_dev - ref["scale"]) <= np.max(eps, axis=1) / 7 * 1.01
                  + 2 ** -23 * ref["scale"])
    flips = compare_codes(q_dev, ref["codes"], ref["v"], ref["x_rot"], eps, s_dev, ref["scale"], True)
    assert flips <= max(3, q_dev.size * 1e-4), flips
    exact = oracle.gemm(q_dev, s_dev, True, pw["codes"], pw["w_scale"])["Y"]
    assert np.array_equal(Y[rows].view(np.uint16), exact.view(np.uint16))
    y_orc = oracle.gemm(ref["codes"], ref["scale"], True, pw["codes"], pw["w_scale"])["Y"]
    check_y_tolerance(Y[rows], y_orc)
