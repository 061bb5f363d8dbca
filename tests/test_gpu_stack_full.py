"""GPU parity of the full synthetic action-head stack -- 16 layers x 8 denoising steps at M = 1600
tokens, hidden 1024, ffn 4096, block 128, per-linear per-step tables -- against the CPU oracle,
through the C ABI, in the launch configuration the benchmark times.

Tokens never mix in this stack (attention is the identity and every scale is a per-step scalar),
so the oracle runs on a few sampled rows while the device runs all 1600. Two comparisons:

- teacher-forced, per layer and linear: the oracle takes the device's own fp16 input of each linear
  (and its residual) on the sampled rows. Then (i) the step scale is the table entry bit for bit,
  (ii) the device codes equal the oracle's except for certified near-tie flips (the device rotation
  is within the derived error bound of the fp64 one and the oracle's value lies within that bound of
  a rounding boundary), and (iii) given the device codes, the oracle's integer GEMM and
  dequantization reproduce the device output bit for bit (GELU within one fp16 ulp);
- free-running: the oracle chains its own fp16 outputs and residuals through all 16 layers of every
  step from the same inputs, and every linear's output is compared with the device's at the
  end-to-end fp16 tolerance (max abs <= 1e-2 max|Y|, relative Frobenius <= 2e-3). The two chains are
  flip-synchronized: where the device's code differs from the oracle's at a certified near-tie --
  the oracle's value lies within the rotation's error bound (plus the propagated difference of the
  two chains' inputs, which differ only by the GELU's last-ulp evaluation) of a rounding boundary, so
  both codes are correct -- the oracle continues with the device's code. Without that, one
  legitimate near-tie flip grows through the quantized residual stack (each requantization turns a
  difference far below one quantization step into whole-step code changes with proportional
  probability) until the chains no longer agree within fp16 tolerance: the oracle alone, with its
  rotated values perturbed by 2^-17 relative, shows a single flip at layer 7 growing to a 21%
  relative difference by layer 11. Any other difference (a wrong code, scale, wiring, residual or
  step index) fails the comparison.

The zigzag permutations, SVD factors and act_scale_tables are the oracle's (the tables calibrated
on eight calibration rows per step through the oracle's stack) and are inputs to both sides.

Pages: gist.science (pt) "Metodologia" 1-2 (rotation before quantization; per-step table looked up
at every denoising step); vnrobo.com "Build DiT action head pack" (--num-steps 8, --a-bits 4).
"""
import numpy as np
import pytest

import oracle
from oracle.reference import EPI_GELU, EPI_NONE, EPI_RESIDUAL
from w4a4_post_quantized_zigzag_amd import inputs
from w4a4_post_quantized_zigzag_amd.stack import LINEARS, DeviceStack

from parity_util import (check_y_tolerance, compare_codes, dev, host, propagated_difference,
                         rotation_error_bound)

pytestmark = pytest.mark.gpu
B = 128
ROWS = np.array([0, 555, 1234, 1599])
EPI = {"qkv": EPI_NONE, "o": EPI_RESIDUAL, "up": EPI_GELU, "down": EPI_RESIDUAL}


@pytest.fixture(scope="module")
def stack_run():
    torch = __import__("torch")
    S = inputs.STACK
    W = inputs.stack_weights()
    A = inputs.stack_activations(calib=1)
    layers = oracle.stack_prepare(W, B)
    tables = oracle.stack_calibrate(layers, [[A["X_calib"][t][0][:8]] for t in range(S["steps"])], B)
    calib = [{n: (dev(l[n]["perm"]), dev(l[n]["U"])) for n in LINEARS} for l in layers]
    ds = DeviceStack(W, B, S["steps"], calib=calib)
    ds.set_tables(tables)
    rows_d = torch.from_numpy(ROWS).cuda()
    per_step = []
    for t in range(S["steps"]):
        outs, codes = [], []
        ds.run(dev(A["X_steps"][t]), t, outputs=outs, codes=codes, rows=rows_d)
        per_step.append(([tuple(None if a is None else host(a) for a in o) for o in outs],
                         [(host(q), host(s)) for q, s in codes]))
    return layers, tables, A, per_step


def test_stack_16x8_teacher_forced(stack_run):
    layers, tables, A, per_step = stack_run
    T = len(per_step)
    flips = total = 0
    for t in range(T):
        outs, codes = per_step[t]
        assert len(outs) == len(codes) == 4 * len(layers)
        for i, ((y_dev, x_in, res), (xq_dev, xs_dev)) in enumerate(zip(outs, codes)):
            li, name = divmod(i, 4)
            name = LINEARS[name]
            lin = layers[li][name]
            pw = lin["pack"]
            table = tables[li][name]
            K = pw["codes"].shape[1]
            # (i) the step's scale is the table entry
            assert xs_dev.view(np.uint32)[0] == np.float32(table[t]).view(np.uint32), (t, li, name)
            # (ii) codes: certified near-tie flips only
            act = oracle.rotate_quant_act(x_in, lin["perm"], lin["U"], B, "per_step", table, T, t,
                                          R=pw["R"])
            q_dev = oracle.unpack_int4(xq_dev, K)
            eps = rotation_error_bound(x_in, lin["perm"], pw["R"], B)
            flips += compare_codes(q_dev, act["codes"], act["v"], act["x_rot"], eps,
                                   np.full(len(ROWS), xs_dev[0]), act["scale"], False)
            total += q_dev.size
            # (iii) given the device codes, the integer GEMM and the dequantization are exact
            y = oracle.gemm(q_dev, xs_dev[:1], False, pw["codes"], pw["w_scale"], EPI[name],
                            res)["Y"]
            if EPI[name] == EPI_GELU:
                d = np.abs(y_dev.view(np.int16).astype(np.int32) - y.view(np.int16).astype(np.int32))
                assert d.max() <= 1, (t, li, name)
            else:
                assert np.array_equal(y_dev.view(np.uint16), y.view(np.uint16)), (t, li, name)
    assert flips <= max(3, total * 1e-4), (flips, total)


def test_stack_16x8_free_running(stack_run):
    layers, tables, A, per_step = stack_run
    T = len(per_step)
    h = inputs.STACK["hidden"]
    flips = total = 0
    for t in range(T):
        outs, codes = per_step[t]
        cur = A["X_steps"][t][ROWS].astype(np.float16)
        i = 0

        def lin(name, x_orc, res_orc):
            nonlocal i, flips, total
            L = layers[i // 4][name]
            pw = L["pack"]
            y_dev, x_dev, _ = outs[i]
            xq_dev, xs_dev = codes[i]
            K = pw["codes"].shape[1]
            act = oracle.rotate_quant_act(x_orc, L["perm"], L["U"], B, "per_step",
                                          tables[i // 4][name], T, t, R=pw["R"])
            eps = (rotation_error_bound(x_orc, L["perm"], pw["R"], B)
                   + propagated_difference(x_dev.astype(np.float64) - x_orc.astype(np.float64),
                                           L["perm"], pw["R"], B))
            q_dev = oracle.unpack_int4(xq_dev, K)
            flips += compare_codes(q_dev, act["codes"], act["v"], act["x_rot"], eps,
                                   np.full(len(ROWS), xs_dev[0]), act["scale"], False)
            total += q_dev.size
            # certified: the device codes are a correct choice at every position; continue with them
            y = oracle.gemm(q_dev, act["scale"][:1], False, pw["codes"], pw["w_scale"], EPI[name],
                            res_orc)["Y"]
            check_y_tolerance(y_dev, y)
            i += 1
            return y

        for li in range(len(layers)):
            qkv = lin("qkv", cur, None)
            h2 = lin("o", np.ascontiguousarray(qkv[:, 2 * h:3 * h]), cur)
            g = lin("up", h2, None)
            cur = lin("down", g, h2)
        assert i == len(outs)
    assert flips <= max(3, total * 1e-4), (flips, total)
