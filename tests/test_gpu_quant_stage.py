"""Quantize-stage parity on the device: scale selection, reciprocal, rounding, clamping and packing
must be exactly the oracle's quantizer applied to the device's own rotated activations.

The rotation is a floating-point sum whose order differs between the device (fp16 matrix cores,
fp32 accumulation) and the oracle (fp64), so end-to-end codes are compared with certified near-tie
flips elsewhere. The quantizer that follows is a fixed fp32 recipe (per-step: s = table[step];
per-token: s = fp32(max |x'| / qmax); r = fp32(1/s); q = clamp(rint(fp32(x' r)))). Given the device's
x' (the xrot_dbg test hook holds exactly the fp32 values the kernel quantizes) the codes and scales
have one correct answer, so here they must match bit for bit with no allowance, on every launch path
of the activation side, for int4 and int8 codes, per-step and per-token, and for the group-wise
table. The kernels that write xrot_dbg are separate instantiations of the production kernels, so
each case also runs the production instantiation (no xrot_dbg) and requires the same bytes. FP6
operands (written without xrot_dbg) must decode to the pinned int4 codes.

Pages: gist.science (pt) "Metodologia" item 1 (the rotation is applied before quantization) and
item 2 (per-step scale looked up from the table); vnrobo.com "Build DiT action head pack"
(--a-bits 4); FoldQuantVLA summary key change 2 (dynamic per-token scales) and key change 5
(int8 linears).
"""
import numpy as np
import pytest

import oracle
from w4a4_post_quantized_zigzag_amd import binding as bd

from parity_util import dev, host

pytestmark = pytest.mark.gpu

# tag: (M, K, B, x dtype, permutation, kernel the shape selects)
PATHS = {
    "few_perm_b128": (50, 1024, 128, np.float16, "zigzag", "few-token kernel"),
    "few_perm_b64": (33, 512, 64, np.float16, "zigzag", "few-token kernel"),
    "few_ident_nb3": (256, 384, 128, np.float16, "identity", "few-token kernel"),
    "ring_ident": (600, 8192, 128, np.float16, "identity", "streaming ring"),
    "ring_permuted": (520, 8192, 128, np.float16, "zigzag", "permutation pass + ring"),
    "ring_permuted_b64": (300, 2048, 64, np.float16, "zigzag", "permutation pass + ring"),
    "gather": (300, 1024, 128, np.float16, "zigzag", "register-staged gather"),
    "stack_qkv_shape": (1600, 1024, 128, np.float16, "zigzag", "register-staged gather"),
    "long_k_gather": (260, 131072, 128, np.float16, "zigzag", "register-staged gather"),
    "fp32_valu": (70, 512, 64, np.float32, "zigzag", "fp32 vector kernel"),
    "fp16_b32_valu": (40, 256, 32, np.float16, "zigzag", "fp32 vector kernel"),
}


def _inputs(M, K, B, xdt, perm_kind, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 15.0
    X = X.astype(xdt)
    W = rng.normal(0.0, 0.02, (64, K))
    perm = (oracle.zigzag_perm(W, B) if perm_kind == "zigzag" else np.arange(K, dtype=np.int32))
    U = oracle.block_svd(W, perm, B)
    return X, perm, U


def _rot(perm, U, B, K, bits):
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B, bits=bits)
    return rot


def _codes(xq, K, bits):
    return oracle.unpack_int4(xq, K) if bits == 4 else xq.view(np.int8).astype(np.int8)


def _same_f32(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


def _run(X, perm_d, rot, B, table, step, bits, with_dbg):
    torch = __import__("torch")
    xrot = torch.empty(X.shape, dtype=torch.float32, device="cuda") if with_dbg else None
    tab = dev(table) if table is not None else None
    xq, xs = bd.rotate_quant_act(dev(X), perm_d, rot, B, tab, 0 if table is None else len(table),
                                 step, xrot_dbg=xrot, bits=bits)
    return host(xq), host(xs), (host(xrot) if with_dbg else None)


def _stage_check(X, perm, U, B, mode, bits, table=None, step=0, dev_perm=True):
    K = X.shape[1]
    rot = _rot(perm, U, B, K, bits)
    pd = dev(perm) if dev_perm else None
    q_dbg, s_dbg, xr = _run(X, pd, rot, B, table, step, bits, True)
    q_prod, s_prod, _ = _run(X, pd, rot, B, table, step, bits, False)
    # production and test-hook instantiations agree byte for byte
    assert np.array_equal(q_dbg, q_prod)
    assert _same_f32(s_dbg, s_prod)
    ref = oracle.quantize_act(xr.astype(np.float64), mode, table, None if table is None else len(table),
                              step, bits)
    assert np.array_equal(_codes(q_dbg, K, bits), ref["codes"])
    if mode == "per_token":
        assert _same_f32(s_dbg, ref["scale"])
    else:
        assert _same_f32(s_dbg[:1], ref["scale"][:1])
    return q_prod, s_prod, xr


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("mode", ["per_step", "per_token"])
@pytest.mark.parametrize("tag", list(PATHS))
def test_quantize_stage_exact(tag, mode, bits):
    M, K, B, xdt, perm_kind, _ = PATHS[tag]
    if bits == 8 and K > 65536:
        pytest.skip("int8 activations of this length are not a linear the int8 GEMM takes")
    X, perm, U = _inputs(M, K, B, xdt, perm_kind, seed=len(tag) + 7 * bits)
    if mode == "per_token":
        _stage_check(X, perm, U, B, mode, bits, dev_perm=(perm_kind == "zigzag"))
        return
    # a calibrated entry and a coarse one that clips (codes at both ends of the grid)
    t0 = oracle.calibrate_table([[X]], perm, U, B, bits=bits)[0]
    table = np.array([t0, t0 / 8, np.float32(0.37)], np.float32)
    for step in range(3):
        _stage_check(X, perm, U, B, mode, bits, table, step, dev_perm=(perm_kind == "zigzag"))


@pytest.mark.parametrize("M", [50, 300, 1600])
def test_quantize_stage_grouped(M):
    torch = __import__("torch")
    K, B = 2048, 128
    X, perm, U = _inputs(M, K, B, np.float16, "zigzag", seed=M)
    tg = oracle.calibrate_table_grouped([[X]], perm, U, B)
    table = np.concatenate([tg, tg / 4], axis=0).astype(np.float32)
    rot = _rot(perm, U, B, K, 4)
    for step in range(2):
        xrot = torch.empty(X.shape, dtype=torch.float32, device="cuda")
        xq, xs = bd.rotate_quant_act_grouped(dev(X), dev(perm), rot, B, dev(table), 2, step,
                                             xrot_dbg=xrot)
        xq2, xs2 = bd.rotate_quant_act_grouped(dev(X), dev(perm), rot, B, dev(table), 2, step)
        q, s, xr = host(xq), host(xs), host(xrot)
        assert np.array_equal(q, host(xq2)) and _same_f32(s, host(xs2))
        ref = oracle.quantize_act_grouped(xr.astype(np.float64), B, table, 2, step)
        assert np.array_equal(oracle.unpack_int4(q, K), ref["codes"])
        assert _same_f32(s, ref["scale"])


@pytest.mark.parametrize("mode", ["per_step", "per_token"])
@pytest.mark.parametrize("M,K,perm_kind", [(1600, 1024, "identity"), (600, 2048, "zigzag"),
                                           (50, 1024, "zigzag")])
def test_quantize_stage_fp6_output(M, K, perm_kind, mode):
    """FP6 operands carry the same codes and scales as the pinned int4 output."""
    B = 128
    X, perm, U = _inputs(M, K, B, np.float16, perm_kind, seed=K + M)
    table = None
    if mode == "per_step":
        t0 = oracle.calibrate_table([[X]], perm, U, B)[0]
        table = np.array([t0 / 2], np.float32)
    pd = dev(perm) if perm_kind == "zigzag" else None
    q4, s4, _ = _stage_check(X, perm, U, B, mode, 4, table, 0, dev_perm=(perm_kind == "zigzag"))
    rot = _rot(perm, U, B, K, 4)
    xf, xs = bd.rotate_quant_act_f6(dev(X), pd, rot, B, None if table is None else dev(table),
                                    0 if table is None else 1, 0)
    assert np.array_equal(oracle.f6_codes(host(xf), M, K), oracle.unpack_int4(q4, K))
    assert _same_f32(host(xs), s4)


# ------------------------------------------------------------------ unusable table entries

BAD_ENTRIES = [0.0, -0.5, np.inf, np.nan]


@pytest.mark.parametrize("tag", ["few_perm_b128", "ring_ident", "ring_permuted", "gather",
                                 "fp32_valu"])
@pytest.mark.parametrize("bits", [4, 8])
def test_unusable_table_entry_gives_nan_output(tag, bits):
    """A table entry that is not a positive finite scale: every code 0 and a NaN scale on both
    sides, and every output of the GEMM NaN (the oracle's rule for an uncalibrated or damaged
    table; aiexpert.news: a wrong or truncated table is a failure mode)."""
    M, K, B, xdt, perm_kind, _ = PATHS[tag]
    X, perm, U = _inputs(M, K, B, xdt, perm_kind, seed=3)
    W = np.random.Generator(np.random.PCG64(4)).normal(0, 0.02, (96, K)).astype(np.float32)
    wq, sw, rot = bd.pack_weights(dev(W), dev(perm), dev(U), B, bits=bits)
    good = oracle.calibrate_table([[X]], perm, U, B, bits=bits)[0]
    table = np.array([good] + BAD_ENTRIES, np.float32)
    pd = dev(perm) if perm_kind == "zigzag" else None
    for step in range(1, len(table)):
        xq, xs = bd.rotate_quant_act(dev(X), pd, rot, B, dev(table), len(table), step, bits=bits)
        ref = oracle.rotate_quant_act(X, perm, U, B, "per_step", table, len(table), step, bits=bits)
        assert not ref["codes"].any() and np.isnan(ref["scale"][0])
        assert not host(xq).any()
        assert np.isnan(host(xs)[0])
        Y = host(bd.gemm(xq, xs, False, wq, sw, K, bits=bits))
        assert np.all(np.isnan(Y.astype(np.float32)))


def test_unusable_table_entry_grouped():
    K, B, M = 1024, 128, 64
    X, perm, U = _inputs(M, K, B, np.float16, "zigzag", seed=9)
    rot = _rot(perm, U, B, K, 4)
    table = oracle.calibrate_table_grouped([[X]], perm, U, B)
    table[0, 2] = 0.0
    table[0, 5] = np.nan
    xq, xs = bd.rotate_quant_act_grouped(dev(X), dev(perm), rot, B, dev(table), 1, 0)
    ref = oracle.rotate_quant_act(X, perm, U, B, "per_token")  # rotation only, for the layout
    q = oracle.unpack_int4(host(xq), K)
    refg = oracle.quantize_act_grouped(ref["x_rot"], B, table, 1, 0)
    s = host(xs)
    assert np.isnan(s[2]) and np.isnan(s[5]) and np.all(np.isfinite(np.delete(s, [2, 5])))
    assert np.isnan(refg["scale"][2]) and np.isnan(refg["scale"][5])
    for g in (2, 5):
        assert not q[:, g * B:(g + 1) * B].any() and not refg["codes"][:, g * B:(g + 1) * B].any()


@pytest.mark.parametrize("perm_kind", ["zigzag", "identity"])
@pytest.mark.parametrize("mode", ["per_step", "per_token"])
def test_codes_at_an_unaligned_address(perm_kind, mode):
    # int4 codes may start at any byte: the kernels that stage a tile's codes for 16-byte stores
    # fall back to byte stores there; the bytes must equal those written to an aligned buffer
    torch = __import__("torch")
    M, K, B = 300, 1024, 128
    X, perm, U = _inputs(M, K, B, np.float16, perm_kind, seed=21)
    rot = _rot(perm, U, B, K, 4)
    pd = dev(perm) if perm_kind == "zigzag" else None
    table = None
    if mode == "per_step":
        table = dev(np.array([oracle.calibrate_table([[X]], perm, U, B)[0]], np.float32))
    T = 1 if table is not None else 0
    q_ref, s_ref = bd.rotate_quant_act(dev(X), pd, rot, B, table, T, 0)
    raw = torch.zeros(M * (K // 2) + 16, dtype=torch.uint8, device="cuda")
    q_odd = raw[1:1 + M * (K // 2)].view(M, K // 2)
    assert q_odd.data_ptr() % 16 == 1
    _, s_odd = bd.rotate_quant_act(dev(X), pd, rot, B, table, T, 0, xq=q_odd)
    assert np.array_equal(host(q_odd), host(q_ref))
    assert np.array_equal(host(s_odd).view(np.uint32), host(s_ref).view(np.uint32))
    assert host(raw)[0] == 0 and not host(raw)[1 + M * (K // 2):].any()
