"""GPU parity of the FP6 (E3M2) operand path against the CPU oracle, through the C ABI.

- w4a4_codes_to_f6: operand bytes must equal the oracle's encoding bit for bit (odd and even row
  counts with the zero pad row, one and several 128-k stages).
- w4a4_gemm_f6_i32: the FP6 matrix instructions' fp32 accumulators hold exact integers (every
  partial sum is an integer below 2^24), so they must equal the oracle's int64 sums bit for bit.
  Shapes reach the 128 x 128, 128 x 256 and 256 x 256 tiles with ragged M and N, the split-K
  reduction, one-row and odd-row operands; the largest are compared on sampled outputs; the extremes
  (all -8 against all -8 and +7) run up to K = 2^18, where 64 K = 2^24 is the largest sum.
- w4a4_gemm_f6: the dequantization and epilogues follow the same fp32 sequence as the oracle, so
  fp16 outputs must match bit for bit (GELU within one fp16 ulp, as for the int8 path).
- w4a4_rotate_quant_act_f6: the FP6 operand, decoded with the oracle's decoder, holds the oracle's
  codes except for certified near-tie flips (as for the packed int4 output), the pad row is zero,
  and a whole linear (rotate-quantize into FP6, FP6 GEMM) meets the end-to-end tolerances.
"""
import numpy as np
import pytest

import oracle
from oracle.reference import EPI_GELU, EPI_NONE, EPI_RESIDUAL
from w4a4_post_quantized_zigzag_amd import binding as bd
from w4a4_post_quantized_zigzag_amd import inputs

from parity_util import dev, host

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed=0):
    xq = inputs.random_packed(M, K, seed=3000 + seed + M)
    wq = inputs.random_packed(N, K, seed=4000 + seed + N)
    return xq, wq


def _f6(packed, K):
    return bd.codes_to_f6(dev(packed), K)


@pytest.mark.parametrize("rows,K", [(1, 128), (7, 256), (64, 1024), (301, 384)])
def test_codes_to_f6_bit_exact(rows, K):
    packed = inputs.random_packed(rows, K, seed=rows + K)
    got = host(_f6(packed, K))
    ref = oracle.f6_operand(oracle.unpack_int4(packed, K))
    assert got.size == ref.size == bd.lib().w4a4_f6_operand_bytes(rows, K)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M,N,K", [
    (65, 72, 128),       # 128 x 128 tile, ragged M and N
    (1, 300, 256),       # one row (pad row in the operand)
    (130, 200, 384),
    (1023, 513, 1280),   # odd M and N
    (257, 129, 4096),    # 4 K splits
    (256, 256, 16384),   # 16 K splits
    (1100, 4100, 384),   # 128 x 256 tiles
    (2100, 4100, 256),   # 256 x 256 tiles
])
def test_gemm_f6_i32_bit_exact(M, N, K):
    xq, wq = _operands(M, N, K)
    acc = host(bd.gemm_f6_i32(_f6(xq, K), M, _f6(wq, K), N, K))
    ref = oracle.int_gemm(oracle.unpack_int4(xq, K), oracle.unpack_int4(wq, K))
    assert np.array_equal(acc.astype(np.int64), ref)


@pytest.mark.parametrize("M,N,K", [(1024, 16384, 2048), (1024, 2048, 16384), (1600, 3072, 1024),
                                   (4096, 4096, 4096)])
def test_gemm_f6_i32_full_size_sampled(M, N, K):
    xq, wq = _operands(M, N, K, seed=7)
    acc = host(bd.gemm_f6_i32(_f6(xq, K), M, _f6(wq, K), N, K)).astype(np.int64)
    rng = np.random.Generator(np.random.PCG64(M + N + K))
    mi = np.concatenate([rng.integers(0, M, 1500), [0, M - 1, M - 1, 0]])
    ni = np.concatenate([rng.integers(0, N, 1500), [0, N - 1, 0, N - 1]])
    rows, cols = np.unique(mi), np.unique(ni)
    q = oracle.unpack_int4(xq[rows], K)
    p = oracle.unpack_int4(wq[cols], K)
    ref = oracle.int_gemm_sampled(q, p, np.searchsorted(rows, mi), np.searchsorted(cols, ni))
    assert np.array_equal(acc[mi, ni], ref)


@pytest.mark.parametrize("K", [128, 4096, 1 << 18])
def test_gemm_f6_i32_extremes(K):
    neg = _f6(inputs.constant_packed(70, K, 0x88), K)   # all codes -8
    pos = _f6(inputs.constant_packed(130, K, 0x77), K)  # all codes +7
    negw = _f6(inputs.constant_packed(65, K, 0x88), K)
    a = host(bd.gemm_f6_i32(neg, 70, negw, 65, K))
    assert np.all(a == 64 * K)
    b = host(bd.gemm_f6_i32(neg, 70, pos, 130, K))
    assert np.all(b == -56 * K)


@pytest.mark.parametrize("per_token", [True, False])
@pytest.mark.parametrize("epi", [EPI_NONE, EPI_RESIDUAL, EPI_GELU])
@pytest.mark.parametrize("M,N,K", [(200, 300, 512), (1100, 4100, 384), (2100, 4100, 256),
                                   (257, 129, 4096), (1024, 16384, 2048)])
def test_gemm_f6_dequant_epilogue(per_token, epi, M, N, K):
    xq, wq = _operands(M, N, K, seed=3)
    sx = inputs.random_scales(M if per_token else 1, seed=M, lo=1e-3, hi=5e-2)
    sw = inputs.random_scales(N, seed=N, lo=1e-3, hi=5e-2)
    res = (np.random.Generator(np.random.PCG64(5)).standard_normal((M, N)) * 4).astype(np.float16)
    Y = host(bd.gemm_f6(_f6(xq, K), M, dev(sx), per_token, _f6(wq, K), N, dev(sw), K, epilogue=epi,
                        residual=dev(res) if epi == EPI_RESIDUAL else None))
    if M * N * K > 2 ** 31:
        rows = np.arange(0, M, 97)
        acc = oracle.int_gemm(oracle.unpack_int4(xq[rows], K), oracle.unpack_int4(wq, K))
        ref, _ = oracle.dequant(acc, sx[rows] if per_token else sx, per_token, sw, epi,
                                res[rows] if epi == EPI_RESIDUAL else None)
        Yc = Y[rows]
    else:
        acc = oracle.int_gemm(oracle.unpack_int4(xq, K), oracle.unpack_int4(wq, K))
        ref, _ = oracle.dequant(acc, sx, per_token, sw, epi, res)
        Yc = Y
    got = Yc.view(np.float16)
    if epi == EPI_GELU:
        gi = got.view(np.int16).astype(np.int32)
        ri = ref.view(np.int16).astype(np.int32)
        assert np.max(np.abs(gi - ri)) <= 1
    else:
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def test_gemm_f6_row_stride_and_empty():
    M, N, K = 150, 96, 256
    xq, wq = _operands(M, N, K)
    sx = inputs.random_scales(M, 1)
    sw = inputs.random_scales(N, 2)
    torch = __import__("torch")
    big = torch.zeros((M, 200), dtype=torch.float16, device="cuda")
    Yv = big[:, 50:50 + N]
    bd.gemm_f6(_f6(xq, K), M, dev(sx), True, _f6(wq, K), N, dev(sw), K, Y=Yv)
    acc = oracle.int_gemm(oracle.unpack_int4(xq, K), oracle.unpack_int4(wq, K))
    ref, _ = oracle.dequant(acc, sx, True, sw)
    full = host(big)
    assert np.array_equal(full[:, 50:50 + N].view(np.uint16), ref.view(np.uint16))
    assert not full[:, :50].any() and not full[:, 50 + N:].any()
    empty = bd.gemm_f6(_f6(xq[:0], K), 0, dev(sx[:0]), True, _f6(wq, K), N, dev(sw), K)
    assert tuple(empty.shape) == (0, N)


# ---- rotate-quantize writing the FP6 operand directly

def _act_inputs(M, K, B, perm_kind, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 15.0
    X = X.astype(np.float16)
    W = rng.normal(0.0, 0.02, (64, K))
    perm = (oracle.zigzag_perm(W, B) if perm_kind == "zigzag" else np.arange(K, dtype=np.int32))
    return X, perm, oracle.block_svd(W, perm, B)


# (M, K, mode, permutation): the streaming kernel writing the layout itself (rows already in
# zigzag order, or after the permutation pass; odd M exercises the zero pad row), and the shapes
# that quantize into the workspace and re-encode (few tokens, per-element gather)
F6_ACT = {
    "ring_step_ident_odd": (301, 1024, "per_step", "identity"),
    "ring_token_permuted": (300, 2048, "per_token", "zigzag"),
    "ring_token_permuted_odd": (517, 4096, "per_token", "zigzag"),
    "ring_step_permuted": (513, 8192, "per_step", "zigzag"),
    "few_step": (50, 1024, "per_step", "zigzag"),
    "few_token_odd": (33, 512, "per_token", "zigzag"),
    "gather_step": (300, 1024, "per_step", "zigzag"),
}


@pytest.mark.parametrize("tag", list(F6_ACT))
def test_rotate_quant_act_f6(tag):
    from parity_util import compare_codes, rotation_error_bound
    M, K, mode, perm_kind = F6_ACT[tag]
    B = 128
    X, perm, U = _act_inputs(M, K, B, perm_kind, seed=len(tag) + M)
    R = oracle.rotation(U, B)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B)
    table = None
    if mode == "per_step":
        t0 = oracle.calibrate_table([[X]], perm, U, B)[0]
        table = np.array([t0, t0 / 8], np.float32)
    dperm = dev(perm) if perm_kind == "zigzag" else None
    for step in ([0, 1] if table is not None else [0]):
        xf, xs = bd.rotate_quant_act_f6(dev(X), dperm, rot, B, dev(table) if table is not None else None,
                                        0 if table is None else len(table), step)
        buf = host(xf)
        assert buf.size == bd.lib().w4a4_f6_operand_bytes(M, K)
        q_dev = oracle.f6_codes(buf, M, K)   # raises on a field that is not an int4 code
        if M % 2:
            R2 = M + 1
            stage = buf.reshape(K // 128, R2 * 96)
            assert not stage[:, M * 64:R2 * 64].any()
            assert not stage[:, R2 * 64:].reshape(K // 128, 4, R2, 8)[:, :, M].any()
        ref = oracle.rotate_quant_act(X, perm, U, B, mode, table, None, step, R=R)
        eps = rotation_error_bound(X, perm, R, B)
        s_dev = host(xs)
        if mode == "per_token":
            assert np.all(np.abs(s_dev - ref["scale"]) <= np.max(eps, axis=1) / 7 * 1.01
                          + 2 ** -23 * ref["scale"])
        else:
            assert s_dev[0] == table[step]
        flips = compare_codes(q_dev, ref["codes"], ref["v"], ref["x_rot"], eps,
                              s_dev if mode == "per_token" else np.full(M, s_dev[0]),
                              ref["scale"], mode == "per_token")
        assert flips <= max(3, q_dev.size * 1e-4), flips


def test_f6_linear_end_to_end():
    # rotate-quantize straight into the FP6 operand, FP6 GEMM with the FP6 weights: within the
    # end-to-end tolerances of the oracle's linear
    from parity_util import check_y_tolerance
    M, K, N, B = 600, 2048, 768, 128
    X, perm, _ = _act_inputs(M, K, B, "zigzag", seed=77)
    W = np.random.Generator(np.random.PCG64(78)).normal(0.0, 0.02, (N, K)).astype(np.float16)
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    wq, sw, rot = bd.pack_weights(dev(W), dev(perm), dev(U), B)
    xf, xs = bd.rotate_quant_act_f6(dev(X), dev(perm), rot, B)
    Y = host(bd.gemm_f6(xf, M, xs, True, bd.codes_to_f6(wq, K), N, sw, K))
    ref = oracle.linear(X, W, B, "per_token", perm=perm, U=U)
    check_y_tolerance(Y, ref["Y"])


@pytest.mark.parametrize("M,mode", [(300, "per_step"), (300, "per_token"), (1, "per_token")])
def test_rotate_quant_act_f6_strided_and_single_row(M, mode):
    # rows 4 halves longer than K (no 16-byte tile loads: the element gather and the re-encoding
    # fallback) and a one-token batch; codes against the oracle as above
    from parity_util import compare_codes, rotation_error_bound
    torch = __import__("torch")
    K, B = 512, 128
    X, perm, U = _act_inputs(M, K, B, "zigzag", seed=M + 11)
    R = oracle.rotation(U, B)
    _, _, rot = bd.pack_weights(dev(np.zeros((1, K), np.float32)), dev(perm), dev(U), B)
    wide = np.zeros((M, K + 4), np.float16)
    wide[:, :K] = X
    xd = torch.from_numpy(wide).cuda()[:, :K]
    table = None
    if mode == "per_step":
        table = np.array([oracle.calibrate_table([[X]], perm, U, B)[0]], np.float32)
    xf, xs = bd.rotate_quant_act_f6(xd, dev(perm), rot, B, dev(table) if table is not None else None,
                                    0 if table is None else 1, 0)
    q_dev = oracle.f6_codes(host(xf), M, K)
    ref = oracle.rotate_quant_act(X, perm, U, B, mode, table, None, 0, R=R)
    eps = rotation_error_bound(X, perm, R, B)
    s_dev = host(xs)
    flips = compare_codes(q_dev, ref["codes"], ref["v"], ref["x_rot"], eps,
                          s_dev if mode == "per_token" else np.full(M, s_dev[0]), ref["scale"],
                          mode == "per_token")
    assert flips <= max(3, q_dev.size * 1e-4), flips
