"""GPU parity of w4a4_gemm_rq_next: the W4A4 GEMM followed by the next linear's per-step
rotate-quantize of a column range of its output, through the C ABI.

The contract is "w4a4_gemm, then w4a4_rotate_quant_act on Y[:, col0:col0+K_next] with perm = NULL"
(the columns already hold the next linear's input in its zigzag order). So, on every case:
  - Y equals w4a4_gemm's output bit for bit;
  - the codes and the scale equal the standalone rotate-quantize of the device's own Y slice bit for
    bit (the fused epilogue runs the streaming kernel's arithmetic in the same order; the fallback
    runs the standalone call itself), and the standalone call is pinned to the oracle's quantizer by
    the quantize-stage tests;
  - on one shape the codes are also compared with the oracle's fp64 rotate-quantize of that slice
    directly (certified near-tie flips only).
Cases cover the stack shapes that use the fused epilogue (QKV feeding O through its V columns, the
up-projection with GELU feeding down, O and down over all their columns on the split-group tiles),
ragged row counts, shapes that take the fallback (few tokens, block 64, a K split), the empty call
and the argument errors.

Pages: gist.science (pt) "Metodologia" 1 (rotation of each linear's input before quantization) and 2
(per-step scale looked up from the table).
"""
import numpy as np
import pytest

import oracle
from oracle.reference import EPI_GELU, EPI_NONE, EPI_RESIDUAL
from w4a4_post_quantized_zigzag_amd import binding as bd

from parity_util import compare_codes, dev, host, rotation_error_bound

pytestmark = pytest.mark.gpu


def _case(M, N, K, K_next, B, epi, seed):
    torch = __import__("torch")
    rng = np.random.Generator(np.random.PCG64(seed))
    xq = dev(rng.integers(0, 256, (M, K // 2), dtype=np.uint8))
    wq = dev(rng.integers(0, 256, (N, K // 2), dtype=np.uint8))
    xs = dev(np.array([0.02], np.float32))
    ws = dev(rng.uniform(0.5, 1.5, N).astype(np.float32) * np.float32(0.02 / np.sqrt(K)))
    res = dev(rng.standard_normal((M, N)).astype(np.float16)) if epi == EPI_RESIDUAL else None
    Wn = rng.normal(0.0, 0.02, (64, K_next))
    perm_n = oracle.zigzag_perm(Wn, B)
    U_n = oracle.block_svd(Wn, perm_n, B)
    _, _, rot_n = bd.pack_weights(dev(np.zeros((1, K_next), np.float32)), dev(perm_n), dev(U_n), B)
    # per-step scales: the largest per-token scale of the slice at step 0, a quarter of it at step 1
    Y0 = bd.gemm(xq, xs, False, wq, ws, K, epilogue=epi, residual=res)
    return dict(xq=xq, wq=wq, xs=xs, ws=ws, res=res, rot=rot_n, U=U_n, Y0=Y0, torch=torch)


def _table_for(d, col0, K_next, B):
    _, s_tok = bd.rotate_quant_act(d["Y0"][:, col0:col0 + K_next], None, d["rot"], B)
    smax = float(host(s_tok).max())
    return dev(np.array([smax, smax / 4], np.float32))


def _same(a, b):
    return np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8))


CASES = {
    # name: (M, N, K, col0, K_next, block, epilogue)
    "qkv_to_o": (1600, 3072, 1024, 2048, 1024, 128, EPI_NONE),
    "up_to_down_gelu": (1600, 4096, 1024, 0, 4096, 128, EPI_GELU),
    "ragged_residual": (333, 768, 512, 256, 512, 128, EPI_RESIDUAL),
    "rows_130_mid_cols": (130, 512, 256, 128, 256, 128, EPI_NONE),
    "few_tokens_fallback": (50, 1024, 1024, 0, 1024, 128, EPI_GELU),
    "block64_fallback": (300, 512, 512, 0, 512, 64, EPI_NONE),
    "k_split_fallback": (260, 256, 16384, 0, 256, 128, EPI_NONE),
    # the split-group tile kind (64 x 128, two k groups per tile) with the fused epilogue: the
    # stack's O and down shapes over all columns, a ragged row count feeding part of the columns
    # (tiles ordered by row band), and GELU with a long K
    "o_shape_split_group": (1600, 1024, 1024, 0, 1024, 128, EPI_RESIDUAL),
    "down_shape_split_group": (1600, 1024, 4096, 0, 1024, 128, EPI_RESIDUAL),
    "split_group_ragged_part": (700, 512, 2048, 128, 256, 128, EPI_NONE),
    "split_group_gelu": (1000, 1024, 4096, 256, 512, 128, EPI_GELU),
    # the 80-row pipelined tiles (the stack's QKV plan) with a ragged last row band
    "rows_80_tiles_ragged": (1590, 3072, 1024, 2048, 1024, 128, EPI_NONE),
    "rows_80_tiles_residual": (1590, 3072, 1024, 0, 1024, 128, EPI_RESIDUAL),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gemm_rq_next_matches_gemm_then_rotate_quantize(name):
    M, N, K, col0, K_next, B, epi = CASES[name]
    d = _case(M, N, K, K_next, B, epi, 11 + list(CASES).index(name))
    table = _table_for(d, col0, K_next, B)
    torch = d["torch"]
    for step, store in ((0, True), (1, True), (1, False)):
        # store=False: the next linear's columns of Y may be left unwritten (pre-filled here with
        # a stand-in value); the other columns, the codes and the scale are unchanged
        Yb = torch.full(tuple(d["Y0"].shape), -3.0, dtype=torch.float16, device="cuda")
        Y, q, s = bd.gemm_rq_next(d["xq"], d["xs"], False, d["wq"], d["ws"], K, col0, K_next, B,
                                  d["rot"], table, 2, step, Y=Yb, epilogue=epi, residual=d["res"],
                                  store_next_cols=store)
        if store:
            assert _same(Y, d["Y0"]), (name, step)
        else:
            keep = np.ones(d["Y0"].shape[1], bool)
            keep[col0:col0 + K_next] = False
            assert np.array_equal(host(Y)[:, keep].view(np.uint16), host(d["Y0"])[:, keep].view(np.uint16))
        q_ref, s_ref = bd.rotate_quant_act(d["Y0"][:, col0:col0 + K_next], None, d["rot"], B,
                                           table, 2, step)
        assert _same(s, s_ref), (name, step, store)
        qa, qb = host(q), host(q_ref)
        if not np.array_equal(qa, qb):
            bad = np.argwhere(qa != qb)[:5]
            raise AssertionError(f"{name} step {step} store {store}: {int((qa != qb).sum())} code "
                                 f"bytes differ, e.g. {bad.tolist()}")


@pytest.mark.parametrize("mode", ["tiny", "edge"])
def test_gemm_rq_next_scales_near_the_fp32_normal_limit(mode):
    # the fused up-projection tile (GELU, next linear's codes) with its activation scale just
    # below or just above 2^-118 and weight scales near 2^108: the fp16 output and the codes equal
    # those of the plain GEMM followed by the stand-alone rotate-quantize, bit for bit
    M, N, K, K_next, B = 1600, 4096, 1024, 4096, 128
    d = _case(M, N, K, K_next, B, EPI_GELU, 31)
    rng = np.random.Generator(np.random.PCG64(32))
    xs = np.float32(np.ldexp(rng.uniform(1.0, 2.0), -120 if mode == "tiny" else -117))
    ws = (rng.uniform(0.5, 1.0, N) * 2.0 ** 100).astype(np.float32)
    d["xs"], d["ws"] = dev(np.array([xs], np.float32)), dev(ws)
    d["Y0"] = bd.gemm(d["xq"], d["xs"], False, d["wq"], d["ws"], K, epilogue=EPI_GELU)
    assert np.all(np.isfinite(host(d["Y0"]).astype(np.float32)))
    table = _table_for(d, 0, K_next, B)
    Y, q, s = bd.gemm_rq_next(d["xq"], d["xs"], False, d["wq"], d["ws"], K, 0, K_next, B,
                              d["rot"], table, 2, 0, epilogue=EPI_GELU, store_next_cols=True)
    assert _same(Y, d["Y0"])
    q_ref, s_ref = bd.rotate_quant_act(d["Y0"], None, d["rot"], B, table, 2, 0)
    assert _same(s, s_ref) and _same(q, q_ref)


def test_gemm_rq_next_codes_against_the_oracle():
    M, N, K, col0, K_next, B, epi = 200, 1024, 512, 512, 512, 128, EPI_NONE
    d = _case(M, N, K, K_next, B, epi, 7)
    table = _table_for(d, col0, K_next, B)
    Y, q, s = bd.gemm_rq_next(d["xq"], d["xs"], False, d["wq"], d["ws"], K, col0, K_next, B,
                              d["rot"], table, 2, 0)
    Xs = host(Y)[:, col0:col0 + K_next].astype(np.float64)
    ident = np.arange(K_next, dtype=np.int32)
    tab = host(table)
    ref = oracle.rotate_quant_act(Xs, ident, d["U"], B, "per_step", tab, 2, 0)
    assert host(s)[0] == tab[0]
    q_dev = oracle.unpack_int4(host(q), K_next)
    eps = rotation_error_bound(Xs, ident, oracle.rotation(d["U"], B), B)
    flips = compare_codes(q_dev, ref["codes"], ref["v"], ref["x_rot"], eps,
                          np.full(M, host(s)[0]), ref["scale"], False)
    assert flips <= max(3, q_dev.size * 1e-4), flips


def test_gemm_rq_next_empty_and_errors():
    torch = __import__("torch")
    d = _case(130, 512, 256, 256, 128, EPI_NONE, 3)
    table = dev(np.array([0.1, 0.2], np.float32))
    # M = 0: nothing to do, no error
    e = torch.empty((0, 128), dtype=torch.uint8, device="cuda")
    Y0 = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    bd.gemm_rq_next(e, d["xs"], False, d["wq"], d["ws"], 256, 0, 256, 128, d["rot"], table, 2, 0,
                    Y=Y0)
    bad = [
        (dict(col0=384, K_next=256), bd.W4A4_ERR_SHAPE),      # columns past N
        (dict(col0=0, K_next=200), bd.W4A4_ERR_SHAPE),        # not a multiple of the block
        (dict(step=2), bd.W4A4_ERR_STEP_RANGE),               # step outside the table
        (dict(table=None), bd.W4A4_ERR_ARG),                  # per-step scale is required
    ]
    for kw, code in bad:
        args = dict(col0=0, K_next=256, step=0, table=table)
        args.update(kw)
        with pytest.raises(bd.W4A4Error) as ei:
            bd.gemm_rq_next(d["xq"], d["xs"], False, d["wq"], d["ws"], 256, args["col0"],
                            args["K_next"], 128, d["rot"], args["table"], 2, args["step"])
        assert ei.value.status == code, (kw, ei.value)


@pytest.mark.parametrize("per_token_in,ld_pad", [(True, 0), (False, 64), (True, 192)])
def test_gemm_rq_next_per_token_input_and_strided_output(per_token_in, ld_pad):
    # the GEMM's own input scales per token, and Y a view into a wider buffer (ldy = N + ld_pad):
    # the fused epilogue must address Y, the residual and the codes by their own strides
    torch = __import__("torch")
    M, N, K, col0, K_next, B, epi = 400, 768, 512, 256, 512, 128, EPI_RESIDUAL
    d = _case(M, N, K, K_next, B, epi, 41 + ld_pad)
    xs = d["xs"]
    if per_token_in:
        rng = np.random.Generator(np.random.PCG64(7))
        xs = dev(rng.uniform(0.01, 0.03, M).astype(np.float32))
    Y0 = bd.gemm(d["xq"], xs, per_token_in, d["wq"], d["ws"], K, epilogue=epi, residual=d["res"])
    d["Y0"] = Y0
    table = _table_for(d, col0, K_next, B)
    big = torch.full((M, N + ld_pad), 7.0, dtype=torch.float16, device="cuda")
    Yv = big[:, :N]
    Y, q, s = bd.gemm_rq_next(d["xq"], xs, per_token_in, d["wq"], d["ws"], K, col0, K_next, B,
                              d["rot"], table, 2, 1, Y=Yv, epilogue=epi, residual=d["res"])
    assert _same(Yv, Y0)
    if ld_pad:
        assert np.all(host(big[:, N:]).astype(np.float32) == 7.0)  # the padding is untouched
    q_ref, s_ref = bd.rotate_quant_act(Y0[:, col0:col0 + K_next], None, d["rot"], B, table, 2, 1)
    assert _same(q, q_ref) and _same(s, s_ref)


# residual column map: output column n adds residual[:, res_cols[n]]. Expected Y: w4a4_gemm with the
# residual's columns gathered on the host side of the comparison (torch indexing), bit for bit; the
# codes, when a next linear is given, as the standalone rotate-quantize of that Y's columns.
MAP_CASES = {
    # name: (M, N, K, col0, K_next, per_token input scales)
    "o_shape_fused_split_group": (1600, 1024, 1024, 0, 1024, False),   # map read in the epilogue
    "down_shape_last_layer": (1600, 1024, 4096, 0, 0, False),          # no next linear
    "ragged_fused_split_group": (700, 1024, 2048, 0, 1024, False),
    "pipelined_plan": (333, 768, 512, 256, 512, False),     # residual gathered into the workspace
    "few_tokens": (50, 1024, 1024, 0, 0, False),            # small-M kernel, gathered first
    "per_token_calibration": (300, 1024, 1024, 0, 0, True),
    "k_split": (260, 256, 16384, 0, 0, False),               # split-K partials and the gather
    "partial_last_tile": (700, 1000, 2048, 0, 0, False),     # a last tile of 104 columns
}


def _gather_order(cols):
    # each 128-column tile's columns sorted by the residual column they read
    N = len(cols)
    order = np.empty(N, np.int64)
    for t0 in range(0, N, 128):
        seg = cols[t0:t0 + 128]
        order[t0:t0 + len(seg)] = t0 + np.argsort(seg, kind="stable")
    return order


@pytest.mark.parametrize("with_order", [False, True])
@pytest.mark.parametrize("name", list(MAP_CASES))
def test_gemm_residual_column_map(name, with_order):
    torch = __import__("torch")
    M, N, K, col0, K_next, per_tok = MAP_CASES[name]
    B = 128
    idx = list(MAP_CASES).index(name)
    d = _case(M, N, K, K_next or 128, B, EPI_RESIDUAL, 101 + idx)
    rng = np.random.Generator(np.random.PCG64(201 + idx))
    # a permutation, except one case that maps several outputs to the same residual column
    cols = rng.permutation(N) if idx % 2 == 0 else rng.integers(0, N, N)
    rmap = dev(cols.astype(np.int32))
    xs = d["xs"]
    if per_tok:
        xs = dev(rng.uniform(0.01, 0.03, M).astype(np.float32))
    res_g = d["res"][:, torch.from_numpy(cols).cuda()].contiguous()
    Y_ref = bd.gemm(d["xq"], xs, per_tok, d["wq"], d["ws"], K, epilogue=EPI_RESIDUAL, residual=res_g)
    table = dev(np.array([0.05, 0.02], np.float32))
    if K_next:
        table = _table_for(dict(d, Y0=Y_ref), col0, K_next, B)
    # the gather order only changes which lane fetches which column: same results
    rord = dev(_gather_order(cols).astype(np.int32)) if with_order else None
    Y, q, s = bd.gemm_rq_next(d["xq"], xs, per_tok, d["wq"], d["ws"], K, col0, K_next, B, d["rot"],
                              table, 2, 1, epilogue=EPI_RESIDUAL, residual=d["res"], res_cols=rmap,
                              res_order=rord)
    assert _same(Y, Y_ref), name
    if K_next:
        q_ref, s_ref = bd.rotate_quant_act(Y_ref[:, col0:col0 + K_next], None, d["rot"], B, table,
                                           2, 1)
        assert _same(q, q_ref) and _same(s, s_ref), name


def test_gemm_residual_column_map_against_the_oracle():
    # the mapped residual through the oracle's integer GEMM and dequantization, bit for bit
    M, N, K = 200, 512, 512
    d = _case(M, N, K, 128, 128, EPI_RESIDUAL, 5)
    cols = np.random.Generator(np.random.PCG64(6)).permutation(N)
    Y, _, _ = bd.gemm_rq_next(d["xq"], d["xs"], False, d["wq"], d["ws"], K, 0, 0, 128, None, None,
                              1, 0, epilogue=EPI_RESIDUAL, residual=d["res"],
                              res_cols=dev(cols.astype(np.int32)))
    ref = oracle.gemm(oracle.unpack_int4(host(d["xq"]), K), host(d["xs"]), False,
                      oracle.unpack_int4(host(d["wq"]), K), host(d["ws"]), EPI_RESIDUAL,
                      host(d["res"])[:, cols])["Y"]
    assert np.array_equal(host(Y).view(np.uint16), ref.view(np.uint16))


def test_gemm_residual_column_map_errors():
    d = _case(130, 512, 256, 128, 128, EPI_NONE, 3)
    rmap = dev(np.arange(512, dtype=np.int32))
    table = dev(np.array([0.1], np.float32))
    # a map without the residual epilogue; K_next = 0 with col0 != 0
    with pytest.raises(bd.W4A4Error) as ei:
        bd.gemm_rq_next(d["xq"], d["xs"], False, d["wq"], d["ws"], 256, 0, 0, 128, None, None, 1, 0,
                        res_cols=rmap)
    assert ei.value.status == bd.W4A4_ERR_ARG
    with pytest.raises(bd.W4A4Error) as ei:
        bd.gemm_rq_next(d["xq"], d["xs"], False, d["wq"], d["ws"], 256, 128, 0, 128, d["rot"], table,
                        1, 0)
    assert ei.value.status == bd.W4A4_ERR_SHAPE
