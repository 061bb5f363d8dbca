"""Host-side checks of the C ABI (no GPU): the library loads, exports every function that
include/w4a4.h declares, and rejects bad arguments on the host before anything is launched.

The rejected calls below pass fake, never-dereferenced device addresses: validation returns before
any HIP call, so these run without a GPU. The step-range rule follows the aiexpert.news page (a step
count mismatch or truncated act_scale_table is a failure mode, so the library reports it instead of
clamping the step).
"""
import ctypes
import os
import re

import pytest

from w4a4_post_quantized_zigzag_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a4.h")

FAKE = ctypes.c_void_p(0x10000)      # 256-byte aligned stand-in address
FAKE_ODD = ctypes.c_void_p(0x10004)  # 4-byte aligned only
NULL = None


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return bd.lib()


def test_every_declared_function_is_exported_and_bound(L):
    names = header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n
        assert n in bd.SIGNATURES, f"{n} missing from the binding"
    assert set(bd.SIGNATURES) == set(names)


def test_status_strings_and_version(L):
    assert L.w4a4_abi_version() == 1
    assert L.w4a4_status_string(3) == b"W4A4_ERR_STEP_RANGE"
    assert L.w4a4_status_string(99) == b"W4A4_ERR_UNKNOWN"


def _rq(L, *, M=16, K=256, ldx=256, block=64, dt=bd.W4A4_F16, X=FAKE, rot=FAKE, table=FAKE,
        steps=8, step=0, ws=NULL, wsb=0):
    return L.w4a4_rotate_quant_act(X, dt, M, K, ldx, block, FAKE, rot, table, steps, step, FAKE,
                                   FAKE, NULL, ws, wsb, NULL)


@pytest.mark.parametrize("step,steps", [(8, 8), (-1, 8), (100, 8), (0, 0)])
def test_step_outside_table_is_an_error(L, step, steps):
    assert _rq(L, step=step, steps=steps) == bd.W4A4_ERR_STEP_RANGE
    assert b"step" in L.w4a4_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(block=3), bd.W4A4_ERR_UNSUPPORTED),
    (dict(block=512), bd.W4A4_ERR_UNSUPPORTED),
    (dict(block=0), bd.W4A4_ERR_UNSUPPORTED),
    (dict(K=250, ldx=250, block=1 << 1), bd.W4A4_ERR_SHAPE),   # fine for block 2 ...
    (dict(K=255, ldx=255, block=1), bd.W4A4_ERR_SHAPE),        # odd K
    (dict(K=192, ldx=192, block=128), bd.W4A4_ERR_SHAPE),      # K not a multiple of the block
    (dict(ldx=100), bd.W4A4_ERR_SHAPE),
    (dict(X=NULL), bd.W4A4_ERR_ARG),
    (dict(M=-1), bd.W4A4_ERR_ARG),
    (dict(dt=7), bd.W4A4_ERR_ARG),
    (dict(rot=FAKE_ODD), bd.W4A4_ERR_ALIGN),
    (dict(rot=NULL), bd.W4A4_ERR_ARG),
    (dict(table=NULL), bd.W4A4_ERR_WORKSPACE),                 # per-token needs a workspace
])
def test_rotate_quant_rejects(L, kw, code):
    if kw.get("K") == 250:
        # K=250 is even and a multiple of block 2, so it is accepted; use M=0 to stay on the host
        assert _rq(L, M=0, **kw) == bd.W4A4_OK
        return
    assert _rq(L, **kw) == code
    assert L.w4a4_last_error() != b""


def _rqh(L, *, M=16, K=256, ldx=256, block=64, dt=bd.W4A4_F16, X=FAKE, table=FAKE, steps=8,
         step=0, xq=FAKE):
    return L.w4a4_rotate_quant_act_hadamard(X, dt, M, K, ldx, block, FAKE, table, steps, step, xq,
                                            FAKE, NULL, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(block=32), bd.W4A4_ERR_UNSUPPORTED),            # the butterfly kernel takes 64 or 128
    (dict(block=256, K=512, ldx=512), bd.W4A4_ERR_UNSUPPORTED),
    (dict(K=1 << 17, ldx=1 << 17), bd.W4A4_ERR_UNSUPPORTED),  # row longer than the LDS stage
    (dict(K=1 << 16, ldx=1 << 16, dt=bd.W4A4_F32), bd.W4A4_ERR_UNSUPPORTED),
    (dict(step=8), bd.W4A4_ERR_STEP_RANGE),
    (dict(steps=0), bd.W4A4_ERR_STEP_RANGE),
    (dict(xq=ctypes.c_void_p(0x10004)), bd.W4A4_ERR_ALIGN),
    (dict(xq=NULL), bd.W4A4_ERR_ARG),
    (dict(K=192, ldx=192, block=128), bd.W4A4_ERR_SHAPE),
    (dict(ldx=100), bd.W4A4_ERR_SHAPE),
])
def test_rotate_quant_hadamard_rejects(L, kw, code):
    assert _rqh(L, **kw) == code
    assert L.w4a4_last_error() != b""


def test_hadamard_empty_batch_and_limits(L):
    assert _rqh(L, M=0) == bd.W4A4_OK
    assert _rqh(L, M=0, table=NULL) == bd.W4A4_OK
    assert _rqh(L, M=0, K=1 << 16, ldx=1 << 16) == bd.W4A4_OK            # 128 KB fp16 row
    assert _rqh(L, M=0, K=1 << 15, ldx=1 << 15, dt=bd.W4A4_F32) == bd.W4A4_OK


def test_empty_batch_is_a_valid_call(L):
    assert _rq(L, M=0) == bd.W4A4_OK
    assert _rq(L, M=0, table=NULL) == bd.W4A4_OK
    assert L.w4a4_gemm(NULL, NULL, 0, FAKE, FAKE, 0, 64, 256, NULL, 64, 0, NULL, 0, NULL, 0,
                       NULL) == bd.W4A4_OK
    assert L.w4a4_gemm_i32(NULL, FAKE, 0, 64, 256, NULL, NULL, 0, NULL) == bd.W4A4_OK


def _gemm(L, *, M=16, N=64, K=256, ldy=64, epi=0, res=NULL, ldr=0, Y=FAKE, ws=NULL, wsb=0):
    return L.w4a4_gemm(FAKE, FAKE, 1, FAKE, FAKE, M, N, K, Y, ldy, epi, res, ldr, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(epi=5), bd.W4A4_ERR_ARG),
    (dict(epi=2), bd.W4A4_ERR_ARG),                 # residual epilogue without residual
    (dict(epi=2, res=FAKE, ldr=10), bd.W4A4_ERR_SHAPE),
    (dict(ldy=10), bd.W4A4_ERR_SHAPE),
    (dict(K=255), bd.W4A4_ERR_SHAPE),
    (dict(N=0), bd.W4A4_ERR_ARG),
    (dict(Y=NULL), bd.W4A4_ERR_ARG),
    (dict(Y=ctypes.c_void_p(0x10001)), bd.W4A4_ERR_ALIGN),
    (dict(K=1 << 25), bd.W4A4_ERR_UNSUPPORTED),
])
def test_gemm_rejects(L, kw, code):
    assert _gemm(L, **kw) == code


def test_gemm_split_k_workspace_is_required(L):
    need = L.w4a4_gemm_workspace_bytes(1024, 2048, 16384)
    assert need > 0
    assert _gemm(L, M=1024, N=2048, K=16384, ldy=2048) == bd.W4A4_ERR_WORKSPACE
    assert _gemm(L, M=1024, N=2048, K=16384, ldy=2048, ws=FAKE, wsb=need - 1) == bd.W4A4_ERR_WORKSPACE


@pytest.mark.parametrize("M,K", [(130, (1 << 20) + 128), (130, 1 << 21), (65, 1 << 24)])
def test_gemm_beyond_one_int32_split_plans_k_pieces(L, M, K):
    # more than 2^16 k per tile accumulator: the plan cuts K into pieces of at most 2^16 k, whose
    # exact int32 partials need a workspace of at least ceil(K / 2^16) partial tiles
    need = L.w4a4_gemm_workspace_bytes(M, 64, K)
    assert need >= -(-K // (1 << 16)) * M * 64 * 4
    assert _gemm(L, M=M, N=64, K=K, ldy=64) == bd.W4A4_ERR_WORKSPACE


def test_pack_and_calibration_reject(L):
    ws = L.w4a4_pack_workspace_bytes(256, 256, 64)
    assert ws >= 256 * 64 * 8
    assert L.w4a4_pack_weights(FAKE, 0, 256, 256, 256, 64, FAKE, FAKE, FAKE, FAKE, FAKE_ODD, FAKE,
                               ws, NULL) == bd.W4A4_ERR_ALIGN
    # U may be NULL (U_b = I), the outputs may not
    assert L.w4a4_pack_weights(FAKE, 0, 256, 256, 256, 64, FAKE, NULL, NULL, FAKE, FAKE, FAKE, ws,
                               NULL) == bd.W4A4_ERR_ARG
    assert L.w4a4_pack_weights(FAKE, 0, 256, 256, 256, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               ws - 8, NULL) == bd.W4A4_ERR_WORKSPACE
    assert L.w4a4_block_svd(FAKE, 0, 64, 512, 512, 256, FAKE, FAKE, FAKE, 1 << 30,
                            NULL) == bd.W4A4_ERR_UNSUPPORTED
    assert L.w4a4_zigzag_perm(FAKE, 0, 0, 256, 256, 64, FAKE, FAKE, 1 << 20, NULL) == bd.W4A4_ERR_ARG
    assert L.w4a4_calibrate_act_scale(FAKE, 0, 16, 256, 256, 64, FAKE, FAKE, NULL, FAKE, 256,
                                      NULL) == bd.W4A4_ERR_ARG


def test_workspace_and_operand_sizes(L):
    # the rotation operand holds an fp32 copy and a two-part fp16 split of every R_b
    assert L.w4a4_rot_bytes(1024, 128) >= 1024 * 128 * (4 + 2 + 2)
    assert L.w4a4_rot_bytes(1000, 128) == 0
    assert L.w4a4_act_workspace_bytes(1024, 2048, 128, 0) == 0
    assert L.w4a4_act_workspace_bytes(1024, 2048, 128, 1) >= 4 * 1024
    assert L.w4a4_block_svd_workspace_bytes(4096, 1024, 128) >= 1024 * 128 * 8 * 3
    assert L.w4a4_zigzag_workspace_bytes(16384) >= 16384 * 8


# ---- group-wise scales: host-side validation (nothing is launched on these paths)

def _rqg(L, *, M=16, K=256, ldx=256, block=128, dt=bd.W4A4_F16, table=FAKE, steps=8, step=3,
         xq=FAKE, ws=NULL, wsb=0):
    return L.w4a4_rotate_quant_act_grouped(FAKE, dt, M, K, ldx, block, FAKE, FAKE, table, steps,
                                           step, xq, FAKE, NULL, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(block=64), bd.W4A4_ERR_UNSUPPORTED),           # GEMM folds one 128-k block per stage
    (dict(dt=bd.W4A4_F32), bd.W4A4_ERR_UNSUPPORTED),
    (dict(step=8), bd.W4A4_ERR_STEP_RANGE),
    (dict(step=-1), bd.W4A4_ERR_STEP_RANGE),
    (dict(steps=0), bd.W4A4_ERR_STEP_RANGE),
    (dict(table=NULL), bd.W4A4_ERR_ARG),                  # no per-token form of group-wise scales
    (dict(xq=NULL), bd.W4A4_ERR_ARG),
    (dict(K=192, ldx=192), bd.W4A4_ERR_SHAPE),
])
def test_rotate_quant_grouped_rejects(L, kw, code):
    assert _rqg(L, **kw) == code
    assert L.w4a4_last_error() != b""


def _gg(L, *, M=16, N=64, K=256, block=128, xq=FAKE, wq=FAKE, epi=0, res=NULL, ldr=0, ldy=64):
    return L.w4a4_gemm_grouped(xq, FAKE, wq, FAKE, M, N, K, block, FAKE, ldy, epi, res, ldr, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(block=64), bd.W4A4_ERR_UNSUPPORTED),
    (dict(K=320), bd.W4A4_ERR_SHAPE),
    (dict(xq=ctypes.c_void_p(0x10008)), bd.W4A4_ERR_ALIGN),
    (dict(wq=ctypes.c_void_p(0x10004)), bd.W4A4_ERR_ALIGN),
    (dict(ldy=32), bd.W4A4_ERR_SHAPE),
    (dict(epi=2), bd.W4A4_ERR_ARG),                       # residual epilogue without residual
    (dict(epi=7), bd.W4A4_ERR_ARG),
    (dict(N=0), bd.W4A4_ERR_ARG),
])
def test_gemm_grouped_rejects(L, kw, code):
    assert _gg(L, **kw) == code


def test_grouped_empty_batch_and_calibration_checks(L):
    assert _rqg(L, M=0) == bd.W4A4_OK
    assert _gg(L, M=0, xq=NULL) == bd.W4A4_OK
    assert L.w4a4_calibrate_act_scale_grouped(FAKE, bd.W4A4_F16, 16, 256, 256, 64, FAKE, FAKE, FAKE,
                                              NULL, 0, NULL) == bd.W4A4_ERR_UNSUPPORTED
    assert L.w4a4_calibrate_act_scale_grouped(FAKE, bd.W4A4_F16, 16, 256, 256, 128, FAKE, FAKE, NULL,
                                              NULL, 0, NULL) == bd.W4A4_ERR_ARG
    # the calibration workspace holds one maximum per rotation block even for few rows
    assert L.w4a4_calibrate_workspace_bytes(2, 128 * 512, 128) >= 512 * 4


# ---- GPTQ solver: host-side validation

def test_gptq_rejects(L):
    # K above the solver's limit, bad damping, missing buffers, short workspace
    assert L.w4a4_gptq_factor(FAKE, 8192, ctypes.c_double(0.05), FAKE, NULL, FAKE, 1 << 30,
                              NULL) == bd.W4A4_ERR_UNSUPPORTED
    assert L.w4a4_gptq_factor(FAKE, 256, ctypes.c_double(-1.0), FAKE, NULL, FAKE, 1 << 30,
                              NULL) == bd.W4A4_ERR_ARG
    assert L.w4a4_gptq_factor(NULL, 256, ctypes.c_double(0.05), FAKE, NULL, FAKE, 1 << 30,
                              NULL) == bd.W4A4_ERR_ARG
    assert L.w4a4_gptq_factor(FAKE, 256, ctypes.c_double(0.05), FAKE, NULL, FAKE, 16,
                              NULL) == bd.W4A4_ERR_WORKSPACE
    assert L.w4a4_gptq_hessian(FAKE, bd.W4A4_F16, 16, 8192, 8192, 128, FAKE, FAKE, FAKE, 0, FAKE,
                               1 << 30, NULL) == bd.W4A4_ERR_UNSUPPORTED
    assert L.w4a4_gptq_hessian(FAKE, bd.W4A4_F16, 16, 256, 256, 128, FAKE, FAKE, NULL, 0, FAKE,
                               1 << 30, NULL) == bd.W4A4_ERR_ARG
    assert L.w4a4_pack_weights_gptq(FAKE, bd.W4A4_F16, 16, 256, 256, 128, FAKE, FAKE, NULL, NULL,
                                    FAKE, FAKE, FAKE, FAKE, 1 << 30, NULL) == bd.W4A4_ERR_ARG
    assert L.w4a4_pack_weights_gptq(FAKE, bd.W4A4_F16, 16, 256, 256, 128, FAKE, FAKE, FAKE, NULL,
                                    FAKE, FAKE, FAKE, FAKE, 64, NULL) == bd.W4A4_ERR_WORKSPACE
    assert L.w4a4_pack_gptq_workspace_bytes(16, 256, 128) >= 16 * 256 * 9


# ---- FP6 operands: host-side validation (nothing is launched on these paths)

def _gemm_f6(L, *, M=256, N=256, K=256, xf=FAKE, wf=FAKE, ws=NULL, wsb=0):
    return L.w4a4_gemm_f6(xf, FAKE, 1, wf, FAKE, M, N, K, FAKE, N, 0, NULL, 0, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(K=192), bd.W4A4_ERR_SHAPE),                     # K not a multiple of 128
    (dict(K=(1 << 18) + 128), bd.W4A4_ERR_UNSUPPORTED),   # 64 K above 2^24
    (dict(xf=ctypes.c_void_p(0x10008)), bd.W4A4_ERR_ALIGN),
    (dict(wf=NULL), bd.W4A4_ERR_ARG),
    (dict(N=0), bd.W4A4_ERR_ARG),
])
def test_gemm_f6_rejects(L, kw, code):
    assert _gemm_f6(L, **kw) == code


def test_codes_to_f6_rejects_and_sizes(L):
    assert L.w4a4_f6_operand_bytes(3, 256) == 4 * 256 * 3 // 4   # rows rounded up to even
    assert L.w4a4_f6_operand_bytes(4, 256) == 4 * 256 * 3 // 4
    assert L.w4a4_f6_operand_bytes(4, 200) == 0
    assert L.w4a4_codes_to_f6(FAKE, 4, 192, FAKE, NULL) == bd.W4A4_ERR_SHAPE
    assert L.w4a4_codes_to_f6(FAKE_ODD, 4, 256, FAKE, NULL) == bd.W4A4_ERR_ALIGN
    assert L.w4a4_codes_to_f6(FAKE, 4, 256, NULL, NULL) == bd.W4A4_ERR_ARG
    assert L.w4a4_codes_to_f6(FAKE, -1, 256, FAKE, NULL) == bd.W4A4_ERR_ARG
    assert L.w4a4_codes_to_f6(FAKE, 0, 256, FAKE, NULL) == bd.W4A4_OK  # empty: nothing launched
    need = L.w4a4_gemm_f6_workspace_bytes(256, 256, 16384)
    assert need >= 2 * 256 * 256 * 4   # split K
    assert _gemm_f6(L, K=16384) == bd.W4A4_ERR_WORKSPACE


def test_rotate_quant_act_f6_rejects(L):
    def call(block=128, K=256, xf=FAKE, ws=FAKE, wsb=1 << 30):
        return L.w4a4_rotate_quant_act_f6(FAKE, bd.W4A4_F16, 300, K, K, block, FAKE, FAKE, NULL, 0, 0,
                                          xf, FAKE, ws, wsb, NULL)
    assert call(block=64) == bd.W4A4_ERR_UNSUPPORTED
    assert call(xf=ctypes.c_void_p(0x10008)) == bd.W4A4_ERR_ALIGN
    assert call(xf=NULL) == bd.W4A4_ERR_ARG
    assert call(wsb=16) == bd.W4A4_ERR_WORKSPACE
    assert L.w4a4_act_f6_workspace_bytes(300, 256, 128, 1) >= 300 * 128 + L.w4a4_act_workspace_bytes(300, 256, 128, 1)
    assert L.w4a4_act_f6_workspace_bytes(300, 256, 64, 1) == 0


def test_f6_empty_batches_are_valid(L):
    assert L.w4a4_rotate_quant_act_f6(FAKE, bd.W4A4_F16, 0, 256, 256, 128, FAKE, FAKE, NULL, 0, 0,
                                      NULL, NULL, NULL, 0, NULL) == bd.W4A4_OK
    assert L.w4a4_gemm_f6(NULL, NULL, 1, FAKE, FAKE, 0, 64, 256, NULL, 64, 0, NULL, 0, NULL, 0,
                          NULL) == bd.W4A4_OK


def _rqn(L, *, M=16, N=256, K=256, epi=2, res=FAKE, ldr=256, rmap=NULL, rord=NULL, col0=0, kn=128,
         block=128, rot=FAKE, table=FAKE, steps=2, step=0, xqn=FAKE, xsn=FAKE, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = L.w4a4_gemm_rq_next_workspace_bytes(M, N, K, kn, block, 0 if rmap is None else 1)
    return L.w4a4_gemm_rq_next(FAKE, FAKE, 0, FAKE, FAKE, M, N, K, FAKE, N, epi, res, ldr, rmap,
                               rord, col0, kn, block, rot, table, steps, step, xqn, xsn, 1, ws, wsb,
                               NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(epi=0, res=NULL, rmap=FAKE), bd.W4A4_ERR_ARG),         # a map needs the residual epilogue
    (dict(rmap=ctypes.c_void_p(0x10002)), bd.W4A4_ERR_ALIGN),    # int32 map, 4-byte aligned
    (dict(rord=FAKE), bd.W4A4_ERR_ARG),                          # a gather order needs a map
    (dict(rmap=FAKE, rord=ctypes.c_void_p(0x10002)), bd.W4A4_ERR_ALIGN),
    (dict(N=70000, ldr=70000, kn=0, rmap=FAKE), bd.W4A4_ERR_UNSUPPORTED),
    (dict(kn=0, col0=128), bd.W4A4_ERR_SHAPE),                   # no next linear: col0 must be 0
    (dict(kn=-128), bd.W4A4_ERR_SHAPE),
    (dict(col0=192, kn=128), bd.W4A4_ERR_SHAPE),                 # past N
    (dict(kn=200), bd.W4A4_ERR_SHAPE),                           # not a multiple of the block
    (dict(table=NULL), bd.W4A4_ERR_ARG),                         # per-step scale required
    (dict(step=2), bd.W4A4_ERR_STEP_RANGE),
    (dict(xqn=NULL), bd.W4A4_ERR_ARG),
    (dict(M=1024, N=2048, K=16384, ldr=2048, ws=NULL), bd.W4A4_ERR_WORKSPACE),  # split-K plan
])
def test_gemm_rq_next_rejects(L, kw, code):
    assert _rqn(L, **kw) == code


def test_gemm_rq_next_without_next_linear_ignores_its_arguments(L):
    # K_next = 0: the rotate-quantize arguments may be NULL; only the GEMM's are checked (here an
    # empty batch, which launches nothing)
    assert _rqn(L, M=0, kn=0, rot=NULL, table=NULL, xqn=NULL, xsn=NULL, rmap=FAKE) == bd.W4A4_OK


def test_gemm_rq_next_workspace_covers_the_mapped_residual(L):
    # a residual map needs room for the gathered residual (M x N fp16) beyond the GEMM's own
    # workspace, for the tile plans that gather it before the GEMM
    M, N, K = 333, 768, 512
    plain = L.w4a4_gemm_rq_next_workspace_bytes(M, N, K, 0, 128, 0)
    mapped = L.w4a4_gemm_rq_next_workspace_bytes(M, N, K, 0, 128, 1)
    assert mapped >= plain + M * N * 2
    assert L.w4a4_gemm_rq_next_workspace_bytes(0, N, K, 0, 128, 1) == 0
