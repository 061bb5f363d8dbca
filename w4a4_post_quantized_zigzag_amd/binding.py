"""Thin ctypes binding of libw4a4.so (include/w4a4.h). Argument marshalling only: shapes and
pointers are taken from torch tensors that live on the GPU, workspaces are torch allocations, and
every call is enqueued on torch's current stream. All arithmetic runs in the library's HIP kernels;
there is no fallback: if the library is missing, ``lib()`` raises."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libw4a4.so")

W4A4_OK, W4A4_ERR_ARG, W4A4_ERR_SHAPE, W4A4_ERR_STEP_RANGE = 0, 1, 2, 3
W4A4_ERR_UNSUPPORTED, W4A4_ERR_ALIGN, W4A4_ERR_WORKSPACE, W4A4_ERR_HIP = 4, 5, 6, 7
W4A4_F16, W4A4_F32 = 0, 1
EPI_NONE, EPI_GELU, EPI_RESIDUAL = 0, 1, 2

_vp, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/w4a4.h
SIGNATURES = {
    "w4a4_zigzag_workspace_bytes": (_sz, [_i]),
    "w4a4_zigzag_perm": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _sz, _vp]),
    "w4a4_block_svd_workspace_bytes": (_sz, [_i, _i, _i]),
    "w4a4_block_svd": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _sz, _vp]),
    "w4a4_calibrate_workspace_bytes": (_sz, [_i, _i, _i]),
    "w4a4_calibrate_act_scale": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "w4a4_rot_bytes": (_sz, [_i, _i]),
    "w4a4_pack_workspace_bytes": (_sz, [_i, _i, _i]),
    "w4a4_pack_weights": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "w4a4_act_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "w4a4_rotate_quant_act": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp,
                                   _vp, _sz, _vp]),
    "w4a4_rotate_quant_act_hadamard": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _i, _i, _vp, _vp,
                                            _vp, _vp]),
    "w4a4_gemm_rq_next_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "w4a4_gemm_rq_next": (_i, [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _vp, _i64, _i, _vp, _i64, _vp,
                               _vp, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "w4a4_noalloc_scratch_bytes": (_sz, []),
    "w4a4_rotate_quant_act_noalloc": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _i, _i, _vp,
                                           _vp, _vp, _vp]),
    "w4a4_gemm_workspace_bytes": (_sz, [_i, _i, _i]),
    "w4a4_gemm": (_i, [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _vp, _i64, _i, _vp, _i64, _vp, _sz, _vp]),
    "w4a4_gemm_i32": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "w4a4_pack_weights_w8": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                  _vp]),
    "w4a4_calibrate_act_scale_a8": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "w4a4_rotate_quant_act_a8": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _i, _i, _vp, _vp,
                                      _vp, _vp, _sz, _vp]),
    "w4a4_gemm_w8a8_workspace_bytes": (_sz, [_i, _i, _i]),
    "w4a4_gemm_w8a8": (_i, [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _vp, _i64, _i, _vp, _i64, _vp, _sz,
                            _vp]),
    "w4a4_gemm_w8a8_i32": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "w4a4_f6_operand_bytes": (_sz, [_i, _i]),
    "w4a4_codes_to_f6": (_i, [_vp, _i, _i, _vp, _vp]),
    "w4a4_act_f6_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "w4a4_rotate_quant_act_f6": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp,
                                      _sz, _vp]),
    "w4a4_gemm_f6_workspace_bytes": (_sz, [_i, _i, _i]),
    "w4a4_gemm_f6": (_i, [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _vp, _i64, _i, _vp, _i64, _vp, _sz,
                          _vp]),
    "w4a4_gemm_f6_i32": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "w4a4_calibrate_act_scale_grouped": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _vp, _sz,
                                              _vp]),
    "w4a4_rotate_quant_act_grouped": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _i, _i, _vp, _vp,
                                           _vp, _vp, _sz, _vp]),
    "w4a4_gemm_grouped": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _i64, _i, _vp, _i64, _vp]),
    "w4a4_gptq_hessian_workspace_bytes": (_sz, [_i, _i, _i]),
    "w4a4_gptq_hessian": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "w4a4_gptq_factor_workspace_bytes": (_sz, [_i]),
    "w4a4_gptq_factor": (_i, [_vp, _i, ctypes.c_double, _vp, _vp, _vp, _sz, _vp]),
    "w4a4_pack_gptq_workspace_bytes": (_sz, [_i, _i, _i]),
    "w4a4_pack_weights_gptq": (_i, [_vp, _i, _i, _i, _i64, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _sz, _vp]),
    "w4a4_last_error": (ctypes.c_char_p, []),
    "w4a4_status_string": (ctypes.c_char_p, [_i]),
    "w4a4_abi_version": (_i, []),
}

_lib = None


class W4A4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib():
    """Load libw4a4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m w4a4_post_quantized_zigzag_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def check(rc: int):
    if rc != W4A4_OK:
        msg = lib().w4a4_last_error().decode()
        raise W4A4Error(rc, msg)


# ---------------------------------------------------------------------------------------------
# torch-facing helpers (device tensors in, device tensors out)
# ---------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return W4A4_F16
    if t.dtype == torch.float32:
        return W4A4_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ws(nbytes: int, device):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _row_stride(t) -> int:
    assert t.dim() == 2 and t.stride(1) == 1, "expected a row-major 2-D tensor"
    return t.stride(0)


def zigzag_perm(W, block: int):
    torch = _torch()
    N, K = W.shape
    perm = torch.empty(K, dtype=torch.int32, device=W.device)
    ws, nb = _ws(lib().w4a4_zigzag_workspace_bytes(K), W.device)
    check(lib().w4a4_zigzag_perm(_p(W), _dtype_code(W), N, K, _row_stride(W), block, _p(perm),
                                 _p(ws), nb, _stream()))
    return perm


def block_svd(W, perm, block: int):
    torch = _torch()
    N, K = W.shape
    U = torch.empty((K // block, block, block), dtype=torch.float32, device=W.device)
    ws, nb = _ws(lib().w4a4_block_svd_workspace_bytes(N, K, block), W.device)
    check(lib().w4a4_block_svd(_p(W), _dtype_code(W), N, K, _row_stride(W), block, _p(perm), _p(U),
                               _p(ws), nb, _stream()))
    return U


def _code_cols(K: int, bits: int) -> int:
    if bits not in (4, 8):
        raise ValueError(f"bits must be 4 or 8, not {bits}")
    return K // 2 if bits == 4 else K


def pack_weights(W, perm, U, block: int, bits: int = 4):
    """Returns (wq uint8 [N, K/2] (int4) or [N, K] (int8), w_scale fp32 [N], rot uint8 [rot_bytes]).
    U None: U_b = I."""
    torch = _torch()
    N, K = W.shape
    wq = torch.empty((N, _code_cols(K, bits)), dtype=torch.uint8, device=W.device)
    w_scale = torch.empty(N, dtype=torch.float32, device=W.device)
    rot = torch.empty(lib().w4a4_rot_bytes(K, block), dtype=torch.uint8, device=W.device)
    ws, nb = _ws(lib().w4a4_pack_workspace_bytes(N, K, block), W.device)
    fn = lib().w4a4_pack_weights if bits == 4 else lib().w4a4_pack_weights_w8
    check(fn(_p(W), _dtype_code(W), N, K, _row_stride(W), block, _p(perm), _p(U), _p(wq),
             _p(w_scale), _p(rot), _p(ws), nb, _stream()))
    return wq, w_scale, rot


def calibrate_act_scale(X, perm, rot, block: int, out=None, ws=None, bits: int = 4):
    """fp32 scale for one (linear, step) entry from stacked calibration activations X [M, K]."""
    torch = _torch()
    M, K = X.shape
    _code_cols(K, bits)
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=X.device)
    if ws is None:
        ws, nb = _ws(lib().w4a4_calibrate_workspace_bytes(M, K, block), X.device)
    else:
        nb = ws.numel()
    fn = lib().w4a4_calibrate_act_scale if bits == 4 else lib().w4a4_calibrate_act_scale_a8
    check(fn(_p(X), _dtype_code(X), M, K, _row_stride(X), block, _p(perm), _p(rot), _p(out), _p(ws),
             nb, _stream()))
    return out


def rotate_quant_act(X, perm, rot, block: int, table=None, num_steps: int = 0, step: int = 0,
                     xq=None, x_scale=None, xrot_dbg=None, ws=None, bits: int = 4):
    torch = _torch()
    M, K = X.shape
    per_token = table is None
    if xq is None:
        xq = torch.empty((M, _code_cols(K, bits)), dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(max(M, 1) if per_token else 1, dtype=torch.float32, device=X.device)
    need = lib().w4a4_act_workspace_bytes(M, K, block, 1 if per_token else 0)
    if ws is None:
        ws, nb = _ws(need, X.device)
    else:
        nb = ws.numel()
    fn = lib().w4a4_rotate_quant_act if bits == 4 else lib().w4a4_rotate_quant_act_a8
    check(fn(_p(X), _dtype_code(X), M, K, _row_stride(X), block, _p(perm), _p(rot), _p(table),
             num_steps, step, _p(xq), _p(x_scale), _p(xrot_dbg), _p(ws), nb, _stream()))
    return xq, x_scale


def rotate_quant_act_noalloc(X, perm, rot, block: int, table=None, num_steps: int = 0,
                             step: int = 0, xq=None, x_scale=None, xrot_dbg=None):
    """rotate_quant_act through the allocation-free entry point (int4 codes; the library's own
    scratch instead of a workspace). xq and x_scale are allocated here only when not given."""
    torch = _torch()
    M, K = X.shape
    per_token = table is None
    if xq is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(max(M, 1) if per_token else 1, dtype=torch.float32, device=X.device)
    check(lib().w4a4_rotate_quant_act_noalloc(_p(X), _dtype_code(X), M, K, _row_stride(X), block,
                                              _p(perm), _p(rot), _p(table), num_steps, step, _p(xq),
                                              _p(x_scale), _p(xrot_dbg), _stream()))
    return xq, x_scale


def rotate_quant_act_hadamard(X, perm, block: int, table=None, num_steps: int = 0, step: int = 0,
                              xq=None, x_scale=None, xrot_dbg=None):
    """Hadamard-only rotation mode (R_b = H_B); per-token scales when table is None."""
    torch = _torch()
    M, K = X.shape
    per_token = table is None
    if xq is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(max(M, 1) if per_token else 1, dtype=torch.float32, device=X.device)
    check(lib().w4a4_rotate_quant_act_hadamard(_p(X), _dtype_code(X), M, K, _row_stride(X), block,
                                               _p(perm), _p(table), num_steps, step, _p(xq),
                                               _p(x_scale), _p(xrot_dbg), _stream()))
    return xq, x_scale


def gemm(xq, x_scale, per_token: bool, wq, w_scale, K: int, Y=None, epilogue: int = EPI_NONE,
         residual=None, ws=None, bits: int = 4):
    """W4A4 GEMM (bits 4, packed int4 operands) or W8A8 GEMM (bits 8, int8 operands)."""
    torch = _torch()
    M, N = xq.shape[0], wq.shape[0]
    _code_cols(K, bits)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=wq.device)
    wsb = lib().w4a4_gemm_workspace_bytes if bits == 4 else lib().w4a4_gemm_w8a8_workspace_bytes
    need = wsb(M, N, K)
    if ws is None:
        ws, nb = _ws(need, wq.device)
    else:
        nb = ws.numel()
    ldr = _row_stride(residual) if residual is not None else 0
    fn = lib().w4a4_gemm if bits == 4 else lib().w4a4_gemm_w8a8
    check(fn(_p(xq), _p(x_scale), 1 if per_token else 0, _p(wq), _p(w_scale), M, N, K, _p(Y),
             _row_stride(Y), epilogue, _p(residual), ldr, _p(ws), nb, _stream()))
    return Y


def gemm_rq_next(xq, x_scale, per_token: bool, wq, w_scale, K: int, col0: int, K_next: int,
                 block_next: int, rot_next, table_next, num_steps: int, step: int, Y=None,
                 epilogue: int = EPI_NONE, residual=None, xq_next=None, x_scale_next=None, ws=None,
                 store_next_cols: bool = True, res_cols=None, res_order=None):
    """W4A4 GEMM, then the next linear's per-step rotate-quantize of Y[:, col0:col0+K_next]
    (fused into the GEMM epilogue where the tile plan allows). store_next_cols=False lets the
    library leave those columns of Y unwritten. K_next = 0: no next linear. res_cols (device int32
    [N]): residual column map, output column n adds residual[:, res_cols[n]]; res_order: optional
    per-tile gather order for it (see w4a4_gemm_rq_next). Returns (Y, xq_next, x_scale_next)."""
    torch = _torch()
    M, N = xq.shape[0], wq.shape[0]
    _code_cols(K, 4)
    dev_ = wq.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=dev_)
    if K_next > 0:
        _code_cols(K_next, 4)
        if xq_next is None:
            xq_next = torch.empty((M, K_next // 2), dtype=torch.uint8, device=dev_)
        if x_scale_next is None:
            x_scale_next = torch.empty(1, dtype=torch.float32, device=dev_)
    L = lib()
    need = L.w4a4_gemm_rq_next_workspace_bytes(M, N, K, K_next, block_next,
                                               0 if res_cols is None else 1)
    if ws is None:
        ws, nb = _ws(need, dev_)
    else:
        nb = ws.numel()
    ldr = _row_stride(residual) if residual is not None else 0
    check(L.w4a4_gemm_rq_next(_p(xq), _p(x_scale), 1 if per_token else 0, _p(wq), _p(w_scale), M, N,
                              K, _p(Y), _row_stride(Y), epilogue, _p(residual), ldr, _p(res_cols),
                              _p(res_order),
                              col0, K_next, block_next, _p(rot_next), _p(table_next), num_steps,
                              step, _p(xq_next), _p(x_scale_next), 1 if store_next_cols else 0,
                              _p(ws), nb, _stream()))
    return Y, xq_next, x_scale_next


def gemm_i32(xq, wq, K: int, bits: int = 4):
    torch = _torch()
    M, N = xq.shape[0], wq.shape[0]
    _code_cols(K, bits)
    acc = torch.empty((M, N), dtype=torch.int32, device=wq.device)
    wsb = lib().w4a4_gemm_workspace_bytes if bits == 4 else lib().w4a4_gemm_w8a8_workspace_bytes
    ws, nb = _ws(wsb(M, N, K), wq.device)
    fn = lib().w4a4_gemm_i32 if bits == 4 else lib().w4a4_gemm_w8a8_i32
    check(fn(_p(xq), _p(wq), M, N, K, _p(acc), _p(ws), nb, _stream()))
    return acc


def codes_to_f6(codes, K: int, out=None):
    """FP6 (E3M2) operand bytes of packed int4 codes [rows][K/2] (flat uint8 tensor)."""
    torch = _torch()
    rows = codes.shape[0]
    nbytes = lib().w4a4_f6_operand_bytes(rows, K)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=codes.device)
    check(lib().w4a4_codes_to_f6(_p(codes), rows, K, _p(out), _stream()))
    return out


def rotate_quant_act_f6(X, perm, rot, block: int, table=None, num_steps: int = 0, step: int = 0,
                        xf=None, x_scale=None, ws=None):
    """Rotate-quantize with the codes written as an FP6 operand (flat uint8) instead of packed int4."""
    torch = _torch()
    M, K = X.shape
    per_token = table is None
    L = lib()
    if xf is None:
        xf = torch.empty(max(L.w4a4_f6_operand_bytes(M, K), 1), dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M if per_token else 1, dtype=torch.float32, device=X.device)
    if ws is None:
        ws, nb = _ws(L.w4a4_act_f6_workspace_bytes(M, K, block, 1 if per_token else 0), X.device)
    else:
        nb = ws.numel()
    check(L.w4a4_rotate_quant_act_f6(_p(X), _dtype_code(X), M, K, _row_stride(X), block, _p(perm),
                                     _p(rot), _p(table), num_steps, step, _p(xf), _p(x_scale),
                                     _p(ws), nb, _stream()))
    return xf, x_scale


def gemm_f6(xf, M: int, x_scale, per_token: bool, wf, N: int, w_scale, K: int, Y=None,
            epilogue: int = EPI_NONE, residual=None, ws=None):
    """The W4A4 GEMM on FP6 operands (``codes_to_f6`` of the activation and weight codes)."""
    torch = _torch()
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=wf.device)
    need = lib().w4a4_gemm_f6_workspace_bytes(M, N, K)
    if ws is None:
        ws, nb = _ws(need, wf.device)
    else:
        nb = ws.numel()
    ldr = _row_stride(residual) if residual is not None else 0
    check(lib().w4a4_gemm_f6(_p(xf), _p(x_scale), 1 if per_token else 0, _p(wf), _p(w_scale), M, N,
                             K, _p(Y), _row_stride(Y), epilogue, _p(residual), ldr, _p(ws), nb,
                             _stream()))
    return Y


def gemm_f6_i32(xf, M: int, wf, N: int, K: int):
    torch = _torch()
    acc = torch.empty((M, N), dtype=torch.int32, device=wf.device)
    ws, nb = _ws(lib().w4a4_gemm_f6_workspace_bytes(M, N, K), wf.device)
    check(lib().w4a4_gemm_f6_i32(_p(xf), _p(wf), M, N, K, _p(acc), _p(ws), nb, _stream()))
    return acc


def calibrate_act_scale_grouped(X, perm, rot, block: int, out=None, ws=None):
    """Group-wise calibration: K / block fp32 scales (one per rotation block) for one step."""
    torch = _torch()
    M, K = X.shape
    if out is None:
        out = torch.empty(K // block, dtype=torch.float32, device=X.device)
    if ws is None:
        ws, nb = _ws(lib().w4a4_calibrate_workspace_bytes(M, K, block), X.device)
    else:
        nb = ws.numel()
    check(lib().w4a4_calibrate_act_scale_grouped(_p(X), _dtype_code(X), M, K, _row_stride(X), block,
                                                 _p(perm), _p(rot), _p(out), _p(ws), nb, _stream()))
    return out


def rotate_quant_act_grouped(X, perm, rot, block: int, table, num_steps: int, step: int, xq=None,
                             x_scale=None, xrot_dbg=None, ws=None):
    """Rotate-quantize with group-wise scales: table [num_steps, K / block]."""
    torch = _torch()
    M, K = X.shape
    if xq is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(K // block, dtype=torch.float32, device=X.device)
    if ws is None:
        ws, nb = _ws(lib().w4a4_act_workspace_bytes(M, K, block, 0), X.device)
    else:
        nb = ws.numel()
    check(lib().w4a4_rotate_quant_act_grouped(_p(X), _dtype_code(X), M, K, _row_stride(X), block,
                                              _p(perm), _p(rot), _p(table), num_steps, step, _p(xq),
                                              _p(x_scale), _p(xrot_dbg), _p(ws), nb, _stream()))
    return xq, x_scale


def gemm_grouped(xq, x_scales, wq, w_scale, K: int, block: int, Y=None, epilogue: int = EPI_NONE,
                 residual=None):
    """W4A4 GEMM with group-wise activation scales x_scales [K / block]."""
    torch = _torch()
    M, N = xq.shape[0], wq.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=wq.device)
    ldr = _row_stride(residual) if residual is not None else 0
    check(lib().w4a4_gemm_grouped(_p(xq), _p(x_scales), _p(wq), _p(w_scale), M, N, K, block, _p(Y),
                                  _row_stride(Y), epilogue, _p(residual), ldr, _stream()))
    return Y


def gptq_hessian(X, perm, U, block: int, H=None, accumulate: bool = False):
    """H (+)= X'^T X' in fp64 [K, K] for the rotated calibration activations X' (GPTQ solver)."""
    torch = _torch()
    M, K = X.shape
    if H is None:
        H = torch.zeros((K, K), dtype=torch.float64, device=X.device)
    ws, nb = _ws(lib().w4a4_gptq_hessian_workspace_bytes(M, K, block), X.device)
    check(lib().w4a4_gptq_hessian(_p(X), _dtype_code(X), M, K, _row_stride(X), block, _p(perm),
                                  _p(U), _p(H), 1 if accumulate else 0, _p(ws), nb, _stream()))
    return H


def gptq_factor(H, damp_percent: float = 0.05):
    """Upper Cholesky factor of the damped inverse Hessian and the dead-channel flags."""
    torch = _torch()
    K = H.shape[0]
    Hf = torch.empty((K, K), dtype=torch.float64, device=H.device)
    dead = torch.empty(K, dtype=torch.uint8, device=H.device)
    ws, nb = _ws(lib().w4a4_gptq_factor_workspace_bytes(K), H.device)
    check(lib().w4a4_gptq_factor(_p(H), K, float(damp_percent), _p(Hf), _p(dead), _p(ws), nb,
                                 _stream()))
    return Hf, dead


def pack_weights_gptq(W, perm, U, block: int, Hf, dead=None):
    """GPTQ-quantized packed int4 weights (same outputs as pack_weights)."""
    torch = _torch()
    N, K = W.shape
    wq = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    w_scale = torch.empty(N, dtype=torch.float32, device=W.device)
    rot = torch.empty(lib().w4a4_rot_bytes(K, block), dtype=torch.uint8, device=W.device)
    ws, nb = _ws(lib().w4a4_pack_gptq_workspace_bytes(N, K, block), W.device)
    check(lib().w4a4_pack_weights_gptq(_p(W), _dtype_code(W), N, K, _row_stride(W), block, _p(perm),
                                       _p(U), _p(Hf), _p(dead), _p(wq), _p(w_scale), _p(rot), _p(ws),
                                       nb, _stream()))
    return wq, w_scale, rot
