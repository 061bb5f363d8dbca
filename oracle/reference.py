"""Python face of the CPU oracle (TEST INFRASTRUCTURE ONLY; see the package docstring).

The arithmetic lives in ``w4a4_oracle.c`` (plain fp64 loops, built with -ffp-contract=off).
This module adds the steps for which a library routine is the plain definition: the singular
value decomposition (LAPACK through numpy), the stable sort that orders channels, and the IEEE
binary16 rounding of outputs (numpy's round-to-nearest-even conversion).

Sources, cited by page title and section:
 [P1] "Omega-QVLA: Nen VLA W4A4 tren Edge" -- "Y tuong paper: xoay truoc, scale theo step sau"
      (composite rotation, per-step act_scale_table) and "Build DiT action head pack"
      (--use-rtn --w-bits 4 --a-bits 4 --num-steps 8 --duquant-block-size 64 --svd-rank 0).
 [P2] gist.science (pt) "Resumo Tecnico", "Metodologia" 1 (SVD W = U Sigma V^T with R_SVD = U,
      normalized Hadamard H, R = R_SVD . H, block implementation, zigzag permutation by weight column
      norms) and 2 (per-step DiT activation scaling from calibration trajectories).
 [P3] aiexpert.news: a step-count mismatch or a truncated table is a failure mode.
 [P5] FoldQuantVLA summary, key change 2: dynamic per-token activation quantization.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_w4a4_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build() -> str:
    """Compile the oracle's C core (gcc, -O2 -ffp-contract=off, single-threaded)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC",
           "-o", _LIB_PATH, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if (not os.path.exists(_LIB_PATH)
            or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_colnorm2.argtypes = [_dp, _i64, _i64, _dp]
    lib.orc_hadamard.argtypes = [_i64, _dp]
    lib.orc_rotation.argtypes = [_fp, _i64, _i64, _dp]
    lib.orc_rotate_rows.argtypes = [_dp, _i64, _i64, _i64, _i64, _i32p, _dp, _dp]
    lib.orc_weight_rtn.argtypes = [_dp, _i64, _i64, _fp, _i8p]
    lib.orc_act_quant.argtypes = [_dp, _i64, _i64, ctypes.c_int, ctypes.c_float, _fp, _fp, _i8p, _fp]
    lib.orc_weight_rtn_q.argtypes = [_dp, _i64, _i64, ctypes.c_int, _fp, _i8p]
    lib.orc_act_quant_q.argtypes = [_dp, _i64, _i64, ctypes.c_int, ctypes.c_float, ctypes.c_int, _fp,
                                    _fp, _i8p, _fp]
    lib.orc_pack.argtypes = [_i8p, _i64, _i64, _u8p]
    lib.orc_unpack.argtypes = [_u8p, _i64, _i64, _i8p]
    lib.orc_int_gemm.argtypes = [_i8p, _i8p, _i64, _i64, _i64, _i64p]
    lib.orc_int_gemm_sampled.argtypes = [_i8p, _i8p, _i64, _i64, _i64p, _i64p, _i64p]
    lib.orc_dequant.argtypes = [_i64p, _i64, _i64, _fp, ctypes.c_int, _fp, _fp]
    lib.orc_gelu.argtypes = [_fp, _i64, _dp]
    lib.orc_act_quant_grouped.argtypes = [_dp, _i64, _i64, _i64, _fp, _fp, _fp, _i8p]
    lib.orc_int_gemm_grouped.argtypes = [_i8p, _i8p, _i64, _i64, _i64, _i64, _i64p]
    lib.orc_dequant_grouped.argtypes = [_i64p, _i64, _i64, _i64, _fp, _fp, _fp]
    lib.orc_gptq_sweep.argtypes = [_dp, _i64, _i64, _dp, _fp, _dp, _i8p]
    for f in ("orc_colnorm2", "orc_hadamard", "orc_rotation", "orc_rotate_rows", "orc_weight_rtn",
              "orc_act_quant", "orc_pack", "orc_unpack", "orc_int_gemm", "orc_int_gemm_sampled",
              "orc_dequant", "orc_gelu", "orc_weight_rtn_q", "orc_act_quant_q",
              "orc_act_quant_grouped", "orc_int_gemm_grouped", "orc_dequant_grouped",
              "orc_gptq_sweep"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


def _f64(a) -> np.ndarray:
    """Stored fp16/fp32 values widened exactly to fp64."""
    return np.ascontiguousarray(np.asarray(a).astype(np.float64))


def _check_block(K: int, B: int):
    if B < 1 or (B & (B - 1)) != 0:
        raise ValueError(f"block size {B} is not a power of two")
    if K % B != 0:
        raise ValueError(f"K={K} is not a multiple of the block size {B}")


# ----------------------------------------------------------------------------------------------
# Offline side: zigzag permutation, per-block SVD factor, composite rotation
# ----------------------------------------------------------------------------------------------

def colnorm2(W) -> np.ndarray:
    """Squared L2 norm of every input channel (column of W [N, K]), fp64, rows summed in order."""
    W64 = _f64(W)
    N, K = W64.shape
    c2 = np.empty(K, np.float64)
    _load().orc_colnorm2(_ptr(W64, _dp), N, K, _ptr(c2, _dp))
    return c2


def zigzag_perm(W, B: int) -> np.ndarray:
    """Zigzag channel permutation [P2 Metodologia 1, "Implementacao em Blocos"; P4 "Implementation
    par Blocs"]: channels are reordered by weight column norm so that high- and low-norm channels
    are spread evenly over the rotation blocks.

    Reading taken: rank channels by descending norm (stable, ties to the lower index), then deal the
    ranks over the nb = K/B blocks like a boustrophedon: ranks [p*nb, (p+1)*nb) form pass p; in an
    even pass rank p*nb + j goes to block j, in an odd pass to block nb-1-j; inside a block, pass p
    takes position p. Returns perm int32[K] with perm[b*B + p] = original channel index.
    """
    W = np.asarray(W)
    N, K = W.shape
    _check_block(K, B)
    nb = K // B
    c2 = colnorm2(W)
    order = np.argsort(-c2, kind="stable")
    perm = np.empty(K, np.int32)
    for r in range(K):
        pss, j = divmod(r, nb)
        b = j if pss % 2 == 0 else nb - 1 - j
        perm[b * B + pss] = order[r]
    return perm


def block_svd(W, perm, B: int, return_fp64: bool = False):
    """Per-block SVD factor [P2 Metodologia 1, "Rotacao SVD": W = U Sigma V^T, R_SVD = U].

    Reading taken: the rotation acts on input channels, so for each block b the factor is the B x B
    orthogonal matrix of right singular vectors of W_b = W[:, perm[bB:(b+1)B]] (N x B), columns in
    descending singular value, so that the columns of W_b . U_b have norms sigma_i ("each row's energy
    controlled by the singular spectrum" in the [in, out] layout the page writes W in). Each column's
    sign is fixed so that its largest-magnitude entry is positive (first index on ties).
    Returns U fp32 [nb, B, B] with U[b][i][j] = entry (i, j) of U_b; with return_fp64 also the
    unrounded fp64 factors and the singular values [nb, B] (zeros padded when N < B).
    """
    W64 = _f64(W)
    N, K = W64.shape
    _check_block(K, B)
    nb = K // B
    perm = np.asarray(perm, np.int64)
    U64 = np.empty((nb, B, B), np.float64)
    sig = np.zeros((nb, B), np.float64)
    for b in range(nb):
        Wb = W64[:, perm[b * B:(b + 1) * B]]
        # the thin decomposition already holds all B right singular vectors when N >= B; the full
        # one (an N x N left factor) is needed only to complete the basis when N < B
        _, s, Vt = np.linalg.svd(Wb, full_matrices=N < B)
        V = Vt.T.copy()
        idx = np.argmax(np.abs(V), axis=0)
        sgn = np.where(V[idx, np.arange(B)] < 0, -1.0, 1.0)
        V *= sgn[None, :]
        U64[b] = V
        sig[b, :len(s)] = s
    U32 = U64.astype(np.float32)
    if return_fp64:
        return U32, U64, sig
    return U32


def hadamard(B: int) -> np.ndarray:
    """Normalized natural-order Sylvester Hadamard matrix H_B, fp64 [P2 "Rotacao Hadamard"]."""
    if B < 1 or (B & (B - 1)) != 0:
        raise ValueError(f"Hadamard size {B} is not a power of two")
    H = np.empty((B, B), np.float64)
    _load().orc_hadamard(B, _ptr(H, _dp))
    return H


def rotation(U, B: int) -> np.ndarray:
    """Composite rotation R_b = U_b . H_B of every block, fp64 [nb, B, B] [P2: R = R_SVD . H]."""
    U = np.ascontiguousarray(np.asarray(U, np.float32))
    nb = U.shape[0]
    assert U.shape == (nb, B, B)
    K = nb * B
    R = np.empty((nb, B, B), np.float64)
    _load().orc_rotation(_ptr(U, _fp), K, B, _ptr(R, _dp))
    return R


def rotate_rows(A, perm, R, B: int) -> np.ndarray:
    """A[:, perm] . blockdiag(R_b), fp64, for weights or activations (rows independent)."""
    A64 = _f64(A)
    rows, K = A64.shape
    _check_block(K, B)
    perm = np.ascontiguousarray(np.asarray(perm, np.int32))
    R = np.ascontiguousarray(np.asarray(R, np.float64))
    assert perm.shape == (K,) and R.shape == (K // B, B, B)
    Y = np.empty((rows, K), np.float64)
    _load().orc_rotate_rows(_ptr(A64, _dp), rows, K, K, B, _ptr(perm, _i32p), _ptr(R, _dp),
                            _ptr(Y, _dp))
    return Y


BITS_QMAX = {4: 7, 8: 127}  # symmetric grids [-(qmax + 1), qmax]


def _qmax(bits: int) -> int:
    if bits not in BITS_QMAX:
        raise ValueError(f"bits must be 4 or 8, not {bits}")
    return BITS_QMAX[bits]


def weight_rtn(Wr, bits: int = 4) -> tuple[np.ndarray, np.ndarray]:
    """Per-output-channel symmetric RTN of rotated weights: (s_w fp32 [N], codes int8 [N, K]).
    bits 4 is the W4A4 grid; bits 8 the W8A8 grid of the FoldQuantVLA summary (key change 5)."""
    Wr = np.ascontiguousarray(np.asarray(Wr, np.float64))
    N, K = Wr.shape
    s_w = np.empty(N, np.float32)
    p = np.empty((N, K), np.int8)
    if bits == 4:
        _load().orc_weight_rtn(_ptr(Wr, _dp), N, K, _ptr(s_w, _fp), _ptr(p, _i8p))
    else:
        _load().orc_weight_rtn_q(_ptr(Wr, _dp), N, K, _qmax(bits), _ptr(s_w, _fp), _ptr(p, _i8p))
    return s_w, p


def pack_codes(q, bits: int) -> np.ndarray:
    """Device byte layout of codes: int4 nibble pairs (uint8 [rows, K/2]) or int8 bytes
    (uint8 [rows, K], two's complement)."""
    if bits == 4:
        return pack_int4(q)
    _qmax(bits)
    return np.ascontiguousarray(np.asarray(q, np.int8)).view(np.uint8)


def pack_int4(q) -> np.ndarray:
    """Two's-complement nibbles, two per byte, low nibble = even k: uint8 [rows, K/2]."""
    q = np.ascontiguousarray(np.asarray(q, np.int8))
    rows, K = q.shape
    if K % 2:
        raise ValueError("K must be even to pack two int4 codes per byte")
    out = np.empty((rows, K // 2), np.uint8)
    _load().orc_pack(_ptr(q, _i8p), rows, K, _ptr(out, _u8p))
    return out


def unpack_int4(packed, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(np.asarray(packed, np.uint8))
    rows = packed.shape[0]
    q = np.empty((rows, K), np.int8)
    _load().orc_unpack(_ptr(packed, _u8p), rows, K, _ptr(q, _i8p))
    return q


def pack_weights(W, perm, U, B: int, rows=None, bits: int = 4) -> dict:
    """Offline weight rotate + per-channel RTN + pack (optionally only the given output rows).

    W' = W[:, perm] . blockdiag(U_b H_B) in fp64; s_w, codes and packed bytes as in ``weight_rtn``.
    """
    W = np.asarray(W)
    if rows is not None:
        W = W[np.asarray(rows)]
    K = W.shape[1]
    R = rotation(U, B)
    Wr = rotate_rows(W, perm, R, B)
    s_w, p = weight_rtn(Wr, bits)
    return {"w_rot": Wr, "w_scale": s_w, "codes": p, "wq": pack_codes(p, bits), "R": R}


def quantize_act(Xr, mode: str, table=None, num_steps: int | None = None, step: int | None = None,
                 bits: int = 4):
    """Activation quantization (int4, or int8 with bits=8) of rotated activations Xr (fp64 [M, K]).

    mode "per_step": s = table[step]; a step outside [0, num_steps) or a table shorter than
      num_steps is an error, never clamped [P3: a step-count mismatch or truncated table is a
      failure mode]; mode "per_token": s_m from the row absmax.
    Returns dict(x32, v, codes, scale, xq).
    """
    Xr = np.ascontiguousarray(np.asarray(Xr, np.float64))
    M, K = Xr.shape
    if mode == "per_step":
        table = np.asarray(table, np.float32)
        if num_steps is None:
            num_steps = len(table)
        if len(table) < num_steps:
            raise ValueError("act_scale_table is shorter than the number of steps")
        if step is None or not (0 <= step < num_steps):
            raise ValueError(f"step {step} outside [0, {num_steps})")
        s = float(table[step])
        imode, ts = 0, s
    elif mode == "per_token":
        imode, ts = 1, 1.0
    else:
        raise ValueError(mode)
    x32 = np.empty((M, K), np.float32)
    v = np.empty((M, K), np.float32)
    q = np.empty((M, K), np.int8)
    sc = np.empty(M, np.float32)
    if bits == 4:
        _load().orc_act_quant(_ptr(Xr, _dp), M, K, imode, ts, _ptr(x32, _fp), _ptr(v, _fp),
                              _ptr(q, _i8p), _ptr(sc, _fp))
    else:
        _load().orc_act_quant_q(_ptr(Xr, _dp), M, K, imode, ts, _qmax(bits), _ptr(x32, _fp),
                                _ptr(v, _fp), _ptr(q, _i8p), _ptr(sc, _fp))
    if mode == "per_step" and not _usable_scale(ts):
        # an entry that is not a positive finite number is no scale: no code is produced (all 0)
        # and the NaN scale carries into every dequantized output
        v[:] = 0.0
        q[:] = 0
        sc[:] = np.float32(np.nan)
    xq = pack_codes(q, bits) if (bits == 8 or K % 2 == 0) else None
    return {"x32": x32, "v": v, "codes": q, "scale": sc, "xq": xq}


def _usable_scale(s) -> bool:
    """A table entry is a scale only if it is a positive finite fp32 number."""
    s = np.float32(s)
    return bool(s > 0 and np.isfinite(s))


def rotate_quant_act(X, perm, U, B: int, mode: str, table=None, num_steps=None, step=None, R=None,
                     bits: int = 4):
    """Runtime activation path: zigzag gather, block rotation, scale, quantize (int4 or int8), pack."""
    if R is None:
        R = rotation(U, B)
    Xr = rotate_rows(X, perm, R, B)
    out = quantize_act(Xr, mode, table, num_steps, step, bits)
    out["x_rot"] = Xr
    return out


def int_gemm(q, p) -> np.ndarray:
    """acc = q . p^T in int64 (q [M, K], p [N, K] int8 codes)."""
    q = np.ascontiguousarray(np.asarray(q, np.int8))
    p = np.ascontiguousarray(np.asarray(p, np.int8))
    M, K = q.shape
    N = p.shape[0]
    assert p.shape[1] == K
    acc = np.empty((M, N), np.int64)
    _load().orc_int_gemm(_ptr(q, _i8p), _ptr(p, _i8p), M, N, K, _ptr(acc, _i64p))
    return acc


def int_gemm_sampled(q, p, mi, ni) -> np.ndarray:
    q = np.ascontiguousarray(np.asarray(q, np.int8))
    p = np.ascontiguousarray(np.asarray(p, np.int8))
    mi = np.ascontiguousarray(np.asarray(mi, np.int64))
    ni = np.ascontiguousarray(np.asarray(ni, np.int64))
    K = q.shape[1]
    acc = np.empty(len(mi), np.int64)
    _load().orc_int_gemm_sampled(_ptr(q, _i8p), _ptr(p, _i8p), K, len(mi), _ptr(mi, _i64p),
                                 _ptr(ni, _i64p), _ptr(acc, _i64p))
    return acc


EPI_NONE, EPI_GELU, EPI_RESIDUAL = 0, 1, 2


def dequant(acc, x_scale, per_token: bool, w_scale, epilogue: int = EPI_NONE, residual=None):
    """Y = fp16_rne(fp32(fp32(acc * s_x) * s_w[n])), then the optional epilogue:
    EPI_GELU: fp16(erf-GELU computed in fp64 of the fp32 dequantized value);
    EPI_RESIDUAL: fp16(fp32(dequant) + fp32(residual)). Returns (Y fp16, y32 fp32 dequant)."""
    acc = np.ascontiguousarray(np.asarray(acc, np.int64))
    M, N = acc.shape
    if np.any(np.abs(acc) >= 2 ** 31):
        raise OverflowError("accumulator leaves int32")
    sx = np.ascontiguousarray(np.asarray(x_scale, np.float32).reshape(-1))
    sw = np.ascontiguousarray(np.asarray(w_scale, np.float32))
    y32 = np.empty((M, N), np.float32)
    _load().orc_dequant(_ptr(acc, _i64p), M, N, _ptr(sx, _fp), 1 if per_token else 0,
                        _ptr(sw, _fp), _ptr(y32, _fp))
    return _epilogue(y32, epilogue, residual), y32


def _epilogue(y32, epilogue, residual):
    """fp16 output of the fp32 dequantized values, after the optional GELU or residual add."""
    M, N = y32.shape
    if epilogue == EPI_NONE:
        Y = y32.astype(np.float16)
    elif epilogue == EPI_GELU:
        g = np.empty((M, N), np.float64)
        _load().orc_gelu(_ptr(y32, _fp), M * N, _ptr(g, _dp))
        Y = g.astype(np.float16)
    elif epilogue == EPI_RESIDUAL:
        Y = (y32 + np.asarray(residual, np.float16).astype(np.float32)).astype(np.float16)
    else:
        raise ValueError(epilogue)
    return Y


def gemm(xq_codes, x_scale, per_token, w_codes, w_scale, epilogue=EPI_NONE, residual=None):
    """Integer GEMM of int4 codes followed by dequantization (codes given unpacked, int8)."""
    acc = int_gemm(xq_codes, w_codes)
    Y, y32 = dequant(acc, x_scale, per_token, w_scale, epilogue, residual)
    return {"acc": acc, "Y": Y, "y32": y32}


def calibrate_table(X_samples_per_step, perm, U, B: int, R=None, bits: int = 4) -> np.ndarray:
    """Per-step act_scale_table from calibration trajectories [P1 "Y tuong paper"; P2 item 2
    "Calibracao por Passo"]. Reading taken: one scale per (linear, step), the absmax statistic over
    every calibration sample, token and channel of the rotated activation, stored as a scale:
    table[t] = fp32(max |fp32(x')| / 7) (1.0f when the max is 0), with 127 in place of 7 for int8
    activations. X_samples_per_step[t] is a list of [M, K] arrays for step t."""
    qmax = float(_qmax(bits))
    if R is None:
        R = rotation(U, B)
    T = len(X_samples_per_step)
    table = np.empty(T, np.float32)
    for t in range(T):
        amax = np.float32(0.0)
        for Xs in X_samples_per_step[t]:
            x32 = rotate_rows(Xs, perm, R, B).astype(np.float32)
            amax = max(amax, np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0))
        table[t] = np.float32(float(amax) / qmax) if amax > 0 else np.float32(1.0)
    return table


# ----------------------------------------------------------------------------------------------
# Group-wise (per rotation block) per-step activation scales: the integer-GEMM form of the pages'
# per-channel act_scale_table [P1 "Y tuong paper": the table is per layer, per step, per channel;
# P2 item 2 "Calibracao por Passo"]. One scale per (linear, step, rotation block): the integer GEMM
# keeps one int32 partial per block and folds it in with that block's scale.
# ----------------------------------------------------------------------------------------------

def quantize_act_grouped(Xr, B: int, table, num_steps=None, step=None) -> dict:
    """Int4 quantization of rotated activations Xr (fp64 [M, K]) with the scales of row `step` of a
    [num_steps, K/B] table: position k uses s = table[step][k // B]. Same step-range rules as the
    per-step mode. Returns dict(x32, v, codes, scale (the K/B scales used), xq)."""
    Xr = np.ascontiguousarray(np.asarray(Xr, np.float64))
    M, K = Xr.shape
    _check_block(K, B)
    table = np.asarray(table, np.float32)
    if table.ndim != 2 or table.shape[1] != K // B:
        raise ValueError("grouped act_scale_table must be [num_steps, K / block]")
    if num_steps is None:
        num_steps = table.shape[0]
    if table.shape[0] < num_steps:
        raise ValueError("act_scale_table is shorter than the number of steps")
    if step is None or not (0 <= step < num_steps):
        raise ValueError(f"step {step} outside [0, {num_steps})")
    sg = np.ascontiguousarray(table[step])
    bad = ~((sg > 0) & np.isfinite(sg))
    x32 = np.empty((M, K), np.float32)
    v = np.empty((M, K), np.float32)
    q = np.empty((M, K), np.int8)
    _load().orc_act_quant_grouped(_ptr(Xr, _dp), M, K, B, _ptr(np.where(bad, np.float32(1), sg), _fp),
                                  _ptr(x32, _fp), _ptr(v, _fp), _ptr(q, _i8p))
    if bad.any():
        # blocks whose entry is no scale (see quantize_act): codes 0 and a NaN scale
        for g in np.nonzero(bad)[0]:
            v[:, g * B:(g + 1) * B] = 0.0
            q[:, g * B:(g + 1) * B] = 0
        sg = np.where(bad, np.float32(np.nan), sg).astype(np.float32)
    xq = pack_int4(q) if K % 2 == 0 else None
    return {"x32": x32, "v": v, "codes": q, "scale": sg.copy(), "xq": xq}


def int_gemm_grouped(q, p, B: int) -> np.ndarray:
    """acc[g] = q[:, block g] . p[:, block g]^T in int64 ([K/B, M, N])."""
    q = np.ascontiguousarray(np.asarray(q, np.int8))
    p = np.ascontiguousarray(np.asarray(p, np.int8))
    M, K = q.shape
    N = p.shape[0]
    assert p.shape[1] == K and K % B == 0
    acc = np.empty((K // B, M, N), np.int64)
    _load().orc_int_gemm_grouped(_ptr(q, _i8p), _ptr(p, _i8p), M, N, K, B, _ptr(acc, _i64p))
    return acc


def dequant_grouped(acc_g, x_scales, w_scale, epilogue: int = EPI_NONE, residual=None):
    """y = fma chain over blocks in order (y = fmaf(acc_g, s_g, y) from y = 0), then
    fp32(y * s_w[n]), then the epilogue as in dequant. Returns (Y fp16, y32)."""
    acc_g = np.ascontiguousarray(np.asarray(acc_g, np.int64))
    nb, M, N = acc_g.shape
    if np.any(np.abs(acc_g.sum(axis=0)) >= 2 ** 31):
        raise OverflowError("accumulator leaves int32")
    sg = np.ascontiguousarray(np.asarray(x_scales, np.float32).reshape(-1))
    assert sg.shape[0] == nb
    sw = np.ascontiguousarray(np.asarray(w_scale, np.float32))
    y32 = np.empty((M, N), np.float32)
    _load().orc_dequant_grouped(_ptr(acc_g, _i64p), nb, M, N, _ptr(sg, _fp), _ptr(sw, _fp),
                                _ptr(y32, _fp))
    return _epilogue(y32, epilogue, residual), y32


def gemm_grouped(xq_codes, x_scales, w_codes, w_scale, B: int, epilogue=EPI_NONE, residual=None):
    """Group-wise integer GEMM (int4 codes given unpacked) and dequantization."""
    acc_g = int_gemm_grouped(xq_codes, w_codes, B)
    Y, y32 = dequant_grouped(acc_g, x_scales, w_scale, epilogue, residual)
    return {"acc_g": acc_g, "acc": acc_g.sum(axis=0), "Y": Y, "y32": y32}


def calibrate_table_grouped(X_samples_per_step, perm, U, B: int, R=None) -> np.ndarray:
    """[T, K/B] table: table[t][g] = fp32(max |fp32(x')| over every calibration sample and token of
    step t and the channels of rotation block g, / 7) (1.0f for a zero max), the per-step
    statistic of calibrate_table taken per block."""
    if R is None:
        R = rotation(U, B)
    T = len(X_samples_per_step)
    K = np.asarray(X_samples_per_step[0][0]).shape[1]
    nb = K // B
    table = np.empty((T, nb), np.float32)
    for t in range(T):
        amax = np.zeros(nb, np.float32)
        for Xs in X_samples_per_step[t]:
            x32 = rotate_rows(Xs, perm, R, B).astype(np.float32)
            if x32.size:
                amax = np.maximum(amax, np.abs(x32).reshape(-1, nb, B).max(axis=(0, 2)))
        for g in range(nb):
            table[t, g] = np.float32(float(amax[g]) / 7.0) if amax[g] > 0 else np.float32(1.0)
    return table


# ----------------------------------------------------------------------------------------------
# GPTQ weight solver on calibration activations [vnrobo "Kien truc thuc thi": the backbone pack is
# "SVD-Hadamard rotation + GPTQ pack"; "Build LLM pack": --gptq-block-size 128
# --gptq-damp-percent 0.05]. The plain sequential form of the column sweep; the 128-column lazy
# batches of the flag only reorder the same updates.
# ----------------------------------------------------------------------------------------------

GPTQ_DAMP = 0.05


def gptq_hessian(X_samples, perm, U, B: int, R=None) -> np.ndarray:
    """H = sum over the calibration samples of X'^T X' (fp64 [K, K]), X' = X[:, perm] . R the
    rotated activations the linear quantizes."""
    if R is None:
        R = rotation(U, B)
    H = None
    for Xs in X_samples:
        Xr = rotate_rows(Xs, perm, R, B)
        H = Xr.T @ Xr if H is None else H + Xr.T @ Xr
    return H


def gptq_factor(H, damp_percent: float = GPTQ_DAMP):
    """Upper Cholesky factor Hf of the damped inverse Hessian (Hf^T Hf = (H + d I)^-1, d =
    damp_percent * mean(diag H)), after giving dead channels (zero diagonal) a unit diagonal.
    Returns (Hf, dead)."""
    H = np.array(H, np.float64, copy=True)
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    H[np.diag_indices_from(H)] += damp_percent * float(np.mean(np.diag(H)))
    L = np.linalg.cholesky(np.linalg.inv(H))
    return np.ascontiguousarray(L.T), dead


def gptq_pack(W, perm, U, B: int, Hf, dead=None) -> dict:
    """GPTQ int4 codes of the rotated weights: per-row scales are the RTN scales of W' (fixed before
    the sweep), dead input channels are zeroed, then every row runs the sequential sweep with Hf.
    Same outputs as pack_weights (codes, packed wq, w_scale, R)."""
    R = rotation(U, B)
    Wr = rotate_rows(W, perm, R, B)
    s_w, _ = weight_rtn(Wr)
    Ws = np.array(Wr, copy=True)
    if dead is not None:
        Ws[:, np.asarray(dead, bool)] = 0.0
    Ws = np.ascontiguousarray(Ws)
    N, K = Ws.shape
    Hf = np.ascontiguousarray(np.asarray(Hf, np.float64))
    assert Hf.shape == (K, K)
    q = np.empty((N, K), np.int8)
    row = np.empty(K, np.float64)
    _load().orc_gptq_sweep(_ptr(Ws, _dp), N, K, _ptr(Hf, _dp), _ptr(s_w, _fp), _ptr(row, _dp),
                           _ptr(q, _i8p))
    return {"w_rot": Wr, "w_scale": s_w, "codes": q, "wq": pack_int4(q), "R": R}


def linear(X, W, B: int, mode: str, table=None, num_steps=None, step=None, perm=None, U=None,
           epilogue=EPI_NONE, residual=None, bits: int = 4) -> dict:
    """The whole quantized linear on the CPU (W4A4, or W8A8 with bits=8): offline (perm, U, pack)
    then runtime (rotate-quant, GEMM). mode "per_block" takes a [num_steps, K/B] table of
    group-wise scales (int4 only)."""
    if perm is None:
        perm = zigzag_perm(W, B)
    if U is None:
        U = block_svd(W, perm, B)
    pw = pack_weights(W, perm, U, B, bits=bits)
    if mode == "per_block":
        if bits != 4:
            raise ValueError("group-wise scales are defined for int4 activations")
        Xr = rotate_rows(X, perm, pw["R"], B)
        act = quantize_act_grouped(Xr, B, table, num_steps, step)
        act["x_rot"] = Xr
        g = gemm_grouped(act["codes"], act["scale"], pw["codes"], pw["w_scale"], B, epilogue,
                         residual)
        return {"perm": perm, "U": U, "pack": pw, "act": act, **g}
    act = rotate_quant_act(X, perm, U, B, mode, table, num_steps, step, R=pw["R"], bits=bits)
    g = gemm(act["codes"], act["scale"], mode == "per_token", pw["codes"], pw["w_scale"],
             epilogue, residual)
    return {"perm": perm, "U": U, "pack": pw, "act": act, **g}


# ----------------------------------------------------------------------------------------------
# Synthetic action-head stack (benchmark workload): per layer QKV -> V slice (attention replaced by
# identity) -> O + residual -> up -> erf-GELU -> down + residual, every linear W4A4. Composed only
# of the functions above; tokens never mix, so any subset of rows can be run on its own.
# ----------------------------------------------------------------------------------------------

STACK_LINEARS = ("qkv", "o", "up", "down")


def stack_prepare(weights, B: int, calib=None, w8=()):
    """Offline side for every linear: zigzag perm, SVD factor (or the given ones) and the pack.
    Linears named in w8 (e.g. ("o", "down"), the FoldQuantVLA summary's W8A8 attention-output and
    FFN-down projections) use the int8 grid, the others int4."""
    layers = []
    for li, lw in enumerate(weights):
        layer = {}
        for name in STACK_LINEARS:
            W = lw[name]
            if calib is None:
                perm = zigzag_perm(W, B)
                U = block_svd(W, perm, B)
            else:
                perm, U = calib[li][name]
            bits = 8 if name in w8 else 4
            layer[name] = {"perm": perm, "U": U, "bits": bits,
                           "pack": pack_weights(W, perm, U, B, bits=bits)}
        layers.append(layer)
    return layers


def _stack_linear(lin, X, B, mode, table, steps, step, epilogue=EPI_NONE, residual=None):
    act = rotate_quant_act(X, lin["perm"], lin["U"], B, mode, table, steps, step,
                           R=lin["pack"]["R"], bits=lin.get("bits", 4))
    g = gemm(act["codes"], act["scale"], mode == "per_token", lin["pack"]["codes"],
             lin["pack"]["w_scale"], epilogue, residual)
    return g["Y"], act


def stack_run(layers, X, B: int, mode: str, tables=None, steps=None, step=0, outputs=None,
              record_tables=None):
    """One pass of the stack on fp16 X [rows, h]. mode "per_step" uses tables[layer][name][step];
    mode "per_token" quantizes per token, and with record_tables (a list of per-layer dicts) stores
    each linear's calibration entry fp32(max |fp32(x')| / 7) (1.0 for a zero max; 127 in place of 7
    for an int8 linear) for `step`. Returns the fp16 output; appends each linear's fp16 output to
    `outputs` if given."""
    h = X.shape[1]
    cur = np.asarray(X, np.float16)
    for li, layer in enumerate(layers):
        def lin(name, inp, epi=EPI_NONE, res=None):
            tab = None if mode == "per_token" else tables[li][name]
            Y, act = _stack_linear(layer[name], inp, B, mode, tab, steps, step, epi, res)
            if record_tables is not None:
                amax = float(np.max(np.abs(act["x32"]))) if act["x32"].size else 0.0
                qmax = float(_qmax(layer[name].get("bits", 4)))
                record_tables[li][name][step] = np.float32(amax / qmax) if amax > 0 else 1.0
            if outputs is not None:
                outputs.append(Y)
            return Y

        qkv = lin("qkv", cur)
        h2 = lin("o", np.ascontiguousarray(qkv[:, 2 * h:3 * h]), EPI_RESIDUAL, cur)
        g = lin("up", h2, EPI_GELU)
        cur = lin("down", g, EPI_RESIDUAL, h2)
    return cur


def stack_calibrate(layers, X_calib_per_step, B: int):
    """Per-linear per-step act_scale_tables: for each step, the stacked calibration draws go through
    the stack in per-token mode and every linear records the scale of its rotated input."""
    T = len(X_calib_per_step)
    tables = [{name: np.ones(T, np.float32) for name in STACK_LINEARS} for _ in layers]
    for t, draws in enumerate(X_calib_per_step):
        X = np.concatenate(draws, axis=0)
        stack_run(layers, X, B, "per_token", steps=T, step=t, record_tables=tables)
    return tables


# ------------------------------------------------------------------ FP6 matrix-core operands
#
# Not a step of the pages' method: an exact re-encoding of the int4 codes for the GEMM's FP6 matrix
# instructions. The OCP Microscaling E3M2 six-bit float (sign bit 5, exponent bits 4..2 with bias 3,
# mantissa bits 1..0; value (-1)^s 2^(e-3) (1 + m/4) for e >= 1 and (-1)^s 2^-2 (m/4) for e = 0)
# holds every integer in [-8, 7], so a product of two encoded codes is the exact integer product.
#
# Operand layout of a [rows][K] code matrix (K % 128 == 0, R2 = rows rounded up to even; row R2-1
# is all zeros when rows is odd): k is cut into stages of 128 and each stage into four groups of
# 32 consecutive k. A group's 32 codes, as 6-bit fields with code i at bits 6i..6i+5 of a 192-bit
# little-endian string, are split into a 16-byte head (bits 0..127) and an 8-byte tail (bits
# 128..191). Stage s occupies the R2*96 bytes from s*R2*96: first the heads, at row*64 + 16*group,
# then the tails, at R2*64 + (group*R2 + row)*8. Total R2*K*3/4 bytes.

def e3m2_value(code: int) -> float:
    """Value of a 6-bit E3M2 code, from the format's definition."""
    code = int(code)
    if not 0 <= code < 64:
        raise ValueError("E3M2 codes are 6 bits")
    s, e, m = (code >> 5) & 1, (code >> 2) & 7, code & 3
    mag = 2.0 ** (e - 3) * (1.0 + m / 4.0) if e else 2.0 ** -2 * (m / 4.0)
    return -mag if s else mag


def e3m2_encode(q: int) -> int:
    """The E3M2 code of the integer q in [-8, 7]: the code whose value is q (+0 for 0)."""
    q = int(q)
    if not -8 <= q <= 7:
        raise ValueError("int4 codes lie in [-8, 7]")
    if q == 0:
        return 0
    hits = [c for c in range(64) if e3m2_value(c) == q]
    assert len(hits) == 1
    return hits[0]


def f6_bytes(rows: int, K: int) -> int:
    return ((rows + 1) // 2 * 2) * K * 3 // 4


def _f6_split(buf, rows: int, K: int):
    """Views of an FP6 operand buffer: heads [stage][row][group][16], tails [stage][group][row][8]."""
    R2 = (rows + 1) // 2 * 2
    stage = buf.reshape(K // 128, R2 * 96)
    return (stage[:, :R2 * 64].reshape(K // 128, R2, 4, 16),
            stage[:, R2 * 64:].reshape(K // 128, 4, R2, 8))


def f6_operand(q) -> np.ndarray:
    """FP6 operand bytes (uint8 [f6_bytes(rows, K)]) of int4 codes q [rows, K] (int8 values)."""
    q = np.asarray(q, np.int64)
    rows, K = q.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    lut = np.array([e3m2_encode(v) for v in range(-8, 8)], np.uint8)
    codes = lut[q + 8].reshape(rows, K // 128, 4, 32)           # [row][stage][group][field]
    bits = ((codes[..., None] >> np.arange(6)) & 1).astype(np.uint8)  # field i -> bits 6i..6i+5
    raw = np.packbits(bits.reshape(rows, K // 128, 4, 192), axis=-1, bitorder="little")
    out = np.zeros(f6_bytes(rows, K), np.uint8)
    head, tail = _f6_split(out, rows, K)
    head[:, :rows] = raw[..., :16].transpose(1, 0, 2, 3)
    tail[:, :, :rows] = raw[..., 16:].transpose(1, 2, 0, 3)
    return out


def f6_codes(buf, rows: int, K: int) -> np.ndarray:
    """Inverse of ``f6_operand``: the int4 codes [rows, K] held by an FP6 operand buffer."""
    buf = np.asarray(buf, np.uint8)
    if buf.size != f6_bytes(rows, K):
        raise ValueError("buffer size does not match rows and K")
    head, tail = _f6_split(buf, rows, K)
    raw = np.concatenate([head[:, :rows].transpose(1, 0, 2, 3),
                          tail[:, :, :rows].transpose(2, 0, 1, 3)], axis=-1)  # [row][stage][group][24]
    bits = np.unpackbits(raw, axis=-1, bitorder="little").reshape(rows, K // 128, 4, 32, 6)
    fields = (bits.astype(np.int64) << np.arange(6)).sum(axis=-1)
    value = np.array([e3m2_value(c) for c in range(64)])
    v = value[fields]
    if not np.all((v == np.round(v)) & (v >= -8) & (v <= 7)):
        raise ValueError("not an int4 code")
    return v.reshape(rows, K).astype(np.int8)
