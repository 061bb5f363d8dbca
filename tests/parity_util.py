"""Helpers shared by the GPU parity tests: device transfers, oracle-side calibration caches and the
comparison rules.

Comparison rules (the arithmetic that justifies them is written next to each function):
 - integer and byte results (perm, packed weights, int32 accumulators) must match bit for bit;
 - fp16 outputs computed from identical integer accumulators and scales must match bit for bit;
 - activation codes come from an fp32 rotation evaluated in a different order than the oracle's
   fp64 one, so a code may differ only where the oracle's pre-rounding value lies within the
   rotation's error bound of a rounding boundary (either neighbour is then a correct code);
 - end-to-end fp16 outputs: max abs error <= 1e-2 * max|Y| and relative Frobenius <= 2e-3.
"""
from __future__ import annotations

import functools

import numpy as np

import oracle

U32 = 2.0 ** -24


def torch():
    import torch as _t
    return _t


def dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch().cuda.synchronize()
    return t.detach().cpu().numpy()


@functools.lru_cache(maxsize=16)
def _calib_cached(key):
    W, B = _CALIB_IN[key]
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    return perm, U


_CALIB_IN = {}


def oracle_calibration(tag: str, W: np.ndarray, B: int):
    """Zigzag perm and SVD factor of W computed by the oracle (cached per tag)."""
    _CALIB_IN[tag] = (W, B)
    return _calib_cached(tag)


def rotation_error_bound(X, perm, R, B, mfma_split: bool = True) -> np.ndarray:
    """Per-element bound on |x'_device - x'_exact| for the device's fp32 rotation.

    The device sums B products in fp32 (any order): error <= (B + 2) u sum_i |x_i R_ij| with
    u = 2^-24; the rotation operand itself carries a relative error <= 2^-22 (two-part fp16 split)
    or 2^-24 (fp32 copy). A factor 2 of margin is applied."""
    Xp = np.abs(np.asarray(X, np.float64)[:, np.asarray(perm)])
    M, K = Xp.shape
    A = np.empty((M, K))
    for b in range(K // B):
        A[:, b * B:(b + 1) * B] = Xp[:, b * B:(b + 1) * B] @ np.abs(R[b])
    rel = (B + 2) * U32 + (2.0 ** -22 if mfma_split else U32)
    return 2.0 * rel * A + 2.0 * U32


def propagated_difference(dX, perm, R, B) -> np.ndarray:
    """Bound on how far a difference dX of the inputs moves the rotated values: |dX[:, perm]| . |R_b|
    block by block (exact propagation through the rotation, in absolute value)."""
    Xp = np.abs(np.asarray(dX, np.float64)[:, np.asarray(perm)])
    out = np.empty_like(Xp)
    for b in range(Xp.shape[1] // B):
        out[:, b * B:(b + 1) * B] = Xp[:, b * B:(b + 1) * B] @ np.abs(R[b])
    return out


def compare_codes(q_dev, q_orc, v_orc, x_orc, eps, scale_dev, scale_orc, per_token: bool):
    """Codes agree, or differ by one where the oracle's value v = x32 * r sits within tau of the
    boundary between the two codes. tau covers the rotation error (eps * r) and, per token, the
    relative difference of the two scales. Returns the number of certified flips."""
    q_dev = q_dev.astype(np.int64)
    q_orc = q_orc.astype(np.int64)
    diff = q_dev != q_orc
    if not diff.any():
        return 0
    # scales: one per row (per-step broadcast or per-token), or a 2-D array broadcastable to the
    # codes (one scale per column group)
    s_orc = np.asarray(scale_orc, np.float64)
    s_dev = np.asarray(scale_dev, np.float64)
    s_orc = s_orc if s_orc.ndim == 2 else s_orc.reshape(-1, 1)
    s_dev = s_dev if s_dev.ndim == 2 else s_dev.reshape(-1, 1)
    r = 1.0 / s_orc
    srel = np.abs(s_dev - s_orc) / s_orc + 2.0 ** -22
    tau = eps * r + np.abs(v_orc) * srel + 1e-6
    lo = np.minimum(q_dev, q_orc)
    boundary = lo + 0.5
    near = np.abs(v_orc.astype(np.float64) - boundary) <= tau
    ok = (np.abs(q_dev - q_orc) == 1) & near
    bad = diff & ~ok
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(i), int(q_dev[tuple(i)]), int(q_orc[tuple(i)]), float(v_orc[tuple(i)]),
                   float(tau[tuple(i)] if np.ndim(tau) else tau)) for i in idx]
        raise AssertionError(f"{int(bad.sum())} uncertified code mismatches, e.g. {detail}")
    return int(diff.sum())


def check_y_tolerance(Y_dev, Y_ref):
    Yd = Y_dev.astype(np.float64)
    Yr = Y_ref.astype(np.float64)
    assert np.all(np.isfinite(Yd)) == np.all(np.isfinite(Yr))
    mx = np.max(np.abs(Yr))
    err = np.max(np.abs(Yd - Yr))
    rel = np.linalg.norm(Yd - Yr) / max(np.linalg.norm(Yr), 1e-300)
    assert err <= 1e-2 * mx, (err, mx)
    assert rel <= 2e-3, rel
    return err / mx, rel
