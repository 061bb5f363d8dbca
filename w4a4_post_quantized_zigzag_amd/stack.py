"""Synthetic action-head stack driven through the C ABI: per layer QKV -> V slice (attention
replaced by identity) -> O with residual -> up with erf-GELU -> down with residual, every linear a
W4A4 linear (or, for the linears named in w8, a W8A8 linear: the FoldQuantVLA summary's mixed
configuration keeps the attention-output and FFN-down projections at W8A8) with its own zigzag
permutation, block SVD factor, packed weights and per-step act_scale_table. This module only
sequences library calls and owns buffers; all arithmetic runs in libw4a4.so.

Per-step tables follow the pages' per-step scaling (vnrobo "Y tuong paper": the runtime looks up the
current denoising step's scale; gist.science item 2: tables from calibration trajectories): for each
step, the stack is run in per-token mode over that step's stacked calibration draws, and each
linear's table entry is the scale of its rotated input on the way.
"""
from __future__ import annotations

import numpy as np

from . import binding as bd

LINEARS = ("qkv", "o", "up", "down")


def _torch():
    import torch
    return torch


class DeviceLinear:
    """One linear's device state. row_perm (optional, device int64 [N]) reorders the output
    channels: the packed weights hold rows W[row_perm], so output column j is channel row_perm[j].
    The zigzag permutation and block SVD are computed on W itself (the row order of W does not
    change them); only the packed rows move."""

    def __init__(self, W, block: int, steps: int, perm=None, U=None, bits: int = 4, row_perm=None):
        torch = _torch()
        Wd = W if isinstance(W, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(W)).cuda()
        self.N, self.K = Wd.shape
        self.B = block
        self.perm = bd.zigzag_perm(Wd, block) if perm is None else perm
        self.U = bd.block_svd(Wd, self.perm, block) if U is None else U
        self.bits = bits
        Wp = Wd if row_perm is None else Wd.index_select(0, row_perm).contiguous()
        self.wq, self.w_scale, self.rot = bd.pack_weights(Wp, self.perm, self.U, block, bits=bits)
        self.row_perm = row_perm
        self.table = torch.empty(steps, dtype=torch.float32, device="cuda")
        self.steps = steps


class _Buffers:
    def __init__(self, rows: int, h: int, f: int, block: int):
        torch = _torch()
        e = lambda shape, dt=torch.float16: torch.empty(shape, dtype=dt, device="cuda")  # noqa: E731
        self.qkv, self.h2, self.g = e((rows, 3 * h)), e((rows, h)), e((rows, f))
        self.hs = [e((rows, h)), e((rows, h))]
        self.xs = e(max(rows, 1), torch.float32)
        self.xq = {(K, b): e((rows, K // 2 if b == 4 else K), torch.uint8)
                   for K in (h, f) for b in (4, 8)}
        self.ws = {K: e(max(256, bd.lib().w4a4_act_workspace_bytes(rows, K, block, 1)), torch.uint8)
                   for K in (h, f)}
        self.cws = {K: e(max(256, bd.lib().w4a4_calibrate_workspace_bytes(rows, K, block)),
                         torch.uint8) for K in (h, f)}
        self.gws = {(N, K, b): e(max(256, (bd.lib().w4a4_gemm_workspace_bytes if b == 4 else
                                           bd.lib().w4a4_gemm_w8a8_workspace_bytes)(rows, N, K)),
                                 torch.uint8)
                    for N, K in ((3 * h, h), (h, h), (f, h), (h, f)) for b in (4, 8)}
        # codes and scale of O's and down's inputs written by the producing GEMM (QKV, up): apart
        # from xq / xs, which that GEMM is still reading
        self.xqn = {K: e((rows, K // 2), torch.uint8) for K in (h, f)}
        self.xsn = e(1, torch.float32)
        self.fws = {(N, K, Kn): e(max(256, bd.lib().w4a4_gemm_rq_next_workspace_bytes(
            rows, N, K, Kn, block)), torch.uint8) for N, K, Kn in ((3 * h, h, h), (f, h, f))}


class DeviceStack:
    """weights: list (one per layer) of dicts qkv [3h,h], o [h,h], up [f,h], down [h,f] (fp16).
    calib: optional list of per-layer dicts name -> (perm, U) device tensors to use instead of the
    device calibration kernels. w8: names of the linears run as W8A8 (e.g. ("o", "down")).
    fold_perms: the V slice of QKV and the up-projection output each feed one linear only (O and
    down), so their producers store them directly in that consumer's zigzag order (QKV's V rows and
    up's rows are packed permuted) and O and down quantize contiguous rows with perm = NULL. The
    arithmetic is unchanged: a permutation is exact."""

    def __init__(self, weights, block: int, steps: int, calib=None, w8=(), fold_perms: bool = True):
        torch = _torch()
        self.block, self.steps = block, steps
        self.h = weights[0]["o"].shape[0]
        self.f = weights[0]["up"].shape[0]
        self.fold = fold_perms
        h = self.h
        self.layers = []
        for li, lw in enumerate(weights):
            layer = {}
            pu = lambda n: calib[li][n] if calib is not None else (None, None)  # noqa: E731
            bits = lambda n: 8 if n in w8 else 4  # noqa: E731
            for name in ("o", "down"):
                layer[name] = DeviceLinear(lw[name], block, steps, *pu(name), bits=bits(name))
            rp_qkv = rp_up = None
            if fold_perms:
                po = layer["o"].perm.to(torch.int64)
                rp_qkv = torch.cat([torch.arange(2 * h, device="cuda", dtype=torch.int64), 2 * h + po])
                rp_up = layer["down"].perm.to(torch.int64)
            layer["qkv"] = DeviceLinear(lw["qkv"], block, steps, *pu("qkv"), bits=bits("qkv"),
                                        row_perm=rp_qkv)
            layer["up"] = DeviceLinear(lw["up"], block, steps, *pu("up"), bits=bits("up"),
                                       row_perm=rp_up)
            self.layers.append({n: layer[n] for n in LINEARS})
        self._bufs = {}

    def bufs(self, rows: int) -> _Buffers:
        if rows not in self._bufs:
            self._bufs[rows] = _Buffers(rows, self.h, self.f, self.block)
        return self._bufs[rows]

    def set_tables(self, tables):
        """tables: list per layer of dict name -> fp32 array [steps]."""
        torch = _torch()
        for layer, tl in zip(self.layers, tables):
            for name in LINEARS:
                layer[name].table.copy_(torch.from_numpy(np.asarray(tl[name], np.float32)))

    def _linear(self, lin, X, Y, step, calib, bufs, epi=bd.EPI_NONE, res=None, in_order=False,
                record=None, pre=False, nxt=None, col0=0, keep=False):
        """Rotate-quantize X (unless pre: the producing GEMM already wrote this linear's codes into
        bufs.xqn / bufs.xsn), then the GEMM; with nxt (the next linear, whose input is Y[:, col0:]
        in its zigzag order), the GEMM also writes nxt's codes (w4a4_gemm_rq_next) and, unless keep
        (the test hooks read them), does not store those fp16 columns, whose only consumer is nxt."""
        b = lin.bits
        perm = None if in_order else lin.perm  # in_order: X already holds the zigzag order
        if pre:
            xq, xs = bufs.xqn[lin.K], bufs.xsn
        else:
            if calib:
                bd.calibrate_act_scale(X, perm, lin.rot, self.block, out=lin.table[step:step + 1],
                                       ws=bufs.cws[lin.K], bits=b)
            xq, xs = bufs.xq[(lin.K, b)], bufs.xs
            bd.rotate_quant_act(X, perm, lin.rot, self.block, None if calib else lin.table,
                                self.steps, step, xq=xq, x_scale=xs, ws=bufs.ws[lin.K], bits=b)
        if record is not None:
            record(xq, xs[:X.shape[0] if calib else 1])
        if nxt is not None:
            bd.gemm_rq_next(xq, xs, False, lin.wq, lin.w_scale, lin.K, col0, nxt.K, self.block,
                            nxt.rot, nxt.table, self.steps, step, Y=Y, epilogue=epi, residual=res,
                            xq_next=bufs.xqn[nxt.K], x_scale_next=bufs.xsn,
                            ws=bufs.fws[(lin.N, lin.K, nxt.K)], store_next_cols=keep)
            return
        bd.gemm(xq, xs, calib, lin.wq, lin.w_scale, lin.K, Y=Y, epilogue=epi, residual=res,
                ws=bufs.gws[(lin.N, lin.K, b)], bits=b)

    def run(self, X, step: int, calib: bool = False, outputs=None, codes=None, rows=None):
        """One pass of the stack for denoising step `step` on X fp16 [rows, h] (device). In calib
        mode the linears quantize per token and record their table entry for `step`. Test hooks:
        if `outputs` is a list, each linear's output (columns in natural channel order) and its
        input are appended as (output, input, residual or None); if `codes` is a list, each linear's
        activation codes and scale are appended as (codes, x_scale). `rows` (device int64 index)
        keeps only those token rows in what the hooks record."""
        bufs = self.bufs(X.shape[0])
        h = self.h
        cur = X
        pick = (lambda t: t.clone()) if rows is None else (lambda t: t.index_select(0, rows))
        cr = None
        if codes is not None:
            def cr(xq, xs):
                codes.append((pick(xq), xs.clone() if xs.numel() == 1 else pick(xs)))
        for li, layer in enumerate(self.layers):
            nxt = bufs.hs[li % 2]
            x_in = pick(cur) if outputs is not None else None
            # O's and down's inputs are quantized by the GEMM that produces them when both sides
            # are W4A4 and their channels come out in the consumer's zigzag order
            fo = self.fold and not calib and layer["qkv"].bits == 4 and layer["o"].bits == 4
            fd = self.fold and not calib and layer["up"].bits == 4 and layer["down"].bits == 4
            keep = outputs is not None
            self._linear(layer["qkv"], cur, bufs.qkv, step, calib, bufs, record=cr,
                         nxt=layer["o"] if fo else None, col0=2 * h, keep=keep)
            self._linear(layer["o"], bufs.qkv[:, 2 * h:3 * h], bufs.h2, step, calib, bufs,
                         bd.EPI_RESIDUAL, cur, in_order=self.fold, record=cr, pre=fo)
            self._linear(layer["up"], bufs.h2, bufs.g, step, calib, bufs, bd.EPI_GELU, record=cr,
                         nxt=layer["down"] if fd else None, keep=keep)
            self._linear(layer["down"], bufs.g, nxt, step, calib, bufs, bd.EPI_RESIDUAL, bufs.h2,
                         in_order=self.fold, record=cr, pre=fd)
            if outputs is not None:
                qkv = pick(self._natural(layer["qkv"], bufs.qkv))
                h2 = pick(bufs.h2)
                g = pick(self._natural(layer["up"], bufs.g))
                out = pick(nxt)
                outputs.extend([(qkv, x_in, None), (h2, qkv[:, 2 * h:3 * h], x_in), (g, h2, None),
                                (out, g, h2)])
            cur = nxt
        return cur

    @staticmethod
    def _natural(lin, Y):
        """Copy of Y with its columns back in the natural channel order (test hook)."""
        if lin.row_perm is None:
            return Y.clone()
        out = Y.clone()
        out[:, lin.row_perm] = Y
        return out

    def calibrate(self, X_calib_per_step):
        """X_calib_per_step[t]: list of fp16 numpy arrays [rows, h] (calibration draws of step t)."""
        torch = _torch()
        for t, draws in enumerate(X_calib_per_step):
            X = torch.from_numpy(np.ascontiguousarray(np.concatenate(draws, axis=0))).cuda()
            self.run(X, t, calib=True)
        torch.cuda.synchronize()
        self._bufs = {k: v for k, v in self._bufs.items() if k < 4096}
