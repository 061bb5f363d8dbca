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
    change them); only the packed rows move, when pack() is called.
    perm / U are the zigzag permutation and SVD factor; gperm / gU the order in which the
    activation's channels are gathered within each block (the same blocks, see _regroup) and the
    factor with its rows in that order, from which the activation-side rotation operand rot is
    built. The weights are always packed from perm / U."""

    def __init__(self, W, block: int, steps: int, perm=None, U=None, bits: int = 4):
        torch = _torch()
        self._W = W if isinstance(W, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(W)).cuda()
        self.N, self.K = self._W.shape
        self.B = block
        self.perm = bd.zigzag_perm(self._W, block) if perm is None else perm
        self.U = bd.block_svd(self._W, self.perm, block) if U is None else U
        self.bits = bits
        self.gperm, self.gU = self.perm, self.U
        self.table = torch.empty(steps, dtype=torch.float32, device="cuda")
        self.steps = steps

    def pack(self, row_perm=None):
        torch = _torch()
        W = self._W if row_perm is None else self._W.index_select(0, row_perm).contiguous()
        self.wq, self.w_scale, self.rot = bd.pack_weights(W, self.perm, self.U, self.B, bits=self.bits)
        if self.gperm is not self.perm:
            # the rotation operand for the regrouped gather order (R'_b = U'_b H_B: R_b's rows in
            # the new order); the one-row weight pack beside it is discarded
            one = torch.zeros((1, self.K), dtype=W.dtype, device=W.device)
            self.rot = bd.pack_weights(one, self.gperm, self.gU, self.B, bits=self.bits)[2]
        self.row_perm = row_perm
        self._W = None
        return self


def _gather_order(cols):
    """w4a4_gemm_rq_next's res_order for the residual map cols (int32 [N], N % 128 == 0): each
    128-column tile's columns sorted by the residual column they read (ties by column)."""
    torch = _torch()
    t = cols.to(torch.int64).view(-1, 128)
    idx = torch.argsort(t * 128 + torch.arange(128, device=t.device).view(1, 128), dim=1)
    base = torch.arange(0, cols.numel(), 128, device=t.device).view(-1, 1)
    return (idx + base).reshape(-1).to(torch.int32).contiguous()


def _regroup(perm, U, key, B: int):
    """Reorder the channels inside each rotation block of perm by key[channel] (stable), and U's
    rows with them. A block is the same set of channels, so x_b R_b is the same rotation (R'_b =
    U'_b H_B holds R_b's rows in the new order): only the order of the products in its sums
    changes. Used to make the channels one output tile reads from a residual stream stored in this
    order sit in runs of adjacent columns."""
    torch = _torch()
    nb = perm.numel() // B
    p = perm.to(torch.int64).view(nb, B)
    comp = key[p] * B + torch.arange(B, device=p.device, dtype=torch.int64).view(1, B)
    idx = torch.argsort(comp, dim=1)
    p2 = torch.gather(p, 1, idx).reshape(-1).to(torch.int32).contiguous()
    U2 = torch.gather(U, 1, idx.unsqueeze(-1).expand(nb, B, B)).contiguous()
    return p2, U2


def _inverse(p):
    torch = _torch()
    inv = torch.empty_like(p)
    inv[p] = torch.arange(p.numel(), device=p.device, dtype=p.dtype)
    return inv


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
        # codes and scale written by a producing GEMM for the next linear: apart from xq / xs,
        # which that GEMM is still reading
        self.xqn = {K: e((rows, K // 2), torch.uint8) for K in (h, f)}
        self.xsn = e(1, torch.float32)
        # w4a4_gemm_rq_next workspaces, by (N, K, K_next, residual map)
        self.fws = {key: e(max(256, bd.lib().w4a4_gemm_rq_next_workspace_bytes(
            rows, key[0], key[1], key[2], block, key[3])), torch.uint8)
            for key in ((3 * h, h, h, 0), (h, h, h, 1), (f, h, f, 0), (h, f, h, 1), (h, h, 0, 1),
                        (h, f, 0, 1))}


class DeviceStack:
    """weights: list (one per layer) of dicts qkv [3h,h], o [h,h], up [f,h], down [h,f] (fp16).
    calib: optional list of per-layer dicts name -> (perm, U) device tensors to use instead of the
    device calibration kernels. w8: names of the linears run as W8A8 (e.g. ("o", "down")).

    fold_perms: each linear's zigzag permutation is folded into the row order of the linear that
    produces its input, so that input comes out already in zigzag order and is rotated and quantized
    from contiguous columns (perm = NULL). The arithmetic is unchanged: a permutation is exact, and
    every output handed to the test hooks is put back in natural channel order.
      - With a W8A8 linear in the stack, only the single-consumer activations are folded: QKV's V
        rows in O's order and up's rows in down's order.
      - With every linear W4A4, the residual stream is folded as well: O's rows come out in up's
        order and down's rows in the next layer's QKV order (the last layer's in natural order).
        The residual that O and down add is then read through a column map (w4a4_gemm_rq_next's
        res_cols). Outside calibration every rotate-quantize but layer 0's QKV input then runs in
        the epilogue of the GEMM that produces the activation."""

    def __init__(self, weights, block: int, steps: int, calib=None, w8=(), fold_perms: bool = True):
        torch = _torch()
        self.block, self.steps = block, steps
        self.h = weights[0]["o"].shape[0]
        self.f = weights[0]["up"].shape[0]
        self.fold = fold_perms
        self.stream = fold_perms and not w8
        h = self.h
        nl = len(weights)
        lin = []
        for li, lw in enumerate(weights):
            pu = lambda n: calib[li][n] if calib is not None else (None, None)  # noqa: E731
            lin.append({n: DeviceLinear(lw[n], block, steps, *pu(n), bits=8 if n in w8 else 4)
                        for n in LINEARS})
        # Gather orders: QKV's input channels grouped, inside each of its blocks, by the up block
        # they belong to, and up's by the block of the next layer's QKV (the last layer's by
        # 64-channel line of the natural order): the residual O adds (stream stored in QKV's order)
        # and the one down adds (O's output, stored in up's order) are then read in runs.
        for li in range(nl):
            q, u = lin[li]["qkv"], lin[li]["up"]
            q.gperm, q.gU = _regroup(q.perm, q.U, _inverse(u.perm.to(torch.int64)) // block, block)
            if li + 1 < nl:
                key = _inverse(lin[li + 1]["qkv"].perm.to(torch.int64)) // block
            else:
                key = torch.arange(u.K, device="cuda", dtype=torch.int64) // 64
            u.gperm, u.gU = _regroup(u.perm, u.U, key, block)
        perm = lambda li, n: lin[li][n].gperm.to(torch.int64)  # noqa: E731
        self.res_map = []
        for li in range(nl):
            rp = dict.fromkeys(LINEARS)
            if fold_perms:
                rp["qkv"] = torch.cat([torch.arange(2 * h, device="cuda", dtype=torch.int64),
                                       2 * h + perm(li, "o")])
                rp["up"] = perm(li, "down")
            maps = {}
            if self.stream:
                # storage order of the residual stream entering layer li (None: natural) and of
                # the one leaving it
                q_in = perm(li, "qkv") if li > 0 else None
                q_out = perm(li + 1, "qkv") if li + 1 < nl else None
                rp["o"] = perm(li, "up")
                rp["down"] = q_out
                # O's column j adds channel rp["o"][j] of the stream, stored at inv(q_in)[...];
                # down's column j adds channel rp["down"][j] of O's output, stored in up's order
                m_o = rp["o"] if q_in is None else _inverse(q_in)[rp["o"]]
                inv_u = _inverse(rp["o"])
                m_d = inv_u if q_out is None else inv_u[q_out]
                maps = {"o": m_o.to(torch.int32).contiguous(), "down": m_d.to(torch.int32).contiguous()}
                if h % 128 == 0:
                    maps.update(o_order=_gather_order(maps["o"]), down_order=_gather_order(maps["down"]))
            for n in LINEARS:
                lin[li][n].pack(rp[n])
            self.res_map.append(maps)
        self.layers = lin
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

    def layer_plan(self, li: int, cur, out, calib: bool, bufs: _Buffers, keep: bool = False):
        """How the four linears of layer li run: one dict per linear with its input X (None when
        the producing GEMM already wrote its codes), the perm relative to X's column order, its
        codes buffers cin, output Y, epilogue, residual and residual map, and the next linear whose
        codes the GEMM writes (nxt, col0, into cout; store: whether those fp16 columns are stored
        too). keep: the test hooks read every output."""
        h, f = self.h, self.f
        L = self.layers[li]
        qkv, o, up, down = (L[n] for n in LINEARS)
        cq = lambda lin: (bufs.xq[(lin.K, lin.bits)], bufs.xs)  # noqa: E731
        plan = [dict(name=n, lin=L[n]) for n in LINEARS]
        P = {d["name"]: d for d in plan}
        if self.stream:
            maps = self.res_map[li]
            last = li + 1 == len(self.layers)
            fuse = not calib
            A, B, F = (bufs.xq[(h, 4)], bufs.xs), (bufs.xqn[h], bufs.xsn), (bufs.xqn[f], bufs.xsn)
            first = li == 0 or calib
            P["qkv"].update(X=cur if first else None, perm=qkv.gperm if li == 0 else None, cin=A,
                            Y=bufs.qkv, epi=bd.EPI_NONE, nxt=o if fuse else None, col0=2 * h,
                            cout=B, store=keep)
            P["o"].update(X=None if fuse else bufs.qkv[:, 2 * h:3 * h], perm=None,
                          cin=B if fuse else A, Y=bufs.h2, epi=bd.EPI_RESIDUAL, res=cur,
                          res_map=maps["o"], res_order=maps.get("o_order"), nxt=up if fuse else None,
                          cout=A, store=True)
            P["up"].update(X=None if fuse else bufs.h2, perm=None, cin=A, Y=bufs.g, epi=bd.EPI_GELU,
                           nxt=down if fuse else None, cout=F, store=keep)
            P["down"].update(X=None if fuse else bufs.g, perm=None, cin=F if fuse else cq(down),
                             Y=out, epi=bd.EPI_RESIDUAL, res=bufs.h2, res_map=maps["down"],
                             res_order=maps.get("down_order"),
                             nxt=None if (last or not fuse) else self.layers[li + 1]["qkv"],
                             cout=A, store=True)
            return plan
        # single-consumer folds only (or none): O and down quantize in their own launches unless
        # the producer and consumer are both W4A4
        fo = self.fold and not calib and qkv.bits == 4 and o.bits == 4
        fd = self.fold and not calib and up.bits == 4 and down.bits == 4
        P["qkv"].update(X=cur, perm=qkv.gperm, cin=cq(qkv), Y=bufs.qkv, epi=bd.EPI_NONE,
                        nxt=o if fo else None, col0=2 * h, cout=(bufs.xqn[h], bufs.xsn), store=keep)
        P["o"].update(X=None if fo else bufs.qkv[:, 2 * h:3 * h], perm=None if self.fold else o.gperm,
                      cin=(bufs.xqn[h], bufs.xsn) if fo else cq(o), Y=bufs.h2, epi=bd.EPI_RESIDUAL,
                      res=cur)
        P["up"].update(X=bufs.h2, perm=up.gperm, cin=cq(up), Y=bufs.g, epi=bd.EPI_GELU,
                       nxt=down if fd else None, cout=(bufs.xqn[f], bufs.xsn), store=keep)
        P["down"].update(X=None if fd else bufs.g, perm=None if self.fold else down.gperm,
                         cin=(bufs.xqn[f], bufs.xsn) if fd else cq(down), Y=out,
                         epi=bd.EPI_RESIDUAL, res=bufs.h2)
        return plan

    def rotate_quant_call(self, e, step: int, calib: bool, bufs: _Buffers):
        """The linear's own rotate-quantize (none when e["X"] is None)."""
        lin, X = e["lin"], e.get("X")
        if X is None:
            return
        xq, xs = e["cin"]
        if calib:
            bd.calibrate_act_scale(X, e.get("perm"), lin.rot, self.block,
                                   out=lin.table[step:step + 1], ws=bufs.cws[lin.K], bits=lin.bits)
        bd.rotate_quant_act(X, e.get("perm"), lin.rot, self.block, None if calib else lin.table,
                            self.steps, step, xq=xq, x_scale=xs, ws=bufs.ws[lin.K], bits=lin.bits)

    def gemm_call(self, e, step: int, calib: bool, bufs: _Buffers):
        """The linear's GEMM with its epilogue (and, with e["nxt"], the next linear's codes)."""
        lin, nxt, rmap = e["lin"], e.get("nxt"), e.get("res_map")
        xq, xs = e["cin"]
        if nxt is not None or rmap is not None:
            kn = nxt.K if nxt is not None else 0
            cout = e.get("cout") or (None, None)
            bd.gemm_rq_next(xq, xs, calib, lin.wq, lin.w_scale, lin.K, e.get("col0", 0) if kn else 0,
                            kn, self.block, nxt.rot if kn else None, nxt.table if kn else None,
                            self.steps, step, Y=e["Y"], epilogue=e["epi"], residual=e.get("res"),
                            xq_next=cout[0] if kn else None, x_scale_next=cout[1] if kn else None,
                            ws=bufs.fws[(lin.N, lin.K, kn, 0 if rmap is None else 1)],
                            store_next_cols=e.get("store", True), res_cols=rmap,
                            res_order=e.get("res_order"))
            return
        bd.gemm(xq, xs, calib, lin.wq, lin.w_scale, lin.K, Y=e["Y"], epilogue=e["epi"],
                residual=e.get("res"), ws=bufs.gws[(lin.N, lin.K, lin.bits)], bits=lin.bits)

    def run(self, X, step: int, calib: bool = False, outputs=None, codes=None, rows=None):
        """One pass of the stack for denoising step `step` on X fp16 [rows, h] (device); returns the
        last layer's output in natural channel order. In calib mode the linears quantize per token
        and record their table entry for `step`. Test hooks: if `outputs` is a list, each linear's
        output (columns in natural channel order) and its input are appended as (output, input,
        residual or None); if `codes` is a list, each linear's activation codes and scale are
        appended as (codes, x_scale). `rows` (device int64 index) keeps only those token rows in
        what the hooks record."""
        bufs = self.bufs(X.shape[0])
        h = self.h
        cur = X
        pick = (lambda t: t.clone()) if rows is None else (lambda t: t.index_select(0, rows))
        keep = outputs is not None
        x_nat = pick(X) if keep else None
        for li in range(len(self.layers)):
            out = bufs.hs[li % 2]
            for e in self.layer_plan(li, cur, out, calib, bufs, keep):
                self.rotate_quant_call(e, step, calib, bufs)
                if codes is not None:
                    xq, xs = e["cin"]
                    codes.append((pick(xq), pick(xs[:xq.shape[0]]) if calib else xs[:1].clone()))
                self.gemm_call(e, step, calib, bufs)
            if keep:
                L = self.layers[li]
                qkv = pick(self._natural(L["qkv"], bufs.qkv))
                h2 = pick(self._natural(L["o"], bufs.h2))
                g = pick(self._natural(L["up"], bufs.g))
                y = pick(self._natural(L["down"], out))
                outputs.extend([(qkv, x_nat, None), (h2, qkv[:, 2 * h:3 * h], x_nat), (g, h2, None),
                                (y, g, h2)])
                x_nat = y
            cur = out
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
