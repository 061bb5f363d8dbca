"""Benchmark of the W4A4 quantized linear on one MI355X.

Default workload (the headline): the full synthetic DiT action-head stack -- 16 layers x 8
denoising steps, M = 1600 tokens (32 episodes x 50 action tokens), hidden 1024, ffn 4096; per layer
QKV 1024->3072, O 1024->1024 on the V slice (attention is the identity) with a residual, up
1024->4096 with erf-GELU, down 4096->1024 with a residual; every linear W4A4 with block-128
composite rotation and its own per-step act_scale_table. One bench step = one pass over all 8
denoising steps: 512 rotate-quantize calls (zigzag gather, block rotation, step scale, int4 pack)
and 512 W4A4 GEMMs (int8 MFMA, fused dequantization and epilogue, fp16 store). The offline side
(device zigzag, block SVD, weight rotate + RTN pack, table calibration) runs once before timing
and is reported separately.

Timing: inputs, packed weights and tables are resident in HBM; W warmup steps, then K steps replayed
from a HIP graph of one pass, bracketed by synchronizations, timed with HIP events on the launch
stream. value = integer operations of the 512 GEMMs (2 M N K each) per second. The dominant
kernel's average launch duration is measured with HIP events on the same stream (a graph of
back-to-back launches of that kernel with the stack's own buffers). Prints one JSON line.
Other workloads: --workload dit_mlp_up | linear_small (few-token per-step linears).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA (POP/s x 1000)
PROFILE_TABLE_ENTRY = 0.5    # per-step scale of every linear in kernel-trace mode
FP6_PEAK_TOPS = 10100.0      # MI355X dense FP6 / FP4 MFMA
PROFILE_DIR = os.path.join(ROOT, "profiles")


def _torch():
    import torch
    return torch


def dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).cuda()


def gemm_bytes(M, N, K, per_token):
    return M * K / 2 + N * K / 2 + 4 * N + 4 * (M if per_token else 1) + 2 * M * N


def rq_bytes(M, K, B, xbytes, per_token):
    return M * K * xbytes + M * K / 2 + 4 * (M if per_token else 1) + 4 * K + 4 * K * B


class Linear:
    """Device state of one W4A4 linear: calibration, packed weights and preallocated buffers."""

    def __init__(self, W, block, bd):
        torch = _torch()
        self.bd = bd
        self.N, self.K = W.shape
        self.B = block
        Wd = dev(W)
        t0 = time.perf_counter()
        self.perm = bd.zigzag_perm(Wd, block)
        self.U = bd.block_svd(Wd, self.perm, block)
        self.wq, self.w_scale, self.rot = bd.pack_weights(Wd, self.perm, self.U, block)
        torch.cuda.synchronize()
        self.offline_s = time.perf_counter() - t0
        del Wd
        self.table = None

    def buffers(self, M, per_token):
        torch = _torch()
        self.xq = torch.empty((M, self.K // 2), dtype=torch.uint8, device="cuda")
        self.xs = torch.empty(M if per_token else 1, dtype=torch.float32, device="cuda")
        n = self.bd.lib().w4a4_act_workspace_bytes(M, self.K, self.B, 1 if per_token else 0)
        self.act_ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
        g = self.bd.lib().w4a4_gemm_workspace_bytes(M, self.N, self.K)
        self.gemm_ws = torch.empty(max(g, 256), dtype=torch.uint8, device="cuda")

    def rq(self, X, step=0, xrot=None):
        self.bd.rotate_quant_act(X, self.perm, self.rot, self.B, self.table,
                                 0 if self.table is None else self.table.numel(), step,
                                 xq=self.xq, x_scale=self.xs, xrot_dbg=xrot, ws=self.act_ws)

    def gemm(self, Y, epilogue=0, residual=None):
        self.bd.gemm(self.xq, self.xs, self.table is None, self.wq, self.w_scale, self.K, Y=Y,
                     epilogue=epilogue, residual=residual, ws=self.gemm_ws)

    def f6_buffers(self, M):
        """FP6 operands for the large-M GEMM: the weights re-encoded once (offline); the activations
        written in the FP6 layout by the rotate-quantize call itself."""
        torch = _torch()
        L = self.bd.lib()
        self.M6 = M
        self.wf = self.bd.codes_to_f6(self.wq, self.K)
        self.xf = torch.empty(max(L.w4a4_f6_operand_bytes(M, self.K), 256), dtype=torch.uint8,
                              device="cuda")
        g = L.w4a4_gemm_f6_workspace_bytes(M, self.N, self.K)
        self.f6_ws = torch.empty(max(g, 256), dtype=torch.uint8, device="cuda")
        a = L.w4a4_act_f6_workspace_bytes(M, self.K, self.B, 1 if self.table is None else 0)
        self.act_f6_ws = torch.empty(max(a, 256), dtype=torch.uint8, device="cuda")

    def to_f6(self):
        self.bd.codes_to_f6(self.xq, self.K, out=self.xf)

    def rq_f6(self, X, step=0):
        self.bd.rotate_quant_act_f6(X, self.perm, self.rot, self.B, self.table,
                                    0 if self.table is None else self.table.numel(), step,
                                    xf=self.xf, x_scale=self.xs, ws=self.act_f6_ws)

    def gemm_f6(self, Y, epilogue=0, residual=None):
        self.bd.gemm_f6(self.xf, self.M6, self.xs, self.table is None, self.wf, self.N, self.w_scale,
                        self.K, Y=Y, epilogue=epilogue, residual=residual, ws=self.f6_ws)


def time_graph(fn, steps, warmup):
    """Capture fn into a HIP graph, replay `warmup` untimed then `steps` timed. Returns ms/step."""
    torch = _torch()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager run on the side stream before capture (allocator warm-up)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_kernel_calls(calls, reps, replays=5):
    """Average duration (ms) of one launch of `calls` (each call enqueues one kernel): a HIP graph
    holding `reps` back-to-back rounds of the calls is replayed `replays` times in a row between two
    HIP events recorded on the launch stream (after two untimed replays), and the elapsed time is
    divided by the number of launches. The graph keeps host launch overhead out of the figure, and
    the back-to-back replays keep the queue ahead of the GPU (a single replay left about 1 us idle
    between its launches while the host was still submitting them); the gap between consecutive
    graph nodes stays in."""
    torch = _torch()

    def body():
        for _ in range(reps):
            for c in calls:
                c()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * reps * len(calls))


def source_hash(name):
    with open(os.path.join(ROOT, "w4a4_post_quantized_zigzag_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel_file, workload):
    """HBM bytes per launch from a committed PMC summary, if it was taken on the current source."""
    p = os.path.join(PROFILE_DIR, f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_sha256_16") != source_hash(kernel_file):
        return None
    return d.get("bytes_per_launch")


# ----------------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------------

def setup_per_step_linear(name, bd, inputs):
    torch = _torch()
    d = inputs.linear_inputs(name)
    lin = Linear(d["W"], d["block"], bd)
    T = d["steps"]
    lin.table = torch.empty(T, dtype=torch.float32, device="cuda")
    for t in range(T):
        stacked = dev(np.concatenate(d["X_calib"][t], axis=0))
        bd.calibrate_act_scale(stacked, lin.perm, lin.rot, lin.B, out=lin.table[t:t + 1])
    M = d["M"]
    lin.buffers(M, per_token=False)
    Xs = [dev(x) for x in d["X_steps"]]
    Ys = [torch.empty((M, lin.N), dtype=torch.float16, device="cuda") for _ in range(T)]

    def step():
        for t in range(T):
            lin.rq(Xs[t], t)
            lin.gemm(Ys[t])

    torch.cuda.synchronize()
    return d, lin, Xs, Ys, step


def grouped_scales(bd, inputs, steps):
    """Group-wise (per rotation block) per-step scales on the DiT MLP up-projection: device
    calibration of the [8, K/128] table, then the same 8-step pass as the headline with the
    group-wise rotate-quantize and GEMM; plus the group-wise GEMM alone on a stack-shaped
    projection (M = 1600) against the single-scale GEMM of the same shape."""
    torch = _torch()
    d = inputs.linear_inputs("dit_mlp_up")
    lin = Linear(d["W"], d["block"], bd)
    T, M, K, N, B = d["steps"], d["M"], d["K"], d["N"], d["block"]
    nb = K // B
    table = torch.empty((T, nb), dtype=torch.float32, device="cuda")
    for t in range(T):
        stacked = dev(np.concatenate(d["X_calib"][t], axis=0))
        bd.calibrate_act_scale_grouped(stacked, lin.perm, lin.rot, B, out=table[t])
    lin.buffers(M, per_token=False)
    xs = torch.empty(nb, dtype=torch.float32, device="cuda")
    Xs = [dev(x) for x in d["X_steps"]]
    Ys = [torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in range(T)]

    def step():
        for t in range(T):
            bd.rotate_quant_act_grouped(Xs[t], lin.perm, lin.rot, B, table, T, t, xq=lin.xq,
                                        x_scale=xs, ws=lin.act_ws)
            bd.gemm_grouped(lin.xq, xs, lin.wq, lin.w_scale, K, B, Y=Ys[t])

    ms = time_graph(step, steps, 5)
    gemm_ms = time_kernel_calls([lambda t=t: bd.gemm_grouped(lin.xq, xs, lin.wq, lin.w_scale, K, B,
                                                             Y=Ys[t]) for t in range(T)], 50)
    out = {"dit_mlp_up": {"M": M, "K": K, "N": N, "block": B, "denoising_steps": T,
                          "ms_per_step": ms, "tops": T * 2.0 * M * N * K / (ms * 1e-3) / 1e12,
                          "gemm_us": gemm_ms * 1e3}}
    del lin, Xs, Ys
    g = torch.Generator(device="cuda").manual_seed(3)
    M2, N2, K2 = 1600, 3072, 1024
    xq = torch.randint(0, 256, (M2, K2 // 2), generator=g, dtype=torch.uint8, device="cuda")
    wq = torch.randint(0, 256, (N2, K2 // 2), generator=g, dtype=torch.uint8, device="cuda")
    sx = torch.rand(K2 // B, generator=g, device="cuda") * 1e-2 + 1e-3
    sw = torch.rand(N2, generator=g, device="cuda") * 1e-2 + 1e-3
    Y = torch.empty((M2, N2), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(256, bd.lib().w4a4_gemm_workspace_bytes(M2, N2, K2)), dtype=torch.uint8,
                     device="cuda")
    tg = time_kernel_calls([lambda: bd.gemm_grouped(xq, sx, wq, sw, K2, B, Y=Y)], 20)
    tp = time_kernel_calls([lambda: bd.gemm(xq, sx[:1], False, wq, sw, K2, Y=Y, ws=ws)], 20)
    ops = 2.0 * M2 * N2 * K2
    out["gemm_1600x3072x1024"] = {"grouped_us": tg * 1e3, "grouped_tops": ops / (tg * 1e-3) / 1e12,
                                  "single_scale_us": tp * 1e3,
                                  "single_scale_tops": ops / (tp * 1e-3) / 1e12}
    return out


def gptq_offline(bd, inputs):
    """Offline GPTQ pack of the DiT MLP up-projection weights (4096 x 1024) on the device: Hessian
    over the 80 calibration draws, damped inverse factor, column sweep and pack; wall time of each
    phase (device synchronized)."""
    torch = _torch()
    d = inputs.linear_inputs("dit_mlp_up")
    W = dev(d["W"])
    B = d["block"]
    perm = bd.zigzag_perm(W, B)
    U = bd.block_svd(W, perm, B)
    draws = [dev(x) for t in range(d["steps"]) for x in d["X_calib"][t]]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    H = None
    for x in draws:
        H = bd.gptq_hessian(x, perm, U, B, H=H, accumulate=H is not None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    Hf, dead = bd.gptq_factor(H)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    bd.pack_weights_gptq(W, perm, U, B, Hf, dead)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    return {"N": int(W.shape[0]), "K": int(W.shape[1]), "calibration_rows": sum(int(x.shape[0]) for x in draws),
            "hessian_s": t1 - t0, "factor_s": t2 - t1, "sweep_and_pack_s": t3 - t2}


def setup_per_token_linear(name, bd, inputs):
    torch = _torch()
    d = inputs.linear_inputs(name)
    lin = Linear(d["W"], d["block"], bd)
    M = d["M"]
    lin.buffers(M, per_token=True)
    X = dev(d["X"])
    Y = torch.empty((M, lin.N), dtype=torch.float16, device="cuda")

    def step():
        lin.rq(X)
        lin.gemm(Y)

    torch.cuda.synchronize()
    return d, lin, [X], [Y], step


def setup_stack(bd, inputs, layers=None, w8=(), calibrate=True):
    """Synthetic action-head stack (16 layers of QKV -> V slice -> O + residual -> up + GELU -> down
    + residual, M = 1600 tokens, 8 denoising steps): device calibration (zigzag, block SVD, pack,
    per-linear per-step tables from the stacked calibration draws), then one pass = 8 steps x 16
    layers x 4 linears (W4A4, or W8A8 for the names in w8). calibrate=False sets every table entry
    to PROFILE_TABLE_ENTRY instead of running the calibration chain (for kernel traces that must
    hold only the pass's launches; no kernel's duration depends on the table's values)."""
    from w4a4_post_quantized_zigzag_amd.stack import DeviceStack
    torch = _torch()
    cfg = inputs.STACK
    Wl = inputs.stack_weights(layers=layers)
    act = inputs.stack_activations()
    T, B, M = cfg["steps"], cfg["block"], cfg["M"]
    t0 = time.perf_counter()
    ds = DeviceStack(Wl, B, T, w8=w8)
    torch.cuda.synchronize()
    offline = time.perf_counter() - t0
    del Wl
    t1 = time.perf_counter()
    if calibrate:
        ds.calibrate(act["X_calib"])
    else:
        ds.set_tables([{n: np.full(T, PROFILE_TABLE_ENTRY, np.float32) for n in ds.layers[0]}
                       for _ in ds.layers])
    calib_s = time.perf_counter() - t1
    Xs = [dev(x) for x in act["X_steps"]]
    ds.bufs(M)

    def step():
        for t in range(T):
            ds.run(Xs[t], t)

    torch.cuda.synchronize()
    info = dict(layers=len(ds.layers), M=M, hidden=ds.h, ffn=ds.f, steps=T, offline_s=offline,
                calib_s=calib_s)
    return info, ds, Xs, None, step


# ----------------------------------------------------------------------------------------------

def cpu_baseline_per_step(d, budget_s=12.0):
    """The oracle (single-threaded C, fp64) on the same workload: its own calibration, then the
    runtime path (rotate-quantize + integer GEMM + dequantization) for as many denoising steps as
    fit in the budget (at least one). Returns ops/s and a description of the sample."""
    import oracle
    W, B = d["W"], d["block"]
    perm = oracle.zigzag_perm(W, B)
    U = oracle.block_svd(W, perm, B)
    pw = oracle.pack_weights(W, perm, U, B)
    table = oracle.calibrate_table(d["X_calib"], perm, U, B)
    M, K, N = d["M"], d["K"], d["N"]
    t0 = time.perf_counter()
    done = 0
    outs = []
    for t, X in enumerate(d["X_steps"]):
        act = oracle.rotate_quant_act(X, perm, U, B, "per_step", table, d["steps"], t, R=pw["R"])
        g = oracle.gemm(act["codes"], act["scale"], False, pw["codes"], pw["w_scale"])
        outs.append(g["Y"])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    ops = done * 2.0 * M * N * K
    return ops / el, f"{done} of {d['steps']} denoising steps of the same workload (runtime path)", \
        outs


def host_cpu():
    """CPU model and logical core count of the host that runs the oracle."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "nproc": os.cpu_count()}


def cpu_oracle_stages(inputs, rows=16, cols=1024):
    """The oracle's runtime stages (rotation, quantization, integer GEMM, dequantization) timed one
    by one on a bounded sample: `rows` activation rows and at most `cols` output channels of each
    linear, on one host thread. Rotation and quantization cost grows with M, the GEMM and the
    dequantization with M x N, so each stage is extrapolated to the full shape by that factor; the
    action stack's layer-step (its four linears on inputs of their own shapes) is further scaled by
    its 128 layer-steps. Weights are packed offline for the sampled output channels only, with
    identity U blocks (untimed; the stages' cost does not depend on the rotation's values)."""
    import oracle
    from oracle.reference import EPI_GELU, EPI_NONE, EPI_RESIDUAL

    def linear(W, X, B, mode, epi):
        perm = oracle.zigzag_perm(W, B)
        # the stages' cost does not depend on U's values: identity blocks spare the oracle's SVD
        U = np.stack([np.eye(B, dtype=np.float32)] * (W.shape[1] // B))
        n = min(cols, W.shape[0])
        pw = oracle.pack_weights(W, perm, U, B, rows=np.arange(n))
        res = np.zeros((X.shape[0], n), np.float16) if epi == EPI_RESIDUAL else None
        clk = time.perf_counter
        t0 = clk()
        Xr = oracle.rotate_rows(X, perm, pw["R"], B)
        t1 = clk()
        table = None
        if mode == "per_step":
            table = np.array([np.float32(np.max(np.abs(Xr)) / 7.0)], np.float32)
        t1b = clk()
        act = oracle.quantize_act(Xr, mode, table, 1 if table is not None else None,
                                  0 if table is not None else None)
        t2 = clk()
        acc = oracle.int_gemm(act["codes"], pw["codes"][:n])
        t3 = clk()
        oracle.dequant(acc, act["scale"], mode == "per_token", pw["w_scale"][:n], epi, res)
        t4 = clk()
        return {"rotate": t1 - t0, "quantize": t2 - t1b, "int_gemm": t3 - t2, "dequant": t4 - t3,
                "n": n}

    def scaled(st, M, N, K, reps=1):
        fm, fn = M / rows, N / st["n"]
        us = {"rotate": st["rotate"] * fm, "quantize": st["quantize"] * fm,
              "int_gemm": st["int_gemm"] * fm * fn, "dequant": st["dequant"] * fm * fn}
        return {k: v * reps * 1e6 for k, v in us.items()}

    out = {"kind": "oracle", "cores": 1, "host": host_cpu(),
           "sample": f"{rows} activation rows x at most {cols} output channels per linear, "
                     "each stage extrapolated linearly to the full shape"}
    rng = np.random.Generator(np.random.PCG64(11))
    for name in ("prefill_proj", "longk_down"):
        d = inputs.linear_inputs(name, M=rows)
        M, K, N = inputs.LINEAR_WORKLOADS[name]["M"], d["K"], d["N"]
        st = linear(d["W"], d["X"], d["block"], "per_token", EPI_NONE)
        us = scaled(st, M, N, K)
        tot = sum(us.values())
        out[name] = {"M": M, "N": N, "K": K, "stage_us": us, "total_us": tot,
                     "tops": 2.0 * M * N * K / (tot * 1e-6) / 1e12}
    S = inputs.STACK
    lw = inputs.stack_weights(layers=1)[0]
    h, f, M = S["hidden"], S["ffn"], S["M"]
    layer = {}
    ops = 0.0
    for nm, epi in (("qkv", EPI_NONE), ("o", EPI_RESIDUAL), ("up", EPI_GELU), ("down", EPI_RESIDUAL)):
        W = lw[nm]
        X = rng.standard_normal((rows, W.shape[1])).astype(np.float16)
        st = linear(W, X, S["block"], "per_step", epi)
        layer[nm] = scaled(st, M, W.shape[0], W.shape[1], reps=S["layers"] * S["steps"])
        ops += 2.0 * M * W.shape[0] * W.shape[1] * S["layers"] * S["steps"]
    tot = sum(sum(v.values()) for v in layer.values())
    stages = {k: sum(v[k] for v in layer.values()) for k in ("rotate", "quantize", "int_gemm", "dequant")}
    out["action_stack"] = {"M": M, "layer_steps": S["layers"] * S["steps"], "stage_us": stages,
                           "total_us": tot, "tops": ops / (tot * 1e-6) / 1e12}
    return out


STACK_LINEAR_SHAPES = (("qkv", "N=3072, K=1024"), ("o", "N=1024, K=1024"), ("up", "N=4096, K=1024"),
                       ("down", "N=1024, K=4096"))


def stack_kernel_times(bd, ds, Xs, reps=30):
    """Average launch duration (ms) of each linear's calls in the stack pass, on the stack's own
    buffers and wiring (layer 1 at step 0, a layer whose every input arrives quantized by the
    producing GEMM when the residual stream is folded), each from a HIP graph of back-to-back
    launches timed with HIP events on the launch stream. Where a GEMM writes the next linear's
    codes in its epilogue, that GEMM entry is the fused call and the consumer has no rotate-quantize
    of its own (None). layer0_input_rotate_quant_ms: the rotate-quantize of layer 0's QKV input
    (the stack's input, gathered through QKV's zigzag permutation), once per step."""
    bufs = ds.bufs(Xs[0].shape[0])
    li = 1 if len(ds.layers) > 1 else 0
    plan = ds.layer_plan(li, bufs.hs[0], bufs.hs[1], False, bufs)
    out = {}
    for e in plan:
        lin = e["lin"]
        rq = (lambda e=e: ds.rotate_quant_call(e, 0, False, bufs)) if e.get("X") is not None else None
        gm = lambda e=e: ds.gemm_call(e, 0, False, bufs)  # noqa: E731
        if rq is not None:
            rq()
        gm()
        nxt = e.get("nxt")
        fuses = None if nxt is None else ("next layer's qkv" if e["name"] == "down" else
                                          next(n for n, l2 in ds.layers[li].items() if l2 is nxt))
        out[e["name"]] = {"N": lin.N, "K": lin.K,
                          "rotate_quant_ms": None if rq is None else time_kernel_calls([rq], reps),
                          "gemm_ms": time_kernel_calls([gm], reps),
                          "gemm_fuses_rotate_quant_of": fuses,
                          "residual_column_map": e.get("res_map") is not None}
    e0 = ds.layer_plan(0, Xs[0], bufs.hs[1], False, bufs)[0]
    rq0 = lambda: ds.rotate_quant_call(e0, 0, False, bufs)  # noqa: E731
    rq0()
    return out, time_kernel_calls([rq0], reps)


def cpu_baseline_stack(inputs, M=1600):
    """The oracle (single-threaded C, fp64) on one layer-step of the stack: the four linears of
    layer 0 at step 0 on all M tokens (rotate-quantize, integer GEMM, dequantization with the
    layer's epilogues), chained as in the stack. Weights are packed and the per-step scales set
    before the clock starts. Returns the integer ops per second (one layer-step is 1/128 of a pass,
    so the rate is that of a pass) and a description of the sample."""
    import oracle
    from oracle.reference import EPI_GELU, EPI_NONE, EPI_RESIDUAL
    S = inputs.STACK
    B, h = S["block"], S["hidden"]
    lw = inputs.stack_weights(layers=1)[0]
    X = inputs.stack_activations(M=M, steps=1, calib=0)["X_steps"][0]
    lin = {}
    for nm in ("qkv", "o", "up", "down"):
        W = lw[nm]
        perm = oracle.zigzag_perm(W, B)
        U = oracle.block_svd(W, perm, B)
        lin[nm] = {"perm": perm, "U": U, "pack": oracle.pack_weights(W, perm, U, B)}

    def run(name, Xin, epi, res, table):
        L = lin[name]
        act = oracle.rotate_quant_act(Xin, L["perm"], L["U"], B, "per_step", table, 1, 0,
                                      R=L["pack"]["R"])
        return oracle.gemm(act["codes"], act["scale"], False, L["pack"]["codes"],
                           L["pack"]["w_scale"], epi, res)["Y"]

    # per-step scales: the absmax of each linear's rotated input on the first 16 tokens (an untimed
    # dry run of the chain; the values do not change the work)
    tables = {}

    def linear(name, xin, epi, res):
        if name not in tables:
            L = lin[name]
            tables[name] = oracle.calibrate_table([[xin]], L["perm"], L["U"], B, R=L["pack"]["R"])
        return run(name, xin, epi, res, tables[name])

    def chain(x):
        qkv = linear("qkv", x, EPI_NONE, None)
        h2 = linear("o", np.ascontiguousarray(qkv[:, 2 * h:3 * h]), EPI_RESIDUAL, x)
        g = linear("up", h2, EPI_GELU, None)
        return linear("down", g, EPI_RESIDUAL, h2)

    chain(X[:16])
    t0 = time.perf_counter()
    chain(X)
    el = time.perf_counter() - t0
    ops = 2.0 * M * (3 * h * h + h * h + S["ffn"] * h + h * S["ffn"])
    return ops / el, el, (f"one layer-step of the same stack (QKV, O, up, down of layer 0 at step 0, "
                          f"all {M} tokens, rotate-quantize + integer GEMM + dequantization); the "
                          f"pass is 128 such layer-steps, so the rate is extrapolated x128 "
                          f"({el:.1f} s measured for the layer-step)")


def stack_headline(bd, inputs, args, result):
    torch = _torch()
    info, ds, Xs, _, step = setup_stack(bd, inputs, calibrate=not args.profile_timed_only)
    M, h, f, T, L = info["M"], info["hidden"], info["ffn"], info["steps"], info["layers"]
    ms = time_graph(step, args.steps, args.warmup)
    ops = T * L * 2.0 * M * (3 * h * h + h * h + f * h + h * f)
    if args.profile_timed_only:
        # the trace holds the offline pack and the timed passes only: no calibration chain, no
        # per-kernel timing graphs, no oracle
        result.update(value=ops / (ms * 1e-3) / 1e12, ms_per_step=ms,
                      config={"workload": "action_stack (kernel-trace mode: fixed per-step tables)"})
        return
    kt, rq0_ms = stack_kernel_times(bd, ds, Xs)
    calls = T * L  # launches of each linear's kernels per pass
    # the dominant kernel: the largest total time per pass among the per-linear kernels
    totals = {}
    for name, d in kt.items():
        totals[(name, "gemm")] = d["gemm_ms"] * calls
        if d["rotate_quant_ms"] is not None:
            totals[(name, "rotate_quant")] = d["rotate_quant_ms"] * calls
    (dn, dk) = max(totals, key=totals.get)
    d = kt[dn]
    if dk == "gemm":
        op = 2.0 * M * d["N"] * d["K"]
        ach = op / (d["gemm_ms"] * 1e-3) / 1e12
        also = d.get("gemm_fuses_rotate_quant_of")
        kname = f"{dn} GEMM ({M}x{d['N']}x{d['K']}, int8 MFMA)" + (
            f", with {also}'s rotate-quantize in its epilogue" if also else "")
        roof = {"bound": "mfma", "kernel": kname,
                "achieved": ach, "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                "frac": ach / INT8_PEAK_TOPS,
                "traffic": traffic_from_profile("k_gemm.hip", f"action_stack_{dn}_gemm"),
                "algorithmic_ops_per_launch": op, "avg_launch_us": d["gemm_ms"] * 1e3}
    else:
        by = rq_bytes(M, d["K"], ds.block, 2, False)
        ach = by / (d["rotate_quant_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": f"{dn} rotate-quantize ({M}x{d['K']})", "achieved": ach,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                "traffic": traffic_from_profile("k_act.hip", f"action_stack_{dn}_rq"),
                "algorithmic_bytes_per_launch": by, "avg_launch_us": d["rotate_quant_ms"] * 1e3}
    kernels = {}
    for name, d in kt.items():
        op = 2.0 * M * d["N"] * d["K"]
        by = rq_bytes(M, d["K"], ds.block, 2, False)
        kernels[name] = {"gemm_us": d["gemm_ms"] * 1e3,
                         "gemm_tops": op / (d["gemm_ms"] * 1e-3) / 1e12,
                         "gemm_frac_int8_peak": op / (d["gemm_ms"] * 1e-3) / 1e12 / INT8_PEAK_TOPS,
                         "gemm_fuses_rotate_quant_of": d["gemm_fuses_rotate_quant_of"],
                         "residual_column_map": d["residual_column_map"]}
        if d["rotate_quant_ms"] is not None:
            kernels[name].update(
                rotate_quant_us=d["rotate_quant_ms"] * 1e3,
                rotate_quant_gbps=by / (d["rotate_quant_ms"] * 1e-3) / 1e9,
                rotate_quant_frac_hbm=by / (d["rotate_quant_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS)
        else:
            kernels[name]["rotate_quant_us"] = "in the producing GEMM's epilogue"
    by0 = rq_bytes(M, h, ds.block, 2, False)
    kernels["layer0_input"] = {
        "rotate_quant_us": rq0_ms * 1e3, "launches_per_pass": T,
        "rotate_quant_gbps": by0 / (rq0_ms * 1e-3) / 1e9,
        "note": "the stack input's rotate-quantize (gather through layer 0's QKV permutation); "
                "every later activation is quantized in its producer's epilogue"}
    result.update(
        value=ops / (ms * 1e-3) / 1e12, ms_per_step=ms,
        config={"workload": f"action_stack: {L} layers x {T} denoising steps, M = {M} tokens "
                            f"(32 episodes x 50), hidden {h}, ffn {f}; per layer QKV, O (+residual), "
                            f"up (+erf-GELU), down (+residual), all W4A4, block {ds.block}, "
                            f"per-linear per-step act_scale_tables",
                "M": M, "hidden": h, "ffn": f, "layers": L, "denoising_steps": T,
                "block": ds.block, "linear_calls_per_step": 4 * L * T, "scale_mode": "per_step"},
        roofline=roof, kernels=kernels,
        frac_int8_peak_whole_pass=ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS,
        offline={"device_zigzag_svd_pack_s": info["offline_s"],
                 "device_table_calibration_s": info["calib_s"]})
    if not args.no_cpu_baseline:
        v, el, sample = cpu_baseline_stack(inputs, M)
        result["cpu_baseline"] = {"value": v / 1e12, "unit": "TOPS", "cores": 1, "kind": "oracle",
                                  "sample": sample, "host": host_cpu()}
    del ds, Xs, step
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="action_stack",
                    choices=["action_stack", "dit_mlp_up", "linear_small"])
    ap.add_argument("--profile-timed-only", action="store_true",
                    help="kernel-trace mode: fixed per-step tables instead of the calibration "
                         "chain, and nothing launched after the timed passes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-supplementary", action="store_true")
    ap.add_argument("--supp-steps", type=int, default=30)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of known size (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the W4A4 linear "
              "shards over tokens with no exchange, so N GPUs would run N copies of this line).",
              file=sys.stderr)
        sys.exit(2)

    torch = _torch()
    from w4a4_post_quantized_zigzag_amd import binding as bd
    from w4a4_post_quantized_zigzag_amd import inputs
    bd.lib()
    torch.cuda.set_device(0)

    result = {"metric": "W4A4 linear TOPS and GB/s (% of int8-MFMA / HBM roofline), 1 MI355X",
              "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int4",
              "data": "synthetic (seeded draws of the workload's shapes and distributions; "
                      "random-init weights)"}

    name = args.workload
    if name == "action_stack":
        stack_headline(bd, inputs, args, result)
    elif name in ("dit_mlp_up", "linear_small"):
        d, lin, Xs, Ys, step = setup_per_step_linear(name, bd, inputs)
        M, K, N, B, T = d["M"], d["K"], d["N"], d["block"], d["steps"]
        ms = time_graph(step, args.steps, args.warmup)
        ops = T * 2.0 * M * N * K
        xb = 2 if d["xdtype"] == np.float16 else 4
        bytes_step = T * (gemm_bytes(M, N, K, False) + rq_bytes(M, K, B, xb, False))
        gemm_ms = time_kernel_calls([lambda t=t: lin.gemm(Ys[t]) for t in range(T)], 50)
        lin.rq(Xs[0], 0)
        rq_ms = time_kernel_calls([lambda t=t: lin.rq(Xs[t], t) for t in range(T)], 50)
        gb = gemm_bytes(M, N, K, False)
        result.update(value=ops / (ms * 1e-3) / 1e12, ms_per_step=ms,
                      config={"workload": f"{name}: X fp16 [{M},{K}] x 8 denoising steps in order, "
                                          f"W fp16 [{N},{K}], block {B}, per-step act_scale_table",
                              "M": M, "K": K, "N": N, "block": B, "denoising_steps": T,
                              "scale_mode": "per_step"},
                      bandwidth_gbps=bytes_step / (ms * 1e-3) / 1e9)
        result["roofline"] = {"bound": "hbm",
                              "kernel": "k_gemm_smallm_wide<4, 1, 8, 4> (16 output columns per "
                                        "workgroup, K split over its 8 waves)",
                              "achieved": gb / (gemm_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                              "unit": "GB/s", "frac": gb / (gemm_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                              "traffic": traffic_from_profile("k_gemm.hip", name),
                              "algorithmic_bytes_per_launch": gb,
                              "avg_launch_us": gemm_ms * 1e3}
        result["kernels"] = {"gemm_avg_us": gemm_ms * 1e3, "rotate_quant_avg_us": rq_ms * 1e3,
                             "rotate_quant_gbps": rq_bytes(M, K, B, xb, False) / (rq_ms * 1e-3) / 1e9}
        result["offline"] = {"calibrate_and_pack_s": lin.offline_s}
        if not args.no_cpu_baseline:
            v, sample, _ = cpu_baseline_per_step(d)
            result["cpu_baseline"] = {"value": v / 1e12, "unit": "TOPS", "cores": 1,
                                      "kind": "oracle", "sample": sample, "host": host_cpu()}

    if not args.no_supplementary:
        result["supplementary"] = supplementary(bd, inputs, args.supp_steps)
        if not args.no_cpu_baseline:
            result["supplementary"]["cpu_oracle_stages"] = cpu_oracle_stages(inputs)
    print(json.dumps(result))


COLD_BYTES = 512 << 20  # distinct operand copies cycled per round: twice the 256 MB last-level cache


def cold_hbm(bd, inputs):
    """HBM-bound kernels on cold operands: each timed launch reads a different copy of its large
    operand, and the copies add up to COLD_BYTES, so by the time a copy comes round again the
    last-level cache has been flushed by the others.
    - small-M GEMM sweep, M in {16, 50, 64} with N = K = 16384 (128 MB of packed weights per copy),
      where the weight stream is long enough for its bandwidth to be measurable;
    - the prefill GEMM (1024 x 16384 x 2048) with int4 and FP6 operands, cycling weight copies;
    - rotate-quantize of the prefill and long-K workloads (per-token, zigzag order), cycling copies
      of X (4 MB and 32 MB)."""
    torch = _torch()
    out = {"note": "cold: operands cycled over distinct copies totalling 512 MB",
           "small_m_gemm": [], "rotate_quant": []}
    N = K = 16384
    g = torch.Generator(device="cuda").manual_seed(7)
    wbytes = N * K // 2
    copies = max(2, COLD_BYTES // wbytes)
    wqs = [torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8, device="cuda")
           for _ in range(copies)]
    w_scale = torch.rand(N, generator=g, device="cuda") * 1e-2
    for M in (16, 50, 64):
        xq = torch.randint(0, 256, (M, K // 2), generator=g, dtype=torch.uint8, device="cuda")
        xs = torch.ones(1, device="cuda")
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        ws = torch.empty(max(256, bd.lib().w4a4_gemm_workspace_bytes(M, N, K)), dtype=torch.uint8,
                         device="cuda")
        ms = time_kernel_calls([lambda w=w: bd.gemm(xq, xs, False, w, w_scale, K, Y=Y, ws=ws)
                                for w in wqs], 10)
        gbps = gemm_bytes(M, N, K, False) / (ms * 1e-3) / 1e9
        out["small_m_gemm"].append({"M": M, "N": N, "K": K, "weight_copies": copies,
                                    "gemm_us": ms * 1e3, "gbps": gbps,
                                    "frac_hbm": gbps / HBM_PEAK_GBPS,
                                    "tops": 2.0 * M * N * K / (ms * 1e-3) / 1e12})
    del wqs
    torch.cuda.empty_cache()
    # large-M GEMM (prefill shape) with cold weights, int4 and FP6 operands: the weight bytes per
    # launch are 16 MB and 24 MB, a small part of the operand traffic of a compute-bound tile loop
    M, N, K = 1024, 16384, 2048
    xq = torch.randint(0, 256, (M, K // 2), generator=g, dtype=torch.uint8, device="cuda")
    xs = torch.full((M,), 1e-3, device="cuda")
    w_scale = torch.rand(N, generator=g, device="cuda") * 1e-2
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    L = bd.lib()
    gws = torch.empty(max(256, L.w4a4_gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda")
    fws = torch.empty(max(256, L.w4a4_gemm_f6_workspace_bytes(M, N, K)), dtype=torch.uint8,
                      device="cuda")
    xf = bd.codes_to_f6(xq, K)
    res = {"M": M, "N": N, "K": K}
    ops = 2.0 * M * N * K
    for fmt, wbytes in (("int4", N * K // 2), ("fp6", L.w4a4_f6_operand_bytes(N, K))):
        copies = max(2, COLD_BYTES // wbytes)
        ws_ = []
        for _ in range(copies):
            w = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8, device="cuda")
            ws_.append(w if fmt == "int4" else bd.codes_to_f6(w, K))
        if fmt == "int4":
            calls = [lambda w=w: bd.gemm(xq, xs, True, w, w_scale, K, Y=Y, ws=gws) for w in ws_]
        else:
            calls = [lambda w=w: bd.gemm_f6(xf, M, xs, True, w, N, w_scale, K, Y=Y, ws=fws)
                     for w in ws_]
        ms = time_kernel_calls(calls, 4)
        res[fmt] = {"weight_copies": copies, "gemm_us": ms * 1e3,
                    "tops": ops / (ms * 1e-3) / 1e12,
                    "frac_int8_peak": ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS}
        del ws_, calls
        torch.cuda.empty_cache()
    out["large_m_gemm_prefill"] = res
    del xq, xf, Y, gws, fws
    torch.cuda.empty_cache()
    for name in ("prefill_proj", "longk_down"):
        d = inputs.linear_inputs(name, M=1)  # weights only; X copies are drawn on the device
        M, K = inputs.LINEAR_WORKLOADS[name]["M"], d["K"]
        lin = Linear(d["W"], d["block"], bd)
        lin.buffers(M, per_token=True)
        xcopies = max(2, COLD_BYTES // (M * K * 2))
        Xs = [torch.randn((M, K), generator=g, device="cuda").half() for _ in range(xcopies)]
        ms = time_kernel_calls([lambda X=X: lin.rq(X) for X in Xs], 4)
        gbps = rq_bytes(M, K, d["block"], 2, True) / (ms * 1e-3) / 1e9
        out["rotate_quant"].append({"workload": name, "M": M, "K": K, "x_copies": xcopies,
                                    "scale_mode": "per_token", "rq_us": ms * 1e3, "gbps": gbps,
                                    "frac_hbm": gbps / HBM_PEAK_GBPS})
        del Xs, lin
        torch.cuda.empty_cache()
    return out


COPY_BYTES = 1 << 30


def copy_calibration(reps=3):
    """A plain copy of COPY_BYTES (larger than the 256 MB last-level cache, so it streams from and
    to HBM), `reps` times: under rocprofv3 --pmc its FETCH_SIZE and WRITE_SIZE per dispatch give the
    factor from those counters to bytes."""
    torch = _torch()
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "reps": reps}))


def square_gemm(bd, n):
    """Kernel ceiling on a large square GEMM (seeded random codes, per-token scales): the int4
    pipelined kernel against the FP6-operand kernel, outputs compared bit for bit."""
    torch = _torch()
    g = torch.Generator(device="cuda").manual_seed(0)
    xq = torch.randint(0, 256, (n, n // 2), generator=g, device="cuda", dtype=torch.uint8)
    wq = torch.randint(0, 256, (n, n // 2), generator=g, device="cuda", dtype=torch.uint8)
    xs = torch.full((n,), 1e-3, device="cuda")
    ws_ = torch.full((n,), 1e-3, device="cuda")
    Y = torch.empty((n, n), dtype=torch.float16, device="cuda")
    Y6 = torch.empty_like(Y)
    L = bd.lib()
    gws = torch.empty(max(L.w4a4_gemm_workspace_bytes(n, n, n), 256), dtype=torch.uint8, device="cuda")
    fws = torch.empty(max(L.w4a4_gemm_f6_workspace_bytes(n, n, n), 256), dtype=torch.uint8, device="cuda")
    xf, wf = bd.codes_to_f6(xq, n), bd.codes_to_f6(wq, n)
    i4 = time_kernel_calls([lambda: bd.gemm(xq, xs, True, wq, ws_, n, Y=Y, ws=gws)], 5)
    f6 = time_kernel_calls([lambda: bd.gemm_f6(xf, n, xs, True, wf, n, ws_, n, Y=Y6, ws=fws)], 5)
    torch.cuda.synchronize()
    ops = 2.0 * n ** 3
    res = {"M": n, "N": n, "K": n,
           "int4_gemm_us": i4 * 1e3, "int4_gemm_tops": ops / (i4 * 1e-3) / 1e12,
           "fp6_gemm_us": f6 * 1e3, "fp6_gemm_tops": ops / (f6 * 1e-3) / 1e12,
           "fp6_gemm_frac_int8_peak": ops / (f6 * 1e-3) / 1e12 / INT8_PEAK_TOPS,
           "same_output_bits": bool(torch.equal(Y.view(torch.int16), Y6.view(torch.int16)))}
    del xq, wq, Y, Y6, xf, wf, gws, fws
    torch.cuda.empty_cache()
    return res


def few_token_line(bd, inputs, name, steps):
    """The few-token per-step linear (the DiT MLP up-projection, X fp16 [50, 1024] x 8 denoising
    steps, W [4096, 1024]): one step = the 8 denoising steps in order; plus each kernel's average
    launch duration."""
    d, lin, Xs, Ys, step = setup_per_step_linear(name, bd, inputs)
    M, K, N, B, T = d["M"], d["K"], d["N"], d["block"], d["steps"]
    ms = time_graph(step, steps, 10)
    gemm_ms = time_kernel_calls([lambda t=t: lin.gemm(Ys[t]) for t in range(T)], 50)
    lin.rq(Xs[0], 0)
    rq_ms = time_kernel_calls([lambda t=t: lin.rq(Xs[t], t) for t in range(T)], 50)
    gb = gemm_bytes(M, N, K, False)
    xb = 2 if d["xdtype"] == np.float16 else 4
    return {"M": M, "K": K, "N": N, "block": B, "denoising_steps": T, "ms_per_step": ms,
            "tops": T * 2.0 * M * N * K / (ms * 1e-3) / 1e12,
            "gemm_us": gemm_ms * 1e3, "gemm_gbps": gb / (gemm_ms * 1e-3) / 1e9,
            "gemm_frac_hbm": gb / (gemm_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "rotate_quant_us": rq_ms * 1e3,
            "rotate_quant_gbps": rq_bytes(M, K, B, xb, False) / (rq_ms * 1e-3) / 1e9,
            "traffic_gemm_bytes_per_launch": traffic_from_profile("k_gemm.hip", name),
            "note": "single launches of 2.5 MB (GEMM) and 0.1 MB (rotate-quantize) are bound by "
                    "launch and two dependent load latencies, not by HBM bandwidth"}


def supplementary(bd, inputs, steps):
    """Shorter runs of the other workloads: the few-token DiT linear, the large-M per-token
    linears (int4 and FP6 operands), a square GEMM, cold-HBM sweeps, group-wise scales, the GPTQ
    pack and the mixed W4A4/W8A8 stack."""
    torch = _torch()
    out = {}
    for name in ("prefill_proj", "longk_down"):
        d, lin, Xs, Ys, step = setup_per_token_linear(name, bd, inputs)
        M, K, N, B = d["M"], d["K"], d["N"], d["block"]
        ms = time_graph(step, steps, 5)
        gemm_ms = time_kernel_calls([lambda: lin.gemm(Ys[0])], 20)
        rq_ms = time_kernel_calls([lambda: lin.rq(Xs[0])], 20)
        ops = 2.0 * M * N * K
        out[name] = {"M": M, "K": K, "N": N, "block": B, "scale_mode": "per_token",
                     "linear_ms": ms, "linear_tops": ops / (ms * 1e-3) / 1e12,
                     "gemm_us": gemm_ms * 1e3, "gemm_tops": ops / (gemm_ms * 1e-3) / 1e12,
                     "gemm_frac_int8_peak": ops / (gemm_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS,
                     "rotate_quant_us": rq_ms * 1e3,
                     "rotate_quant_gbps": rq_bytes(M, K, B, 2, True) / (rq_ms * 1e-3) / 1e9,
                     "rotate_quant_frac_hbm": rq_bytes(M, K, B, 2, True) / (rq_ms * 1e-3) / 1e9
                     / HBM_PEAK_GBPS,
                     "calibrate_and_pack_s": lin.offline_s}
        # the same linear with FP6 (E3M2) matrix-core operands: weights re-encoded offline, the
        # activation codes after each rotate-quantize; outputs must be the int4 path's bits
        lin.f6_buffers(M)
        Y6 = torch.empty_like(Ys[0])

        def step_f6():
            lin.rq_f6(Xs[0])
            lin.gemm_f6(Y6)

        ms6 = time_graph(step_f6, steps, 5)
        f6_ms = time_kernel_calls([lambda: lin.gemm_f6(Y6)], 20)
        rq6 = time_kernel_calls([lambda: lin.rq_f6(Xs[0])], 20)
        rq4 = time_kernel_calls([lambda: lin.rq(Xs[0])], 20)
        lin.rq(Xs[0])
        cvt_ms = time_kernel_calls([lin.to_f6], 20)
        step()
        step_f6()
        torch.cuda.synchronize()
        out[name]["fp6_operands"] = {
            "linear_ms": ms6, "linear_tops": ops / (ms6 * 1e-3) / 1e12,
            "gemm_us": f6_ms * 1e3, "gemm_tops": ops / (f6_ms * 1e-3) / 1e12,
            "gemm_frac_int8_peak": ops / (f6_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS,
            "gemm_frac_fp6_peak": ops / (f6_ms * 1e-3) / 1e12 / FP6_PEAK_TOPS,
            "rotate_quant_to_fp6_us": rq6 * 1e3,
            "rotate_quant_to_int4_us_same_run": rq4 * 1e3,
            "separate_codes_to_fp6_us": cvt_ms * 1e3,
            "same_output_bits_as_int4_path": bool(torch.equal(Y6.view(torch.int16),
                                                              Ys[0].view(torch.int16)))}
        del lin, Xs, Ys, Y6
        torch.cuda.empty_cache()
    out["square_gemm_8192"] = square_gemm(bd, 8192)
    out["cold_hbm"] = cold_hbm(bd, inputs)
    out["group_wise_scales"] = grouped_scales(bd, inputs, max(20, steps))
    out["gptq_offline_pack"] = gptq_offline(bd, inputs)
    out["dit_mlp_up"] = few_token_line(bd, inputs, "dit_mlp_up", max(50, steps))
    for name, w8 in (("action_stack_mixed", ("o", "down")),):
        info, lins, Xs, rb, step = setup_stack(bd, inputs, w8=w8)
        ms = time_graph(step, max(3, steps // 5), 2)
        M, h, f, T, L = info["M"], info["hidden"], info["ffn"], info["steps"], info["layers"]
        ops = T * L * 2.0 * M * (3 * h * h + h * h + f * h + h * f)
        out[name] = {"layers": L, "M": M, "hidden": h, "ffn": f, "steps": T,
                     "w8a8_linears": list(w8), "linear_calls": T * L * 4, "ms_per_pass": ms,
                     "tops": ops / (ms * 1e-3) / 1e12,
                     "frac_int8_peak": ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS,
                     "offline_pack_s": info["offline_s"], "calibration_s": info["calib_s"]}
        del lins, Xs, step
        torch.cuda.empty_cache()
    out["vendor_int8_gemm_reference"] = vendor_int8_gemm_reference(max(20, steps))
    return out


def vendor_int8_gemm_reference(reps):
    """The vendor library's int8 GEMM (torch._int_mm, int8 operands [M,K] x [K,N] -> int32) on the
    benchmark's GEMM shapes, timed like the library's kernels: a measured reference for what the
    matrix cores reach at these shapes, not part of the W4A4 path (its operands are int8, twice the
    packed int4 bytes, and it has no dequantization epilogue)."""
    torch = _torch()
    g = torch.Generator(device="cuda").manual_seed(0)
    out = {}
    for name, M, N, K in (("stack_qkv", 1600, 3072, 1024), ("stack_o", 1600, 1024, 1024),
                          ("stack_up", 1600, 4096, 1024), ("stack_down", 1600, 1024, 4096),
                          ("prefill_proj", 1024, 16384, 2048), ("longk_down", 1024, 2048, 16384)):
        A = torch.randint(-8, 8, (M, K), generator=g, dtype=torch.int8, device="cuda")
        Bt = torch.randint(-8, 8, (N, K), generator=g, dtype=torch.int8, device="cuda")
        try:
            torch._int_mm(A, Bt.t())
            us = time_kernel_calls([lambda: torch._int_mm(A, Bt.t())], reps) * 1e3
        except RuntimeError as e:  # not every torch build has the int8 product on this device
            out[name] = {"error": str(e)[:200]}
            continue
        tops = 2.0 * M * N * K / (us * 1e-6) / 1e12
        out[name] = {"M": M, "N": N, "K": K, "us": us, "tops": tops,
                     "frac_int8_peak": tops / INT8_PEAK_TOPS}
    return out


if __name__ == "__main__":
    main()
