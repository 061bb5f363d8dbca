"""Seeded synthetic inputs for the W4A4 linear workloads.

This module only draws numbers: activation and weight tensors with the shapes, value distributions
and outlier structure of the five workloads below. It holds none of the quantizer's arithmetic (no
permutation, rotation, scale or rounding to codes), so the GPU path and the CPU oracle can both be
fed from it. Every draw comes from numpy's PCG64 generator with a fixed seed and a fixed draw order;
values are drawn in fp64 and stored in the workload's dtype (round to nearest even).

Workloads (sizes and distributions as the benchmark suite states them):
  linear_small   X fp32 [16, 256] N(0,1), 4 channels x20, one draw per step (8 steps);
                 W fp32 [256, 256] N(0, 0.02^2), 2 rows x10; block 64; per-step scales.
  dit_mlp_up     X fp16 [50, 1024] per step t=0..7 N(0, s_t^2), s_t = 3.0 - 2.5 t / 7, 1% channels x15,
                 plus 10 calibration draws per step; W fp16 [4096, 1024] N(0, 0.02^2); block 128.
  prefill_proj   X fp16 [1024, 2048] Laplace(0, 1), 0.5% channels x30; W fp16 [16384, 2048]
                 N(0, 0.015^2), 1% rows x8; block 128; per-token scales.
  longk_down     X fp16 [1024, 16384] GELU(N(0,1)), 0.2% channels x40; W fp16 [2048, 16384]
                 N(0, 0.008^2); block 128; per-token scales.
  action_stack   16 layers of {QKV 1024->3072, O 1024->1024, up 1024->4096, down 4096->1024},
                 W fp16 N(0, 0.02^2); per step X fp16 [1600, 1024] N(0,1), 1% channels x20, and 10
                 calibration draws per step; block 128; per-step scales.
The standard deviation reading is used for "N(0, 0.02)". Outlier counts are round(fraction * size),
chosen without replacement and kept fixed across steps and calibration draws.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

SEEDS = {"linear_small": 0, "dit_mlp_up": 1, "prefill_proj": 2, "longk_down": 3, "action_stack": 4}

LINEAR_WORKLOADS = {
    # name: M, K, N, block, x dtype, mode, steps
    "linear_small": dict(M=16, K=256, N=256, block=64, xdtype=np.float32, mode="per_step", steps=8),
    "dit_mlp_up": dict(M=50, K=1024, N=4096, block=128, xdtype=np.float16, mode="per_step", steps=8),
    "prefill_proj": dict(M=1024, K=2048, N=16384, block=128, xdtype=np.float16, mode="per_token",
                         steps=1),
    "longk_down": dict(M=1024, K=16384, N=2048, block=128, xdtype=np.float16, mode="per_token",
                       steps=1),
}

STACK = dict(layers=16, M=1600, hidden=1024, ffn=4096, block=128, steps=8, calib=10)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _count(frac: float, n: int) -> int:
    return max(1, int(round(frac * n)))


def _gelu_normal(rng, shape):
    z = rng.standard_normal(shape)
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def linear_inputs(name: str, M: int | None = None, K: int | None = None, N: int | None = None,
                  seed: int | None = None, calib: int | None = None) -> dict:
    """Draw one linear workload. Sizes may be overridden (parity cases at reduced size keep the
    recipe and scale the outlier counts with the new sizes)."""
    cfg = dict(LINEAR_WORKLOADS[name])
    M = cfg["M"] if M is None else M
    K = cfg["K"] if K is None else K
    N = cfg["N"] if N is None else N
    rng = _rng(SEEDS[name] if seed is None else seed)
    xdt = cfg["xdtype"]
    out = dict(name=name, M=M, K=K, N=N, block=cfg["block"], mode=cfg["mode"], steps=cfg["steps"],
               xdtype=xdt)
    if name == "linear_small":
        W = rng.normal(0.0, 0.02, (N, K))
        W[rng.choice(N, min(2, N), replace=False)] *= 10.0
        ch = rng.choice(K, min(4, K), replace=False)
        Xs = []
        for _ in range(cfg["steps"]):
            X = rng.standard_normal((M, K))
            X[:, ch] *= 20.0
            Xs.append(X.astype(xdt))
        out.update(W=W.astype(np.float32), X_steps=Xs, X_calib=[[x] for x in Xs])
    elif name == "dit_mlp_up":
        W = rng.normal(0.0, 0.02, (N, K))
        ch = rng.choice(K, _count(0.01, K), replace=False)
        nc = 10 if calib is None else calib
        Xs, Xc = [], []
        for t in range(cfg["steps"]):
            sig = 3.0 - 2.5 * t / 7.0
            X = rng.normal(0.0, sig, (M, K))
            X[:, ch] *= 15.0
            Xs.append(X.astype(xdt))
            cal = []
            for _ in range(nc):
                C = rng.normal(0.0, sig, (M, K))
                C[:, ch] *= 15.0
                cal.append(C.astype(xdt))
            Xc.append(cal)
        out.update(W=W.astype(np.float16), X_steps=Xs, X_calib=Xc)
    elif name == "prefill_proj":
        W = rng.normal(0.0, 0.015, (N, K))
        W[rng.choice(N, _count(0.01, N), replace=False)] *= 8.0
        X = rng.laplace(0.0, 1.0, (M, K))
        X[:, rng.choice(K, _count(0.005, K), replace=False)] *= 30.0
        out.update(W=W.astype(np.float16), X=X.astype(xdt))
    elif name == "longk_down":
        W = rng.normal(0.0, 0.008, (N, K))
        X = _gelu_normal(rng, (M, K))
        X[:, rng.choice(K, _count(0.002, K), replace=False)] *= 40.0
        out.update(W=W.astype(np.float16), X=X.astype(xdt))
    else:
        raise KeyError(name)
    return out


def stack_weights(layers: int | None = None, hidden: int | None = None, ffn: int | None = None,
                  seed: int | None = None) -> list:
    """Weights of the synthetic action-head stack: per layer fp16 qkv [3h, h], o [h, h],
    up [f, h], down [h, f], all N(0, 0.02^2)."""
    L = STACK["layers"] if layers is None else layers
    h = STACK["hidden"] if hidden is None else hidden
    f = STACK["ffn"] if ffn is None else ffn
    rng = _rng(SEEDS["action_stack"] if seed is None else seed)
    out = []
    for _ in range(L):
        lw = {}
        for nm, shp in (("qkv", (3 * h, h)), ("o", (h, h)), ("up", (f, h)), ("down", (h, f))):
            lw[nm] = rng.normal(0.0, 0.02, shp).astype(np.float16)
        out.append(lw)
    return out


def stack_activations(M: int | None = None, hidden: int | None = None, steps: int | None = None,
                      calib: int | None = None, seed: int | None = None) -> dict:
    """Stack inputs: per step one fp16 [M, h] draw N(0,1) with 1% channels x20, plus `calib`
    calibration draws per step from the same distribution."""
    M = STACK["M"] if M is None else M
    h = STACK["hidden"] if hidden is None else hidden
    T = STACK["steps"] if steps is None else steps
    nc = STACK["calib"] if calib is None else calib
    rng = _rng(1000 + (SEEDS["action_stack"] if seed is None else seed))
    ch = rng.choice(h, _count(0.01, h), replace=False)

    def draw():
        X = rng.standard_normal((M, h))
        X[:, ch] *= 20.0
        return X.astype(np.float16)

    X_steps = [draw() for _ in range(T)]
    X_calib = [[draw() for _ in range(nc)] for _ in range(T)]
    return dict(X_steps=X_steps, X_calib=X_calib, outlier_channels=ch)


def random_packed(rows: int, K: int, seed: int) -> np.ndarray:
    """Uniform random bytes uint8 [rows, K/2]: every byte is a valid pair of int4 codes, so these are
    packed int4 operands covering the whole code range, for integer-GEMM cases."""
    return _rng(seed).integers(0, 256, size=(rows, K // 2), dtype=np.uint8)


def constant_packed(rows: int, K: int, byte: int) -> np.ndarray:
    return np.full((rows, K // 2), byte, np.uint8)


def random_scales(n: int, seed: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    return _rng(seed).uniform(lo, hi, n).astype(np.float32)
