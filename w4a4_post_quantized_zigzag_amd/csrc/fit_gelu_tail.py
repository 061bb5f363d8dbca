"""Coefficients of the normal-tail polynomial used by the GEMM's GELU epilogue (k_gemm.hip).

GELU(v) = v * Phi(v) with Phi the standard normal CDF. For w = |v|, Phi(-w) = 0.5 erfc(w / sqrt 2)
= exp(-w^2 / 2) * g(w), and g(w) = 0.5 erfc(w / sqrt 2) exp(w^2 / 2) is smooth and slowly varying
(0.5 at w = 0, about 1 / (w sqrt(2 pi)) for large w). The kernel evaluates g as a degree-7
polynomial in t = 1 / (1 + 0.3 w) on w in [0, 6] (w is clamped to 6: beyond it Phi(-w) < 1e-9, far
below fp16 resolution of GELU), then Phi(v) = 1 - exp(-v^2/2) g for v >= 0 and exp(-v^2/2) g
otherwise. This script fits the polynomial by relative least squares on Chebyshev nodes of [0, 6]
and prints its coefficients (lowest degree first) and the maximum relative error of g (about
1.6e-7). Run: python fit_gelu_tail.py
"""
import numpy as np
from scipy.special import erfc

WMAX, A, DEG, NODES = 6.0, 0.3, 7, 4000


def g(w):
    return 0.5 * erfc(w / np.sqrt(2.0)) * np.exp(w * w / 2.0)


def fit():
    k = np.arange(NODES)
    w = 0.5 * WMAX * (1.0 - np.cos(np.pi * (k + 0.5) / NODES))
    t = 1.0 / (1.0 + A * w)
    y = g(w)
    basis = np.vander(t, DEG + 1, increasing=True) / y[:, None]
    c, *_ = np.linalg.lstsq(basis, np.ones(NODES), rcond=None)
    return c


if __name__ == "__main__":
    c = fit().astype(np.float32)
    w = np.linspace(0.0, WMAX, 200001)
    rel = np.polynomial.polynomial.polyval(1.0 / (1.0 + A * w), c.astype(np.float64)) / g(w) - 1.0
    print("coefficients:", ", ".join(f"{v:.9g}f" for v in c))
    print(f"max relative error of g on [0, {WMAX}]: {np.max(np.abs(rel)):.2e}")
