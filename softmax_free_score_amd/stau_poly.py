"""Coefficients of the polynomial that the s^tau tile kernels use for
log2(1 + t) / t on 0 <= t <= 1 (t = 2^-|y|, so that t * P(t) = log2(1 + 2^-|y|),
the softplus term of the s^tau map in base-2 units).

The fit is minimax in relative error, by Lawson's algorithm: weighted least
squares on a Chebyshev grid, each point's weight multiplied by its absolute
error after every pass, which converges to the best uniform approximation.
The coefficients are then rounded to fp32 and the error of fp32 Horner
evaluation is measured on a dense grid.

    python -m softmax_free_score_amd.stau_poly        # prints coefficients and error
"""
from __future__ import annotations

import numpy as np

DEGREE = 4


def target(t: np.ndarray) -> np.ndarray:
    """log2(1 + t) / t, with its limit 1/ln 2 at t = 0."""
    t = np.asarray(t, dtype=np.float64)
    safe = np.where(t > 0, t, 1.0)
    return np.where(t > 0, np.log1p(safe) / safe, 1.0) / np.log(2.0)


def fit(degree: int = DEGREE, points: int = 4001, passes: int = 400) -> np.ndarray:
    """Monomial coefficients c_0..c_degree (fp64) of the relative-error minimax fit."""
    x = np.cos(np.pi * (np.arange(points) + 0.5) / points)  # Chebyshev nodes on [-1, 1]
    t = 0.5 * (x + 1.0)
    f = target(t)
    vander = np.vander(t, degree + 1, increasing=True) / f[:, None]  # relative error
    w = np.full(points, 1.0 / points)
    for _ in range(passes):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(vander * sw[:, None], sw, rcond=None)
        err = np.abs(vander @ c - 1.0)
        w = w * err
        w /= w.sum()
    return c


def horner_f32(coef: np.ndarray, t: np.ndarray) -> np.ndarray:
    """The kernels' evaluation order: fp32 fused multiply-adds from the top."""
    c = np.asarray(coef, dtype=np.float32)
    t = np.asarray(t, dtype=np.float32)
    acc = np.full_like(t, c[-1])
    for a in c[-2::-1]:
        acc = (acc.astype(np.float64) * t + np.float64(a)).astype(np.float32)  # one rounding
    return acc


def max_rel_error(coef: np.ndarray, n: int = 1 << 20) -> float:
    t = np.linspace(0.0, 1.0, n + 1)
    return float(np.max(np.abs(horner_f32(coef, t).astype(np.float64) / target(t) - 1.0)))


if __name__ == "__main__":
    c = fit().astype(np.float32)
    for i, a in enumerate(c):
        print(f"c{i} = {float(a)!r}f  // {np.float32(a).view(np.uint32):#010x}")
    print(f"max relative error (fp32 Horner): {max_rel_error(c):.3e}")
