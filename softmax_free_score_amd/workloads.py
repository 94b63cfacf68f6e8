"""Seeded synthetic inputs for the attention forward.

This module holds shapes, value distributions and the rounding of draws to
the storage dtype -- nothing of the method's arithmetic.  The tests, the
benchmark and the oracle-side checks all take their inputs from here, so both
sides of a parity check see the same bytes.

The six workloads stand in for the pages' models (a character-level GPT with
6 layers, 4 heads, width 192 and context 128 in "The Kernel Between the
Roles", "The run"; Qwen3-1.7B-class GQA attention for the s^tau post; the
cross-attention shapes T_q != T_k, d_v != d_k of "NNX Scaled Dot-Product
Attention", "Shapes and the three steps"):

=========  ====================================================================
tiny       B=1, H=1, T=64, d=16, fp32, causal; q,k,v ~ N(0,1); b_raw = eps_raw
           = 0; seed 0
gpt_small  B=32, H=6, T=256, d=32, bf16, causal; q,k ~ N(0, 3^2); v ~ N(0,1);
           b_raw, eps_raw ~ N(0, variance 0.5); seed 1
long_yat   B=4, H=16, T=4096, d=128, bf16, causal; q,k ~ N(0, 2^2);
           v ~ N(0,1); b_raw ~ U(-1,1); eps_raw ~ U(-3,0); seed 2
stau_gqa   B=2, Hq=16, Hkv=8, T=2048, d=128, bf16, causal; q,k,v ~ N(0,1);
           log_tau ~ U(-1,2); seed 3
cross      B=8, H=8, Tq=1024, Tk=8192, dk=64, dv=128, bf16, non-causal;
           q,k ~ N(0,1); v ~ U(-1,1); seed 4
decode     B=8, Hq=16, Hkv=8, Tq=1, Tk=8192, d=128, bf16, non-causal: one new
           query row per head against a long key cache (the Qwen3-1.7B-class
           head layout of the s^tau post, at inference); q,k,v ~ N(0,1); seed 5
=========  ====================================================================

Draw order is fixed: q, k, v, b_raw, eps_raw, log_tau, each as fp32 from
``numpy.random.default_rng(seed)``; q, k, v are then rounded to bf16
(round-to-nearest-even) for bf16 workloads.  Parameters a workload does not
specify are drawn anyway from b_raw ~ U(-1,1), eps_raw ~ U(-3,0),
log_tau ~ U(-1,2) so that every branch can run on every workload.  A "tied"
workload sets k := q after rounding (the Yat peak kappa(q,q) is then on the
diagonal).
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int
    dk: int
    dv: int
    dtype: str          # "bf16" or "f32"
    causal: bool
    seed: int
    qk_std: float
    v_dist: str         # "normal" or "uniform"
    b_dist: tuple       # ("normal", std) | ("uniform", lo, hi) | ("zero",)
    eps_dist: tuple
    variants: tuple

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def allowed_pairs(self) -> int:
        """Number of (query, key) pairs the mask allows, over all heads."""
        if self.causal:
            per_head = self.Tq * (self.Tq + 1) // 2
        else:
            per_head = self.Tq * self.Tk
        return self.B * self.Hq * per_head


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 64, 64, 16, 16, "f32", True, 0, 1.0, "normal",
                     ("zero",), ("zero",), ("yat", "softmax", "stau")),
    "gpt_small": Workload("gpt_small", 32, 6, 6, 256, 256, 32, 32, "bf16", True, 1, 3.0,
                          "normal", ("normal", float(np.sqrt(0.5))),
                          ("normal", float(np.sqrt(0.5))), ("yat", "softmax")),
    "long_yat": Workload("long_yat", 4, 16, 16, 4096, 4096, 128, 128, "bf16", True, 2, 2.0,
                         "normal", ("uniform", -1.0, 1.0), ("uniform", -3.0, 0.0),
                         ("yat", "softmax")),
    "stau_gqa": Workload("stau_gqa", 2, 16, 8, 2048, 2048, 128, 128, "bf16", True, 3, 1.0,
                         "normal", ("uniform", -1.0, 1.0), ("uniform", -3.0, 0.0),
                         ("stau",)),
    "cross": Workload("cross", 8, 8, 8, 1024, 8192, 64, 128, "bf16", False, 4, 1.0,
                      "uniform", ("uniform", -1.0, 1.0), ("uniform", -3.0, 0.0),
                      ("softmax", "yat", "stau")),
    "decode": Workload("decode", 8, 16, 8, 1, 8192, 128, 128, "bf16", False, 5, 1.0,
                       "normal", ("uniform", -1.0, 1.0), ("uniform", -3.0, 0.0),
                       ("yat", "softmax", "stau")),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the fp32 values they encode (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """One seeded problem.  ``q``, ``k``, ``v`` hold the stored values as fp32
    (exactly representable in the storage dtype); ``q_bits`` etc. hold bf16
    bit patterns for bf16 workloads (None for fp32)."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    b_raw: np.ndarray
    eps_raw: np.ndarray
    log_tau: np.ndarray
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None

    def f64(self):
        return (self.q.astype(np.float64), self.k.astype(np.float64),
                self.v.astype(np.float64))

    def params(self):
        return dict(b_raw=self.b_raw, eps_raw=self.eps_raw, log_tau=self.log_tau)


def _draw_param(rng, dist, n):
    if dist[0] == "zero":
        return np.zeros(n, np.float32)
    if dist[0] == "normal":
        return (rng.standard_normal(n, dtype=np.float32) * np.float32(dist[1])).astype(np.float32)
    if dist[0] == "uniform":
        return rng.uniform(dist[1], dist[2], n).astype(np.float32)
    raise ValueError(dist)


def make_inputs(wl: Workload, tied: bool = False) -> Inputs:
    rng = np.random.default_rng(wl.seed)
    std = np.float32(wl.qk_std)
    q = rng.standard_normal((wl.B, wl.Hq, wl.Tq, wl.dk), dtype=np.float32) * std
    k = rng.standard_normal((wl.B, wl.Hkv, wl.Tk, wl.dk), dtype=np.float32) * std
    if wl.v_dist == "normal":
        v = rng.standard_normal((wl.B, wl.Hkv, wl.Tk, wl.dv), dtype=np.float32)
    else:
        v = rng.uniform(-1.0, 1.0, (wl.B, wl.Hkv, wl.Tk, wl.dv)).astype(np.float32)
    b_raw = _draw_param(rng, wl.b_dist, wl.Hq)
    eps_raw = _draw_param(rng, wl.eps_dist, wl.Hq)
    log_tau = rng.uniform(-1.0, 2.0, wl.Hq).astype(np.float32)
    qb = kb = vb = None
    if wl.dtype == "bf16":
        qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
        q, k, v = bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb)
    if tied:
        if wl.Tq != wl.Tk or wl.Hq != wl.Hkv:
            raise ValueError("a tied workload needs Tq == Tk and Hq == Hkv")
        k = q.copy()
        kb = None if qb is None else qb.copy()
    return Inputs(wl, q, k, v, b_raw, eps_raw, log_tau, qb, kb, vb)


def make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, dtype="bf16", causal=True, seed=0, qk_std=1.0,
                v_dist="normal", tied=False) -> Inputs:
    """A small seeded problem of any shape (for edge-case tests)."""
    wl = Workload("custom", B, Hq, Hkv, Tq, Tk, dk, dv, dtype, causal, seed, qk_std, v_dist,
                  ("uniform", -1.0, 1.0), ("uniform", -3.0, 0.0), ("yat", "softmax", "stau"))
    return make_inputs(wl, tied=tied)


def make_grad_out(inp: Inputs, seed_offset: int = 1000):
    """The output gradient dL/dout for a backward on ``inp``: N(0, 1) of the
    output's shape [B, Hq, Tq, dv], drawn from default_rng(seed + seed_offset)
    and rounded to the storage dtype like q, k, v.  Returns (values as fp32,
    bf16 bit patterns or None)."""
    wl = inp.wl
    rng = np.random.default_rng(wl.seed + seed_offset)
    g = rng.standard_normal((wl.B, wl.Hq, wl.Tq, wl.dv), dtype=np.float32)
    if wl.dtype == "bf16":
        bits = bf16_bits(g)
        return bf16_bits_to_f32(bits), bits
    return g, None
