"""Helpers for GPU-vs-oracle parity: device upload of seeded inputs, one call
through the C ABI, and the tolerance checks.

Tolerances (fixed here, derived from the stated bar):
  fp32 storage: out max|d| <= 1e-5 * max|ref| (normwise over the tensor);
                mass |d| <= 1e-5 * |ref| per row;
                max_score |d| <= 1e-5 * |ref| + 1e-6 * max|ref| per row.
  bf16 storage: out, element by element, |d| <= 2e-2 * rms(V) + 2^-7 * |ref|:
                the first term covers the weights rounded to bf16 before the
                value contraction (2^-9 relative per weight, averaged over the
                keys of a row), the second the output's own rounding to bf16
                (at most 2^-9 relative) with room for the fp32 sums; and the
                mean |d| over the tensor <= 5e-3 * rms(V);
                mass |d| <= 1e-2 * |ref| per row;
                max_score |d| <= 1e-2 * |ref| + 1e-3 * max|ref| per row.
"""
import sys

import numpy as np
import torch

import oracle
from softmax_free_score_amd import attn

TOL = {
    "f32": dict(out=1e-5, mass=1e-5, mx=1e-5, mx_floor=1e-6),
    "bf16": dict(out=2e-2, out_rel=2.0 ** -7, mean=5e-3, mass=1e-2, mx=1e-2, mx_floor=1e-3),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(inp, tied_copy=True):
    """Device tensors (q, k, v, params) holding exactly the oracle's values."""
    dev = torch.device("cuda:0")
    if inp.wl.dtype == "bf16":
        def t(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        q, k, v = t(inp.q_bits), t(inp.k_bits), t(inp.v_bits)
    else:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (inp.q, inp.k, inp.v))
    prm = {n: torch.from_numpy(np.ascontiguousarray(a)).to(dev) for n, a in inp.params().items()}
    return q, k, v, prm


def run_gpu(q, k, v, prm, variant, causal, yat_opts=None, **kw):
    """One call through the C ABI: attn_fwd, or attn_fwd_yat when ``yat_opts``
    = (power, bias_free) is given."""
    if yat_opts is not None:
        out, mass, mx = attn.attn_fwd_yat(q, k, v, prm["b_raw"], prm["eps_raw"],
                                          power=yat_opts[0], bias_free=yat_opts[1],
                                          causal=causal, **kw)
    else:
        out, mass, mx = attn.attn_fwd(q, k, v, variant, causal=causal, **prm, **kw)
    torch.cuda.synchronize()
    return out, mass, mx


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _yat_kw(yat_opts):
    return {} if yat_opts is None else dict(yat_power=yat_opts[0], yat_bias_free=yat_opts[1])


def oracle_full(inp, variant, causal, yat_opts=None):
    q, k, v = inp.f64()
    return oracle.attn_fwd_np(q, k, v, variant, causal=causal, **_yat_kw(yat_opts),
                              **{n: a.astype(np.float64) for n, a in inp.params().items()})


def oracle_rows(inp, variant, causal, rows, yat_opts=None):
    q, k, v = inp.f64()
    return oracle.attn_fwd_c(q, k, v, variant, causal=causal, rows=rows, **_yat_kw(yat_opts),
                             **{n: a.astype(np.float64) for n, a in inp.params().items()})


def check(dtype, got, ref, label="", v_rms=None):
    """got, ref: (out, mass, max_score) as float64 arrays of equal shape.
    v_rms: rms of the values (bf16): the scale of the output bound."""
    tol = TOL[dtype]
    out_g, mass_g, mx_g = got
    out_r, mass_r, mx_r = ref
    assert np.all(np.isfinite(out_g)) and np.all(np.isfinite(mass_g)) and np.all(np.isfinite(mx_g)), \
        f"{label}: non-finite GPU output"
    e_mean = 0.0
    if not out_r.size:
        e_out = 0.0
    elif dtype == "bf16":
        assert v_rms is not None and v_rms > 0, "the bf16 bound needs rms(V)"
        diff = np.abs(out_g - out_r)
        e_out = (diff / (tol["out"] * v_rms + tol["out_rel"] * np.abs(out_r))).max()
        e_mean = diff.mean() / v_rms
        e_abs = diff.max() / v_rms
    else:
        e_out = np.abs(out_g - out_r).max() / (tol["out"] * max(np.abs(out_r).max(), 1e-30))
    e_mass = (np.abs(mass_g - mass_r) / np.maximum(np.abs(mass_r), 1e-30)).max()
    mx_bound = tol["mx"] * np.abs(mx_r) + tol["mx_floor"] * np.abs(mx_r).max()
    e_mx = (np.abs(mx_g - mx_r) / np.maximum(mx_bound, 1e-30)).max()
    extra = f" (max|d| {e_abs:.2e} rms(V))" if dtype == "bf16" and out_r.size else ""
    say(f"  {label}: out err/bound {e_out:.3f}{extra}, mean {e_mean:.2e} rms(V), "
        f"mass rel err {e_mass:.3e} (tol {tol['mass']:.0e}), max_score err/bound {e_mx:.3f}")
    assert e_out <= 1.0, f"{label}: out error outside its bound (ratio {e_out:.3f})"
    if dtype == "bf16":
        assert e_mean <= tol["mean"], f"{label}: mean out error {e_mean:.3e} > 5e-3 rms(V)"
    assert e_mass <= tol["mass"], f"{label}: mass error {e_mass:.3e} > {tol['mass']}"
    assert e_mx <= 1.0, f"{label}: max_score outside bound (ratio {e_mx:.3f})"
    return e_out, e_mass
