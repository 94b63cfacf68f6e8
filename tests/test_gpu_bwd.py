"""GPU parity of the backward (attn_bwd through the C ABI) against the fp64
oracle ``oracle.attn_bwd_np`` on the same seeded bf16 inputs.

The forward that feeds the backward (its mass and max_score) is the HIP
forward, as a caller would use it; the oracle takes only the seeded inputs.

Tolerances (bf16 storage, fp32 arithmetic):
  dq, dk, dv   max |d| <= 1.5e-2 * S per tensor and mean |d| <= 5e-3 * S_mean,
               with S = max(max |ref|, 2^-12 max |scale|) and S_mean the same
               with means; "scale" is the oracle's error scale (every factor
               by its absolute value, dw - D by |dw| + |D|).  Normally max
               |ref| is the larger; the scale only matters where the exact
               gradient cancels to about 0 (rows with one allowed key, whose q
               and k gradients are 0 up to 1e-9 / kappa in Yat), and there an
               fp32 evaluation can only be as close as a few rounding units of
               the terms that cancel.  The products run on bf16 operands: the weights and
               gradient scores are rounded to bf16 (relative 2^-9 each), as are
               the stored gradients.  Measured: max 2.5-6.5e-3 (1.3-3.3 x 2^-9),
               mean 2.0-3.3e-3; the bounds are 8 x 2^-9 and 2.5 x 2^-9.
  parameters   |d| <= 1e-6 * scale per head: the gradient of b_raw, eps_raw
               or log_tau is a sum of per-pair terms of both signs, each with
               the factor dw - D, evaluated in fp32 from fp32 terms (no bf16
               rounding) and added in fp64 across workgroups; its error is
               measured against the same sum of absolute values (measured
               below 1e-7).
"""
import numpy as np
import pytest
import torch

import oracle
from parity import run_gpu, say, to_device, to_np
from softmax_free_score_amd import attn
from softmax_free_score_amd.workloads import WORKLOADS, make_custom, make_grad_out, make_inputs

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN, TOL_PARAM = 1.5e-2, 5e-3, 1e-6
FLOOR = 2.0 ** -12
PARAMS = {"yat": ("db_raw", "deps_raw"), "stau": ("dlog_tau",), "softmax": ()}


def dout_device(inp):
    g, bits = make_grad_out(inp)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return g.astype(np.float64), t


def gpu_fwd_bwd(inp, variant, causal):
    q, k, v, prm = to_device(inp)
    _, dout = dout_device(inp)
    _, mass, mx = run_gpu(q, k, v, prm, variant, causal)
    g = attn.attn_bwd(q, k, v, dout, variant, mass, mx, causal=causal, **prm)
    torch.cuda.synchronize()
    return g


def oracle_bwd(inp, variant, causal, heads=None, batches=None):
    """The oracle on the whole problem, or on the query heads ``heads`` (all of
    one key/value group) and batches ``batches``."""
    q, k, v = inp.f64()
    g, _ = make_grad_out(inp)
    g = g.astype(np.float64)
    prm = {n: a.astype(np.float64) for n, a in inp.params().items()}
    if heads is not None:
        grp = inp.wl.Hq // inp.wl.Hkv
        hk = heads[0] // grp
        assert list(heads) == list(range(hk * grp, (hk + 1) * grp))
        bs = slice(None) if batches is None else batches
        q, g = q[bs][:, heads], g[bs][:, heads]
        k, v = k[bs][:, hk:hk + 1], v[bs][:, hk:hk + 1]
        prm = {n: a[heads] for n, a in prm.items()}
    return oracle.attn_bwd_np(q, k, v, g, variant, causal=causal, return_abs=True, **prm)


def check_bwd(got, ref, variant, label, params=True):
    errs = {}
    for name in ("dq", "dk", "dv"):
        g, r, a = got[name], ref[name], ref[name + "_abs"]
        assert np.all(np.isfinite(g)), f"{label}: non-finite {name}"
        scale = max(np.abs(r).max(), FLOOR * a.max(), 1e-30)
        e_max = np.abs(g - r).max() / scale
        e_mean = np.abs(g - r).mean() / max(np.abs(r).mean(), FLOOR * a.mean(), 1e-30)
        errs[name] = (e_max, e_mean)
    msg = ", ".join(f"{n} {a:.2e}/{b:.2e}" for n, (a, b) in errs.items())
    perr = {}
    if params:
        for name in PARAMS[variant]:
            g, r, a = got[name], ref[name], ref[name + "_abs"]
            assert np.all(np.isfinite(g)), f"{label}: non-finite {name}"
            perr[name] = (np.abs(g - r) / np.maximum(a, 1e-30)).max()
        msg += "".join(f", {n} {e:.2e}" for n, e in perr.items())
    say(f"  {label}: max/mean rel err {msg}")
    for name, (e_max, e_mean) in errs.items():
        assert e_max <= TOL_MAX, f"{label}: {name} max error {e_max:.3e} > {TOL_MAX}"
        assert e_mean <= TOL_MEAN, f"{label}: {name} mean error {e_mean:.3e} > {TOL_MEAN}"
    for name, e in perr.items():
        assert e <= TOL_PARAM, f"{label}: {name} error {e:.3e} > {TOL_PARAM}"


def grads_np(g):
    return {n: to_np(t) for n, t in g.items() if t is not None}


def case(inp, variant, causal, label):
    w = inp.wl
    say(f"[gpu-bwd] {label} {variant} causal={causal} B{w.B} Hq{w.Hq} Hkv{w.Hkv} Tq{w.Tq} "
        f"Tk{w.Tk} dk{w.dk} dv{w.dv}")
    got = grads_np(gpu_fwd_bwd(inp, variant, causal))
    ref = oracle_bwd(inp, variant, causal)
    check_bwd(got, ref, variant, f"{label}/{variant}")
    return got


SHAPES = [
    # B, Hq, Hkv, Tq, Tk, dk, dv, causal
    (1, 2, 2, 128, 128, 128, 128, True),
    (2, 4, 2, 333, 333, 128, 128, True),
    (1, 2, 1, 200, 517, 64, 128, False),
    (2, 3, 3, 130, 130, 32, 32, True),
    (1, 4, 4, 97, 97, 16, 16, True),
    (1, 2, 2, 150, 260, 128, 64, False),
    (1, 2, 1, 70, 70, 16, 128, True),
    (1, 2, 2, 65, 300, 128, 16, False),
    (1, 4, 1, 257, 257, 64, 32, True),
]


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_shapes(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=11, qk_std=1.5)
    case(inp, variant, causal, "shape")


@pytest.mark.parametrize("variant", ["yat", "softmax"])
def test_bwd_gpt_small(variant):
    case(make_inputs(WORKLOADS["gpt_small"]), variant, True, "gpt_small")


def test_bwd_tied_yat():
    """k := q: every diagonal pair sits on the Yat peak (|q|^2 + b)^2 / eps,
    where the distance term of the gradient must cancel exactly."""
    inp = make_custom(1, 3, 3, 300, 300, 128, 128, "bf16", True, seed=9, qk_std=2.0, tied=True)
    case(inp, "yat", True, "tied")
    inp = make_inputs(WORKLOADS["gpt_small"], tied=True)
    case(inp, "yat", True, "gpt_small_tied")


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", [(1, 2, 1, 1, 1, 64, 64, False), (2, 2, 2, 1, 300, 128, 128, False),
                                   (1, 2, 2, 300, 1, 32, 16, False), (1, 1, 1, 1, 1, 16, 16, True),
                                   (1, 2, 2, 33, 33, 128, 128, True)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bwd_degenerate_sizes(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=12)
    case(inp, variant, causal, "degenerate")


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_bwd_no_query_rows_gives_zero_key_gradients(variant):
    inp = make_custom(1, 2, 1, 4, 100, 64, 32, "bf16", False, seed=13)
    q, k, v, prm = to_device(inp)
    q0 = q[:, :, :0]
    dout = torch.empty((1, 2, 0, 32), dtype=torch.bfloat16, device="cuda:0")
    mass = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda:0")
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    say(f"[gpu-bwd] Tq=0 {variant}")
    attn.attn_bwd(q0, k, v, dout, variant, mass, mass, causal=False, dk=dk, dv=dv, **prm)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_bwd_strided_layout_and_determinism(variant):
    """[B, T, H, d] storage viewed as [B, H, T, d] (row stride H*d) for every
    tensor, and two calls give identical bits."""
    B, Hq, Hkv, T, dk, dv = 2, 4, 2, 190, 64, 64
    inp = make_custom(B, Hq, Hkv, T, T, dk, dv, "bf16", True, seed=14, qk_std=1.5)
    q, k, v, prm = to_device(inp)

    def btHd(t):
        s = torch.empty((t.shape[0], t.shape[2], t.shape[1], t.shape[3]), dtype=t.dtype,
                        device=t.device)
        s.copy_(t.transpose(1, 2))
        return s.transpose(1, 2)

    qs, ks, vs = btHd(q), btHd(k), btHd(v)
    _, dout = dout_device(inp)
    say(f"[gpu-bwd] strided {variant}")
    _, mass, mx = run_gpu(qs, ks, vs, prm, variant, True)
    douts = btHd(dout)   # dout in the [B, T, H, d] layout as well
    g1 = attn.attn_bwd(qs, ks, vs, douts, variant, mass, mx, causal=True, **prm)
    g2 = attn.attn_bwd(qs, ks, vs, douts, variant, mass, mx, causal=True, **prm)
    torch.cuda.synchronize()
    assert g1["dq"].stride() == qs.stride() and g1["dk"].stride() == ks.stride()
    for n in g1:
        if g1[n] is not None:
            a, b = g1[n], g2[n]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), n
    ref = oracle_bwd(inp, variant, True)
    check_bwd(grads_np(g1), ref, variant, f"strided/{variant}")


# ----------------------------------------------------------- full sizes

FULL = [("long_yat", "yat"), ("long_yat", "softmax"), ("stau_gqa", "stau")]


@pytest.mark.parametrize("name,variant", FULL)
def test_bwd_full_size_sampled_heads(name, variant):
    """The full workload on the GPU; the oracle recomputes every gradient of
    one key/value group (all batches), including the parameter gradients of
    its query heads."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    say(f"[gpu-bwd] full {name} {variant} B{wl.B} Hq{wl.Hq} Hkv{wl.Hkv} T{wl.Tq} d{wl.dk}")
    g = gpu_fwd_bwd(inp, variant, wl.causal)
    got = grads_np(g)
    grp = wl.Hq // wl.Hkv
    for hk in (0, wl.Hkv - 1):
        heads = list(range(hk * grp, (hk + 1) * grp))
        say(f"  oracle for kv head {hk} (query heads {heads})")
        ref = oracle_bwd(inp, variant, wl.causal, heads=heads)
        sub = dict(dq=got["dq"][:, heads], dk=got["dk"][:, hk:hk + 1],
                   dv=got["dv"][:, hk:hk + 1])
        for n in PARAMS[variant]:
            sub[n] = got[n][heads]
        check_bwd(sub, ref, variant, f"{name}/{variant}/kv{hk}")
