"""Fp64 CPU oracle for the attention forward and backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it, and
it shares no code with the HIP path: it neither imports ``softmax_free_score_amd``
nor reads its headers or constants.

Two independent fp64 implementations of the same closed form live here:

* ``attn_fwd_c`` -- plain C loops (``attn_oracle.c``), OpenMP over query rows;
  also the CPU baseline that the benchmark times.
* ``attn_fwd_np`` -- a numpy transcription (library matmuls as the two
  contraction steps, everything else elementwise in the pages' order).

What each computes, with the pages it follows:

* Yat ("Softmax-Free Attention in JAX/Flax NNX", "One module, two
  compatibility functions"; "The Kernel Between the Roles", "What the
  exponential was hired to do"): dots = q.k, d2 = |q|^2 + |k|^2 - 2 dots,
  b = softplus(b_raw), eps = softplus(eps_raw) per head,
  kappa = (dots + b)^2 / (max(d2, 0) + eps), kappa = 0 where masked,
  mass = sum_j kappa, w = kappa / (mass + 1e-9), out = w @ v.
* softmax ("NNX Scaled Dot-Product Attention", "Shapes and the three steps",
  "Mask before softmax"): s = q.k / sqrt(d_k), blocked scores -inf, softmax
  over keys after subtracting the row maximum, out = w @ v.
* s^tau ("s^tau" forum post, core formula): s = q.k / sqrt(d_k),
  phi = softplus(s) + 1e-6, tau = softplus(log_tau) + 1 per head,
  w = phi^tau / sum phi^tau over allowed keys, out = w @ v.

* ``attn_bwd_np`` -- gradients of L = sum(dout * out) with respect to q, k, v
  and the per-head parameters (b_raw, eps_raw, log_tau) of the three maps
  above: the chain rule through their closed forms, written out in fp64
  (the pages train these models by automatic differentiation and print no
  backward formulas; the derivation is in the function's docstring).

Readings of points the pages leave open (GQA mapping h -> h // (Hq/Hkv),
causal j <= i with Tq == Tk, masked keys weigh exactly 0 in all branches,
mass and max_score per branch) are those stated in ``attn_oracle.c``.

Parity status: every function here is pinned by tests in
``tests/test_oracle_pins.py`` (worked examples printed on the pages, closed
forms, invariants and brute force).  The mass and max_score conventions for
softmax and s^tau and the GQA mapping are conventions chosen here, pinned
only by brute force and self-consistency (parity unpinned by the pages).
``attn_bwd_np`` is pinned in ``tests/test_oracle_bwd_pins.py`` to central
finite differences of the C forward, to PyTorch autograd through its own
scaled dot-product attention (softmax), and to closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

SOFTMAX, YAT, STAU = 0, 1, 2
VARIANTS = {"softmax": SOFTMAX, "yat": YAT, "stau": STAU}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, IEEE arithmetic, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-shared", "-fPIC",
           _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("SFS_ORACLE_LIBRARY")   # another build of the same source
        if not path:
            path = _LIB_PATH
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build()
        lib = ctypes.CDLL(path)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_attn_fwd.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, i64,
                                        i64, i64, d, d, d, d, d, d,
                                        ctypes.POINTER(i64), i64, d, d, d]
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_fwd_yat.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, i64,
                                            d, d, d, d, d, ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(i64), i64, d, d, d]
        lib.oracle_attn_fwd_yat.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _dptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _as_f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def attn_fwd_c(q, k, v, variant, b_raw=None, eps_raw=None, log_tau=None, causal=False,
               rows=None, yat_power=1, yat_bias_free=False):
    """C oracle.  q [B,Hq,Tq,dk], k [B,Hkv,Tk,dk], v [B,Hkv,Tk,dv] (any float
    dtype; upcast exactly to fp64).  ``rows`` optionally lists flat row ids
    (b*Hq + h)*Tq + i to evaluate.  Returns (out, mass, max_score); with
    ``rows`` they are [n_rows, dv], [n_rows], [n_rows], otherwise shaped
    [B,Hq,Tq,dv] and [B,Hq,Tq]."""
    variant = VARIANTS.get(variant, variant)
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, Tq, dk = q.shape
    _, Hkv, Tk, dv = v.shape
    params = [_as_f64(p) for p in (b_raw, eps_raw, log_tau)]
    if rows is None:
        n = B * Hq * Tq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.size
    out = np.empty((n, dv), np.float64)
    mass = np.empty(n, np.float64)
    mx = np.empty(n, np.float64)
    rows_p = None if rows_arr is None else rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    if variant == YAT and (yat_power != 1 or yat_bias_free):
        rc = _load().oracle_attn_fwd_yat(
            int(bool(causal)), B, Hq, Hkv, Tq, Tk, dk, dv, _dptr(q), _dptr(k), _dptr(v),
            _dptr(params[0]), _dptr(params[1]), int(yat_power), int(bool(yat_bias_free)),
            rows_p, n, _dptr(out), _dptr(mass), _dptr(mx))
    else:
        rc = _load().oracle_attn_fwd(
            int(variant), int(bool(causal)), B, Hq, Hkv, Tq, Tk, dk, dv, _dptr(q), _dptr(k),
            _dptr(v), *[_dptr(p) for p in params], rows_p, n, _dptr(out), _dptr(mass), _dptr(mx))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd rejected its arguments (code {rc})")
    if rows is None:
        return out.reshape(B, Hq, Tq, dv), mass.reshape(B, Hq, Tq), mx.reshape(B, Hq, Tq)
    return out, mass, mx


def softplus(x):
    """log(1 + e^x) without overflow in either tail; softplus(0) = ln 2."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def attn_fwd_np(q, k, v, variant, b_raw=None, eps_raw=None, log_tau=None, causal=False,
                yat_power=1, yat_bias_free=False):
    """numpy fp64 oracle; same contract as ``attn_fwd_c`` without ``rows``.

    Yat options ("The Kernel Between the Roles", "The run"): numerator
    (q.k + b)^(2 yat_power); b = 0 exactly when ``yat_bias_free``."""
    variant = VARIANTS.get(variant, variant)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, Hq, Tq, dk = q.shape
    _, Hkv, Tk, dv = v.shape
    if Hq % Hkv or (causal and Tq != Tk):
        raise ValueError("bad shape")
    g = Hq // Hkv
    # query head h reads key/value head h // g
    kh = np.repeat(k, g, axis=1)
    vh = np.repeat(v, g, axis=1)
    dots = q @ np.swapaxes(kh, -1, -2)  # (B,Hq,Tq,Tk)
    allowed = np.ones((Tq, Tk), bool)
    if causal:
        allowed = np.tril(allowed)
    if variant == YAT:
        bias = 0.0 if yat_bias_free else softplus(b_raw)[None, :, None, None]
        eps = softplus(eps_raw)[None, :, None, None]
        d2 = (np.sum(q * q, -1, keepdims=True) + np.swapaxes(np.sum(kh * kh, -1, keepdims=True), -1, -2)
              - 2.0 * dots)
        kappa = ((dots + bias) ** 2) ** int(yat_power) / (np.maximum(d2, 0.0) + eps)
        kappa = np.where(allowed, kappa, 0.0)
        mass = kappa.sum(-1)
        w = kappa / (mass[..., None] + 1e-9)
        max_score = np.where(allowed, kappa, -np.inf).max(-1)
    elif variant == SOFTMAX:
        s = np.where(allowed, dots / np.sqrt(dk), -np.inf)
        m = s.max(-1, keepdims=True)
        e = np.exp(s - m)
        mass = e.sum(-1)
        w = e / mass[..., None]
        max_score = m[..., 0]
    elif variant == STAU:
        s = dots / np.sqrt(dk)
        tau = (softplus(log_tau) + 1.0)[None, :, None, None]
        u = np.where(allowed, (softplus(s) + 1e-6) ** tau, 0.0)
        mass = u.sum(-1)
        w = u / mass[..., None]
        max_score = np.where(allowed, s, -np.inf).max(-1)
    else:
        raise ValueError(f"unknown variant {variant}")
    return w @ vh, mass, max_score


def telemetry_np(q, k, variant, b_raw=None, eps_raw=None, log_tau=None, causal=False,
                 sparsity_threshold=1e-6):
    """Attention telemetry, fp64 (numpy).  Returns (row_entropy, row_sparsity,
    tau_star): row_entropy and row_sparsity [B,Hq,Tq], tau_star [Hq].

    * row_entropy: the entropy of the row's weights over its allowed keys,
      -sum w ln w, divided by ln(n) for n allowed keys (0 for n = 1): 0 for a
      row that puts everything on one key, 1 for uniform weights ("The Kernel
      Between the Roles", "The run").
    * row_sparsity: the fraction of allowed keys whose weight is below the
      threshold (the s^tau post's sparsity, weights < 1e-6).
    * tau_star: per query head, Cov(s, ln phi(s)) / Var(ln phi(s)) over every
      allowed (query, key) pair of the head, s = q.k / sqrt(d_k),
      phi = softplus(s) + 1e-6 (the s^tau post's closed form for the tau that
      makes s^tau closest to softmax); NaN when Var = 0.

    The weights are those of the forward for ``variant`` (Yat: kappa /
    (mass + 1e-9); softmax; s^tau), computed here from q and k."""
    variant = VARIANTS.get(variant, variant)
    q, k = (np.asarray(a, dtype=np.float64) for a in (q, k))
    B, Hq, Tq, dk = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    kh = np.repeat(k, g, axis=1)
    dots = q @ np.swapaxes(kh, -1, -2)
    allowed = np.tril(np.ones((Tq, Tk), bool)) if causal else np.ones((Tq, Tk), bool)
    allowed = np.broadcast_to(allowed, dots.shape)
    eye = np.eye(Tk)
    if variant == YAT:
        # the forward's weights, read off with V = identity
        w = attn_fwd_np(q, k, np.broadcast_to(eye, (B, Hkv, Tk, Tk)), YAT, b_raw, eps_raw,
                        causal=causal)[0]
    else:
        w = attn_fwd_np(q, k, np.broadcast_to(eye, (B, Hkv, Tk, Tk)), variant, b_raw, eps_raw,
                        log_tau, causal=causal)[0]
    n = allowed.sum(-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        wlnw = np.where(allowed & (w > 0), w * np.log(np.where(w > 0, w, 1.0)), 0.0)
    ent = -wlnw.sum(-1)
    row_entropy = np.where(n > 1, ent / np.log(np.maximum(n, 2)), 0.0)
    row_sparsity = np.where(allowed, w < sparsity_threshold, False).sum(-1) / n
    s = dots / np.sqrt(dk)
    L = np.log(softplus(s) + 1e-6)
    tau = np.empty(Hq)
    for h in range(Hq):
        m = allowed[:, h]
        sv, lv = s[:, h][m], L[:, h][m]
        cov = np.mean(sv * lv) - np.mean(sv) * np.mean(lv)
        var = np.mean(lv * lv) - np.mean(lv) ** 2
        tau[h] = cov / var if var > 0 else np.nan
    return row_entropy, row_sparsity, tau


def sigmoid(x):
    """1 / (1 + e^-x), the derivative of softplus, without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, 1.0 / (1.0 + np.exp(-np.abs(x))), np.exp(-np.abs(x)) / (1.0 + np.exp(-np.abs(x))))


def _bwd_forward(q, k, v, dout, variant, b_raw, eps_raw, log_tau, causal):
    """The forward quantities the backward needs (fp64): per query head the
    repeated keys and values, q.k, the mask, the unnormalised weights u, the
    normaliser Z, w = u / Z, dw = dout . v and D = dout . out, plus the
    branch's own arrays (Yat: b, den; s^tau: s, tau, phi)."""
    variant = VARIANTS.get(variant, variant)
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    B, Hq, Tq, dk = q.shape
    _, Hkv, Tk, dv = v.shape
    g = Hq // Hkv
    f = dict(variant=variant, q=q, dout=dout, g=g, shape=(B, Hq, Hkv, Tq, Tk, dk, dv))
    f["kh"] = kh = np.repeat(k, g, axis=1)
    vh = np.repeat(v, g, axis=1)
    f["dots"] = dots = q @ np.swapaxes(kh, -1, -2)
    allowed = np.tril(np.ones((Tq, Tk), bool)) if causal else np.ones((Tq, Tk), bool)
    f["allowed"] = allowed = np.broadcast_to(allowed, dots.shape)
    if variant == YAT:
        f["bias"] = bias = softplus(b_raw)[None, :, None, None]
        eps = softplus(eps_raw)[None, :, None, None]
        d2 = (np.sum(q * q, -1, keepdims=True) + np.swapaxes(np.sum(kh * kh, -1, keepdims=True), -1, -2)
              - 2.0 * dots)
        f["den"] = den = np.maximum(d2, 0.0) + eps
        u = np.where(allowed, (dots + bias) ** 2 / den, 0.0)
        Z = u.sum(-1, keepdims=True) + 1e-9
    elif variant == SOFTMAX:
        s = np.where(allowed, dots / np.sqrt(dk), -np.inf)
        u = np.exp(s - s.max(-1, keepdims=True))
        Z = u.sum(-1, keepdims=True)
    else:
        f["s"] = s = dots / np.sqrt(dk)
        f["tau"] = tau = (softplus(log_tau) + 1.0)[None, :, None, None]
        f["phi"] = phi = softplus(s) + 1e-6
        u = np.where(allowed, phi ** tau, 0.0)
        Z = u.sum(-1, keepdims=True)
    f["u"], f["Z"] = u, Z
    f["w"] = w = u / Z
    out = w @ vh
    f["dw"] = dout @ np.swapaxes(vh, -1, -2)
    f["D"] = np.sum(dout * out, -1, keepdims=True)
    return f


def attn_bwd_np(q, k, v, dout, variant, b_raw=None, eps_raw=None, log_tau=None, causal=False,
                return_abs=False):
    """Gradients of L = sum(dout * out) for the forward of ``attn_fwd_np``
    (fp64, numpy).  Returns dict(dq, dk, dv, db_raw, deps_raw, dlog_tau) with
    the shapes of the inputs (the parameter gradients of the other branches are
    zeros).  K/V gradients sum over the query heads that share a key/value head.
    With ``return_abs`` the dict also holds the error scales of
    ``attn_bwd_scales_np`` under the names dq_abs, dk_abs, ..., dlog_tau_abs.

    The chain rule, written out for the closed forms of the forward:
      out_i = sum_j w_ij v_j,  w_ij = u_ij / Z_i,  Z_i = sum_j u_ij (+ 1e-9, Yat)
      dv_j  = sum_i w_ij dout_i;   dw_ij = dout_i . v_j
      du_ij = (dw_ij - D_i) / Z_i,  D_i = sum_j w_ij dw_ij = dout_i . out_i
      softmax: u = e^(s - m), s = q.k / sqrt(d_k):  ds = du u
      s^tau:   u = phi^tau, phi = softplus(s) + 1e-6:  ds = du tau u sigmoid(s) / phi,
               dtau = sum du u ln phi, tau = softplus(log_tau) + 1
      Yat:     u = kappa = (q.k + b)^2 / (|q - k|^2 + eps) (the clamp max(d2, 0)
               is inactive in exact arithmetic):
               dkappa/dq = [2 (q.k + b) k - 2 kappa (q - k)] / den,
               dkappa/dk = [2 (q.k + b) q - 2 kappa (k - q)] / den,
               dkappa/db = 2 (q.k + b) / den,  dkappa/deps = -kappa / den,
               b = softplus(b_raw), eps = softplus(eps_raw), d softplus = sigmoid."""
    f = _bwd_forward(q, k, v, dout, variant, b_raw, eps_raw, log_tau, causal)
    variant, q, dout, kh, dots, allowed = (f[n] for n in ("variant", "q", "dout", "kh", "dots",
                                                         "allowed"))
    B, Hq, Hkv, Tq, Tk, dk, dv = f["shape"]
    g = f["g"]
    u, Z, w = f["u"], f["Z"], f["w"]
    zeros_h = np.zeros(Hq)
    db_raw, deps_raw, dlog_tau = zeros_h.copy(), zeros_h.copy(), zeros_h.copy()
    dvh = np.swapaxes(w, -1, -2) @ dout                     # per query head
    du = np.where(allowed, (f["dw"] - f["D"]) / Z, 0.0)
    if variant == YAT:
        bias, den = f["bias"], f["den"]
        A = np.where(allowed, 2.0 * du * (dots + bias) / den, 0.0)   # coefficient of k in dq
        Bc = np.where(allowed, 2.0 * du * u / den, 0.0)               # coefficient of (q - k)
        dq = (A + Bc) @ kh - Bc.sum(-1, keepdims=True) * q
        dkh = np.swapaxes(A + Bc, -1, -2) @ q - np.swapaxes(Bc.sum(-2, keepdims=True), -1, -2) * kh
        db_raw = sigmoid(b_raw) * np.sum(A, axis=(0, 2, 3))          # dkappa/db = A / du
        deps_raw = sigmoid(eps_raw) * np.sum(du * np.where(allowed, -u / den, 0.0), axis=(0, 2, 3))
    else:
        if variant == SOFTMAX:
            ds = du * u
        else:
            s, tau, phi = f["s"], f["tau"], f["phi"]
            ds = np.where(allowed, du * tau * u * sigmoid(s) / phi, 0.0)
            dlog_tau = sigmoid(log_tau) * np.sum(np.where(allowed, du * u * np.log(phi), 0.0),
                                                 axis=(0, 2, 3))
        ds = ds / np.sqrt(dk)
        dq = ds @ kh
        dkh = np.swapaxes(ds, -1, -2) @ q
    dk_out = dkh.reshape(B, Hkv, g, Tk, dk).sum(2)
    dv_out = dvh.reshape(B, Hkv, g, Tk, dv).sum(2)
    res = dict(dq=dq, dk=dk_out, dv=dv_out, db_raw=db_raw, deps_raw=deps_raw, dlog_tau=dlog_tau)
    if return_abs:
        sc = attn_bwd_scales_np(q, k, v, dout, variant, b_raw, eps_raw, log_tau, causal, _f=f)
        res.update({n + "_abs": a for n, a in sc.items()})
    return res


def attn_bwd_scales_np(q, k, v, dout, variant, b_raw=None, eps_raw=None, log_tau=None,
                       causal=False, _f=None):
    """Error scales for tests of a finite-precision backward (not gradients):
    the sums of ``attn_bwd_np`` with du_ij = (dw_ij - D_i) / Z_i replaced by
    (|dw_ij| + |D_i|) / Z_i and every other factor by its absolute value.  A
    floating-point evaluation that forms dw - D, or rounds any factor, errs by
    a multiple of the rounding unit times this scale; it is the only scale
    left where the two terms cancel (e.g. a row with one allowed key, whose
    exact q and k gradients are 0)."""
    f = _f if _f is not None else _bwd_forward(q, k, v, dout, variant, b_raw, eps_raw, log_tau,
                                               causal)
    variant, q, dout, kh, dots, allowed = (f[n] for n in ("variant", "q", "dout", "kh", "dots",
                                                         "allowed"))
    B, Hq, Hkv, Tq, Tk, dk, dv = f["shape"]
    g = f["g"]
    u, Z, w = f["u"], f["Z"], f["w"]
    zeros_h = np.zeros(Hq)
    db, de, dt = zeros_h.copy(), zeros_h.copy(), zeros_h.copy()
    ma = np.where(allowed, (np.abs(f["dw"]) + np.abs(f["D"])) / Z, 0.0)
    qa, ka = np.abs(q), np.abs(kh)
    if variant == YAT:
        bias, den = f["bias"], f["den"]
        A = np.where(allowed, 2.0 * ma * np.abs(dots + bias) / den, 0.0)
        Bc = np.where(allowed, 2.0 * ma * u / den, 0.0)
        dq = (A + Bc) @ ka + Bc.sum(-1, keepdims=True) * qa
        dkh = np.swapaxes(A + Bc, -1, -2) @ qa + np.swapaxes(Bc.sum(-2, keepdims=True), -1, -2) * ka
        db = sigmoid(b_raw) * np.sum(A, axis=(0, 2, 3))
        de = sigmoid(eps_raw) * np.sum(Bc, axis=(0, 2, 3)) / 2.0
    else:
        if variant == SOFTMAX:
            ds = ma * u
        else:
            s, tau, phi = f["s"], f["tau"], f["phi"]
            ds = np.where(allowed, ma * tau * u * sigmoid(s) / phi, 0.0)
            dt = sigmoid(log_tau) * np.sum(np.where(allowed, ma * u * np.abs(np.log(phi)), 0.0),
                                           axis=(0, 2, 3))
        ds = ds / np.sqrt(dk)
        dq = ds @ ka
        dkh = np.swapaxes(ds, -1, -2) @ qa
    dvh = np.swapaxes(w, -1, -2) @ np.abs(dout)
    return dict(dq=dq, dk=dkh.reshape(B, Hkv, g, Tk, dk).sum(2),
                dv=dvh.reshape(B, Hkv, g, Tk, dv).sum(2), db_raw=db, deps_raw=de, dlog_tau=dt)
