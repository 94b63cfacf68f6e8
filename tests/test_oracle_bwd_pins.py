"""Pins for the fp64 backward oracle (``oracle.attn_bwd_np``).

The backward has no worked example on the pages; it is pinned to things other
than its own chain-rule algebra:

* central finite differences of the forward oracle in plain C loops
  (``oracle.attn_fwd_c``, itself pinned to the pages), for every input and
  per-head parameter, with and without the causal mask and with grouped
  query heads;
* for softmax, PyTorch's autograd through its own scaled dot-product
  attention (a library routine, fp64 on the CPU);
* closed forms at a zero query, where every branch's weights are uniform or
  known, and invariants (value gradients sum to the output gradients, softmax
  key gradients sum to zero, Yat with b = 0 and eps -> 0 is homogeneous of
  degree 0 in (q, k)).
CPU only."""
import math

import numpy as np
import pytest

import oracle

VARIANTS = ["softmax", "yat", "stau"]
GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "b_raw": "db_raw", "eps_raw": "deps_raw",
           "log_tau": "dlog_tau"}


def make(seed, B, Hq, Hkv, Tq, Tk, dk, dv, scale=1.0):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.standard_normal((B, Hq, Tq, dk)) * scale,
             k=rng.standard_normal((B, Hkv, Tk, dk)) * scale,
             v=rng.standard_normal((B, Hkv, Tk, dv)),
             b_raw=rng.uniform(-1, 1, Hq), eps_raw=rng.uniform(-2, 0.5, Hq),
             log_tau=rng.uniform(-1, 1.5, Hq))
    dout = rng.standard_normal((B, Hq, Tq, dv))
    return x, dout


def loss_c(x, dout, variant, causal):
    out, _, _ = oracle.attn_fwd_c(x["q"], x["k"], x["v"], variant, b_raw=x["b_raw"],
                                  eps_raw=x["eps_raw"], log_tau=x["log_tau"], causal=causal)
    return float(np.sum(dout * out))


def finite_difference(x, dout, variant, causal, name):
    arr = x[name]
    g = np.zeros_like(arr)
    for idx in np.ndindex(arr.shape):
        h = 1e-6 * max(1.0, abs(arr[idx]))
        old = arr[idx]
        arr[idx] = old + h
        lp = loss_c(x, dout, variant, causal)
        arr[idx] = old - h
        lm = loss_c(x, dout, variant, causal)
        arr[idx] = old
        g[idx] = (lp - lm) / (2 * h)
    return g


def bwd(x, dout, variant, causal):
    return oracle.attn_bwd_np(x["q"], x["k"], x["v"], dout, variant, b_raw=x["b_raw"],
                              eps_raw=x["eps_raw"], log_tau=x["log_tau"], causal=causal)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", [(1, 2, 1, 5, 5, 3, 2, True), (2, 4, 2, 4, 4, 3, 2, False),
                                   (1, 2, 2, 3, 6, 4, 3, False), (1, 4, 2, 6, 6, 2, 3, True)])
def test_gradients_match_finite_differences_of_the_c_forward(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    x, dout = make(31, B, Hq, Hkv, Tq, Tk, dk, dv, scale=1.2)
    g = bwd(x, dout, variant, causal)
    names = ["q", "k", "v"] + {"yat": ["b_raw", "eps_raw"], "stau": ["log_tau"],
                                "softmax": []}[variant]
    for name in names:
        fd = finite_difference(x, dout, variant, causal, name)
        got = g[GRAD_OF[name]]
        assert got.shape == fd.shape, name
        np.testing.assert_allclose(got, fd, rtol=0, atol=2e-6 * max(1.0, np.abs(fd).max()),
                                   err_msg=f"{variant} d{name}")
    # the other branches' parameters do not enter: their gradients are zero
    for name in {"b_raw", "eps_raw", "log_tau"} - set(names):
        assert np.all(g[GRAD_OF[name]] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_matches_torch_autograd_sdpa(causal):
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, T, dk, dv = 2, 4, 2, 7, 5, 3
    x, dout = make(32, B, Hq, Hkv, T, T, dk, dv, scale=1.5)
    g = bwd(x, dout, "softmax", causal)
    q = torch.tensor(x["q"], requires_grad=True)
    k = torch.tensor(x["k"], requires_grad=True)
    v = torch.tensor(x["v"], requires_grad=True)
    rep = Hq // Hkv
    out = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(rep, dim=1), v.repeat_interleave(rep, dim=1), is_causal=causal)
    (out * torch.tensor(dout)).sum().backward()
    for name, t in (("dq", q), ("dk", k), ("dv", v)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=name)


def test_zero_query_closed_forms():
    """q = 0: softmax and s^tau weights are uniform, 1/n, whatever the keys.
    Then dL/dq = c * (1/n) sum_j (g_j - mean g) k_j with g_j = dout . v_j and
    c = 1/sqrt(d_k) for softmax, c = tau * sigmoid(0) / phi(0) / sqrt(d_k)
    for s^tau (phi(0) = ln 2 + 1e-6); dL/dv_j = dout / n."""
    B, Hq, Hkv, T, dk, dv = 1, 1, 1, 6, 4, 3
    x, dout = make(33, B, Hq, Hkv, 1, T, dk, dv)
    x["q"][:] = 0.0
    n = T
    kk, vv, do = x["k"][0, 0], x["v"][0, 0], dout[0, 0, 0]
    gj = vv @ do
    base = ((gj - gj.mean())[:, None] * kk).sum(0) / n
    tau = math.log1p(math.exp(x["log_tau"][0])) + 1.0
    phi0 = math.log(2.0) + 1e-6
    for variant, c in (("softmax", 1.0 / math.sqrt(dk)),
                       ("stau", tau * 0.5 / phi0 / math.sqrt(dk))):
        g = bwd(x, dout, variant, False)
        np.testing.assert_allclose(g["dq"][0, 0, 0], c * base, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g["dv"][0, 0], np.tile(do / n, (T, 1)), rtol=1e-12)
        # uniform weights do not depend on tau
        if variant == "stau":
            assert abs(g["dlog_tau"][0]) < 1e-14


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_value_gradients_sum_to_output_gradients(variant, causal):
    """sum_j w_ij = 1 (Yat: mass / (mass + 1e-9)), so sum_j dv_j = sum_i dout_i
    over the query heads of the group."""
    B, Hq, Hkv, T, dk, dv = 2, 4, 2, 9, 4, 5
    x, dout = make(34, B, Hq, Hkv, T, T, dk, dv)
    g = bwd(x, dout, variant, causal)
    row_sum = np.ones((B, Hq, T, 1))
    if variant == "yat":
        _, mass, _ = oracle.attn_fwd_c(x["q"], x["k"], x["v"], "yat", b_raw=x["b_raw"],
                                       eps_raw=x["eps_raw"], causal=causal)
        row_sum = (mass / (mass + 1e-9))[..., None]
    lhs = g["dv"].sum(2)                                       # [B, Hkv, dv]
    rhs = (dout * row_sum).reshape(B, Hkv, Hq // Hkv, T, dv).sum((2, 3))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_key_gradients_sum_to_zero(causal):
    """Adding one vector c to every key shifts each row's scores by q.c / sqrt(d),
    which softmax ignores: the key gradients of each key/value head sum to 0."""
    x, dout = make(35, 2, 4, 2, 8, 8, 5, 3, scale=1.5)
    g = bwd(x, dout, "softmax", causal)
    s = np.abs(g["dk"]).max()
    assert np.abs(g["dk"].sum(2)).max() < 1e-12 * max(1.0, s) * 8


def test_yat_bias_free_is_scale_invariant():
    """b = 0 (b_raw = -inf) and eps -> 0: kappa(lambda q, lambda k) =
    lambda^2 kappa(q, k), so the weights, and L, do not depend on lambda, and
    by Euler's theorem sum q . dq + sum k . dk = 0."""
    x, dout = make(36, 1, 2, 1, 6, 6, 4, 3, scale=1.3)
    x["b_raw"][:] = -np.inf
    x["eps_raw"][:] = -40.0          # eps = 4e-18
    g = bwd(x, dout, "yat", False)
    euler = np.sum(x["q"] * g["dq"]) + np.sum(x["k"] * g["dk"])
    scale = np.sum(np.abs(x["q"] * g["dq"])) + np.sum(np.abs(x["k"] * g["dk"]))
    assert scale > 1e-3
    assert abs(euler) < 1e-9 * scale
    # with a bias the identity breaks (the pin can fail)
    x["b_raw"][:] = 0.5
    g = bwd(x, dout, "yat", False)
    euler = np.sum(x["q"] * g["dq"]) + np.sum(x["k"] * g["dk"])
    assert abs(euler) > 1e-4


def test_single_key_has_no_score_gradient():
    """With one allowed key the softmax and s^tau weight is 1 whatever the
    scores: dq = dk = 0 and dv = dout."""
    x, dout = make(37, 1, 2, 2, 1, 1, 4, 3)
    for variant in ("softmax", "stau"):
        g = bwd(x, dout, variant, False)
        assert np.abs(g["dq"]).max() < 1e-15 and np.abs(g["dk"]).max() < 1e-15
        np.testing.assert_allclose(g["dv"], dout, rtol=1e-14)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_error_scales_bound_the_gradients(variant, causal):
    """The error scales replace every factor by its absolute value and the
    difference dw - D by |dw| + |D|, so by the triangle inequality each one
    bounds its gradient elementwise; and with one allowed key per row the q
    and k gradients vanish while their scales do not."""
    x, dout = make(38, 2, 4, 2, 9, 9, 5, 3, scale=1.3)
    g = oracle.attn_bwd_np(x["q"], x["k"], x["v"], dout, variant, b_raw=x["b_raw"],
                           eps_raw=x["eps_raw"], log_tau=x["log_tau"], causal=causal,
                           return_abs=True)
    for n in ("dq", "dk", "dv", "db_raw", "deps_raw", "dlog_tau"):
        assert np.all(np.abs(g[n]) <= g[n + "_abs"] * (1 + 1e-12) + 1e-300), n
    x, dout = make(39, 1, 2, 2, 4, 1, 5, 3)
    g = oracle.attn_bwd_np(x["q"], x["k"], x["v"], dout, variant, b_raw=x["b_raw"],
                           eps_raw=x["eps_raw"], log_tau=x["log_tau"], return_abs=True)
    # softmax and s^tau: w = 1 exactly; Yat: w = kappa / (kappa + 1e-9), so the
    # gradient is that 1e-9 / (kappa + 1e-9) fraction of the terms
    bound = 1e-4 if variant == "yat" else 1e-12
    assert np.abs(g["dq"]).max() < bound * g["dq_abs"].max()
    assert np.abs(g["dk"]).max() < bound * g["dk_abs"].max()
    assert g["dq_abs"].min() > 0
