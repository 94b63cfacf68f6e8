"""Pins for the fp64 oracle: values the pages print, closed forms, invariants
and brute force.  Each pin is checked against both oracle implementations
(plain C loops and the numpy transcription).  CPU only."""
import math

import numpy as np
import pytest

import oracle
from conftest import load_golden

IMPLS = ["c", "np"]
LN2 = math.log(2.0)


def run(impl, q, k, v, variant, causal=False, b_raw=None, eps_raw=None, log_tau=None,
        yat_power=1, yat_bias_free=False):
    """Oracle on single-head 2-D inputs (Tq x dk, Tk x dk, Tk x dv) or 4-D."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    two_d = q.ndim == 2
    if two_d:
        q, k, v = q[None, None], k[None, None], v[None, None]
    Hq = q.shape[1]
    b_raw = np.zeros(Hq) if b_raw is None else np.broadcast_to(np.asarray(b_raw, float), (Hq,))
    eps_raw = np.zeros(Hq) if eps_raw is None else np.broadcast_to(np.asarray(eps_raw, float), (Hq,))
    log_tau = np.zeros(Hq) if log_tau is None else np.broadcast_to(np.asarray(log_tau, float), (Hq,))
    fn = oracle.attn_fwd_c if impl == "c" else oracle.attn_fwd_np
    opts = {} if variant != "yat" else dict(yat_power=yat_power, yat_bias_free=yat_bias_free)
    out, mass, mx = fn(q, k, v, variant, b_raw=b_raw, eps_raw=eps_raw, log_tau=log_tau,
                       causal=causal, **opts)
    if two_d:
        return out[0, 0], mass[0, 0], mx[0, 0]
    return out, mass, mx


def weights(impl, q, k, variant, causal=False, **kw):
    """The weight matrix, observed through V = identity (d_v = T_k)."""
    Tk = np.asarray(k).shape[-2]
    out, _, _ = run(impl, q, k, np.eye(Tk), variant, causal=causal, **kw)
    return out


# --------------------------------------------------------------------------
# Softmax branch: values printed on "NNX Scaled Dot-Product Attention"

@pytest.mark.parametrize("impl", IMPLS)
def test_sdpa_worked_example(impl):
    g = load_golden("sdpa_worked_example.json")
    q = np.array([[LN2], [0.0]])
    out, _, _ = run(impl, q, g["k"], g["v"], "softmax")
    np.testing.assert_allclose(out, g["out"], rtol=0, atol=1e-14)
    w = weights(impl, q, g["k"], "softmax")
    np.testing.assert_allclose(w, g["weights"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("impl", IMPLS)
def test_softmax_share_of_matching_key(impl):
    g = load_golden("softmax_share.json")
    # d_k = 1 so the 1/sqrt(d_k) scale is 1 and the scores are the keys
    w = weights(impl, [[1.0]], np.array(g["scores"])[:, None], "softmax")[0]
    np.testing.assert_allclose(w, g["weights_rounded"], rtol=0, atol=g["abs_tol"])
    assert abs(w.sum() - 1.0) < 1e-15


@pytest.mark.parametrize("impl", IMPLS)
def test_weighted_average_of_values(impl):
    g = load_golden("weighted_average.json")
    w0, w1 = g["weights"]
    # scores differing by ln(w1/w0) produce exactly these weights
    k = [[0.0], [math.log(w1 / w0)]]
    out, _, _ = run(impl, [[1.0]], k, np.array(g["values"])[:, None], "softmax")
    assert abs(out[0, 0] - g["out"]) < 1e-14


@pytest.mark.parametrize("impl", IMPLS)
def test_softmax_divides_by_sqrt_dk(impl):
    # q.k = 4 with d_k = 4 -> score 4 / 2 = 2 against a zero score
    q = [[1.0, 1.0, 1.0, 1.0]]
    k = [[1.0, 1.0, 1.0, 1.0], [0.0, 0.0, 0.0, 0.0]]
    w = weights(impl, q, k, "softmax")[0]
    e2 = math.exp(2.0)
    np.testing.assert_allclose(w, [e2 / (e2 + 1), 1 / (e2 + 1)], rtol=1e-14)
    _, mass, mx = run(impl, q, k, np.eye(2), "softmax")
    assert abs(mx[0] - 2.0) < 1e-15                  # max scaled logit
    assert abs(mass[0] - (1.0 + math.exp(-2.0))) < 1e-15  # sum exp(s - max)


@pytest.mark.parametrize("impl", IMPLS)
def test_softmax_shift_invariance(impl):
    # with d_k = 1 and q = 2, adding 5 to every key adds 10 to every score
    rng = np.random.default_rng(11)
    k = rng.standard_normal((7, 1))
    v = rng.standard_normal((7, 3))
    a, _, _ = run(impl, [[2.0]], k, v, "softmax")
    b, _, _ = run(impl, [[2.0]], k + 5.0, v, "softmax")
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("impl", IMPLS)
def test_zero_query_averages_values(impl):
    # "The zero query scores both keys equally, so it returns the ordinary average"
    rng = np.random.default_rng(12)
    k = rng.standard_normal((5, 3))
    v = rng.standard_normal((5, 4))
    out, _, _ = run(impl, np.zeros((1, 3)), k, v, "softmax")
    np.testing.assert_allclose(out[0], v.mean(0), rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# Masks and normalisation, all branches

@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("variant", ["softmax", "yat", "stau"])
def test_causal_masked_weights_exactly_zero_and_rows_normalised(impl, variant):
    rng = np.random.default_rng(13)
    T = 9
    q = rng.standard_normal((T, 4))
    k = rng.standard_normal((T, 4))
    kw = dict(b_raw=0.3, eps_raw=-0.5, log_tau=0.7)
    w = weights(impl, q, k, variant, causal=True, **kw)
    assert np.all(w[np.triu_indices(T, 1)] == 0.0)
    assert np.all(w >= 0.0)
    out, mass, _ = run(impl, q, k, np.ones((T, 1)), variant, causal=True, **kw)
    if variant == "yat":
        # w = kappa / (mass + 1e-9) sums to mass / (mass + 1e-9)
        np.testing.assert_allclose(out[:, 0], mass / (mass + 1e-9), rtol=1e-14)
    else:
        np.testing.assert_allclose(out[:, 0], 1.0, rtol=1e-14)
    # the first row has one allowed key and returns its value
    v = rng.standard_normal((T, 3))
    out, _, _ = run(impl, q, k, v, variant, causal=True, **kw)
    if variant == "yat":
        _, m0, _ = run(impl, q[:1], k[:1], v[:1], variant, **kw)
        np.testing.assert_allclose(out[0], v[0] * m0[0] / (m0[0] + 1e-9), rtol=1e-14)
    else:
        np.testing.assert_allclose(out[0], v[0], rtol=1e-14)


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("variant", ["softmax", "yat", "stau"])
def test_causality_future_keys_do_not_matter(impl, variant):
    rng = np.random.default_rng(14)
    T = 8
    q, k, v = rng.standard_normal((T, 3)), rng.standard_normal((T, 3)), rng.standard_normal((T, 2))
    kw = dict(b_raw=0.1, eps_raw=0.2, log_tau=0.3)
    a = run(impl, q, k, v, variant, causal=True, **kw)
    k2, v2 = k.copy(), v.copy()
    k2[5:] += 10.0
    v2[5:] -= 3.0
    b = run(impl, q, k2, v2, variant, causal=True, **kw)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x[:5], y[:5])


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("variant", ["softmax", "yat", "stau"])
def test_key_permutation_invariance_noncausal(impl, variant):
    rng = np.random.default_rng(15)
    q, k, v = rng.standard_normal((4, 5)), rng.standard_normal((11, 5)), rng.standard_normal((11, 3))
    perm = rng.permutation(11)
    kw = dict(b_raw=-0.2, eps_raw=0.4, log_tau=1.1)
    a = run(impl, q, k, v, variant, **kw)
    b = run(impl, q, k[perm], v[perm], variant, **kw)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# Yat kernel: closed forms from "The Kernel Between the Roles"

@pytest.mark.parametrize("impl", IMPLS)
def test_yat_softplus_zero_is_ln2_and_peak_at_query(impl):
    g = load_golden("yat_peak.json")
    assert abs(oracle.softplus(0.0) - g["softplus_zero"]) < 1e-16
    rng = np.random.default_rng(16)
    q = rng.standard_normal((1, 6))
    nq = (q @ q.T).item()
    # b_raw = eps_raw = 0 -> b = eps = ln 2; a key equal to the query
    _, mass, mx = run(impl, q, q, np.ones((1, 1)), "yat", b_raw=0.0, eps_raw=0.0)
    peak = (nq + LN2) ** 2 / LN2
    assert abs(mass[0] - peak) <= 1e-13 * peak
    assert abs(mx[0] - peak) <= 1e-13 * peak


@pytest.mark.parametrize("impl", IMPLS)
def test_yat_distance_from_dots(impl):
    # q = (1, 0), k = (1, 1): q.k = 1, |q - k|^2 = 1
    b, e = math.log1p(math.exp(0.5)), math.log1p(math.exp(-1.0))
    _, mass, _ = run(impl, [[1.0, 0.0]], [[1.0, 1.0]], [[1.0]], "yat", b_raw=0.5, eps_raw=-1.0)
    assert abs(mass[0] - (1.0 + b) ** 2 / (1.0 + e)) < 1e-14
    # q = (2, -1), k = (-1, 3): q.k = -5, |q - k|^2 = 9 + 16 = 25
    _, mass, _ = run(impl, [[2.0, -1.0]], [[-1.0, 3.0]], [[1.0]], "yat", b_raw=0.5, eps_raw=-1.0)
    assert abs(mass[0] - (-5.0 + b) ** 2 / (25.0 + e)) < 1e-14


@pytest.mark.parametrize("impl", IMPLS)
def test_yat_zero_query(impl):
    k = np.array([[0.5, -2.0, 1.0]])
    b, e = math.log1p(math.exp(0.3)), math.log1p(math.exp(-0.7))
    _, mass, _ = run(impl, np.zeros((1, 3)), k, [[1.0]], "yat", b_raw=0.3, eps_raw=-0.7)
    assert abs(mass[0] - b * b / ((k @ k.T).item() + e)) < 1e-15


@pytest.mark.parametrize("impl", IMPLS)
def test_yat_bias_free_orthogonal_pair_scores_zero(impl):
    # b = softplus(-inf) = 0: an orthogonal pair scores exactly 0 however near
    out, mass, mx = run(impl, [[1.0, 0.0]], [[0.0, 1e-3]], [[7.0, -3.0]], "yat",
                        b_raw=-np.inf, eps_raw=0.0)
    assert mass[0] == 0.0 and mx[0] == 0.0
    # the 1e-9 floor keeps the weights finite: w = 0 / (0 + 1e-9) = 0
    assert np.all(out == 0.0)


@pytest.mark.parametrize("impl", IMPLS)
def test_yat_symmetric_and_nonnegative(impl):
    rng = np.random.default_rng(17)
    for _ in range(5):
        a, c = rng.standard_normal((1, 4)), rng.standard_normal((1, 4))
        _, m1, _ = run(impl, a, c, [[1.0]], "yat", b_raw=0.2, eps_raw=-0.3)
        _, m2, _ = run(impl, c, a, [[1.0]], "yat", b_raw=0.2, eps_raw=-0.3)
        assert m1[0] >= 0.0
        assert abs(m1[0] - m2[0]) <= 1e-14 * m1[0]


@pytest.mark.parametrize("impl", IMPLS)
def test_yat_mass_is_sum_of_pair_scores(impl):
    # the mass of a row is the sum of its one-key masses
    rng = np.random.default_rng(18)
    q, k = rng.standard_normal((1, 5)), rng.standard_normal((6, 5))
    _, mass, mx = run(impl, q, k, np.ones((6, 1)), "yat", b_raw=0.4, eps_raw=0.1)
    singles = [run(impl, q, k[j:j + 1], [[1.0]], "yat", b_raw=0.4, eps_raw=0.1)[1][0]
               for j in range(6)]
    assert abs(mass[0] - sum(singles)) <= 1e-13 * mass[0]
    assert mx[0] == max(singles)


# --------------------------------------------------------------------------
# Yat kernel-family options ("The Kernel Between the Roles", "The run"): the
# numerator power (q.k + b)^(2m) and the b = 0 ablation

@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("m", [1, 2, 3])
@pytest.mark.parametrize("bias_free", [False, True])
def test_yat_power_peak_at_query(impl, m, bias_free):
    # a key equal to its query: distance 0, so kappa = (|q|^2 + b)^(2m) / eps
    rng = np.random.default_rng(40 + m)
    q = rng.standard_normal((1, 5))
    nq = (q @ q.T).item()
    _, mass, mx = run(impl, q, q, [[1.0]], "yat", b_raw=0.0, eps_raw=0.0, yat_power=m,
                      yat_bias_free=bias_free)
    b = 0.0 if bias_free else LN2
    peak = (nq + b) ** (2 * m) / LN2
    assert abs(mass[0] - peak) <= 1e-13 * peak and mx[0] == mass[0]


@pytest.mark.parametrize("impl", IMPLS)
def test_yat_power_hand_values(impl):
    b, e = math.log1p(math.exp(0.5)), math.log1p(math.exp(-1.0))
    # q = (1, 0), k = (1, 1): q.k = 1, |q - k|^2 = 1
    # q = (2, -1), k = (-1, 3): q.k = -5, |q - k|^2 = 25
    for q, k, dot_, d2 in (([[1.0, 0.0]], [[1.0, 1.0]], 1.0, 1.0),
                           ([[2.0, -1.0]], [[-1.0, 3.0]], -5.0, 25.0)):
        for m in (2, 3, 4):
            _, mass, _ = run(impl, q, k, [[1.0]], "yat", b_raw=0.5, eps_raw=-1.0, yat_power=m)
            want = (dot_ + b) ** (2 * m) / (d2 + e)
            assert abs(mass[0] - want) <= 1e-14 * want
            # the bias-free kernel ignores b_raw
            _, mass0, _ = run(impl, q, k, [[1.0]], "yat", b_raw=0.5, eps_raw=-1.0, yat_power=m,
                              yat_bias_free=True)
            want0 = dot_ ** (2 * m) / (d2 + e)
            assert abs(mass0[0] - want0) <= 1e-14 * want0


@pytest.mark.parametrize("impl", IMPLS)
def test_yat_bias_free_equals_softplus_minus_infinity(impl):
    # the explicit flag and b_raw = -inf are the same kernel (b = 0 exactly)
    rng = np.random.default_rng(44)
    q, k, v = rng.standard_normal((4, 3)), rng.standard_normal((6, 3)), rng.standard_normal((6, 2))
    a = run(impl, q, k, v, "yat", b_raw=3.0, eps_raw=-0.5, yat_bias_free=True)
    c = run(impl, q, k, v, "yat", b_raw=-np.inf, eps_raw=-0.5)
    for x, y in zip(a, c):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("m", [1, 2, 4])
def test_yat_bias_free_orthogonal_pair_scores_zero_any_power(impl, m):
    out, mass, mx = run(impl, [[1.0, 0.0]], [[0.0, 1e-3]], [[7.0, -3.0]], "yat", b_raw=2.0,
                        eps_raw=0.0, yat_power=m, yat_bias_free=True)
    assert mass[0] == 0.0 and mx[0] == 0.0 and np.all(out == 0.0)


# --------------------------------------------------------------------------
# s^tau: the core formula and its softmax identity ("s^tau" forum post)

def _tau_for(t):
    """log_tau with softplus(log_tau) + 1 = t (t > 1)."""
    return math.log(math.expm1(t - 1.0))


@pytest.mark.parametrize("impl", IMPLS)
def test_stau_power_of_large_scores(impl):
    # for s >> 1, phi(s) = s to ~1e-9 relative, so weights -> s^tau / sum s^tau
    k = [[30.0], [10.0]]
    w = weights(impl, [[1.0]], k, "stau", log_tau=-np.inf)[0]     # tau = 1
    np.testing.assert_allclose(w, [0.75, 0.25], atol=2e-6)
    w = weights(impl, [[1.0]], k, "stau", log_tau=_tau_for(2.0))[0]  # tau = 2
    np.testing.assert_allclose(w, [0.9, 0.1], atol=2e-6)
    w = weights(impl, [[1.0]], [[100.0], [10.0], [1.0]], "stau", log_tau=_tau_for(5.0))[0]
    # the page's tau = 5 illustration: 100^5, 10^5, 1^5 (phi(1) = 1.3133;
    # phi(10) exceeds 10 by 4.5e-5, i.e. 2.3e-5 relative after the 5th power)
    expect = np.array([1e10, 1e5, (math.log1p(math.e) + 1e-6) ** 5])
    np.testing.assert_allclose(w, expect / expect.sum(), rtol=3e-5)


@pytest.mark.parametrize("impl", IMPLS)
def test_stau_tau_init_weak_pin(impl):
    g = load_golden("stau_tau_init.json")
    # recover tau from two large scores: w0/w1 = (s0/s1)^tau
    w = weights(impl, [[1.0]], [[60.0], [20.0]], "stau", log_tau=g["log_tau"])[0]
    tau = math.log(w[0] / w[1]) / math.log(3.0)
    assert abs(tau - g["tau_printed"]) < g["abs_tol"]


@pytest.mark.parametrize("impl", IMPLS)
def test_stau_equals_softmax_of_tau_log_phi(impl):
    # the page's equivalence: phi^tau / sum phi^tau = softmax(tau log phi(s))
    rng = np.random.default_rng(19)
    q, k = rng.standard_normal((3, 4)), rng.standard_normal((7, 4))
    log_tau = 0.8
    tau = float(oracle.softplus(log_tau)) + 1.0
    w = weights(impl, q, k, "stau", log_tau=log_tau)
    s = (q @ k.T) / 2.0
    for i in range(3):
        logits = tau * np.log(oracle.softplus(s[i]) + 1e-6)
        # the softmax oracle with d_k = 1 and query 1 turns keys into logits
        ws = weights(impl, [[1.0]], logits[:, None], "softmax")[0]
        np.testing.assert_allclose(w[i], ws, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("impl", IMPLS)
def test_stau_max_score_and_mass(impl):
    q, k = [[1.0, 1.0, 1.0, 1.0]], [[1.0, 1.0, 1.0, 1.0], [-1.0, -1.0, 0.0, 0.0]]
    _, mass, mx = run(impl, q, k, np.ones((2, 1)), "stau", log_tau=-np.inf)  # tau = 1
    # scores 2 and -1; phi = softplus + 1e-6
    assert abs(mx[0] - 2.0) < 1e-15
    sp = lambda x: math.log1p(math.exp(x))
    assert abs(mass[0] - (sp(2.0) + sp(-1.0) + 2e-6)) < 1e-14


# --------------------------------------------------------------------------
# Shapes: GQA mapping, T_q != T_k, d_v != d_k, brute force

@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("variant", ["softmax", "yat", "stau"])
def test_gqa_equals_repeated_kv(impl, variant):
    rng = np.random.default_rng(20)
    B, Hq, Hkv, Tq, Tk, dk, dv = 2, 6, 2, 5, 7, 4, 3
    q = rng.standard_normal((B, Hq, Tq, dk))
    k = rng.standard_normal((B, Hkv, Tk, dk))
    v = rng.standard_normal((B, Hkv, Tk, dv))
    kw = dict(b_raw=rng.uniform(-1, 1, Hq), eps_raw=rng.uniform(-3, 0, Hq),
              log_tau=rng.uniform(-1, 2, Hq))
    a = run(impl, q, k, v, variant, **kw)
    b = run(impl, q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), variant, **kw)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def brute_force(q, k, v, variant, b_raw, eps_raw, log_tau, causal, yat_power=1,
                yat_bias_free=False):
    """Pure-Python loops over 4-D nested lists; tiny inputs only."""
    B, Hq, Tq, dk = q.shape
    Hkv, Tk, dv = k.shape[1], k.shape[2], v.shape[3]
    sp = lambda x: max(x, 0.0) + math.log1p(math.exp(-abs(x)))
    out = np.zeros((B, Hq, Tq, dv)); mass = np.zeros((B, Hq, Tq)); mx = np.zeros((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(Tq):
                keys = range(i + 1) if causal else range(Tk)
                sc = {}
                for j in keys:
                    d = sum(float(q[b, h, i, t]) * float(k[b, hk, j, t]) for t in range(dk))
                    if variant == "yat":
                        nq = sum(float(x) ** 2 for x in q[b, h, i])
                        nk = sum(float(x) ** 2 for x in k[b, hk, j])
                        bb = 0.0 if yat_bias_free else sp(b_raw[h])
                        num = 1.0
                        for _ in range(yat_power):
                            num *= (d + bb) * (d + bb)
                        sc[j] = num / (max(nq + nk - 2 * d, 0.0) + sp(eps_raw[h]))
                    else:
                        sc[j] = d / math.sqrt(dk)
                if variant == "yat":
                    tot = sum(sc.values()); wts = {j: s / (tot + 1e-9) for j, s in sc.items()}
                    mx[b, h, i] = max(sc.values())
                elif variant == "softmax":
                    m = max(sc.values()); e = {j: math.exp(s - m) for j, s in sc.items()}
                    tot = sum(e.values()); wts = {j: x / tot for j, x in e.items()}
                    mx[b, h, i] = m
                else:
                    tau = sp(log_tau[h]) + 1.0
                    u = {j: (sp(s) + 1e-6) ** tau for j, s in sc.items()}
                    tot = sum(u.values()); wts = {j: x / tot for j, x in u.items()}
                    mx[b, h, i] = max(sc.values())
                mass[b, h, i] = tot
                for t in range(dv):
                    out[b, h, i, t] = sum(wts[j] * float(v[b, hk, j, t]) for j in wts)
    return out, mass, mx


@pytest.mark.parametrize("variant", ["softmax", "yat", "stau"])
@pytest.mark.parametrize("shape", [(1, 2, 1, 3, 5, 2, 4, False), (2, 2, 2, 4, 4, 3, 2, True),
                                   (1, 4, 2, 6, 6, 5, 3, True)])
def test_brute_force_tiny(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    rng = np.random.default_rng(21)
    q = rng.standard_normal((B, Hq, Tq, dk)) * 1.5
    k = rng.standard_normal((B, Hkv, Tk, dk)) * 1.5
    v = rng.standard_normal((B, Hkv, Tk, dv))
    prm = dict(b_raw=rng.uniform(-1, 1, Hq), eps_raw=rng.uniform(-3, 0, Hq),
               log_tau=rng.uniform(-1, 2, Hq))
    ref = brute_force(q, k, v, variant, causal=causal, **prm)
    for impl in IMPLS:
        got = run(impl, q, k, v, variant, causal=causal, **prm)
        for x, y in zip(got, ref):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("opts", [(2, False), (3, True), (1, True)])
def test_brute_force_tiny_yat_options(opts):
    m, bias_free = opts
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = 1, 4, 2, 5, 5, 3, 2, True
    rng = np.random.default_rng(23)
    q = rng.standard_normal((B, Hq, Tq, dk))
    k = rng.standard_normal((B, Hkv, Tk, dk))
    v = rng.standard_normal((B, Hkv, Tk, dv))
    prm = dict(b_raw=rng.uniform(-1, 1, Hq), eps_raw=rng.uniform(-3, 0, Hq), log_tau=None)
    ref = brute_force(q, k, v, "yat", causal=causal, yat_power=m, yat_bias_free=bias_free, **prm)
    for impl in IMPLS:
        got = run(impl, q, k, v, "yat", causal=causal, yat_power=m, yat_bias_free=bias_free,
                  **prm)
        for x, y in zip(got, ref):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("variant", ["softmax", "yat", "stau"])
@pytest.mark.parametrize("causal", [False, True])
def test_c_and_numpy_oracles_agree(variant, causal):
    rng = np.random.default_rng(22)
    B, Hq, Hkv, T, dk, dv = 2, 4, 2, 40, 16, 24
    q = rng.standard_normal((B, Hq, T, dk)) * 2
    k = rng.standard_normal((B, Hkv, T, dk)) * 2
    v = rng.standard_normal((B, Hkv, T, dv))
    prm = dict(b_raw=rng.uniform(-1, 1, Hq), eps_raw=rng.uniform(-3, 0, Hq),
               log_tau=rng.uniform(-1, 2, Hq))
    a = oracle.attn_fwd_c(q, k, v, variant, causal=causal, **prm)
    b = oracle.attn_fwd_np(q, k, v, variant, causal=causal, **prm)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-12)
    # a row subset gives the same rows
    rows = np.array([0, 7, 39, 40, 100, B * Hq * T - 1])
    c = oracle.attn_fwd_c(q, k, v, variant, causal=causal, rows=rows, **prm)
    for x, y in zip(c, a):
        np.testing.assert_array_equal(x, y.reshape(B * Hq * T, -1)[rows].reshape(x.shape))


def test_oracle_rejects_bad_arguments():
    q = np.zeros((1, 3, 4, 2)); k = np.zeros((1, 2, 4, 2)); v = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):      # Hq % Hkv != 0
        oracle.attn_fwd_c(q, k, v, "softmax")
    q = np.zeros((1, 1, 3, 2)); k = np.zeros((1, 1, 4, 2)); v = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):      # causal needs Tq == Tk
        oracle.attn_fwd_c(q, k, v, "softmax", causal=True)
    with pytest.raises(ValueError):      # out-of-range row id
        oracle.attn_fwd_c(q, k, v, "softmax", rows=[3])
    with pytest.raises(ValueError):      # Yat numerator power below 1
        oracle.attn_fwd_c(q, k, v, "yat", b_raw=np.zeros(1), eps_raw=np.zeros(1), yat_power=0)


# --------------------------------------------------------------------------
# Telemetry: normalised row entropy ("The Kernel Between the Roles", "The
# run"), sparsity and tau* (the s^tau post)

def tel(q, k, variant, causal=False, **kw):
    q, k = np.asarray(q, float)[None, None], np.asarray(k, float)[None, None]
    prm = dict(b_raw=np.zeros(1), eps_raw=np.zeros(1), log_tau=np.zeros(1))
    prm.update(kw)
    e, s, t = oracle.telemetry_np(q, k, variant, causal=causal, **prm)
    return e[0, 0], s[0, 0], t[0]


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_entropy_of_equal_keys_is_one(variant):
    # identical keys get identical weights: the entropy is ln n, normalised 1
    e, s, _ = tel([[0.3, -1.2], [2.0, 0.5]], [[1.0, 0.4]] * 5, variant)
    # (Yat weights sum to mass / (mass + 1e-9), which moves the entropy by ~1e-9)
    np.testing.assert_allclose(e, 1.0, rtol=0, atol=1e-8 if variant == "yat" else 1e-12)
    assert np.all(s == 0.0)


def test_entropy_two_keys_is_binary_entropy():
    # softmax over two logits a, b: p = 1 / (1 + e^(b - a)); H = -p ln p - q ln q
    a, b = 0.7, -1.9
    e, _, _ = tel([[1.0]], [[a], [b]], "softmax")
    p = 1.0 / (1.0 + math.exp(b - a))
    h = -(p * math.log(p) + (1 - p) * math.log(1 - p)) / math.log(2.0)
    assert abs(e[0] - h) < 1e-13


def test_entropy_one_allowed_key_is_zero():
    e, s, _ = tel([[1.0], [2.0]], [[0.5], [0.1]], "yat", causal=True)
    assert e[0] == 0.0 and s[0] == 0.0          # row 0 sees one key


def test_sparsity_counts_weights_below_threshold():
    # logits 0, -20, -20, 0: two weights e^-20 / (2 + 2 e^-20) < 1e-6
    _, s, _ = tel([[1.0]], [[0.0], [-20.0], [-20.0], [0.0]], "softmax")
    assert s[0] == 0.5
    _, s, _ = tel([[1.0]], [[0.0], [-20.0], [-20.0], [0.0]], "softmax", sparsity_threshold=1e-12)
    assert s[0] == 0.0


def test_tau_star_two_score_values_is_the_slope():
    # with two distinct scores the least-squares slope of s on ln phi(s) runs
    # through both points: tau* = (s1 - s2) / (ln phi(s1) - ln phi(s2))
    s1, s2 = 1.5, -0.25
    _, _, t = tel([[1.0]], [[s1], [s2], [s1]], "stau")
    lp = lambda s: math.log(max(s, 0.0) + math.log1p(math.exp(-abs(s))) + 1e-6)
    assert abs(t - (s1 - s2) / (lp(s1) - lp(s2))) < 1e-12


def test_tau_star_ignores_masked_pairs_and_is_undefined_without_spread():
    # causal: row 0 sees only key 0; all allowed scores equal -> Var = 0 -> NaN
    _, _, t = tel([[1.0], [1.0]], [[0.5], [9.0]], "softmax", causal=True)
    assert math.isnan(t) is False                # keys 0.5 (x2) and 9.0 differ
    _, _, t = tel([[1.0], [1.0]], [[0.5], [0.5]], "softmax")
    assert math.isnan(t)
