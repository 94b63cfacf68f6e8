"""The polynomial behind the s^tau tile kernels' map, on the CPU.

The kernels take log2(1 + t), t = 2^-|y|, as t P(t) with P a degree-4
polynomial for log2(1 + t) / t on [0, 1] (bf16_common.h, StauPoly).  These
tests read the coefficients from that header and check them against the
mathematics: the fit in softmax_free_score_amd/stau_poly.py reproduces them,
their relative error in fp32 Horner evaluation is below the 5.7e-5 the header
states, and the whole base-2 map, emulated in fp32 with exactly rounded
exp2/log2, gives phi^tau / (ln 2)^tau with phi = softplus(s) + 1e-6 ("s^tau"
forum post, core formula) to within tau times that error."""
import os
import re

import numpy as np
import pytest

from conftest import ROOT
from softmax_free_score_amd import stau_poly

HEADER = os.path.join(ROOT, "softmax_free_score_amd", "csrc", "bf16_common.h")
BOUND = 5.7e-5
F32 = np.float32


def header_coefficients():
    text = open(HEADER).read()
    m = re.search(r"StauPoly s\{([^}]*)\}", text)
    assert m, "StauPoly initialiser not found"
    vals = [float(v.strip().rstrip("f")) for v in m.group(1).split(",")]
    assert len(vals) == stau_poly.DEGREE + 1
    return np.array(vals, dtype=np.float32)


def test_header_matches_fit():
    fitted = stau_poly.fit().astype(np.float32)
    got = header_coefficients()
    assert np.allclose(got, fitted, rtol=1e-5, atol=0), (got, fitted)


def test_relative_error_bound():
    err = stau_poly.max_rel_error(header_coefficients())
    assert err < BOUND, err
    # and the fit is not loose: a degree lower cannot meet the bound
    assert stau_poly.max_rel_error(stau_poly.fit(stau_poly.DEGREE - 1)) > 4 * BOUND


def test_target_special_values():
    # log2(1 + t) / t -> 1/ln 2 at 0, 1 at t = 1, and t P(t) is log2(1 + t)
    assert stau_poly.target(np.array([0.0]))[0] == pytest.approx(1 / np.log(2), rel=1e-15)
    assert stau_poly.target(np.array([1.0]))[0] == pytest.approx(1.0, rel=1e-15)
    t = np.array([2.0 ** -30, 2.0 ** -10, 0.25, 0.75])
    assert np.allclose(t * stau_poly.target(t), np.log2(1 + t), rtol=1e-14)


def r32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def emulate_map(x, tau, c_sm, coef):
    """The kernel's stau_weight2 step by step in fp32 (fma: one rounding;
    exp2 and log2: exactly rounded)."""
    c = coef.astype(np.float64)
    floor2 = r32(1e-6 * np.log2(np.e))
    y = r32(x.astype(np.float64) * c_sm + floor2)
    t = r32(np.exp2(-np.abs(y.astype(np.float64))))
    l = r32(c[-1] * t + c[-2])
    for a in c[-3::-1]:
        l = r32(l.astype(np.float64) * t + a)
    z = r32(l.astype(np.float64) * t + np.maximum(y, floor2))
    lz = r32(np.log2(z.astype(np.float64)))
    return r32(np.exp2(r32(np.float64(tau) * lz).astype(np.float64)))


@pytest.mark.parametrize("tau", [0.37, 1.0, 2.5, 7.4])
def test_map_against_definition(tau):
    dk = 128
    c_sm = float(r32(np.log2(np.e) / np.sqrt(dk)))
    s = np.concatenate([np.linspace(-40.0, 40.0, 160001), [-1e-3, 0.0, 1e-3]])
    x = r32(s * np.sqrt(dk))  # raw q.k
    sx = x.astype(np.float64) / np.sqrt(dk)
    phi = np.logaddexp(0.0, sx) + 1e-6
    want = phi ** tau / np.log(2.0) ** tau
    got = emulate_map(x, tau, c_sm, header_coefficients()).astype(np.float64)
    rel = np.abs(got / want - 1.0)
    # relative error of Z: the polynomial's, the floor folded into y (2^-|y|
    # off by a factor 2^(1e-6 log2 e), i.e. 1e-6 relative) and a few fp32
    # roundings; the power multiplies it by tau.  Then the roundings of
    # tau log2 Z (relative 2^-24 of it) and of exp2.
    bound = tau * (BOUND + 1e-6 + 2.0 ** -21) \
        + 2.0 ** -22 * np.abs(tau * np.log2(phi / np.log(2))) + 2.0 ** -22
    # weights below the fp32 normal range (tau large, s very negative) keep
    # only an absolute precision
    tiny = want < 2.0 ** -126
    assert np.all(np.abs(got - want)[tiny] <= 2.0 ** -126)
    ok = ~tiny
    assert np.all(rel[ok] <= bound[ok]), (rel[ok].max(), s[ok][np.argmax(rel[ok] / bound[ok])])
