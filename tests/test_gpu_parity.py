"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Small and medium problems are compared element by
element; the full-size workloads run in the benchmark's launch configuration
and are compared on every row with the C oracle."""
import numpy as np
import pytest
import torch

import oracle

from softmax_free_score_amd import attn
from parity import check, oracle_full, oracle_rows, run_gpu, say, to_device, to_np
from softmax_free_score_amd.workloads import WORKLOADS, make_custom, make_inputs

pytestmark = pytest.mark.gpu


def v_rms(inp):
    return float(np.sqrt(np.mean(np.square(inp.v, dtype=np.float64))))


# bf16 kernels by query rows per workgroup (0: the library's own choice)
BLOCK_ROWS = (0, 64, 128, 256)


def full_check(inp, variant, causal, label, block_rows=(0,), yat_opts=None, kv_splits=0):
    say(f"[gpu] {label} {variant} causal={causal} shape B{inp.wl.B} Hq{inp.wl.Hq} "
        f"Hkv{inp.wl.Hkv} Tq{inp.wl.Tq} Tk{inp.wl.Tk} dk{inp.wl.dk} dv{inp.wl.dv} {inp.wl.dtype}"
        f"{'' if yat_opts is None else f' yat_opts={yat_opts}'}")
    q, k, v, prm = to_device(inp)
    ref = oracle_full(inp, variant, causal, yat_opts)
    for rows in block_rows:
        got = [to_np(t) for t in run_gpu(q, k, v, prm, variant, causal, yat_opts=yat_opts,
                                         block_rows=rows, kv_splits=kv_splits)]
        check(inp.wl.dtype, got, ref, f"{label}/{variant}/rows{rows}",
              v_rms=v_rms(inp))


# ---------------------------------------------------------------- small sizes

@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_tiny_fp32(variant):
    inp = make_inputs(WORKLOADS["tiny"])
    full_check(inp, variant, True, "tiny")


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_gpt_small_full(variant):
    inp = make_inputs(WORKLOADS["gpt_small"])
    full_check(inp, variant, True, "gpt_small")


def test_gpt_small_tied_yat():
    # k := q puts the Yat peak (|q|^2 + b)^2 / eps on the diagonal
    inp = make_inputs(WORKLOADS["gpt_small"], tied=True)
    full_check(inp, "yat", True, "gpt_small_tied", BLOCK_ROWS)


MEDIUM = [
    # B, Hq, Hkv, Tq, Tk, dk, dv, causal
    (2, 4, 2, 333, 333, 128, 128, True),
    (1, 2, 1, 200, 517, 64, 128, False),
    (2, 3, 3, 130, 130, 32, 32, True),
    (1, 4, 4, 97, 97, 16, 16, True),
    (1, 2, 2, 150, 260, 128, 64, False),
    (1, 2, 1, 70, 70, 16, 128, True),
    (1, 2, 2, 65, 300, 128, 16, False),
    (1, 2, 2, 257, 257, 64, 32, True),
]


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", MEDIUM, ids=lambda s: "x".join(map(str, s)))
def test_medium_shapes_bf16(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=7, qk_std=1.5)
    full_check(inp, variant, causal, "medium", BLOCK_ROWS)


# Short key ranges: the small-grid kernels preload every tile (at most 4 per
# workgroup: T_k <= 256 for 128-row and <= 128 for 64-row workgroups, d <= 64)
PRELOAD = [
    (2, 4, 2, 256, 256, 32, 32, True),    # 4 full tiles (128 rows)
    (2, 2, 1, 100, 128, 64, 64, False),   # 4 full 32-key tiles (64 rows), 2 (128 rows)
    (1, 4, 2, 300, 60, 16, 32, False),    # one ragged tile, T_q > T_k
    (3, 2, 2, 33, 33, 64, 16, True),      # one tile, one query tile
    (1, 2, 2, 190, 190, 32, 64, True),    # ragged third tile
    (1, 2, 2, 129, 257, 64, 64, False),   # one key past the preload range
]


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", PRELOAD, ids=lambda s: "x".join(map(str, s)))
def test_short_key_ranges_bf16(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=28, qk_std=1.5)
    full_check(inp, variant, causal, "preload", BLOCK_ROWS)


# 128-row workgroups whose key range spans >= 8 tiles of 64 keys take two key
# halves: two waves per 32 query rows, alternate tiles, partials merged in LDS.
# Causal (short and long query tiles in one launch), ragged tails, odd tile
# counts, GQA, and d_k <= 32 (Yat norms formed in the kernel).
KEY_HALVES = [
    (1, 4, 2, 600, 600, 128, 128, True),
    (2, 2, 2, 515, 515, 64, 64, True),
    (1, 2, 1, 130, 1000, 32, 128, False),
    (1, 2, 2, 257, 520, 16, 16, False),
]


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", KEY_HALVES, ids=lambda s: "x".join(map(str, s)))
def test_key_halves_bf16(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=29, qk_std=1.5)
    full_check(inp, variant, causal, "key_halves", block_rows=(128,))


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", [(1, 2, 1, 100, 100, 32, 64, True),
                                   (2, 2, 2, 33, 90, 128, 16, False)],
                         ids=lambda s: "x".join(map(str, s)))
def test_medium_shapes_fp32(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "f32", causal, seed=8)
    full_check(inp, variant, causal, "medium_f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tied_medium_yat(dtype):
    inp = make_custom(1, 3, 3, 300, 300, 128, 128, dtype, True, seed=9, qk_std=2.0, tied=True)
    full_check(inp, "yat", True, "tied_medium", BLOCK_ROWS if dtype == "bf16" else (0,))


# ------------------------------------------- Yat options (attn_fwd_yat)

YAT_OPTS = [(2, False), (3, True), (1, True)]


@pytest.mark.parametrize("opts", YAT_OPTS, ids=lambda o: f"m{o[0]}{'_nobias' if o[1] else ''}")
@pytest.mark.parametrize("shape", [MEDIUM[0], MEDIUM[1], MEDIUM[3], MEDIUM[6]],
                         ids=lambda s: "x".join(map(str, s)))
def test_yat_options_bf16(shape, opts):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=15, qk_std=1.0)
    full_check(inp, "yat", causal, "yat_opts", BLOCK_ROWS, yat_opts=opts)


@pytest.mark.parametrize("opts", YAT_OPTS, ids=lambda o: f"m{o[0]}{'_nobias' if o[1] else ''}")
def test_yat_options_fp32(opts):
    inp = make_custom(1, 2, 1, 100, 100, 32, 64, "f32", True, seed=16)
    full_check(inp, "yat", True, "yat_opts_f32", yat_opts=opts)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_yat_power_tied_peak(dtype):
    # k := q: the diagonal carries the peak (|q|^2 + b)^(2m) / eps
    inp = make_custom(1, 2, 2, 160, 160, 64, 64, dtype, True, seed=17, qk_std=1.0, tied=True)
    full_check(inp, "yat", True, "yat_pow_tied", BLOCK_ROWS if dtype == "bf16" else (0,),
               yat_opts=(2, False))


def test_yat_options_full_size_every_row():
    wl = WORKLOADS["cross"]
    inp = make_inputs(wl)
    say("[gpu] full-size cross yat power 2: every row")
    q, k, v, prm = to_device(inp)
    got = [to_np(t) for t in run_gpu(q, k, v, prm, "yat", wl.causal, yat_opts=(2, False))]
    ref = oracle_rows(inp, "yat", wl.causal, None, yat_opts=(2, False))
    check(wl.dtype, got, ref, "cross/yat_m2", v_rms=v_rms(inp))


def test_yat_default_options_match_attn_fwd():
    # opts (1, no bias-free) is the standard kernel, bit for bit
    inp = make_custom(2, 4, 2, 300, 300, 128, 128, "bf16", True, seed=18)
    q, k, v, prm = to_device(inp)
    a = run_gpu(q, k, v, prm, "yat", True)
    b = run_gpu(q, k, v, prm, "yat", True, yat_opts=(1, False))
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ------------------------------------- key splits (partials + combine)

SPLITS = [(64, 2), (64, 5), (128, 3), (0, 0)]   # (block_rows, kv_splits); (0, 0): library's plan


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", [MEDIUM[0], MEDIUM[1], MEDIUM[2], MEDIUM[6],
                                   (1, 4, 2, 64, 1500, 128, 128, False)],
                         ids=lambda s: "x".join(map(str, s)))
def test_kv_splits_bf16(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=19, qk_std=1.5)
    say(f"[gpu] kv splits {variant} {shape}")
    q, k, v, prm = to_device(inp)
    ref = oracle_full(inp, variant, causal)
    for rows, splits in SPLITS:
        got = [to_np(t) for t in run_gpu(q, k, v, prm, variant, causal, block_rows=rows,
                                         kv_splits=splits)]
        check("bf16", got, ref, f"splits/{variant}/rows{rows}/s{splits}",
              v_rms=v_rms(inp))


# Key splits whose chunks span >= 8 tiles take two key halves inside each chunk:
# chunks starting at an odd tile (27 tiles in 3 chunks of 9), and causal rows
# whose second chunk is empty for the early query tiles.
@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("case", [((1, 4, 2, 64, 1728, 128, 128, False), 3),
                                  ((1, 2, 1, 1100, 1100, 64, 64, True), 2)],
                         ids=lambda c: "x".join(map(str, c[0])) + f"_s{c[1]}")
def test_kv_splits_key_halves(variant, case):
    (B, Hq, Hkv, Tq, Tk, dk, dv, causal), splits = case
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=31, qk_std=1.5)
    full_check(inp, variant, causal, "splits_key_halves", block_rows=(128,), kv_splits=splits)


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", [(2, 8, 2, 1, 3000, 128, 128), (4, 16, 8, 4, 2049, 64, 64),
                                   (1, 2, 1, 7, 9000, 128, 32)],
                         ids=lambda s: "x".join(map(str, s)))
def test_decode_shapes(variant, shape):
    # few query rows against long keys: the library splits the keys by itself
    B, Hq, Hkv, Tq, Tk, dk, dv = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", False, seed=20, qk_std=1.0)
    full_check(inp, variant, False, "decode")


DECODE_FORCED = [
    # B, Hq, Hkv, Tq, Tk, dk, dv, causal; Hq/Hkv * Tq <= 8
    (2, 4, 2, 1, 1000, 64, 128, False),
    (1, 8, 1, 1, 300, 128, 16, False),      # g = 8, d_v = 16
    (3, 6, 3, 2, 257, 128, 128, False),     # 4 packed rows, one key past a chunk
    (1, 4, 4, 2, 700, 16, 64, False),       # d_k = 16
    (1, 2, 2, 3, 3, 32, 32, True),          # causal, fewer keys than a chunk
    (2, 2, 1, 4, 4, 128, 128, True),        # causal, 8 packed rows
    (1, 2, 1, 1, 17000, 64, 64, False),     # 67 chunks: the merge reads more than 64
    (1, 2, 1, 1, 70001, 64, 32, False),     # 274 chunks, ragged last one
    (2, 3, 3, 1, 513, 32, 32, False),       # one row per kv head, ragged last chunk
    (1, 8, 2, 1, 600, 16, 32, False),       # d_k = 16, 4 rows: each lane maps 2 rows
    (1, 8, 1, 1, 300, 16, 16, False),       # d_k = 16, 8 rows: each lane maps 4 rows
    (2, 4, 1, 2, 520, 32, 64, False),       # d_k = 32, 8 rows: each lane maps 2 rows
    (1, 4, 1, 2, 2, 16, 16, True),          # causal, d_k = 16, 8 rows
]


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", DECODE_FORCED, ids=lambda s: "x".join(map(str, s)))
def test_decode_kernel(variant, shape):
    # the packed vector kernel (block_rows = 8) and the library's own choice
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=23, qk_std=1.5)
    full_check(inp, variant, causal, "decode_kernel", block_rows=(8, 0))


def test_decode_kernel_tied_and_yat_options():
    # k := q puts the peak (|q|^2 + b)^2 / eps on the diagonal; the kernel's
    # |q|^2, |k|^2 and q.k share one v_dot2 order, so d2 is exactly 0 there
    inp = make_custom(1, 4, 4, 2, 2, 128, 128, "bf16", True, seed=24, qk_std=2.0, tied=True)
    full_check(inp, "yat", True, "decode_tied", block_rows=(8,))
    inp = make_custom(2, 8, 2, 1, 900, 128, 128, "bf16", False, seed=25, qk_std=1.0)
    for opts in ((2, False), (3, True), (1, True)):
        full_check(inp, "yat", False, "decode_yat_opts", block_rows=(8,), yat_opts=opts)


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_decode_kernel_strided_gqa_determinism(variant):
    """The decode kernel's arithmetic per row does not depend on how rows are
    packed or on the storage strides: [B, T, H, d] storage, K/V repeated to one
    query row per key/value head, and a second call all give identical bits."""
    inp = make_custom(2, 8, 2, 1, 1000, 128, 128, "bf16", False, seed=28)
    q, k, v, prm = to_device(inp)
    a = run_gpu(q, k, v, prm, variant, False, block_rows=8)
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    assert ks.stride(2) == 2 * 128
    b = run_gpu(qs, ks, vs, prm, variant, False, block_rows=8)
    c = run_gpu(q, k.repeat_interleave(4, dim=1).contiguous(),
                v.repeat_interleave(4, dim=1).contiguous(), prm, variant, False, block_rows=8)
    d = run_gpu(q, k, v, prm, variant, False, block_rows=8)
    for x, y, z, u in zip(a, b, c, d):
        assert torch.equal(x, y) and torch.equal(x, z) and torch.equal(x, u)


@pytest.mark.parametrize("shape,rows", [
    ((2, 4, 4, 200, 200, 128, 128), BLOCK_ROWS),     # every tile kernel
    ((1, 2, 2, 100, 100, 64, 32), BLOCK_ROWS),
    ((1, 4, 4, 2, 2, 128, 128), (8,)),               # the decode kernel
    ((2, 6, 6, 256, 256, 32, 32), (64, 128)),        # small-grid kernels, norms formed in-kernel
    ((1, 2, 2, 100, 100, 16, 16), (64, 128)),
    ((1, 2, 2, 600, 600, 128, 128), (128,)),        # two key halves
    ((1, 2, 2, 600, 600, 32, 32), (128,)),          # two key halves, norms in-kernel
])
def test_yat_tied_keys_with_tiny_eps(shape, rows):
    """k := q and eps = softplus(-20) ~ 2e-9: the diagonal weight is
    (|q|^2 + b)^2 / eps only if the kernel's d2 = |q|^2 + |k|^2 - 2 q.k is
    exactly 0 there (a residual of one rounding unit of |q|^2 would shrink it
    by orders of magnitude), so mass and max_score pin that cancellation."""
    B, Hq, Hkv, Tq, Tk, dk, dv = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", True, seed=26, qk_std=1.5, tied=True)
    inp.eps_raw = np.full_like(inp.eps_raw, -20.0)
    full_check(inp, "yat", True, "yat_tied_tiny_eps", block_rows=rows)


@pytest.mark.parametrize("causal", [True, False])
def test_head_grouped_dispatch(causal):
    # 32 (batch, head) slices: the 256-row kernel hands each XCD its heads in
    # groups of 4 (workgroup i -> XCD i % 8); every tile must still be computed
    # exactly once, with GQA and a ragged last query tile
    inp = make_custom(2, 16, 8, 600, 600, 64, 64, "bf16", causal, seed=27, qk_std=1.5)
    for variant in ("yat", "softmax"):
        full_check(inp, variant, causal, "head_grouped", block_rows=(256,))


def test_kv_splits_more_chunks_than_tiles():
    # 64 chunks over 4 tiles of keys: most chunks are empty and write neutral partials
    inp = make_custom(1, 2, 2, 40, 100, 64, 64, "bf16", False, seed=21)
    for variant in ("yat", "softmax", "stau"):
        full_check(inp, variant, False, "splits64", block_rows=(64,), kv_splits=64)


def test_kv_splits_with_yat_options_and_determinism():
    inp = make_custom(1, 4, 2, 96, 2000, 128, 128, "bf16", False, seed=22, qk_std=1.0)
    full_check(inp, "yat", False, "splits_yat_opts", block_rows=(64, 128), yat_opts=(2, True),
               kv_splits=4)
    q, k, v, prm = to_device(inp)
    a = run_gpu(q, k, v, prm, "softmax", False, kv_splits=6)
    b = run_gpu(q, k, v, prm, "softmax", False, kv_splits=6)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ------------------------------------------------- telemetry (attn_telemetry)

# Tolerances: the pass recomputes each weight in fp32 from the same bf16
# inputs and the forward's fp32 row normaliser, so weights carry ~1e-5
# relative error: entropy |d| <= 2e-3; sparsity may differ by weights that sit
# at the threshold: |d| <= 2 / n + 1e-3; tau* (fp32 per-lane sums, fp64 above)
# |d| <= 2e-3 |ref|.
TEL_SHAPES = [(2, 4, 2, 200, 200, 64, 64, True), (1, 2, 1, 70, 300, 128, 128, False),
              (1, 4, 4, 97, 97, 16, 16, True), (1, 2, 2, 130, 130, 32, 32, False)]


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", TEL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_telemetry_parity(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, "bf16", causal, seed=24, qk_std=2.0)
    say(f"[gpu] telemetry {variant} {shape}")
    q, k, v, prm = to_device(inp)
    _, mass, mx = run_gpu(q, k, v, prm, variant, causal)
    from softmax_free_score_amd import attn
    ent, spa, tau = attn.attn_telemetry(q, k, variant, mass, mx, causal=causal, **prm)
    torch.cuda.synchronize()
    qq, kk, _ = inp.f64()
    r_ent, r_spa, r_tau = oracle.telemetry_np(
        qq, kk, variant, causal=causal, **{n: a.astype(np.float64) for n, a in inp.params().items()})
    n = (np.arange(Tq)[:, None] >= np.arange(Tk)[None, :]).sum(1) if causal else np.full(Tq, Tk)
    assert np.abs(to_np(ent) - r_ent).max() <= 2e-3
    assert np.all(np.abs(to_np(spa) - r_spa) <= 2.0 / n + 1e-3)
    assert np.all(np.abs(to_np(tau) - r_tau) <= 2e-3 * np.abs(r_tau))


@pytest.mark.parametrize("variant", ["yat", "softmax"])
def test_telemetry_full_size_properties(variant):
    wl = WORKLOADS["long_yat"]
    inp = make_inputs(wl)
    say(f"[gpu] telemetry full-size long_yat {variant}")
    q, k, v, prm = to_device(inp)
    _, mass, mx = run_gpu(q, k, v, prm, variant, True)
    from softmax_free_score_amd import attn
    ent, spa, tau = attn.attn_telemetry(q, k, variant, mass, mx, causal=True, **prm)
    torch.cuda.synchronize()
    assert torch.all((ent >= 0) & (ent <= 1 + 1e-5)) and torch.all((spa >= 0) & (spa <= 1))
    assert torch.all(torch.isfinite(tau))
    # row 0 of every head sees one key: entropy 0, sparsity 0
    assert torch.all(ent[:, :, 0] == 0) and torch.all(spa[:, :, 0] == 0)


def test_telemetry_outputs_are_optional_and_sparsity_threshold():
    inp = make_custom(1, 2, 2, 64, 64, 64, 64, "bf16", False, seed=25, qk_std=3.0)
    q, k, v, prm = to_device(inp)
    _, mass, mx = run_gpu(q, k, v, prm, "softmax", False)
    from softmax_free_score_amd import attn
    e1, s1, t1 = attn.attn_telemetry(q, k, "softmax", mass, mx, **prm)
    e2, s2, t2 = attn.attn_telemetry(q, k, "softmax", mass, mx, entropy=False, tau_star=False,
                                     sparsity_threshold=1e-30, **prm)
    torch.cuda.synchronize()
    assert e2 is None and t2 is None and torch.all(s2 <= s1)
    assert float(s1.mean()) > 0.0     # qk_std 3: many weights below 1e-6


# --------------------------------------------------------------- edge cases

@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 64, 64, True), (1, 2, 2, 1, 1, 32, 32, False),
                                   (2, 2, 1, 1, 1000, 128, 128, False),
                                   (1, 1, 1, 5, 3, 16, 32, False)],
                         ids=lambda s: "x".join(map(str, s)))
def test_degenerate_sizes(variant, shape):
    B, Hq, Hkv, Tq, Tk, dk, dv, causal = shape
    for dtype in ("bf16", "f32"):
        inp = make_custom(B, Hq, Hkv, Tq, Tk, dk, dv, dtype, causal, seed=10)
        full_check(inp, variant, causal, f"degenerate_{dtype}",
                   BLOCK_ROWS if dtype == "bf16" else (0,))


def test_empty_batch_is_a_no_op():
    from softmax_free_score_amd import attn
    q = torch.empty((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    out, mass, mx = attn.attn_fwd(q, k, k, "softmax", causal=True)
    assert out.shape == (0, 2, 16, 64)


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_strided_layout_and_null_statistics(variant):
    # tensors stored as [B, T, H, d] and viewed as [B, H, T, d]
    inp = make_custom(2, 4, 2, 150, 150, 64, 128, "bf16", True, seed=11)
    q, k, v, prm = to_device(inp)
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    assert qs.stride(2) == 4 * 64 and ks.stride(2) == 2 * 64
    out_s = torch.empty((2, 150, 4, 128), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    from softmax_free_score_amd import attn
    attn.attn_fwd(qs, ks, vs, variant, causal=True, out=out_s, **prm)
    ref_out, ref_mass, ref_mx = run_gpu(q, k, v, prm, variant, True)
    torch.cuda.synchronize()
    assert torch.equal(out_s, ref_out)
    # no statistics requested: same output
    out_n = torch.empty_like(ref_out)
    lib = attn.load_library()
    desc = attn.make_desc(q, k, v, out_n)
    ws = torch.empty(max(attn.workspace_bytes(q, k, v, variant), 16), dtype=torch.uint8,
                     device="cuda")
    st = attn.call_raw(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(), attn.VARIANTS[variant],
                       prm["b_raw"].data_ptr(), prm["eps_raw"].data_ptr(),
                       prm["log_tau"].data_ptr(), 1, out_n.data_ptr(), 0, 0, ws.data_ptr(),
                       ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.attn_last_error()
    torch.cuda.synchronize()
    assert torch.equal(out_n, ref_out)


# ------------------------------------------------------------- invariances

@pytest.mark.parametrize("rows", BLOCK_ROWS[1:])
@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_causality_and_determinism(variant, rows):
    inp = make_custom(1, 2, 2, 384, 384, 128, 128, "bf16", True, seed=12)
    q, k, v, prm = to_device(inp)
    a = run_gpu(q, k, v, prm, variant, True, block_rows=rows)
    b = run_gpu(q, k, v, prm, variant, True, block_rows=rows)
    for x, y in zip(a, b):
        assert torch.equal(x, y), "two identical calls differ"
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 200:] = -k2[:, :, 200:]
    v2[:, :, 200:] = 3.0
    c = run_gpu(q, k2, v2, prm, variant, True, block_rows=rows)
    for x, y in zip(a, c):
        assert torch.equal(x[:, :, :200], y[:, :, :200]), "a row saw a future key"


@pytest.mark.parametrize("rows", BLOCK_ROWS[1:])
@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_gqa_equals_repeated_kv(variant, rows):
    inp = make_custom(2, 8, 2, 200, 200, 64, 64, "bf16", True, seed=13)
    q, k, v, prm = to_device(inp)
    a = run_gpu(q, k, v, prm, variant, True, block_rows=rows)
    b = run_gpu(q, k.repeat_interleave(4, dim=1).contiguous(),
                v.repeat_interleave(4, dim=1).contiguous(), prm, variant, True, block_rows=rows)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("variant", ["yat", "softmax", "stau"])
def test_unit_values_give_weight_sums(variant):
    inp = make_custom(1, 2, 2, 256, 256, 128, 32, "bf16", True, seed=14)
    q, k, v, prm = to_device(inp)
    v1 = torch.ones_like(v)
    out, mass, _ = run_gpu(q, k, v1, prm, variant, True)
    o = to_np(out)
    if variant == "yat":
        m = to_np(mass)[..., None]
        expect = m / (m + 1e-9)
    else:
        expect = np.ones_like(o)
    # weights are rounded to bf16 before the value contraction: 2^-8 relative
    assert np.abs(o - expect).max() < 8e-3


def test_side_stream_call():
    # a call on a stream other than torch's current one: outputs and workspace
    # are allocated on that stream, and the results are those of the current
    # stream's call bit for bit
    inp = make_custom(2, 8, 4, 700, 700, 128, 128, "bf16", True, seed=21)
    q, k, v, prm = to_device(inp)
    ref = run_gpu(q, k, v, prm, "yat", True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        got = attn.attn_fwd(q, k, v, "yat", causal=True, stream=side, **prm)
        side.synchronize()
        for x, y in zip(ref, got):
            assert torch.equal(x, y)


# ------------------------------------------------- full sizes, every row

FULL = [("long_yat", "yat", False), ("long_yat", "softmax", False), ("long_yat", "yat", True),
        ("stau_gqa", "stau", False), ("cross", "softmax", False), ("cross", "yat", False),
        ("cross", "stau", False), ("gpt_small", "yat", True), ("decode", "yat", False),
        ("decode", "softmax", False), ("decode", "stau", False)]


@pytest.mark.parametrize("name,variant,tied", FULL, ids=lambda x: str(x))
def test_full_size_every_row(name, variant, tied):
    # the benchmark's launch configuration, against the C oracle on every row
    # (OpenMP over rows: about 13 s for long_yat on 16 host cores)
    wl = WORKLOADS[name]
    inp = make_inputs(wl, tied=tied)
    say(f"[gpu] full-size {name} tied={tied} {variant}: every row")
    q, k, v, prm = to_device(inp)
    out, mass, mx = run_gpu(q, k, v, prm, variant, wl.causal)
    got = (to_np(out), to_np(mass), to_np(mx))
    ref = oracle_rows(inp, variant, wl.causal, None)
    check(wl.dtype, got, ref, f"{name}{'_tied' if tied else ''}/{variant}", v_rms=v_rms(inp))
    m = got[1]
    assert (m > 0).all()
    if variant == "softmax":
        assert (m >= 0.999).all()   # the maximal key contributes exp(0) = 1
