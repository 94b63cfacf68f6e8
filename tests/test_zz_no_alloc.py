"""attn_fwd_noalloc, the forward that allocates nothing, against attn_fwd with a
caller workspace: the same kernels run on the same inputs, so the outputs must
agree bit for bit.  Each case makes two calls in a row, the second on a
smaller problem, so the second runs on a scratch that still holds the first
call's contents."""
import ctypes

import pytest
import torch

from parity import say, to_device
from softmax_free_score_amd import attn
from softmax_free_score_amd.workloads import make_custom

pytestmark = pytest.mark.gpu


def _desc(q, k, v, out, block_rows=0, kv_splits=0):
    B, Hq, Tq, dk = q.shape
    Hkv, Tk, dv = k.shape[1], k.shape[2], v.shape[3]
    d = attn.AttnDesc()
    assert attn.load_library().attn_desc_init(ctypes.byref(d), B, Hq, Hkv, Tq, Tk, dk, dv,
                                              attn.ATTN_BF16) == 0
    d.block_rows, d.kv_splits = block_rows, kv_splits
    return d


def _pair(inp, variant, causal, block_rows=0, kv_splits=0):
    """One problem through both entry points; returns the two result triples."""
    q, k, v, prm = to_device(inp)
    B, Hq, Tq, _ = q.shape
    dv = v.shape[3]
    d = _desc(q, k, v, None, block_rows, kv_splits)
    lib = attn.load_library()
    need = int(lib.attn_fwd_workspace_bytes(ctypes.byref(d), variant))
    assert 0 < need <= attn.ATTN_NOALLOC_SCRATCH_BYTES
    res = []
    for noalloc in (False, True):
        out = torch.full((B, Hq, Tq, dv), float("nan"), dtype=q.dtype, device=q.device)
        mass = torch.full((B, Hq, Tq), float("nan"), dtype=torch.float32, device=q.device)
        mx = torch.full((B, Hq, Tq), float("nan"), dtype=torch.float32, device=q.device)
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), variant, prm["b_raw"].data_ptr(),
                prm["eps_raw"].data_ptr(), prm["log_tau"].data_ptr(), int(causal),
                out.data_ptr(), mass.data_ptr(), mx.data_ptr())
        stream = torch.cuda.current_stream().cuda_stream
        if noalloc:
            st = attn.call_raw_noalloc(d, *args, stream)
        else:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
            st = attn.call_raw(d, *args, ws.data_ptr(), need, stream)
        assert st == 0, lib.attn_last_error().decode()
        torch.cuda.synchronize()
        res.append((out, mass, mx))
    return res


def _same(a, b, label):
    for name, x, y in zip(("out", "mass", "max_score"), a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)), \
            f"{label}: {name} differs"


# (first problem, second smaller problem): (B, Hq, Hkv, Tq, Tk, dk, dv), variant,
# causal, block_rows, kv_splits
CASES = {
    "yat_prefill": (((4, 8, 8, 2048, 2048, 128, 128), attn.ATTN_YAT, True, 0, 0),
                    ((2, 4, 2, 333, 517, 128, 128), attn.ATTN_YAT, False, 0, 0)),
    "yat_keysplit": (((2, 32, 8, 1, 16384, 128, 128), attn.ATTN_YAT, False, 0, 16),
                     ((1, 8, 2, 3, 1000, 128, 128), attn.ATTN_YAT, False, 0, 4)),
    "softmax_decode": (((4, 32, 8, 1, 8192, 128, 128), attn.ATTN_SOFTMAX, False, 0, 0),
                       ((1, 4, 1, 2, 777, 64, 64), attn.ATTN_SOFTMAX, False, 0, 0)),
    "stau_keysplit": (((2, 16, 4, 1, 8192, 128, 128), attn.ATTN_STAU, False, 0, 8),
                      ((1, 16, 4, 1, 999, 128, 128), attn.ATTN_STAU, False, 0, 3)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_matches_workspace_call(case):
    for i, (shape, variant, causal, rows, splits) in enumerate(CASES[case]):
        label = f"{case} call {i + 1}: shape={shape} variant={variant} causal={causal} " \
                f"block_rows={rows} kv_splits={splits}"
        say("noalloc:", label)
        inp = make_custom(*shape, causal=causal, seed=7 + i)
        a, b = _pair(inp, variant, causal, rows, splits)
        assert torch.isfinite(a[0].float()).all(), label
        _same(a, b, label)


def test_noalloc_torch_binding_matches():
    inp = make_custom(2, 8, 4, 300, 300, 128, 128, causal=True, seed=11)
    q, k, v, prm = to_device(inp)
    ref = attn.attn_fwd(q, k, v, attn.ATTN_YAT, causal=True, **prm)
    got = attn.attn_fwd_noalloc(q, k, v, attn.ATTN_YAT, causal=True, **prm)
    torch.cuda.synchronize()
    _same(ref, got, "torch binding")



@pytest.mark.parametrize("case", ["yat_prefill", "stau_keysplit"])
def test_noalloc_in_a_captured_graph(case):
    # the caller the entry point is for: the call captured once into a HIP
    # graph on fixed buffers, then replayed on new inputs copied into them;
    # every replay must equal an eager attn_fwd on the same inputs
    shape, variant, causal, rows, splits = CASES[case][1]
    inputs = [make_custom(*shape, causal=causal, seed=40 + i) for i in range(3)]
    bufs = [t.clone() for t in to_device(inputs[0])[:3]]
    prm = to_device(inputs[0])[3]
    B, Hq, Tq, _ = bufs[0].shape
    out = torch.empty(B, Hq, Tq, bufs[2].shape[3], dtype=bufs[0].dtype, device=bufs[0].device)
    mass = torch.empty(B, Hq, Tq, dtype=torch.float32, device=out.device)
    mx = torch.empty_like(mass)
    kw = dict(causal=causal, block_rows=rows, kv_splits=splits, out=out, mass=mass, max_score=mx,
              **prm)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        attn.attn_fwd_noalloc(*bufs, variant, stream=side.cuda_stream, **kw)  # first call: set-up
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            attn.attn_fwd_noalloc(*bufs, variant, stream=side.cuda_stream, **kw)
    torch.cuda.synchronize()
    for i, inp in enumerate(inputs):
        say(f"noalloc graph {case}: replay {i}")
        q, k, v, _ = to_device(inp)
        for dst, src in zip(bufs, (q, k, v)):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = attn.attn_fwd(q, k, v, variant, causal=causal, block_rows=rows, kv_splits=splits,
                            **prm)
        torch.cuda.synchronize()
        _same(ref, (out, mass, mx), f"{case} replay {i}")
