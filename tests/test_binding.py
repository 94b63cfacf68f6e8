"""The Python binding's own checks, on the CPU: every tensor argument is
checked for dtype, device, contiguity and size before the first library call,
and a bad one raises ValueError.  The library is replaced by a stub that fails
the test if it is reached."""
import pytest
import torch

from softmax_free_score_amd import attn

B, HQ, HKV, T, D = 2, 4, 2, 16, 32


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def reached():
        raise AssertionError("the library was reached before the arguments were checked")
    monkeypatch.setattr(attn, "load_library", reached)


def qkv(dtype=torch.bfloat16):
    q = torch.zeros(B, HQ, T, D, dtype=dtype)
    k = torch.zeros(B, HKV, T, D, dtype=dtype)
    v = torch.zeros(B, HKV, T, D, dtype=dtype)
    return q, k, v


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def fwd(**kw):
    q, k, v = qkv()
    args = dict(q=q, k=k, v=v, variant="yat", b_raw=f32(HQ), eps_raw=f32(HQ))
    args.update(kw)
    return attn.attn_fwd(**args)


BAD_FWD = {
    "k dtype": dict(k=torch.zeros(B, HKV, T, D, dtype=torch.float32)),
    "v dtype": dict(v=torch.zeros(B, HKV, T, D, dtype=torch.float16)),
    "v device": dict(v=torch.zeros(B, HKV, T, D, dtype=torch.bfloat16, device="meta")),
    "q dtype": dict(q=torch.zeros(B, HQ, T, D, dtype=torch.float16),
                    k=torch.zeros(B, HKV, T, D, dtype=torch.float16),
                    v=torch.zeros(B, HKV, T, D, dtype=torch.float16)),
    "k 3-D": dict(k=torch.zeros(HKV, T, D, dtype=torch.bfloat16)),
    "k shape": dict(k=torch.zeros(B, HKV, T + 1, D, dtype=torch.bfloat16)),
    "out shape": dict(out=torch.zeros(B, HQ, T, D + 1, dtype=torch.bfloat16)),
    "out dtype": dict(out=torch.zeros(B, HQ, T, D, dtype=torch.float32)),
    "out device": dict(out=torch.zeros(B, HQ, T, D, dtype=torch.bfloat16, device="meta")),
    "out last axis": dict(out=torch.zeros(B, HQ, D, T, dtype=torch.bfloat16).transpose(2, 3)),
    "mass dtype": dict(mass=torch.zeros(B, HQ, T, dtype=torch.float64)),
    "mass size": dict(mass=f32(B, HQ, T - 1)),
    "mass strided": dict(mass=f32(B, HQ, 2 * T)[:, :, ::2]),
    "max_score size": dict(max_score=f32(B * HQ * T + 1)),
    "max_score device": dict(max_score=torch.zeros(B, HQ, T, device="meta")),
    "b_raw dtype": dict(b_raw=torch.zeros(HQ, dtype=torch.float64)),
    "b_raw size": dict(b_raw=f32(HQ - 1)),
    "eps_raw strided": dict(eps_raw=f32(2 * HQ)[::2]),
    "eps_raw device": dict(eps_raw=torch.zeros(HQ, device="meta")),
    "log_tau size": dict(log_tau=f32(1)),
    "workspace device": dict(workspace=torch.zeros(64, dtype=torch.uint8, device="meta")),
    "workspace strided": dict(workspace=torch.zeros(64, dtype=torch.uint8)[::2]),
}


@pytest.mark.parametrize("case", list(BAD_FWD))
def test_fwd_rejects(case):
    with pytest.raises(ValueError):
        fwd(**BAD_FWD[case])


def test_fwd_host_tensors_rejected():
    # well-formed arguments in host memory: refused before the library
    with pytest.raises(ValueError, match="GPU"):
        fwd(out=torch.zeros(B, HQ, T, D, dtype=torch.bfloat16), mass=f32(B, HQ, T),
            max_score=f32(B, HQ, T), log_tau=f32(HQ))


@pytest.mark.parametrize("case", ["v dtype", "out shape", "mass size", "b_raw size"])
def test_other_forward_entry_points_reject(case):
    q, k, v = qkv()
    args = dict(q=q, k=k, v=v, b_raw=f32(HQ), eps_raw=f32(HQ))
    args.update(BAD_FWD[case])
    with pytest.raises(ValueError):
        attn.attn_fwd_noalloc(variant="yat", **args)
    args.pop("log_tau", None)
    with pytest.raises(ValueError):
        attn.attn_fwd_yat(**args)


def telemetry(**kw):
    q, k, _ = qkv()
    args = dict(q=q, k=k, variant="softmax", mass=f32(B, HQ, T), max_score=f32(B, HQ, T))
    args.update(kw)
    return attn.attn_telemetry(**args)


@pytest.mark.parametrize("kw", [
    dict(k=torch.zeros(B, HKV, T, D, dtype=torch.float32)),
    dict(mass=f32(B, HQ, T + 1)),
    dict(mass=torch.zeros(B, HQ, T, dtype=torch.bfloat16)),
    dict(max_score=torch.zeros(B, HQ, T, device="meta")),
    dict(log_tau=f32(HQ - 1)),
    dict(b_raw=torch.zeros(HQ, dtype=torch.float64)),
    dict(workspace=torch.zeros(8, dtype=torch.uint8, device="meta")),
], ids=["k dtype", "mass size", "mass dtype", "max_score device", "log_tau size",
        "b_raw dtype", "workspace device"])
def test_telemetry_rejects(kw):
    with pytest.raises(ValueError):
        telemetry(**kw)


def test_telemetry_host_tensors_rejected():
    with pytest.raises(ValueError, match="GPU"):
        telemetry()


def bwd(**kw):
    q, k, v = qkv()
    args = dict(q=q, k=k, v=v, dout=torch.zeros(B, HQ, T, D, dtype=torch.bfloat16),
                variant="softmax", mass=f32(B, HQ, T), max_score=f32(B, HQ, T))
    args.update(kw)
    return attn.attn_bwd(**args)


@pytest.mark.parametrize("kw", [
    dict(dout=torch.zeros(B, HQ, T, D + 1, dtype=torch.bfloat16)),
    dict(dout=torch.zeros(B, HQ, T, D, dtype=torch.float32)),
    dict(v=torch.zeros(B, HKV, T, D, dtype=torch.float32)),
    dict(dq=torch.zeros(B, HQ, T, D, dtype=torch.float32)),
    dict(dk=torch.zeros(B, HKV, T + 1, D, dtype=torch.bfloat16)),
    dict(dv=torch.zeros(B, HKV, D, T, dtype=torch.bfloat16).transpose(2, 3)),
    dict(mass=f32(B, HQ, T - 1)),
    dict(max_score=torch.zeros(B, HQ, T, dtype=torch.float64)),
    dict(eps_raw=f32(HQ - 1)),
    dict(workspace=torch.zeros(8, dtype=torch.uint8)[::2]),
], ids=["dout shape", "dout dtype", "v dtype", "dq dtype", "dk shape", "dv strides",
        "mass size", "max_score dtype", "eps_raw size", "workspace strided"])
def test_bwd_rejects(kw):
    with pytest.raises(ValueError):
        bwd(**kw)


def test_bwd_host_tensors_rejected():
    with pytest.raises(ValueError, match="GPU"):
        bwd()
