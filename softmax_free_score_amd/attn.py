"""ctypes binding of ``libsfs_attn.so`` (the C ABI in ``include/sfs_attn.h``).

Argument marshalling only: shapes, strides and device pointers of torch
tensors go in, the library validates and enqueues the kernels on the current
HIP stream.  Every step of the attention forward runs in the library; there is
no fallback -- without the built library every call raises.

    out, mass, max_score = attn_fwd(q, k, v, "yat", b_raw=..., eps_raw=...,
                                    causal=True)

q [B,Hq,Tq,dk], k [B,Hkv,Tk,dk], v [B,Hkv,Tk,dv] and out [B,Hq,Tq,dv] are
device tensors of one dtype (bfloat16 or float32) whose last axis is
contiguous; any strides on the other axes that are multiples of 16 bytes are
accepted.  b_raw, eps_raw and log_tau are float32 [Hq] device tensors.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

# SFS_ATTN_LIBRARY names another build of the same library (e.g. the host
# code built with sanitizers); by default the in-tree one is loaded.
_LIB_PATH = os.environ.get("SFS_ATTN_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libsfs_attn.so")

ATTN_SOFTMAX, ATTN_YAT, ATTN_STAU = 0, 1, 2
ATTN_F32, ATTN_BF16 = 0, 1
VARIANTS = {"softmax": ATTN_SOFTMAX, "yat": ATTN_YAT, "stau": ATTN_STAU}
STATUS = {0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_UNSUPPORTED",
          -4: "ATTN_ERR_PARAM", -5: "ATTN_ERR_WORKSPACE", -6: "ATTN_ERR_HIP"}
EXPORTS = ("attn_desc_init", "attn_fwd_workspace_bytes", "attn_fwd", "attn_fwd_noalloc",
           "attn_fwd_yat",
           "attn_telemetry_workspace_bytes", "attn_telemetry", "attn_bwd_workspace_bytes",
           "attn_bwd", "attn_status_string", "attn_last_error")
ATTN_YAT_MAX_POWER = 8
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20


class AttnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("Tq", ctypes.c_int64), ("Tk", ctypes.c_int64), ("dk", ctypes.c_int64),
                ("dv", ctypes.c_int64), ("dtype", ctypes.c_int32), ("block_rows", ctypes.c_int32),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
                ("kv_splits", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class AttnYatOpts(ctypes.Structure):
    _fields_ = [("power", ctypes.c_int32), ("bias_free", ctypes.c_int32)]


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Open the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m softmax_free_score_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.attn_desc_init.argtypes = [ctypes.POINTER(AttnDesc), i64, i64, i64, i64, i64, i64,
                                       i64, ctypes.c_int32]
        lib.attn_desc_init.restype = ctypes.c_int
        lib.attn_fwd_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc), ctypes.c_int]
        lib.attn_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_fwd.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                 ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.attn_fwd.restype = ctypes.c_int
        lib.attn_fwd_noalloc.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, ctypes.c_int, vp,
                                         vp, vp, ctypes.c_int, vp, vp, vp, vp]
        lib.attn_fwd_noalloc.restype = ctypes.c_int
        lib.attn_fwd_yat.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp,
                                     ctypes.POINTER(AttnYatOpts), ctypes.c_int, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
        lib.attn_fwd_yat.restype = ctypes.c_int
        lib.attn_telemetry_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc), ctypes.c_int]
        lib.attn_telemetry_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_telemetry.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, ctypes.c_int, vp, vp,
                                       vp, ctypes.c_int, vp, vp, ctypes.c_float, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
        lib.attn_telemetry.restype = ctypes.c_int
        lib.attn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc), ctypes.c_int]
        lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_bwd.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, ctypes.c_int, vp,
                                 vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 ctypes.c_size_t, vp]
        lib.attn_bwd.restype = ctypes.c_int
        lib.attn_status_string.argtypes = [ctypes.c_int]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_desc(q, k, v, out=None, block_rows=0, kv_splits=0) -> AttnDesc:
    """Descriptor from 4-D tensors (strides in elements, last axis contiguous).
    ``block_rows`` 0 lets the library pick the bf16 kernel; 64/128/256 force a
    tile kernel, 8 the decode kernel (at most 8 query rows per key/value head).
    ``kv_splits`` 0 lets the library decide whether to split the keys; 1 never;
    n >= 2 forces n chunks."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t is None:
            continue
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, T, d]")
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name} needs a contiguous last axis")
    B, Hq, Tq, dk = q.shape
    Hkv, Tk, dv = v.shape[1], v.shape[2], v.shape[3]
    if k.shape != (B, Hkv, Tk, dk) or v.shape[0] != B:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    d = AttnDesc()
    d.B, d.Hq, d.Hkv, d.Tq, d.Tk, d.dk, d.dv = B, Hq, Hkv, Tq, Tk, dk, dv
    d.dtype = _dtype_code(q)
    d.block_rows = int(block_rows)
    d.kv_splits = int(kv_splits)
    for field, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        if t is not None:
            getattr(d, field)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    return d


def workspace_bytes(q, k, v, variant, block_rows=0, kv_splits=0) -> int:
    d = make_desc(q, k, v, None, block_rows, kv_splits)
    return int(load_library().attn_fwd_workspace_bytes(ctypes.byref(d),
                                                       VARIANTS.get(variant, variant)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_qkv(q, k, v=None):
    """q, k (and v): 4-D tensors of one supported dtype on one device."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D tensor [B, H, T, d]")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} is {t.dtype}, q is {q.dtype}: they must match")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}: they must match")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported dtype {q.dtype} (bfloat16 or float32)")


def _check_f32(name, t, device, numel, exact=False):
    """A float32 contiguous tensor on ``device`` of ``numel`` elements (at least
    ``numel`` unless ``exact``); None passes (the library checks presence)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
        raise ValueError(f"{name} must be a float32 tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, q on {device}: they must match")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if (t.numel() != numel) if exact else (t.numel() < numel):
        want = "exactly" if exact else "at least"
        raise ValueError(f"{name} has {t.numel()} elements, needs {want} {numel}")


def _check_params(q, Hq, b_raw, eps_raw, log_tau):
    for name, t in (("b_raw", b_raw), ("eps_raw", eps_raw), ("log_tau", log_tau)):
        _check_f32(name, t, q.device, Hq)


def _check_like(name, t, shape, dtype, device):
    """An output tensor given by the caller: this shape, dtype and device, last
    axis contiguous (other strides are the library's to check)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape):
        got = tuple(t.shape) if isinstance(t, torch.Tensor) else type(t).__name__
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {got}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, q on {device}: they must match")


def _check_workspace(workspace, device):
    if workspace is None:
        return
    if not isinstance(workspace, torch.Tensor) or workspace.device != device:
        raise ValueError("workspace must be a tensor on q's device")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _check_on_gpu(q):
    if not q.is_cuda:
        raise ValueError(f"tensors are on {q.device}: the library needs GPU (HIP) device memory")


def _stream_handle(stream, device):
    """(raw stream handle, allocation context): tensors allocated here for a
    call on a stream other than torch's current one are allocated on that
    stream, so the caching allocator does not hand their memory to other work
    before the call's kernels are done with it."""
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream, contextlib.nullcontext()
    handle = stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)
    if handle == torch.cuda.current_stream(device).cuda_stream:
        return handle, contextlib.nullcontext()
    return handle, torch.cuda.stream(torch.cuda.ExternalStream(handle, device=device))


def _prepare(q, k, v, variant, out, mass, max_score, workspace, stream, block_rows,
             kv_splits=0, allocate_workspace=True, params=(None, None, None)):
    # every check on the arguments comes before the first library call
    _check_qkv(q, k, v)
    B, Hq, Tq, _ = q.shape
    dv = v.shape[3]
    _check_like("out", out, (B, Hq, Tq, dv), q.dtype, q.device)
    _check_f32("mass", mass, q.device, B * Hq * Tq, exact=True)
    _check_f32("max_score", max_score, q.device, B * Hq * Tq, exact=True)
    _check_params(q, Hq, *params)
    _check_workspace(workspace, q.device)
    desc = make_desc(q, k, v, out, block_rows, kv_splits)
    _check_on_gpu(q)
    lib = load_library()
    stream, alloc = _stream_handle(stream, q.device)
    need = int(lib.attn_fwd_workspace_bytes(ctypes.byref(desc), variant))
    with alloc:
        if out is None:
            out = torch.empty((B, Hq, Tq, dv), dtype=q.dtype, device=q.device)
            desc = make_desc(q, k, v, out, block_rows, kv_splits)
        if mass is None:
            mass = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
        if max_score is None:
            max_score = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
        if workspace is None and need > 0 and allocate_workspace:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return lib, desc, out, mass, max_score, workspace, ws_bytes, stream


def attn_fwd(q, k, v, variant, b_raw=None, eps_raw=None, log_tau=None, causal=False, out=None,
             mass=None, max_score=None, workspace=None, stream=None, block_rows=0,
             kv_splits=0):
    """Enqueue the fused forward; returns (out, mass, max_score).

    Outputs that are not given are allocated (out like q with d_v columns;
    mass and max_score float32 [B,Hq,Tq]); a workspace of the required size is
    allocated when not given.  ``stream`` defaults to torch's current stream
    on q's device.  Raises AttnError with the library's status on failure."""
    variant = VARIANTS.get(variant, variant)
    lib, desc, out, mass, max_score, workspace, ws_bytes, stream = _prepare(
        q, k, v, variant, out, mass, max_score, workspace, stream, block_rows, kv_splits,
        params=(b_raw, eps_raw, log_tau))
    st = lib.attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), variant, _ptr(b_raw),
                      _ptr(eps_raw), _ptr(log_tau), int(bool(causal)), _ptr(out), _ptr(mass),
                      _ptr(max_score), _ptr(workspace), ws_bytes,
                      ctypes.c_void_p(stream) if stream else None)
    if st != 0:
        raise AttnError(st, lib.attn_last_error().decode())
    return out, mass, max_score


def attn_fwd_noalloc(q, k, v, variant, b_raw=None, eps_raw=None, log_tau=None, causal=False,
                     out=None, mass=None, max_score=None, stream=None, block_rows=0,
                     kv_splits=0):
    """``attn_fwd`` without a workspace: the library's per-GPU scratch of
    ATTN_NOALLOC_SCRATCH_BYTES serves instead, and the library allocates
    nothing.  Outputs that are not given are allocated here, as in
    ``attn_fwd``.  Calls that may overlap on one GPU race on the scratch."""
    variant = VARIANTS.get(variant, variant)
    lib, desc, out, mass, max_score, _, _, stream = _prepare(
        q, k, v, variant, out, mass, max_score, None, stream, block_rows, kv_splits,
        allocate_workspace=False, params=(b_raw, eps_raw, log_tau))
    st = lib.attn_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), variant,
                              _ptr(b_raw), _ptr(eps_raw), _ptr(log_tau), int(bool(causal)),
                              _ptr(out), _ptr(mass), _ptr(max_score),
                              ctypes.c_void_p(stream) if stream else None)
    if st != 0:
        raise AttnError(st, lib.attn_last_error().decode())
    return out, mass, max_score


def attn_fwd_yat(q, k, v, b_raw=None, eps_raw=None, power=1, bias_free=False, causal=False,
                 out=None, mass=None, max_score=None, workspace=None, stream=None, block_rows=0,
                 kv_splits=0):
    """The Yat forward with kernel-family options: numerator (q.k + b)^(2 power),
    and b = 0 exactly when ``bias_free`` (b_raw then unused).  Otherwise as
    ``attn_fwd(..., "yat", ...)``."""
    lib, desc, out, mass, max_score, workspace, ws_bytes, stream = _prepare(
        q, k, v, ATTN_YAT, out, mass, max_score, workspace, stream, block_rows, kv_splits,
        params=(b_raw, eps_raw, None))
    opts = AttnYatOpts(int(power), int(bool(bias_free)))
    st = lib.attn_fwd_yat(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(b_raw),
                          _ptr(eps_raw), ctypes.byref(opts), int(bool(causal)), _ptr(out),
                          _ptr(mass), _ptr(max_score), _ptr(workspace), ws_bytes,
                          ctypes.c_void_p(stream) if stream else None)
    if st != 0:
        raise AttnError(st, lib.attn_last_error().decode())
    return out, mass, max_score


def call_raw(desc: AttnDesc, q, k, v, variant, b_raw, eps_raw, log_tau, causal, out, mass,
             max_score, workspace, workspace_bytes, stream) -> int:
    """The C entry point with raw integer pointers (0 = NULL); returns the status."""
    lib = load_library()
    p = lambda x: ctypes.c_void_p(x) if x else None
    dp = ctypes.byref(desc) if desc is not None else None
    return int(lib.attn_fwd(dp, p(q), p(k), p(v), int(variant), p(b_raw),
                            p(eps_raw), p(log_tau), int(causal), p(out), p(mass), p(max_score),
                            p(workspace), int(workspace_bytes), p(stream)))


def call_raw_noalloc(desc: AttnDesc, q, k, v, variant, b_raw, eps_raw, log_tau, causal, out,
                     mass, max_score, stream) -> int:
    """attn_fwd_noalloc with raw integer pointers (0 = NULL); returns the status."""
    lib = load_library()
    p = lambda x: ctypes.c_void_p(x) if x else None
    dp = ctypes.byref(desc) if desc is not None else None
    return int(lib.attn_fwd_noalloc(dp, p(q), p(k), p(v), int(variant), p(b_raw), p(eps_raw),
                                    p(log_tau), int(causal), p(out), p(mass), p(max_score),
                                    p(stream)))


def call_raw_yat(desc: AttnDesc, q, k, v, b_raw, eps_raw, opts, causal, out, mass, max_score,
                 workspace, workspace_bytes, stream) -> int:
    """attn_fwd_yat with raw integer pointers (0 = NULL) and an AttnYatOpts or
    None; returns the status."""
    lib = load_library()
    p = lambda x: ctypes.c_void_p(x) if x else None
    dp = ctypes.byref(desc) if desc is not None else None
    op = ctypes.byref(opts) if opts is not None else None
    return int(lib.attn_fwd_yat(dp, p(q), p(k), p(v), p(b_raw), p(eps_raw), op, int(causal),
                                p(out), p(mass), p(max_score), p(workspace),
                                int(workspace_bytes), p(stream)))


def attn_telemetry(q, k, variant, mass, max_score=None, b_raw=None, eps_raw=None, log_tau=None,
                   causal=False, sparsity_threshold=1e-6, entropy=True, sparsity=True,
                   tau_star=True, workspace=None, stream=None):
    """One telemetry pass after a forward with the same inputs: returns
    (row_entropy [B,Hq,Tq], row_sparsity [B,Hq,Tq], tau_star [Hq]) as float32
    device tensors (None for the ones not asked for).  ``mass`` and
    ``max_score`` are the forward's outputs."""
    variant = VARIANTS.get(variant, variant)
    _check_qkv(q, k)
    B, Hq, Tq, _ = q.shape
    _check_f32("mass", mass, q.device, B * Hq * Tq, exact=True)
    _check_f32("max_score", max_score, q.device, B * Hq * Tq, exact=True)
    _check_params(q, Hq, b_raw, eps_raw, log_tau)
    _check_workspace(workspace, q.device)
    desc = make_desc(q, k, k, q)   # v and out are not used; k and q give valid shapes
    _check_on_gpu(q)
    lib = load_library()
    stream, alloc = _stream_handle(stream, q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    need = int(lib.attn_telemetry_workspace_bytes(ctypes.byref(desc), variant))
    with alloc:
        ent = torch.empty((B, Hq, Tq), **f32) if entropy else None
        spa = torch.empty((B, Hq, Tq), **f32) if sparsity else None
        tau = torch.empty((Hq,), **f32) if tau_star else None
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.attn_telemetry(ctypes.byref(desc), _ptr(q), _ptr(k), variant, _ptr(b_raw),
                            _ptr(eps_raw), _ptr(log_tau), int(bool(causal)), _ptr(mass),
                            _ptr(max_score), float(sparsity_threshold), _ptr(ent), _ptr(spa),
                            _ptr(tau), _ptr(workspace), ws_bytes,
                            ctypes.c_void_p(stream) if stream else None)
    if st != 0:
        raise AttnError(st, lib.attn_last_error().decode())
    return ent, spa, tau


def bwd_workspace_bytes(q, k, v, variant) -> int:
    d = make_desc(q, k, v, None)
    return int(load_library().attn_bwd_workspace_bytes(ctypes.byref(d),
                                                       VARIANTS.get(variant, variant)))


def attn_bwd(q, k, v, dout, variant, mass, max_score=None, b_raw=None, eps_raw=None,
             log_tau=None, causal=False, dq=None, dk=None, dv=None, param_grads=True,
             workspace=None, stream=None):
    """Enqueue the backward of a forward with the same inputs; returns a dict
    with dq, dk, dv (bf16, laid out like q, k, v) and, when ``param_grads``,
    the per-head parameter gradients of the variant (db_raw and deps_raw for
    Yat, dlog_tau for s^tau; float32 [Hq]).  ``mass`` and ``max_score`` are
    the forward's row statistics (softmax needs both; Yat and s^tau read
    neither and take None); ``dout`` is dL/dout [B, Hq, Tq, dv]."""
    variant = VARIANTS.get(variant, variant)
    _check_qkv(q, k, v)
    B, Hq, Tq, _ = q.shape
    _check_like("dout", dout, (B, Hq, Tq, v.shape[3]), q.dtype, q.device)
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_like(name, t, like.shape, like.dtype, like.device)
        if t is not None and t.stride() != like.stride():
            raise ValueError(f"{name} must have the strides of its input")
    _check_f32("mass", mass, q.device, B * Hq * Tq, exact=True)
    _check_f32("max_score", max_score, q.device, B * Hq * Tq, exact=True)
    _check_params(q, Hq, b_raw, eps_raw, log_tau)
    _check_workspace(workspace, q.device)
    desc = make_desc(q, k, v, dout)
    _check_on_gpu(q)
    lib = load_library()
    stream, alloc = _stream_handle(stream, q.device)
    need = int(lib.attn_bwd_workspace_bytes(ctypes.byref(desc), variant))
    f32 = dict(dtype=torch.float32, device=q.device)
    want_p = bool(param_grads)
    grads = {}
    with alloc:
        for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            grads[name] = t if t is not None else torch.empty_strided(
                like.shape, like.stride(), dtype=like.dtype, device=like.device)
        grads["db_raw"] = torch.empty(Hq, **f32) if want_p and variant == ATTN_YAT else None
        grads["deps_raw"] = torch.empty(Hq, **f32) if want_p and variant == ATTN_YAT else None
        grads["dlog_tau"] = torch.empty(Hq, **f32) if want_p and variant == ATTN_STAU else None
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                      variant, _ptr(b_raw), _ptr(eps_raw), _ptr(log_tau), int(bool(causal)),
                      _ptr(mass), _ptr(max_score), _ptr(grads["dq"]), _ptr(grads["dk"]),
                      _ptr(grads["dv"]), _ptr(grads["db_raw"]), _ptr(grads["deps_raw"]),
                      _ptr(grads["dlog_tau"]), _ptr(workspace), ws_bytes,
                      ctypes.c_void_p(stream) if stream else None)
    if st != 0:
        raise AttnError(st, lib.attn_last_error().decode())
    return grads
