"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad calls with the documented status before touching
the device.  Pointers here are fake (never dereferenced: validation fails, or
no device is present, before any launch)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT
from softmax_free_score_amd import attn

HEADER = os.path.join(ROOT, "include", "sfs_attn.h")
OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_PARAM, ERR_WS, ERR_HIP = 0, -1, -2, -3, -4, -5, -6
A, K, V, O, BR, ER, LT, M, X, W = (0x10000 * i for i in range(1, 11))


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(attn_\w+)\s*\(", text, flags=re.M))


def test_library_exports_every_declared_function():
    lib = attn.load_library()
    declared = header_functions()
    assert declared == set(attn.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def desc(B=1, Hq=2, Hkv=1, Tq=64, Tk=64, dk=64, dv=64, dtype=attn.ATTN_BF16):
    d = attn.AttnDesc()
    assert attn.load_library().attn_desc_init(ctypes.byref(d), B, Hq, Hkv, Tq, Tk, dk, dv,
                                              dtype) == OK
    return d


def call(d, variant=attn.ATTN_SOFTMAX, causal=1, q=A, k=K, v=V, out=O, b=BR, e=ER, lt=LT,
         mass=M, mx=X, ws=W, ws_bytes=1 << 20):
    return attn.call_raw(d, q, k, v, variant, b, e, lt, causal, out, mass, mx, ws, ws_bytes, 0)


def test_desc_init_strides():
    d = desc(B=2, Hq=4, Hkv=2, Tq=10, Tk=12, dk=32, dv=16)
    assert list(d.q_stride) == [4 * 10 * 32, 10 * 32, 32]
    assert list(d.k_stride) == [2 * 12 * 32, 12 * 32, 32]
    assert list(d.v_stride) == [2 * 12 * 16, 12 * 16, 16]
    assert list(d.o_stride) == [4 * 10 * 16, 10 * 16, 16]
    assert attn.load_library().attn_desc_init(None, 1, 1, 1, 1, 1, 16, 16, 0) == ERR_NULL


def test_null_pointers():
    assert attn.call_raw(None, A, K, V, 0, 0, 0, 0, 0, O, 0, 0, 0, 0, 0) == ERR_NULL
    for kw in ("q", "k", "v", "out"):
        assert call(desc(), **{kw: 0}) == ERR_NULL


@pytest.mark.parametrize("field,value", [("B", -1), ("Hq", 0), ("Hkv", 0), ("Tq", -1),
                                         ("Tk", 0), ("dk", 0), ("dv", -2)])
def test_bad_sizes(field, value):
    d = desc()
    setattr(d, field, value)
    assert call(d, causal=0) == ERR_SHAPE


def test_head_grouping_and_causal_shape():
    assert call(desc(Hq=3, Hkv=2)) == ERR_SHAPE
    assert call(desc(Tq=32, Tk=64), causal=1) == ERR_SHAPE


def test_unsupported():
    assert call(desc(dk=48)) == ERR_UNSUP
    assert call(desc(dv=256)) == ERR_UNSUP
    assert call(desc(dtype=7)) == ERR_UNSUP
    assert call(desc(), variant=3) == ERR_UNSUP
    assert call(desc(), q=A + 8) == ERR_UNSUP        # misaligned base
    assert call(desc(), mass=M + 2) == ERR_UNSUP     # misaligned statistics
    d = desc()
    d.k_stride[2] = 68                               # 136 bytes: not a multiple of 16
    assert call(d) == ERR_UNSUP
    d = desc()
    d.v_stride[2] = 32                               # rows overlap
    assert call(d) == ERR_UNSUP
    d = desc(Tq=70000, Tk=70000, dk=128)
    d.q_stride[2] = 1 << 14                          # one slice spans >= 2^31 bytes
    assert call(d) == ERR_UNSUP


@pytest.mark.parametrize("rows,dtype,status", [(32, attn.ATTN_BF16, ERR_UNSUP),
                                               (512, attn.ATTN_BF16, ERR_UNSUP),
                                               (-64, attn.ATTN_BF16, ERR_UNSUP),
                                               (64, attn.ATTN_F32, ERR_UNSUP),
                                               (64, attn.ATTN_BF16, ERR_HIP),
                                               (128, attn.ATTN_BF16, ERR_HIP),
                                               (256, attn.ATTN_BF16, ERR_HIP)])
def test_block_rows(rows, dtype, status):
    # valid choices pass validation and then fail on the missing device
    d = desc(dtype=dtype)
    assert d.block_rows == 0                          # attn_desc_init: library's choice
    d.block_rows = rows
    assert call(d) == status


def test_missing_per_head_parameters():
    assert call(desc(), variant=attn.ATTN_YAT, b=0) == ERR_PARAM
    assert call(desc(), variant=attn.ATTN_YAT, e=0) == ERR_PARAM
    assert call(desc(), variant=attn.ATTN_STAU, lt=0) == ERR_PARAM


def test_workspace_rules():
    lib = attn.load_library()
    d = desc(B=2, Hq=4, Hkv=2, Tq=100, Tk=100)
    need = lib.attn_fwd_workspace_bytes(ctypes.byref(d), attn.ATTN_YAT)
    assert need == 2 * 4 * 128 * 4                   # |k|^2 + b per query head, rows padded to 64
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(d), attn.ATTN_SOFTMAX) == 0
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(d), attn.ATTN_STAU) == 0
    assert lib.attn_fwd_workspace_bytes(None, attn.ATTN_YAT) == 0
    assert call(d, variant=attn.ATTN_YAT, ws=0) == ERR_WS
    assert call(d, variant=attn.ATTN_YAT, ws_bytes=need - 4) == ERR_WS
    assert call(d, variant=attn.ATTN_YAT, ws=W + 4) == ERR_WS


def call_noalloc(d, variant=attn.ATTN_SOFTMAX, causal=1, q=A, k=K, v=V, out=O, b=BR, e=ER,
                 lt=LT, mass=M, mx=X):
    return attn.call_raw_noalloc(d, q, k, v, variant, b, e, lt, causal, out, mass, mx, 0)


def test_noalloc_rules():
    lib = attn.load_library()
    # 64 batches x 64 query heads x 4096 keys of |k|^2 + b: 64 MiB > the scratch
    big = desc(B=64, Hq=64, Hkv=64, Tq=4096, Tk=4096, dk=128, dv=128)
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(big), attn.ATTN_YAT) > \
        attn.ATTN_NOALLOC_SCRATCH_BYTES
    assert call_noalloc(big, variant=attn.ATTN_YAT) == ERR_WS
    assert "ATTN_NOALLOC_SCRATCH_BYTES" in lib.attn_last_error().decode()
    # the ordinary checks come first, as in attn_fwd
    assert call_noalloc(None) == ERR_NULL
    assert call_noalloc(desc(), out=0) == ERR_NULL
    assert call_noalloc(desc(Tq=64, Tk=32)) == ERR_SHAPE
    assert call_noalloc(desc(), variant=attn.ATTN_YAT, b=0) == ERR_PARAM
    assert call_noalloc(desc(B=0), q=0, k=0, v=0, out=0) == OK


def test_noalloc_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert call_noalloc(desc(), variant=attn.ATTN_YAT) == ERR_HIP
    assert call_noalloc(desc(), variant=attn.ATTN_SOFTMAX) == ERR_HIP


@pytest.mark.parametrize("B,Hq,Tq,Tk", [
    (2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1),   # products overflow int64
    (2 ** 31, 1, 1, 1),                                     # an extent past 32 bits
    (2 ** 16, 2 ** 8, 2 ** 8, 2 ** 8),                      # 2^32 query rows
    (2 ** 10, 2 ** 10, 1, 2 ** 21),                         # 2^41 key rows
])
def test_oversized_problems_are_refused(B, Hq, Tq, Tk):
    lib = attn.load_library()
    d = attn.AttnDesc()
    assert lib.attn_desc_init(ctypes.byref(d), 1, 1, 1, 1, 1, 64, 64, attn.ATTN_BF16) == OK
    d.B, d.Hq, d.Hkv, d.Tq, d.Tk = B, Hq, 1, Tq, Tk
    for variant in (attn.ATTN_SOFTMAX, attn.ATTN_YAT, attn.ATTN_STAU):
        assert lib.attn_fwd_workspace_bytes(ctypes.byref(d), variant) == 0
        assert lib.attn_bwd_workspace_bytes(ctypes.byref(d), variant) == 0
        assert lib.attn_telemetry_workspace_bytes(ctypes.byref(d), variant) == 0
        assert call(d, variant=variant, causal=0) == ERR_UNSUP
        assert call_noalloc(d, variant=variant, causal=0) == ERR_UNSUP
    d.dk = d.dv = 8192
    d.B, d.Hq, d.Tq, d.Tk = 1, 1, 1, 1
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(d), attn.ATTN_YAT) == 0
    assert call(d, variant=attn.ATTN_YAT) == ERR_UNSUP


def test_empty_problem_is_a_no_op():
    assert call(desc(B=0), q=0, k=0, v=0, out=0) == OK
    assert call(desc(Tq=0, Tk=5), causal=0, q=0, k=0, v=0, out=0) == OK


def test_valid_call_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert call(desc(), variant=attn.ATTN_SOFTMAX) == ERR_HIP
    assert "hip" in attn.load_library().attn_last_error().decode().lower()


def test_status_strings():
    lib = attn.load_library()
    for code in (OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_PARAM, ERR_WS, ERR_HIP):
        assert lib.attn_status_string(code)
    assert lib.attn_status_string(99) == b"unknown status"


def call_yat(d, opts, b=BR, e=ER, causal=1):
    return attn.call_raw_yat(d, A, K, V, b, e, opts, causal, O, M, X, W, 1 << 20, 0)


@pytest.mark.parametrize("opts,b,status", [
    (attn.AttnYatOpts(0, 0), BR, ERR_UNSUP),                       # power below 1
    (attn.AttnYatOpts(attn.ATTN_YAT_MAX_POWER + 1, 0), BR, ERR_UNSUP),
    (attn.AttnYatOpts(2, 0), 0, ERR_PARAM),                        # b_raw needed
    (attn.AttnYatOpts(2, 1), 0, ERR_HIP),                          # bias-free: b_raw unused
    (None, BR, ERR_HIP),                                           # NULL opts: standard kernel
    (attn.AttnYatOpts(attn.ATTN_YAT_MAX_POWER, 1), BR, ERR_HIP)])
def test_yat_options_validation(opts, b, status):
    assert call_yat(desc(), opts, b=b) == status


def test_yat_options_need_eps_and_desc():
    assert call_yat(desc(), attn.AttnYatOpts(1, 1), e=0) == ERR_PARAM
    assert call_yat(None, None) == ERR_NULL


@pytest.mark.parametrize("splits,dtype,rows,reserved,status", [
    (-1, attn.ATTN_BF16, 0, 0, ERR_UNSUP),
    (65, attn.ATTN_BF16, 0, 0, ERR_UNSUP),
    (2, attn.ATTN_F32, 0, 0, ERR_UNSUP),          # splitting is a bf16-path feature
    (2, attn.ATTN_BF16, 256, 0, ERR_UNSUP),       # not with the 256-row kernel
    (0, attn.ATTN_BF16, 0, 1, ERR_UNSUP),         # reserved must be 0
    (2, attn.ATTN_BF16, 64, 0, ERR_HIP),          # valid: fails only for want of a device
    (64, attn.ATTN_BF16, 128, 0, ERR_HIP),
    (1, attn.ATTN_F32, 0, 0, ERR_HIP)])
def test_kv_splits_validation(splits, dtype, rows, reserved, status):
    d = desc(dtype=dtype)
    assert d.kv_splits == 0 and d.reserved == 0     # attn_desc_init: library's choice
    d.kv_splits, d.block_rows, d.reserved = splits, rows, reserved
    assert call(d, ws_bytes=1 << 30) == status


def ws(d, variant):
    return attn.load_library().attn_fwd_workspace_bytes(ctypes.byref(d), variant)


def test_workspace_bytes_with_splits():
    # decode-like: 1 query row against 4096 keys -> the plan splits the keys
    d = desc(B=2, Hq=8, Hkv=2, Tq=1, Tk=4096, dk=128, dv=128)
    assert ws(d, attn.ATTN_SOFTMAX) > 0
    d.kv_splits = 1                                   # no split: softmax needs nothing
    assert ws(d, attn.ATTN_SOFTMAX) == 0
    d.kv_splits = 3                                   # 3 chunks x 16 rows x (128 + 4) floats
    assert ws(d, attn.ATTN_SOFTMAX) == 3 * 16 * 132 * 4
    nk = 2 * 8 * 4096 * 4                             # Yat: |k|^2 + b rows first (256-aligned)
    assert ws(d, attn.ATTN_YAT) == nk + 3 * 16 * 132 * 4
    d.dtype = attn.ATTN_F32
    assert ws(d, attn.ATTN_SOFTMAX) == 0


def call_tel(d, variant=attn.ATTN_SOFTMAX, mass=M, mx=X, thr=1e-6, ent=O, spa=O + 0x100,
             tau=O + 0x200, b=BR, e=ER, lt=LT):
    lib = attn.load_library()
    p = lambda x: ctypes.c_void_p(x) if x else None
    return lib.attn_telemetry(ctypes.byref(d) if d is not None else None, p(A), p(K), variant,
                              p(b), p(e), p(lt), 1, p(mass), p(mx), ctypes.c_float(thr), p(ent),
                              p(spa), p(tau), p(W), 1 << 30, None)


def test_telemetry_validation():
    assert call_tel(desc()) == ERR_HIP                               # valid, no device
    assert call_tel(desc(dtype=attn.ATTN_F32)) == ERR_UNSUP
    assert call_tel(desc(), mass=0) == ERR_NULL
    assert call_tel(desc(), mx=0) == ERR_NULL                        # softmax needs max_score
    assert call_tel(desc(), variant=attn.ATTN_YAT, mx=0) == ERR_HIP  # Yat does not
    assert call_tel(desc(), ent=0, spa=0, tau=0) == ERR_NULL
    assert call_tel(desc(), thr=0.0) == ERR_PARAM
    assert call_tel(desc(), variant=attn.ATTN_YAT, b=0) == ERR_PARAM
    assert call_tel(None) == ERR_NULL


def test_telemetry_workspace_bytes():
    lib = attn.load_library()
    d = desc(B=2, Hq=4, Hkv=2, Tq=130, Tk=100, dk=64, dv=64)
    n_qt = 3                                                          # 130 rows / 64
    tau_bytes = 4 * 2 * n_qt * 8 * 8
    assert lib.attn_telemetry_workspace_bytes(ctypes.byref(d), attn.ATTN_SOFTMAX) == tau_bytes
    nk = 2 * 2 * 128 * 4                                              # |k|^2 rows, pitch 128
    assert lib.attn_telemetry_workspace_bytes(ctypes.byref(d), attn.ATTN_YAT) == \
        (nk + 255) // 256 * 256 + tau_bytes


DO, DQ, DKG, DVG, GB, GE, GT = (0x200000 + 0x10000 * i for i in range(7))


def call_bwd(d, variant=attn.ATTN_SOFTMAX, causal=1, q=A, k=K, v=V, dout=DO, mass=M,
             mx=X, dq=DQ, dk=DKG, dv=DVG, b=BR, e=ER, lt=LT, gb=GB, ge=GE, gt=GT, ws=W,
             ws_bytes=1 << 30):
    lib = attn.load_library()
    p = lambda x: ctypes.c_void_p(x) if x else None
    return lib.attn_bwd(ctypes.byref(d) if d is not None else None, p(q), p(k), p(v),
                        p(dout), variant, p(b), p(e), p(lt), causal, p(mass), p(mx), p(dq),
                        p(dk), p(dv), p(gb), p(ge), p(gt), p(ws), ws_bytes, None)


def test_bwd_validation():
    assert call_bwd(desc()) == ERR_HIP                               # valid, no device
    assert call_bwd(None) == ERR_NULL
    assert call_bwd(desc(dtype=attn.ATTN_F32)) == ERR_UNSUP
    for kw in ("q", "k", "v", "dout", "dq", "dk", "dv", "mass"):
        assert call_bwd(desc(), **{kw: 0}) == ERR_NULL, kw
    assert call_bwd(desc(), mx=0) == ERR_NULL                        # softmax needs max_score
    assert call_bwd(desc(), variant=attn.ATTN_YAT, mx=0) == ERR_HIP  # Yat does not
    assert call_bwd(desc(), variant=attn.ATTN_YAT, mass=0, mx=0) == ERR_HIP  # nor the mass
    assert call_bwd(desc(), variant=attn.ATTN_STAU, mass=0, mx=0) == ERR_HIP  # s^tau neither
    assert call_bwd(desc(), variant=attn.ATTN_YAT, b=0) == ERR_PARAM
    assert call_bwd(desc(), variant=attn.ATTN_STAU, lt=0) == ERR_PARAM
    # parameter gradients are optional
    assert call_bwd(desc(), variant=attn.ATTN_YAT, gb=0, ge=0) == ERR_HIP
    assert call_bwd(desc(), dq=DQ + 8) == ERR_UNSUP                  # misaligned
    assert call_bwd(desc(), variant=attn.ATTN_YAT, gb=GB + 2) == ERR_UNSUP
    assert call_bwd(desc(Tq=64, Tk=32)) == ERR_SHAPE                 # causal needs Tq == Tk
    assert call_bwd(desc(dk=48)) == ERR_UNSUP
    assert call_bwd(desc(), ws=0) == ERR_WS
    assert call_bwd(desc(), ws_bytes=16) == ERR_WS
    # empty problems: B == 0 enqueues nothing; Tq == 0 still writes dk = dv = 0
    assert call_bwd(desc(B=0)) == OK
    assert call_bwd(desc(Tq=0), causal=0) == ERR_HIP
    assert call_bwd(desc(Tq=0), causal=0, dk=0) == ERR_NULL


def test_bwd_workspace_bytes():
    lib = attn.load_library()
    d = desc(B=2, Hq=4, Hkv=2, Tq=130, Tk=100, dk=64, dv=64)
    rows = 2 * 4 * 192 * 4                                    # Tq pitch 192 (multiple of 64)
    n_qt = 2                                                  # 130 rows / 128
    prm = 4 * 2 * n_qt * 2 * 8
    al = lambda x: (x + 255) // 256 * 256
    ws = lambda v: lib.attn_bwd_workspace_bytes(ctypes.byref(d), v)
    assert ws(attn.ATTN_SOFTMAX) == 2 * al(rows)
    assert ws(attn.ATTN_STAU) == 2 * al(rows) + prm
    nk = 2 * 4 * 128 * 4                                      # |k|^2 + b per query head
    assert ws(attn.ATTN_YAT) == al(nk) + 3 * al(rows) + prm
    assert ws(7) == 0
    d.dtype = attn.ATTN_F32
    assert ws(attn.ATTN_SOFTMAX) == 0


@pytest.mark.parametrize("shape,rows,splits,dtype,status", [
    ((1, 2, 1, 4, 64), 8, 0, attn.ATTN_BF16, ERR_HIP),    # 2 x 4 = 8 packed rows: valid
    ((1, 2, 1, 5, 64), 8, 0, attn.ATTN_BF16, ERR_UNSUP),  # 10 rows per kv head
    ((1, 8, 1, 1, 64), 8, 0, attn.ATTN_BF16, ERR_HIP),
    ((1, 8, 1, 1, 64), 8, 2, attn.ATTN_BF16, ERR_UNSUP),  # the decode kernel chunks by itself
    ((1, 8, 1, 1, 64), 8, 0, attn.ATTN_F32, ERR_UNSUP)])
def test_decode_kernel_validation(shape, rows, splits, dtype, status):
    B, Hq, Hkv, Tq, Tk = shape
    d = desc(B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, dtype=dtype)
    d.block_rows, d.kv_splits = rows, splits
    assert call(d, causal=0, ws_bytes=1 << 30) == status


def test_decode_kernel_workspace():
    # 4 query rows per kv head: the decode kernel, 256-key chunks, partials for
    # every chunk (2 x 8 x 1 = 16 rows x (128 + 4) floats), also when one chunk
    d = desc(B=2, Hq=8, Hkv=2, Tq=1, Tk=4096, dk=128, dv=128)
    assert ws(d, attn.ATTN_SOFTMAX) == 16 * 16 * 132 * 4
    assert ws(d, attn.ATTN_YAT) == 16 * 16 * 132 * 4     # no |k|^2 pre-pass buffer
    d = desc(B=2, Hq=8, Hkv=2, Tq=1, Tk=100, dk=128, dv=128)
    assert ws(d, attn.ATTN_SOFTMAX) == 1 * 16 * 132 * 4
    d.block_rows = 64                                    # forced tile kernel: no partials
    assert ws(d, attn.ATTN_SOFTMAX) == 0

