"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host (before any HIP call),
with the documented status codes.  No compute call is made here."""

import ctypes
import os
import re

import pytest

from mla_decode_attention_paged_amd import binding
from mla_decode_attention_paged_amd.binding import MlaPlan, MlaShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_paged.h")

OK, NULL, SHAPE, RANGE, UNSUP, WS, HIP = range(7)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mla_status|const char\*|int32_t|size_t)\s+(mla_\w+)\s*\(",
                                 text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.lib_path()):
        pytest.fail("libmla_paged.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 7, names
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert binding.mla_abi_version() == 5
    for code in range(7):
        assert lib.mla_status_string(code).decode()
    assert lib.mla_status_string(99).decode() == "unknown status"


def good_shape(**kw):
    d = dict(batch=2, num_q_heads=128, head_dim=576, v_dim=512, num_blocks=64, kv_dim=1, num_layers=1,
             page_size=64, num_kv_heads=1, num_scale_blocks=64, scale_groups=1, max_pages=8)
    d.update(kw)
    return MlaShape(**d)


def call(lib, shape, *, layer=0, q_len=1, sm=0.07, nulls=(), ws=None, ws_bytes=0, splits=None):
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(7)]
    for i in nulls:
        fake[i] = None
    q, blocks, scales, lt, cl, out, _ = fake
    args = (q, blocks, scales, lt, None, cl, layer, q_len, ctypes.c_float(sm), out,
            ctypes.byref(shape) if shape is not None else None, ws, ws_bytes)
    if splits is None:
        return lib.mla_decode_paged_fp8(*args, None)
    return lib.mla_decode_paged_fp8_splits(*args, splits, None)


@pytest.mark.parametrize("idx", range(6))
def test_null_pointers_rejected(lib, idx):
    assert call(lib, good_shape(), nulls=(idx,)) == NULL


def test_null_shape_rejected(lib):
    assert call(lib, None) == NULL


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(num_q_heads=-1), SHAPE), (dict(page_size=0), SHAPE),
    (dict(scale_groups=5), SHAPE),            # 576 % 5 != 0: granularity must divide head_dim
    (dict(v_dim=600), SHAPE),
    (dict(head_dim=512, scale_groups=1), UNSUP), (dict(v_dim=256), UNSUP),
    (dict(num_kv_heads=2), UNSUP), (dict(scale_groups=3), UNSUP), (dict(page_size=24), UNSUP),
    (dict(num_q_heads=70000), UNSUP),
])
def test_bad_shapes_rejected(lib, kw, code):
    assert call(lib, good_shape(**kw)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(layer=1), RANGE), (dict(layer=-1), RANGE), (dict(q_len=0), RANGE),
    (dict(sm=0.0), RANGE), (dict(sm=float("nan")), RANGE), (dict(splits=-2), RANGE),
])
def test_bad_ranges_rejected(lib, kw, code):
    assert call(lib, good_shape(), **kw) == code


def test_explicit_splits_need_workspace(lib):
    assert call(lib, good_shape(max_pages=64), splits=4) == WS
    assert call(lib, good_shape(max_pages=64), splits=4, ws=ctypes.c_void_p(0x9000), ws_bytes=16) == WS


def plan(lib, shape, q_len=1, splits=0):
    p = MlaPlan()
    st = lib.mla_decode_paged_fp8_plan(ctypes.byref(shape), q_len, splits, ctypes.byref(p))
    return st, p


def test_plan_covers_the_key_range(lib):
    for B, H, Q, maxp, P in [(16, 128, 1, 64, 64), (1, 128, 1, 1024, 128), (64, 128, 1, 128, 64),
                             (128, 128, 4, 512, 64), (2, 16, 1, 7, 16)]:
        st, p = plan(lib, good_shape(batch=B, num_q_heads=H, max_pages=maxp, page_size=P,
                                     num_blocks=maxp * B), q_len=Q)
        assert st == OK
        assert p.row_groups == (Q * H + 31) // 32
        assert p.tokens_per_split % 128 == 0
        assert p.num_splits * p.tokens_per_split >= maxp * P
        assert (p.num_splits - 1) * p.tokens_per_split < maxp * P
        assert p.grid % 8 == 0 and p.grid >= B * ((p.row_groups + 1) // 2) * p.num_splits
        if p.num_splits == 1:
            assert p.workspace_bytes == 0
        else:
            units = B * p.row_groups * p.num_splits
            # 288 KiB of split completion flags, then O and lse partials
            assert p.workspace_bytes == 294912 + units * 32 * 512 * 4 + units * 32 * 4


def test_plan_explicit_splits_clamped(lib):
    st, p = plan(lib, good_shape(max_pages=2, page_size=64), splits=50)   # 128 keys -> 1 chunk
    assert st == OK and p.num_splits == 1


def test_split_plans_limited_to_the_merge_counters(lib):
    # 8192 (request, row-group pair) units have completion counters; more
    # units run unsplit (automatic plan) or are refused (explicit count)
    shape = good_shape(batch=8193, num_q_heads=64, max_pages=256, page_size=64, num_blocks=64)
    st, p = plan(lib, shape)
    assert st == OK and p.num_splits == 1 and p.workspace_bytes == 0
    st, p = plan(lib, shape, splits=2)
    assert st == UNSUP
    shape = good_shape(batch=8192, num_q_heads=64, max_pages=256, page_size=64, num_blocks=64)
    st, p = plan(lib, shape, splits=2)
    assert st == OK and p.num_splits == 2


def test_resolve_rejects_bad_args(lib):
    f = ctypes.c_void_p(0x1000)
    assert lib.mla_resolve_pages(None, None, f, 2, 4, 16, 64, f, f, f, None) == NULL
    assert lib.mla_resolve_pages(f, None, f, 0, 4, 16, 64, f, f, f, None) == SHAPE
    assert lib.mla_resolve_pages(f, None, f, 2, 4, 16, 0, f, f, f, None) == SHAPE


def call_append(lib, shape, *, layer=0, q_len=1, nulls=()):
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(5)]
    for i in nulls:
        fake[i] = None
    kv, blocks, scales, lt, cl = fake
    return lib.mla_append_kv_fp8(kv, blocks, scales, lt, None, cl, layer, q_len,
                                 ctypes.byref(shape) if shape is not None else None, None)


@pytest.mark.parametrize("idx", range(5))
def test_append_null_pointers_rejected(lib, idx):
    assert call_append(lib, good_shape(), nulls=(idx,)) == NULL


@pytest.mark.parametrize("kw,shape_kw,code", [
    (dict(layer=1), {}, RANGE), (dict(layer=-1), {}, RANGE), (dict(q_len=0), {}, RANGE),
    ({}, dict(batch=0), SHAPE), ({}, dict(scale_groups=5), SHAPE), ({}, dict(scale_groups=3), UNSUP),
    ({}, dict(head_dim=512), UNSUP), ({}, dict(page_size=24), UNSUP),
])
def test_append_bad_arguments_rejected(lib, kw, shape_kw, code):
    assert call_append(lib, good_shape(**shape_kw), **kw) == code
    assert call_append(lib, None) == NULL


def call_bf16(lib, shape, *, layer=0, q_len=1, sm=0.07, nulls=()):
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(5)]
    for i in nulls:
        fake[i] = None
    q, blocks, lt, cl, out = fake
    return lib.mla_decode_paged_bf16(q, blocks, lt, cl, layer, q_len, ctypes.c_float(sm), out,
                                     ctypes.byref(shape) if shape is not None else None, None, 0, None)


@pytest.mark.parametrize("idx", range(5))
def test_bf16_null_pointers_rejected(lib, idx):
    assert call_bf16(lib, good_shape(), nulls=(idx,)) == NULL


@pytest.mark.parametrize("kw,shape_kw,code", [
    (dict(layer=1), {}, RANGE), (dict(q_len=0), {}, RANGE), (dict(sm=-1.0), {}, RANGE),
    ({}, dict(batch=0), SHAPE), ({}, dict(head_dim=512), UNSUP), ({}, dict(page_size=24), UNSUP),
    ({}, dict(num_kv_heads=2), UNSUP),
])
def test_bf16_bad_arguments_rejected(lib, kw, shape_kw, code):
    assert call_bf16(lib, good_shape(**shape_kw), **kw) == code
    assert call_bf16(lib, None) == NULL


def test_bf16_ignores_scale_fields():
    """The scale fields of the shape do not apply to an unquantized cache: values
    that the FP8 entry rejects pass the host checks here (checked with a NULL q so
    that nothing is launched)."""
    lib = binding.load_library()
    for kw in (dict(scale_groups=5), dict(scale_groups=0, num_scale_blocks=0)):
        assert call(lib, good_shape(**kw)) in (SHAPE, UNSUP)
        assert call_bf16(lib, good_shape(**kw), nulls=(0,)) == NULL
        assert call_bf16(lib, good_shape(**kw), layer=5) == RANGE


@pytest.mark.parametrize("idx", [0, 1, 5])
def test_misaligned_pointers_rejected(lib, idx):
    """q, blocks and out must be 16-byte aligned (checked before any HIP call)."""
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(6)]
    fake[idx] = ctypes.c_void_p(0x1000 * (idx + 1) + 8)
    q, blocks, scales, lt, cl, out = fake
    st = lib.mla_decode_paged_fp8(q, blocks, scales, lt, None, cl, 0, 1, ctypes.c_float(0.07), out,
                                  ctypes.byref(good_shape()), None, 0, None)
    assert st == UNSUP
    if idx != 2:
        st = lib.mla_decode_paged_bf16(q, blocks, lt, cl, 0, 1, ctypes.c_float(0.07), out,
                                       ctypes.byref(good_shape()), None, 0, None)
        assert st == UNSUP


def test_misaligned_table_rejected(lib):
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(6)]
    q, blocks, scales, lt, cl, out = fake
    lt = ctypes.c_void_p(0x4002)
    st = lib.mla_decode_paged_fp8(q, blocks, scales, lt, None, cl, 0, 1, ctypes.c_float(0.07), out,
                                  ctypes.byref(good_shape()), None, 0, None)
    assert st == UNSUP


def test_plan_two_waves_for_large_batches(lib):
    """With >= 32 requests the automatic plan sizes for two waves of workgroups
    (the kernel deals key ranges largest first), as long as a split keeps at
    least 2048 keys; otherwise one wave.  (CPU: the CU count defaults to 256.)"""
    def splits(B, maxp, P=64, Q=1):
        st, p = plan(lib, good_shape(batch=B, max_pages=maxp, page_size=P, num_blocks=maxp * B), q_len=Q)
        assert st == OK
        return p.num_splits, p.tokens_per_split
    assert splits(64, 128) == (4, 2048)         # 128 units -> 512 workgroups
    assert splits(16, 64) == (8, 512)           # few requests: one wave
    assert splits(4, 1024, P=128) == (32, 4096)
    assert splits(32, 16) == (4, 256)           # two waves would cut splits below 2048 keys
    assert splits(300, 16)[0] == 1              # more units than compute units already


def test_block_offsets_entry_rejects_bad_args(lib):
    """The debug entry with the decode kernel's own resolution record checks its
    extra arguments on the host: a NULL record, a non-positive or too small
    block count (one record per 16 keys of max_pages * page_size) and a
    misaligned record are rejected before anything is launched."""
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(6)]
    q, blocks, scales, lt, cl, out = fake
    f = lib.mla_decode_paged_fp8_block_offsets

    def go(rec, nblk, shape=None):
        return f(q, blocks, scales, lt, None, cl, 0, 1, ctypes.c_float(0.07), out,
                 ctypes.byref(shape or good_shape()), None, 0, 0, rec, nblk, None)
    rec = ctypes.c_void_p(0x20000)
    assert go(None, 64) == NULL
    assert go(rec, 0) == SHAPE
    assert go(rec, 31) == SHAPE                      # 8 pages x 64 keys = 512 keys = 32 blocks
    assert go(ctypes.c_void_p(0x20004), 32) == UNSUP
    assert go(rec, 32, good_shape(batch=0)) == SHAPE


def test_binding_checks_q_len_against_q():
    """The kernels stride q and out by q_len rows per request, so the binding
    refuses a q_len that differs from q's second dimension (on meta tensors:
    no device is needed and nothing is launched)."""
    import torch
    meta = torch.device("meta")
    q = torch.empty((2, 4, 128, 576), dtype=torch.bfloat16, device=meta)
    blocks = torch.empty((8, 1, 1, 64, 1, 576), dtype=torch.uint8, device=meta)
    scales = torch.empty((8, 1, 1, 64, 1, 1), dtype=torch.float32, device=meta)
    lt = torch.empty((2, 4), dtype=torch.int32, device=meta)
    cl = torch.empty((2,), dtype=torch.int32, device=meta)
    out = torch.empty((2, 4, 128, 512), dtype=torch.bfloat16, device=meta)
    binding._check_shapes(q, blocks, scales, lt, None, cl, out, 4)
    for bad in (1, 3, 5):
        with pytest.raises(ValueError, match="q_len"):
            binding._check_shapes(q, blocks, scales, lt, None, cl, out, bad)
    with pytest.raises(ValueError, match="scales dims"):
        binding._check_shapes(q, blocks, scales[:, :, :, :32], lt, None, cl, out, 4)
    with pytest.raises(ValueError, match="scales_lookup_table"):
        binding._check_shapes(q, blocks, scales, lt, lt[:, :2], cl, out, 4)


def test_ragged_entry_rejects_bad_args(lib):
    """The per-request query-count entry checks its offsets pointer and the usual
    arguments on the host (max_q_len plays q_len's part) before any launch."""
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(7)]
    q, offs, blocks, scales, lt, cl, out = fake
    f = lib.mla_decode_paged_fp8_ragged

    def go(offsets, max_q_len=4, shape=None, layer=0):
        return f(q, offsets, blocks, scales, lt, None, cl, layer, max_q_len, ctypes.c_float(0.07), out,
                 ctypes.byref(shape or good_shape()), None, 0, 0, None)
    assert go(None) == NULL
    assert go(ctypes.c_void_p(0x2002)) == UNSUP                # not 4-byte aligned
    assert go(offs, max_q_len=0) == RANGE
    assert go(offs, layer=3) == RANGE
    assert go(offs, shape=good_shape(batch=0)) == SHAPE
