"""ctypes binding of libmla_paged.so: torch tensors in, C-ABI call out.

Argument marshalling only: every step of the decode runs in the HIP kernels
behind ``include/mla_paged.h``.  torch provides the device memory (inputs,
output, split workspace) and the current stream.  There is no fallback: if the
library is missing or the tensors are not on a GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmla_paged.so"

# mla_status codes (include/mla_paged.h)
MLA_OK = 0


class MlaError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({_status_string(status)})")
        self.status = status


class MlaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("kv_dim", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_scale_blocks", ctypes.c_int64),
        ("scale_groups", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
    ]


class MlaPlan(ctypes.Structure):
    _fields_ = [
        ("row_groups", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("tokens_per_split", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Open the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    vp, u32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    common = [vp, vp, f32p, u32p, u32p, u32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
              vp, ctypes.POINTER(MlaShape), vp, ctypes.c_size_t]
    lib.mla_decode_paged_fp8.argtypes = common + [vp]
    lib.mla_decode_paged_fp8.restype = ctypes.c_int
    lib.mla_decode_paged_fp8_splits.argtypes = common + [ctypes.c_int32, vp]
    lib.mla_decode_paged_fp8_splits.restype = ctypes.c_int
    lib.mla_decode_paged_fp8_profiled.argtypes = common + [ctypes.c_int32, vp, vp, vp]
    lib.mla_decode_paged_fp8_profiled.restype = ctypes.c_int
    lib.mla_decode_paged_fp8_mfma8.argtypes = common + [ctypes.c_int32, vp, vp, vp]
    lib.mla_decode_paged_fp8_mfma8.restype = ctypes.c_int
    lib.mla_decode_paged_fp8_mfma8_kv.argtypes = common + [ctypes.c_int32, vp, vp, vp]
    lib.mla_decode_paged_fp8_mfma8_kv.restype = ctypes.c_int
    lib.mla_decode_paged_fp8_noalloc.argtypes = [vp, vp, f32p, u32p, u32p, u32p, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_float, vp, ctypes.POINTER(MlaShape), ctypes.c_int32, vp]
    lib.mla_decode_paged_fp8_noalloc.restype = ctypes.c_int
    lib.mla_noalloc_scratch_bytes.argtypes = []
    lib.mla_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.mla_decode_paged_fp8_block_offsets.argtypes = common + [ctypes.c_int32, vp, ctypes.c_int32, vp]
    lib.mla_decode_paged_fp8_block_offsets.restype = ctypes.c_int
    lib.mla_decode_paged_fp8_ragged.argtypes = [vp, u32p, vp, f32p, u32p, u32p, u32p, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_float, vp, ctypes.POINTER(MlaShape), vp,
                                                ctypes.c_size_t, ctypes.c_int32, vp]
    lib.mla_decode_paged_fp8_ragged.restype = ctypes.c_int
    bf16_common = [vp, vp, u32p, u32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, vp,
                   ctypes.POINTER(MlaShape), vp, ctypes.c_size_t]
    lib.mla_decode_paged_bf16.argtypes = bf16_common + [vp]
    lib.mla_decode_paged_bf16.restype = ctypes.c_int
    lib.mla_decode_paged_bf16_profiled.argtypes = bf16_common + [ctypes.c_int32, vp, vp, vp]
    lib.mla_decode_paged_bf16_profiled.restype = ctypes.c_int
    lib.mla_decode_paged_fp8_plan.argtypes = [ctypes.POINTER(MlaShape), ctypes.c_int32, ctypes.c_int32,
                                              ctypes.POINTER(MlaPlan)]
    lib.mla_decode_paged_fp8_plan.restype = ctypes.c_int
    lib.mla_append_kv_fp8.argtypes = [vp, vp, f32p, u32p, u32p, u32p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(MlaShape), vp]
    lib.mla_append_kv_fp8.restype = ctypes.c_int
    lib.mla_resolve_pages.argtypes = [u32p, u32p, u32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, u32p, u32p, u32p, vp]
    lib.mla_resolve_pages.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_abi_version.argtypes = []
    lib.mla_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().mla_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - only used inside error paths
        return "unknown"


def mla_abi_version() -> int:
    return int(load_library().mla_abi_version())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(q, blocks, scales, lookup_table) -> MlaShape:
    B, Q, H, D = q.shape
    NB, KVD, NL, P, HKV, D2 = blocks.shape
    return MlaShape(batch=B, num_q_heads=H, head_dim=D, v_dim=512, num_blocks=NB, kv_dim=KVD,
                    num_layers=NL, page_size=P, num_kv_heads=HKV, num_scale_blocks=scales.shape[0],
                    scale_groups=scales.shape[-1], max_pages=lookup_table.shape[1])


def _check_tensor(name, t, dtypes, ndim, device):
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous row-major")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _check_q_len(q, q_len):
    """The kernels stride q and out by q_len rows per request: q_len must be q's
    second dimension (a larger value would read past q and write past out)."""
    if int(q_len) != q.shape[1]:
        raise ValueError(f"q_len ({int(q_len)}) must equal q.shape[1] ({q.shape[1]})")


def _check_shapes(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, out, q_len):
    """Cross-tensor shape checks that the C struct cannot express."""
    B = q.shape[0]
    _check_q_len(q, q_len)
    if blocks.shape[1:5] != scales.shape[1:5]:
        raise ValueError("scales dims 1..4 must equal blocks dims 1..4")
    if blocks.shape[5] != q.shape[3]:
        raise ValueError("head_dim of q and blocks differ")
    if lookup_table.shape[0] != B or cache_lengths.shape[0] != B:
        raise ValueError("lookup_table / cache_lengths batch size differs from q")
    if scales_lookup_table is not None and scales_lookup_table.shape != lookup_table.shape:
        raise ValueError("scales_lookup_table shape must equal lookup_table shape")
    if tuple(out.shape) != (B, q.shape[1], q.shape[2], 512):
        raise ValueError(f"out must be [B, q_len, H, 512], got {tuple(out.shape)}")


def mla_decode_paged_fp8_plan(q_shape, blocks_shape, scales_shape, lookup_shape, q_len, num_splits=0):
    """The library's work plan for these tensor shapes (host-only call)."""
    lib = load_library()
    B, Q, H, D = q_shape
    NB, KVD, NL, P, HKV, _ = blocks_shape
    shp = MlaShape(batch=B, num_q_heads=H, head_dim=D, v_dim=512, num_blocks=NB, kv_dim=KVD,
                   num_layers=NL, page_size=P, num_kv_heads=HKV, num_scale_blocks=scales_shape[0],
                   scale_groups=scales_shape[-1], max_pages=lookup_shape[1])
    plan = MlaPlan()
    st = lib.mla_decode_paged_fp8_plan(ctypes.byref(shp), int(q_len), int(num_splits), ctypes.byref(plan))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_paged_fp8_plan")
    return {"row_groups": plan.row_groups, "num_splits": plan.num_splits,
            "tokens_per_split": plan.tokens_per_split, "grid": plan.grid,
            "workspace_bytes": int(plan.workspace_bytes)}


# Bytes of split completion counters at the start of every split workspace.
SPLIT_FLAG_BYTES = 288 * 1024


def new_workspace(nbytes, device):
    """A device workspace of nbytes (uint8) whose split counters are zero, as
    the library needs before a buffer's first use; later calls keep them zero."""
    ws = torch.empty(max(int(nbytes), SPLIT_FLAG_BYTES), dtype=torch.uint8, device=device)
    ws[:SPLIT_FLAG_BYTES].zero_()
    return ws


def workspace_bytes(q, blocks, scales, lookup_table, q_len, num_splits=0) -> int:
    return mla_decode_paged_fp8_plan(tuple(q.shape), tuple(blocks.shape), tuple(scales.shape),
                                     tuple(lookup_table.shape), q_len, num_splits)["workspace_bytes"]


def mla_decode_paged_fp8(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                         layer_idx, q_len, softmax_scale, out=None, workspace=None, num_splits=None,
                         main_events=None, block_offsets=None, fp8_mfma=None):
    """Decode attention over the paged FP8 cache; returns `out` (bf16 [B, q_len, H, 512]).

    q bf16 [B, q_len, H, 576]; blocks uint8 (E4M3FN bytes) [NB, KVD, NL, P, 1, 576];
    scales float32 [NBs, KVD, NL, P, 1, 576 / granularity]; lookup_table and
    scales_lookup_table (or None) uint32 ids stored in int32 tensors [B, max_pages];
    cache_lengths uint32 in an int32 tensor [B].  workspace: a uint8 device
    tensor from new_workspace() (its split counters zeroed once; every call
    leaves them zero), or None to have one allocated per the plan.
    num_splits: None for the automatic plan, or an explicit count.
    main_events: optional (begin, end) raw hipEvent_t handles that take the
    decode launch's own start and end timestamps.
    block_offsets: optional int64 device tensor [B, max_blocks, 2] (debug): the
    decode kernel writes the row and scale offsets it computed for every
    16-key block it loads (mla_decode_paged_fp8_block_offsets in the C ABI).
    fp8_mfma: None (default), "v" (the value contraction on the FP8 MFMA,
    mla_decode_paged_fp8_mfma8) or "kv" (both contractions,
    mla_decode_paged_fp8_mfma8_kv); per-token scales only.
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("mla_decode_paged_fp8 runs on the GPU only; got tensors on " + str(dev))
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], q.shape[2], 512), dtype=torch.bfloat16, device=dev)
    _check_tensor("q", q, (torch.bfloat16,), 4, dev)
    _check_tensor("blocks", blocks, (torch.uint8, torch.float8_e4m3fn), 6, dev)
    _check_tensor("scales", scales, (torch.float32,), 6, dev)
    _check_tensor("lookup_table", lookup_table, (torch.int32,), 2, dev)
    if scales_lookup_table is not None:
        _check_tensor("scales_lookup_table", scales_lookup_table, (torch.int32,), 2, dev)
    _check_tensor("cache_lengths", cache_lengths, (torch.int32,), 1, dev)
    _check_tensor("out", out, (torch.bfloat16,), 4, dev)
    _check_shapes(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, out, q_len)
    shp = _shape(q, blocks, scales, lookup_table)
    want = 0 if num_splits is None else int(num_splits)
    if workspace is None:
        need = workspace_bytes(q, blocks, scales, lookup_table, q_len, want)
        workspace = new_workspace(need, dev) if need > 0 else None
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(blocks), _ptr(scales), _ptr(lookup_table), _ptr(scales_lookup_table),
            _ptr(cache_lengths), int(layer_idx), int(q_len), float(softmax_scale), _ptr(out),
            ctypes.byref(shp), ws_ptr, ws_bytes)
    if fp8_mfma is not None:
        if fp8_mfma not in ("v", "kv"):
            raise ValueError('fp8_mfma must be None, "v" or "kv"')
        if block_offsets is not None:
            raise ValueError("fp8_mfma does not combine with block_offsets")
        ev = main_events if main_events is not None else (None, None)
        fn = lib.mla_decode_paged_fp8_mfma8 if fp8_mfma == "v" else lib.mla_decode_paged_fp8_mfma8_kv
        st = fn(*args, want, ctypes.c_void_p(ev[0]), ctypes.c_void_p(ev[1]), _stream_handle(dev))
    elif block_offsets is not None:
        if (block_offsets.dtype != torch.int64 or block_offsets.dim() != 3 or block_offsets.shape[0] != q.shape[0]
                or block_offsets.shape[2] != 2 or not block_offsets.is_contiguous() or block_offsets.device != dev):
            raise ValueError("block_offsets must be a contiguous int64 [B, max_blocks, 2] tensor on the device")
        st = lib.mla_decode_paged_fp8_block_offsets(*args, want, _ptr(block_offsets), int(block_offsets.shape[1]),
                                                    _stream_handle(dev))
    elif main_events is not None:
        st = lib.mla_decode_paged_fp8_profiled(*args, want, ctypes.c_void_p(main_events[0]),
                                               ctypes.c_void_p(main_events[1]), _stream_handle(dev))
    elif num_splits is None:
        st = lib.mla_decode_paged_fp8(*args, _stream_handle(dev))
    else:
        st = lib.mla_decode_paged_fp8_splits(*args, int(num_splits), _stream_handle(dev))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_paged_fp8")
    return out


def mla_decode_paged_fp8_ragged(q, q_offsets, blocks, scales, lookup_table, scales_lookup_table,
                                cache_lengths, layer_idx, softmax_scale, max_q_len=None, out=None,
                                workspace=None, num_splits=None):
    """Decode with per-request query counts; returns `out` (bf16 [T, H, 512]).

    q bf16 [T, H, 576] packed request after request; q_offsets int32 [B + 1]
    on the device (request b owns rows q_offsets[b] .. q_offsets[b + 1] - 1);
    the cache arguments as for mla_decode_paged_fp8.  max_q_len: the largest
    per-request count; when None the offsets are copied to the host (a
    synchronisation), checked, and the largest count taken from them.
    workspace / num_splits as for mla_decode_paged_fp8.
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("mla_decode_paged_fp8_ragged runs on the GPU only; got tensors on " + str(dev))
    _check_tensor("q", q, (torch.bfloat16,), 3, dev)
    _check_tensor("q_offsets", q_offsets, (torch.int32,), 1, dev)
    _check_tensor("blocks", blocks, (torch.uint8, torch.float8_e4m3fn), 6, dev)
    _check_tensor("scales", scales, (torch.float32,), 6, dev)
    _check_tensor("lookup_table", lookup_table, (torch.int32,), 2, dev)
    if scales_lookup_table is not None:
        _check_tensor("scales_lookup_table", scales_lookup_table, (torch.int32,), 2, dev)
    _check_tensor("cache_lengths", cache_lengths, (torch.int32,), 1, dev)
    T, H, D = q.shape
    B = lookup_table.shape[0]
    if q_offsets.shape[0] != B + 1 or cache_lengths.shape[0] != B:
        raise ValueError("q_offsets must hold batch + 1 entries and cache_lengths batch entries")
    if blocks.shape[1:5] != scales.shape[1:5]:
        raise ValueError("scales dims 1..4 must equal blocks dims 1..4")
    if blocks.shape[5] != D:
        raise ValueError("head_dim of q and blocks differ")
    if scales_lookup_table is not None and scales_lookup_table.shape != lookup_table.shape:
        raise ValueError("scales_lookup_table shape must equal lookup_table shape")
    if max_q_len is None:
        offs = q_offsets.cpu().tolist()
        counts = [offs[b + 1] - offs[b] for b in range(B)]
        if offs[0] != 0 or offs[-1] != T or min(counts) < 0:
            raise ValueError("q_offsets must be non-decreasing from 0 to q.shape[0]")
        max_q_len = max(1, max(counts))
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    _check_tensor("out", out, (torch.bfloat16,), 3, dev)
    if tuple(out.shape) != (T, H, 512):
        raise ValueError(f"out must be [T, H, 512], got {tuple(out.shape)}")
    NB, KVD, NL, P, HKV, _ = blocks.shape
    shp = MlaShape(batch=B, num_q_heads=H, head_dim=D, v_dim=512, num_blocks=NB, kv_dim=KVD, num_layers=NL,
                   page_size=P, num_kv_heads=HKV, num_scale_blocks=scales.shape[0],
                   scale_groups=scales.shape[-1], max_pages=lookup_table.shape[1])
    want = 0 if num_splits is None else int(num_splits)
    if workspace is None:
        need = mla_decode_paged_fp8_plan((B, int(max_q_len), H, D), tuple(blocks.shape), tuple(scales.shape),
                                         tuple(lookup_table.shape), int(max_q_len), want)["workspace_bytes"]
        workspace = new_workspace(need, dev) if need > 0 else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.mla_decode_paged_fp8_ragged(_ptr(q), _ptr(q_offsets), _ptr(blocks), _ptr(scales), _ptr(lookup_table),
                                         _ptr(scales_lookup_table), _ptr(cache_lengths), int(layer_idx),
                                         int(max_q_len), float(softmax_scale), _ptr(out), ctypes.byref(shp),
                                         _ptr(workspace), ws_bytes, want, _stream_handle(dev))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_paged_fp8_ragged")
    return out


def mla_decode_paged_fp8_noalloc(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                                 layer_idx, q_len, softmax_scale, out, num_splits=0):
    """mla_decode_paged_fp8 through the entry point that allocates nothing: the
    split partials use the library's per-GPU scratch.  `out` (bf16 [B, q_len, H,
    512]) must be given; nothing is allocated here either.  num_splits 0 picks
    the automatic plan within the scratch."""
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("mla_decode_paged_fp8_noalloc runs on the GPU only; got tensors on " + str(dev))
    _check_tensor("q", q, (torch.bfloat16,), 4, dev)
    _check_tensor("blocks", blocks, (torch.uint8, torch.float8_e4m3fn), 6, dev)
    _check_tensor("scales", scales, (torch.float32,), 6, dev)
    _check_tensor("lookup_table", lookup_table, (torch.int32,), 2, dev)
    if scales_lookup_table is not None:
        _check_tensor("scales_lookup_table", scales_lookup_table, (torch.int32,), 2, dev)
    _check_tensor("cache_lengths", cache_lengths, (torch.int32,), 1, dev)
    _check_tensor("out", out, (torch.bfloat16,), 4, dev)
    _check_shapes(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, out, q_len)
    shp = _shape(q, blocks, scales, lookup_table)
    st = lib.mla_decode_paged_fp8_noalloc(_ptr(q), _ptr(blocks), _ptr(scales), _ptr(lookup_table),
                                          _ptr(scales_lookup_table), _ptr(cache_lengths), int(layer_idx),
                                          int(q_len), float(softmax_scale), _ptr(out), ctypes.byref(shp),
                                          int(num_splits), _stream_handle(dev))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_paged_fp8_noalloc")
    return out


def mla_decode_paged_bf16(q, blocks, lookup_table, cache_lengths, layer_idx, q_len, softmax_scale,
                          out=None, workspace=None, num_splits=None, main_events=None):
    """Decode attention over an unquantized paged cache; returns `out` (bf16 [B, q_len, H, 512]).

    q bf16 [B, q_len, H, 576]; blocks bf16 [NB, KVD, NL, P, 1, 576];
    lookup_table uint32 ids in an int32 tensor [B, max_pages]; cache_lengths
    uint32 in an int32 tensor [B].  workspace, num_splits and main_events as
    for mla_decode_paged_fp8 (the split plan is the same).
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("mla_decode_paged_bf16 runs on the GPU only; got tensors on " + str(dev))
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], q.shape[2], 512), dtype=torch.bfloat16, device=dev)
    _check_tensor("q", q, (torch.bfloat16,), 4, dev)
    _check_tensor("blocks", blocks, (torch.bfloat16,), 6, dev)
    _check_tensor("lookup_table", lookup_table, (torch.int32,), 2, dev)
    _check_tensor("cache_lengths", cache_lengths, (torch.int32,), 1, dev)
    _check_tensor("out", out, (torch.bfloat16,), 4, dev)
    B = q.shape[0]
    _check_q_len(q, q_len)
    if blocks.shape[5] != q.shape[3]:
        raise ValueError("head_dim of q and blocks differ")
    if lookup_table.shape[0] != B or cache_lengths.shape[0] != B:
        raise ValueError("lookup_table / cache_lengths batch size differs from q")
    if tuple(out.shape) != (B, q.shape[1], q.shape[2], 512):
        raise ValueError(f"out must be [B, q_len, H, 512], got {tuple(out.shape)}")
    NB, KVD, NL, P, HKV, D = blocks.shape
    shp = MlaShape(batch=B, num_q_heads=q.shape[2], head_dim=q.shape[3], v_dim=512, num_blocks=NB,
                   kv_dim=KVD, num_layers=NL, page_size=P, num_kv_heads=HKV, num_scale_blocks=1,
                   scale_groups=1, max_pages=lookup_table.shape[1])
    want = 0 if num_splits is None else int(num_splits)
    if workspace is None:
        need = mla_decode_paged_fp8_plan(tuple(q.shape), tuple(blocks.shape), (1, KVD, NL, P, HKV, 1),
                                         tuple(lookup_table.shape), q_len, want)["workspace_bytes"]
        workspace = new_workspace(need, dev) if need > 0 else None
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(blocks), _ptr(lookup_table), _ptr(cache_lengths), int(layer_idx), int(q_len),
            float(softmax_scale), _ptr(out), ctypes.byref(shp), ws_ptr, ws_bytes)
    if main_events is not None or num_splits is not None:
        ev = main_events if main_events is not None else (None, None)
        st = lib.mla_decode_paged_bf16_profiled(*args, want, ctypes.c_void_p(ev[0]), ctypes.c_void_p(ev[1]),
                                                _stream_handle(dev))
    else:
        st = lib.mla_decode_paged_bf16(*args, _stream_handle(dev))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_paged_bf16")
    return out


def mla_append_kv_fp8(kv_new, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                      layer_idx, q_len, num_q_heads=128):
    """Quantise the latent rows of the q_len new tokens of every request into the paged
    FP8 cache, in place (blocks and scales are written); returns (blocks, scales).

    kv_new bf16 [B, q_len, 576]; blocks uint8 (E4M3FN bytes) [NB, KVD, NL, P, 1, 576];
    scales float32 [NBs, KVD, NL, P, 1, 576 / granularity]; tables and cache_lengths as
    for mla_decode_paged_fp8 (cache_lengths count the new tokens).  num_q_heads only
    fills the shape description the library validates.
    """
    lib = load_library()
    dev = kv_new.device
    if dev.type != "cuda":
        raise ValueError("mla_append_kv_fp8 runs on the GPU only; got tensors on " + str(dev))
    _check_tensor("kv_new", kv_new, (torch.bfloat16,), 3, dev)
    _check_tensor("blocks", blocks, (torch.uint8, torch.float8_e4m3fn), 6, dev)
    _check_tensor("scales", scales, (torch.float32,), 6, dev)
    _check_tensor("lookup_table", lookup_table, (torch.int32,), 2, dev)
    if scales_lookup_table is not None:
        _check_tensor("scales_lookup_table", scales_lookup_table, (torch.int32,), 2, dev)
    _check_tensor("cache_lengths", cache_lengths, (torch.int32,), 1, dev)
    B, Q, D = kv_new.shape
    if Q != q_len or D != blocks.shape[-1] or lookup_table.shape[0] != B or cache_lengths.shape[0] != B:
        raise ValueError("mla_append_kv_fp8: kv_new, tables and cache_lengths disagree on batch / q_len / depth")
    NB, KVD, NL, P, HKV, _ = blocks.shape
    shp = MlaShape(batch=B, num_q_heads=int(num_q_heads), head_dim=D, v_dim=512, num_blocks=NB, kv_dim=KVD,
                   num_layers=NL, page_size=P, num_kv_heads=HKV, num_scale_blocks=scales.shape[0],
                   scale_groups=scales.shape[-1], max_pages=lookup_table.shape[1])
    st = lib.mla_append_kv_fp8(_ptr(kv_new), _ptr(blocks), _ptr(scales), _ptr(lookup_table),
                               _ptr(scales_lookup_table), _ptr(cache_lengths), int(layer_idx), int(q_len),
                               ctypes.byref(shp), _stream_handle(dev))
    if st != MLA_OK:
        raise MlaError(st, "mla_append_kv_fp8")
    return blocks, scales


def mla_resolve_pages(lookup_table, scales_lookup_table, cache_lengths, page_size, max_tokens):
    """Device-side page resolution (debug): (page, slot, spage) int32 tensors [B, max_tokens]
    holding uint32 bits; 0xFFFFFFFF past each request's length."""
    lib = load_library()
    dev = lookup_table.device
    B, max_pages = lookup_table.shape
    outs = [torch.empty((B, max_tokens), dtype=torch.int32, device=dev) for _ in range(3)]
    st = lib.mla_resolve_pages(_ptr(lookup_table), _ptr(scales_lookup_table), _ptr(cache_lengths),
                               int(B), int(max_pages), int(page_size), int(max_tokens),
                               _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _stream_handle(dev))
    if st != MLA_OK:
        raise MlaError(st, "mla_resolve_pages")
    return tuple(outs)
