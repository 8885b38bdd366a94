"""FP64 CPU oracle for MLA decode over a paged FP8 KV cache with separately stored scales.

THIS IS TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import or call it.  The HIP
path never imports it, and it imports nothing from the HIP path.

What it computes, and where each piece comes from
--------------------------------------------------
Storage and indexing follow two Modular API pages:

* "generic_get_paged_cache_with_scales" (Mojo function page, section "Args"):
  - ``blocks``  is ``[num_blocks, kv_dim, num_layers, page_size, num_heads, head_dim]``;
  - ``scales``  is ``[num_blocks, kv_dim, num_layers, page_size, num_heads,
    head_dim_granularity]``;
  - ``lookup_table`` is ``[batch_size, max_pages]`` of uint32 page ids;
  - ``cache_lengths`` is ``[batch_size]`` of uint32;
  - ``max_prompt_length`` is the query length (here ``q_len``);
  - ``scales_lookup_table`` (optional) is a second ``[batch_size, max_pages]``
    table for when the scale pages carry their own ids; when it is absent the
    scale pages resolve through ``lookup_table``.
* "KVCacheScalesMHAOperand" (Mojo struct page, description and the
  ``scales_raw_ptr`` method): per-token scales live in the scales field of the
  K cache when ``quantization_granularity`` equals the head size, and the scale
  element type is Float32.

The attention itself (multi-head latent attention decode: a 576-wide latent
key of which the first 512 dims are the value, one latent KV head shared by all
query heads) is named on the "KVLoad2CvtProducer" page (MLA decode, FP8 KV
tiles converted for the QK depth ``q_depth``) and by the workload description.

Readings taken where the pages are silent (each listed in the design doc):
  R1  cache_lengths[b] counts every valid cached token, the q_len new ones
      included; query row i (0-based among the q_len new tokens) sees keys
      j <= L_b - q_len + i.
  R2  kv_dim index 0 holds the latent cache; kv head 0 is the single latent head.
  R3  scale group of element d is floor(d / granularity); groups are contiguous.
  R4  dequantised value = e4m3fn_value(code) * scale.
  R5  "FP8" is OCP E4M3FN (bias 7, max 448, no infinities, NaN = S.1111.111).
  R6  scales are float32.
  R7  V_j = K_j[:dv] with the same scales (dv = 512 for the MLA workloads).
  R8  softmax_scale multiplies the full-depth dot product; q already carries rope.
  R9  rows with no visible key give O = 0 and lse = -inf.
  R16 per-request query counts ("generic_get_paged_cache_with_scales", Args:
      ``max_prompt_length`` is the largest query length of the batch, so the
      requests' own lengths may differ; "KVCacheScalesMHAOperand",
      ``create_ragged_tma_tile``: ragged rows): the queries of all requests are
      packed request after request along the first axis, request b owning
      rows [q_offsets[b], q_offsets[b + 1]) of an offsets array of batch + 1
      non-decreasing entries starting at 0; its count n_b may be 0 (no rows)
      and R1 applies to it with q_len = n_b.

Everything is evaluated in float64 with no blocking, fusion or reordering: the
gather is a per-token integer loop over the page table, and the contractions are
plain numpy dot products.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "E4M3FN_TABLE",
    "e4m3fn_value",
    "bf16_round",
    "resolve",
    "gather_dequant",
    "attention_rows",
    "decode",
    "decode_range",
    "decode_ragged",
    "merge_partials",
]


# --------------------------------------------------------------------------- FP8
def e4m3fn_value(code: int) -> float:
    """Value of one OCP E4M3FN byte (reading R5).

    sign = bit 7, exponent = bits 6..3 with bias 7, mantissa = bits 2..0.
    Exponent field 0 is subnormal: 2^-6 * m/8.  Field 15 with mantissa 7 is
    NaN; there is no infinity, so field 15 with m < 7 is an ordinary normal.
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m / 8.0, -6)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E4M3FN_TABLE.setflags(write=False)


# --------------------------------------------------------------------------- BF16
def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range
    (normal >= 2^-126, subnormal spacing 2^-133).  The rounding is done once,
    directly from float64 (no intermediate float32 step).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    mant, exp = np.frexp(xf)             # xf = mant * 2^exp, 0.5 <= |mant| < 1
    # quantum of the bf16 grid at this magnitude: 2^(exp-8) for normals,
    # 2^-133 below the normal range
    q_exp = np.maximum(exp - 8, -133)
    scaled = np.ldexp(xf, -q_exp)        # exact: power-of-two scaling
    r = np.ldexp(np.rint(scaled), q_exp)  # np.rint rounds half to even
    # overflow past the largest bf16 (0x7F7F = (2 - 2^-7) * 2^127) goes to inf
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


# ---------------------------------------------------------------- page resolution
def resolve(lookup_table, scales_lookup_table, cache_lengths, page_size):
    """Resolve every valid token of every request to (page id, slot, scale page id).

    Follows the lookup-table arguments of generic_get_paged_cache_with_scales:
    token t of request b lives in page ``lookup_table[b, t // page_size]`` at
    slot ``t % page_size``; its scales live in page
    ``scales_lookup_table[b, t // page_size]`` when that table is given, else in
    the same page id as the values.

    Returns a list with one int64 array of shape [L_b, 3] per request.
    """
    lt = np.asarray(lookup_table)
    slt = lt if scales_lookup_table is None else np.asarray(scales_lookup_table)
    out = []
    for b in range(lt.shape[0]):
        L = int(cache_lengths[b])
        rows = np.empty((L, 3), dtype=np.int64)
        for t in range(L):
            col = t // page_size
            rows[t, 0] = int(lt[b, col])
            rows[t, 1] = t % page_size
            rows[t, 2] = int(slt[b, col])
        out.append(rows)
    return out


def gather_dequant(blocks, scales, resolved_rows, layer_idx, granularity):
    """Dequantised latent rows K_j (float64 [L, head_dim]) of one request.

    ``blocks`` holds raw E4M3FN bytes (uint8); element d of token j is
    ``blocks[page, 0, layer, slot, 0, d]`` (reading R2) and its scale is
    ``scales[spage, 0, layer, slot, 0, d // granularity]`` (readings R3, R4, R6).
    The product of a 4-bit and a 24-bit significand is exact in float64.
    """
    head_dim = blocks.shape[-1]
    groups = np.arange(head_dim) // granularity
    L = resolved_rows.shape[0]
    K = np.empty((L, head_dim), dtype=np.float64)
    for j in range(L):
        page, slot, spage = (int(v) for v in resolved_rows[j])
        codes = blocks[page, 0, layer_idx, slot, 0, :]
        s = scales[spage, 0, layer_idx, slot, 0, :].astype(np.float64)
        K[j] = E4M3FN_TABLE[codes] * s[groups]
    return K


# ------------------------------------------------------------------ attention
def attention_rows(q_rows, K, n_visible, softmax_scale, dv):
    """Softmax attention of query rows against the first ``n_visible`` keys.

    q_rows: float64 [R, head_dim]; K: float64 [L, head_dim]; V = K[:, :dv]
    (reading R7).  Scores are ``softmax_scale * q . k`` over the full depth
    (reading R8).  Returns (O [R, dv], lse [R], weights [R, n_visible]) where
    lse = log(sum_j exp(score_j)) in natural log; with no visible key
    O = 0 and lse = -inf (reading R9).
    """
    R = q_rows.shape[0]
    if n_visible <= 0:
        return np.zeros((R, dv)), np.full(R, -np.inf), np.zeros((R, 0))
    Kv = K[:n_visible]
    scores = softmax_scale * (q_rows @ Kv.T)              # [R, n]
    m = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - m)
    denom = e.sum(axis=1, keepdims=True)
    w = e / denom
    O = w @ Kv[:, :dv]
    lse = (m + np.log(denom))[:, 0]
    return O, lse, w


def _check_args(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                layer_idx, q_len):
    B, Q, H, D = q.shape
    if blocks.ndim != 6 or scales.ndim != 6:
        raise ValueError("blocks and scales are 6-D")
    if blocks.shape[-1] != D:
        raise ValueError("head_dim of q and blocks differ")
    if blocks.shape[4] != 1:
        raise ValueError("MLA has one latent KV head")
    if Q != q_len:
        raise ValueError("q.shape[1] must equal q_len")
    if not (0 <= layer_idx < blocks.shape[2]):
        raise ValueError("layer_idx out of range")
    if scales_lookup_table is not None and \
            np.asarray(scales_lookup_table).shape != np.asarray(lookup_table).shape:
        raise ValueError("scales_lookup_table shape must equal lookup_table shape")
    for b in range(B):
        if int(cache_lengths[b]) < 0:
            raise ValueError("negative cache length")


def decode(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
           layer_idx, q_len, softmax_scale, dv=512, batches=None, return_lse=False):
    """MLA decode over the paged FP8 cache: O[b, i, h, :dv] in float64.

    q: float [B, q_len, H, head_dim] (bf16 values); blocks: uint8 E4M3FN codes
    [num_blocks, kv_dim, num_layers, page_size, 1, head_dim]; scales: float32
    [num_scale_blocks, kv_dim, num_layers, page_size, 1, head_dim/granularity];
    lookup_table / scales_lookup_table: [B, max_pages] page ids;
    cache_lengths: [B].  ``batches`` restricts the work to a subset of requests
    (other rows are left as NaN) for sampled checks at large sizes.
    """
    q = np.asarray(q, dtype=np.float64)
    _check_args(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                layer_idx, q_len)
    B, Q, H, D = q.shape
    P = blocks.shape[3]
    G = D // scales.shape[-1]
    if G * scales.shape[-1] != D:
        raise ValueError("head_dim must be a multiple of the scale granularity")
    lt = np.asarray(lookup_table)
    slt = None if scales_lookup_table is None else np.asarray(scales_lookup_table)
    O = np.full((B, Q, H, dv), np.nan)
    lse = np.full((B, Q, H), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(cache_lengths[b])
        rows = resolve(lt[b:b + 1], None if slt is None else slt[b:b + 1], [L], P)[0]
        K = gather_dequant(blocks, scales, rows, layer_idx, G)
        for i in range(Q):
            n_vis = max(0, min(L, L - Q + i + 1))        # reading R1
            o, l, _ = attention_rows(q[b, i], K, n_vis, softmax_scale, dv)
            O[b, i] = o
            lse[b, i] = l
    return (O, lse) if return_lse else O


def decode_ragged(q, q_offsets, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                  layer_idx, softmax_scale, dv=512, requests=None, return_lse=False):
    """MLA decode with per-request query counts (reading R16): O[t, h, :dv].

    q: float [T, H, head_dim], the queries of request b in rows
    q_offsets[b] .. q_offsets[b + 1] - 1 (T = q_offsets[-1]); the other
    arguments as for ``decode``.  Query i (0-based) of request b sees keys
    j <= L_b - n_b + i with n_b = q_offsets[b + 1] - q_offsets[b] (reading
    R1 per request).  ``requests`` restricts the work to a subset (other rows
    are left as NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    offs = [int(x) for x in np.asarray(q_offsets).reshape(-1)]
    B = len(offs) - 1
    T, H, D = q.shape
    if B < 1 or offs[0] != 0 or offs[-1] != T or any(offs[b + 1] < offs[b] for b in range(B)):
        raise ValueError("q_offsets must be batch + 1 non-decreasing entries from 0 to q.shape[0]")
    if blocks.ndim != 6 or scales.ndim != 6 or blocks.shape[-1] != D or blocks.shape[4] != 1:
        raise ValueError("blocks / scales shapes do not match q")
    if not (0 <= layer_idx < blocks.shape[2]):
        raise ValueError("layer_idx out of range")
    P = blocks.shape[3]
    G = D // scales.shape[-1]
    lt = np.asarray(lookup_table)
    slt = None if scales_lookup_table is None else np.asarray(scales_lookup_table)
    O = np.full((T, H, dv), np.nan)
    lse = np.full((T, H), np.nan)
    for b in (range(B) if requests is None else requests):
        first, n = offs[b], offs[b + 1] - offs[b]
        if n == 0:
            continue
        L = int(cache_lengths[b])
        rows = resolve(lt[b:b + 1], None if slt is None else slt[b:b + 1], [L], P)[0]
        K = gather_dequant(blocks, scales, rows, layer_idx, G)
        for i in range(n):
            n_vis = max(0, min(L, L - n + i + 1))        # readings R1, R16
            o, l, _ = attention_rows(q[first + i], K, n_vis, softmax_scale, dv)
            O[first + i] = o
            lse[first + i] = l
    return (O, lse) if return_lse else O


def decode_range(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                 layer_idx, q_len, softmax_scale, t0, t1, dv=512):
    """Partial result of ``decode`` restricted to key positions t0 <= j < t1.

    Returns (O_r, lse_r) float64, O_r normalised within the range, lse_r the
    natural-log sum of exp(scores) over the visible keys of the range
    (-inf and O_r = 0 when the range holds none).  Merging the partials of a
    partition of [0, L) with ``merge_partials`` gives ``decode``'s result.
    """
    q = np.asarray(q, dtype=np.float64)
    _check_args(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                layer_idx, q_len)
    B, Q, H, D = q.shape
    P = blocks.shape[3]
    G = D // scales.shape[-1]
    lt = np.asarray(lookup_table)
    slt = None if scales_lookup_table is None else np.asarray(scales_lookup_table)
    O = np.zeros((B, Q, H, dv))
    lse = np.full((B, Q, H), -np.inf)
    for b in range(B):
        L = int(cache_lengths[b])
        rows = resolve(lt[b:b + 1], None if slt is None else slt[b:b + 1], [L], P)[0]
        K = gather_dequant(blocks, scales, rows, layer_idx, G)
        for i in range(Q):
            hi = min(t1, max(0, min(L, L - Q + i + 1)))
            lo = min(t0, hi)
            if hi <= lo:
                continue
            o, l, _ = attention_rows(q[b, i], K[lo:hi], hi - lo, softmax_scale, dv)
            O[b, i] = o
            lse[b, i] = l
    return O, lse


def merge_partials(parts):
    """Log-sum-exp merge of partial results [(O_r, lse_r), ...] over disjoint key ranges.

    lse = M + log(sum_r exp(lse_r - M)) with M = max_r lse_r, and
    O = sum_r exp(lse_r - lse) * O_r.  Rows whose every part is empty stay
    O = 0, lse = -inf (reading R9).
    """
    lses = np.stack([p[1] for p in parts])            # [R, ...]
    Os = np.stack([p[0] for p in parts])              # [R, ..., dv]
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    w = np.exp(lses - Msafe)                          # exp(-inf) = 0
    tot = w.sum(axis=0)
    lse = np.where(finite, Msafe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    coef = np.where(finite, 1.0, 0.0) * np.exp(lses - np.where(finite, lse, 0.0))
    coef = np.where(np.isfinite(lses), coef, 0.0)
    O = (coef[..., None] * Os).sum(axis=0)
    return O, lse
