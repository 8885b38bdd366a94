"""CPU oracle for appending new latent rows to the paged FP8 cache (quantize + scatter).

THIS IS TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import or call it.  The HIP
path never imports it, and it imports nothing from the HIP path.

What it computes, and where each piece comes from
--------------------------------------------------
The write side of the storage contract that the decode oracle reads
(``mla_oracle``): the "generic_get_paged_cache_with_scales" page, section
"Args", fixes where a token's bytes and scales live -- token t of request b is
``blocks[LT[b, t // P], 0, layer, t % P, 0, :]`` with its scales in
``scales[SLT[b, t // P], 0, layer, t % P, 0, :]`` (SLT = LT when the scales
table is absent); the "KVCacheScalesMHAOperand" page gives the Float32 scale
type and the per-token granularity.  The quantisation recipe is the one the
workloads are described with: per granularity group, scale = amax / 448 in
float32 and code = the E4M3FN value nearest to clip(x / scale, -448, 448).

Readings taken where the pages are silent (each listed in the design doc):
  A1  cache_lengths already count the q_len new tokens (reading R1 of the
      decode oracle): new row i of request b is token t = L_b - q_len + i.
      Rows with t < 0 or t >= max_pages * page_size are not written.
  A2  The floating-point steps that decide a code run in float32, as a kernel
      runs them: s = fl32(fl32(amax) / 448), v = fl32(x / s), v clipped to
      [-448, 448]; the code is the E4M3FN value nearest to v, ties going to the
      even code (bit 0 clear).  The sign bit is v's (so -0.0 -> 0x80).
  A3  A group whose amax is 0 gets scale 0 and all codes 0x00.
  A4  The new rows are bf16 [B, q_len, head_dim] (the latent row of the single
      KV head); they go to kv index 0, head 0, layer ``layer_idx``.
  A5  Non-finite inputs are outside the contract.

No blocking or fusion: a per-row Python loop over the page table; the nearest
E4M3FN value is found by a search over the sorted table of all finite codes.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import E4M3FN_TABLE

__all__ = ["FP8_MAX", "e4m3fn_round", "quantize_row", "append_kv"]

FP8_MAX = 448.0

# non-negative finite codes 0x00..0x7E in increasing value
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3FN_TABLE[:0x7F].copy()


def e4m3fn_round(v) -> np.ndarray:
    """E4M3FN codes (uint8) of float values with |v| <= 448: nearest value, ties to even.

    For each |v| the two neighbouring table values are compared; on an exact
    tie the code with bit 0 clear wins.  The sign bit is copied from v.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > FP8_MAX) or not np.all(np.isfinite(v)):
        raise ValueError("e4m3fn_round takes finite values within [-448, 448]")
    hi = np.searchsorted(_POS_VALUES, a, side="left")       # first table value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    mag = np.where(_POS_VALUES[hi] == a, _POS_CODES[hi], mag)   # exact hits
    sign = np.signbit(v).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


def quantize_row(x, granularity: int):
    """Codes (uint8 [D]) and float32 scales ([D / granularity]) of one latent row.

    x: the row's values (bf16 values held in any float dtype).  Reading A2 for
    the float32 steps, A3 for all-zero groups.
    """
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[0]
    groups = d // granularity
    codes = np.zeros(d, dtype=np.uint8)
    scales = np.zeros(groups, dtype=np.float32)
    for g in range(groups):
        xg = x[g * granularity:(g + 1) * granularity]
        amax = np.float32(np.max(np.abs(xg)))
        s = np.float32(amax / np.float32(FP8_MAX))
        scales[g] = s
        if amax == 0:
            continue
        v = np.clip(np.float32(xg / s), -FP8_MAX, FP8_MAX)   # float32 division (RNE)
        codes[g * granularity:(g + 1) * granularity] = e4m3fn_round(v)
    return codes, scales


def append_kv(kv_new, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
              layer_idx: int, q_len: int):
    """New (blocks, scales) copies with the q_len new rows of every request written.

    kv_new: [B, q_len, head_dim] bf16 values (float array); blocks uint8
    [NB, KVD, NL, P, 1, head_dim]; scales float32 [NBs, KVD, NL, P, 1, NG];
    tables [B, max_pages] of uint32 ids; cache_lengths [B].
    """
    kv_new = np.asarray(kv_new, dtype=np.float32)
    blocks = np.array(blocks, dtype=np.uint8, copy=True)
    scales = np.array(scales, dtype=np.float32, copy=True)
    lt = np.asarray(lookup_table).astype(np.int64)
    slt = lt if scales_lookup_table is None else np.asarray(scales_lookup_table).astype(np.int64)
    B, max_pages = lt.shape
    P = blocks.shape[3]
    head_dim = blocks.shape[-1]
    granularity = head_dim // scales.shape[-1]
    for b in range(B):
        L = int(cache_lengths[b])
        for i in range(q_len):
            t = L - q_len + i
            if t < 0 or t >= max_pages * P:
                continue
            page, slot, spage = int(lt[b, t // P]), t % P, int(slt[b, t // P])
            codes, s = quantize_row(kv_new[b, i], granularity)
            blocks[page, 0, layer_idx, slot, 0, :] = codes
            scales[spage, 0, layer_idx, slot, 0, :] = s
    return blocks, scales
