"""FP64 CPU oracle for MLA decode over an unquantized (bf16) paged KV cache.

THIS IS TEST INFRASTRUCTURE, NOT PRODUCT CODE (same rules as ``mla_oracle``:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it).

The "KVCacheScalesMHAOperand" page (Mojo struct page, the
``quantization_enabled`` alias) makes quantization a property of the cache
type: a cache may also hold its latent rows unquantized, with no scales.  The
storage is then the ``blocks`` tensor of "generic_get_paged_cache_with_scales"
(section "Args") with a 16-bit element type, and the page lookup, cache
lengths and query length are read exactly as for the FP8 cache.

Reading U1: the unquantized element type is bfloat16 (the type the FP8 tiles
are converted to on the "KVLoad2CvtProducer" page), and the latent row is
used as stored: K_j[d] = blocks[LT[b, j / P], 0, layer, j % P, 0, d].
Everything else (readings R1, R2, R7, R8, R9 of ``mla_oracle``) is unchanged,
so the attention step is ``mla_oracle.attention_rows`` on these rows.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import attention_rows, resolve

__all__ = ["gather_rows", "decode_unquantized"]


def gather_rows(blocks, resolved_rows, layer_idx):
    """Latent rows K_j (float64 [L, head_dim]) of one request from an unquantized cache.

    ``blocks`` holds the element values (any float dtype; bf16 values widen to
    float64 exactly); token j's row is ``blocks[page, 0, layer, slot, 0, :]``.
    """
    head_dim = blocks.shape[-1]
    L = resolved_rows.shape[0]
    K = np.empty((L, head_dim), dtype=np.float64)
    for j in range(L):
        page, slot = int(resolved_rows[j, 0]), int(resolved_rows[j, 1])
        K[j] = blocks[page, 0, layer_idx, slot, 0, :]
    return K


def decode_unquantized(q, blocks, lookup_table, cache_lengths, layer_idx, q_len, softmax_scale,
                       dv=512, batches=None, return_lse=False):
    """MLA decode over the unquantized paged cache: O[b, i, h, :dv] in float64.

    q: float [B, q_len, H, head_dim]; blocks: float values
    [num_blocks, kv_dim, num_layers, page_size, 1, head_dim]; lookup_table:
    [B, max_pages] page ids; cache_lengths: [B].  Query row i sees keys
    j <= L_b - q_len + i.  ``batches`` restricts the work to some requests
    (other rows stay NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    blocks = np.asarray(blocks)
    B, Q, H, D = q.shape
    if blocks.ndim != 6 or blocks.shape[-1] != D or blocks.shape[4] != 1:
        raise ValueError("blocks is [num_blocks, kv_dim, num_layers, page_size, 1, head_dim]")
    if Q != q_len:
        raise ValueError("q.shape[1] must equal q_len")
    if not (0 <= layer_idx < blocks.shape[2]):
        raise ValueError("layer_idx out of range")
    P = blocks.shape[3]
    lt = np.asarray(lookup_table)
    O = np.full((B, Q, H, dv), np.nan)
    lse = np.full((B, Q, H), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(cache_lengths[b])
        rows = resolve(lt[b:b + 1], None, [L], P)[0]
        K = gather_rows(blocks, rows, layer_idx)
        for i in range(Q):
            n_vis = max(0, min(L, L - Q + i + 1))
            o, l, _ = attention_rows(q[b, i], K, n_vis, softmax_scale, dv)
            O[b, i] = o
            lse[b, i] = l
    return (O, lse) if return_lse else O
