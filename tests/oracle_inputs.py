"""Convert synthetic workloads (torch) into the numpy arrays the oracle takes."""

import numpy as np
import torch

from mla_decode_attention_paged_amd.synth import u32_numpy


def to_numpy(w):
    """(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths) as numpy."""
    q = w.q.detach().to("cpu").to(torch.float64).numpy()
    blocks = w.blocks.detach().to("cpu")
    # bf16 rows of an unquantized cache widen exactly to float64
    blocks = blocks.to(torch.float64).numpy() if blocks.dtype == torch.bfloat16 else blocks.numpy()
    scales = None if w.scales is None else w.scales.detach().to("cpu").numpy()
    lt = u32_numpy(w.lookup_table)
    slt = None if w.scales_lookup_table is None else u32_numpy(w.scales_lookup_table)
    cl = u32_numpy(w.cache_lengths)
    return q, blocks, scales, lt, slt, cl


def oracle_decode(w, batches=None, return_lse=False):
    from oracle import decode
    q, blocks, scales, lt, slt, cl = to_numpy(w)
    return decode(q, blocks, scales, lt, slt, cl, w.layer_idx, w.q_len, w.softmax_scale,
                  batches=batches, return_lse=return_lse)


def oracle_decode_ragged(w, requests=None, return_lse=False):
    from oracle import decode_ragged
    q, blocks, scales, lt, slt, cl = to_numpy(w)
    offs = w.q_offsets.cpu().numpy().astype(np.int64)
    return decode_ragged(q, offs, blocks, scales, lt, slt, cl, w.layer_idx, w.softmax_scale,
                         requests=requests, return_lse=return_lse)


def oracle_decode_unquantized(w, batches=None, return_lse=False):
    from oracle import decode_unquantized
    q, blocks, _, lt, _, cl = to_numpy(w)
    return decode_unquantized(q, blocks, lt, cl, w.layer_idx, w.q_len, w.softmax_scale,
                              batches=batches, return_lse=return_lse)


def gate_stats(gpu, ref64):
    """Normalised error e = |gpu - bf16(ref)| / max(1, |ref|) and literal errors."""
    from oracle import bf16_round
    ref_bf = bf16_round(ref64)
    d = np.abs(np.asarray(gpu, dtype=np.float64) - ref_bf)
    e = d / np.maximum(1.0, np.abs(ref64))
    return {"max_norm": float(e.max()), "mean_norm": float(e.mean()),
            "max_abs": float(d.max()), "mean_abs": float(d.mean())}
