"""Pins of the unquantized-cache oracle (oracle/unquantized.py).

* a cache whose bf16 rows are exactly the dequantized rows of an FP8 cache
  (power-of-two scales make e4m3 x scale representable in bf16) gives the
  FP8 oracle's result bit for bit, poisoned slots, pages and layers included;
* brute force with scalar loops and math.fsum on tiny inputs (random page
  table, causal q_len = 3, a second layer);
* permuting the physical page ids (and moving the pages with them) leaves
  the result unchanged.
"""

import math

import numpy as np
import torch

from mla_decode_attention_paged_amd.synth import make_workload
from oracle import E4M3FN_TABLE, decode, decode_unquantized
from tests.oracle_inputs import to_numpy


def _bf16_values(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_equals_fp8_oracle_on_dequantized_rows():
    w = make_workload(3, 16, [37, 100, 5], 16, 64, q_len=2, num_layers=2, layer_idx=1, spare_blocks=4,
                      seed=31, poison=True)
    rng = np.random.default_rng(4)
    scales = w.scales.numpy().copy()
    live = np.isfinite(scales)
    scales[live] = np.exp2(rng.integers(-8, 3, size=live.sum())).astype(np.float32)
    codes = w.blocks.numpy()
    NG = scales.shape[-1]
    deq = E4M3FN_TABLE[codes] * np.repeat(scales, 576 // NG, axis=-1).astype(np.float64)
    as_bf16 = torch.from_numpy(deq).to(torch.bfloat16)
    live_rows = np.isfinite(deq)
    assert np.array_equal(as_bf16.double().numpy()[live_rows], deq[live_rows])   # exact in bf16
    q, _, _, lt, _, cl = to_numpy(w)
    ref = decode(q, codes, scales, lt, None, cl, w.layer_idx, w.q_len, w.softmax_scale)
    got = decode_unquantized(q, _bf16_values(as_bf16), lt, cl, w.layer_idx, w.q_len, w.softmax_scale)
    assert np.isfinite(got).all()
    assert np.array_equal(got, ref)


def _brute(q, rows_of, lengths, q_len, sm):
    B, Q, H, D = q.shape
    out = np.zeros((B, Q, H, 512))
    for b in range(B):
        for i in range(Q):
            n = lengths[b] - q_len + i + 1
            for h in range(H):
                if n <= 0:
                    continue
                s = [sm * math.fsum(q[b, i, h, d] * rows_of(b, j)[d] for d in range(D)) for j in range(n)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = math.fsum(e)
                for c in range(512):
                    out[b, i, h, c] = math.fsum(e[j] * rows_of(b, j)[c] for j in range(n)) / z
    return out


def test_brute_force_tiny():
    rng = np.random.default_rng(9)
    P, D, NL, layer, q_len = 4, 576, 2, 1, 3
    lengths = [7, 3]
    max_pages = 2
    NB = 6
    blocks = torch.full((NB, 1, NL, P, 1, D), float("nan"), dtype=torch.bfloat16)
    lt = np.array([[4, 1], [2, 5]], dtype=np.uint32)
    store = {}
    for b, L in enumerate(lengths):
        for t in range(L):
            row = torch.from_numpy(rng.standard_normal(D) * 2.0).to(torch.bfloat16)
            blocks[lt[b, t // P], 0, layer, t % P, 0] = row
            store[(b, t)] = row.double().numpy()
    q = torch.from_numpy(rng.standard_normal((2, q_len, 2, D))).to(torch.bfloat16).double().numpy()
    sm = 0.07
    got = decode_unquantized(q, _bf16_values(blocks), lt, lengths, layer, q_len, sm)
    ref = _brute(q, lambda b, j: store[(b, j)], lengths, q_len, sm)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_page_permutation_invariance():
    w = make_workload(2, 8, [40, 70], 16, 576, spare_blocks=3, seed=12, poison=True, kv_dtype="bf16")
    q, blocks, _, lt, _, cl = to_numpy(w)
    ref = decode_unquantized(q, blocks, lt, cl, 0, 1, w.softmax_scale)
    perm = np.random.default_rng(2).permutation(blocks.shape[0])
    moved = np.empty_like(blocks)
    moved[perm] = blocks
    lt2 = lt.copy()
    used = lt2 < blocks.shape[0]
    lt2[used] = perm[lt2[used]]
    got = decode_unquantized(q, moved, lt2, cl, 0, 1, w.softmax_scale)
    assert np.isfinite(got).all()
    assert np.array_equal(got, ref)
