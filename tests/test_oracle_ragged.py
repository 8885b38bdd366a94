"""Pins of the oracle's per-request query counts (decode_ragged).

The requests' queries are packed request after request (q [T, H, 576], request
b owning rows q_offsets[b] .. q_offsets[b + 1] - 1), each request causal among
its own n_b new tokens ("generic_get_paged_cache_with_scales", Args:
max_prompt_length is the batch's largest query count).  Pinned against:
* brute force with scalar loops and math.fsum on tiny inputs with mixed
  counts, an empty request and a request with fewer keys than queries;
* the batched decode (itself pinned in test_oracle_attention.py) when every
  request has the same count, and per request with q_len = n_b;
* a permutation of the requests permuting the output rows;
* an empty request contributing no rows, and a one-query request equal to a
  q_len = 1 decode of the same request.
"""

import math

import numpy as np
import pytest

from mla_decode_attention_paged_amd.synth import make_ragged_workload
from oracle import E4M3FN_TABLE, decode, decode_ragged
from tests.oracle_inputs import to_numpy


def _np(w):
    q, blocks, scales, lt, slt, cl = to_numpy(w)
    return q, w.q_offsets.cpu().numpy().astype(np.int64), blocks, scales, lt, slt, cl


def _brute_force_ragged(q, offs, blocks, scales, lt, slt, cl, layer, sm, P, G, cols=(0, 77, 511)):
    """Scalar restatement: per request b, query i < n_b and head, keys j <= L_b - n_b + i."""
    out = {}
    for b in range(len(offs) - 1):
        n = int(offs[b + 1] - offs[b])
        L = int(cl[b])
        K = []
        for t in range(L):
            page, slot = int(lt[b][t // P]), t % P
            spage = int((slt if slt is not None else lt)[b][t // P])
            K.append([E4M3FN_TABLE[int(blocks[page][0][layer][slot][0][d])] *
                      float(scales[spage][0][layer][slot][0][d // G]) for d in range(576)])
        for i in range(n):
            vis = max(0, min(L, L - n + i + 1))
            for h in range(q.shape[1]):
                row = int(offs[b]) + i
                if vis == 0:
                    for c in cols:
                        out[(row, h, c)] = 0.0
                    continue
                s = [sm * math.fsum(float(q[row, h, d]) * K[j][d] for d in range(576)) for j in range(vis)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                den = math.fsum(e)
                for c in cols:
                    out[(row, h, c)] = math.fsum(e[j] / den * K[j][c] for j in range(vis))
    return out


@pytest.mark.parametrize("gran,indep", [(576, False), (64, True)])
def test_brute_force_mixed_counts(gran, indep):
    # counts 3, 0, 1, 2 (request 1 empty); request 3 has one key for two queries
    w = make_ragged_workload([3, 0, 1, 2], 2, [7, 5, 4, 1], 16, gran, seed=21, num_layers=2, layer_idx=1,
                             independent_scales=indep, spare_blocks=2, spare_scale_blocks=2)
    q, offs, blocks, scales, lt, slt, cl = _np(w)
    got = decode_ragged(q, offs, blocks, scales, lt, slt, cl, 1, w.softmax_scale)
    assert got.shape == (6, 2, 512)
    ref = _brute_force_ragged(q, offs, blocks, scales, lt, slt, cl, 1, w.softmax_scale, 16, gran)
    for (row, h, c), v in ref.items():
        assert abs(got[row, h, c] - v) <= 1e-12 * max(1.0, abs(v)), (row, h, c)
    # the first query of request 3 sees no key (L - n + 0 + 1 = 0): zeros
    assert np.all(got[4] == 0.0)


def test_equal_counts_match_batched_decode():
    w = make_ragged_workload([4, 4, 4], 3, [40, 9, 70], 16, 64, seed=22, independent_scales=True)
    q, offs, blocks, scales, lt, slt, cl = _np(w)
    got = decode_ragged(q, offs, blocks, scales, lt, slt, cl, 0, w.softmax_scale)
    ref = decode(q.reshape(3, 4, 3, 576), blocks, scales, lt, slt, cl, 0, 4, w.softmax_scale)
    assert np.array_equal(got, ref.reshape(12, 3, 512))


def test_each_request_equals_its_own_decode():
    counts = [1, 4, 0, 16, 2]
    w = make_ragged_workload(counts, 2, [30, 12, 8, 50, 2], 16, 576, seed=23)
    q, offs, blocks, scales, lt, slt, cl = _np(w)
    got = decode_ragged(q, offs, blocks, scales, lt, slt, cl, 0, w.softmax_scale)
    for b, n in enumerate(counts):
        if n == 0:
            continue
        qb = q[offs[b]:offs[b + 1]][None]
        ref = decode(qb, blocks, scales, lt[b:b + 1], None, cl[b:b + 1], 0, n, w.softmax_scale)
        assert np.array_equal(got[offs[b]:offs[b + 1]], ref[0])


def test_request_permutation_permutes_rows():
    counts = [2, 5, 1, 3]
    w = make_ragged_workload(counts, 2, [20, 33, 6, 9], 16, 64, seed=24, independent_scales=True)
    q, offs, blocks, scales, lt, slt, cl = _np(w)
    got = decode_ragged(q, offs, blocks, scales, lt, slt, cl, 0, w.softmax_scale)
    perm = [2, 0, 3, 1]
    q2 = np.concatenate([q[offs[b]:offs[b + 1]] for b in perm])
    offs2 = np.concatenate([[0], np.cumsum([counts[b] for b in perm])])
    got2 = decode_ragged(q2, offs2, blocks, scales, lt[perm], slt[perm], cl[perm], 0, w.softmax_scale)
    assert np.array_equal(got2, np.concatenate([got[offs[b]:offs[b + 1]] for b in perm]))


def test_one_query_request_is_a_single_token_decode():
    w = make_ragged_workload([1, 3], 2, [25, 25], 16, 576, seed=25)
    q, offs, blocks, scales, lt, slt, cl = _np(w)
    got = decode_ragged(q, offs, blocks, scales, lt, slt, cl, 0, w.softmax_scale)
    ref = decode(q[0:1][None], blocks, scales, lt[0:1], None, cl[0:1], 0, 1, w.softmax_scale)
    assert np.array_equal(got[0], ref[0, 0])


@pytest.mark.parametrize("offs", [[1, 3], [0, 3, 2, 5], [0, 2]])
def test_bad_offsets_rejected(offs):
    w = make_ragged_workload([2, 3], 2, [9, 9], 16, 576, seed=26)
    q, _, blocks, scales, lt, slt, cl = _np(w)
    with pytest.raises(ValueError):
        decode_ragged(q, np.array(offs), blocks, scales, lt, slt, cl, 0, w.softmax_scale)
