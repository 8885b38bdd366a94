"""GPU parity: per-request query counts (mla_decode_paged_fp8_ragged, through
the C ABI) against the oracle's decode_ragged.

Queries are packed request after request; each request is causal among its
own new tokens.  Cases mix counts 1, 4 and 16 (and 0: an empty request) in
one batch, with per-token and group scales, shared and independent scale
tables, forced and automatic split counts, a request with fewer keys than
queries, and more workgroups than compute units.  Gate as in
test_gpu_parity.py.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_paged_amd import mla_decode_paged_fp8, mla_decode_paged_fp8_ragged
from mla_decode_attention_paged_amd.synth import make_ragged_workload
from tests.gpu_helpers import check_gate, say
from tests.oracle_inputs import oracle_decode_ragged

pytestmark = pytest.mark.gpu


def _w(gpu_device, *args, **kw):
    kw.setdefault("device", gpu_device)
    return make_ragged_workload(*args, **kw)


def run_ragged(w, num_splits=None, max_q_len=None):
    out = mla_decode_paged_fp8_ragged(w.q, w.q_offsets, w.blocks, w.scales, w.lookup_table,
                                      w.scales_lookup_table, w.cache_lengths, w.layer_idx, w.softmax_scale,
                                      max_q_len=max_q_len, num_splits=num_splits)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("gran,indep,splits", [(576, False, None), (64, True, None), (576, False, 3),
                                               (64, True, 7)])
def test_mixed_counts(gpu_device, gran, indep, splits):
    counts = [1, 4, 16, 0, 4, 1]
    lengths = [300, 1000, 2000, 50, 16, 3000]
    say("ragged counts", counts, "granularity", gran, "independent", indep, "splits", splits)
    w = _w(gpu_device, counts, 128, lengths, 64, gran, independent_scales=indep, spare_blocks=3,
           spare_scale_blocks=3, seed=301, poison=True, unused_table_id=0xFFFFFFFF)
    out = run_ragged(w, num_splits=splits)
    assert out.shape == (sum(counts), 128, 512)
    check_gate(out, oracle_decode_ragged(w), f"ragged gran {gran} splits {splits}")


def test_fewer_keys_than_queries(gpu_device):
    """16 queries over 5 keys: the first 11 queries see no key and give zeros."""
    say("ragged: 16 queries, 5 keys")
    w = _w(gpu_device, [16, 2], 64, [5, 700], 16, 576, seed=302, poison=True)
    out = run_ragged(w)
    assert (out[:11] == 0).all()
    check_gate(out, oracle_decode_ragged(w), "fewer keys than queries")


def test_equal_counts_match_uniform_entry_bitwise(gpu_device):
    """With every count equal the packed layout is the [B, Q, H, 576] layout, and
    the ragged entry must reproduce the uniform entry bit for bit."""
    say("ragged: equal counts vs uniform entry")
    w = _w(gpu_device, [4, 4, 4], 128, [900, 64, 2500], 64, 64, independent_scales=True, seed=303, poison=True)
    out = run_ragged(w, num_splits=2)
    uni = mla_decode_paged_fp8(w.q.view(3, 4, 128, 576), w.blocks, w.scales, w.lookup_table,
                               w.scales_lookup_table, w.cache_lengths, w.layer_idx, 4, w.softmax_scale,
                               num_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(out, uni.view(12, 128, 512))


@pytest.mark.parametrize("heads", [16, 128])
def test_many_requests_default_plan(gpu_device, heads):
    """24 requests with counts in {0, 1, 4, 16}: the default plan (largest key
    ranges first once the workgroups outnumber the compute units)."""
    rng = np.random.default_rng(304 + heads)
    counts = rng.choice([0, 1, 4, 16], size=24).tolist()
    counts[0], counts[1] = 16, 0
    lengths = [int(max(c, v)) for c, v in zip(counts, rng.integers(1, 5000, size=24))]
    say("ragged: 24 requests, heads", heads, "counts", counts)
    w = _w(gpu_device, counts, heads, lengths, 64, 576, spare_blocks=2, seed=305, poison=True)
    check_gate(run_ragged(w), oracle_decode_ragged(w), f"ragged B=24 H={heads}")


def test_explicit_max_q_len(gpu_device):
    """max_q_len given by the caller (no host copy of the offsets): the same result."""
    say("ragged: explicit max_q_len")
    w = _w(gpu_device, [3, 0, 9], 32, [40, 10, 300], 16, 576, seed=306, poison=True)
    a = run_ragged(w)
    b = run_ragged(w, max_q_len=9)
    assert torch.equal(a, b)
    check_gate(a, oracle_decode_ragged(w), "explicit max_q_len")
