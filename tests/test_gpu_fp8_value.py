"""GPU parity of the FP8-MFMA paths against the FP64 oracle, through the C
ABI.  Both are lossy opt-in modes, checked against their documented bound
(two bf16 ulps at |O| <= 2, and the gate's mean), not the gate itself:

  "v"  (mla_decode_paged_fp8_mfma8): P' V on v_mfma_scale_f32_32x32x64_f8f6f4,
       P' = p * key scale as two E4M3 parts with a power-of-two exponent per
       query row and 32-key tile, V as its E4M3 codes;
  "kv" (mla_decode_paged_fp8_mfma8_kv): also q K^T on the FP8 MFMA
       (v_mfma_scale_f32_16x16x128_f8f6f4), q as two E4M3 parts per row, K as
       its codes, in the one-wave-per-SIMD kernel.

The CPU emulation of these recipes under the measured accumulation model
(tests/test_numerics_budget.py) meets the gate on its cases; these tests check the
kernels: poisoned unused slots, ragged tails and steps with one tile, split
counts 1 to 24, causal q_len 4, a reference max that jumps (the rare rescale
paths), and the full-size uniform workload on sampled requests.  Group
scales are refused.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_paged_amd import MlaError, mla_decode_paged_fp8
from mla_decode_attention_paged_amd.synth import make_workload, uniform
from tests.gpu_helpers import GATE_MEAN, say
from tests.oracle_inputs import gate_stats, oracle_decode

pytestmark = pytest.mark.gpu


def _w(gpu_device, *args, **kw):
    kw.setdefault("device", gpu_device)
    return make_workload(*args, **kw)


MODES = ["v", "kv"]

# Both modes are lossy opt-in modes checked against their documented bound,
# two bf16 ulps at |O| <= 2 (2^-6), not the gate: "kv" because the FP8 key
# contraction's accumulation adds up to about one more bf16 ulp at |O| ~ 1
# (measured 1.11e-2 on test_fp8_mfma_empty_and_short_requests), "v" because
# P' in two E4M3 parts keeps about 8 significant bits (measured 1.17e-2 on
# test_multi_block_merge_fp8_mfma's 32 requests x 128 heads).
KV_MAX = 2.0 ** -6


def check(mode, out, ref, what):
    g = out.to(torch.float64).cpu().numpy()
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    st = gate_stats(g, ref)
    say(what, st)
    assert st["max_norm"] <= KV_MAX and st["mean_norm"] <= GATE_MEAN, (what, st)
    return st


def run_f8(w, mode, num_splits=None):
    out = mla_decode_paged_fp8(w.q, w.blocks, w.scales, w.lookup_table, w.scales_lookup_table, w.cache_lengths,
                               w.layer_idx, w.q_len, w.softmax_scale, num_splits=num_splits, fp8_mfma=mode)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("lengths,page,splits", [([37, 100], 16, None), ([3000, 700], 64, None),
                                                 ([3000, 700], 64, 1), ([3000, 700], 64, 3),
                                                 ([1, 31, 33, 64, 65, 96], 16, None),
                                                 ([20000, 3000, 5], 128, 24)])
@pytest.mark.parametrize("mode", MODES)
def test_fp8_mfma_parity(gpu_device, mode, lengths, page, splits):
    say("fp8 mfma", mode, lengths, page, splits)
    w = _w(gpu_device, len(lengths), 128, lengths, page, 576, spare_blocks=3, seed=401 + len(lengths),
           poison=True, unused_table_id=0xFFFFFFFF)
    check(mode, run_f8(w, mode, splits), oracle_decode(w), f"fp8 mfma {mode} {lengths} splits {splits}")


@pytest.mark.parametrize("mode", MODES)
def test_fp8_mfma_causal_q4(gpu_device, mode):
    say("fp8 mfma", mode, "q_len 4, layer 2 of 4")
    w = _w(gpu_device, 3, 128, [900, 4, 77], 64, 576, q_len=4, num_layers=4, layer_idx=2, independent_scales=True,
           spare_scale_blocks=2, seed=411, poison=True)
    check(mode, run_f8(w, mode), oracle_decode(w), f"fp8 mfma {mode} q_len 4")


@pytest.mark.parametrize("mode", MODES)
def test_fp8_mfma_empty_and_short_requests(gpu_device, mode):
    """An empty request, requests with fewer keys than queries (q_len 4) and a
    long one in one batch: rows that see no key are 0, the others meet the gate."""
    say("fp8 mfma", mode, "empty and short requests")
    w = _w(gpu_device, 4, 128, [0, 2, 5, 2500], 16, 576, q_len=4, seed=414, poison=True,
           unused_table_id=0xFFFFFFFF)
    out = run_f8(w, mode)
    assert (out[0] == 0).all() and (out[1, :2] == 0).all()
    check(mode, out, oracle_decode(w), f"fp8 mfma {mode} empty and short")


@pytest.mark.parametrize("heads", [16, 40])
def test_fp8_mfma_kv_partial_row_groups(gpu_device, heads):
    """Fewer heads than a row-group pair holds (16: one group; 40: a second,
    partial group): the one-wave-per-SIMD kernel's waves without rows."""
    say("fp8 mfma kv, heads", heads)
    w = _w(gpu_device, 2, heads, [700, 3000], 64, 576, seed=413 + heads, poison=True)
    check("kv", run_f8(w, "kv"), oracle_decode(w), f"fp8 mfma kv heads {heads}")


@pytest.mark.parametrize("mode", MODES)
def test_fp8_mfma_reference_max_jumps(gpu_device, mode):
    """Low scores first, far higher ones later: the reference moves after O has
    accumulated ("v": P' records made against an older reference are rescaled
    before their MFMAs; "kv": O is rescaled in its accumulators)."""
    say("fp8 mfma", mode, "reference max jumps")
    w = _w(gpu_device, 2, 128, [1500, 700], 64, 576, seed=91, poison=True)
    lt = (w.lookup_table.to(torch.int64) & 0xFFFFFFFF).cpu()
    P = w.page_size
    for b, L in enumerate(w.lengths()):
        for t in range(min(L, 128)):
            w.scales[int(lt[b, t // P]), 0, 0, t % P, 0, :] *= 1e-3
    w.q.mul_(8.0)
    torch.cuda.synchronize()
    ref = oracle_decode(w)
    check(mode, run_f8(w, mode, num_splits=1), ref, f"fp8 mfma {mode} jump, one split")
    check(mode, run_f8(w, mode), ref, f"fp8 mfma {mode} jump, auto plan")


@pytest.mark.parametrize("mode", MODES)
def test_fp8_mfma_full_size_uniform(gpu_device, mode):
    """16 x 4096 keys, 128 heads, the launch the benchmark times: all requests
    finite, four sampled requests against the oracle."""
    say("fp8 mfma", mode, "uniform 16 x 4096")
    w = uniform(device=gpu_device)
    out = run_f8(w, mode)
    assert torch.isfinite(out.float()).all()
    batches = [0, 5, 10, 15]
    ref = oracle_decode(w, batches=batches)
    check(mode, out[batches], ref[batches], f"fp8 mfma {mode} uniform sampled")


@pytest.mark.parametrize("mode", MODES)
def test_fp8_mfma_refuses_group_scales(gpu_device, mode):
    w = _w(gpu_device, 2, 16, [40, 50], 16, 64, seed=412)
    with pytest.raises(MlaError):
        run_f8(w, mode)
