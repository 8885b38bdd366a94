"""GPU parity of the FP8-MFMA value contraction (mla_decode_paged_fp8_mfma8,
through the C ABI) against the FP64 oracle, same gate as test_gpu_parity.py.

P' = p * key scale enters the v_mfma_scale_f32_32x32x64_f8f6f4 MFMA as two
E4M3 parts per element with a power-of-two exponent per query row and 32-key
tile; V enters as its E4M3 codes.  The CPU emulation of this recipe under the
measured accumulation model (tests/test_numerics_budget.py) meets the gate;
these tests check the kernel: poisoned unused slots, ragged tails and steps
with one tile, split counts 1 to 24, causal q_len 4, a reference max that
jumps (the rare rescale of P' records), and the full-size uniform workload on
sampled requests.  Group scales are refused.
"""

import pytest
import torch

from mla_decode_attention_paged_amd import MlaError, mla_decode_paged_fp8
from mla_decode_attention_paged_amd.synth import make_workload, uniform
from tests.gpu_helpers import check_gate, say
from tests.oracle_inputs import oracle_decode

pytestmark = pytest.mark.gpu


def _w(gpu_device, *args, **kw):
    kw.setdefault("device", gpu_device)
    return make_workload(*args, **kw)


def run_f8(w, num_splits=None):
    out = mla_decode_paged_fp8(w.q, w.blocks, w.scales, w.lookup_table, w.scales_lookup_table, w.cache_lengths,
                               w.layer_idx, w.q_len, w.softmax_scale, num_splits=num_splits, value_fp8=True)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("lengths,page,splits", [([37, 100], 16, None), ([3000, 700], 64, None),
                                                 ([3000, 700], 64, 1), ([3000, 700], 64, 3),
                                                 ([1, 31, 33, 64, 65, 96], 16, None),
                                                 ([20000, 3000, 5], 128, 24)])
def test_fp8_value_parity(gpu_device, lengths, page, splits):
    say("fp8 value contraction", lengths, page, splits)
    w = _w(gpu_device, len(lengths), 128, lengths, page, 576, spare_blocks=3, seed=401 + len(lengths),
           poison=True, unused_table_id=0xFFFFFFFF)
    check_gate(run_f8(w, splits), oracle_decode(w), f"fp8 value {lengths} splits {splits}")


def test_fp8_value_causal_q4(gpu_device):
    say("fp8 value contraction, q_len 4, layer 2 of 4")
    w = _w(gpu_device, 3, 128, [900, 4, 77], 64, 576, q_len=4, num_layers=4, layer_idx=2, independent_scales=True,
           spare_scale_blocks=2, seed=411, poison=True)
    check_gate(run_f8(w), oracle_decode(w), "fp8 value q_len 4")


def test_fp8_value_reference_max_jumps(gpu_device):
    """Low scores first, far higher ones later: P' records made against an older
    reference are rescaled (decoded, scaled, split again) before their MFMAs."""
    say("fp8 value contraction, reference max jumps")
    w = _w(gpu_device, 2, 128, [1500, 700], 64, 576, seed=91, poison=True)
    lt = (w.lookup_table.to(torch.int64) & 0xFFFFFFFF).cpu()
    P = w.page_size
    for b, L in enumerate(w.lengths()):
        for t in range(min(L, 128)):
            w.scales[int(lt[b, t // P]), 0, 0, t % P, 0, :] *= 1e-3
    w.q.mul_(8.0)
    torch.cuda.synchronize()
    ref = oracle_decode(w)
    check_gate(run_f8(w, num_splits=1), ref, "fp8 value jump, one split")
    check_gate(run_f8(w), ref, "fp8 value jump, auto plan")


def test_fp8_value_full_size_uniform(gpu_device):
    """16 x 4096 keys, 128 heads, the launch the benchmark times: all requests
    finite, four sampled requests against the oracle."""
    say("fp8 value contraction, uniform 16 x 4096")
    w = uniform(device=gpu_device)
    out = run_f8(w)
    assert torch.isfinite(out.float()).all()
    batches = [0, 5, 10, 15]
    ref = oracle_decode(w, batches=batches)
    check_gate(out[batches], ref[batches], "fp8 value uniform sampled")


def test_fp8_value_refuses_group_scales(gpu_device):
    w = _w(gpu_device, 2, 16, [40, 50], 16, 64, seed=412)
    with pytest.raises(MlaError):
        run_f8(w)
