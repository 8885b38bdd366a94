"""GPU parity of the append-and-quantise kernel (through the C ABI) against the oracle.

Codes and scales are compared bit for bit over the whole blocks and scales
tensors, so a byte written where it should not be fails as surely as a wrong
code.  The rows include exact rounding ties (a row whose largest magnitude is
448 has scale 1, so its other values reach the E4M3FN grid unscaled), all-zero
groups, negative zeros and tiny values.  A decode after the append is checked
against the oracle's decode of the oracle-appended cache.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_paged_amd import mla_append_kv_fp8
from mla_decode_attention_paged_amd.synth import make_workload, u32_numpy
from oracle import append_kv
from tests.gpu_helpers import check_gate, run_gpu, say
from tests.oracle_inputs import oracle_decode

pytestmark = pytest.mark.gpu

TIES = [1.0625, -1.1875, 2.0 ** -10, 3 * 2.0 ** -10, -5 * 2.0 ** -10, 248.0, -9.5, 0.3125, 13.0, -0.0]


def _new_rows(B, q_len, gran, seed, device):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn((B, q_len, 576), generator=g) * torch.exp(torch.randn((B, q_len, 1), generator=g))
    x[0, 0, :] = 0.0                                   # an all-zero row: scale 0, codes 0
    if q_len > 1 or B > 1:
        r = x[-1, -1]
        r[:] = torch.randn(576, generator=g).clamp(-3, 3)
        for grp in range(576 // gran):
            base = grp * gran
            r[base] = 448.0                           # scale 1 for this group
            for k, v in enumerate(TIES):
                r[base + 1 + k] = v
    if gran == 64 and B > 1:
        x[1, 0, 64:128] = 0.0                          # one zero group inside a live row
        x[1, 0, 130] = 2.0 ** -20                      # tiny value next to larger ones
    return x.to(torch.bfloat16).to(device)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


@pytest.mark.parametrize("gran,indep,page,q_len,layers", [
    (576, False, 16, 1, 1), (576, True, 64, 4, 3), (64, True, 64, 1, 1), (64, False, 16, 4, 2),
])
def test_append_bit_exact(gpu_device, gran, indep, page, q_len, layers):
    say("append", gran, indep, page, q_len, layers)
    lengths = [q_len, 37, 200, 3 * page]
    layer = layers - 1
    w = make_workload(len(lengths), 16, lengths, page, gran, q_len=q_len, num_layers=layers, layer_idx=layer,
                      independent_scales=indep, spare_blocks=2, spare_scale_blocks=3, seed=90 + gran + page,
                      device=gpu_device, poison=True, unused_table_id=0xFFFFFFFF)
    kv = _new_rows(len(lengths), q_len, gran, 7 + page, gpu_device)
    lt = u32_numpy(w.lookup_table)
    slt = None if w.scales_lookup_table is None else u32_numpy(w.scales_lookup_table)
    ref_b, ref_s = append_kv(kv.float().cpu().numpy(), w.blocks.cpu().numpy(), w.scales.cpu().numpy(),
                             lt, slt, [int(v) for v in w.lengths()], layer, q_len)
    mla_append_kv_fp8(kv, w.blocks, w.scales, w.lookup_table, w.scales_lookup_table, w.cache_lengths,
                      layer, q_len)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(w.blocks), ref_b.view(np.uint8))
    assert np.array_equal(_bits(w.scales), ref_s.view(np.uint8))


def test_append_skips_rows_without_a_table_entry(gpu_device):
    """Request 0 is shorter than q_len (its first rows have t < 0); request 1's
    last rows fall past max_pages * page_size."""
    say("append out-of-table rows")
    q_len, page = 4, 16
    w = make_workload(2, 16, [2, 32], page, 576, q_len=1, seed=5, device=gpu_device, poison=True)
    w.cache_lengths.copy_(torch.tensor([2, 34], dtype=torch.int32))
    kv = _new_rows(2, q_len, 576, 3, gpu_device)
    lt = u32_numpy(w.lookup_table)
    ref_b, ref_s = append_kv(kv.float().cpu().numpy(), w.blocks.cpu().numpy(), w.scales.cpu().numpy(),
                             lt, None, [2, 34], 0, q_len)
    mla_append_kv_fp8(kv, w.blocks, w.scales, w.lookup_table, None, w.cache_lengths, 0, q_len)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(w.blocks), ref_b.view(np.uint8))
    assert np.array_equal(_bits(w.scales), ref_s.view(np.uint8))


@pytest.mark.parametrize("gran", [576, 64])
def test_decode_after_append(gpu_device, gran):
    say("decode after append", gran)
    q_len = 4
    lengths = [4, 300, 1030]
    w = make_workload(3, 128, lengths, 64, gran, q_len=q_len, independent_scales=gran == 64, spare_blocks=1,
                      spare_scale_blocks=1, seed=123 + gran, device=gpu_device, poison=True)
    kv = _new_rows(3, q_len, gran, 11, gpu_device)
    host_b, host_s = w.blocks.cpu().numpy(), w.scales.cpu().numpy()
    mla_append_kv_fp8(kv, w.blocks, w.scales, w.lookup_table, w.scales_lookup_table, w.cache_lengths,
                      w.layer_idx, q_len)
    torch.cuda.synchronize()
    lt = u32_numpy(w.lookup_table)
    slt = None if w.scales_lookup_table is None else u32_numpy(w.scales_lookup_table)
    ref_b, ref_s = append_kv(kv.float().cpu().numpy(), host_b, host_s, lt, slt, lengths, w.layer_idx, q_len)
    assert np.array_equal(_bits(w.blocks), ref_b.view(np.uint8))
    w_ref = w.to("cpu")
    w_ref.blocks = torch.from_numpy(ref_b)
    w_ref.scales = torch.from_numpy(ref_s)
    check_gate(run_gpu(w), oracle_decode(w_ref), f"decode after append g{gran}")
