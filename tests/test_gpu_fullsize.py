"""Full-size workloads on the GPU, in the launch configuration the benchmark
times, checked against the oracle on sampled requests (the oracle computes
those requests one by one from a compact copy of their pages), plus
properties that hold at any size: finite outputs and bit-exact page
resolution over the whole batch."""

import numpy as np
import pytest
import torch

from mla_decode_attention_paged_amd import mla_resolve_pages
from mla_decode_attention_paged_amd import synth
from oracle import resolve
from tests.gpu_helpers import check_gate, run_gpu, sampled_oracle, say

pytestmark = pytest.mark.gpu


def _resolve_exact(w):
    lens = w.lengths()
    pg, sl, sp = mla_resolve_pages(w.lookup_table, w.scales_lookup_table, w.cache_lengths,
                                   w.page_size, max(lens))
    torch.cuda.synchronize()
    lt = synth.u32_numpy(w.lookup_table)
    slt = None if w.scales_lookup_table is None else synth.u32_numpy(w.scales_lookup_table)
    rows = resolve(lt, slt, lens, w.page_size)
    got = [synth.u32_numpy(t) for t in (pg, sl, sp)]
    for b, L in enumerate(lens):
        for k in range(3):
            assert np.array_equal(got[k][b, :L].astype(np.int64), rows[b][:, k]), (w.name, b, k)


def _check(w, batches):
    out = run_gpu(w)
    assert torch.isfinite(out.float()).all()
    ref = sampled_oracle(w, batches)
    check_gate(out[batches], ref, f"{w.name} sample {batches}")
    _resolve_exact(w)


def test_uniform_16x4096(gpu_device):
    say("uniform B=16 L=4096 P=64 per-token scales")
    w = synth.uniform(device=gpu_device)
    _check(w, [0, 15])


def test_ragged_64_group_scales(gpu_device):
    say("ragged B=64 L~U[1,8192] group scales, independent scale table")
    w = synth.ragged(device=gpu_device)
    lens = w.lengths()
    _check(w, [int(np.argmin(lens)), int(np.argmax(lens)), 7])


@pytest.mark.parametrize("batch", [1, 4])
def test_long_context(gpu_device, batch):
    say("long context B=%d L=131072 P=128" % batch)
    w = synth.long_context(device=gpu_device, batch=batch)
    _check(w, [batch - 1])


def test_speculative_128x4(gpu_device):
    say("speculative B=128 q_len 4, layer 2 of 4, group scales")
    w = synth.speculative(device=gpu_device)
    lens = w.lengths()
    _check(w, [int(np.argmin(lens)), int(np.argmax(lens))])
