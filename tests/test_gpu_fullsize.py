"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (the automatic plan), checked against the oracle request by request
(the oracle computes each request from a compact copy of its pages), plus the
decode kernel's own page and scale-page resolution over the whole batch, bit
for bit.

Every request of the uniform, ragged and long-context workloads is checked;
for the speculative batch (128 requests of up to 32768 keys and 4 query
positions) the shortest and longest requests, one request from each length
decile and requests whose length sits at a multiple of the plan's split
length (or one key past it) are checked, at least 16 in all."""

import numpy as np
import pytest
import torch

from mla_decode_attention_paged_amd import mla_decode_paged_fp8_plan, synth
from tests.gpu_helpers import check_block_offsets, check_gate, sampled_oracle, say

pytestmark = pytest.mark.gpu


def _check(w, batches, chunk=8):
    out = check_block_offsets(w, what=w.name)
    assert torch.isfinite(out.float()).all()
    for i in range(0, len(batches), chunk):
        part = batches[i:i + chunk]
        ref = sampled_oracle(w, part)
        check_gate(out[part], ref, f"{w.name} requests {part}")


def test_uniform_16x4096(gpu_device):
    say("uniform B=16 L=4096 P=64 per-token scales, all requests")
    w = synth.uniform(device=gpu_device)
    _check(w, list(range(w.batch)))


def test_ragged_64_group_scales(gpu_device):
    say("ragged B=64 L~U[1,8192] group scales, independent scale table, all requests")
    w = synth.ragged(device=gpu_device)
    _check(w, list(range(w.batch)))


@pytest.mark.parametrize("batch", [1, 4])
def test_long_context(gpu_device, batch):
    say("long context B=%d L=131072 P=128, all requests" % batch)
    w = synth.long_context(device=gpu_device, batch=batch)
    _check(w, list(range(w.batch)), chunk=1)


def _speculative_sample(w):
    lens = np.array(w.lengths())
    order = np.argsort(lens, kind="stable")
    pick = {int(order[0]), int(order[-1])}
    for d in range(10):                                   # one request per length decile
        pick.add(int(order[min(len(order) - 1, (2 * d + 1) * len(order) // 20)]))
    plan = mla_decode_paged_fp8_plan(tuple(w.q.shape), tuple(w.blocks.shape), tuple(w.scales.shape),
                                     tuple(w.lookup_table.shape), w.q_len)
    T = plan["tokens_per_split"]
    # lengths nearest to a multiple of the split length (from either side)
    dist = np.minimum(lens % T, T - lens % T)
    for b in np.argsort(dist, kind="stable")[:4]:
        pick.add(int(b))
    b = 0
    while len(pick) < 16:
        pick.add(b)
        b += 1
    return sorted(pick), T


def test_speculative_128x4(gpu_device):
    say("speculative B=128 q_len 4, layer 2 of 4, group scales")
    w = synth.speculative(device=gpu_device)
    batches, T = _speculative_sample(w)
    say("speculative requests checked:", batches, "split length", T)
    _check(w, batches, chunk=4)
