"""Helpers shared by the GPU tests: run the HIP path, compare with the oracle."""

import sys

import numpy as np
import torch

from mla_decode_attention_paged_amd import mla_decode_paged_fp8
from mla_decode_attention_paged_amd.synth import Workload, _u32_view, u32_numpy
from tests.oracle_inputs import gate_stats, oracle_decode

GATE_MAX = 1e-2      # max of |gpu - bf16(oracle)| / max(1, |oracle|)
GATE_MEAN = 1e-3     # mean of the same


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_gpu(w, num_splits=None, workspace=None):
    out = mla_decode_paged_fp8(w.q, w.blocks, w.scales, w.lookup_table, w.scales_lookup_table,
                               w.cache_lengths, w.layer_idx, w.q_len, w.softmax_scale,
                               num_splits=num_splits, workspace=workspace)
    torch.cuda.synchronize()
    return out


def check_gate(gpu_out, ref, what=""):
    g = gpu_out.to(torch.float64).cpu().numpy()
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    st = gate_stats(g, ref)
    say(what, st)
    assert st["max_norm"] <= GATE_MAX and st["mean_norm"] <= GATE_MEAN, (what, st)
    return st


def extract_requests(w, batches):
    """A compact copy of workload w holding only the requests in `batches`,
    with the same key rows (for sampled oracle checks of very large pools).
    Page ids are renumbered; resolution itself is checked bit-exactly by the
    resolve tests at full size."""
    P = w.page_size
    lens = w.lengths()
    lt = u32_numpy(w.lookup_table).astype(np.int64)
    slt = lt if w.scales_lookup_table is None else u32_numpy(w.scales_lookup_table).astype(np.int64)
    pages, spages, new_lt, new_slt, new_len = [], [], [], [], []
    maxp = max(1, max((lens[b] + P - 1) // P for b in batches))
    for b in batches:
        n = (lens[b] + P - 1) // P
        row, srow = [], []
        for c in range(n):
            row.append(len(pages))
            srow.append(len(spages))
            pages.append(int(lt[b, c]))
            spages.append(int(slt[b, c]))
        new_lt.append(row + [0] * (maxp - n))
        new_slt.append(srow + [0] * (maxp - n))
        new_len.append(lens[b])
    if not pages:
        pages, spages = [0], [0]
    dev = w.blocks.device
    blocks = w.blocks[torch.as_tensor(pages, device=dev)][:, :, :, :, :, :].contiguous()
    scales = None if w.scales is None else w.scales[torch.as_tensor(spages, device=dev)].contiguous()
    return Workload(
        q=w.q[torch.as_tensor(batches, device=w.q.device)].contiguous(), blocks=blocks, scales=scales,
        lookup_table=_u32_view(torch.tensor(new_lt)).to(dev),
        scales_lookup_table=None if w.scales_lookup_table is None else _u32_view(torch.tensor(new_slt)).to(dev),
        cache_lengths=_u32_view(torch.tensor(new_len)).to(dev), layer_idx=w.layer_idx, q_len=w.q_len,
        softmax_scale=w.softmax_scale, page_size=P, granularity=w.granularity, name=w.name + "_sample")


def sampled_oracle(w, batches):
    """Oracle rows for the sampled requests of a (large) GPU workload."""
    sub = extract_requests(w, batches).to("cpu")
    return oracle_decode(sub)
