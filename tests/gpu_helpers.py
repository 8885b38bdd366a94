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
    with the same key rows (for oracle checks of very large pools one request
    at a time).  Page ids are renumbered; the full-size tests check the decode
    kernel's own resolution of the original tables bit for bit
    (check_block_offsets)."""
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


def check_block_offsets(w, num_splits=None, what=""):
    """Run the decode with the kernel's own resolution record and compare it bit
    for bit with the oracle's page resolution: for every key t < L_b the row the
    kernel addresses (its block's recorded offset + (t % 16) rows) must be the
    row of blocks[LT[b, t // P], 0, layer, t % P, 0, :], and likewise for the
    scale row through the scales table; blocks past a request's length stay
    unwritten.  Offsets are counted from (page 0, kv 0, layer, slot 0), the
    expected ones come from numpy's row-major index arithmetic on the tensor
    shapes.  Returns the decode output."""
    from oracle import resolve
    B = w.batch
    P = w.page_size
    lens = w.lengths()
    max_blocks = (w.lookup_table.shape[1] * P + 15) // 16
    rec = torch.full((B, max_blocks, 2), -1, dtype=torch.int64, device=w.q.device)
    out = mla_decode_paged_fp8(w.q, w.blocks, w.scales, w.lookup_table, w.scales_lookup_table,
                               w.cache_lengths, w.layer_idx, w.q_len, w.softmax_scale,
                               num_splits=num_splits, block_offsets=rec)
    torch.cuda.synchronize()
    got = rec.cpu().numpy()
    lt = u32_numpy(w.lookup_table)
    slt = None if w.scales_lookup_table is None else u32_numpy(w.scales_lookup_table)
    bshape = tuple(w.blocks.shape)
    sshape = tuple(w.scales.shape)
    base_b = np.ravel_multi_index((0, 0, w.layer_idx, 0, 0, 0), bshape)
    base_s = np.ravel_multi_index((0, 0, w.layer_idx, 0, 0, 0), sshape)
    for b, L in enumerate(lens):
        rows = resolve(lt[b:b + 1], None if slt is None else slt[b:b + 1], [L], P)[0]
        nb = (L + 15) // 16
        t = np.arange(L)
        z = np.zeros(L, dtype=np.int64)
        want_row = np.ravel_multi_index((rows[:, 0], z, z + w.layer_idx, rows[:, 1], z, z), bshape) - base_b
        want_srow = np.ravel_multi_index((rows[:, 2], z, z + w.layer_idx, rows[:, 1], z, z), sshape) - base_s
        got_row = got[b, t // 16, 0] + (t % 16) * bshape[-1]
        got_srow = got[b, t // 16, 1] + (t % 16) * sshape[-1]
        assert np.array_equal(got_row, want_row), (what, b, "row offsets")
        assert np.array_equal(got_srow, want_srow), (what, b, "scale row offsets")
        assert (got[b, nb:] == -1).all(), (what, b, "records past the request's length")
    say(what, "kernel page resolution bit-exact over", sum(lens), "keys")
    return out
