"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle.

Gate (floating point): e = |gpu - bf16(oracle)| / max(1, |oracle|), max e <=
1e-2 and mean e <= 1e-3 on the bf16 outputs.  Index work (page / slot / scale
page resolution) is compared bit-exactly.  Sizes here are ones the oracle
finishes in seconds while still spanning several 32-key tiles, several waves
and ragged tails; the full-size workloads are checked on sampled requests in
test_gpu_fullsize.py.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_paged_amd import mla_resolve_pages
from mla_decode_attention_paged_amd.synth import make_workload, tiny, u32_numpy
from oracle import resolve
from tests.gpu_helpers import check_block_offsets, check_gate, run_gpu, say
from tests.oracle_inputs import oracle_decode

pytestmark = pytest.mark.gpu


def _w(gpu_device, *args, **kw):
    kw.setdefault("device", gpu_device)
    return make_workload(*args, **kw)


# ------------------------------------------------------------------ resolution
@pytest.mark.parametrize("page,indep,lengths", [
    (16, False, [37, 100]), (64, True, [1, 64, 65, 4000]), (128, True, [131, 9000]),
])
def test_resolve_bit_exact(gpu_device, page, indep, lengths):
    say("resolve", page, indep, lengths)
    w = _w(gpu_device, len(lengths), 4, lengths, page, 64, independent_scales=indep,
           spare_blocks=3, spare_scale_blocks=5, unused_table_id=0xFFFFFFFF, seed=page)
    max_tokens = max(lengths) + 40
    pg, sl, sp = mla_resolve_pages(w.lookup_table, w.scales_lookup_table, w.cache_lengths, page, max_tokens)
    torch.cuda.synchronize()
    lt = u32_numpy(w.lookup_table)
    slt = None if w.scales_lookup_table is None else u32_numpy(w.scales_lookup_table)
    rows = resolve(lt, slt, lengths, page)
    got = [u32_numpy(t) for t in (pg, sl, sp)]
    for b, L in enumerate(lengths):
        for k in range(3):
            assert np.array_equal(got[k][b, :L].astype(np.int64), rows[b][:, k]), (b, k)
            assert (got[k][b, L:] == 0xFFFFFFFF).all()


@pytest.mark.parametrize("page,gran,indep,splits", [
    (16, 576, False, 1), (16, 64, True, None), (64, 576, True, 3), (64, 64, False, None),
    (128, 576, False, None), (128, 64, True, 2),
])
def test_kernel_resolution_bit_exact(gpu_device, page, gran, indep, splits):
    """The decode kernel's own page and scale-page resolution (the offsets it
    loads from), recorded by the kernel itself, equals the oracle's resolution
    bit for bit; layer 1 of 3 selected; ragged lengths across pages and
    windows of 64 blocks; unused table columns hold 0xFFFFFFFF."""
    say("kernel resolution", page, gran, indep, splits)
    w = _w(gpu_device, 4, 128, [1, 16 * page + 5, 33, 70 * 16 + 3], page, gran, num_layers=3, layer_idx=1,
           independent_scales=indep, spare_blocks=3, spare_scale_blocks=4, unused_table_id=0xFFFFFFFF,
           seed=100 + page + gran, poison=True)
    out = check_block_offsets(w, num_splits=splits, what=f"P{page} G{gran} indep={indep} splits={splits}")
    check_gate(out, oracle_decode(w), "kernel resolution output")


# ------------------------------------------------------------------ parity, small
def test_tiny_workload(gpu_device):
    say("tiny (B=2, H=16, L={37,100}, P=16, per-token scales, NaN poison)")
    w = tiny(device=gpu_device, poison=True)
    check_gate(run_gpu(w), oracle_decode(w), "tiny")


@pytest.mark.parametrize("gran", [576, 64])
def test_128_heads_ragged_lengths(gpu_device, gran):
    say("128 heads ragged", gran)
    w = _w(gpu_device, 4, 128, [1, 77, 1000, 33], 64, gran, independent_scales=gran == 64,
           spare_blocks=2, spare_scale_blocks=3, seed=21 + gran, poison=True,
           unused_table_id=0xFFFFFFFF)
    check_gate(run_gpu(w), oracle_decode(w), f"ragged g{gran}")


@pytest.mark.parametrize("gran", [576, 64])
@pytest.mark.parametrize("seed", [177, 179, 181])
def test_many_rows_several_seeds(gpu_device, gran, seed):
    """4,096 query rows (32 requests x 128 heads, lengths spread over
    1..1,500 keys with one empty request), default plan: every element within
    the gate, across seeds (the worst element sits at the one-ulp floor)."""
    say("many rows", gran, seed)
    lengths = [(97 * b) % 1500 + 1 for b in range(32)]
    lengths[5] = 0
    w = _w(gpu_device, 32, 128, lengths, 64, gran, independent_scales=gran == 64, seed=seed, poison=True)
    check_gate(run_gpu(w), oracle_decode(w), f"many rows g{gran} seed {seed}")


@pytest.mark.parametrize("page", [16, 128])
def test_page_sizes(gpu_device, page):
    say("page size", page)
    w = _w(gpu_device, 2, 128, [513, 250], page, 576, seed=31 + page, poison=True)
    check_gate(run_gpu(w), oracle_decode(w), f"page {page}")


def test_causal_four_queries_layer_select(gpu_device):
    say("q_len 4, layer 2 of 4, group scales, own scale table")
    w = _w(gpu_device, 3, 128, [4, 70, 1500], 64, 64, q_len=4, num_layers=4, layer_idx=2,
           independent_scales=True, spare_blocks=2, spare_scale_blocks=2, seed=41, poison=True)
    check_gate(run_gpu(w), oracle_decode(w), "causal q4")


@pytest.mark.parametrize("q_len,heads,gran", [(16, 128, 64), (64, 16, 576)])
def test_longer_query_runs(gpu_device, q_len, heads, gran):
    """Chunked-prefill shapes (q_len >> 4) over the paged cache: many row
    groups, each query position with its own causal limit."""
    say("q_len", q_len, "heads", heads, "gran", gran)
    w = _w(gpu_device, 3, heads, [q_len, 300, 1000], 64, gran, q_len=q_len,
           independent_scales=gran == 64, spare_blocks=2, spare_scale_blocks=2, seed=43 + q_len,
           poison=True)
    check_gate(run_gpu(w), oracle_decode(w), f"q{q_len} h{heads}")


def test_rows_mixing_query_positions(gpu_device):
    """16 heads x 4 queries: one 32-row group holds two query positions."""
    say("H=16, q_len 4")
    w = _w(gpu_device, 2, 16, [9, 300], 16, 576, q_len=4, seed=51, poison=True)
    check_gate(run_gpu(w), oracle_decode(w), "h16 q4")


def test_odd_head_count(gpu_device):
    say("H=40 (partial row group)")
    w = _w(gpu_device, 2, 40, [3, 200], 64, 64, seed=52, poison=True)
    check_gate(run_gpu(w), oracle_decode(w), "h40")


def test_empty_request_gives_zeros(gpu_device):
    say("L = 0 request")
    w = _w(gpu_device, 3, 128, [0, 5, 0], 64, 576, seed=61, poison=True)
    out = run_gpu(w)
    assert (out[0] == 0).all() and (out[2] == 0).all()
    check_gate(out[1:2], oracle_decode(w)[1:2], "L=0 neighbours")


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_forced_splits(gpu_device, splits):
    say("forced splits", splits)
    w = _w(gpu_device, 2, 128, [3000, 700], 64, 64, independent_scales=True, seed=71, poison=True)
    ref = oracle_decode(w)
    out = run_gpu(w, num_splits=splits)
    check_gate(out, ref, f"splits {splits}")
    base = run_gpu(w, num_splits=1)
    check_gate(base, ref, "splits 1")


def test_long_split_many_page_windows(gpu_device):
    """One split per request over up to 20000 keys with 16-key pages: the
    workgroup walks 20 windows of 64 page-table entries, each prefetched while
    the previous one is in use."""
    say("long split over many page windows")
    w = _w(gpu_device, 2, 128, [9000, 20000], 16, 64, independent_scales=True, spare_blocks=3,
           spare_scale_blocks=3, seed=77, poison=True, unused_table_id=0xFFFFFFFF)
    ref = oracle_decode(w)
    check_gate(run_gpu(w, num_splits=1), ref, "one split, 20000 keys")
    check_gate(run_gpu(w), ref, "auto plan")


# ------------------------------------------------------------------ invariances on the GPU
def test_page_permutation_bitwise(gpu_device):
    say("permutation invariance")
    w = _w(gpu_device, 2, 128, [200, 90], 16, 64, independent_scales=True, spare_blocks=5,
           spare_scale_blocks=5, seed=81, poison=True)
    out1 = run_gpu(w, num_splits=1)
    NB = w.blocks.shape[0]
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(1)).to(gpu_device)
    blocks2 = torch.empty_like(w.blocks)
    blocks2[perm] = w.blocks
    lt = w.lookup_table.to(torch.int64) & 0xFFFFFFFF
    lt2 = perm[lt.clamp(max=NB - 1)].to(torch.int32)
    w2 = type(w)(**{**w.__dict__, "blocks": blocks2, "lookup_table": lt2.contiguous()})
    out2 = run_gpu(w2, num_splits=1)
    assert torch.equal(out1, out2)


def test_shared_table_equals_independent_copy(gpu_device):
    say("shared vs independent table")
    w = _w(gpu_device, 2, 128, [130, 400], 64, 576, seed=82, poison=True)
    out1 = run_gpu(w)
    w2 = type(w)(**{**w.__dict__, "scales_lookup_table": w.lookup_table.clone()})
    out2 = run_gpu(w2)
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("gran", [576, 64])
def test_reference_max_jumps(gpu_device, gran):
    """The first 128 keys (the first tiles of both score waves) score near zero,
    later keys score far higher (q scaled by 8): each score wave's reference
    max jumps mid-range, the partner follows it, and the value waves rescale
    their accumulators and the P' tiles that were made against an older
    reference.  Key scales stay in the workload's range (scaling them up would
    inflate |V| far beyond |O|, where no f16 P' meets the gate)."""
    say("reference max jumps", gran)
    w = _w(gpu_device, 2, 128, [1500, 700], 64, gran, independent_scales=gran == 64,
           spare_scale_blocks=2, seed=91, poison=True)
    lt = (w.lookup_table.to(torch.int64) & 0xFFFFFFFF).cpu()
    slt = lt if w.scales_lookup_table is None else (w.scales_lookup_table.to(torch.int64) & 0xFFFFFFFF).cpu()
    P = w.page_size
    for b, L in enumerate(w.lengths()):
        for t in range(min(L, 128)):
            w.scales[int(slt[b, t // P]), 0, 0, t % P, 0, :] *= 1e-3
    w.q.mul_(8.0)
    torch.cuda.synchronize()
    ref = oracle_decode(w)
    check_gate(run_gpu(w, num_splits=1), ref, "jump, one split")
    check_gate(run_gpu(w), ref, "jump, auto plan")


def _q1_calls_match_q4_rows(w, run):
    """Row i of a q_len = 4 call equals a q_len = 1 call on the same cache with
    cache_lengths L - 3 + i (the causal rule); the two launches group rows and
    track reference maxima differently, so they agree to the gate's rounding
    (two bf16 units at most), not bit for bit."""
    import dataclasses
    out4 = run(w).to(torch.float64).cpu().numpy()
    for i in range(4):
        w1 = dataclasses.replace(w, q=w.q[:, i:i + 1].contiguous(), q_len=1,
                                 cache_lengths=(w.cache_lengths - (3 - i)).contiguous())
        out1 = run(w1).to(torch.float64).cpu().numpy()[:, 0]
        d = np.abs(out4[:, i] - out1) / np.maximum(1.0, np.abs(out1))
        say(f"q4 row {i} vs q1 call: max {d.max():.3g} mean {d.mean():.3g}")
        assert d.max() <= 1.6e-2 and d.mean() <= 1e-3, (i, d.max(), d.mean())


@pytest.mark.parametrize("gran", [576, 64])
def test_q4_rows_equal_q1_calls(gpu_device, gran):
    say("q4 rows vs q1 calls", gran)
    w = _w(gpu_device, 3, 128, [40, 700, 2100], 64, gran, q_len=4, independent_scales=gran == 64,
           spare_blocks=2, spare_scale_blocks=2, seed=71 + gran, poison=True)
    _q1_calls_match_q4_rows(w, run_gpu)


@pytest.mark.parametrize("gran,e", [(576, 14), (64, 11)])
def test_split_partials_beyond_f16_range(gpu_device, gran, e):
    """Large scales: scales x 2^e and q x 2^-e leave every score unchanged and
    multiply O by 2^e exactly (powers of two).  With per-token scales (e = 14)
    the outputs pass f16's largest finite value (65504): the fp32 split
    partials and the split merge must carry them, and the per-tile threshold
    must keep P' = p * s finite in f16.  With group scales (e = 11) the scales
    reach the range where P' = p * s_g depends on the threshold's bound
    p <= 2^8 (the documented contract is s_g <= 255)."""
    say("large scales", gran, e)
    w = _w(gpu_device, 2, 128, [3000, 700], 64, gran, independent_scales=gran == 64, seed=73, poison=True)
    w.scales.mul_(2.0 ** e)
    w.q.mul_(2.0 ** -e)
    ref = oracle_decode(w)
    if gran == 576:
        assert np.abs(ref).max() > 65504.0
    else:
        assert 64.0 < float(w.scales[torch.isfinite(w.scales)].max()) <= 255.0
    # the gate is read at the unscaled magnitudes (division by 2^e is exact)
    for splits in (1, 2, 7):
        out = run_gpu(w, num_splits=splits).to(torch.float64) * 2.0 ** -e
        check_gate(out, ref * 2.0 ** -e, f"G{gran} x2^{e} splits {splits}")


@pytest.mark.parametrize("splits", [24, 40, 157])
def test_many_splits_ragged(gpu_device, splits):
    """Many key splits (the merge workgroups then fold them in several waves per wave block)
    with requests that use fewer splits than the plan, or none."""
    say("many splits", splits)
    w = _w(gpu_device, 3, 128, [20000, 3000, 5], 128, 576, seed=75, poison=True)
    ref = oracle_decode(w)
    check_gate(run_gpu(w, num_splits=splits), ref, f"splits {splits}")


def test_longest_first_order(gpu_device):
    """More workgroups than compute units: requests are ranked by length on the
    device (ties by index) and dealt to the XCDs longest first; a batch that is
    not a multiple of 8 leaves empty ranks."""
    rng = np.random.default_rng(77)
    lengths = rng.integers(4, 400, size=37).tolist()
    lengths[5] = lengths[6] = lengths[30] = 257                  # ties
    say("longest-first order, B=37, q_len 4")
    w = _w(gpu_device, 37, 128, lengths, 64, 64, q_len=4, independent_scales=True, spare_blocks=2,
           spare_scale_blocks=2, seed=77, poison=True)
    check_gate(run_gpu(w), oracle_decode(w), "lpt B=37")


def test_largest_key_ranges_first(gpu_device):
    """Splits with more workgroups than compute units: (request, split) key
    ranges are ordered by size on the device -- full splits, then the
    requests' remainders by size, then empty ranges -- covering requests that
    are empty, exact multiples of the split length, or ragged."""
    rng = np.random.default_rng(78)
    lengths = rng.integers(1, 2000, size=40).tolist()
    lengths[3] = lengths[17] = 0
    lengths[8] = 512
    lengths[9] = 1024
    lengths[20] = lengths[21] = 700                      # equal remainders
    say("largest key ranges first, B=40, 4 splits")
    w = _w(gpu_device, 40, 128, lengths, 64, 576, spare_blocks=2, seed=78, poison=True)
    out = run_gpu(w, num_splits=4)
    assert (out[3] == 0).all() and (out[17] == 0).all()
    keep = [b for b in range(40) if lengths[b] > 0]
    check_gate(out[keep], oracle_decode(w)[keep], "lpt splits 4")


@pytest.mark.parametrize("case", [
    # (batch, heads, q_len, page, granularity, max length, seed): default plans that
    # put more workgroups than compute units in flight (largest-first order), with
    # one, two and seven splits per request
    (200, 128, 1, 16, 576, 200, 81),
    (48, 128, 2, 64, 64, 3000, 82),
    (40, 64, 1, 128, 576, 4300, 83),
    (200, 16, 1, 16, 576, 300, 84),           # one row group: the pair's second group is absent
])
def test_default_plans_over_one_wave(gpu_device, case):
    B, H, Q, P, G, lmax, seed = case
    rng = np.random.default_rng(seed)
    lengths = rng.integers(Q, lmax + 1, size=B).tolist()
    lengths[0] = lmax
    lengths[-1] = Q
    say("default plan over one wave", case)
    w = _w(gpu_device, B, H, lengths, P, G, q_len=Q, independent_scales=G == 64, spare_blocks=2,
           spare_scale_blocks=2, seed=seed, poison=True)
    check_gate(run_gpu(w), oracle_decode(w), f"plan {case}")
