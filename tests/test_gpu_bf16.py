"""GPU parity of the unquantized (bf16 cache) decode, through the C ABI,
against the FP64 oracle of oracle/unquantized.py.

The gate is the one of the FP8 path: e = |gpu - bf16(oracle)| / max(1, |oracle|),
max e <= 1e-2 and mean e <= 1e-3.  Cases cover NaN-poisoned unused slots,
pages and layers, ragged tails around the 32-key tile and 16-key load block,
lengths below q_len, empty requests, forced split counts (partials merged by
the split merge of the same launch), causal q_len > 1, odd head counts, and the full-size
uniform workload (16 x 4096 keys, 128 heads) on sampled requests in the
launch configuration the benchmark times.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_paged_amd import mla_decode_paged_bf16
from mla_decode_attention_paged_amd.synth import make_workload, uniform_bf16
from tests.gpu_helpers import check_gate, extract_requests, say
from tests.oracle_inputs import oracle_decode_unquantized

pytestmark = pytest.mark.gpu


def run_bf16(w, num_splits=None):
    out = mla_decode_paged_bf16(w.q, w.blocks, w.lookup_table, w.cache_lengths, w.layer_idx, w.q_len,
                                w.softmax_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out


def _w(gpu_device, *args, **kw):
    kw.setdefault("device", gpu_device)
    kw["kv_dtype"] = "bf16"
    return make_workload(*args, **kw)


def test_tiny_poisoned(gpu_device):
    say("bf16 tiny (B=2, H=16, L={37,100}, P=16, NaN poison)")
    w = _w(gpu_device, 2, 16, [37, 100], 16, 576, spare_blocks=6, seed=1, poison=True,
           unused_table_id=0xFFFFFFFF)
    check_gate(run_bf16(w), oracle_decode_unquantized(w), "bf16 tiny")


@pytest.mark.parametrize("splits", [None, 1, 3])
def test_ragged_tails(gpu_device, splits):
    lengths = [1, 15, 16, 17, 31, 32, 33, 100, 129, 1000]
    say("bf16 ragged tails, splits", splits)
    w = _w(gpu_device, len(lengths), 128, lengths, 64, 576, spare_blocks=2, seed=7, poison=True)
    check_gate(run_bf16(w, num_splits=splits), oracle_decode_unquantized(w), f"bf16 ragged s{splits}")


@pytest.mark.parametrize("q_len,heads,page", [(4, 128, 64), (4, 16, 16), (16, 128, 128), (3, 24, 32)])
def test_causal_queries(gpu_device, q_len, heads, page):
    say("bf16 causal", q_len, heads, page)
    lengths = [q_len, q_len + 5, 300, 2100]
    w = _w(gpu_device, len(lengths), heads, lengths, page, 576, q_len=q_len, num_layers=3, layer_idx=1,
           kv_dim=2, spare_blocks=3, seed=11 + q_len + heads, poison=True)
    check_gate(run_bf16(w), oracle_decode_unquantized(w), f"bf16 causal q{q_len} h{heads} p{page}")


def test_empty_and_short_requests(gpu_device):
    """cache_lengths 0 yields zeros; lengths below q_len leave the first rows empty."""
    say("bf16 empty / short")
    w = _w(gpu_device, 4, 16, [5, 2, 40, 9], 16, 576, q_len=4, spare_blocks=1, seed=3, poison=True)
    w.cache_lengths[0] = 0
    out = run_bf16(w)
    assert torch.count_nonzero(out[0]).item() == 0
    ref = oracle_decode_unquantized(w.to("cpu"))
    assert (ref[0] == 0).all() and (ref[1, :2] == 0).all()     # request 1: rows 0, 1 see no key
    assert np.isfinite(out.float().cpu().numpy()).all()
    check_gate(out[1:], ref[1:], "bf16 short")


def test_uniform_full_size_sampled(gpu_device):
    """16 x 4096 keys, 128 heads, page 64, in the automatic plan (the benchmark's
    launch configuration); requests 0, 7 and 15 against the oracle."""
    say("bf16 uniform full size")
    w = uniform_bf16(device=gpu_device)
    out = run_bf16(w)
    batches = [0, 7, 15]
    sub = extract_requests(w, batches).to("cpu")
    ref = oracle_decode_unquantized(sub)
    check_gate(out[batches], ref, "bf16 uniform sampled")
    assert np.isfinite(out.float().cpu().numpy()).all()


def test_long_context_sampled(gpu_device):
    """One request of 131072 keys (page 128): many splits merged by the split merge."""
    say("bf16 long 131072")
    w = _w(gpu_device, 1, 128, [131072], 128, 576, seed=3001, poison=False)
    check_gate(run_bf16(w), oracle_decode_unquantized(w.to("cpu")), "bf16 long")


def test_q4_rows_equal_q1_calls(gpu_device):
    from tests.test_gpu_parity import _q1_calls_match_q4_rows
    say("bf16 q4 rows vs q1 calls")
    w = _w(gpu_device, 3, 128, [40, 700, 2100], 64, 576, q_len=4, spare_blocks=2, seed=77, poison=True)
    _q1_calls_match_q4_rows(w, run_bf16)


def test_reference_max_jumps(gpu_device):
    """The first 128 keys score near zero (their rows scaled by 1e-3) and later
    keys far higher (q scaled by 8): each score wave's reference jumps
    mid-range and the other key half's wave follows it a tile later, so the
    value waves rescale O and the P tiles that were made against an older
    reference (both rare paths), in one split and in the automatic plan."""
    say("bf16 reference max jumps")
    w = _w(gpu_device, 2, 128, [1500, 700], 64, 576, seed=91, poison=True)
    lt = (w.lookup_table.to(torch.int64) & 0xFFFFFFFF).cpu()
    P = w.page_size
    for b, L in enumerate(w.lengths()):
        for t in range(min(L, 128)):
            w.blocks[int(lt[b, t // P]), 0, w.layer_idx, t % P, 0, :] *= 1e-3
    w.q.mul_(8.0)
    torch.cuda.synchronize()
    ref = oracle_decode_unquantized(w)
    check_gate(run_bf16(w, num_splits=1), ref, "bf16 jump, one split")
    check_gate(run_bf16(w), ref, "bf16 jump, auto plan")


@pytest.mark.parametrize("splits", [24, 157])
def test_many_splits_ragged(gpu_device, splits):
    """Many key splits (splits of one to four tiles, so the two-ahead tile
    stream starts and drains inside a few steps) with requests that use fewer
    splits than the plan, or one."""
    say("bf16 many splits", splits)
    w = _w(gpu_device, 3, 128, [20000, 3000, 5], 128, 576, seed=75, poison=True)
    check_gate(run_bf16(w, num_splits=splits), oracle_decode_unquantized(w), f"bf16 splits {splits}")


def test_split_partials_beyond_f16_range(gpu_device):
    """Cache rows x 2^14 and q x 2^-14: the same scores, O x 2^14, past f16's
    largest finite value; the fp32 split partials and the split merge must carry
    such outputs, and P (bf16 hi + lo) must stay exact enough at that scale."""
    say("bf16 cache, partials beyond the f16 range")
    w = _w(gpu_device, 2, 128, [3000, 700], 64, 576, seed=74, poison=True, kv_dtype="bf16")
    w.blocks.mul_(2.0 ** 14)
    w.q.mul_(2.0 ** -14)
    ref = oracle_decode_unquantized(w)
    assert np.abs(ref).max() > 65504.0
    # the gate is read at the unscaled magnitudes (division by 2^14 is exact)
    for splits in (1, 2, 7):
        out = run_bf16(w, num_splits=splits).to(torch.float64) * 2.0 ** -14
        check_gate(out, ref * 2.0 ** -14, f"bf16 x2^14 splits {splits}")


def test_largest_key_ranges_first(gpu_device):
    """More workgroups than compute units over the bf16 cache: key ranges run
    largest first, with empty requests and exact multiples of the split."""
    rng = np.random.default_rng(79)
    lengths = rng.integers(1, 2000, size=40).tolist()
    lengths[2] = 0
    lengths[11] = 512
    lengths[30] = lengths[31] = 900
    say("bf16 cache, largest key ranges first, B=40, 4 splits")
    w = _w(gpu_device, 40, 128, lengths, 64, 576, spare_blocks=2, seed=79, poison=True)
    out = run_bf16(w, num_splits=4)
    assert (out[2] == 0).all()
    keep = [b for b in range(40) if lengths[b] > 0]
    check_gate(out[keep], oracle_decode_unquantized(w)[keep], "bf16 lpt splits 4")
