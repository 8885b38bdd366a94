"""GPU: the split merge that runs in the decode launch itself.

A split call's workspace starts with 288 KiB of completion flags (zero
before a buffer's first use); every call must return them to zero, so one
workspace serves call after call, of any shape, and graph replays.  Outputs
are compared bit for bit with the same call on a fresh workspace (the
kernels are deterministic) and against the FP64 oracle, including the merge
plan's multi-block chunks (each wave of a merge workgroup merging two or four
wave blocks in turn) in both decode kernels.
"""

import pytest
import torch

from mla_decode_attention_paged_amd import mla_decode_paged_fp8, mla_decode_paged_fp8_plan, new_workspace
from mla_decode_attention_paged_amd.synth import make_workload
from tests.gpu_helpers import check_gate, run_gpu, say
from tests.oracle_inputs import oracle_decode

pytestmark = pytest.mark.gpu

FLAG_BYTES = 288 * 1024


def _w(gpu_device, *args, **kw):
    kw.setdefault("device", gpu_device)
    return make_workload(*args, **kw)


def _need(w, splits):
    scales_shape = tuple(w.scales.shape)
    return mla_decode_paged_fp8_plan(tuple(w.q.shape), tuple(w.blocks.shape), scales_shape,
                                     tuple(w.lookup_table.shape), w.q_len, splits)["workspace_bytes"]


def _cases(gpu_device):
    lengths40 = [(37 * b) % 1900 + 1 for b in range(40)]
    lengths40[3] = 0
    return [
        (_w(gpu_device, 2, 128, [3000, 700], 64, 64, independent_scales=True, seed=171, poison=True), 3),
        (_w(gpu_device, 3, 16, [20000, 3000, 5], 128, 576, seed=172, poison=True), 24),    # one row group
        (_w(gpu_device, 40, 128, lengths40, 64, 576, seed=173, poison=True), 4),           # largest first
        (_w(gpu_device, 2, 16, [2100, 900], 64, 64, q_len=3, seed=174, poison=True), 5),  # 48 rows
    ]


def test_one_workspace_across_shapes(gpu_device):
    cases = _cases(gpu_device)
    ws = new_workspace(max(_need(w, s) for w, s in cases), gpu_device)
    for rep in range(2):
        for k, (w, splits) in enumerate(cases):
            say("shared workspace, case", k, "pass", rep)
            out = run_gpu(w, num_splits=splits, workspace=ws)
            assert int(torch.count_nonzero(ws[:FLAG_BYTES])) == 0, "split counters not returned to zero"
            fresh = run_gpu(w, num_splits=splits)
            assert torch.equal(out, fresh), f"case {k}: shared workspace result differs"


@pytest.mark.parametrize("k", [0, 1, 3])
def test_merge_cases_against_oracle(gpu_device, k):
    w, splits = _cases(gpu_device)[k]
    say("split merge vs oracle, case", k)
    check_gate(run_gpu(w, num_splits=splits), oracle_decode(w), f"case {k}, splits {splits}")


def test_graph_replays(gpu_device):
    """The split call captured in a HIP graph: every replay (with eager decode
    calls and synchronizations between them) equals the eager result."""
    w = _w(gpu_device, 2, 128, [3000, 700], 64, 64, independent_scales=True, seed=175, poison=True)
    other = _w(gpu_device, 3, 16, [20000, 3000, 5], 128, 576, seed=176, poison=True)
    splits = 3
    ws = new_workspace(_need(w, splits), gpu_device)
    out = torch.empty((w.batch, w.q_len, w.num_heads, 512), dtype=torch.bfloat16, device=gpu_device)

    def call():
        mla_decode_paged_fp8(w.q, w.blocks, w.scales, w.lookup_table, w.scales_lookup_table, w.cache_lengths,
                             w.layer_idx, w.q_len, w.softmax_scale, out=out, workspace=ws, num_splits=splits)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                   # warm the side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        say("graph replay", rep)
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        assert int(torch.count_nonzero(ws[:FLAG_BYTES])) == 0
        run_gpu(other, num_splits=24)            # eager work between replays


def _many_groups(gpu_device, kv_dtype, seed):
    """32 requests x 128 heads = 128 row groups: with splits the merge plan
    takes chunks of 16 wave blocks, so each wave of a merge workgroup merges
    two (the 8-wave kernels) or four (the 4-wave kernel of the FP8-MFMA "kv"
    mode) blocks in turn."""
    lengths = [(97 * b) % 1500 + 1 for b in range(32)]
    lengths[5] = 0
    return _w(gpu_device, 32, 128, lengths, 64, 576, seed=seed, poison=True, kv_dtype=kv_dtype)


@pytest.mark.parametrize("splits", [2, 5])
def test_multi_block_merge_fp8(gpu_device, splits):
    w = _many_groups(gpu_device, "fp8", 177)
    say("multi-block merge, fp8, splits", splits)
    check_gate(run_gpu(w, num_splits=splits), oracle_decode(w), f"fp8 multi-block merge, splits {splits}")


@pytest.mark.parametrize("splits", [2, 5])
def test_multi_block_merge_bf16(gpu_device, splits):
    from mla_decode_attention_paged_amd import mla_decode_paged_bf16
    from tests.oracle_inputs import oracle_decode_unquantized
    w = _many_groups(gpu_device, "bf16", 178)
    say("multi-block merge, bf16, splits", splits)
    out = mla_decode_paged_bf16(w.q, w.blocks, w.lookup_table, w.cache_lengths, w.layer_idx, w.q_len,
                                w.softmax_scale, num_splits=splits)
    torch.cuda.synchronize()
    check_gate(out, oracle_decode_unquantized(w), f"bf16 multi-block merge, splits {splits}")


@pytest.mark.parametrize("mode", ["v", "kv"])
def test_multi_block_merge_fp8_mfma(gpu_device, mode):
    """The FP8-MFMA entry points with 128 row groups and 2 splits: merge
    chunks of 16 wave blocks, two per wave in the 8-wave kernel ("v") and
    four per wave in the 4-wave kernel ("kv", the only kernel that takes the
    four-block form); each mode against its own bound."""
    from tests.test_gpu_fp8_value import check, run_f8
    w = _many_groups(gpu_device, "fp8", 179)
    say("multi-block merge, fp8 mfma", mode)
    check(mode, run_f8(w, mode, 2), oracle_decode(w), f"fp8 mfma {mode} multi-block merge")
