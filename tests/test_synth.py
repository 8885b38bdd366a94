"""The seeded input generators (synth.py): determinism and the structure the
workload recipe promises (page ids a permutation of the pool, unused table
columns and slots filled as documented, scale = amax / 448 per group)."""

import numpy as np
import torch

from mla_decode_attention_paged_amd.synth import make_workload, u32_numpy


def _bits(t):
    """Bit pattern of a tensor (so that poison NaNs compare equal)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _draw(seed, **kw):
    base = dict(spare_blocks=3, spare_scale_blocks=2, seed=seed, poison=True, unused_table_id=0xFFFFFFFF)
    base.update(kw)
    return make_workload(3, 8, [5, 70, 33], 16, 64, independent_scales=True, **base)


def test_same_seed_same_inputs():
    a, b = _draw(17), _draw(17)
    for f in ("q", "blocks", "scales", "lookup_table", "scales_lookup_table", "cache_lengths"):
        assert torch.equal(_bits(getattr(a, f)), _bits(getattr(b, f))), f


def test_different_seed_different_inputs():
    a, b = _draw(17), _draw(18)
    assert not torch.equal(_bits(a.q), _bits(b.q))
    assert not torch.equal(a.lookup_table, b.lookup_table)


def test_page_ids_are_a_permutation_and_unused_columns_marked():
    w = _draw(5)
    lt = u32_numpy(w.lookup_table)
    slt = u32_numpy(w.scales_lookup_table)
    lens, P = w.lengths(), w.page_size
    used = [lt[b, c] for b, L in enumerate(lens) for c in range((L + P - 1) // P)]
    sused = [slt[b, c] for b, L in enumerate(lens) for c in range((L + P - 1) // P)]
    assert len(set(used)) == len(used) and max(used) < w.blocks.shape[0]
    assert len(set(sused)) == len(sused) and max(sused) < w.scales.shape[0]
    for b, L in enumerate(lens):
        assert (lt[b, (L + P - 1) // P:] == 0xFFFFFFFF).all()
        assert (slt[b, (L + P - 1) // P:] == 0xFFFFFFFF).all()


def test_scales_are_group_amax_over_448_and_unused_slots_poisoned():
    w = _draw(9)
    lt, slt = u32_numpy(w.lookup_table), u32_numpy(w.scales_lookup_table)
    blocks, scales = w.blocks.numpy(), w.scales.numpy()
    P = w.page_size
    codes_max = []
    for b, L in enumerate(w.lengths()):
        for t in range(L):
            row = blocks[lt[b, t // P], 0, 0, t % P, 0]
            s = scales[slt[b, t // P], 0, 0, t % P, 0]
            assert np.isfinite(s).all() and (s > 0).all()
            # the group's largest code is 448 in magnitude (0x7E / 0xFE): scale = amax / 448
            codes_max.append((row.reshape(9, 64) & 0x7F).max(axis=1))
        # slots past the request's last token in its last page hold the NaN code
        if L % P:
            assert (blocks[lt[b, (L - 1) // P], 0, 0, L % P:, 0] == 0x7F).all()
    assert (np.concatenate(codes_max) == 0x7E).all()


def test_unquantized_cache_rows_and_poison():
    w = make_workload(2, 4, [20, 3], 16, 576, spare_blocks=2, seed=3, poison=True, kv_dtype="bf16")
    assert w.scales is None and w.blocks.dtype == torch.bfloat16
    lt = u32_numpy(w.lookup_table)
    finite = torch.isfinite(w.blocks.float())
    for b, L in enumerate(w.lengths()):
        for t in range(L):
            assert finite[lt[b, t // 16], 0, 0, t % 16, 0].all()
    assert int(finite.all(dim=-1).sum()) == sum(w.lengths())
