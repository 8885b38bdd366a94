"""Pins for the append-and-quantise oracle (oracle/kv_append.py).

Each check ties the oracle to something other than itself: torch's
float8_e4m3fn cast (a library routine), the OCP E4M3FN grid in closed form
(ties, subnormals, the largest value), the half-step error bound of
round-to-nearest, and the decode oracle's own gather (what the append writes is
what decode reads).
"""

import math

import numpy as np
import pytest
import torch

from mla_decode_attention_paged_amd.synth import _quantize_rows
from oracle import E4M3FN_TABLE, FP8_MAX, append_kv, e4m3fn_round, gather_dequant, quantize_row, resolve


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16_values(shape, rng, scale=1.0):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return x.to(torch.bfloat16).to(torch.float32).numpy()


# ------------------------------------------------------------------ rounding
def test_round_matches_torch_cast():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000),          # subnormal range and its edge
        rng.standard_normal(20000) * 30,
    ]).astype(np.float32)
    v = np.clip(v, -FP8_MAX, FP8_MAX)
    assert np.array_equal(e4m3fn_round(v), _torch_e4m3(v))


def test_round_midpoints_go_to_even_codes():
    pos = E4M3FN_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0                     # exact in float32 (short significands)
    codes = e4m3fn_round(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes.astype(np.int64), want)
    assert np.array_equal(codes, _torch_e4m3(mids))       # the library agrees on every tie


def test_round_closed_form_examples():
    ex = [(448.0, 0x7E), (-448.0, 0xFE), (240.0, 0x77), (1.0, 0x38), (1.0625, 0x38), (1.1875, 0x3A),
          (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
          (0.0, 0x00), (-0.0, 0x80), (-2.0 ** -11, 0x80)]
    got = e4m3fn_round(np.array([v for v, _ in ex], dtype=np.float32))
    assert [int(c) for c in got] == [c for _, c in ex]


# ------------------------------------------------------------------ one row
@pytest.mark.parametrize("gran", [576, 64])
def test_quantize_row_half_step_bound(gran):
    rng = np.random.default_rng(gran)
    for k in range(20):
        x = _bf16_values(576, rng, scale=math.exp(rng.normal(0, 2)))
        codes, s = quantize_row(x, gran)
        for g in range(576 // gran):
            xg = x[g * gran:(g + 1) * gran].astype(np.float64)
            amax = np.max(np.abs(xg))
            assert s[g] == np.float32(np.float32(amax) / np.float32(448))
            cg = codes[g * gran:(g + 1) * gran]
            deq = E4M3FN_TABLE[cg] * float(s[g])
            # the largest magnitude maps to +-448 exactly
            j = int(np.argmax(np.abs(xg)))
            assert cg[j] & 0x7F == 0x7E
            # every element within half a grid step of x / s (plus the float32 division's rounding)
            v = xg / float(s[g])
            ex = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
            half_step = np.ldexp(1.0, (ex - 3).astype(int)) / 2
            err = np.abs(v - deq / float(s[g]))
            assert np.all(err <= half_step * (1 + 1e-6) + np.abs(v) * 2.0 ** -23)


def test_zero_group_gets_zero_scale_and_codes():
    x = np.zeros(576, dtype=np.float32)
    x[:64] = 1.5
    codes, s = quantize_row(x, 64)
    assert s[0] == np.float32(1.5 / 448) and np.all(s[1:] == 0)
    assert np.all(codes[64:] == 0)
    codes, s = quantize_row(np.zeros(576, dtype=np.float32), 576)
    assert s[0] == 0 and np.all(codes == 0)


def test_group_scales_equal_token_scale_when_group_maxima_agree():
    rng = np.random.default_rng(9)
    x = _bf16_values(576, rng).reshape(9, 64)
    x[:, 0] = 3.25                                        # every group's amax is 3.25
    x = np.clip(x, -3.0, 3.25).reshape(576)
    c576, s576 = quantize_row(x, 576)
    c64, s64 = quantize_row(x, 64)
    assert np.all(s64 == s576[0]) and np.array_equal(c64, c576)


def test_quantize_matches_torch_recipe():
    """The workload generator quantises float32 rows with torch (fp32 scale, torch's cast)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 576)).astype(np.float32) * np.exp(rng.normal(0, 0.5, (64, 1))).astype(np.float32)
    for gran in (576, 64):
        tc, ts = _quantize_rows(torch.from_numpy(x), gran)
        for r in range(64):
            codes, s = quantize_row(x[r], gran)
            assert np.array_equal(codes, tc[r].numpy()) and np.array_equal(s, ts[r].numpy())


# ------------------------------------------------------------------ the scatter
def _cache(rng, NB, NL, P, NG, poison=0xA5):
    blocks = np.full((NB, 1, NL, P, 1, 576), poison, dtype=np.uint8)
    scales = np.full((NB, 1, NL, P, 1, NG), np.float32(-7.0), dtype=np.float32)
    return blocks, scales


@pytest.mark.parametrize("gran,indep", [(576, False), (64, True)])
def test_append_writes_exactly_the_new_rows(gran, indep):
    rng = np.random.default_rng(13)
    P, NL, layer, q_len, max_pages = 16, 3, 1, 4, 4
    lengths = [4, 17, 33, 64]
    B = len(lengths)
    NB = B * max_pages + 2
    ids = rng.permutation(NB)[:B * max_pages].reshape(B, max_pages).astype(np.uint32)
    sids = rng.permutation(NB)[:B * max_pages].reshape(B, max_pages).astype(np.uint32) if indep else None
    blocks, scales = _cache(rng, NB, NL, P, 576 // gran)
    kv = _bf16_values((B, q_len, 576), rng, scale=2.0)
    nb, ns = append_kv(kv, blocks, scales, ids, sids, lengths, layer, q_len)
    written = np.zeros(blocks.shape[:4], dtype=bool)
    swritten = np.zeros(scales.shape[:4], dtype=bool)
    rows = resolve(ids, sids, lengths, P)
    for b, L in enumerate(lengths):
        for i in range(q_len):
            t = L - q_len + i
            page, slot, spage = rows[b][t]
            codes, s = quantize_row(kv[b, i], gran)
            assert np.array_equal(nb[page, 0, layer, slot, 0], codes)
            assert np.array_equal(ns[spage, 0, layer, slot, 0], s)
            written[page, 0, layer, slot] = True
            swritten[spage, 0, layer, slot] = True
        # the decode oracle's gather reads back code x scale
        K = gather_dequant(nb, ns, rows[b][L - q_len:L], layer, gran)
        for i in range(q_len):
            codes, s = quantize_row(kv[b, i], gran)
            assert np.array_equal(K[i], E4M3FN_TABLE[codes] * np.repeat(s.astype(np.float64), gran))
    assert np.all(nb[~written] == 0xA5) and np.all(ns[~swritten] == np.float32(-7.0))


def test_append_skips_rows_outside_the_table():
    rng = np.random.default_rng(17)
    P, max_pages, q_len = 16, 2, 4
    lengths = [2, 34]          # request 0: t = -2, -1 (skipped), 0, 1; request 1: t = 30..33, 32 and 33 past the table
    ids = np.array([[0, 1], [2, 3]], dtype=np.uint32)
    blocks, scales = _cache(rng, 4, 1, P, 1)
    kv = _bf16_values((2, q_len, 576), rng)
    nb, ns = append_kv(kv, blocks, scales, ids, None, lengths, 0, q_len)
    assert np.array_equal(nb[0, 0, 0, 0, 0], quantize_row(kv[0, 2], 576)[0])
    assert np.array_equal(nb[0, 0, 0, 1, 0], quantize_row(kv[0, 3], 576)[0])
    assert np.array_equal(nb[3, 0, 0, 14, 0], quantize_row(kv[1, 0], 576)[0])
    assert np.array_equal(nb[3, 0, 0, 15, 0], quantize_row(kv[1, 1], 576)[0])
    changed = np.argwhere(np.any(nb != 0xA5, axis=(1, 2, 4, 5)))
    assert sorted(map(tuple, changed.tolist())) == [(0, 0), (0, 1), (3, 14), (3, 15)]
