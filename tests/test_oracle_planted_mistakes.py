"""Planted mistakes: the oracle's pins must catch plausible errors in it.

Each mutant is a copy of oracle/mla_oracle.py with one small textual change of
the kind that slips into such code -- a dropped term, a wrong sign, an index
off by one, a swapped table or operand, a wrong rounding mode -- executed as a
module of its own on the CPU.  The real oracle must pass every pin below; every
mutant must fail at least one (an exception counts as a failure).  The pins
are restatements of the ones in test_oracle_*.py, sized to run in seconds:
the OCP E4M3FN decode against torch's float8_e4m3fn; bf16 rounding against
torch's bfloat16 cast; the hand-worked resolution and two-key examples
(tests/golden/); identity paging against torch's scaled_dot_product_attention;
rows summing to 1; one cached key returning its value row; the causal rule;
equal group scales against per-token scales; page permutation invariance; the
log-sum-exp merge; a scalar brute force with math.fsum; and the same brute
force over per-request query counts.
"""

import json
import math
import os
import types

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "mla_oracle.py")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_variant(replace=None):
    """The oracle module, or a copy with one planted change (old -> new, which
    must occur exactly once in the source)."""
    src = open(ORACLE_SRC).read()
    if replace is not None:
        old, new = replace
        assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_variant")
    exec(compile(src, ORACLE_SRC, "exec"), mod.__dict__)
    return mod


# --------------------------------------------------------------------- pins
def pin_codec(o):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.asarray(o.E4M3FN_TABLE)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(ref)], ref[~np.isnan(ref)])


def pin_bf16(o):
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    # float32 is exact for these test values' bf16 neighbours only when x is a float32; compare on float32 inputs
    got = o.bf16_round(x.astype(np.float32).astype(np.float64))
    assert np.array_equal(got, ref)


def pin_resolve_golden(o):
    with open(os.path.join(GOLDEN, "resolve_worked_example.json")) as f:
        g = json.load(f)
    rows = o.resolve(np.array(g["lookup_table"], dtype=np.uint32),
                     np.array(g["scales_lookup_table"], dtype=np.uint32), g["cache_lengths"], g["page_size"])
    for tok in g["tokens"]:
        assert tuple(rows[tok["b"]][tok["t"]]) == (tok["page"], tok["slot"], tok["spage"])


def pin_two_keys(o):
    with open(os.path.join(GOLDEN, "attention_two_keys.json")) as f:
        g = json.load(f)
    P, D = g["page_size"], 576
    blocks = np.zeros((1, 1, 1, P, 1, D), dtype=np.uint8)
    scales = np.zeros((1, 1, 1, P, 1, 1), dtype=np.float32)
    for j, key in enumerate(g["keys"]):
        for d, code in key["codes"].items():
            blocks[0, 0, 0, j, 0, int(d)] = int(code, 16)
        scales[0, 0, 0, j, 0, 0] = key["scale"]
    q = np.zeros((1, 1, 1, D))
    for d, v in g["q_nonzero"].items():
        q[0, 0, 0, int(d)] = v
    O, lse = o.decode(q, blocks, scales, np.zeros((1, 1), dtype=np.uint32), None, [2], 0, 1,
                      g["softmax_scale"], return_lse=True)
    e = math.e
    expect = np.zeros(512)
    expect[0] = e / (1 + e)
    expect[1] = 2.0 / (1 + e) + 0.5 * e / (1 + e)
    assert np.allclose(O[0, 0, 0], expect, rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(1 + e)) < 1e-15


def _closed_form_e4m3(code):
    code = int(code)
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    return s * (m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))


def _random_cache(seed, lengths, P=16, G=576, NL=1, layer=0, indep=False, H=3, Q=1, spare=2):
    """A small paged cache with random page ids, poisoned spare pages and layers."""
    rng = np.random.default_rng(seed)
    D, NG = 576, 576 // G
    pages = [(L + P - 1) // P for L in lengths]
    used = sum(pages)
    NB = used + spare
    blocks = np.full((NB, 1, NL, P, 1, D), 0x7F, dtype=np.uint8)
    scales = np.full((NB, 1, NL, P, 1, NG), np.nan, dtype=np.float32)
    finite = np.flatnonzero(np.isfinite([_closed_form_e4m3(c) for c in range(256)]))
    perm = rng.permutation(NB)[:used]
    sperm = rng.permutation(NB)[:used] if indep else perm
    lt = np.full((len(lengths), max(pages)), 0xFFFFFFFF, dtype=np.uint32)
    slt = lt.copy()
    k = 0
    for b, L in enumerate(lengths):
        for c in range(pages[b]):
            lt[b, c], slt[b, c] = perm[k], sperm[k]
            n = min(P, L - c * P)
            blocks[perm[k], 0, layer, :n, 0, :] = rng.choice(finite, size=(n, D))
            scales[sperm[k], 0, layer, :n, 0, :] = rng.uniform(0.01, 0.05, size=(n, NG))
            k += 1
    q = rng.standard_normal((len(lengths), Q, H, D))
    return q, blocks, scales, lt, (slt if indep else None)


def pin_dense(o):
    """Identity paging, unit scales: textbook attention (torch SDPA, float64)."""
    rng = np.random.default_rng(1)
    L, P, H, D = 21, 16, 3, 576
    finite = np.flatnonzero(np.isfinite(np.asarray([_closed_form_e4m3(c) for c in range(256)])) &
                            (np.abs([_closed_form_e4m3(c) if c not in (0x7F, 0xFF) else 0 for c in range(256)]) <= 4))
    blocks = rng.choice(finite, size=(2, 1, 1, P, 1, D)).astype(np.uint8)
    scales = np.ones((2, 1, 1, P, 1, 1), dtype=np.float32)
    lt = np.array([[0, 1]], dtype=np.uint32)
    q = rng.standard_normal((1, 1, H, D))
    sm = 0.0721
    O = o.decode(q, blocks, scales, lt, None, [L], 0, 1, sm)
    K = torch.tensor([[_closed_form_e4m3(c) for c in row] for row in blocks[:, 0, 0, :, 0, :].reshape(-1, D)[:L]],
                     dtype=torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0]).unsqueeze(0), K.unsqueeze(0).unsqueeze(0).expand(1, H, L, D),
        K[:, :512].unsqueeze(0).unsqueeze(0).expand(1, H, L, 512), scale=sm)[0]
    assert np.allclose(O[0, 0], ref.numpy(), rtol=0, atol=1e-12)


def pin_rows_sum(o):
    rng = np.random.default_rng(2)
    K = rng.standard_normal((37, 576))
    _, _, w = o.attention_rows(rng.standard_normal((4, 576)), K, 30, 0.1, 512)
    assert w.shape == (4, 30)
    assert np.all(w >= 0) and np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def pin_one_key(o):
    q, blocks, scales, lt, slt = _random_cache(3, [1, 1], indep=True)
    O = o.decode(q, blocks, scales, lt, slt, [1, 1], 0, 1, 0.07)
    for b in range(2):
        page, spage = lt[b, 0], slt[b, 0]
        v = np.array([_closed_form_e4m3(c) for c in blocks[page, 0, 0, 0, 0, :512]]) * float(scales[spage, 0, 0, 0, 0, 0])
        assert np.array_equal(O[b, 0], np.broadcast_to(v, O[b, 0].shape))


def pin_causal(o):
    lengths = [9, 40]
    q, blocks, scales, lt, slt = _random_cache(4, lengths, Q=4)
    O4 = o.decode(q, blocks, scales, lt, slt, lengths, 0, 4, 0.09)
    for i in range(4):
        O1 = o.decode(q[:, i:i + 1], blocks, scales, lt, slt, [L - 3 + i for L in lengths], 0, 1, 0.09)
        assert np.allclose(O4[:, i], O1[:, 0], rtol=0, atol=1e-12)


def pin_group_equal(o):
    lengths = [20, 33]
    q, blocks, scales, lt, slt = _random_cache(5, lengths)
    scales9 = np.repeat(scales, 9, axis=-1)
    a = o.decode(q, blocks, scales, lt, slt, lengths, 0, 1, 0.08)
    b = o.decode(q, blocks, scales9, lt, slt, lengths, 0, 1, 0.08)
    assert np.array_equal(a, b)
    # and a group scale that differs from the others changes exactly what it should
    scales9[..., 3] *= 2.0
    c = o.decode(q, blocks, scales9, lt, slt, lengths, 0, 1, 0.08)
    assert not np.allclose(a, c)


def pin_perm(o):
    lengths = [23, 50]
    q, blocks, scales, lt, slt = _random_cache(6, lengths, indep=True, spare=3)
    a = o.decode(q, blocks, scales, lt, slt, lengths, 0, 1, 0.08)
    NB = blocks.shape[0]
    perm = np.random.default_rng(7).permutation(NB)
    blocks2 = np.empty_like(blocks)
    blocks2[perm] = blocks
    lt2 = np.where(lt == 0xFFFFFFFF, lt, perm[np.minimum(lt, NB - 1)]).astype(np.uint32)
    b = o.decode(q, blocks2, scales, lt2, slt, lengths, 0, 1, 0.08)
    assert np.array_equal(a, b)


def pin_merge(o):
    lengths = [45, 17]
    q, blocks, scales, lt, slt = _random_cache(8, lengths, Q=2, indep=True)
    full, lse = o.decode(q, blocks, scales, lt, slt, lengths, 0, 2, 0.08, return_lse=True)
    parts = [o.decode_range(q, blocks, scales, lt, slt, lengths, 0, 2, 0.08, t0, t1)
             for t0, t1 in ((0, 7), (7, 30), (30, 64))]
    O, l = o.merge_partials(parts)
    assert np.allclose(O, full, rtol=0, atol=1e-12)
    assert np.allclose(l, lse, rtol=0, atol=1e-12)


def pin_brute(o):
    """Scalar loops and math.fsum: causal q_len 2, layer 1 of 2, group scales,
    an independent scales table, random page ids."""
    lengths = [5, 19]
    P, G, Q, H, sm, layer = 16, 64, 2, 2, 0.11, 1
    q, blocks, scales, lt, slt = _random_cache(9, lengths, P=P, G=G, NL=2, layer=layer, indep=True, H=H, Q=Q)
    O = o.decode(q, blocks, scales, lt, slt, lengths, layer, Q, sm)
    for b, L in enumerate(lengths):
        K = []
        for t in range(L):
            page, slot, spage = int(lt[b, t // P]), t % P, int(slt[b, t // P])
            K.append([_closed_form_e4m3(blocks[page, 0, layer, slot, 0, d]) *
                      float(scales[spage, 0, layer, slot, 0, d // G]) for d in range(576)])
        for i in range(Q):
            n = L - Q + i + 1
            for h in range(H):
                s = [sm * math.fsum(q[b, i, h, d] * K[j][d] for d in range(576)) for j in range(n)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                den = math.fsum(e)
                for c in (0, 100, 511):
                    ref = math.fsum(e[j] / den * K[j][c] for j in range(n))
                    assert abs(O[b, i, h, c] - ref) <= 1e-12 * max(1.0, abs(ref))


def pin_ragged(o):
    """Per-request query counts (3, 0, 2, 1): scalar loops and math.fsum, each
    request causal among its own new tokens."""
    lengths, counts = [6, 4, 9, 3], [3, 0, 2, 1]
    P, G, H, sm = 16, 64, 2, 0.09
    _, blocks, scales, lt, slt = _random_cache(13, lengths, P=P, G=G, indep=True, H=H)
    rng = np.random.default_rng(14)
    offs = np.concatenate([[0], np.cumsum(counts)])
    q = rng.standard_normal((int(offs[-1]), H, 576))
    O = o.decode_ragged(q, offs, blocks, scales, lt, slt, lengths, 0, sm)
    for b, L in enumerate(lengths):
        K = []
        for t in range(L):
            page, slot, spage = int(lt[b, t // P]), t % P, int(slt[b, t // P])
            K.append([_closed_form_e4m3(blocks[page, 0, 0, slot, 0, d]) *
                      float(scales[spage, 0, 0, slot, 0, d // G]) for d in range(576)])
        n = counts[b]
        for i in range(n):
            vis = L - n + i + 1
            for h in range(H):
                row = int(offs[b]) + i
                s = [sm * math.fsum(q[row, h, d] * K[j][d] for d in range(576)) for j in range(vis)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                den = math.fsum(e)
                for c in (0, 300, 511):
                    ref = math.fsum(e[j] / den * K[j][c] for j in range(vis))
                    assert abs(O[row, h, c] - ref) <= 1e-12 * max(1.0, abs(ref))


PINS = [pin_codec, pin_bf16, pin_resolve_golden, pin_two_keys, pin_dense, pin_rows_sum, pin_one_key,
        pin_causal, pin_group_equal, pin_perm, pin_merge, pin_brute, pin_ragged]

MUTANTS = {
    "softmax scale dropped": ("scores = softmax_scale * (q_rows @ Kv.T)", "scores = (q_rows @ Kv.T)"),
    "value from the last 512 dims": ("O = w @ Kv[:, :dv]", "O = w @ Kv[:, -dv:]"),
    "causal limit off by one": ("n_vis = max(0, min(L, L - Q + i + 1))", "n_vis = max(0, min(L, L - Q + i))"),
    "scale page from the value table": ("rows[t, 2] = int(slt[b, col])", "rows[t, 2] = int(lt[b, col])"),
    "slot and column swapped": ("rows[t, 1] = t % page_size", "rows[t, 1] = t // page_size"),
    "scale groups reversed": ("groups = np.arange(head_dim) // granularity",
                              "groups = (np.arange(head_dim) // granularity)[::-1]"),
    "sign of the max subtraction": ("e = np.exp(scores - m)", "e = np.exp(m - scores)"),
    "exponent bias 8": ("return sign * math.ldexp(1.0 + m / 8.0, e - 7)",
                        "return sign * math.ldexp(1.0 + m / 8.0, e - 8)"),
    "subnormal scale 2^-7": ("return sign * math.ldexp(m / 8.0, -6)", "return sign * math.ldexp(m / 8.0, -7)"),
    "layer index ignored": ("codes = blocks[page, 0, layer_idx, slot, 0, :]", "codes = blocks[page, 0, 0, slot, 0, :]"),
    "scales read through the value page": ("s = scales[spage, 0, layer_idx, slot, 0, :]",
                                           "s = scales[page, 0, layer_idx, slot, 0, :]"),
    "q depth reversed against K": ("scores = softmax_scale * (q_rows @ Kv.T)",
                                   "scores = softmax_scale * (q_rows[:, ::-1] @ Kv.T)"),
    "bf16 rounding truncates": ("r = np.ldexp(np.rint(scaled), q_exp)", "r = np.ldexp(np.floor(scaled), q_exp)"),
    "lse without the max": ("lse = (m + np.log(denom))[:, 0]", "lse = (np.log(denom))[:, 0]"),
    "weights not normalised": ("w = e / denom", "w = e / (denom + 1.0)"),
    "merge weights against the max, not the lse": (
        "coef = np.where(finite, 1.0, 0.0) * np.exp(lses - np.where(finite, lse, 0.0))",
        "coef = np.where(finite, 1.0, 0.0) * np.exp(lses - np.where(finite, Msafe, 0.0))"),
    "range causal limit off by one": ("hi = min(t1, max(0, min(L, L - Q + i + 1)))",
                                      "hi = min(t1, max(0, min(L, L - Q + i + 2)))"),
    "ragged causal limit from the largest count": (
        "n_vis = max(0, min(L, L - n + i + 1))        # readings R1, R16",
        "n_vis = max(0, min(L, L - max(offs[k + 1] - offs[k] for k in range(B)) + i + 1))"),
    "ragged query rows shifted by one": ("o, l, _ = attention_rows(q[first + i], K, n_vis, softmax_scale, dv)",
                                         "o, l, _ = attention_rows(q[min(first + i + 1, T - 1)], K, n_vis, softmax_scale, dv)"),
    "ragged count from the wrong offsets": ("first, n = offs[b], offs[b + 1] - offs[b]",
                                            "first, n = offs[b], offs[b + 1] - offs[max(b - 1, 0)]"),
}


def _failed_pins(mod):
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception as e:          # an exception counts as a failed pin
            failed.append((pin.__name__, type(e).__name__))
    return failed


def test_real_oracle_passes_every_pin():
    assert _failed_pins(load_variant()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    failed = _failed_pins(load_variant(MUTANTS[name]))
    assert failed, f"no pin catches the planted mistake: {name}"
