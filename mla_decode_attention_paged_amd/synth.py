"""Seeded synthetic workloads for paged-FP8 MLA decode.

This module only draws inputs: random queries, random latent rows quantised to
FP8 E4M3FN with one float32 scale per group (amax / 448), random page-id
permutations and cache lengths.  It holds none of the attention arithmetic and
is shared by the tests, the benchmark and the smoke check.

Tensor shapes follow the "generic_get_paged_cache_with_scales" page (section
"Args"): blocks [num_blocks, kv_dim, num_layers, page_size, num_kv_heads,
head_dim] as raw E4M3FN bytes, scales [num_scale_blocks, kv_dim, num_layers,
page_size, num_kv_heads, head_dim / granularity] float32, lookup tables
[batch, max_pages] uint32, cache_lengths [batch] uint32.

Value recipe (shared by all workloads):
  q      ~ bf16(N(0, 1))                               [B, q_len, H, 576]
  row    = N(0, 1)^576 * m,  m ~ LogNormal(0, 0.5)      per cached token
  scale  = float32(amax(|row_g|) / 448)                 per group g of `granularity`
  code   = e4m3fn(clip(row_g / scale, -448, 448))       round to nearest even
With kv_dtype="bf16" (the unquantized cache) blocks holds bf16(row) and
there are no scales.
Page ids of a request are drawn from a random permutation of the pool, in
(request, page) order; scale pages use their own permutation when the scales
are paged independently.  Slots past a request's length, pages no request
uses, layers other than the selected one and kv_dim entries other than 0 are
filled with `fill_code` (0x7F, an E4M3FN NaN, in poison mode; a bf16 NaN for
the unquantized cache) so that any read of them shows up in the result.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEAD_DIM = 576
V_DIM = 512
FP8_MAX = 448.0
NAN_CODE = 0x7F


@dataclasses.dataclass
class Workload:
    """One decode call's inputs (tensors live on `device`)."""

    q: torch.Tensor                  # bf16 [B, Q, H, 576]
    blocks: torch.Tensor             # uint8 [NB, KVD, NL, P, 1, 576] (bf16 when unquantized)
    scales: torch.Tensor | None      # float32 [NBs, KVD, NL, P, 1, NG]; None when unquantized
    lookup_table: torch.Tensor       # int32 view of uint32 ids [B, max_pages]
    scales_lookup_table: torch.Tensor | None
    cache_lengths: torch.Tensor      # int32 view of uint32 [B]
    layer_idx: int
    q_len: int
    softmax_scale: float
    page_size: int
    granularity: int
    name: str = ""

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def num_heads(self) -> int:
        return self.q.shape[2]

    def lengths(self) -> list[int]:
        return [int(v) for v in self.cache_lengths.cpu().tolist()]

    def to(self, device) -> "Workload":
        f = lambda t: None if t is None else t.to(device)  # noqa: E731
        return dataclasses.replace(
            self, q=f(self.q), blocks=f(self.blocks), scales=f(self.scales),
            lookup_table=f(self.lookup_table),
            scales_lookup_table=f(self.scales_lookup_table),
            cache_lengths=f(self.cache_lengths))


def _quantize_rows(x: torch.Tensor, granularity: int):
    """E4M3FN codes (uint8) and float32 group scales of float32 rows x [N, 576]."""
    n, d = x.shape
    groups = d // granularity
    xg = x.view(n, groups, granularity)
    amax = xg.abs().amax(dim=2)
    scale = (amax / FP8_MAX).to(torch.float32)
    scale = torch.where(scale > 0, scale, torch.ones_like(scale))
    y = (xg / scale[:, :, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).view(n, d)
    return codes, scale


def make_workload(batch, num_heads, cache_lengths, page_size, granularity, *, q_len=1,
                  num_layers=1, layer_idx=0, kv_dim=1, independent_scales=False,
                  spare_blocks=0, spare_scale_blocks=0, max_pages=None, seed=0,
                  softmax_scale=None, device="cpu", poison=True, unused_table_id=0,
                  chunk_tokens=1 << 20, name="", kv_dtype="fp8"):
    """Draw one workload.

    cache_lengths: list of per-request lengths (each >= q_len unless a test
    wants the degenerate case).  max_pages defaults to the longest request's
    page count.  With `poison`, every byte the decode must not read holds the
    NaN code 0x7F (NaN scales likewise); otherwise zeros.  unused_table_id is
    written into table columns past a request's pages (0xFFFFFFFF in poison
    tests: such a column must never be read).  kv_dtype "bf16" draws the
    unquantized cache: blocks hold the bf16 rows themselves, scales is None
    (granularity and independent_scales do not apply).
    """
    if kv_dtype not in ("fp8", "bf16"):
        raise ValueError("kv_dtype is 'fp8' or 'bf16'")
    unquantized = kv_dtype == "bf16"
    if unquantized:
        independent_scales = False
        granularity = HEAD_DIM
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    dgen = torch.Generator(device=device)
    dgen.manual_seed(int(seed) + 7919)
    lengths = [int(v) for v in cache_lengths]
    B = int(batch)
    P = int(page_size)
    pages_per = [(L + P - 1) // P for L in lengths]
    if max_pages is None:
        max_pages = max(1, max(pages_per))
    used = sum(pages_per)
    NB = used + int(spare_blocks)
    NBs = (used + int(spare_scale_blocks)) if independent_scales else NB
    NG = HEAD_DIM // granularity
    fill_code = NAN_CODE if poison else 0
    fill_scale = float("nan") if poison else 0.0

    # page ids: a random permutation of the pool, assigned in (request, page) order
    perm = torch.randperm(NB, generator=gen)
    lt = torch.full((B, max_pages), int(unused_table_id), dtype=torch.int64)
    slt = None
    sperm = torch.randperm(NBs, generator=gen) if independent_scales else None
    if independent_scales:
        slt = torch.full((B, max_pages), int(unused_table_id), dtype=torch.int64)
    k = 0
    for b in range(B):
        for c in range(pages_per[b]):
            lt[b, c] = int(perm[k])
            if independent_scales:
                slt[b, c] = int(sperm[k])
            k += 1

    if unquantized:
        blocks = torch.full((NB, kv_dim, num_layers, P, 1, HEAD_DIM), float("nan") if poison else 0.0,
                            dtype=torch.bfloat16, device=device)
        scales = None
    else:
        blocks = torch.full((NB, kv_dim, num_layers, P, 1, HEAD_DIM), fill_code, dtype=torch.uint8,
                            device=device)
        scales = torch.full((NBs, kv_dim, num_layers, P, 1, NG), fill_scale, dtype=torch.float32,
                            device=device)

    # latent rows of every valid token, drawn in chunks (large pools)
    tok_b = np.repeat(np.arange(B), lengths)
    tok_t = np.concatenate([np.arange(L) for L in lengths]) if lengths else np.zeros(0, np.int64)
    lt_np = lt.numpy()
    slt_np = slt.numpy() if slt is not None else lt_np
    total = len(tok_b)
    for s0 in range(0, total, chunk_tokens):
        s1 = min(total, s0 + chunk_tokens)
        n = s1 - s0
        rows = torch.randn((n, HEAD_DIM), generator=dgen, device=device, dtype=torch.float32)
        mag = torch.exp(0.5 * torch.randn((n, 1), generator=dgen, device=device, dtype=torch.float32))
        bb = tok_b[s0:s1]
        tt = tok_t[s0:s1]
        page = torch.as_tensor(lt_np[bb, tt // P], device=device)
        spage = torch.as_tensor(slt_np[bb, tt // P], device=device)
        slot = torch.as_tensor(tt % P, device=device)
        if unquantized:
            blocks[page, 0, layer_idx, slot, 0, :] = (rows * mag).to(torch.bfloat16)
        else:
            codes, sc = _quantize_rows(rows * mag, granularity)
            blocks[page, 0, layer_idx, slot, 0, :] = codes
            scales[spage, 0, layer_idx, slot, 0, :] = sc

    q = torch.randn((B, q_len, num_heads, HEAD_DIM), generator=dgen, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / math.sqrt(192.0)))
    return Workload(
        q=q, blocks=blocks, scales=scales,
        lookup_table=_u32_view(lt).to(device),
        scales_lookup_table=None if slt is None else _u32_view(slt).to(device),
        cache_lengths=_u32_view(torch.tensor(lengths, dtype=torch.int64)).to(device),
        layer_idx=int(layer_idx), q_len=int(q_len), softmax_scale=float(softmax_scale),
        page_size=P, granularity=int(granularity), name=name)


@dataclasses.dataclass
class RaggedWorkload(Workload):
    """A decode call whose requests have their own query counts: q is packed
    [T, H, 576], request b owning rows q_offsets[b] .. q_offsets[b + 1] - 1;
    q_len holds the largest count (the batch's max_prompt_length)."""

    q_offsets: torch.Tensor | None = None   # int32 [B + 1], from 0 to T

    @property
    def batch(self) -> int:
        return self.q_offsets.shape[0] - 1

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    def q_counts(self) -> list[int]:
        o = [int(v) for v in self.q_offsets.cpu().tolist()]
        return [o[b + 1] - o[b] for b in range(len(o) - 1)]

    def to(self, device) -> "RaggedWorkload":
        w = Workload.to(self, device)
        return dataclasses.replace(w, q_offsets=self.q_offsets.to(device))


def make_ragged_workload(q_counts, num_heads, cache_lengths, page_size, granularity, *, seed=0,
                         device="cpu", **kw):
    """The cache of make_workload (same recipe and keyword arguments) with
    per-request query counts q_counts (each >= 0, normally <= the request's
    cache length): q ~ bf16(N(0, 1)) packed [sum(q_counts), H, 576]."""
    counts = [int(c) for c in q_counts]
    if any(c < 0 for c in counts):
        raise ValueError("query counts are >= 0")
    w = make_workload(len(counts), num_heads, cache_lengths, page_size, granularity, q_len=1,
                      seed=seed, device=device, **kw)
    dgen = torch.Generator(device=device)
    dgen.manual_seed(int(seed) + 104729)
    q = torch.randn((sum(counts), num_heads, HEAD_DIM), generator=dgen, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=device)
    fields = {f.name: getattr(w, f.name) for f in dataclasses.fields(Workload)}
    fields.update(q=q, q_len=max(1, max(counts)))
    return RaggedWorkload(**fields, q_offsets=offs)


def _u32_view(t: torch.Tensor) -> torch.Tensor:
    """int64 ids in [0, 2^32) stored as int32 tensors holding the same 32 bits."""
    t = t.to(torch.int64)
    t = torch.where(t >= 2 ** 31, t - 2 ** 32, t)
    return t.to(torch.int32)


def u32_numpy(t: torch.Tensor) -> np.ndarray:
    """uint32 numpy copy of an int32 tensor holding uint32 bits."""
    return t.detach().cpu().numpy().view(np.uint32)


# ------------------------------------------------------------ named workloads
def tiny(seed=0, device="cpu", poison=True):
    """2 requests of 37 and 100 keys, 16 heads, page 16, per-token scales, 16 blocks."""
    return make_workload(2, 16, [37, 100], 16, HEAD_DIM, spare_blocks=6, seed=seed,
                         device=device, poison=poison, name="tiny")


def uniform(seed=1000, device="cpu", poison=False, batch=16, length=4096):
    """16 requests x 4096 keys, 128 heads, page 64, per-token scales."""
    return make_workload(batch, 128, [length] * batch, 64, HEAD_DIM, seed=seed, device=device,
                         poison=poison, name=f"uniform_b{batch}_l{length}")


def ragged(seed=2000, device="cpu", poison=False, batch=64, lmax=8192):
    """64 requests, lengths U[1, 8192], 128 heads, page 64, 64-wide scale groups, own scale table."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, lmax + 1, size=batch).tolist()
    return make_workload(batch, 128, lengths, 64, 64, independent_scales=True, spare_blocks=3,
                         spare_scale_blocks=11, max_pages=(lmax + 63) // 64, seed=seed,
                         device=device, poison=poison, name=f"ragged_b{batch}")


def long_context(seed=3000, device="cpu", poison=False, batch=1, length=131072):
    """batch x 131072 keys, 128 heads, page 128, per-token scales."""
    return make_workload(batch, 128, [length] * batch, 128, HEAD_DIM, seed=seed, device=device,
                         poison=poison, name=f"long_b{batch}")


def speculative(seed=4000, device="cpu", poison=False, batch=128, lmin=2048, lmax=32768):
    """batch x q_len 4 (causal), lengths U[2048, 32768], 128 heads, page 64,
    4 layers (layer 2 read), 64-wide scale groups, own scale table."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lmin, lmax + 1, size=batch).tolist()
    return make_workload(batch, 128, lengths, 64, 64, q_len=4, num_layers=4, layer_idx=2,
                         independent_scales=True, spare_blocks=5, spare_scale_blocks=9,
                         max_pages=(lmax + 63) // 64, seed=seed, device=device, poison=poison,
                         name=f"spec_b{batch}")


def query_chunk(seed=5000, device="cpu", poison=False, batch=8, q_len=16, length=4096):
    """batch x q_len 16 new tokens (causal) over 4096 cached keys, 128 heads, page 64,
    per-token scales: a chunked-prefill shape over the paged cache."""
    return make_workload(batch, 128, [length] * batch, 64, HEAD_DIM, q_len=q_len, seed=seed, device=device,
                         poison=poison, name=f"chunk_b{batch}_q{q_len}_l{length}")


def uniform_bf16(seed=6000, device="cpu", poison=False, batch=16, length=4096):
    """The uniform shape (16 requests x 4096 keys, 128 heads, page 64) over an
    unquantized bf16 cache."""
    return make_workload(batch, 128, [length] * batch, 64, HEAD_DIM, seed=seed, device=device,
                         poison=poison, kv_dtype="bf16", name=f"uniform_bf16_b{batch}_l{length}")
