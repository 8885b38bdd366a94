// Split-KV merge, fused into the decode launches (shared by the FP8 and the
// bf16 decode kernels).
//
// When a request's keys are split over several decode workgroups (the
// flash-decoding split of a long key range), each split s leaves an fp32
// partial per query row: O_s = (sum_j 2^(c2 x_j - lse_s) v_j) and lse_s =
// log2 sum_j 2^(c2 x_j), over its own keys j.  The row's output is then
// sum_s 2^(lse_s - lse) O_s with lse = log2 sum_s 2^(lse_s): the same softmax
// over all keys, regrouped.
//
// The merge runs in the same launch as the decode: the grid has the decode
// workgroups first (blockIdx < dgrid) and then the merge workgroups.  A merge
// workgroup owns (request, row group, a slice of the group's 32 rows x 512
// columns) and merges the request's split partials of that slice as they
// become ready, in whatever order the decode workgroups finish, so that most
// of the merge overlaps the last decode workgroups.  Waiting is safe because
// workgroups are dispatched in blockIdx order on each XCD: every decode
// workgroup of the XCD is resident or finished before a merge workgroup is
// placed there, and decode workgroups wait on nothing.  It is also bounded
// (kSpinLimit polls, far above any real wait), so the kernel always ends; a
// merge that gives up writes NaN rows rather than a silent wrong value.
//
// Completion words (workspace start, kFlagBytes): one ready word per
// (request, row-group pair, split), whose four bytes the four partial-writing
// waves of that split's decode workgroup set to 1; and one merge count per
// (request, row-group pair).  Wave 0 of a merge workgroup polls the ready
// words of its pair (one lane per split) and publishes them in LDS, where
// the other waves look.  The ready words are written once per call: polling
// words that other workgroups update atomically was measured to stall the
// decode workgroups still running (by up to 40 % of the launch).  The pair's
// last merge workgroup puts its words back to zero, so a workspace that
// starts zeroed stays usable, call after call, with no clearing pass
// (nothing to capture in a graph either).
//
// Visibility across XCDs (each XCD has its own L2, not coherent with the
// others): partials and ready bytes are written, and read, with device-scope
// (sc1) vector accesses, which write through to, and read from, the device's
// coherence point, as the AMDGPU memory model's agent-scope relaxed atomic
// stores and loads do on this family.  A decode wave waits for its partial
// stores to complete (vmcnt 0) before it sets its ready byte, and a merge
// wave issues a split's partial loads only after the split's ready word has
// been read complete.  This orders data and flags the way agent-scope
// release / acquire pairs would, without the whole-L2 writeback and
// invalidate such fences issue (measured: tens of microseconds per launch
// once every workgroup runs them).
#pragma once

#include <hip/hip_runtime.h>

#include "mla_internal.h"
#include "unit_order.h"

namespace mla {
namespace split_merge {

typedef float mf32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mu32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t mu32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t LdsU32;
typedef __attribute__((address_space(3))) float LdsF32;

constexpr int kColBlock = 64;                    // columns per wave block (two 32-column halves)
constexpr int kColBlocks = kVDim / kColBlock;    // 8
constexpr int kRowBlock = 8;                     // rows per wave block
constexpr int kWaveBlocks = (kRows / kRowBlock) * kColBlocks;   // 32 per row group
// Most wave blocks per merge workgroup.  Measured on 64 ragged requests (4
// splits, 256 row groups): 8 blocks 143.8 us, 16 blocks 138.8 us, 32 blocks
// 140.2 us per decode launch; on the bf16 cache's 16 x 4096 keys (4-wave
// workgroups) 4 / 8 / 16 blocks 54.5 / 52.4 / 51.9 us.
constexpr int kMaxChunkBlocks = 16;
constexpr int kSignalWaves = 4;                  // decode waves that write partials (per workgroup)
constexpr uint32_t kReadyAll = 0x01010101u;      // a split's ready word once all four have
constexpr uint32_t kSpinLimit = 1u << 19;        // polls before a merge gives up (about half a second)
constexpr int kStateFloats = 10;                 // M, W, acc[8] per lane
constexpr int kBatch = 8;                        // splits whose loads are in flight together
constexpr int kMaskWords = kMaxSplits / 32;      // LDS ready mask
constexpr int kScDevice = 16;                    // buffer cache-policy bits: sc1 (device scope)
constexpr int kRsrcWord3 = 0x00020000;           // buffer descriptor word 3 for gfx9 (raw byte addressing)
// word offsets in the completion area
constexpr size_t kReadyWord = (size_t)kSplitFlagPairs;  // after the merge counts
static_assert((kReadyWord + kSplitFlagEntries) * sizeof(uint32_t) <= kFlagBytes, "flags fit their region");

// Buffer resource over [base, base + 2 GiB); base must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kRsrcWord3);
}

// Device-scope (write-through) stores and device-scope loads; base
// wave-uniform, byte offsets per lane.
__device__ __forceinline__ void store_dev(float* base, uint32_t byte_off, mf32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(mu32x4, v), rsrc(base), byte_off, 0, kScDevice);
}
__device__ __forceinline__ void store_dev(float* base, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc(base), byte_off, 0, kScDevice);
}
__device__ __forceinline__ mf32x4 load_dev4(const float* base, uint32_t byte_off) {
  return __builtin_bit_cast(mf32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), byte_off, 0, kScDevice));
}
__device__ __forceinline__ float load_dev1(const float* base, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(base), byte_off, 0, kScDevice));
}

// LDS bytes a merge workgroup of `waves` waves uses: the give-up word (padded
// to 16 bytes), the ready mask, then the split groups' states.
constexpr int lds_bytes(int waves) { return 16 + 4 * kMaskWords + waves * kStateFloats * 64 * 4; }

__device__ __forceinline__ size_t pair_index(const DecodeArgs& a, int b, int pair) {
  return (size_t)b * ((a.row_groups + 1) >> 1) + pair;
}

// Splits of request b that hold keys (as the decode kernels count them).
__device__ __forceinline__ int splits_used(const DecodeArgs& a, int b) {
  const int L = (int)min(a.cache_lengths[b], (uint32_t)a.max_pages * (uint32_t)a.page_size);
  return L <= 0 ? 1 : (L + a.tokens_per_split - 1) / a.tokens_per_split;
}

// A decode wave has issued its last partial store (O rows and lse, all
// through store_dev): wait until they have completed, then set its byte
// (slot 0..3) of the split's ready word.  Called once by each of the
// kSignalWaves partial-writing waves of a decode workgroup whose request has
// more than one split.
__device__ __forceinline__ void signal_partials(const DecodeArgs& a, int b, int pair, int split, int slot,
                                                int lane) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0) {
    const size_t e = pair_index(a, b, pair) * a.num_splits + split;
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)1, rsrc(a.ws_flags + kReadyWord + e), slot, 0, kScDevice);
  }
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Merge workgroups that have rows to merge in (request, row-group pair), for a
// request of rows_total query rows.
__device__ __forceinline__ int merges_in_pair(const DecodeArgs& a, int pair, int nch, int rows_total) {
  int n = 0;
  for (int g = 2 * pair; g < min(2 * pair + 2, a.row_groups); ++g) {
    const int rows = min(kRows, rows_total - g * kRows);
    for (int c = 0; c < nch; ++c)      // chunk c holds wave blocks [c * nwb, c * nwb + nwb)
      n += (c * (kWaveBlocks / nch) / kColBlocks) * kRowBlock < rows ? 1 : 0;
  }
  return n;
}

// Wave 0's poll: read the ready words of all nse splits of the pair, publish
// them in the LDS mask; returns true once every split is ready (or the wait
// has given up: then `failed` is set and every bit too).
__device__ __forceinline__ bool poll_ready(const uint32_t* ready, int nse, LdsU32* mask, LdsU32* failed,
                                           uint32_t& polls, int lane) {
  bool all = true;
  for (int s0 = 0; s0 < nse; s0 += 64) {
    const bool mine = s0 + lane < nse;
    const uint32_t w = mine ? __builtin_amdgcn_raw_buffer_load_b32(rsrc(ready + s0), 4 * lane, 0, kScDevice) : kReadyAll;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(w == kReadyAll);
    if (lane == 0) __hip_atomic_store(mask + (s0 >> 5), (uint32_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (lane == 0 && s0 + 32 < nse)
      __hip_atomic_store(mask + (s0 >> 5) + 1, (uint32_t)(bits >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    all = all && bits == ~0ull;
  }
  if (!all && ++polls >= kSpinLimit) {
    if (lane == 0) __hip_atomic_store(failed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int k = lane; k < (nse + 31) / 32; k += 64)
      __hip_atomic_store(mask + k, ~0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    all = true;
  }
  return all;
}

// Merge workgroup `mblock` (blockIdx.x - dgrid) of a launch with kWaves
// waves per workgroup.  A wave block is 8 rows x 64 columns of a row group
// (32 of them per group, row-block major); a merge unit v = (request b, row
// group rg, chunk ch) holds nwb = a.merge_nwb consecutive wave blocks.  With
// fewer blocks than waves, the kWaves / nwb waves on one wave block split the
// request's key splits between them (interleaved), meeting in LDS at the
// end; with more, each wave merges nwb / kWaves blocks in turn.  Units are dealt to
// XCDs in contiguous ranges, as the decode units are.  In a wave, lane (r, c)
// owns row r of its block and columns [4c, 4c + 4) and [32 + 4c, 36 + 4c):
// each load of the wave reads 8 rows x 128 contiguous bytes.
template <int kWaves, int kBpw>
__device__ __forceinline__ void merge_chunk(const DecodeArgs& a, int mblock,
                                            __attribute__((address_space(3))) float* lds) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwb = a.merge_nwb;                   // wave blocks per workgroup
  const int sgp = nwb < kWaves ? kWaves / nwb : 1;   // split groups (waves per block)
  constexpr int bpw = kBpw;                      // blocks per wave (nwb / kWaves when > 1)
  const int nch = kWaveBlocks / nwb;             // chunks per row group
  const int units = a.batch * a.row_groups * nch;
  const int per_x = (units + 7) >> 3;
  const int v = (mblock & 7) * per_x + (mblock >> 3);
  if (v >= units) return;                        // (the whole workgroup)
  const int ch = v % nch;
  const int rg = (v / nch) % a.row_groups;
  const int b = (v / nch) / a.row_groups;
  const RequestRows rq = request_rows(a, b);
  const int rows_total = rq.count * a.num_heads; // this request's query rows
  if (rg * kRows + ((ch * nwb) / kColBlocks) * kRowBlock >= rows_total) return;   // no rows (not counted)
  const int nse = splits_used(a, b);
  if (nse <= 1) return;                          // the decode wrote this request's rows itself

  LdsU32* const failed = (LdsU32*)lds;
  LdsU32* const mask = failed + 4;
  LdsF32* const st = (LdsF32*)(mask + kMaskWords);
  for (int k = tid; k < (nse + 31) / 32; k += kWaves * 64) mask[k] = 0u;
  if (tid == 0) *failed = 0u;
  __syncthreads();

  const size_t p = pair_index(a, b, rg >> 1);
  const uint32_t* const ready = a.ws_flags + kReadyWord + p * a.num_splits;
  const int sgi = nwb < kWaves ? wave / nwb : 0;
  const int nj = sgi < nse ? (nse - sgi + sgp - 1) / sgp : 0;   // this wave's splits: sgi + j sgp
  const size_t pbase = ((size_t)b * a.row_groups + rg) * a.num_splits;
  const float kNegInf = -__builtin_inff();
  bool all_ready = wave != 0;                    // wave 0 polls until every split is ready
  uint32_t polls = 0;
  for (int k = 0; k < bpw; ++k) {               // each block of this wave
    const int wb = ch * nwb + (nwb < kWaves ? wave % nwb : wave + k * kWaves);   // this wave's block
    const int rb = wb / kColBlocks, cb = wb % kColBlocks;
    const int rl = rb * kRowBlock + (lane >> 3);   // row within the group
    const int col0 = cb * kColBlock + 4 * (lane & 7);
    const uint32_t o_off = 4 * (rl * kVDim + col0);
    float M = kNegInf, W = 0.0f;
    mf32x4 acc0 = mf32x4{0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
    // One split at a time, in index order, with the same arithmetic whatever
    // the order in which the splits became ready (so the result does not
    // depend on timing): window of kBatch of this wave's splits, the loads of
    // every ready split of the window issued at once, consumed in order.
    auto fold = [&](float l, mf32x4 x0, mf32x4 x1) __attribute__((always_inline)) {
      if (l > M) {
        const float rs = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - l);
        W *= rs;
        acc0 *= rs;
        acc1 *= rs;
        M = l;
      }
      if (l != kNegInf) {
        const float w = __builtin_amdgcn_exp2f(l - M);
        W += w;
        acc0 += w * x0;
        acc1 += w * x1;
      }
    };
    for (int w0 = 0; w0 < nj; w0 += kBatch) {
      const int nvalid = min(kBatch, nj - w0);
      uint32_t issued = 0;
      int consumed = 0;
      float ls[kBatch];
      mf32x4 o0[kBatch], o1[kBatch];
      while (consumed < nvalid) {
        if (!all_ready) all_ready = poll_ready(ready, nse, mask, failed, polls, lane);
        // ready bits of the window (lane u < nvalid looks up split sgi + (w0 + u) sgp)
        const int sk = sgi + (w0 + lane) * sgp;
        const bool rk = lane < nvalid &&
                        ((__hip_atomic_load(mask + (sk >> 5), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >>
                          (sk & 31)) & 1u);
        const uint32_t fresh = (uint32_t)__builtin_amdgcn_ballot_w64(rk) & ~issued;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if ((fresh >> u) & 1u) {
            const int s = sgi + (w0 + u) * sgp;
            ls[u] = load_dev1(a.ws_lse + (pbase + s) * kRows, 4 * rl);
            const float* const ob = a.ws_o + (pbase + s) * kRows * kVDim;
            o0[u] = load_dev4(ob, o_off);
            o1[u] = load_dev4(ob, o_off + 128);
          }
        }
        issued |= fresh;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (u == consumed && ((issued >> u) & 1u)) {
            fold(ls[u], o0[u], o1[u]);
            ++consumed;
          }
        }
        if (consumed < nvalid && !((issued >> consumed) & 1u)) __builtin_amdgcn_s_sleep(2);
      }
    }
    while (!all_ready) {                           // wave 0: keep publishing for the other waves
      all_ready = poll_ready(ready, nse, mask, failed, polls, lane);
      if (!all_ready) __builtin_amdgcn_s_sleep(2);
    }

    // every wave is past its waits; groups 1.. hand their states to group 0
    if (sgp > 1 && sgi != 0) {
      st[(wave * kStateFloats + 0) * 64 + lane] = M;
      st[(wave * kStateFloats + 1) * 64 + lane] = W;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st[(wave * kStateFloats + 2 + e) * 64 + lane] = acc0[e];
        st[(wave * kStateFloats + 6 + e) * 64 + lane] = acc1[e];
      }
    }
    __syncthreads();
    const bool gave_up = *failed != 0u;
    if (sgi == 0) {
      for (int j = 1; j < sgp; ++j) {
        const int wo = wave + j * nwb;
        const float Mo = st[(wo * kStateFloats + 0) * 64 + lane];
        const float Wo = st[(wo * kStateFloats + 1) * 64 + lane];
        const float Mn = fmaxf(M, Mo);
        const float r0 = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
        const float r1 = Mo == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(Mo - Mn);
        W = W * r0 + Wo * r1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc0[e] = acc0[e] * r0 + st[(wo * kStateFloats + 2 + e) * 64 + lane] * r1;
          acc1[e] = acc1[e] * r0 + st[(wo * kStateFloats + 6 + e) * 64 + lane] * r1;
        }
        M = Mn;
      }
      const int row = rg * kRows + rl;
      if (row < rows_total) {
        const float inv = W > 0.0f ? 1.0f / W : 0.0f;
        mu32x2 lo, hi;
        if (gave_up) {
          lo = hi = mu32x2{0x7fc07fc0u, 0x7fc07fc0u};
        } else {
          lo[0] = (uint32_t)bf16_rne(acc0[0] * inv) | ((uint32_t)bf16_rne(acc0[1] * inv) << 16);
          lo[1] = (uint32_t)bf16_rne(acc0[2] * inv) | ((uint32_t)bf16_rne(acc0[3] * inv) << 16);
          hi[0] = (uint32_t)bf16_rne(acc1[0] * inv) | ((uint32_t)bf16_rne(acc1[1] * inv) << 16);
          hi[1] = (uint32_t)bf16_rne(acc1[2] * inv) | ((uint32_t)bf16_rne(acc1[3] * inv) << 16);
        }
        uint16_t* const orow = a.out + ((size_t)rq.first * a.num_heads + row) * kVDim + col0;
        *(mu32x2*)orow = lo;
        *(mu32x2*)(orow + 32) = hi;
      }
    }
  }
  // Wave 0 counts this workgroup out (every wave of it is past its waits);
  // the pair's last merge workgroup clears the pair's words for the next call.
  if (wave == 0) {
    uint32_t last = 0u;
    if (lane == 0)
      last = __hip_atomic_fetch_add(a.ws_flags + p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (uint32_t)merges_in_pair(a, rg >> 1, nch, rows_total) - 1u ? 1u : 0u;
    if (__builtin_amdgcn_readfirstlane(last)) {
      for (int s = lane; s < nse; s += 64) __builtin_amdgcn_raw_buffer_store_b32(0u, rsrc(ready), 4 * s, 0, kScDevice);
      if (lane == 0) __hip_atomic_store(a.ws_flags + p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The merge workgroup: chunks of more blocks than waves take the
// multi-block form (blocks per wave fixed at compile time, so that the
// decode path that shares the kernel keeps its register allocation).
template <int kWaves>
__device__ __forceinline__ void merge_workgroup(const DecodeArgs& a, int mblock,
                                                __attribute__((address_space(3))) float* lds) {
  static_assert(kMaxChunkBlocks % kWaves == 0 && kMaxChunkBlocks / kWaves <= 4, "chunks of 1, 2 or 4 blocks per wave");
  const int bpw = a.merge_nwb / kWaves;          // (merge_nwb: a power of two, at most kMaxChunkBlocks)
  if constexpr (kMaxChunkBlocks / kWaves >= 4) {
    if (bpw == 4) {
      merge_chunk<kWaves, 4>(a, mblock, lds);
      return;
    }
  }
  if constexpr (kMaxChunkBlocks / kWaves >= 2) {
    if (bpw == 2) {
      merge_chunk<kWaves, 2>(a, mblock, lds);
      return;
    }
  }
  merge_chunk<kWaves, 1>(a, mblock, lds);
}

}  // namespace split_merge
}  // namespace mla
