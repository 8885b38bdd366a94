// Which work unit a decode workgroup runs (shared by the FP8 and the bf16
// decode kernels).  A unit is (request, row-group pair, key split), numbered
// request-major: unit = (request * num_splits + split) * pairs + pair.
#pragma once

#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mla {

typedef __attribute__((address_space(3))) int LdsInt;

// Workgroups are dispatched in blockIdx order and dealt round-robin to the 8
// XCDs (blockIdx % 8).  Returns the unit of this workgroup, or -1 when it has
// none.  Every thread of the workgroup (at least 4 waves) must call it: with
// a.lpt it synchronizes the workgroup and uses the first 3 KiB of `lds`.
__device__ __forceinline__ int workgroup_unit(const DecodeArgs& a, int rgp_count,
                                              __attribute__((address_space(3))) char* lds, int tid, int lane,
                                              int wave) {
  if (!a.lpt) {
    // request order: the units of one request (which read the same keys)
    // land on one XCD, back to back
    const int per_xcd = (a.grid_units + 7) >> 3;
    const int unit = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    return unit < a.grid_units ? unit : -1;
  }
  // More units than compute units: largest key ranges first (the
  // hardware's in-order dispatch then runs a greedy list schedule in
  // decreasing size, which keeps the last wave of workgroups short).  An
  // item is a (request, split) key range; its key count is T for the full
  // splits of a request, the remainder for its last split, 0 past it.
  // Items are ranked by (count desc, index asc): first every full split
  // in index order, then the requests' remainders by size (ties by
  // request; a request without keys has a remainder of 0 keys, so that its
  // zero output is written), then the empty items.  Every workgroup
  // computes the item at its own rank from the cache lengths: a prefix sum
  // of the full-split counts and a ranking of the <= kLptMaxBatch
  // remainders, in LDS.  Item
  // rank q goes to XCD q % 8, the ranks of an XCD in increasing order,
  // each item's row-group pairs back to back.
  LdsInt* const fpre = (LdsInt*)lds;                 // [B + 1] full splits before request b
  LdsInt* const tail = fpre + kLptMaxBatch + 1;      // [B] remainder keys of request b
  LdsInt* const tord = tail + kLptMaxBatch;          // [B] requests by remainder rank
  LdsInt* const wsum = tord + kLptMaxBatch;          // [4] per-wave totals of the scan
  const int T = a.tokens_per_split, S = a.num_splits, B = a.batch;
  const uint32_t cap = (uint32_t)a.max_pages * (uint32_t)a.page_size;
  // full splits (low 16 bits) and remainder flag (high 16 bits) of request tid,
  // scanned over the first four waves (B <= 256)
  // A request with no keys still writes its (zero) output: its split 0
  // counts as a remainder of 0 keys.  tail[b] = -1: no remainder.
  int fb = 0, tb = -1;
  if (tid < B) {
    const int len = (int)min(a.cache_lengths[tid], cap);
    fb = min(S, len / T);
    tb = (fb < S && (len > fb * T || len == 0)) ? len - fb * T : -1;
    tail[tid] = tb;
  }
  int v = fb | ((tb >= 0 ? 1 : 0) << 16);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63 && wave < 4) wsum[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave && w < 4; ++w) v += wsum[w];
  if (tid < B) fpre[tid + 1] = v & 0xffff;
  if (tid == 0) fpre[0] = 0;
  const int tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];     // (all four waves' totals)
  const int F = tot & 0xffff, NT = tot >> 16;
  if (tid < B && tb >= 0) {
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < B; ++j) {
      const int tj = tail[j];
      rank += (tj > tb || (tj == tb && j < tid)) ? 1 : 0;
    }
    tord[rank] = tid;
  }
  __syncthreads();
  const int jx = blockIdx.x >> 3;
  const int q = (jx / rgp_count) * 8 + (blockIdx.x & 7);     // item rank
  int item = -1;
  if (q < F) {
    int lo = 0, hi = B - 1;          // the request b with fpre[b] <= q < fpre[b + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (fpre[mid] <= q) lo = mid; else hi = mid - 1;
    }
    item = lo * S + (q - fpre[lo]);
  } else if (q < F + NT) {
    const int bt = tord[q - F];
    item = bt * S + (fpre[bt + 1] - fpre[bt]);
  }
  __syncthreads();                                  // (the LDS is reused below)
  return item < 0 ? -1 : item * rgp_count + jx % rgp_count;   // (-1: an empty key range)
}

// The queries of request b: the packed index of its first query and its
// query count (q_offsets, when given, holds the per-request counts as prefix
// offsets; otherwise every request has q_len queries).  Query i, head h of
// request b is row (first + i) * num_heads + h of q and of out.
struct RequestRows {
  int first, count;
};
__device__ __forceinline__ RequestRows request_rows(const DecodeArgs& a, int b) {
  if (a.q_offsets == nullptr) return RequestRows{b * a.q_len, a.q_len};
  const __attribute__((address_space(4))) uint32_t* const o = (const __attribute__((address_space(4))) uint32_t*)a.q_offsets;
  const uint32_t first = o[b], next = o[b + 1];
  return RequestRows{(int)first, (int)(next - first)};
}

// Grid of the decode kernels for a.
inline int decode_grid(const DecodeArgs& a) {
  // (largest-first order: 8 * ceil(items / 8) item ranks x row-group pairs per item)
  return a.lpt ? 8 * ((a.batch * a.num_splits + 7) / 8) * ((a.row_groups + 1) / 2) : 8 * ((a.grid_units + 7) / 8);
}

}  // namespace mla
