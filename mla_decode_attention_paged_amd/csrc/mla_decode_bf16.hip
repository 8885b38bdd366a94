// MLA decode over an unquantized (bf16) paged latent cache, for gfx950.
//
// The cache type may hold its latent rows without quantization ("quantization
// enabled" is a property of the cache type on the "KVCacheScalesMHAOperand"
// page); the rows then sit in the blocks tensor of
// "generic_get_paged_cache_with_scales" (section "Args") as bf16, with the
// same page lookup, cache lengths and query length as the FP8 cache, and no
// scales.
//
// Work decomposition and output format are those of the FP8 decode kernel:
// a workgroup owns a pair of 32-row groups (64 query rows) of one request and
// one key range; with several key ranges it writes fp32 partials (O / l and the
// log2-sum-exp) that the merge workgroups of the same launch combine
// (split_merge.h).
//
// Workgroup = 4 waves; wave w owns 16 query rows (rows 16 (w % 2) .. + 15 of
// row group w / 2) against all keys and all 512 value columns, so its softmax
// state never leaves the wave.  Per 32-key tile:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows read from LDS as the A
//     operand, q held in registers as the B operand), 36 MFMAs;
//   * online softmax in fp32, base 2, with a lazy reference maximum;
//   * O^T += V^T P^T on the same MFMA: V^T fragments come straight from the
//     bf16 tile through ds_read_b64_tr_b16, and P is split into a bf16 high
//     part and a bf16 remainder (two MFMAs per block), which keeps P to about
//     16 significant bits; 64 MFMAs.
// K and V^T fragments are read from LDS six MFMAs ahead of use, in an order
// pinned with sched_group_barrier.  Tiles stream global -> LDS by direct-to-LDS
// loads into a ring of four 36 KiB buffers, three tiles ahead; one workgroup
// barrier per tile.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "mla_internal.h"
#include "split_merge.h"
#include "unit_order.h"

namespace mla {
namespace bf16_path {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

constexpr float kNegInf = -__builtin_inff();
constexpr int kRowBytes = 2 * kHeadDim;          // 1152: one bf16 latent row
constexpr int kHalfBytes = 16 * kRowBytes;       // 18432: 16 keys
constexpr int kTileBytesU = 2 * kHalfBytes;      // 36864: one 32-key tile
constexpr int kBufs = 4;                         // LDS ring of tiles
constexpr int kAhead = kBufs - 1;                // tiles in flight ahead of the one in use
constexpr int kThreadsU = 256;
constexpr int kLdsBytes = kBufs * kTileBytesU;   // 147456
static_assert(split_merge::lds_bytes(kThreadsU / 64) <= kLdsBytes, "merge state fits in the LDS");
constexpr int kDepthChunks = kHeadDim / 32;      // 18 MFMA k-steps of 32
constexpr int kVBlocks = kVDim / 16;             // 32 output blocks of 16 columns
// Lazy reference maximum: the reference moves only when a score passes it by
// more than kLazyLog2 / c2, so unnormalised weights stay below 2^kLazyLog2.
constexpr float kLazyLog2 = 16.0f;
constexpr int kKAhead = 6;                       // K fragments in flight (depth chunks)
constexpr int kVAhead = 6;                       // V^T fragments in flight (column blocks)

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query row in
// the MFMA layouts below).  v_permlane16_swap / v_permlane32_swap with both
// operands equal to x hand every lane the values of its partner row / half.
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16 bytes per lane from base + voff + kOff into LDS at ldst + kOff + 16 * lane
// (global_load_lds_dwordx4 with a scalar base: the LDS address is M0 plus the
// instruction offset plus 16 * lane).  Hand-written so that the compiler does
// not insert vmcnt(0) waits for these loads before later LDS reads.
template <int kOff>
__device__ __forceinline__ void tile_dma16(const uint8_t* base, uint32_t voff, uint32_t ldst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3"
               :: "v"(voff), "s"(base), "s"(ldst), "n"(kOff) : "memory", "m0");
}

// LDS tile layout: two halves of 16 keys; in a half, 18 blocks of 1 KiB, block
// bk holding depth bytes [64 bk, 64 bk + 64) of the 16 keys; inside a block,
// 16-byte slot 4 k + (c ^ swz(k / 4)) holds bytes [16 c, 16 c + 16) of key k.
// swz (0, 2, 3, 1 for k / 4 = 0..3) is a permutation, which keeps the 16-key K
// reads (ds_read_b128) on distinct banks, and its bit 1 differs between any
// two groups of four keys that one half-wave of a V transpose read touches
// (groups 0 and 1, 2 and 3, 0 and 2, 1 and 3), which keeps those reads on
// distinct banks too.
__device__ __forceinline__ constexpr int swz(int j) { return (((j ^ (j >> 1)) & 1) << 1) | ((j >> 1) & 1); }

__global__ void __launch_bounds__(kThreadsU) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_bf16_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  LDS_AS char* const L0 = (LDS_AS char*)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4;           // 16-lane group
  const int n = lane & 15;

  // ---- merge workgroups (past the decode grid) combine the split partials
  if ((int)blockIdx.x >= a.dgrid) {
    split_merge::merge_workgroup<kThreadsU / 64>(a, (int)blockIdx.x - a.dgrid, (LDS_AS float*)lds);
    return;
  }

  // ---- unit: (request, row-group pair, key split), in the FP8 kernel's order
  const int rgp_count = (a.row_groups + 1) >> 1;
  const int unit = workgroup_unit(a, rgp_count, L0, tid, lane, wave);
  if (unit < 0) return;
  const int rgp = unit % rgp_count;
  const int bs = unit / rgp_count;
  const int split = bs % a.num_splits;
  const int b = bs / a.num_splits;

  const CONST_AS uint32_t* const lt = (const CONST_AS uint32_t*)a.lt;
  const int L = (int)min(((const CONST_AS uint32_t*)a.cache_lengths)[b],
                         (uint32_t)a.max_pages * (uint32_t)a.page_size);
  const int T = a.tokens_per_split;
  const int nsplit_eff = L <= 0 ? 1 : (L + T - 1) / T;
  if (split >= nsplit_eff) return;
  const RequestRows rq = request_rows(a, b);
  const int rows_total = rq.count * a.num_heads;   // this request's query rows (query-major)
  if (2 * rgp * kRows >= rows_total) return;   // the pair holds none of them
  const size_t row_base = (size_t)rq.first * a.num_heads;
  const int t_lo = split * T;
  const int t_hi = min(L, t_lo + T);
  const int ntiles = (t_hi - t_lo + 31) / 32;
  const float c2 = a.sm_log2;

  // ---- this lane's query row (row n of the wave's 16)
  const int rg = 2 * rgp + (wave >> 1);
  const int row_in_rg = 16 * (wave & 1) + n;
  const int my_row = rg * kRows + row_in_rg;
  const bool row_ok = rg < a.row_groups && my_row < rows_total;
  const int my_i = row_ok ? my_row / a.num_heads : 0;
  // keys visible to this row: j < L - Q + i + 1, clipped to the split
  const int lim = row_ok ? min(L - rq.count + my_i + 1, t_hi) : t_hi;

  // q as the B operand of S^T = K Q^T: lane (n, gq) holds depth 32 kc + 8 gq .. + 7 of its row
  bf16x8 qf[kDepthChunks];
  {
    const uint16_t* qrow = a.q + (row_base + (row_ok ? my_row : 0)) * kHeadDim + 8 * gq;
#pragma unroll
    for (int kc = 0; kc < kDepthChunks; ++kc) {
      const u32x4 v = row_ok ? *(const u32x4*)(qrow + 32 * kc) : u32x4{0, 0, 0, 0};
      qf[kc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- tile loads: wave w fills blocks 9 (w % 2) .. + 8 of half w / 2.  Lane s
  // fills slot s of a block: key s / 4, 16-byte column (s % 4) ^ swz(s / 16).
  // Keys at or past t_hi re-load the last valid key (finite data that the
  // softmax masks out), so nothing past a request's length is read.
  const uint8_t* layer_base = (const uint8_t*)a.blocks + a.layer_offset;
  const int ld_hb = wave >> 1;
  const int ld_bk0 = 9 * (wave & 1);
  const int ld_key = lane >> 2;
  const int ld_col = (lane & 3) ^ swz(lane >> 4);
  auto issue_tile = [&](int j) __attribute__((always_inline)) {
    const int t0 = t_lo + 32 * j;
    const int nvalid = min(32, t_hi - t0);
    const int src_half = nvalid > 16 ? ld_hb : 0;         // half whose page holds this wave's keys
    const int kk = min(16 * ld_hb + ld_key, nvalid - 1) - 16 * src_half;
    const uint32_t tb = (uint32_t)(t0 + 16 * src_half);    // a 16-key block never straddles a page
    const uint32_t P = (uint32_t)a.page_size;
    const uint32_t page = lt[(size_t)b * a.max_pages + tb / P];
    const uint8_t* base = layer_base + (uint64_t)page * (uint64_t)a.page_stride +
                          (uint64_t)(tb % P) * kRowBytes + 64 * ld_bk0;
    const uint32_t voff = (uint32_t)kk * kRowBytes + 16 * ld_col;
    const uint32_t dst = (uint32_t)(uintptr_t)(L0 + (j % kBufs) * kTileBytesU + ld_hb * kHalfBytes + 1024 * ld_bk0);
#define MLA_DMA(cb) tile_dma16<64 * (cb)>(base, voff, dst + (1024 - 64) * (cb))
    MLA_DMA(0); MLA_DMA(1); MLA_DMA(2); MLA_DMA(3); MLA_DMA(4);
    MLA_DMA(5); MLA_DMA(6); MLA_DMA(7); MLA_DMA(8);
#undef MLA_DMA
  };

  // K read (A operand, 16 keys x 32 depth): lane (n, gq) reads key n, 16-byte column gq
  const uint32_t kread = (uint32_t)(16 * (4 * n + (gq ^ swz(n >> 2))));
  // V^T read (A operand via transpose read): provider lane (k, h) = (n / 4, n % 4) of
  // group gq addresses key 4 gq + k, columns 16 nb + 4 h .. + 3; the result gives
  // lane (n, gq) column 16 nb + n of keys 4 gq .. 4 gq + 3.
  const int vk = n >> 2, vh = n & 3;
  const int vkey = 4 * gq + vk;
  uint32_t vread[2];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd)
    vread[odd] = (uint32_t)(64 * vkey + 16 * ((2 * odd + (vh >> 1)) ^ swz(gq)) + 8 * (vh & 1));

  f32x4 o[kVBlocks];
#pragma unroll
  for (int nb = 0; nb < kVBlocks; ++nb) o[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = kNegInf;     // reference maximum of the row (unscaled scores)
  float l_part = 0.0f;       // this lane's share of the row sum against m_ref

  // Tile 0 goes out, then the compiler's own wait for q is forced here, outside
  // the loop (its counter does not see the hand-written tile loads, so a wait
  // placed at the first use of q inside the loop would be a full vmcnt(0) on
  // every tile).  Tile 0 is needed first anyway; the next tiles follow.
  if (ntiles > 0) issue_tile(0);
#pragma unroll
  for (int kc = 0; kc < kDepthChunks; ++kc) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, qf[kc])));
#pragma unroll
  for (int j = 1; j < kAhead; ++j)
    if (j < ntiles) issue_tile(j);

  for (int j = 0; j < ntiles; ++j) {
    // tile j has landed: this wave's loads of it (the younger tiles' loads may
    // still be in flight), then everyone's
    const int younger = min(kAhead - 1, ntiles - 1 - j);
    if (younger >= 2) wait_vmcnt<18>();
    else if (younger == 1) wait_vmcnt<9>();
    else wait_vmcnt<0>();
    lds_barrier();
    // the buffer of tile j - 1 is free again
    if (j + kAhead < ntiles) issue_tile(j + kAhead);

    LDS_AS const char* tb = L0 + (j % kBufs) * kTileBytesU;
    // ---- S^T for keys 0..15 (sA) and 16..31 (sB) of the tile
    // (K fragments are read kKAhead depth chunks ahead of their MFMAs)
    f32x4 sA = {0.0f, 0.0f, 0.0f, 0.0f}, sB = {0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 ka[kKAhead], kb[kKAhead];
#pragma unroll
    for (int kc = 0; kc < kKAhead; ++kc) {
      ka[kc] = *(LDS_AS const bf16x8*)(tb + kread + 1024 * kc);
      kb[kc] = *(LDS_AS const bf16x8*)(tb + kHalfBytes + kread + 1024 * kc);
    }
#pragma unroll
    for (int kc = 0; kc < kDepthChunks; ++kc) {
      sA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kc % kKAhead], qf[kc], sA, 0, 0, 0);
      sB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kc % kKAhead], qf[kc], sB, 0, 0, 0);
      if (kc + kKAhead < kDepthChunks) {
        ka[kc % kKAhead] = *(LDS_AS const bf16x8*)(tb + kread + 1024 * (kc + kKAhead));
        kb[kc % kKAhead] = *(LDS_AS const bf16x8*)(tb + kHalfBytes + kread + 1024 * (kc + kKAhead));
      }
    }
    // keep that order (the scheduler would otherwise sink each read next to its MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kKAhead, 0);
#pragma unroll
    for (int kc = 0; kc < kDepthChunks; ++kc) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (kc + kKAhead < kDepthChunks) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // lane (n, gq): x[r] = score of key 4 gq + r (r < 4) or 16 + 4 gq + r - 4, row n
    const int t0 = t_lo + 32 * j;
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = (t0 + 4 * gq + r < lim) ? sA[r] : kNegInf;
      x[4 + r] = (t0 + 16 + 4 * gq + r < lim) ? sB[r] : kNegInf;
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, x[r]);
    mx = quad_max(mx);
    // lazy reference: move only when a score passes it by more than kLazyLog2 / c2
    const bool move = mx * c2 > m_ref * c2 + kLazyLog2;
    if (wave_any(move)) {
      const float m_new = move ? mx : m_ref;
      const float alpha = (move && m_ref != kNegInf) ? exp2_fast((m_ref - m_new) * c2) : 1.0f;
      if (wave_any(alpha != 1.0f)) {
#pragma unroll
        for (int nb = 0; nb < kVBlocks; ++nb) o[nb] *= alpha;
      }
      l_part *= alpha;
      m_ref = m_new;
    }
    const float mb = m_ref == kNegInf ? 0.0f : m_ref * c2;
    float p[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      p[r] = exp2_fast(__builtin_fmaf(x[r], c2, -mb));
      l_part += p[r];
    }
    // P^T (B operand): k-slot r of lane (n, gq) is the key of x[r]; P = hi + lo in bf16
    bf16x8 ph, pl;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const __bf16 h = (__bf16)p[r];
      ph[r] = h;
      pl[r] = (__bf16)(p[r] - (float)h);
    }
    // ---- O^T += V^T P^T, 16 columns per block (V^T fragments read kVAhead blocks ahead)
    auto read_v = [&](int nb) __attribute__((always_inline)) {
      const uint32_t off = 1024 * (nb >> 1) + vread[nb & 1];
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(tb + off));
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(tb + kHalfBytes + off));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 va[kVAhead];
#pragma unroll
    for (int nb = 0; nb < kVAhead; ++nb) va[nb] = read_v(nb);
    // blocks go in pairs so that the two MFMAs on one accumulator are not back to back
#pragma unroll
    for (int nb = 0; nb < kVBlocks; nb += 2) {
      const bf16x8 v0 = va[nb % kVAhead], v1 = va[(nb + 1) % kVAhead];
      if (nb + kVAhead < kVBlocks) {
        va[nb % kVAhead] = read_v(nb + kVAhead);
        va[(nb + 1) % kVAhead] = read_v(nb + 1 + kVAhead);
      }
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, ph, o[nb], 0, 0, 0);
      o[nb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, ph, o[nb + 1], 0, 0, 0);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pl, o[nb], 0, 0, 0);
      o[nb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, pl, o[nb + 1], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVAhead, 1);
#pragma unroll
    for (int nb = 0; nb < kVBlocks; nb += 2) {
      if (nb + kVAhead < kVBlocks) __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
    }
  }

  // ---- epilogue: lane (n, gq) holds O[row n][16 nb + 4 gq + r] in o[nb][r]
  const float l_row = quad_sum(l_part);
  const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
  if (!row_ok) {
    // no row here; the wave still counts in below
  } else if (nsplit_eff == 1) {
    uint16_t* orow = a.out + (row_base + my_row) * kVDim + 4 * gq;
#pragma unroll
    for (int nb = 0; nb < kVBlocks; ++nb) {
      u32x2 packed;
      packed[0] = f32_to_bf16_bits(o[nb][0] * inv) | (f32_to_bf16_bits(o[nb][1] * inv) << 16);
      packed[1] = f32_to_bf16_bits(o[nb][2] * inv) | (f32_to_bf16_bits(o[nb][3] * inv) << 16);
      *(u32x2*)(orow + 16 * nb) = packed;
    }
  } else {
    // device-scope stores that the merge workgroups read (split_merge.h)
    const size_t pidx = ((size_t)b * a.row_groups + rg) * a.num_splits + split;
    float* const po = a.ws_o + pidx * kRows * kVDim;
    const uint32_t off = 4 * (row_in_rg * kVDim + 4 * gq);
#pragma unroll
    for (int nb = 0; nb < kVBlocks; ++nb) split_merge::store_dev(po, off + 64 * nb, o[nb] * inv);
    if (gq == 0)
      split_merge::store_dev(a.ws_lse + pidx * kRows, 4 * row_in_rg,
                             l_row > 0.0f ? m_ref * c2 + __log2f(l_row) : kNegInf);
  }
  if (nsplit_eff > 1) split_merge::signal_partials(a, b, rgp, split, wave, lane);   // (each of the four waves)
}

}  // namespace bf16_path

// ---------------------------------------------------------------- host launcher
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream, hipEvent_t main_begin,
                              hipEvent_t main_end) {
  static bool attr_set = false;   // per process; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)bf16_path::mla_decode_bf16_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bf16_path::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipError_t e;
  const bool both = main_begin && main_end;
  if (main_begin && !both && (e = hipEventRecord(main_begin, stream)) != hipSuccess) return e;
  DecodeArgs args = a;
  const int grid = decode_grid(a) + plan_merge(args, decode_grid(a), bf16_path::kThreadsU / 64);
  if (both) {
    hipExtLaunchKernelGGL(bf16_path::mla_decode_bf16_kernel, dim3(grid), dim3(bf16_path::kThreadsU),
                          bf16_path::kLdsBytes, stream, main_begin, main_end, 0, args);
  } else {
    hipLaunchKernelGGL(bf16_path::mla_decode_bf16_kernel, dim3(grid), dim3(bf16_path::kThreadsU),
                       bf16_path::kLdsBytes, stream, args);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (main_end && !both && (e = hipEventRecord(main_end, stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
