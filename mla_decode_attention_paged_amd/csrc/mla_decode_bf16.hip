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
// Workgroup = 8 waves, two per SIMD, in two roles, so that one wave's MFMAs
// run while the other of its SIMD does VALU work or waits on the LDS.  A step
// is one 32-key tile.
//   * score waves (w = 0..3; row group r = w / 2 of the pair, key half
//     h = w % 2): S^T = K Q^T for the 16 keys of half h and the 32 rows of
//     group r over the whole 576-deep product, on v_mfma_f32_16x16x32_bf16
//     (K read from LDS as the A operand, q held in registers as the B
//     operand), 36 MFMAs; then the online softmax (fp32, base 2, lazy
//     reference maximum that follows the other half's wave) and P as two bf16
//     numbers, hi = bf16(p) and lo = bf16(p - hi) (about 16 significant bits),
//     handed to the value waves through LDS in their operand order;
//   * value waves (w = 4..7; output columns [128 c, 128 c + 128),
//     c = w - 4): O^T += V^T P^T for the previous step's tile and all 64
//     rows, on the same MFMA, with V^T fragments straight from the bf16 tile
//     through ds_read_b64_tr_b16 and the hi and lo parts of P in two MFMAs
//     per block, 64 MFMAs; they read the V^T fragments of the tile being
//     scored between those MFMAs (so the next step starts on them at once),
//     and they stream the tiles in.
// Tiles go from HBM into LDS by direct-to-LDS loads, two steps ahead, in a
// ring of three tile buffers: a tile's buffer is read only in the step that
// scores it (K by the score waves, V^T into the value waves' registers), so
// the buffer of tile i - 1 takes tile i + 2.  One workgroup barrier per step
// orders the hand-offs.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "mla_internal.h"
#include "split_merge.h"
#include "unit_order.h"

namespace mla {
namespace bf16_path {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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
constexpr int kSlots = 3;                        // tile buffers: two in flight, one being scored
constexpr int kThreadsU = 512;
constexpr int kDepthChunks = kHeadDim / 32;      // 18 MFMA k-steps of 32
constexpr int kColBlocks = 8;                    // 16-column blocks of a value wave (128 columns)
constexpr int kEpStride = 128 + 4;               // floats per row of a value wave's epilogue slice
// LDS: the tile ring, then P^T per tile parity ([row block 0..3][hi, lo][64
// lanes][16 B]), then the references per tile parity and key half ([2][2][64
// rows]), then the score waves' final row statistics ([key half][64 rows] m,
// then l).
constexpr int kPBytes = 4 * 2 * 64 * 16;         // 8192
constexpr int kPOff = kSlots * kTileBytesU;      // 110592
constexpr int kAlphaOff = kPOff + 2 * kPBytes;   // 126976
constexpr int kStatsOff = kAlphaOff + 2 * 2 * 64 * 4;
constexpr int kLdsBytes = kStatsOff + 2 * 2 * 64 * 4;   // 129024
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(4 * kRows * kEpStride * 4 <= kSlots * kTileBytesU, "epilogue slices fit in the tile ring");
static_assert(split_merge::lds_bytes(kThreadsU / 64) <= kLdsBytes, "merge state fits in the LDS");
// Lazy reference maximum: the reference moves only when a score passes it by
// more than kLazyLog2 / c2, so unnormalised weights stay below 2^kLazyLog2.
constexpr float kLazyLog2 = 16.0f;
constexpr int kKAhead = 6;                       // K fragments in flight (depth chunks)


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

__global__ void __attribute__((amdgpu_flat_work_group_size(kThreadsU, kThreadsU), amdgpu_waves_per_eu(2, 2)))
mla_decode_bf16_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  LDS_AS char* const L0 = (LDS_AS char*)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool is_score = wave < 4;
  const int sub = wave & 3;
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

  auto tile_buf = [&](int j) __attribute__((always_inline)) { return L0 + (j % kSlots) * kTileBytesU; };
  auto p_buf = [&](int j) __attribute__((always_inline)) { return L0 + kPOff + (j & 1) * kPBytes; };
  // reference maxima of tile j's key half hh, one per row of the pair (64)
  auto alpha_buf = [&](int j, int hh) __attribute__((always_inline)) {
    return (LDS_AS float*)(L0 + kAlphaOff) + ((j & 1) * 2 + hh) * 64;
  };
  LDS_AS float* const stat_m = (LDS_AS float*)(L0 + kStatsOff);   // [key half][64 rows]
  LDS_AS float* const stat_l = stat_m + 2 * 64;

  // ---- tile loads: wave sub fills blocks 9 (sub % 2) .. + 8 of half sub / 2.
  // Lane s fills slot s of a block: key s / 4, 16-byte column (s % 4) ^
  // swz(s / 16).  Keys at or past t_hi re-load the last valid key (finite data
  // that the softmax masks out), so nothing past a request's length is read.
  const uint8_t* layer_base = (const uint8_t*)a.blocks + a.layer_offset;
  const int ld_hb = sub >> 1;
  const int ld_bk0 = 9 * (sub & 1);
  const int ld_key = lane >> 2;
  const int ld_col = (lane & 3) ^ swz(lane >> 4);
  // Row offsets of the key range's 16-key blocks (a block never straddles a
  // page: pages hold a multiple of 16 keys), 64 blocks (32 tiles) at a time:
  // lane k holds the byte offset of block 64 m + k's first row from the
  // layer's start, so that a tile's address comes from v_readlane rather than
  // from a table read on the step's path.  The page ids of window m + 1 are
  // fetched while window m is in use.
  const int nblk = (t_hi - t_lo + 15) >> 4;
  const uint32_t* ltr = a.lt + (size_t)b * a.max_pages;
  uint32_t nxt_page = 0;
  uint64_t w_off = 0;
  int cur_win = -1;
  auto fetch_window = [&](int m) __attribute__((always_inline)) {
    const int blk = 64 * m + lane;
    if (blk < nblk) nxt_page = ltr[(uint32_t)(t_lo + 16 * blk) / (uint32_t)a.page_size];
  };
  auto enter_window = [&](int m) __attribute__((always_inline)) {
    const uint32_t slot = (uint32_t)(t_lo + 16 * (64 * m + lane)) % (uint32_t)a.page_size;
    w_off = (uint64_t)nxt_page * (uint64_t)a.page_stride + (uint64_t)slot * kRowBytes;
    cur_win = m;
    if (64 * (m + 1) < nblk) fetch_window(m + 1);
  };
  auto issue_tile = [&](int j) __attribute__((always_inline)) {
    const int t0 = t_lo + 32 * j;
    const int nvalid = min(32, t_hi - t0);
    const int src_half = nvalid > 16 ? ld_hb : 0;         // half whose page holds this wave's keys
    const int kk = min(16 * ld_hb + ld_key, nvalid - 1) - 16 * src_half;
    if ((j >> 5) != cur_win) enter_window(j >> 5);
    const int k = ((2 * j) & 63) + src_half;               // the block's lane in the window
    const uint64_t row_off = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(w_off >> 32), k) << 32) |
                             __builtin_amdgcn_readlane((uint32_t)w_off, k);
    const uint8_t* base = layer_base + row_off + 64 * ld_bk0;
    const uint32_t voff = (uint32_t)kk * kRowBytes + 16 * ld_col;
    const uint32_t dst = (uint32_t)(uintptr_t)(tile_buf(j) + ld_hb * kHalfBytes + 1024 * ld_bk0);
#define MLA_DMA(cb) tile_dma16<64 * (cb)>(base, voff, dst + (1024 - 64) * (cb))
    MLA_DMA(0); MLA_DMA(1); MLA_DMA(2); MLA_DMA(3); MLA_DMA(4);
    MLA_DMA(5); MLA_DMA(6); MLA_DMA(7); MLA_DMA(8);
#undef MLA_DMA
  };

  // ================================================================ score waves
  if (is_score) {
    const int r = sub >> 1;          // row group of the pair
    const int h = sub & 1;           // key half of every tile
    const int rg = 2 * rgp + r;
    // this lane's rows: row 16 rb + n of the group (rb = 0, 1)
    int lim[2];
    int lim_min = 0x7fffffff;
    bf16x8 qf[2][kDepthChunks];      // q as the B operand: lane (n, gq) holds depth 32 kc + 8 gq .. + 7
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = rg * kRows + 16 * rb + n;
      const bool ok = rg < a.row_groups && row < rows_total;
      // keys visible to this row: j < L - Q + i + 1, clipped to the split
      lim[rb] = ok ? min(L - rq.count + row / a.num_heads + 1, t_hi) : t_hi;
      lim_min = min(lim_min, lim[rb]);
      const uint16_t* qrow = a.q + (row_base + (ok ? row : 0)) * kHeadDim + 8 * gq;
#pragma unroll
      for (int kc = 0; kc < kDepthChunks; ++kc) {
        const u32x4 v = ok ? *(const u32x4*)(qrow + 32 * kc) : u32x4{0, 0, 0, 0};
        qf[rb][kc] = __builtin_bit_cast(bf16x8, v);
      }
    }
    for (int off = 32; off >= 1; off >>= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off));
    lim_min = __builtin_amdgcn_readfirstlane(lim_min);
    // K read (A operand, 16 keys x 32 depth): lane (n, gq) reads key n, 16-byte column gq
    const uint32_t kread = (uint32_t)(h * kHalfBytes + 16 * (4 * n + (gq ^ swz(n >> 2))));
    const float thr = kLazyLog2 / c2;
    float m_run[2] = {kNegInf, kNegInf};   // reference maximum per row (unscaled scores)
    float l_part[2] = {0.0f, 0.0f};        // this lane's share of the row sum against m_run
    __syncthreads();             // tile 0 has landed (the value waves waited for their loads)

    for (int i = 0; i <= ntiles; ++i) {
      if (i < ntiles) {
        LDS_AS const char* tb = tile_buf(i);
        // the other half's reference after the previous tile (read first: its
        // latency hides under the MFMAs)
        float mo_other[2] = {kNegInf, kNegInf};
        if (i > 0) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) mo_other[rb] = alpha_buf(i - 1, h ^ 1)[32 * r + 16 * rb + n];
        }
        // ---- S^T for the 16 keys of half h and row blocks 0, 1 (K fragments
        // read kKAhead depth chunks ahead of their MFMAs)
        f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
        bf16x8 kf[kKAhead];
#pragma unroll
        for (int kc = 0; kc < kKAhead; ++kc) kf[kc] = *(LDS_AS const bf16x8*)(tb + kread + 1024 * kc);
#pragma unroll
        for (int kc = 0; kc < kDepthChunks; ++kc) {
          const bf16x8 k = kf[kc % kKAhead];
          if (kc + kKAhead < kDepthChunks)
            kf[kc % kKAhead] = *(LDS_AS const bf16x8*)(tb + kread + 1024 * (kc + kKAhead));
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, qf[0][kc], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, qf[1][kc], s1, 0, 0, 0);
        }
        // keep that order (the scheduler would otherwise sink each read next to its MFMA)
        __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
        for (int kc = 0; kc < kDepthChunks; ++kc) {
          if (kc + kKAhead < kDepthChunks) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        // lane (n, gq): x[rb][e] = score of key 4 gq + e of the half, row 16 rb + n
        const int t0 = t_lo + 32 * i + 16 * h;
        float x[2][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[0][e] = s0[e];
          x[1][e] = s1[e];
        }
        if (t0 + 16 > lim_min) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[rb][e] = (t0 + 4 * gq + e < lim[rb]) ? x[rb][e] : kNegInf;
        }
        // The reference moves up to the other half's wave's (as it stood
        // after the previous tile), and lazily to this half's maximum, only
        // when a score here passes the reference by more than thr (then every
        // row of the wave moves to its own maximum).
        float mt[2], mref[2];
        bool pass = false;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          mt[rb] = quad_max(fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3])));
          mref[rb] = fmaxf(m_run[rb], mo_other[rb]);
          pass = pass || mt[rb] > mref[rb] + thr;
        }
        const bool move = wave_any(pass);
        LDS_AS float* const ab = alpha_buf(i, h) + 32 * r;
        float p[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          if (move) mref[rb] = fmaxf(mref[rb], mt[rb]);
          if (wave_any(mref[rb] != m_run[rb])) {
            l_part[rb] *= m_run[rb] == kNegInf ? 0.0f : exp2_fast((m_run[rb] - mref[rb]) * c2);
            m_run[rb] = mref[rb];
          }
          if (gq == 0) ab[16 * rb + n] = m_run[rb];
          const float nm = m_run[rb] == kNegInf ? 0.0f : -m_run[rb] * c2;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[rb][e] = exp2_fast(__builtin_fmaf(x[rb][e], c2, nm));
            l_part[rb] += p[rb][e];
          }
        }
        // P^T as the value waves' B operand: lane (n, gq) of row block 2 r + rb
        // holds row n's keys 4 gq .. + 3 of half 0 in bytes 0-7 and of half 1
        // in bytes 8-15, for the hi and the lo part
        LDS_AS char* const pb = p_buf(i) + 8 * h + 16 * lane;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          bf16x4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hi[e] = (__bf16)p[rb][e];
            lo[e] = (__bf16)(p[rb][e] - (float)hi[e]);
          }
          *(LDS_AS bf16x4*)(pb + ((2 * r + rb) * 2 + 0) * 1024) = hi;
          *(LDS_AS bf16x4*)(pb + ((2 * r + rb) * 2 + 1) * 1024) = lo;
        }
      }
      lds_barrier();             // end of step: P^T and references of tile i are out
    }
    // the rows' final references and sums (against them) for the epilogue
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float l_row = quad_sum(l_part[rb]);
      if (gq == 0) {
        stat_m[h * 64 + 32 * r + 16 * rb + n] = m_run[rb];
        stat_l[h * 64 + 32 * r + 16 * rb + n] = l_row;
      }
    }
    __syncthreads();
    return;
  }

  // ================================================================ value waves
  // They carry the step's critical path (tile loads, reads, 64 MFMAs); a
  // higher issue priority than the score wave of their SIMD shortens it.
  __builtin_amdgcn_s_setprio(1);
  // V^T read (A operand via transpose read): provider lane (k, hq) = (n / 4,
  // n % 4) of group gq addresses key 4 gq + k, columns 16 nb + 4 hq .. + 3; the
  // result gives lane (n, gq) column 16 nb + n of keys 4 gq .. 4 gq + 3.
  const int vk = n >> 2, vh = n & 3;
  const int vkey = 4 * gq + vk;
  uint32_t vread[2];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd)
    vread[odd] = (uint32_t)(64 * vkey + 16 * ((2 * odd + (vh >> 1)) ^ swz(gq)) + 8 * (vh & 1));
  auto read_v = [&](LDS_AS const char* tb, int nb) __attribute__((always_inline)) {
    const uint32_t off = 1024 * (nb >> 1) + vread[nb & 1];
    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(tb + off));
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(tb + kHalfBytes + off));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // O^T blocks: lane (n, gq) holds O[row 16 rb + n][128 sub + 16 nl + 4 gq + e]
  // in o[nl][rb][e], against the reference mo[rb] of its row.
  f32x4 o[kColBlocks][4];
#pragma unroll
  for (int nl = 0; nl < kColBlocks; ++nl)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) o[nl][rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float mo[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  bf16x8 vt[kColBlocks];             // V^T fragments of the tile the next MFMAs use

  if (ntiles > 0) {
    fetch_window(0);
    issue_tile(0);
    if (ntiles > 1) issue_tile(1);
  }
  if (ntiles > 1) wait_vmcnt<9>();   // tile 0 has landed (tile 1 may still be in flight)
  else wait_vmcnt<0>();
  __syncthreads();               // (the score waves loaded q)

  for (int i = 0; i <= ntiles; ++i) {
    if (i + 2 < ntiles) issue_tile(i + 2);   // into the buffer of tile i - 1, read last step
    if (i >= 1) {
      const int j = i - 1;
      LDS_AS const char* pb = p_buf(j) + 16 * lane;
      LDS_AS const float* a0 = alpha_buf(j, 0);
      LDS_AS const float* a1 = alpha_buf(j, 1);
      float ma[2][4];
      bf16x8 ph[4], pl[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        ma[0][rb] = a0[16 * rb + n];
        ma[1][rb] = a1[16 * rb + n];
        ph[rb] = *(LDS_AS const bf16x8*)(pb + (2 * rb + 0) * 1024);
        pl[rb] = *(LDS_AS const bf16x8*)(pb + (2 * rb + 1) * 1024);
      }
      // Bring O and both halves of the tile to one reference per row,
      // max(O's, half 0's, half 1's).  O is rescaled only when a reference
      // moved past O's (rare: references move lazily and follow each other);
      // a half whose reference is below the new one has its P scaled (hi and
      // lo recombined, scaled, split again).
      // (nothing to do unless a reference differs from O's: the common case)
      bool moved = false;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) moved = moved || ma[0][rb] != mo[rb] || ma[1][rb] != mo[rb];
      if (wave_any(moved)) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const float m_new = fmaxf(mo[rb], fmaxf(ma[0][rb], ma[1][rb]));
          if (wave_any(m_new != mo[rb] && mo[rb] != kNegInf)) {
            const float al = mo[rb] == kNegInf ? 0.0f : exp2_fast((mo[rb] - m_new) * c2);
#pragma unroll
            for (int nl = 0; nl < kColBlocks; ++nl) o[nl][rb] *= al;
          }
          mo[rb] = m_new;
          const float f0 = ma[0][rb] == kNegInf ? 0.0f : exp2_fast((ma[0][rb] - m_new) * c2);
          const float f1 = ma[1][rb] == kNegInf ? 0.0f : exp2_fast((ma[1][rb] - m_new) * c2);
          if (wave_any(f0 != 1.0f || f1 != 1.0f)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pv = ((float)ph[rb][e] + (float)pl[rb][e]) * (e < 4 ? f0 : f1);
              ph[rb][e] = (__bf16)pv;
              pl[rb][e] = (__bf16)(pv - (float)ph[rb][e]);
            }
          }
        }
      }
      // O^T += V^T P^T, hi and lo parts; the four row blocks between two
      // MFMAs on one accumulator.  Each V^T fragment, once used, is replaced
      // by the same fragment of tile i (in LDS since this step began), so
      // that the next step's MFMAs start without a read round trip.
      const bool pre = i < ntiles;
      LDS_AS const char* tn = tile_buf(i);
#pragma unroll
      for (int nl = 0; nl < kColBlocks; ++nl) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) o[nl][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[nl], ph[rb], o[nl][rb], 0, 0, 0);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) o[nl][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[nl], pl[rb], o[nl][rb], 0, 0, 0);
        if (pre) vt[nl] = read_v(tn, 8 * sub + nl);
      }
    } else if (ntiles > 0) {
#pragma unroll
      for (int nl = 0; nl < kColBlocks; ++nl) vt[nl] = read_v(tile_buf(0), 8 * sub + nl);
    }
    // this wave's loads of tile i + 1 have landed (those of tile i + 2 may be in flight)
    if (i + 2 < ntiles) wait_vmcnt<9>();
    else if (i + 1 < ntiles) wait_vmcnt<0>();
    lds_barrier();
  }

  // ---- epilogue: the rows' sums against O's references, then O / l.  Each
  // row group's 32 rows x 128 columns go through this wave's own LDS slice
  // (the tile ring is free now), so that every store covers two rows x 128
  // contiguous columns.
  __syncthreads();               // (the score waves' row statistics)
  LDS_AS float* const stage = (LDS_AS float*)(L0 + sub * (kRows * kEpStride * 4));   // [32][kEpStride]
  const int er = lane >> 5, ec = 4 * (lane & 31);   // read-back: rows 2k + er, columns ec .. ec + 3
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rg = 2 * rgp + p;
    if (rg >= a.row_groups) break;           // the pair's second group does not exist
    float lrow[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rb = 2 * p + h;
      const int row64 = 16 * rb + n;
      float lsum = 0.0f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float mh = stat_m[hh * 64 + row64];
        if (mh != kNegInf) lsum += stat_l[hh * 64 + row64] * exp2_fast((mh - mo[rb]) * c2);
      }
      lrow[h] = lsum;
      const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
      for (int nl = 0; nl < kColBlocks; ++nl)
        *(LDS_AS f32x4*)(stage + (16 * h + n) * kEpStride + 16 * nl + 4 * gq) = o[nl][rb] * inv;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const size_t pidx = ((size_t)b * a.row_groups + rg) * a.num_splits + split;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = 2 * k + er;               // row within the group
      if (rg * kRows + r >= rows_total) continue;
      const f32x4 v = *(LDS_AS const f32x4*)(stage + r * kEpStride + ec);
      if (nsplit_eff == 1) {
        u32x2 packed;
        packed[0] = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
        packed[1] = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
        *(u32x2*)(a.out + (row_base + rg * kRows + r) * kVDim + 128 * sub + ec) = packed;
      } else {
        // device-scope stores that the merge workgroups read (split_merge.h)
        split_merge::store_dev(a.ws_o + pidx * kRows * kVDim, 4 * (r * kVDim + 128 * sub + ec), v);
      }
    }
    if (nsplit_eff > 1 && sub == 0 && gq == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rb = 2 * p + h;
        const int row_in_rg = 16 * h + n;
        if (rg * kRows + row_in_rg < rows_total)
          split_merge::store_dev(a.ws_lse + pidx * kRows, 4 * row_in_rg,
                                 lrow[h] > 0.0f ? mo[rb] * c2 + __log2f(lrow[h]) : kNegInf);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // (the slice is rewritten for the next group)
  }
  if (nsplit_eff > 1) split_merge::signal_partials(a, b, rgp, split, sub, lane);   // (each of the four value waves)
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
  const int grid = decode_grid(a) + plan_merge(args, decode_grid(a));
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
