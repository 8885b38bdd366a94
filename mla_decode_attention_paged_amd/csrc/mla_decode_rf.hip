// gfx950 MLA decode over the paged FP8 (E4M3FN) cache with per-token float32
// scales, both contractions on the block-scaled FP8 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4): the "FP8 MFMA with the scales folded
// into the score columns and into P" option for the FP8 KV tiles of the
// "KVLoad2CvtProducer" page, without its widening stage.
//
// Storage as in the "generic_get_paged_cache_with_scales" page (Args) and the
// "KVCacheScalesMHAOperand" page (per-token Float32 scales).  The FP8 key
// bytes enter the MFMAs as they are; the 16-bit operands do not fit E4M3, so
// each is split into two E4M3 parts with power-of-two factors that the MFMA
// applies through its E8M0 operand scales:
//
//   * q (bf16) per query row: q = 2^a (hi + 2^-t lo), a and t chosen so that
//     each part uses the top of the E4M3 range; S^T = K q^T is the hi MFMA (B
//     scale 2^a) plus the lo MFMA (2^(a - t)), in fp32.  The last 64 dims go
//     through one MFMA with hi and lo side by side (the key bytes repeated);
//   * P' = p * key scale per query row, step (two 32-key tiles) and half of
//     the lanes: P' = 2^e (hi + 2^-4 lo), the largest of the 32 values in
//     [2^(e+7), 2^(e+8)); one MFMA per 16 columns takes the step's 64 keys,
//     hi and lo side by side (the V bytes repeated), with A scales 2^e and
//     2^(e-4).
//
// MFMA operand facts used (measured on gfx950): A and B bytes pair by (lane
// group of 16, byte); the E8M0 scale of K block q (32 values: lane groups
// 2(q % 2) and 2(q % 2) + 1, bytes [16 (q / 2), + 16)) for row / column m
// comes from lane 16 q + m.
//
// Workgroup = 4 waves (one per SIMD) on a pair of 32-row groups and one key
// range of one request, the role-split kernel's units.  Wave w owns 16 query
// rows (rows 16 (w % 2) + [0, 16) of row group w / 2 of the pair) and runs the
// whole step for them: scores of both tiles, its own online softmax, O += P' V
// for its 16 rows x 512 columns (fp32 accumulators).  Tiles arrive by direct
// global->LDS loads two steps ahead (four step buffers: the loop reads the
// keys of step j + 1 while it still reads the values of step j), one
// workgroup barrier per step.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <type_traits>

#include "mla_internal.h"
#include "split_merge.h"
#include "unit_order.h"

namespace mla {
namespace rf_path {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

constexpr int kThreads = 256;
constexpr int kTileBytes = kTile * kHeadDim;         // 18432: one 32-key FP8 tile
// In LDS the tile's second 16 keys start 32 bytes past 9 KiB, so that the 8
// keys of a transposing V read (4 from each half) fall on distinct banks.
constexpr int kHalfBytes = 16 * kHeadDim + 32;
constexpr int kTileStride = 2 * kHalfBytes;
constexpr int kSlots = 4;                            // steps of tiles in LDS
constexpr int kScaleBytes = 256;                     // per tile (64 lanes x 4 bytes; keys 0-31 twice)
constexpr int kLdsTiles = 0;
constexpr int kLdsScales = kLdsTiles + kSlots * 2 * kTileStride;
constexpr int kLdsLoop = kLdsScales + kSlots * 2 * kScaleBytes;
// epilogue (the tile buffers are idle): per wave 16 rows x 512 columns of O (fp32, padded rows)
constexpr int kEpStride = kVDim + 4;
constexpr int kLdsEpi = 4 * 16 * kEpStride * 4;
constexpr int kLdsTotal = kLdsEpi > kLdsLoop ? kLdsEpi : kLdsLoop;
static_assert(kLdsTotal <= 160 * 1024, "LDS budget");
static_assert(split_merge::lds_bytes(kThreads / 64) <= kLdsTotal, "merge state fits in the LDS");
static_assert(3 * 1024 <= kLdsScales, "the unit ranking's LDS lies in the tile buffers");

constexpr float kNegInf = -__builtin_inff();

// max / sum over the lanes l, l ^ 16 (v_permlane16_swap pairs 16-lane rows
// 2k and 2k + 1), and over l ^ 32 (v_permlane32_swap pairs the halves)
__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// the value of the lane l ^ 32
__device__ __forceinline__ float xor32_get(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }
template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct global->LDS loads of the tile stream, kept out of the compiler's
// view and waited for explicitly (vmcnt before the step barrier); writing M0
// right before an LDS DMA needs one wait state.
template <int kOff>
__device__ __forceinline__ void tile_dma16(const uint8_t* base, uint32_t voff, uint32_t ldst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3"
               :: "v"(voff), "s"(base), "s"(ldst), "n"(kOff) : "memory", "m0");
}
__device__ __forceinline__ void tile_dma4(const void* gsrc, uint32_t ldst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gsrc), "s"(ldst) : "memory", "m0");
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four floats -> four E4M3 bytes (round to nearest even), in order.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  s16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, a, b, 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}
__device__ __forceinline__ f32x4 e4m3x4_value(uint32_t u) {
  const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u, 1.0f, false);
  const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u, 1.0f, true);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

// The power-of-two factor 2^a with which the largest |x| = m lands in
// (224, 448]: a = ceil(log2(m / 448)) (0 for m = 0).
__device__ __forceinline__ int e4m3_exponent(float m) {
  if (!(m > 0.0f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(m);          // m = f 2^e, f in [0.5, 1)
  const float f = __builtin_amdgcn_frexp_mantf(m);
  return f <= 0.875f ? e - 9 : e - 8;
}

// Eight bf16 (one 16-byte load) scaled by 2^-qa: hi parts (E4M3) into two
// dwords; the unrounded values in y.
__device__ __forceinline__ void split_hi8(u32x4 w, int qa, float (&y)[8], uint32_t& h0, uint32_t& h1) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[2 * e] = __builtin_amdgcn_ldexpf(__uint_as_float(w[e] << 16), -qa);
    y[2 * e + 1] = __builtin_amdgcn_ldexpf(__uint_as_float(w[e] & 0xffff0000u), -qa);
  }
  h0 = e4m3x4(y[0], y[1], y[2], y[3]);
  h1 = e4m3x4(y[4], y[5], y[6], y[7]);
}

// Key (within a tile) of S^T register r % 4 of key block r / 4 in lane group
// g4; also the key (within tile r / 8 of the step) of P' byte r % 8.
__device__ __forceinline__ constexpr int step_key(int r, int g4) { return 16 * (r >> 2) + 4 * g4 + (r & 3); }

__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
mla_decode_rf_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  LDS_AS char* const L0 = (LDS_AS char*)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;         // lane group of 16
  const int n = lane & 15;          // query row (S^T, P') / column (O) within the 16

  if ((int)blockIdx.x >= a.dgrid) {
    split_merge::merge_workgroup<kThreads / 64>(a, (int)blockIdx.x - a.dgrid, (LDS_AS float*)lds);
    return;
  }

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
  const int rows_total = rq.count * a.num_heads;
  if (2 * rgp * kRows >= rows_total) return;
  const size_t row_base = (size_t)rq.first * a.num_heads;
  const int t_lo = split * T;
  const int t_hi = min(L, t_lo + T);
  const int ntiles = (t_hi - t_lo + kTile - 1) / kTile;
  const int nsteps = (ntiles + 1) / 2;
  const float c2 = a.sm_log2;

  const int rg = 2 * rgp + (wave >> 1);          // this wave's row group
  const bool rg_ok = rg < a.row_groups;
  const int row0 = rg * kRows + 16 * (wave & 1); // the wave's first row, within the request
  const int my_row = row0 + n;
  const bool row_ok = rg_ok && my_row < rows_total;
  const int my_i = row_ok ? my_row / a.num_heads : 0;
  const int lim = row_ok ? min(L - rq.count + my_i + 1, t_hi) : t_hi;   // keys < lim are visible
  int lim_min = row_ok ? lim : 0x7fffffff;
  for (int off = 8; off >= 1; off >>= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off));
  lim_min = __builtin_amdgcn_readfirstlane(lim_min);

  auto tile_buf = [&](int step, int tt) __attribute__((always_inline)) {
    return L0 + kLdsTiles + ((step % kSlots) * 2 + tt) * kTileStride;
  };
  auto scale_buf = [&](int step, int tt) __attribute__((always_inline)) {
    return L0 + kLdsScales + ((step % kSlots) * 2 + tt) * kScaleBytes;
  };

  // ---- tile loads (as the role-split kernel's): wave `wave` loads half
  // (wave & 1) of tile (wave >> 1) of a step, 9 blocks of 1 KiB, and that
  // tile's 32 scales.  Keys at or past t_hi are never read: their lanes
  // re-load the last valid key (finite data the softmax masks out).
  const int ld_key = lane >> 2;
  const int ld_col = (lane & 3) ^ ((lane >> 4) & 3);
  const uint8_t* layer_base = a.blocks + a.layer_offset;
  const float* slayer_base = a.scales + a.slayer_offset;
  const int nblk = (t_hi - t_lo + 15) >> 4;
  const uint32_t* ltr = a.lt + (size_t)b * a.max_pages;
  const uint32_t* sltr = a.slt + (size_t)b * a.max_pages;
  uint32_t nxt_page = 0, nxt_spage = 0;
  uint64_t w_off = 0, w_soff = 0;
  int cur_win = -1;
  auto fetch_window = [&](int m) __attribute__((always_inline)) {
    const int blk = 64 * m + lane;
    if (blk < nblk) {
      const uint32_t col = (uint32_t)(t_lo + 16 * blk) / (uint32_t)a.page_size;
      nxt_page = ltr[col];
      nxt_spage = sltr[col];
    }
  };
  auto enter_window = [&](int m) __attribute__((always_inline)) {
    const uint32_t slot = (uint32_t)(t_lo + 16 * (64 * m + lane)) % (uint32_t)a.page_size;
    w_off = (uint64_t)nxt_page * (uint64_t)a.page_stride + (uint64_t)slot * kHeadDim;
    w_soff = (uint64_t)nxt_spage * (uint64_t)a.spage_stride + (uint64_t)slot;
    cur_win = m;
    if (64 * (m + 1) < nblk) fetch_window(m + 1);
  };
  auto lane_u64 = [&](uint64_t v, int k) __attribute__((always_inline)) -> uint64_t {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, k);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), k);
    return ((uint64_t)hi << 32) | lo;
  };
  const int ld_tt = wave >> 1, ld_hb = wave & 1;
  // DMA instructions this wave issues for a step (10: nine blocks and the scales)
  auto dma_count = [&](int step) __attribute__((always_inline)) -> int {
    return (step < nsteps && 2 * step + ld_tt < ntiles) ? 10 : 0;
  };
  auto issue = [&](int step) __attribute__((always_inline)) {
    const int j = 2 * step + ld_tt;
    if (step >= nsteps || j >= ntiles) return;
    const int t0 = t_lo + kTile * j;
    const int nvalid = min(kTile, t_hi - t0);
    if ((step >> 4) != cur_win) enter_window(step >> 4);
    const int blk0 = ((t0 - t_lo) >> 4) & 63;
    const int bh = nvalid > 16 ? 1 : 0;
    const int kk = min(16 * ld_hb + ld_key, nvalid - 1);
    const int half = __builtin_amdgcn_readfirstlane(min(ld_hb, bh));
    const uint8_t* base = layer_base + lane_u64(w_off, blk0 + half);
    const uint32_t voff = (uint32_t)(kk - 16 * half) * kHeadDim + 16 * ld_col;
    LDS_AS char* dst = tile_buf(step, ld_tt) + kHalfBytes * ld_hb;
    // (both waves of a tile write its scales: the same bytes)
    {
      const int key = min(lane & 31, nvalid - 1);
      const uint64_t so0 = lane_u64(w_soff, blk0), so1 = lane_u64(w_soff, blk0 + bh);
      const float* srow = slayer_base + ((key >> 4) ? so1 : so0) + (size_t)(key & 15);
      tile_dma4(srow, (uint32_t)(uintptr_t)scale_buf(step, ld_tt));
    }
#define RF_DMA_CB(cb) tile_dma16<64 * (cb)>(base, voff, (uint32_t)(uintptr_t)dst + (1024 - 64) * (cb))
    RF_DMA_CB(0); RF_DMA_CB(1); RF_DMA_CB(2); RF_DMA_CB(3); RF_DMA_CB(4);
    RF_DMA_CB(5); RF_DMA_CB(6); RF_DMA_CB(7); RF_DMA_CB(8);
#undef RF_DMA_CB
  };
  auto wait_dma = [&](int outstanding) __attribute__((always_inline)) {
    if (outstanding >= 10) wait_vmcnt<10>();
    else wait_vmcnt<0>();
  };
  if (nsteps > 0) fetch_window(0);
  issue(0);
  issue(1);

  // ---- q of row n, in the B-operand order of the QK MFMAs: lane group g4
  // holds depth 128 kb + 32 g4 + [0, 32) for kb = 0..3 (hi and lo parts in
  // separate MFMAs), and depth 512 + 16 g4 + [0, 16) with hi in bytes 0-15 and
  // lo in bytes 16-31 (one MFMA).
  i32x8 qhi[4], qlo[4], qf;
  int sq_hi, sq_lo;                               // B scales (E8M0) of the two parts
  {
    const uint16_t* qrow = a.q + (row_base + (row_ok ? my_row : 0)) * kHeadDim;
    u32x4 raw[4][4], rawf[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int u = 0; u < 4; ++u) raw[kb][u] = *(const u32x4*)(qrow + 128 * kb + 32 * g4 + 8 * u);
#pragma unroll
    for (int u = 0; u < 2; ++u) rawf[u] = *(const u32x4*)(qrow + 512 + 16 * g4 + 8 * u);
    float qm = 0.0f;
    auto absmax = [&](u32x4 w) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qm = fmaxf(qm, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xffff0000u))));
    };
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int u = 0; u < 4; ++u) absmax(raw[kb][u]);
    absmax(rawf[0]);
    absmax(rawf[1]);
    qm = xor32_max(xor16_max(qm));
    const int qa = max(e4m3_exponent(qm), -120);
    // hi parts and the largest residual
    float rm = 0.0f;
    uint32_t hf[4];
    auto hi8 = [&](u32x4 w, uint32_t& h0, uint32_t& h1) __attribute__((always_inline)) {
      float y[8];
      split_hi8(w, qa, y, h0, h1);
      const f32x4 v0 = e4m3x4_value(h0), v1 = e4m3x4_value(h1);
#pragma unroll
      for (int e = 0; e < 4; ++e) rm = fmaxf(rm, fmaxf(fabsf(y[e] - v0[e]), fabsf(y[4 + e] - v1[e])));
    };
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t h0, h1;
        hi8(raw[kb][u], h0, h1);
        qhi[kb][2 * u] = (int)h0;
        qhi[kb][2 * u + 1] = (int)h1;
      }
    hi8(rawf[0], hf[0], hf[1]);
    hi8(rawf[1], hf[2], hf[3]);
    rm = xor32_max(xor16_max(rm));
    const int qt = min(-e4m3_exponent(rm), qa + 127);   // lo = E4M3(r 2^t); 2^(a - t) stays an E8M0 value
    auto lo8 = [&](u32x4 w, uint32_t h0, uint32_t h1, uint32_t& l0, uint32_t& l1) __attribute__((always_inline)) {
      float y[8];
      uint32_t d0, d1;
      split_hi8(w, qa, y, d0, d1);
      const f32x4 v0 = e4m3x4_value(h0), v1 = e4m3x4_value(h1);
      l0 = e4m3x4(__builtin_amdgcn_ldexpf(y[0] - v0[0], qt), __builtin_amdgcn_ldexpf(y[1] - v0[1], qt),
                  __builtin_amdgcn_ldexpf(y[2] - v0[2], qt), __builtin_amdgcn_ldexpf(y[3] - v0[3], qt));
      l1 = e4m3x4(__builtin_amdgcn_ldexpf(y[4] - v1[0], qt), __builtin_amdgcn_ldexpf(y[5] - v1[1], qt),
                  __builtin_amdgcn_ldexpf(y[6] - v1[2], qt), __builtin_amdgcn_ldexpf(y[7] - v1[3], qt));
    };
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t l0, l1;
        lo8(raw[kb][u], (uint32_t)qhi[kb][2 * u], (uint32_t)qhi[kb][2 * u + 1], l0, l1);
        qlo[kb][2 * u] = (int)l0;
        qlo[kb][2 * u + 1] = (int)l1;
      }
    uint32_t lf[4];
    lo8(rawf[0], hf[0], hf[1], lf[0], lf[1]);
    lo8(rawf[1], hf[2], hf[3], lf[2], lf[3]);
    qf = i32x8{(int)hf[0], (int)hf[1], (int)hf[2], (int)hf[3], (int)lf[0], (int)lf[1], (int)lf[2], (int)lf[3]};
    sq_hi = 127 + qa;
    sq_lo = 127 + qa - qt;
  }
  // folded block: K blocks 0 and 1 (scales from lanes 0-31) hold hi, 2 and 3 lo
  const int sq_f = g4 < 2 ? sq_hi : sq_lo;

  // ---- per-lane LDS addresses
  // K (A operand of QK), key m = n of key block kb2: bytes [128 kb + 32 g4, + 32)
  // = 16-byte columns 2 (g4 % 2) + {0, 1} of 64-byte block 2 kb + g4 / 2; the
  // folded block: 16-byte column g4 of block 8.
  const int swk = (n >> 2) & 3;
  const uint32_t ka0 = (uint32_t)(1024 * (g4 >> 1) + 16 * (4 * n + ((2 * (g4 & 1)) ^ swk)));
  const uint32_t ka1 = (uint32_t)(1024 * (g4 >> 1) + 16 * (4 * n + ((2 * (g4 & 1) + 1) ^ swk)));
  const uint32_t kaf = (uint32_t)(1024 * 8 + 16 * (4 * n + (g4 ^ swk)));
  // V (B operand of PV) by transposing reads: provider lane 2k + hh of lane
  // group g4 reads key step_key(k, g4) of a tile at columns 16 cb + 8 hh; the
  // receiving lane (g4, c) gets column 16 cb + c of those 8 keys, key k in byte k.
  const int vk = (lane & 15) >> 1, vhh = lane & 1;
  const int vkey = step_key(vk, g4);             // (vkey & 15) >> 2 == g4
  // column block cb (16 columns) of a tile: vlo[cb % 4] + 1024 (cb / 4)
  uint32_t vlo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    vlo[j] = (uint32_t)(kHalfBytes * (vkey >> 4) + 16 * (4 * (vkey & 15) + (j ^ g4)) + 8 * vhh);

  // ---- state
  f32x4 o[32];                  // O: column block cb (16 columns), rows 4 g4 + [0, 4)
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) o[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = kNegInf;        // reference max of row n (every lane group), unscaled
  float l_part = 0.0f;          // this lane's share of the row sum, against m_run
  const float thr = 16.0f / c2; // the reference moves when a score passes it by thr (p <= 2^16)

  // ---- the stages of a step (two tiles, or the last tile alone: `two`
  // false).  The loop is software-pipelined: the QK MFMAs of step j + 1 run
  // with the softmax of step j between them, then O += P' V of step j.
  //
  // step_sync(j): step j's loads have landed (this wave's, then every
  // wave's); every wave is done with step j - 2 (its V was read before this
  // point), so step j + 2 may load into its buffers.  Steps 0 and 1 were
  // issued before the q prologue.
  auto step_sync = [&](int j) __attribute__((always_inline)) {
    wait_dma(dma_count(j + 1));
    lds_barrier();
    issue(j + 2);
  };

  // S^T of step j: chain c = (tile c / 2, key block c % 2), row n, keys
  // 16 (c % 2) + 4 g4 + [0, 4) of tile c / 2 (chains 2 and 3 only with two
  // tiles).  The chains are interleaved so that back-to-back MFMAs are
  // independent; K is read one depth block ahead; between(kb) is placed with
  // the MFMAs of depth block kb.
  auto qk = [&](int j, auto two_c, f32x4 (&s)[4], auto&& between) __attribute__((always_inline)) {
    constexpr bool two = decltype(two_c)::value;
    constexpr int kC = two ? 4 : 2;
    uint32_t kt0[4], kt1[4];      // (masked as the V addresses: see pv)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t kt = (uint32_t)(uintptr_t)tile_buf(j, c >> 1) + kHalfBytes * (c & 1);
      kt0[c] = (kt + ka0) & 0x3ffffu;
      kt1[c] = (kt + ka1) & 0x3ffffu;
      s[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    i32x8 kc[4];
    auto kload = [&](int c, int kb) __attribute__((always_inline)) -> i32x8 {
      const u32x4 k0 = *(LDS_AS const u32x4*)(uintptr_t)(kt0[c] + 2048 * kb);
      const u32x4 k1 = *(LDS_AS const u32x4*)(uintptr_t)(kt1[c] + 2048 * kb);
      return i32x8{(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3], (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
    };
#pragma unroll
    for (int c = 0; c < kC; ++c) kc[c] = kload(c, 0);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      i32x8 kn[4];
      __builtin_amdgcn_sched_barrier(0);
      if (kb < 3) {
#pragma unroll
        for (int c = 0; c < kC; ++c) kn[c] = kload(c, kb + 1);
      } else {
#pragma unroll
        for (int c = 0; c < kC; ++c) {
          const u32x4 kf = *(LDS_AS const u32x4*)(uintptr_t)(kt0[c] - ka0 + kaf);
          kn[c] = i32x8{(int)kf[0], (int)kf[1], (int)kf[2], (int)kf[3], (int)kf[0], (int)kf[1], (int)kf[2], (int)kf[3]};
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // the next block's reads go out before this block's MFMAs
      between(kb);
#pragma unroll
      for (int c = 0; c < kC; ++c)
        s[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc[c], qhi[kb], s[c], 0, 0, 0, 127, 0, sq_hi);
#pragma unroll
      for (int c = 0; c < kC; ++c)
        s[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc[c], qlo[kb], s[c], 0, 0, 0, 127, 0, sq_lo);
#pragma unroll
      for (int c = 0; c < kC; ++c) kc[c] = kn[c];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < kC; ++c)
      s[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc[c], qf, s[c], 0, 0, 0, 127, 0, sq_f);
  };

  // The softmax of step j from its scores s, in four parts: 0 key scales and
  // mask, 1 the reference (moved lazily: only when a score passes it by thr;
  // O's factor is applied by rescale() before the step's P' V), 2 p and the
  // row sums, 3 P' split into its hi and lo parts (pa, and sp the A scale).
  float x[16], sv[16], pp[16];
  float sm_max = kNegInf, sm_al = 1.0f;
  bool sm_resc = false;
  i32x8 pa = i32x8{};
  int sp = 127;
  auto sm = [&](int k, int j, auto two_c, const f32x4 (&s)[4]) __attribute__((always_inline)) {
    constexpr bool two = decltype(two_c)::value;
    if (k == 0) {
      // x[r]: tile r / 8, key step_key(r % 8, g4) of it.  (A step with one
      // tile: the second tile's scores are -inf and its scales 0, so that its P' is 0.)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 v0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, v1 = v0;
        if (tt == 0 || two) {
          LDS_AS const float* sg = (LDS_AS const float*)scale_buf(j, tt);
          v0 = *(LDS_AS const f32x4*)(sg + 4 * g4);
          v1 = *(LDS_AS const f32x4*)(sg + 16 + 4 * g4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[8 * tt + e] = v0[e];
          sv[8 * tt + 4 + e] = v1[e];
        }
      }
      const int t0 = t_lo + 2 * kTile * j;
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool vis = (r < 8 || two) && t0 + 32 * (r >> 3) + step_key(r & 7, g4) < lim;
        x[r] = vis ? s[r >> 2][r & 3] * sv[r] : kNegInf;
        mx = fmaxf(mx, x[r]);
      }
      sm_max = mx;
    } else if (k == 1) {
      const float mt = xor32_max(xor16_max(sm_max));
      const bool mv = wave_any(mt > m_run + thr);
      const float m_new = mv ? fmaxf(m_run, mt) : m_run;
      sm_al = m_run == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      sm_resc = wave_any(m_new != m_run) && wave_any(m_run != kNegInf);
      l_part *= sm_al;              // (1 when the reference stays; l is 0 while it is -inf)
      m_run = m_new;
    } else if (k == 2) {
      const float nm = m_run == kNegInf ? 0.0f : -m_run * c2;
      float psum = 0.0f, pmax = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], c2, nm));
        psum += p;
        pp[r] = p * sv[r];
        pmax = fmaxf(pmax, pp[r]);
      }
      l_part += psum;
      sm_max = pmax;
    } else {
      // exponents: of this lane's pair of groups (g4 / 2) and of the other pair
      const float pm_own = xor16_max(sm_max);
      const float pm_other = xor32_get(pm_own);
      const int e_own = pm_own > 0.0f ? max(__builtin_amdgcn_frexp_expf(pm_own) - 8, -120) : 0;
      const int e_other = pm_other > 0.0f ? max(__builtin_amdgcn_frexp_expf(pm_other) - 8, -120) : 0;
      // A scale this lane gives: K block g4 (0: hi of groups 0-1, 1: hi of 2-3, 2: lo of 0-1, 3: lo of 2-3)
      sp = g4 == 0 ? 127 + e_own : g4 == 1 ? 127 + e_other : g4 == 2 ? 123 + e_other : 123 + e_own;
      // P' operand: byte r = hi part of x[r]'s key, byte 16 + r its lo part
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = __builtin_amdgcn_ldexpf(pp[4 * qd + e], -e_own);
        const uint32_t hu = e4m3x4(y[0], y[1], y[2], y[3]);
        const f32x4 hv = e4m3x4_value(hu);
        pa[qd] = (int)hu;
        pa[4 + qd] = (int)e4m3x4((y[0] - hv[0]) * 16.0f, (y[1] - hv[1]) * 16.0f, (y[2] - hv[2]) * 16.0f,
                                 (y[3] - hv[3]) * 16.0f);
      }
    }
  };
  auto softmax = [&](int j, auto two_c, const f32x4 (&s)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sm(k, j, two_c, s);
  };
  // O rows 4 g4 + e take the factor of their row (lane 4 g4 + e) when the
  // step moved the reference (rare).  (The empty asm statements keep O in
  // the accumulation registers outside this block: otherwise the compiler
  // moves all of O through ordinary registers on every step.)
  auto rescale = [&]() __attribute__((always_inline)) {
    if (sm_resc) {
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) asm volatile("" : "+a"(o[cb]));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = __shfl(sm_al, 4 * g4 + e);
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) o[cb][e] *= f;
      }
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) asm volatile("" : "+a"(o[cb]));
    }
  };
  // O += P' V of step j, 16 columns at a time; V bytes 0-7 from tile 0, 8-15
  // from tile 1 (zeros for a step with one tile), repeated.  Batches of four
  // column blocks: the next batch's reads go out before this batch's MFMAs.
  auto pv = [&](int j, auto two_c) __attribute__((always_inline)) {
    constexpr bool two = decltype(two_c)::value;
    // (LDS byte addresses masked to the 160 KiB range: with the sign bit
    // known clear the column-block steps fold into the reads' offsets)
    uint32_t vb0[4], vb1[4];
    const uint32_t tb0 = (uint32_t)(uintptr_t)tile_buf(j, 0), tb1 = (uint32_t)(uintptr_t)tile_buf(j, 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      vb0[q] = (tb0 + vlo[q]) & 0x3ffffu;
      vb1[q] = (tb1 + vlo[q]) & 0x3ffffu;
    }
    i32x2 wa[4][2], wb[4][2];
    auto vbatch = [&](int bt, i32x2 (&w)[4][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[k][0] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(uintptr_t)(vb0[k] + 1024 * bt));
        w[k][1] = two ? __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(uintptr_t)(vb1[k] + 1024 * bt))
                      : i32x2{0, 0};
      }
    };
    vbatch(0, wa);
#pragma unroll
    for (int bt = 0; bt < 8; ++bt) {
      __builtin_amdgcn_sched_barrier(0);
      if (bt < 7) vbatch(bt + 1, wb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const i32x8 vb = i32x8{wa[k][0][0], wa[k][0][1], wa[k][1][0], wa[k][1][1],
                               wa[k][0][0], wa[k][0][1], wa[k][1][0], wa[k][1][1]};
        o[4 * bt + k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pa, vb, o[4 * bt + k], 0, 0, 0, sp, 0, 127);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        wa[k][0] = wb[k][0];
        wa[k][1] = wb[k][1];
      }
    }
  };

  const int nfull = ntiles >> 1;     // steps with two tiles; an odd count ends with a one-tile step
  const std::true_type kTwo{};
  const std::false_type kOne{};
  auto none = [](int) {};
  f32x4 sa[4], sb[4];
  if (nsteps > 0) step_sync(0);
  if (nfull == 0) {
    if (ntiles == 1) {
      qk(0, kOne, sa, none);
      softmax(0, kOne, sa);
      rescale();
      pv(0, kOne);
    }
  } else {
    qk(0, kTwo, sa, none);
    for (int i = 0; i + 1 < nfull; ++i) {
      step_sync(i + 1);
      qk(i + 1, kTwo, sb, [&](int kb) __attribute__((always_inline)) { sm(kb, i, kTwo, sa); });
      rescale();
      pv(i, kTwo);
#pragma unroll
      for (int c = 0; c < 4; ++c) sa[c] = sb[c];
    }
    if (ntiles & 1) {
      step_sync(nfull);
      qk(nfull, kOne, sb, [&](int kb) __attribute__((always_inline)) { sm(kb, nfull - 1, kTwo, sa); });
      rescale();
      pv(nfull - 1, kTwo);
      softmax(nfull, kOne, sb);
      rescale();
      pv(nfull, kOne);
    } else {
      softmax(nfull - 1, kTwo, sa);
      rescale();
      pv(nfull - 1, kTwo);
    }
  }

  // ---- epilogue: O / l per row, out through LDS (row-major, 16 rows per wave)
  const float l_row = xor32_sum(xor16_sum(l_part));
  __syncthreads();              // the tile buffers are idle
  LDS_AS float* const ep = (LDS_AS float*)(L0) + wave * 16 * kEpStride;
  {
    const float inv_n = l_row > 0.0f ? 1.0f / l_row : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float inv = __shfl(inv_n, 4 * g4 + e);
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) ep[(4 * g4 + e) * kEpStride + 16 * cb + n] = o[cb][e] * inv;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the rows are in LDS before this wave reads them back
  if (rg_ok) {
    if (nsplit_eff == 1) {
      // final rows: 8 columns (16 bytes of bf16) per lane, one row per pass
#pragma unroll
      for (int rl = 0; rl < 16; ++rl) {
        const int row = row0 + rl;
        const f32x4 v0 = *(LDS_AS const f32x4*)(ep + rl * kEpStride + 8 * lane);
        const f32x4 v1 = *(LDS_AS const f32x4*)(ep + rl * kEpStride + 8 * lane + 4);
        if (row < rows_total) {
          u32x4 packed;
          packed[0] = (uint32_t)bf16_bits(v0[0]) | ((uint32_t)bf16_bits(v0[1]) << 16);
          packed[1] = (uint32_t)bf16_bits(v0[2]) | ((uint32_t)bf16_bits(v0[3]) << 16);
          packed[2] = (uint32_t)bf16_bits(v1[0]) | ((uint32_t)bf16_bits(v1[1]) << 16);
          packed[3] = (uint32_t)bf16_bits(v1[2]) | ((uint32_t)bf16_bits(v1[3]) << 16);
          *(u32x4*)(a.out + (row_base + row) * kVDim + 8 * lane) = packed;
        }
      }
    } else {
      const size_t pidx = ((size_t)b * a.row_groups + rg) * a.num_splits + split;
      float* po = a.ws_o + (pidx * kRows + 16 * (wave & 1)) * kVDim;
      // 4 columns (16 bytes) per lane, half a row per pass; device-scope stores
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int rl = k >> 1, c4 = 256 * (k & 1) + 4 * lane;
        split_merge::store_dev(po, 4 * (rl * kVDim + c4), *(LDS_AS const f32x4*)(ep + rl * kEpStride + c4));
      }
      if (g4 == 0) {
        // the row's log2-sum-exp
        split_merge::store_dev(a.ws_lse + pidx * kRows + 16 * (wave & 1), 4 * n,
                               l_row > 0.0f ? m_run * c2 + __log2f(l_row) : kNegInf);
      }
    }
  }
  if (nsplit_eff > 1) split_merge::signal_partials(a, b, rgp, split, wave, lane);
}

}  // namespace rf_path

hipError_t launch_decode_rf(const DecodeArgs& a, hipStream_t stream, hipEvent_t begin, hipEvent_t end) {
  using namespace rf_path;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mla_decode_rf_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsTotal);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  DecodeArgs args = a;
  const int grid = decode_grid(a) + plan_merge(args, decode_grid(a));
  if (begin && end) {
    hipExtLaunchKernelGGL(mla_decode_rf_kernel, dim3(grid), dim3(kThreads), kLdsTotal, stream, begin, end, 0, args);
  } else {
    hipLaunchKernelGGL(mla_decode_rf_kernel, dim3(grid), dim3(kThreads), kLdsTotal, stream, args);
  }
  return hipGetLastError();
}

}  // namespace mla
