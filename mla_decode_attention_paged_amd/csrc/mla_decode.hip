// gfx950 kernels: MLA decode over a paged FP8 (E4M3FN) latent cache with
// separately stored float32 scales.
//
// Storage follows the "generic_get_paged_cache_with_scales" page (section
// "Args": blocks / scales tensors, lookup_table, optional scales_lookup_table,
// cache_lengths) and the "KVCacheScalesMHAOperand" page (per-token Float32
// scales kept in the scales field).  The "KVLoad2CvtProducer" page describes a
// Blackwell pipeline in which producer warps stage FP8 KV tiles in shared
// memory, convert them to a 16-bit type, and hand them to MMA warps.  On CDNA4:
//
//   * FP8 key bytes go from HBM straight into LDS (global_load_lds_dwordx4,
//     no VGPR staging) and are widened in registers right before the MFMAs
//     that use them: to bf16 for QK^T (exact; q is bf16 as given, so every
//     product is exact and the fp32 accumulation is the only rounding) and to
//     f16 for PV, with P' = f16(p * scale).  gfx950's block-scaled FP8 MFMA
//     would skip the widening, but its internal accumulation keeps only about
//     12 bits of the products' magnitude sum, which large scores turn into
//     visible softmax weight errors; an FP8 P' is not accurate enough either;
//   * the roles are split between waves (four score waves and four value
//     waves, one of each per SIMD) so
//     that each keeps its operands in registers: q for the score waves, the
//     O accumulators for the value waves;
//   * the softmax is online, base 2, in fp32, with lazy rescaling;
//   * a workgroup either writes final bf16 rows or, when a request's keys are
//     split across workgroups, an fp32 partial (O / l, log2-sum-exp) that the
//     merge workgroups of the same launch combine (split_merge.h).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "mla_internal.h"
#include "split_merge.h"
#include "unit_order.h"

namespace mla {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
// Read-only kernel inputs read at wave-uniform addresses (page tables, cache
// lengths) go through the constant address space, so they become scalar loads.
#define CONST_AS __attribute__((address_space(4)))

constexpr int kTileBytes = kTile * kHeadDim;   // 18432: one 32-key FP8 tile
constexpr float kNegInf = -__builtin_inff();


// ---------------------------------------------------------------- page resolution
// Token t of request b: value page = LT[b, t / P], slot = t % P, scale page =
// SLT[b, t / P] (SLT is LT when no separate table was given).  Used by the
// resolve debug kernel; the decode kernel resolves whole 16-key blocks in its
// page windows (fetch_window / enter_window) and can record what it computed
// there (DecodeArgs::dbg_offsets).
struct PageRef {
  uint32_t page, slot, spage;
};

template <typename Ptr>
__device__ __forceinline__ PageRef resolve_token(Ptr lt, Ptr slt, int max_pages, int b, uint32_t t,
                                                 uint32_t page_size) {
  const uint32_t col = t / page_size;
  const size_t idx = (size_t)b * (size_t)max_pages + col;
  PageRef r;
  r.page = lt[idx];
  r.slot = t - col * page_size;
  r.spage = slt[idx];
  return r;
}

// ---------------------------------------------------------------- small helpers
__device__ __forceinline__ f16x8 fp8x8_to_f16(uint32_t lo, uint32_t hi) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Combine the values of lanes l and l^32.  v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second; with both set to
// x the two results hold (x_lo, x_lo) and (x_hi, x_hi) per half, so a symmetric
// combination of the two gives every lane op(x_lo, x_hi).
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Scheduling fence: keeps the compiler from hoisting loads of a later phase into
// an earlier one (which would raise peak register pressure past the budget).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// True in every lane when the predicate holds in any lane (wave-uniform result).
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Waits on the vector-memory counter with a compiler memory barrier, so that no
// LDS read of a tile is scheduled above the wait for that tile's DMA loads.
template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void lds_dma16(const void* gsrc, LDS_AS void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, ldst, 16, 0, 0);
}
// Same, with an immediate offset added to both the global and the LDS address.
template <int kOff>
__device__ __forceinline__ void lds_dma16_off(const void* gsrc, LDS_AS void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, ldst, 16, kOff, 0);
}
__device__ __forceinline__ void lds_dma4(const void* gsrc, LDS_AS void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, ldst, 4, 0, 0);
}

// The same direct global->LDS loads written out by hand for the tile stream.
// The compiler counts its own LDS DMA as a pending LDS write and makes every
// later LDS read (and every workgroup barrier) wait for it; a tile loaded a
// step ahead lands in a buffer nobody reads before the end-of-step wait, so the
// stream is kept out of the compiler's view and waited for explicitly
// (wait_vmcnt before the end-of-step barrier).  Writing M0 right before an LDS
// DMA needs one wait state, hence the s_nop.
// 16 bytes per lane from base + voff + kOff into LDS ldst + kOff + 16 * lane.
template <int kOff>
__device__ __forceinline__ void tile_dma16(const uint8_t* base, uint32_t voff, uint32_t ldst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3"
               :: "v"(voff), "s"(base), "s"(ldst), "n"(kOff) : "memory", "m0");
}
// 4 bytes per lane from gsrc into LDS ldst + 4 * lane.
__device__ __forceinline__ void tile_dma4(const void* gsrc, uint32_t ldst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gsrc), "s"(ldst) : "memory", "m0");
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS accesses are
// complete, then s_barrier.  Unlike __syncthreads it does not wait for vector
// memory, so tile loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Key position (within a 32-key tile) held by accumulator register r of an
// S^T = K Q^T 32x32 MFMA result, for lane half g = lane / 32.
__device__ __forceinline__ constexpr int tile_key(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// ---------------------------------------------------------------- the decode kernel
//
// Workgroup = 8 waves on a pair of 32-row groups (64 query rows: q position x
// head) and one key range [t_lo, t_hi) of one request.  The key range is cut
// into 32-key tiles; a "step" is two consecutive tiles, loaded once into LDS
// and used by both row groups.  Wave w runs on SIMD w % 4, so every SIMD
// hosts one score and one value wave; their phases are arranged so that one
// wave's VALU work (FP8 widening, softmax) overlaps the other's MFMAs.
//
//   score waves (w = 0..3; tile parity t = w / 2, depth half d = w % 2): for
//     tile 2i + t of step i, compute the partial S^T = K Q^T of both row
//     groups over their half of the 576-deep dot product (bytes [32d, 32d+32)
//     of every 64-byte block), on v_mfma_f32_32x32x16_bf16 with q (bf16) in
//     registers and the keys widened FP8 -> bf16 once for both groups.  The
//     two halves of a tile swap partial sums through LDS at the mid-step
//     barrier; then wave (t, d) finishes row group d: key scales (fp32),
//     online softmax against a reference max that follows the other tile's
//     wave and moves lazily, and the hand-off of P' (f16) and the tile's
//     reference max to the value waves.
//   value waves (w = 4..7; column quarter c = w - 4): own output columns
//     [128c, 128c + 128) of both row groups and compute O += P' V on
//     v_mfma_f32_32x32x16_f16 for the two tiles of the previous step (one
//     before the mid-step barrier, one after), widening each V fragment once
//     for both groups.  When a tile's reference differs from O's, the smaller
//     side is scaled to the larger (rare: references move lazily).  The
//     value waves also issue the tile loads, one step ahead.
//
// Tiles arrive by direct global->LDS dwordx4 loads; a tile buffer lives three
// steps (loaded, scored, consumed).  Two workgroup barriers per step order the
// hand-offs.
constexpr int kWaveCount = 8;
constexpr int kThreads = 64 * kWaveCount;
constexpr int kEpStride = 128 + 4;            // floats per row of a value wave's epilogue transpose
constexpr int kEpSlice = kRows * kEpStride;   // floats of one value wave's epilogue slice

// F8: the value contraction on the FP8 MFMA (per-token scales only): P' per
// tile and row group as 32 records of kF8Rec bytes, one per query row: the
// high E4M3 parts of its 32 keys, the low parts, and the row's power-of-two
// exponent (int32), padded so that the records spread over the LDS banks.
constexpr int kF8Rec = 80;
template <int NG, bool F8 = false>
struct Layout {
  static_assert(!F8 || NG == 1, "the FP8 value contraction serves per-token scales");
  static constexpr int kScaleBytes = NG == 1 ? 256 : 1280;      // per tile
  static constexpr int kPBytes = F8 ? kRows * kF8Rec : NG == 1 ? 2048 : 4096;   // P' (E4M3 / f16) or p (fp32) per tile and group
  static constexpr int kXBytes = 4096;                           // a 32 x 32 fp32 partial score tile
  static constexpr int kSlots = 3;                               // steps of tiles live at once
  static constexpr int kTiles = 0;                               // kSlots steps x 2 tiles
  static constexpr int kScales = kTiles + 2 * kSlots * kTileBytes;
  static constexpr int kP = kScales + 2 * kSlots * kScaleBytes;  // [step % 2][tile][row group]
  static constexpr int kAlphaBytes = 128;                        // 32 row maxima
  static constexpr int kAlpha = kP + 8 * kPBytes;                // [step % 2][tile][row group]
  static constexpr int kStats = kAlpha + 8 * kAlphaBytes;        // [row group][m0, m1, l0, l1][32]
  static constexpr int kMO = kStats + 2 * 4 * kRows * 4;         // [value wave][row group][32]: O's reference
  // partial-score exchange [tile][row group]: its own region when a P slot is
  // smaller than a score tile, else the P slot of the step being scored (its
  // owner reads the exchange before writing P' there)
  static constexpr bool kXOwn = kPBytes < kXBytes;
  static constexpr int kX = kMO + 8 * kRows * 4;
  static constexpr int kTotal = kX + (kXOwn ? 4 * kXBytes : 0);
};
static_assert(Layout<1>::kTotal <= 160 * 1024 && Layout<9>::kTotal <= 160 * 1024 &&
              Layout<1, true>::kTotal <= 160 * 1024, "LDS budget");
static_assert(4 * kEpSlice * 4 <= 6 * kTileBytes, "epilogue transposes fit in the tile buffers");
static_assert(2 * 2 * 18 * 64 * 16 <= 4 * kTileBytes, "q staging fits in the tile buffers of steps 1 and 2");
static_assert(split_merge::lds_bytes(kThreads / 64) <= Layout<1>::kTotal &&
              split_merge::lds_bytes(kThreads / 64) <= Layout<9>::kTotal, "merge state fits in the LDS");

// kRecord: also write the block offsets this kernel computes to a.dbg_offsets
// (the debug entry point's instantiation; the production one carries no such
// code, so that its registers are not spent on it).
template <int NG, bool kRecord, bool kF8 = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
mla_decode_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  using LY = Layout<NG, kF8>;
  LDS_AS char* const L0 = (LDS_AS char*)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const bool is_score = wave < 4;
  const int sub = wave & 3;
  const int g = lane >> 5;          // lane half
  const int n = lane & 31;          // MFMA column / row within the half

  // ---- Merge workgroups (past the decode grid) combine the split partials.
  if ((int)blockIdx.x >= a.dgrid) {
    split_merge::merge_workgroup<kThreads / 64>(a, (int)blockIdx.x - a.dgrid, (LDS_AS float*)lds);
    return;
  }

  // ---- The work unit (request, row-group pair, key split) of this
  // workgroup: request order, or largest key ranges first (unit_order.h).
  // In the largest-first order the unit is known only once the cache
  // lengths have arrived; meanwhile the value waves touch 256 evenly spaced
  // entries of the page tables and rows of q, so that the workgroup's first
  // reads of them find their address translations (and many lines) warm.
  // (Volatile reads whose values are never used: nothing waits for them
  // until the prologue's own waits.)
  if (a.lpt && !is_score) {
    const int k = sub * 64 + lane;
    const size_t nlt = (size_t)a.batch * a.max_pages;
    (void)*(volatile const uint32_t*)(a.lt + nlt * k / 256);
    (void)*(volatile const uint32_t*)(a.slt + nlt * k / 256);
    if (a.q_offsets == nullptr) {
      const size_t nrow = (size_t)a.batch * a.q_len * a.num_heads;
      (void)*(volatile const uint32_t*)(a.q + nrow * k / 256 * kHeadDim);
    }
  }
  const int rgp_count = (a.row_groups + 1) >> 1;
  const int unit = workgroup_unit(a, rgp_count, L0, tid, lane, wave);
  if (unit < 0) return;
  const int rgp = unit % rgp_count;
  const int bs = unit / rgp_count;
  const int split = bs % a.num_splits;
  const int b = bs / a.num_splits;

  const CONST_AS uint32_t* const lt = (const CONST_AS uint32_t*)a.lt;
  const CONST_AS uint32_t* const slt = (const CONST_AS uint32_t*)a.slt;
  // cache length, clipped to what the page table can address
  const int L = (int)min(((const CONST_AS uint32_t*)a.cache_lengths)[b],
                         (uint32_t)a.max_pages * (uint32_t)a.page_size);
  const int T = a.tokens_per_split;
  const int nsplit_eff = L <= 0 ? 1 : (L + T - 1) / T;
  if (split >= nsplit_eff) return;             // no keys here; nothing to write
  const RequestRows rq = request_rows(a, b);
  const int rows_total = rq.count * a.num_heads;   // this request's query rows (query-major)
  if (2 * rgp * kRows >= rows_total) return;   // the pair holds none of them (fewer queries than the largest)
  const size_t row_base = (size_t)rq.first * a.num_heads;
  const int t_lo = split * T;
  const int t_hi = min(L, t_lo + T);
  const int ntiles = (t_hi - t_lo + kTile - 1) / kTile;
  const int nsteps = (ntiles + 1) / 2;
  const float c2 = a.sm_log2;                  // scores are kept unscaled; exponents are c2 * (x - m)

  // ---- LDS regions
  auto tile_buf = [&](int step, int tt) __attribute__((always_inline)) {
    return L0 + LY::kTiles + ((step % LY::kSlots) * 2 + tt) * kTileBytes;
  };
  auto scale_buf = [&](int step, int tt) __attribute__((always_inline)) {
    return L0 + LY::kScales + ((step % LY::kSlots) * 2 + tt) * LY::kScaleBytes;
  };
  auto p_buf = [&](int step, int tt, int r) __attribute__((always_inline)) {
    return L0 + LY::kP + (((step & 1) * 2 + tt) * 2 + r) * LY::kPBytes;
  };
  auto alpha_buf = [&](int step, int tt, int r) __attribute__((always_inline)) {
    return (LDS_AS float*)(L0 + LY::kAlpha + (((step & 1) * 2 + tt) * 2 + r) * LY::kAlphaBytes);
  };
  auto x_buf = [&](int step, int tt, int r) __attribute__((always_inline)) {
    return LY::kXOwn ? L0 + LY::kX + (tt * 2 + r) * LY::kXBytes : p_buf(step, tt, r);
  };
  auto stats = [&](int r) __attribute__((always_inline)) {   // [m0, m1, l0, l1][32] of row group r
    return (LDS_AS float*)(L0 + LY::kStats) + r * 4 * kRows;
  };

  // ---- tile loads.  Global->LDS tile layout: 18 blocks of 1 KiB, block
  // 9*(key/16) + col/64; inside a block, 16-byte slot 4*(key%16) +
  // ((c%4) ^ ((key%16)/4 % 4)) holds bytes [16c, 16c+16) of that key (c = 16-byte
  // column).  The XOR spreads the 16 keys of an MFMA read over all LDS banks.
  const int ld_key = lane >> 2;                                   // key % 16 loaded by this lane
  const int ld_col = (lane & 3) ^ ((lane >> 4) & 3);              // 16B column % 4 loaded by this lane
  const uint8_t* layer_base = a.blocks + a.layer_offset;
  const float* slayer_base = a.scales + a.slayer_offset;

  // Row offsets of the key range's 16-key blocks (a block never straddles a
  // page: pages hold a multiple of 16 keys), 64 blocks (16 steps) at a time:
  // lane k of the value waves holds the byte offset of block 64 m + k's first
  // row in blocks[.., layer] and the float offset of its scale row, so that a
  // step's addresses come from v_readlane rather than from memory.  The page
  // ids of window m + 1 are prefetched while window m is in use.
  const int nblk = (t_hi - t_lo + 15) >> 4;
  const uint32_t* ltr = a.lt + (size_t)b * a.max_pages;
  const uint32_t* sltr = a.slt + (size_t)b * a.max_pages;
  uint32_t nxt_page = 0, nxt_spage = 0;          // raw page ids of the prefetched window
  uint64_t w_off = 0, w_soff = 0;                // offsets of the current window
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
    w_soff = (uint64_t)nxt_spage * (uint64_t)a.spage_stride + (uint64_t)slot * NG;
    cur_win = m;
    if (64 * (m + 1) < nblk) fetch_window(m + 1);
  };
  auto lane_u64 = [&](uint64_t v, int k) __attribute__((always_inline)) -> uint64_t {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, k);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), k);
    return ((uint64_t)hi << 32) | lo;
  };

  // Value wave sub loads half (sub & 1) of tile (sub >> 1) of `step` (9
  // blocks), and the scales of that tile when it loads half 0.  Keys at or past
  // t_hi are never read: their lanes re-load the last valid key (finite data
  // that the softmax masks out), so slots, pages and table columns past a
  // request's length stay untouched.  The nine block loads go out in three
  // parts of three, spread over the step, so that no wave stalls long on a full
  // memory pipeline and the request stream stays even.
  // source of the pending loads: a wave-uniform block-row base plus this lane's
  // 32-bit offset (scalar-base addressing)
  const uint8_t* dma_base = layer_base;
  uint32_t dma_voff = 0;
  auto issue_part = [&](int step, int part) __attribute__((always_inline)) {
    const int tt = sub >> 1, hb = sub & 1;
    const int j = 2 * step + tt;
    if (j >= ntiles) return;
    LDS_AS char* dst = tile_buf(step, tt) + 1024 * 9 * hb;
    if (part == 0) {
      const int t0 = t_lo + kTile * j;
      const int nvalid = min(kTile, t_hi - t0);     // >= 1
      if ((step >> 4) != cur_win) enter_window(step >> 4);
      const int blk0 = ((t0 - t_lo) >> 4) & 63;     // lane of the tile's first block in the window
      const int bh = nvalid > 16 ? 1 : 0;           // block of the second half (clamped)
      const int kk = min(16 * hb + ld_key, nvalid - 1);
      const int half = __builtin_amdgcn_readfirstlane(min(hb, bh));   // half holding this wave's keys
      const uint64_t row_off = lane_u64(w_off, blk0 + half);
      dma_base = layer_base + row_off;
      dma_voff = (uint32_t)(kk - 16 * half) * kHeadDim + 16 * ld_col;
      if (kRecord && lane == 0)
        a.dbg_offsets[2 * ((size_t)b * a.dbg_blocks + (t0 >> 4) + half)] = row_off;
      if (hb == 0) {
        LDS_AS char* sdst = scale_buf(step, tt);
        const int key = min(lane & 31, nvalid - 1);
        const uint64_t so0 = lane_u64(w_soff, blk0), so1 = lane_u64(w_soff, blk0 + bh);
        if (kRecord && lane == 0) {
          uint64_t* rec = a.dbg_offsets + 2 * ((size_t)b * a.dbg_blocks + (t0 >> 4)) + 1;
          rec[0] = so0;
          if (bh) rec[2] = so1;
        }
        const float* srow = slayer_base + ((key >> 4) ? so1 : so0) + (size_t)(key & 15) * NG;
        const uint32_t sd = (uint32_t)(uintptr_t)sdst;
        if constexpr (NG == 1) {
          tile_dma4(srow, sd);
        } else {
          // [group][key] layout: lane covers group 2i + lane/32 for key lane%32
#pragma unroll
          for (int i = 0; i < 5; ++i) tile_dma4(srow + min(2 * i + (lane >> 5), NG - 1), sd + 256 * i);
        }
      }
    }
    // The three loads of a part share one address register: column block cb
    // sits 64 B further in HBM, given by the instruction's immediate offset.
    // That offset also moves the LDS address, so the LDS base steps by 1024 - 64.
#define MLA_DMA_CB(cb) tile_dma16<64 * (cb)>(dma_base, dma_voff, (uint32_t)(uintptr_t)dst + (1024 - 64) * (cb))
    if (part == 0) { MLA_DMA_CB(0); MLA_DMA_CB(1); MLA_DMA_CB(2); }
    if (part == 1) { MLA_DMA_CB(3); MLA_DMA_CB(4); MLA_DMA_CB(5); }
    if (part == 2) { MLA_DMA_CB(6); MLA_DMA_CB(7); MLA_DMA_CB(8); }
#undef MLA_DMA_CB
  };

  // Scales of the 16 keys a lane holds in the S^T layout: per-key (NG == 1) or
  // of group gv ([group][key] layout, NG == 9).
  auto lane_scales = [&](LDS_AS const char* sb, int gv, float (&sv16)[16]) __attribute__((always_inline)) {
    LDS_AS const float* sg = (LDS_AS const float*)sb + 32 * gv;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const f32x4 sv = *(LDS_AS const f32x4*)(sg + 8 * qq + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) sv16[4 * qq + e] = sv[e];
    }
  };

  // ================================================================ the step loops
  // Each role runs its own copy of the step loop (so that the register
  // allocator never sees q and the accumulators live together); both copies
  // pass the same number of workgroup barriers.
  if (is_score) {
    const int par = sub >> 1;      // tile parity this wave scores
    const int d = sub & 1;         // depth half; also the row group it finishes
    // rows of row group d (the softmax side) in the S^T layout: lane column n
    const int my_row = (2 * rgp + d) * kRows + n;
    const bool row_ok = my_row < rows_total;
    const int my_i = row_ok ? my_row / a.num_heads : 0;
    // keys visible to this row: j < L - Q + i + 1, clipped to this split
    const int lim = row_ok ? min(L - rq.count + my_i + 1, t_hi) : t_hi;
    int lim_min = row_ok ? lim : 0x7fffffff;
    for (int off = 16; off >= 1; off >>= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off));
    lim_min = __builtin_amdgcn_readfirstlane(min(lim_min, __shfl_xor(lim_min, 32)));
    // K read (A operand): lane (key n, half g) reads 16-byte column 4s + 2d + g
    // of its key for 64-byte block s.
    const uint32_t kread = (uint32_t)(1024 * 9 * (n >> 4) + 16 * (4 * (n & 15) + ((2 * d + g) ^ ((n >> 2) & 3))));
    // Lazy threshold: the reference moves only when a score passes it by thr,
    // so p <= 2^(c2 thr).  With group scales P' is formed on the value side and
    // thr stays at 8 / c2 (p <= 2^8); with per-token scales it is set per tile
    // so that P' = p * s stays below 2^15 (finite in f16) for the tile's largest
    // scale, at most 16 / c2.
    const float thr8 = 8.0f / c2;

    float m_run = kNegInf;     // running reference max per row (same in both halves), unscaled
    float l_part = 0.0f;       // this lane's share of the row sum, against m_run

    // q of both row groups in the B-operand order of the 32x32x16 MFMAs: for
    // block s the two MFMAs take depths 64s + 32d + 16g + [0,8) and + [8,16) --
    // the same depths as the key bytes each lane reads.
    // The two tile-parity waves of a depth half need the same q: each loads its
    // own row group's share from HBM and passes it to the other through LDS
    // (staged in the tile buffers of steps 1 and 2, which are not loaded yet).
    bf16x8 qk[18], qg[18], qown[18];   // q of the row group this wave keeps (d) / gives (1 - d)
    {
      const int row = (2 * rgp + par) * kRows + n;
      const bool ok = row < rows_total;
      const uint16_t* qrow = a.q + (row_base + (ok ? row : 0)) * kHeadDim + 32 * d + 16 * g;
#pragma unroll
      for (int s = 0; s < 9; ++s) {
        const u32x4* src = (const u32x4*)(qrow + 64 * s);
        u32x4 w0 = src[0], w1 = src[1];
        if (!ok) { w0 = u32x4{0, 0, 0, 0}; w1 = u32x4{0, 0, 0, 0}; }
        qown[2 * s] = __builtin_bit_cast(bf16x8, w0);
        qown[2 * s + 1] = __builtin_bit_cast(bf16x8, w1);
      }
    }
    LDS_AS char* const qstage = L0 + LY::kTiles + 2 * kTileBytes;   // [depth half][row group][18][64 lanes][16 B]
#pragma unroll
    for (int j = 0; j < 18; ++j)
      *(LDS_AS bf16x8*)(qstage + (((d * 2 + par) * 18 + j) * 64 + lane) * 16) = qown[j];
    __syncthreads();            // q shares staged
#pragma unroll
    for (int j = 0; j < 18; ++j) {
      const bf16x8 other = *(LDS_AS const bf16x8*)(qstage + (((d * 2 + (par ^ 1)) * 18 + j) * 64 + lane) * 16);
      qk[j] = par == d ? qown[j] : other;
      qg[j] = par == d ? other : qown[j];
    }
    __syncthreads();            // step 0 has landed (the value waves waited for their loads)

    for (int i = 0; i <= nsteps; ++i) {
      const int j = 2 * i + par;
      const bool have = i < nsteps && j < ntiles;
      const int t0 = t_lo + kTile * j;
      LDS_AS const char* tb = tile_buf(i, par);
      LDS_AS const char* sb = scale_buf(i, par);
      // ---- phase 1: partial scores of both row groups over depth half d:
      // accK for row group d (finished here), accG for row group 1 - d
      f32x16 accK, accG;
      // the other tile's reference after its previous tile (written before the
      // last end-of-step barrier): read now, its latency under the MFMAs
      float m_other = kNegInf;
      if (have && i > 0) m_other = alpha_buf(i - 1, par ^ 1, d)[n];
      if (have) {
        accK = f32x16{};
        accG = f32x16{};
        // all nine key reads are issued up front: one LDS latency per tile (the
        // group-scale variant, short of registers, reads them one block ahead:
        // measured 2.5 % faster on 128 x 4 queries over 2,048..32,768 keys
        // than reading each block where it is used)
        u32x4 kws[9];
        if constexpr (NG == 1) {
#pragma unroll
          for (int s = 0; s < 9; ++s) kws[s] = *(LDS_AS const u32x4*)(tb + kread + 1024 * s);
          sched_fence();
        }
        u32x4 kw_next = NG == 1 ? kws[0] : *(LDS_AS const u32x4*)(tb + kread);
#pragma unroll
        for (int s = 0; s < 9; ++s) {
          const u32x4 kw = NG == 1 ? kws[s] : kw_next;
          if constexpr (NG != 1) {
            if (s + 1 < 9) kw_next = *(LDS_AS const u32x4*)(tb + kread + 1024 * (s + 1));
          }
          const bf16x8 k0 = fp8x8_to_bf16(kw[0], kw[1]);
          const bf16x8 k1 = fp8x8_to_bf16(kw[2], kw[3]);
          if constexpr (NG == 1) {
            accK = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qk[2 * s], accK, 0, 0, 0);
            accG = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qg[2 * s], accG, 0, 0, 0);
            accK = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qk[2 * s + 1], accK, 0, 0, 0);
            accG = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qg[2 * s + 1], accG, 0, 0, 0);
          } else {
            // block s is scale group s: acc += scale * (this half's partial sums)
            f32x16 u0 = f32x16{}, u1 = f32x16{};
            u0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qk[2 * s], u0, 0, 0, 0);
            u1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qg[2 * s], u1, 0, 0, 0);
            u0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qk[2 * s + 1], u0, 0, 0, 0);
            u1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qg[2 * s + 1], u1, 0, 0, 0);
            float sv16[16];
            lane_scales(sb, s, sv16);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              accK[r] = __builtin_fmaf(sv16[r], u0[r], accK[r]);
              accG[r] = __builtin_fmaf(sv16[r], u1[r], accG[r]);
            }
          }
        }
        // the other row group's partial goes to the wave finishing it (same tile, depth 1 - d)
        LDS_AS char* xo = x_buf(i, par, d ^ 1);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          *(LDS_AS f32x4*)(xo + 1024 * qq + 16 * lane) = f32x4{accG[4 * qq], accG[4 * qq + 1], accG[4 * qq + 2], accG[4 * qq + 3]};
      }
      lds_barrier();            // mid-step: partial scores exchanged
      // ---- phase 2: row group d of this tile: full scores, online softmax, P'
      if (have) {
        LDS_AS const char* xi = x_buf(i, par, d);
        float x[16];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const f32x4 o4 = *(LDS_AS const f32x4*)(xi + 1024 * qq + 16 * lane);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * qq + e] = accK[4 * qq + e] + o4[e];
        }
        // x = the scaled score without softmax_scale (exponents use c2 * (x - m))
        float sv16[16];
        float thr = thr8;
        if constexpr (NG == 1) {
          lane_scales(sb, 0, sv16);
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] *= sv16[r];
          float smax = sv16[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) smax = fmaxf(smax, sv16[r]);
          smax = halves_max(smax);                        // the tile's 32 keys
          thr = fminf(16.0f, fmaxf(0.0f, 15.0f - __log2f(smax))) / c2;
        }
        if (t0 + kTile > lim_min) {
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = (t0 + tile_key(r, g) < lim) ? x[r] : kNegInf;
        }
        float mt = x[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
        mt = halves_max(mt);
        // The reference max moves up to the other tile's wave's (as it stood
        // after its previous tile), and lazily to this tile's max, only when a
        // score here passes the reference by more than thr.
        LDS_AS float* ab = alpha_buf(i, par, d);
        float mref = m_run;
        mref = fmaxf(mref, m_other);
        if (wave_any(mt > mref + thr)) mref = fmaxf(mref, mt);
        if (wave_any(mref != m_run)) {
          l_part *= m_run == kNegInf ? 0.0f : exp2_fast((m_run - mref) * c2);
          m_run = mref;
        }
        ab[n] = m_run;                // the tile's reference; both halves write the same value
        const float nm = m_run == kNegInf ? 0.0f : -m_run * c2;
        float p[16];
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = exp2_fast(__builtin_fmaf(x[r], c2, nm));
          psum += p[r];
        }
        l_part += psum;
        LDS_AS char* pb = p_buf(i, par, d);
        if constexpr (kF8) {
          // P' = p * key scale, split per row against a power-of-two exponent
          // e (the row's largest P' in this tile is m 2^(e + 8), m in [0.5, 1)):
          // P' = 2^e (hi + 2^-4 lo) with hi = E4M3(P' 2^-e) <= 256 and lo =
          // E4M3((P' 2^-e - hi) 2^4).  Record of row n: the 32 hi bytes in key
          // order, the 32 lo bytes, e.  This lane holds keys 8j + 4g .. + 3.
          float pp[16];
          float pm = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pp[r] = p[r] * sv16[r];
            pm = fmaxf(pm, pp[r]);
          }
          pm = halves_max(pm);
          const int ex = pm > 0.0f ? max(__builtin_amdgcn_frexp_expf(pm) - 8, -120) : 0;
          LDS_AS char* rec = pb + kF8Rec * n;
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = __builtin_amdgcn_ldexpf(pp[4 * jq + e], -ex);
            s16x2 hw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, y[0], y[1], 1.0f, false);
            hw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hw, y[2], y[3], 1.0f, true);
            const uint32_t hu = __builtin_bit_cast(uint32_t, hw);
            const f32x2 h01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hu, 1.0f, false);
            const f32x2 h23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hu, 1.0f, true);
            s16x2 lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, (y[0] - h01[0]) * 16.0f,
                                                                (y[1] - h01[1]) * 16.0f, 1.0f, false);
            lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw, (y[2] - h23[0]) * 16.0f, (y[3] - h23[1]) * 16.0f,
                                                          1.0f, true);
            *(LDS_AS uint32_t*)(rec + 8 * jq + 4 * g) = hu;
            *(LDS_AS uint32_t*)(rec + 32 + 8 * jq + 4 * g) = __builtin_bit_cast(uint32_t, lw);
          }
          if (g == 0) *(LDS_AS int*)(rec + 64) = ex;
        } else if constexpr (NG == 1) {
          // P' = f16(p * key scale) in the A-operand order of the PV MFMA
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            f16x8 pa;
#pragma unroll
            for (int e = 0; e < 8; ++e) pa[e] = (_Float16)(p[8 * hh + e] * sv16[8 * hh + e]);
            *(LDS_AS f16x8*)(pb + 1024 * hh + 16 * lane) = pa;
          }
        } else {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            *(LDS_AS f32x4*)(pb + 1024 * qq + 16 * lane) = f32x4{p[4 * qq], p[4 * qq + 1], p[4 * qq + 2], p[4 * qq + 3]};
        }
      }
      lds_barrier();            // end of step
    }
    const float l_row = halves_sum(l_part);
    if (g == 0) {
      LDS_AS float* st = stats(d);
      st[par * kRows + n] = m_run;
      st[(2 + par) * kRows + n] = l_row;
    }
    __syncthreads();
    return;
  }

  // ================================================================ value waves
  // With per-token scales the value waves carry the step's critical path
  // (their reads, the tile loads and the PV MFMAs); a higher issue priority
  // than the score waves on the same SIMD shortens it.  (Measured: 7 % on
  // the main kernel with 16 x 4096 keys; with group scales it costs 6 %, so
  // that variant keeps equal priorities.)
  if constexpr (NG == 1) __builtin_amdgcn_s_setprio(1);
  const int vq4 = sub;                // value wave owns columns [128 vq4, 128 vq4 + 128) of both groups
  // O holds sum_j 2^(c2 (x_j - mO)) s_j v_j for the row's reference max mO,
  // kept per row in LDS (C-layout rows 8(r/4) + 4g + r%4) and in a register
  // for the lane's A-layout row n.
  LDS_AS float* const mo_lds = (LDS_AS float*)(L0 + LY::kMO) + 2 * kRows * sub;   // [row group][32]
  float mo_a[2] = {kNegInf, kNegInf};
  if (g == 0) { mo_lds[n] = kNegInf; mo_lds[kRows + n] = kNegInf; }
  // V read (B operand via transpose read): provider lane p = 2k + h of each 16-lane
  // group addresses key tau(g,k) = 4g + (k&3) + 8(k>>2) at column 32nb + 16q + 8h.
  const int vq = (lane >> 4) & 1, vk = (lane & 15) >> 1, vh = lane & 1;
  const int vtau = 4 * g + (vk & 3) + 8 * (vk >> 2);
  const uint32_t vread0 = (uint32_t)(16 * (4 * vtau + ((0 + vq) ^ ((vtau >> 2) & 3))) + 8 * vh);
  const uint32_t vread1 = (uint32_t)(16 * (4 * vtau + ((2 + vq) ^ ((vtau >> 2) & 3))) + 8 * vh);
  f32x16 o[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[r][i] = f32x16{};
  if (nsteps > 0) {
    fetch_window(0);
    issue_part(0, 0);
    issue_part(0, 1);
    issue_part(0, 2);
  }
  __syncthreads();              // (the score waves stage q)
  wait_vmcnt<0>();              // this wave's share of step 0 has landed
  __syncthreads();

  // P' (f16, NG == 1) or p (fp32, NG == 9) of one tile and row group in this
  // lane's A-operand order, as raw dwords.
  typedef u32x4 PRaw[NG == 1 ? 2 : 4];
  auto load_p = [&](LDS_AS const char* pb, PRaw& pr) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < (NG == 1 ? 2 : 4); ++k) pr[k] = *(LDS_AS const u32x4*)(pb + 1024 * k + 16 * lane);
  };
  // Bring O of row group r and both tiles of a step to one reference per row,
  // max(O's, tile 0's, tile 1's): O is rescaled at most once per step, and
  // only when a reference moved (rare: references move lazily); the factors
  // for the tiles' P' come back in pf (1 when nothing changes).
  auto align_step = [&](int r, int step, bool two, const float (&mt)[2], float (&pf)[2], bool (&sp)[2])
      __attribute__((always_inline)) {
    pf[0] = pf[1] = 1.0f;
    sp[0] = sp[1] = false;
    const float mt1 = two ? mt[1] : kNegInf;
    const float m_new = fmaxf(mo_a[r], fmaxf(mt[0], mt1));
    if (wave_any(mt[0] != mo_a[r] || (two && mt1 != mo_a[r]))) {
      if (wave_any(m_new != mo_a[r])) {
        LDS_AS float* mol = mo_lds + r * kRows;
        LDS_AS const float* a0 = alpha_buf(step, 0, r);
        LDS_AS const float* a1 = alpha_buf(step, 1, r);
        // (while every row's reference is still -inf, O is zero: nothing to scale)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          if (!wave_any(mo_a[r] != kNegInf)) break;
          const f32x4 old = *(LDS_AS const f32x4*)(mol + 8 * qq + 4 * g);
          const f32x4 t0 = *(LDS_AS const f32x4*)(a0 + 8 * qq + 4 * g);
          const f32x4 t1 = two ? *(LDS_AS const f32x4*)(a1 + 8 * qq + 4 * g) : f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float nw = fmaxf(old[e], fmaxf(t0[e], t1[e]));
            const float al = old[e] == kNegInf ? 0.0f : exp2_fast((old[e] - nw) * c2);
#pragma unroll
            for (int nl = 0; nl < 4; ++nl) o[r][nl][4 * qq + e] *= al;
          }
        }
        if (g == 0) mol[n] = m_new;
      }
      pf[0] = mt[0] == kNegInf ? 0.0f : exp2_fast((mt[0] - m_new) * c2);
      pf[1] = mt1 == kNegInf ? 0.0f : exp2_fast((mt1 - m_new) * c2);
      sp[0] = wave_any(pf[0] != 1.0f);
      sp[1] = two && wave_any(pf[1] != 1.0f);
      mo_a[r] = m_new;
    }
  };
  // Everything a tile's PV step reads from LDS -- the V fragments (ds_read_b64_tr_b8),
  // P' of both row groups and their reference maxima -- is fetched ahead of the
  // MFMAs, so that the LDS latency is not paid per MFMA.
  typedef i32x2 VFrag[2][4];
  auto fetch_p = [&](int step, int tt, PRaw (&pr)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 2; ++r) load_p(p_buf(step, tt, r), pr[r]);
  };
  auto fetch_v = [&](int step, int tt, VFrag& vr) __attribute__((always_inline)) {
    LDS_AS const char* tb = tile_buf(step, tt);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int nl = 0; nl < 4; ++nl) {
        const int nb = 4 * vq4 + nl;
        vr[hh][nl] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (LDS_AS i32x2*)(tb + ((nb & 1) ? vread1 : vread0) + 1024 * (9 * hh + (nb >> 1))));
      }
  };
  // Per-token scales: the VALU part of a tile (P' brought to the step's
  // reference, V widened to f16) ...
  auto prep_p = [&](const PRaw (&pr)[2], const float (&pf)[2], const bool (&sp)[2], f16x8 (&pa)[2][2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) pa[r][hh] = __builtin_bit_cast(f16x8, pr[r][hh]);
      if (sp[r]) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 8; ++e) pa[r][hh][e] = (_Float16)((float)pa[r][hh][e] * pf[r]);
      }
    }
  };
  auto widen_v = [&](const VFrag& vr, f16x8 (&vb)[2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int nl = 0; nl < 4; ++nl) vb[hh][nl] = fp8x8_to_f16((uint32_t)vr[hh][nl][0], (uint32_t)vr[hh][nl][1]);
  };
  // ... and its MFMA part, O += P' V for both row groups.
  auto mma_tile = [&](const f16x8 (&pa)[2][2], const f16x8 (&vb)[2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int nl = 0; nl < 4; ++nl) {
        o[0][nl] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[0][hh], vb[hh][nl], o[0][nl], 0, 0, 0);
        o[1][nl] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[1][hh], vb[hh][nl], o[1][nl], 0, 0, 0);
      }
  };
  // Group scales: one tile, P'_g = f16(p * s_g) per value group, then O += P'_g V.
  auto compute_tile_g = [&](int step, int tt, const VFrag& vr, const PRaw (&pr)[2], const float (&pf)[2])
      __attribute__((always_inline)) {
    LDS_AS const char* sb = scale_buf(step, tt);
    // value group gv = columns [64gv, 64gv + 64) = blocks nb = 2gv, 2gv + 1
#pragma unroll
    for (int gl = 0; gl < 2; ++gl) {
      const int gv = 2 * vq4 + gl;
      float sv16[16];
      lane_scales(sb, gv, sv16);
      f16x8 pa[2][2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = __builtin_bit_cast(f32x4, pr[r][2 * hh + (e >> 2)])[e & 3];
            pa[r][hh][e] = (_Float16)(pv * pf[r] * sv16[8 * hh + e]);
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) {
          const int nl = 2 * gl + nn;
          const f16x8 vb = fp8x8_to_f16((uint32_t)vr[hh][nl][0], (uint32_t)vr[hh][nl][1]);
          o[0][nl] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[0][hh], vb, o[0][nl], 0, 0, 0);
          o[1][nl] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[1][hh], vb, o[1][nl], 0, 0, 0);
        }
      }
    }
  };

  // F8 value contraction (per-token scales): one 32x32x64 FP8 MFMA covers
  // both tiles of a step.  The MFMA pairs A and B bytes of the same lane half
  // and byte, and takes the E8M0 scale of A's K block 0 (bytes 0-15 of both
  // lane halves) for row m from lane m, of K block 1 (bytes 16-31) from lane
  // 32 + m.  So bytes 0-15 of lane half g hold keys 16 g .. 16 g + 15 of tile
  // 0, bytes 16-31 the same keys of tile 1, and lane (g, n) gives the
  // exponent of tile g's row n.  P' (A) comes from the score waves' records;
  // V (B) from transposing reads of 8 keys each: provider lane 2k + h of a
  // 16-lane group reads key k of the 8 at columns [16 q + 8 h, + 8) of the
  // 32-column block, and receiving lane 8 h + c gets column 16 q + 8 h + c of
  // the 8 keys.  P' = 2^e (hi + 2^-4 lo) enters as two MFMAs whose A scales
  // are 2^e and 2^(e - 4).
  const int f8_kp = (lane & 15) >> 1, f8_h = lane & 1, f8_q = (lane >> 4) & 1;
  // V read r8 (0..3) of 32-column block nb: tile r8 / 2, keys 16 g + 8 (r8 % 2) + [0, 8)
  auto f8_vaddr = [&](int r8, int nb) __attribute__((always_inline)) -> uint32_t {
    const int nba = 4 * vq4 + nb;                       // absolute 32-column block
    const int key = 16 * g + 8 * (r8 & 1) + f8_kp;
    const int c16 = 2 * (nba & 1) + f8_q;               // 16-byte column within the 64-byte block
    return (uint32_t)(1024 * (9 * (key >> 4) + (nba >> 1)) +
                      16 * (4 * (key & 15) + (c16 ^ (((key & 15) >> 2) & 3))) + 8 * f8_h);
  };
  // The 16 P' values of one tile in dwords [4 t, 4 t + 4) of hi and lo,
  // scaled by f (the step's reference moved; rare): decode, scale, split again
  // against an exponent moved by f's binary exponent, so that the other lane
  // half (same row, same tile, same f) moves it alike.  Returns that move.
  auto f8_rescale = [&](i32x8& hi, i32x8& lo, int t, float f) __attribute__((always_inline)) -> int {
    const int dx = __builtin_amdgcn_frexp_expf(f);
    const float fm = __builtin_amdgcn_ldexpf(f, -dx);   // in [0.5, 1)
#pragma unroll
    for (int w = 4 * t; w < 4 * t + 4; ++w) {
      const f32x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)hi[w], 1.0f, false);
      const f32x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)hi[w], 1.0f, true);
      const f32x2 l0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)lo[w], 1.0f, false);
      const f32x2 l1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)lo[w], 1.0f, true);
      const float y[4] = {__builtin_fmaf(l0[0], 0.0625f, h0[0]) * fm, __builtin_fmaf(l0[1], 0.0625f, h0[1]) * fm,
                          __builtin_fmaf(l1[0], 0.0625f, h1[0]) * fm, __builtin_fmaf(l1[1], 0.0625f, h1[1]) * fm};
      s16x2 hw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, y[0], y[1], 1.0f, false);
      hw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hw, y[2], y[3], 1.0f, true);
      const uint32_t hu = __builtin_bit_cast(uint32_t, hw);
      const f32x2 h01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hu, 1.0f, false);
      const f32x2 h23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hu, 1.0f, true);
      s16x2 lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, (y[0] - h01[0]) * 16.0f,
                                                          (y[1] - h01[1]) * 16.0f, 1.0f, false);
      lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw, (y[2] - h23[0]) * 16.0f, (y[3] - h23[1]) * 16.0f, 1.0f, true);
      hi[w] = (int)hu;
      lo[w] = __builtin_bit_cast(int, lw);
    }
    return dx;
  };

  // Phase 1 of a step (the score waves run their QK MFMAs): fetch the previous
  // step's tiles from LDS and do their VALU work.  Phase 2 (the score waves run
  // the softmax): the PV MFMAs.  The next step's loads go out in phase 1.
  for (int i = 0; i <= nsteps; ++i) {
    const bool next = i + 1 < nsteps;
    if constexpr (NG != 1) {
      // (the group-scale variant is short of registers to hold its tile reads
      // across the loads: they go out first)
      if (next) {
        issue_part(i + 1, 0);
        issue_part(i + 1, 1);
        issue_part(i + 1, 2);
      }
    }
    const bool have0 = i >= 1, have1 = i >= 1 && 2 * (i - 1) + 1 < ntiles;
    float pf[2][2];           // [row group][tile]
    bool sp[2][2];
    if (have0) {
      float mt[2][2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        mt[r][0] = alpha_buf(i - 1, 0, r)[n];
        mt[r][1] = alpha_buf(i - 1, 1, r)[n];
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) align_step(r, i - 1, have1, mt[r], pf[r], sp[r]);
    }
    if constexpr (kF8) {
      // bytes 0-15 of lane half g: keys 16 g + [0, 16) of tile 0, bytes 16-31: of tile 1
      i32x8 ahi[2], alo[2], vb8[4];
      int ex[2][2];             // [row group][tile]
      if (have0) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          LDS_AS const char* r0 = p_buf(i - 1, 0, r) + kF8Rec * n;
          LDS_AS const char* r1 = p_buf(i - 1, 1, r) + kF8Rec * n;
          const u32x4 h0 = *(LDS_AS const u32x4*)(r0 + 16 * g), l0 = *(LDS_AS const u32x4*)(r0 + 32 + 16 * g);
          ex[r][0] = *(LDS_AS const int*)(r0 + 64);
          u32x4 h1 = u32x4{0, 0, 0, 0}, l1 = u32x4{0, 0, 0, 0};
          ex[r][1] = 0;
          if (have1) {
            h1 = *(LDS_AS const u32x4*)(r1 + 16 * g);
            l1 = *(LDS_AS const u32x4*)(r1 + 32 + 16 * g);
            ex[r][1] = *(LDS_AS const int*)(r1 + 64);
          }
          ahi[r] = i32x8{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
          alo[r] = i32x8{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
          for (int r8 = 0; r8 < 4; ++r8) {
            i32x2 w = i32x2{0, 0};
            if (r8 < 2 || have1)
              w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(tile_buf(i - 1, r8 >> 1) + f8_vaddr(r8, nb)));
            vb8[nb][2 * r8] = w[0];
            vb8[nb][2 * r8 + 1] = w[1];
          }
        }
      }
      sched_fence();
      if (next) {
        issue_part(i + 1, 0);
        issue_part(i + 1, 1);
      }
      sched_fence();
      int sa[2][2];             // [row group][hi, lo]: this lane's A scales (tile g)
      if (have0) {
        // rare: a tile's reference differs from the step's, its P' is rescaled
#pragma unroll
        for (int r = 0; r < 2; ++r) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (sp[r][t] && pf[r][t] != 1.0f) {
              // (a tile that drops below 2^-112 of the reference contributes nothing)
              bool zero = !(pf[r][t] > 0.0f);
              if (!zero) {
                ex[r][t] += f8_rescale(ahi[r], alo[r], t, pf[r][t]);
                zero = ex[r][t] < -120;
              }
              if (zero) {
#pragma unroll
                for (int w = 4 * t; w < 4 * t + 4; ++w) ahi[r][w] = alo[r][w] = 0;
                ex[r][t] = 0;
              }
            }
          }
          const int e = g == 0 ? ex[r][0] : ex[r][1];   // in [-120, 8]
          sa[r][0] = 127 + e;
          sa[r][1] = 123 + e;
        }
      }
      sched_fence();
      if (next) issue_part(i + 1, 2);
      lds_barrier();            // mid-step
      if (have0) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            o[r][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ahi[r], vb8[nb], o[r][nb], 0, 0, 0,
                                                                       sa[r][0], 0, 127);
            o[r][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(alo[r], vb8[nb], o[r][nb], 0, 0, 0,
                                                                       sa[r][1], 0, 127);
          }
        }
      }
    } else if constexpr (NG == 1) {
      VFrag vr0, vr1;
      PRaw pr0[2], pr1[2];
      f16x8 pa0[2][2], pa1[2][2], vb[2][4];
      if (have0) {
        fetch_v(i - 1, 0, vr0);
        fetch_p(i - 1, 0, pr0);
      }
      if (have1) {
        fetch_v(i - 1, 1, vr1);
        fetch_p(i - 1, 1, pr1);
      }
      // the first two parts of the next step's loads go out while the tile
      // reads are in flight, the third at the end of the phase
      sched_fence();
      if (next) {
        issue_part(i + 1, 0);
        issue_part(i + 1, 1);
      }
      sched_fence();
      // (the second tile's V is widened in phase 2: registers)
      if (have0) {
        prep_p(pr0, {pf[0][0], pf[1][0]}, {sp[0][0], sp[1][0]}, pa0);
        widen_v(vr0, vb);
      }
      if (have1) prep_p(pr1, {pf[0][1], pf[1][1]}, {sp[0][1], sp[1][1]}, pa1);
      sched_fence();
      if (next) issue_part(i + 1, 2);
      lds_barrier();            // mid-step
      if (have0) mma_tile(pa0, vb);
      if (have1) {
        widen_v(vr1, vb);
        mma_tile(pa1, vb);
      }
    } else {
      // the group-scale variant has no registers to hold both tiles: one tile
      // per phase
      VFrag vr;
      PRaw pr[2];
      if (have0) {
        fetch_v(i - 1, 0, vr);
        fetch_p(i - 1, 0, pr);
        sched_fence();
        compute_tile_g(i - 1, 0, vr, pr, {pf[0][0], pf[1][0]});
      }
      lds_barrier();            // mid-step
      if (have1) {
        fetch_v(i - 1, 1, vr);
        fetch_p(i - 1, 1, pr);
        sched_fence();
        compute_tile_g(i - 1, 1, vr, pr, {pf[0][1], pf[1][1]});
      }
    }
    wait_vmcnt<0>();          // this wave's loads of step i + 1 have landed
    lds_barrier();            // end of step
  }
  __syncthreads();             // the score waves' (m, l) are in the stats

  // O / (2^(c2 (m0 - mO)) l0 + 2^(c2 (m1 - mO)) l1) per row, mO >= m0, m1
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int rg = 2 * rgp + r;
    if (rg >= a.row_groups) break;      // the pair's second group does not exist
    LDS_AS const float* st = stats(r);
    LDS_AS const float* mol = mo_lds + r * kRows;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const f32x4 m0 = *(LDS_AS const f32x4*)(st + 0 * kRows + 8 * qq + 4 * g);
      const f32x4 m1 = *(LDS_AS const f32x4*)(st + 1 * kRows + 8 * qq + 4 * g);
      const f32x4 l0 = *(LDS_AS const f32x4*)(st + 2 * kRows + 8 * qq + 4 * g);
      const f32x4 l1 = *(LDS_AS const f32x4*)(st + 3 * kRows + 8 * qq + 4 * g);
      const f32x4 mo = *(LDS_AS const f32x4*)(mol + 8 * qq + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float Lt = (m0[e] == kNegInf ? 0.0f : exp2_fast((m0[e] - mo[e]) * c2) * l0[e]) +
                         (m1[e] == kNegInf ? 0.0f : exp2_fast((m1[e] - mo[e]) * c2) * l1[e]);
        const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
#pragma unroll
        for (int nl = 0; nl < 4; ++nl) o[r][nl][4 * qq + e] *= inv;
      }
    }
    // Rows leave through LDS: the MFMA layout gives a lane one column of 16
    // rows; the transposed copy lets each lane store 16 contiguous bytes.  Each
    // value wave uses its own slice of the (now idle) tile buffers.
    LDS_AS float* const ep = (LDS_AS float*)(L0 + LY::kTiles) + sub * kEpSlice;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
#pragma unroll
      for (int nl = 0; nl < 4; ++nl) ep[tile_key(rr, g) * kEpStride + 32 * nl + n] = o[r][nl][rr];
    if (nsplit_eff == 1) {
      // final rows: out[b, i, h, 128 vq4 + c], 8 columns (16 bytes of bf16) per lane, 4 rows per pass
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int rl = 4 * k + (lane >> 4);
        const int c8 = 8 * (lane & 15);
        const int row = rg * kRows + rl;
        const f32x4 v0 = *(LDS_AS const f32x4*)(ep + rl * kEpStride + c8);
        const f32x4 v1 = *(LDS_AS const f32x4*)(ep + rl * kEpStride + c8 + 4);
        if (row < rows_total) {
          u32x4 packed;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            packed[j] = (uint32_t)f32_to_bf16_bits(v0[2 * j]) | ((uint32_t)f32_to_bf16_bits(v0[2 * j + 1]) << 16);
            packed[2 + j] = (uint32_t)f32_to_bf16_bits(v1[2 * j]) | ((uint32_t)f32_to_bf16_bits(v1[2 * j + 1]) << 16);
          }
          *(u32x4*)(a.out + (row_base + row) * kVDim + 128 * vq4 + c8) = packed;
        }
      }
    } else {
      const size_t pidx = ((size_t)b * a.row_groups + rg) * a.num_splits + split;
      float* po = a.ws_o + pidx * kRows * kVDim + 128 * vq4;
      // 4 columns (16 bytes) per lane, 2 rows per pass; device-scope stores
      // that the merge workgroups read (split_merge.h)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int rl = 2 * k + g;
        split_merge::store_dev(po, 4 * (rl * kVDim + 4 * n), *(LDS_AS const f32x4*)(ep + rl * kEpStride + 4 * n));
      }
      if (vq4 == 0 && g == 0) {
        // the row's log2-sum-exp: c2 mO + log2(L)
        const float m0 = st[n], m1 = st[kRows + n], mo = mol[n];
        const float Lt = (m0 == kNegInf ? 0.0f : exp2_fast((m0 - mo) * c2) * st[2 * kRows + n]) +
                         (m1 == kNegInf ? 0.0f : exp2_fast((m1 - mo) * c2) * st[3 * kRows + n]);
        split_merge::store_dev(a.ws_lse + pidx * kRows, 4 * n, Lt > 0.0f ? mo * c2 + __log2f(Lt) : kNegInf);
      }
    }
  }
  if (nsplit_eff > 1) split_merge::signal_partials(a, b, rgp, split, sub, lane);   // (each value wave)
}

// ---------------------------------------------------------------- resolve (debug)
__global__ void mla_resolve_kernel(const uint32_t* lt, const uint32_t* slt, const uint32_t* cache_lengths,
                                   int batch, int max_pages, int page_size, int max_tokens,
                                   uint32_t* page, uint32_t* slot, uint32_t* spage) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch || t >= max_tokens) return;
  const size_t o = (size_t)b * max_tokens + t;
  // tokens past what the table row can address are not resolved (as in decode)
  if ((uint32_t)t < min(cache_lengths[b], (uint32_t)max_pages * (uint32_t)page_size)) {
    const PageRef r = resolve_token(lt, slt, max_pages, b, (uint32_t)t, (uint32_t)page_size);
    page[o] = r.page;
    slot[o] = r.slot;
    spage[o] = r.spage;
  } else {
    page[o] = 0xffffffffu;
    slot[o] = 0xffffffffu;
    spage[o] = 0xffffffffu;
  }
}

// ---------------------------------------------------------------- host launchers
size_t partial_bytes(int64_t batch, int64_t row_groups, int64_t num_splits) {
  if (num_splits <= 1) return 0;
  const size_t units = (size_t)batch * (size_t)row_groups * (size_t)num_splits;
  return kFlagBytes + units * kRows * kVDim * sizeof(float) + units * kRows * sizeof(float);
}

// Merge grid: units (request, row group, chunk of wave blocks); a chunk is
// the most 8-row x 64-column wave blocks per workgroup (a power of two up to
// half a row group) that still gives about one merge workgroup per compute
// unit.  A workgroup's waves take several blocks each when the chunk holds
// more blocks than waves, or split the key splits of one block when it holds
// fewer (split_merge.h).
int plan_merge(DecodeArgs& a, int dgrid) {
  a.dgrid = dgrid;
  a.merge_nwb = 1;
  if (a.num_splits <= 1) return 0;
  int cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0) cus = c;
  }
  const int64_t groups = (int64_t)a.batch * a.row_groups;
  // as many wave blocks per workgroup as keep about one merge workgroup per
  // compute unit (every merge workgroup holds a whole compute unit, the
  // launch's LDS, so a larger grid queues behind itself), at most
  // kMaxChunkBlocks: a wave merges its blocks one after the other
  int nwb = split_merge::kMaxChunkBlocks;
  while (nwb > 1 && groups * (split_merge::kWaveBlocks / nwb) < cus) nwb >>= 1;
  a.merge_nwb = nwb;
  const int64_t units = groups * (split_merge::kWaveBlocks / nwb);
  return (int)(8 * ((units + 7) / 8));
}

template <int NG, bool kRecord, bool kF8 = false>
static hipError_t launch_main(const DecodeArgs& a, hipStream_t stream, hipEvent_t begin, hipEvent_t end) {
  static bool attr_set = false;   // per process; the attribute is per function
  const int lds_bytes = Layout<NG, kF8>::kTotal;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mla_decode_kernel<NG, kRecord, kF8>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  DecodeArgs args = a;
  const int grid = decode_grid(a) + plan_merge(args, decode_grid(a));
  if (begin && end) {
    // the events take the kernel's own start / end timestamps
    hipExtLaunchKernelGGL((mla_decode_kernel<NG, kRecord, kF8>), dim3(grid), dim3(kThreads), lds_bytes, stream,
                          begin, end, 0, args);
  } else {
    hipLaunchKernelGGL((mla_decode_kernel<NG, kRecord, kF8>), dim3(grid), dim3(kThreads), lds_bytes, stream, args);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int scale_groups, hipStream_t stream,
                         hipEvent_t main_begin, hipEvent_t main_end) {
  hipError_t e;
  const bool both = main_begin && main_end;
  if (main_begin && !both && (e = hipEventRecord(main_begin, stream)) != hipSuccess) return e;
  if (a.dbg_offsets)
    e = scale_groups == 1 ? launch_main<1, true>(a, stream, main_begin, main_end)
                          : launch_main<9, true>(a, stream, main_begin, main_end);
  else if (scale_groups == 1 && a.fp8_mfma == 2)
    e = launch_decode_rf(a, stream, main_begin, main_end);
  else if (scale_groups == 1 && a.fp8_mfma == 1)
    e = launch_main<1, false, true>(a, stream, main_begin, main_end);
  else
    e = scale_groups == 1 ? launch_main<1, false>(a, stream, main_begin, main_end)
                          : launch_main<9, false>(a, stream, main_begin, main_end);
  if (e != hipSuccess) return e;
  if (main_end && !both && (e = hipEventRecord(main_end, stream)) != hipSuccess) return e;
  return e;
}

hipError_t launch_resolve(const uint32_t* lt, const uint32_t* slt, const uint32_t* cache_lengths,
                          int batch, int max_pages, int page_size, int max_tokens,
                          uint32_t* page, uint32_t* slot, uint32_t* spage, hipStream_t stream) {
  dim3 grid((max_tokens + 255) / 256, batch);
  hipLaunchKernelGGL(mla_resolve_kernel, grid, dim3(256), 0, stream, lt, slt, cache_lengths, batch,
                     max_pages, page_size, max_tokens, page, slot, spage);
  return hipGetLastError();
}

}  // namespace mla
