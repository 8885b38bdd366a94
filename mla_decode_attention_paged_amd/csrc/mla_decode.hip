// gfx950 kernels: MLA decode over a paged FP8 (E4M3FN) latent cache with
// separately stored float32 scales.
//
// Storage follows the "generic_get_paged_cache_with_scales" page (section
// "Args": blocks / scales tensors, lookup_table, optional scales_lookup_table,
// cache_lengths) and the "KVCacheScalesMHAOperand" page (per-token Float32
// scales kept in the scales field).  The "KVLoad2CvtProducer" page describes a
// Blackwell pipeline that stages FP8 KV tiles in shared memory and converts
// them to a 16-bit type for the tensor cores; on CDNA4 the same idea becomes:
//
//   * one workgroup = 4 waves on one group of 32 query rows (q position, head);
//     each wave streams its own 32-key tiles through a private, double-buffered
//     LDS tile filled by direct global->LDS dwordx4 loads (no VGPR staging);
//   * S^T = K Q^T on v_mfma_f32_32x32x16_f16: FP8 bytes are widened to f16
//     exactly in registers (scale 1.0 conversion); q (bf16) is held in f16,
//     which is exact for 2^-14 <= |q| <= 65504; the fp32 scale is applied to
//     score columns (one scale per key) or per 64-deep group partial sums;
//   * softmax in fp32, base 2, against a per-wave reference max taken from the
//     wave's first tile: the accumulators are never rescaled (no VALU touches
//     them in the loop, so they stay in AGPRs); P' may exceed 1, and a wave
//     whose P' overflowed f16 repeats its keys once against the exact max;
//   * O = P' V on the same MFMA, with P' = f16(p * scale) and V read from the
//     same LDS tile through ds_read_b64_tr_b8 (8 keys of one column per lane);
//   * the 4 waves merge (m, l, O) through LDS; a workgroup either writes the
//     final bf16 rows or, when a request's keys are split across workgroups,
//     an fp32 partial (O / l, log2-sum-exp) merged by mla_combine.
#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mla {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
// Read-only kernel inputs read at wave-uniform addresses (page tables, cache
// lengths) go through the constant address space, so they become scalar loads.
#define CONST_AS __attribute__((address_space(4)))

constexpr int kTileBytes = kTile * kHeadDim;   // 18432: one 32-key FP8 tile
constexpr float kNegInf = -__builtin_inff();

template <int NG>
struct Layout {
  // scales per tile in LDS: NG == 1 -> 64 floats (lanes 32..63 load duplicates),
  // NG == 9 -> [group][key] 9 x 32 floats plus a 32-float tail for the last load.
  static constexpr int kScaleBytes = NG == 1 ? 256 : 1280;
  static constexpr int kWaveBytes = 2 * kTileBytes + 2 * kScaleBytes + 128;   // + row-factor scratch
  static constexpr int kTotal = kWaves * kWaveBytes;
};
static_assert(Layout<9>::kTotal <= 160 * 1024, "LDS budget");

// ---------------------------------------------------------------- page resolution
// Token t of request b: value page = LT[b, t / P], slot = t % P, scale page =
// SLT[b, t / P] (SLT is LT when no separate table was given).  Shared by the
// decode kernel's tile addressing and by the resolve debug kernel.
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
__device__ __forceinline__ void lds_dma4(const void* gsrc, LDS_AS void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, ldst, 4, 0, 0);
}

// Key position (within a 32-key tile) held by accumulator register r of an
// S^T = K Q^T 32x32 MFMA result, for lane half g = lane / 32.
__device__ __forceinline__ constexpr int tile_key(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// ---------------------------------------------------------------- the decode kernel
template <int NG>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
mla_decode_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  using LY = Layout<NG>;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 5;          // lane half
  const int n = lane & 31;          // MFMA column / row within the half

  // ---- XCD-aware unit mapping: consecutive units (the row groups of one key
  // range) land on the same XCD and are dispatched back to back there.
  const int per_xcd = (a.grid_units + 7) >> 3;
  const int unit = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (unit >= a.grid_units) return;
  const int rg = unit % a.row_groups;
  const int bs = unit / a.row_groups;
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
  const int t_lo = split * T;
  const int t_hi = min(L, t_lo + T);

  const int rows_total = a.q_len * a.num_heads;

  // ---- per-lane row bookkeeping (S^T layout: lane column n is row rg*32 + n)
  const int my_row = rg * kRows + n;
  const bool row_ok = my_row < rows_total;
  const int my_i = row_ok ? my_row / a.num_heads : 0;
  // keys visible to this row: j < L - Q + i + 1, clipped to this split
  int lim = row_ok ? min(L - a.q_len + my_i + 1, t_hi) : t_hi;
  // the earliest limit over the wave's real rows decides whether a tile needs masking
  int lim_min = row_ok ? lim : 0x7fffffff;
  for (int off = 16; off >= 1; off >>= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off));
  lim_min = __builtin_amdgcn_readfirstlane(min(lim_min, __shfl_xor(lim_min, 32)));

  // ---- Q fragments (B operand of S^T = K Q^T), f16, held for the whole key range.
  // k-step s = 2u + v covers depth d = 32u + 16g + 8v + e, e < 8.
  f16x8 qf[36];
  {
    const uint16_t* qrow = a.q + (size_t)(row_ok ? my_row : 0) * kHeadDim + (size_t)b * rows_total * kHeadDim;
#pragma unroll
    for (int u = 0; u < 18; ++u) {
      const u32x4 w0 = *(const u32x4*)(qrow + 32 * u + 16 * g);
      const u32x4 w1 = *(const u32x4*)(qrow + 32 * u + 16 * g + 8);
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const u32x4 w = v ? w1 : w0;
        f16x8 f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = bf16_bits_to_f32(w[k] & 0xffffu);
          const float hi = bf16_bits_to_f32(w[k] >> 16);
          f[2 * k] = row_ok ? (_Float16)lo : (_Float16)0.0f;
          f[2 * k + 1] = row_ok ? (_Float16)hi : (_Float16)0.0f;
        }
        qf[2 * u + v] = f;
      }
    }
  }

  // ---- LDS regions of this wave (address space 3, 32-bit addressing)
  LDS_AS char* const lds0 = (LDS_AS char*)lds;
  LDS_AS char* const wbase = lds0 + wave * LY::kWaveBytes;

  // Global->LDS tile layout: 18 blocks of 1 KiB, block i = 9*(key/16) + col/64;
  // inside a block, 16-byte slot 4*(key%16) + ((c%4) ^ ((key%16)/4 % 4)) holds
  // bytes [16c, 16c+16) of that key, c = 16-byte column index.  The XOR spreads
  // the 16 keys of an MFMA read over all LDS banks.
  const int ld_key = lane >> 2;                                   // key % 16 loaded by this lane
  const int ld_col = (lane & 3) ^ ((lane >> 4) & 3);              // 16B column % 4 loaded by this lane
  const uint32_t ld_off = (uint32_t)ld_key * kHeadDim + 16u * ld_col;   // + 64*(col/4) per block

  // K read (A operand): lane (key n, half g) reads 16B column c = 2u + g
  const uint32_t kread[2] = {
      (uint32_t)(1024 * 9 * (n >> 4) + 16 * (4 * (n & 15) + ((0 + g) ^ ((n >> 2) & 3)))),
      (uint32_t)(1024 * 9 * (n >> 4) + 16 * (4 * (n & 15) + ((2 + g) ^ ((n >> 2) & 3))))};
  // V read (B operand via transpose read): provider lane p = 2k + h of each 16-lane
  // group addresses key tau(g,k) = 4g + (k&3) + 8(k>>2) at column 32nb + 16q + 8h.
  const int vq = (lane >> 4) & 1, vk = (lane & 15) >> 1, vh = lane & 1;
  const int vtau = 4 * g + (vk & 3) + 8 * (vk >> 2);
  const uint32_t vread[2] = {
      (uint32_t)(16 * (4 * vtau + ((0 + vq) ^ ((vtau >> 2) & 3))) + 8 * vh),
      (uint32_t)(16 * (4 * vtau + ((2 + vq) ^ ((vtau >> 2) & 3))) + 8 * vh)};

  const uint8_t* layer_base = a.blocks + a.layer_offset;
  const float* slayer_base = a.scales + a.slayer_offset;

  // Issue the global->LDS loads of the tile starting at key t0 into buffer `buf`.
  // Keys at or past t_hi are never read: their lanes re-load the last valid key
  // (finite data that the softmax masks out), so stale or NaN-holding slots,
  // pages and table columns past a request's length stay untouched.
  auto issue_tile = [&](int t0, int buf) __attribute__((always_inline)) {
    const int nvalid = min(kTile, t_hi - t0);     // >= 1
    // pages of the two 16-key halves (a 16-key half never crosses a page)
    const PageRef p0 = resolve_token(lt, slt, a.max_pages, b, (uint32_t)t0, (uint32_t)a.page_size);
    const uint8_t* rb0 = layer_base + (size_t)p0.page * (size_t)a.page_stride + (size_t)p0.slot * kHeadDim;
    const float* sb0 = slayer_base + (size_t)p0.spage * (size_t)a.spage_stride + (size_t)p0.slot * NG;
    const uint8_t* rb1 = rb0;
    const float* sb1 = sb0;
    if (nvalid > 16) {
      const PageRef p1 = resolve_token(lt, slt, a.max_pages, b, (uint32_t)(t0 + 16), (uint32_t)a.page_size);
      rb1 = layer_base + (size_t)p1.page * (size_t)a.page_stride + (size_t)p1.slot * kHeadDim;
      sb1 = slayer_base + (size_t)p1.spage * (size_t)a.spage_stride + (size_t)p1.slot * NG;
    }
    LDS_AS char* dst = wbase + buf * kTileBytes;
    if (nvalid == kTile) {
#pragma unroll
      for (int i = 0; i < 18; ++i) {
        const uint8_t* src = (i < 9 ? rb0 : rb1) + 64 * (i % 9) + ld_off;
        lds_dma16(src, dst + 1024 * i);
      }
    } else {
      const int kmax0 = min(nvalid, 16) - 1;
      const uint32_t off0 = (uint32_t)min(ld_key, kmax0) * kHeadDim + 16u * ld_col;
      const uint8_t* base1 = nvalid > 16 ? rb1 : rb0 + kmax0 * kHeadDim;
      const uint32_t off1 = (uint32_t)min(ld_key, max(nvalid - 17, 0)) * kHeadDim + 16u * ld_col;
#pragma unroll
      for (int i = 0; i < 18; ++i) {
        const uint8_t* src = (i < 9 ? rb0 + off0 : base1 + off1) + 64 * (i % 9);
        lds_dma16(src, dst + 1024 * i);
      }
    }
    LDS_AS char* sdst = wbase + 2 * kTileBytes + buf * LY::kScaleBytes;
    const int key = min(lane & 31, nvalid - 1);
    const float* srow = (key < 16 ? sb0 : sb1) + (key & 15) * NG;
    if constexpr (NG == 1) {
      lds_dma4(srow, sdst);
    } else {
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int grp = min(2 * i + (lane >> 5), NG - 1);
        lds_dma4(srow + grp, sdst + 256 * i);
      }
    }
  };

  // ---- running state
  f32x16 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x16{};
  // Reference max per row (S^T layout: lane column n; same value in both halves).
  // It is fixed from the wave's first tile and never moved inside the loop, so
  // the accumulators O are never rescaled: P' = f16(2^(x - m_ref) * scale) may
  // exceed 1, which costs no precision in f16; only its overflow matters, and
  // that case is caught after the pass (see the key loop).
  float m_ref = kNegInf;
  float l_part = 0.0f;       // this lane's share of the row sum (keys of its half)

  const int ntiles = (t_hi - t_lo + kTile - 1) / kTile;
  const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  const int t_first = t_lo + kTile * wave;

  // Per-key scales of the keys this lane holds in the S^T layout (NG == 1).
  auto key_scales = [&](LDS_AS const char* sb, float (&sv16)[16]) __attribute__((always_inline)) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const f32x4 sv = *(LDS_AS const f32x4*)((LDS_AS const float*)sb + 8 * qq + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) sv16[4 * qq + e] = sv[e];
    }
  };
  // Scales of group gv ([group][key] layout) for the keys this lane holds (NG == 9).
  auto group_scales = [&](LDS_AS const char* sb, int gv, float (&sv16)[16]) __attribute__((always_inline)) {
    LDS_AS const float* sg = (LDS_AS const float*)sb + 32 * gv;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const f32x4 sv = *(LDS_AS const f32x4*)(sg + 8 * qq + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) sv16[4 * qq + e] = sv[e];
    }
  };
  // Scores of one tile in the log2 domain (masked keys = -inf) and their row max.
  auto tile_scores = [&](LDS_AS const char* tb, LDS_AS const char* sb, int t0, float (&x)[16])
      __attribute__((always_inline)) -> float {
    f32x16 s = f32x16{};
    if constexpr (NG == 1) {
#pragma unroll
      for (int u = 0; u < 18; ++u) {
        const u32x4 kr = *(LDS_AS const u32x4*)(tb + kread[u & 1] + 1024 * (u >> 1));
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(fp8x8_to_f16(kr[0], kr[1]), qf[2 * u], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(fp8x8_to_f16(kr[2], kr[3]), qf[2 * u + 1], s, 0, 0, 0);
        if (u & 1) sched_fence();
      }
      float sv16[16];
      key_scales(sb, sv16);
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (s[r] * sv16[r]) * a.sm_log2;
    } else {
      // one 64-deep scale group = 16-byte columns 4gi..4gi+3 = u in {2gi, 2gi+1}
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        f32x16 t = f32x16{};
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          const int u = 2 * gi + uu;
          const u32x4 kr = *(LDS_AS const u32x4*)(tb + kread[u & 1] + 1024 * (u >> 1));
          t = __builtin_amdgcn_mfma_f32_32x32x16_f16(fp8x8_to_f16(kr[0], kr[1]), qf[2 * u], t, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_32x32x16_f16(fp8x8_to_f16(kr[2], kr[3]), qf[2 * u + 1], t, 0, 0, 0);
        }
        float sv16[16];
        group_scales(sb, gi, sv16);
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_fmaf(sv16[r], t[r], s[r]);
        sched_fence();
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s[r] * a.sm_log2;
    }
    if (t0 + kTile > lim_min) {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (t0 + tile_key(r, g) < lim) ? x[r] : kNegInf;
    }
    float mt = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
    sched_fence();
    return halves_max(mt);
  };

  // Probabilities, row sums, and O += P' V for one tile (P' = f16(p * scale)).
  auto finish_tile = [&](LDS_AS const char* tb, LDS_AS const char* sb, const float (&x)[16])
      __attribute__((always_inline)) {
    const float m_use = m_ref == kNegInf ? 0.0f : m_ref;
    float p[16];
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = exp2_fast(x[r] - m_use);
      psum += p[r];
    }
    l_part += psum;

    if constexpr (NG == 1) {
      float sv16[16];
      key_scales(sb, sv16);
      f16x8 pa[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) pa[hh][e] = (_Float16)(p[8 * hh + e] * sv16[8 * hh + e]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
          const i32x2 vr = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (LDS_AS i32x2*)(tb + vread[nb & 1] + 1024 * (9 * hh + (nb >> 1))));
          o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              pa[hh], fp8x8_to_f16((uint32_t)vr[0], (uint32_t)vr[1]), o[nb], 0, 0, 0);
          if ((nb & 3) == 3) sched_fence();
        }
      }
    } else {
      // value group gv = columns [64gv, 64gv + 64) = output blocks nb = 2gv, 2gv+1
#pragma unroll
      for (int gv = 0; gv < 8; ++gv) {
        float sv16[16];
        group_scales(sb, gv, sv16);
        f16x8 pa[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 8; ++e) pa[hh][e] = (_Float16)(p[8 * hh + e] * sv16[8 * hh + e]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) {
            const int nb = 2 * gv + nn;
            const i32x2 vr = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (LDS_AS i32x2*)(tb + vread[nb & 1] + 1024 * (9 * hh + (nb >> 1))));
            o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                pa[hh], fp8x8_to_f16((uint32_t)vr[0], (uint32_t)vr[1]), o[nb], 0, 0, 0);
          }
        }
        sched_fence();
      }
    }
  };

  // ---- the key loop.  Tile k of this wave starts at t_first + 128k; tile k+1's
  // loads are in flight while tile k is computed.  Tiles run in chunks of
  // kChunk against a reference max that is fixed inside a chunk (no VALU
  // touches O in the tile loop); between chunks, if the running max moved, O
  // and the row sums are rescaled once.  P' <= 2^(m_seen - m_ref) * (largest
  // scale loaded); if that bound passes 2^15 within a chunk, the wave repeats
  // its keys once from zero against the exact max, which it keeps tracking.
  constexpr int kChunk = 4;
  LDS_AS float* const alpha_buf = (LDS_AS float*)(wbase + 2 * kTileBytes + 2 * LY::kScaleBytes);
  float m_all = kNegInf;       // running max over every tile seen (exact at the end)
  for (int pass = 0; pass < 2; ++pass) {
    bool overflow = false;
    if (my_tiles > 0) issue_tile(t_first, 0);
    for (int c0 = 0; c0 < my_tiles; c0 += kChunk) {
      const int c1 = min(my_tiles, c0 + kChunk);
      float m_seen = kNegInf;
      float s_seen = 0.0f;     // largest scale this lane loaded in the chunk (its DMA slots)
      for (int k = c0; k < c1; ++k) {
        const int buf = k & 1;
        const int t0 = t_first + kTile * kWaves * k;
        if (k + 1 < my_tiles) {
          issue_tile(t0 + kTile * kWaves, buf ^ 1);
          if constexpr (NG == 1) wait_vmcnt<19>();   // this tile's loads; the next tile's stay in flight
          else wait_vmcnt<23>();
        } else {
          wait_vmcnt<0>();
        }
        LDS_AS const char* tb = wbase + buf * kTileBytes;
        LDS_AS const char* sb = wbase + 2 * kTileBytes + buf * LY::kScaleBytes;

        float x[16];
        const float mt = tile_scores(tb, sb, t0, x);
        m_seen = fmaxf(m_seen, mt);
        if (k == 0 && pass == 0) m_ref = mt;
        LDS_AS const float* sf = (LDS_AS const float*)sb;
        s_seen = fmaxf(s_seen, sf[lane]);
        if constexpr (NG == 9) {
#pragma unroll
          for (int i = 1; i < 5; ++i) s_seen = fmaxf(s_seen, sf[64 * i + lane]);
        }
        finish_tile(tb, sb, x);
      }
      m_all = fmaxf(m_all, m_seen);
      if (pass == 0) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) s_seen = fmaxf(s_seen, __shfl_xor(s_seen, off));
        const bool risky = m_seen != kNegInf && (m_seen - m_ref) + __log2f(s_seen) > 15.0f;
        if (wave_any(risky)) {
          overflow = true;
          // finish the remaining scores only to learn the exact max
          wait_vmcnt<0>();
          for (int j = c1; j < my_tiles; ++j) {
            const int tj = t_first + kTile * kWaves * j;
            issue_tile(tj, 0);
            wait_vmcnt<0>();
            float xj[16];
            m_all = fmaxf(m_all, tile_scores(wbase, wbase + 2 * kTileBytes, tj, xj));
          }
          break;
        }
      }
      if (c1 < my_tiles && wave_any(m_seen > m_ref)) {
        // move the reference to the running max: O and l scale by 2^(m_ref - m_new)
        const float m_new = fmaxf(m_ref, m_seen);
        const float alpha = m_ref == kNegInf ? 0.0f : exp2_fast(m_ref - m_new);
        l_part *= alpha;
        m_ref = m_new;
        alpha_buf[n] = alpha;      // both halves hold the same value for row n
        wait_lgkmcnt0();
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const f32x4 av = *(LDS_AS const f32x4*)(alpha_buf + 8 * qq + 4 * g);
#pragma unroll
          for (int nb = 0; nb < 16; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[nb][4 * qq + e] *= av[e];
        }
      }
    }
    if (!overflow) break;
    m_ref = m_all;
    l_part = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = f32x16{};
  }

  // ================================================================ merge the 4 waves
  const float l_row = halves_sum(l_part);

  __syncthreads();    // every wave is done with its tiles; LDS is free
  LDS_AS float* const st_m = (LDS_AS float*)lds0;     // [4][32] running max per wave and row
  LDS_AS float* const st_l = st_m + kWaves * kRows;   // [4][32] row sum per wave and row
  if (g == 0) {
    st_m[wave * kRows + n] = m_ref;
    st_l[wave * kRows + n] = l_row;
  }
  __syncthreads();

  // Scale this wave's O rows (PV layout: row 8(r/4) + 4g + r%4) by
  // 2^(m_w - M) / L_total so that the 4 waves' O sum to the result.
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    f32x4 mw[kWaves], lw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = *(LDS_AS const f32x4*)(st_m + w * kRows + 8 * qq + 4 * g);
      lw[w] = *(LDS_AS const f32x4*)(st_l + w * kRows + 8 * qq + 4 * g);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float M = mw[0][e];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[w][e]);
      float Lt = 0.0f, fself = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = mw[w][e] == kNegInf ? 0.0f : exp2_fast(mw[w][e] - M);
        Lt += f * lw[w][e];
        fself = w == wave ? f : fself;
      }
      const float fo = Lt > 0.0f ? fself / Lt : 0.0f;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) o[nb][4 * qq + e] *= fo;
    }
  }
  // the row's log2-sum-exp (S^T layout row n) for split partials
  float lse_row = kNegInf;
  {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st_m[w * kRows + n]);
    float Lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = st_m[w * kRows + n];
      Lt += mw == kNegInf ? 0.0f : exp2_fast(mw - M) * st_l[w * kRows + n];
    }
    lse_row = Lt > 0.0f ? M + __log2f(Lt) : kNegInf;
  }

  // tree sum through LDS: [nb][r][lane] fp32 images, 64 KiB per wave
  LDS_AS float* const red0 = (LDS_AS float*)(lds0 + 1024);
  LDS_AS float* const red1 = red0 + 16 * 16 * 64;
  auto put = [&](LDS_AS float* dst, int nb_lo, int nb_hi) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 16; ++nb)
      if (nb >= nb_lo && nb < nb_hi)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(nb * 16 + r) * 64 + lane] = o[nb][r];
  };
  auto add = [&](LDS_AS const float* src, int nb_lo, int nb_hi) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 16; ++nb)
      if (nb >= nb_lo && nb < nb_hi)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nb][r] += src[(nb * 16 + r) * 64 + lane];
  };
  __syncthreads();
  if (wave == 2) put(red0, 0, 16);
  if (wave == 3) put(red1, 0, 16);
  __syncthreads();
  if (wave == 0) add(red0, 0, 16);
  if (wave == 1) add(red1, 0, 16);
  __syncthreads();
  if (wave == 0) put(red0, 8, 16);
  if (wave == 1) put(red1, 0, 8);
  __syncthreads();
  if (wave == 0) add(red1, 0, 8);
  if (wave == 1) add(red0, 8, 16);
  if (wave >= 2) return;
  const int nb_lo = wave == 0 ? 0 : 8;

  if (nsplit_eff == 1) {
    // final rows: out[b, i, h, 32nb + n]
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rg * kRows + tile_key(r, g);
      if (row < rows_total) {
        uint16_t* orow = a.out + ((size_t)b * rows_total + row) * kVDim;
#pragma unroll
        for (int nb = 0; nb < 16; ++nb)
          if (nb >= nb_lo && nb < nb_lo + 8) orow[32 * nb + n] = f32_to_bf16_bits(o[nb][r]);
      }
    }
  } else {
    const size_t pidx = ((size_t)b * a.row_groups + rg) * a.num_splits + split;
    float* po = a.ws_o + pidx * kRows * kVDim;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float* prow = po + tile_key(r, g) * kVDim;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb)
        if (nb >= nb_lo && nb < nb_lo + 8) prow[32 * nb + n] = o[nb][r];
    }
    if (wave == 0 && g == 0) a.ws_lse[pidx * kRows + n] = lse_row;
  }
}

// ---------------------------------------------------------------- split combine
// out = sum_s 2^(lse_s - lse) O_s with lse = log2 sum_s 2^lse_s, per row.
// One workgroup per (request, row group, 64-column chunk); a thread owns one
// row and 8 columns.
constexpr int kCombineChunks = kVDim / 64;       // 8
constexpr int kCombineThreads = kRows * 8;       // 256

__global__ void __launch_bounds__(kCombineThreads) mla_combine_kernel(DecodeArgs a) {
  const int chunk = blockIdx.x % kCombineChunks;
  const int brg = blockIdx.x / kCombineChunks;
  const int b = brg / a.row_groups;
  const int rg = brg % a.row_groups;
  const int L = (int)min(((const CONST_AS uint32_t*)a.cache_lengths)[b],
                         (uint32_t)a.max_pages * (uint32_t)a.page_size);
  const int T = a.tokens_per_split;
  const int nsplit_eff = L <= 0 ? 1 : (L + T - 1) / T;
  if (nsplit_eff <= 1) return;
  const int rows_total = a.q_len * a.num_heads;
  const int rl = threadIdx.x >> 3;                          // row within the group
  const int col0 = chunk * 64 + (threadIdx.x & 7) * 8;      // 8 columns per thread
  const int row = rg * kRows + rl;
  if (row >= rows_total) return;

  const size_t pbase = ((size_t)b * a.row_groups + rg) * a.num_splits;
  float M = kNegInf;
  for (int s = 0; s < nsplit_eff; ++s) M = fmaxf(M, a.ws_lse[(pbase + s) * kRows + rl]);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  float W = 0.0f;
  if (M != kNegInf) {
    for (int s = 0; s < nsplit_eff; ++s) {
      const float ls = a.ws_lse[(pbase + s) * kRows + rl];
      if (ls == kNegInf) continue;
      const float w = exp2_fast(ls - M);
      W += w;
      const f32x4* src = (const f32x4*)(a.ws_o + ((pbase + s) * kRows + rl) * kVDim + col0);
      const f32x4 v0 = src[0], v1 = src[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = __builtin_fmaf(w, v0[j], acc[j]);
        acc[4 + j] = __builtin_fmaf(w, v1[j], acc[4 + j]);
      }
    }
  }
  const float inv = W > 0.0f ? 1.0f / W : 0.0f;
  uint16_t* orow = a.out + ((size_t)b * rows_total + row) * kVDim + col0;
  u32x4 packed;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    packed[j] = (uint32_t)f32_to_bf16_bits(acc[2 * j] * inv) | ((uint32_t)f32_to_bf16_bits(acc[2 * j + 1] * inv) << 16);
  *(u32x4*)orow = packed;
}

// ---------------------------------------------------------------- resolve (debug)
__global__ void mla_resolve_kernel(const uint32_t* lt, const uint32_t* slt, const uint32_t* cache_lengths,
                                   int batch, int max_pages, int page_size, int max_tokens,
                                   uint32_t* page, uint32_t* slot, uint32_t* spage) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch || t >= max_tokens) return;
  const size_t o = (size_t)b * max_tokens + t;
  if ((uint32_t)t < cache_lengths[b]) {
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
  return units * kRows * kVDim * sizeof(float) + units * kRows * sizeof(float);
}

template <int NG>
static hipError_t launch_main(const DecodeArgs& a, hipStream_t stream) {
  static bool attr_set = false;   // per process; the attribute is per function
  const int lds_bytes = Layout<NG>::kTotal;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mla_decode_kernel<NG>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int per_xcd = (a.grid_units + 7) / 8;
  hipLaunchKernelGGL(mla_decode_kernel<NG>, dim3(8 * per_xcd), dim3(256), lds_bytes, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int scale_groups, hipStream_t stream,
                         hipEvent_t main_begin, hipEvent_t main_end) {
  hipError_t e;
  if (main_begin && (e = hipEventRecord(main_begin, stream)) != hipSuccess) return e;
  e = scale_groups == 1 ? launch_main<1>(a, stream) : launch_main<9>(a, stream);
  if (e != hipSuccess) return e;
  if (main_end && (e = hipEventRecord(main_end, stream)) != hipSuccess) return e;
  if (a.num_splits > 1) {
    hipLaunchKernelGGL(mla_combine_kernel, dim3(a.batch * a.row_groups * kCombineChunks), dim3(kCombineThreads),
                       0, stream, a);
    e = hipGetLastError();
  }
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
