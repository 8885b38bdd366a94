// gfx950 kernel: append the latent rows of new tokens to the paged FP8 cache,
// quantising each to E4M3FN codes with float32 scales.
//
// This is the write side of the storage the decode kernel reads
// ("generic_get_paged_cache_with_scales" page, section "Args"): token t of
// request b goes to blocks[LT[b, t / P], 0, layer, t % P, 0, :] and its scales
// to scales[SLT[b, t / P], 0, layer, t % P, 0, :] (SLT = LT when the scales
// table is absent); the scales are Float32, one per token or per 64-wide group
// ("KVCacheScalesMHAOperand" page).  The quantisation: per group, s = amax / 448
// in float32, code = the E4M3FN value nearest to clip(x / s, -448, 448) (ties
// to the even code); a group with amax = 0 gets s = 0 and codes 0.
//
// One wave per new row: lane l holds elements l + 64k (k = 0..8), so group k of
// a 64-wide granularity is one column of the wave, and every load and store of
// a column is 64 consecutive elements.  HBM-bound; the work per row is a few
// hundred VALU instructions.
#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kAppendWaves = 4;    // rows per workgroup

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// E4M3FN code of v, |v| <= 448, round to nearest with ties to even.  Written
// from the format: for |v| >= 2^-6 (normal), v = m * 2^(e - 3) with m in
// [8, 16) is rounded to an integer m (a tie goes to the even m, which is the
// even code); m = 16 carries into the exponent.  Below 2^-6 the grid is
// uniform with step 2^-9, and the code is round(|v| * 2^9) (the boundary value
// 8 is the first normal code, so both forms meet).
__device__ __forceinline__ uint32_t e4m3fn_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);                 // exact scaling, RNE
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // floor(log2 a)
    uint32_t m = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));   // in [8, 16]
    int ee = e;
    if (m == 16u) { m = 8u; ++ee; }
    mag = ((uint32_t)(ee + 7) << 3) | (m - 8u);
  }
  return sign | mag;
}

template <int NG>
__global__ void __launch_bounds__(64 * kAppendWaves) mla_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  if (row >= a.batch * a.q_len) return;
  // The row's values, its cache length and its table entries are loaded with
  // no branch between them, so that the loads overlap; a token without a
  // table entry (or with a page id past the tensors) writes nothing.
  const uint16_t* src = a.kv_new + (size_t)row * kHeadDim;
  uint16_t xb[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) xb[k] = src[lane + 64 * k];
  const int b = row / a.q_len;
  const int i = row - b * a.q_len;
  const int64_t t = (int64_t)a.cache_lengths[b] - a.q_len + i;
  const bool in_table = t >= 0 && t < (int64_t)a.max_pages * a.page_size;
  const uint32_t tc = in_table ? (uint32_t)t : 0u;                   // < max_pages * page_size
  const uint32_t col = tc / (uint32_t)a.page_size;
  const uint32_t slot = tc - col * (uint32_t)a.page_size;
  const size_t tix = (size_t)b * a.max_pages + col;
  const uint32_t page = a.lt[tix];
  const uint32_t spage = a.slt[tix];
  const bool write = in_table && page < (uint32_t)a.num_blocks && spage < (uint32_t)a.num_scale_blocks;
  __builtin_amdgcn_sched_barrier(0);   // (the table loads go out before any wait for the row)
  float x[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) x[k] = __uint_as_float((uint32_t)xb[k] << 16);   // bf16 -> fp32, exact

  float s[9];
  if constexpr (NG == 1) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 9; ++k) m = fmaxf(m, fabsf(x[k]));
    m = wave_max(m);
    const float sc = __fdiv_rn(m, 448.0f);
#pragma unroll
    for (int k = 0; k < 9; ++k) s[k] = sc;
  } else {
#pragma unroll
    for (int k = 0; k < 9; ++k) s[k] = __fdiv_rn(wave_max(fabsf(x[k])), 448.0f);
  }

  uint32_t code[9];
#pragma unroll
  for (int k = 0; k < 9; ++k)
    code[k] = s[k] > 0.0f ? e4m3fn_rne(fminf(fmaxf(__fdiv_rn(x[k], s[k]), -448.0f), 448.0f)) : 0u;
  if (!write) return;
  uint8_t* dst = a.blocks + (size_t)page * a.page_stride + a.layer_offset + (size_t)slot * kHeadDim;
#pragma unroll
  for (int k = 0; k < 9; ++k) dst[lane + 64 * k] = (uint8_t)code[k];
  float* sdst = a.scales + (size_t)spage * a.spage_stride + a.slayer_offset + (size_t)slot * NG;
#pragma unroll
  for (int k = 0; k < NG; ++k)
    if (lane == k) sdst[k] = s[k];
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int scale_groups, hipStream_t stream) {
  const int rows = a.batch * a.q_len;
  const dim3 grid((rows + kAppendWaves - 1) / kAppendWaves);
  if (scale_groups == 1)
    hipLaunchKernelGGL(mla_append_kernel<1>, grid, dim3(64 * kAppendWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(mla_append_kernel<9>, grid, dim3(64 * kAppendWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
