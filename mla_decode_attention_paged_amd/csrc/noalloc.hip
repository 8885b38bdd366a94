// mla_decode_paged_fp8_noalloc: the decode entry point for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The split partials live in a file-scope
// device array instead of a caller-given workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_internal.h"

namespace {

// Split-partial scratch for mla_decode_paged_fp8_noalloc, one copy per GPU the
// library runs on, held until the process ends.  Its name is a host-side
// stand-in in host code: the device address comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};     // device address of `scratch` per device id

// The scratch's device address on the current device (resolved once per
// device, with that device current).  Returns null and sets *err on failure.
void* scratch_address(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" size_t mla_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" mla_status mla_decode_paged_fp8_noalloc(const void* q, const void* blocks, const float* scales,
                                                   const uint32_t* lookup_table,
                                                   const uint32_t* scales_lookup_table,
                                                   const uint32_t* cache_lengths, int32_t layer_idx,
                                                   int32_t q_len, float softmax_scale, void* out,
                                                   const mla_shape* shape, int32_t num_splits,
                                                   hipStream_t stream) {
  // Every host check before any HIP call: the arguments, then the plan's
  // partials against the scratch (an explicit split count whose partials
  // exceed it is rejected; the automatic plan is limited to it).
  mla_status st = mla::check_decode_args(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                                         layer_idx, q_len, softmax_scale, out, shape, num_splits);
  if (st != MLA_OK) return st;
  size_t need = 0;
  st = mla::plan_workspace(shape, q_len, num_splits, kScratchBytes, &need);
  if (st != MLA_OK) return st;
  if (need > kScratchBytes) return MLA_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ws = scratch_address(&e);
  if (!ws) return MLA_ERR_HIP;
  return mla::decode_with_workspace(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths,
                                    layer_idx, q_len, softmax_scale, out, shape, ws, kScratchBytes,
                                    num_splits, stream);
}
