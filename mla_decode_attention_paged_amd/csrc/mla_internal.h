// Internal interface between the C-ABI layer (api.cpp) and the gfx950 kernels
// (mla_decode.hip).  Not installed; the public interface is include/mla_paged.h.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "mla_paged.h"

namespace mla {

constexpr int kHeadDim = 576;            // latent key depth (512 value dims + 64 rope dims)
constexpr int kVDim = 512;               // value depth: the first 512 latent dims
constexpr int kTile = 32;                // keys per MFMA tile
constexpr int kRows = 32;                // query rows (q position, head) per row group
constexpr int kWaves = 4;                // waves per workgroup, each streaming its own tiles
constexpr int kSplitQuantum = kTile * kWaves;   // split lengths are multiples of this
// The plan keeps splits at most this long whenever the workspace allows, so
// that long requests spread over many workgroups (any split length decodes
// correctly).
constexpr int kMaxSplitKeys = 8192;
// Largest batch whose key ranges the decode kernels order by size on the device.
constexpr int kLptMaxBatch = 256;
// Shortest split the plan accepts when it sizes for two waves of workgroups.
constexpr int kMinWaveSplitKeys = 2048;

// Everything the main kernel needs, by value.  Offsets are precomputed on the
// host from the contiguous row-major shapes of the blocks / scales tensors.
struct DecodeArgs {
  const uint16_t* q;                 // bf16 bits [B, Q, H, 576], or [T, H, 576] with q_offsets
  const uint32_t* q_offsets;         // [B + 1] packed query rows per request, or null (Q each)
  const uint8_t* blocks;             // e4m3fn bytes
  const float* scales;
  const uint32_t* lt;                // [B, max_pages]
  const uint32_t* slt;               // scale page table; == lt when absent
  const uint32_t* cache_lengths;     // [B]
  uint16_t* out;                     // bf16 bits [B, Q, H, 512], or [T, H, 512] with q_offsets
  float* ws_o;                       // split partials O   [B, RG, S, 32, 512] (fp32)
  float* ws_lse;                     // split partials lse [B, RG, S, 32]      (log2 domain)
  uint32_t* ws_flags;                // split completion words (kFlagBytes; split_merge.h)
  int64_t page_stride;               // bytes between pages of blocks (kv_dim*num_layers*P*576)
  int64_t layer_offset;              // bytes to (kv 0, layer_idx, slot 0) inside a page
  int64_t spage_stride;              // floats between pages of scales
  int64_t slayer_offset;             // floats to (kv 0, layer_idx, slot 0) inside a scale page
  int32_t batch, q_len, num_heads, max_pages, page_size;   // q_len: the largest count with q_offsets
  int32_t row_groups, num_splits, tokens_per_split;
  int32_t grid_units;                // batch * row_groups * num_splits
  int32_t lpt;                       // 1: largest (request, split) key ranges first
  int32_t fp8_mfma;                  // per-token scales only: 1 = P'V on the FP8 MFMA (role-split
                                     // kernel), 2 = QK^T and P'V on it (mla_decode_rf.hip); 0 = neither
  int32_t dgrid;                     // decode workgroups; the merge workgroups follow them
  int32_t merge_nwb;                 // 8-row x 64-column wave blocks per merge workgroup
  float sm_log2;                     // softmax_scale * log2(e)
  // Debug record of the decode kernel's own page resolution (null in normal
  // calls): for 16-key block k of request b, [b, k, 0] = byte offset of the
  // block's first row from (page 0, kv 0, layer_idx, slot 0) and [b, k, 1] =
  // float offset of its first scale row from the same place in scales, as
  // the kernel computed them for its loads.  dbg_blocks = blocks per request.
  uint64_t* dbg_offsets;
  int32_t dbg_blocks;
};

// Workspace of a split plan: the completion counters (kFlagBytes, at the
// start, the same place for every plan, so that a workspace reused across
// shapes never finds partial data where counters go), then the partial O,
// then the partial lse.  0 when num_splits <= 1.  Split plans are limited to
// kSplitFlagPairs (request, row-group pair) units.
constexpr int64_t kSplitFlagPairs = 8192;
// ... and kSplitFlagEntries (request, row-group pair, split) units, with at
// most kMaxSplits splits per request.
constexpr int64_t kSplitFlagEntries = 65536;
constexpr int64_t kMaxSplits = 4096;
constexpr size_t kFlagBytes = (size_t)(kSplitFlagPairs + kSplitFlagEntries) * sizeof(uint32_t);   // 288 KiB
size_t partial_bytes(int64_t batch, int64_t row_groups, int64_t num_splits);

// Arguments of the append-and-quantise kernel (kv_append.hip).
struct AppendArgs {
  const uint16_t* kv_new;            // bf16 bits [B, Q, 576]: latent rows of the new tokens
  uint8_t* blocks;                   // e4m3fn bytes, written
  float* scales;                     // written
  const uint32_t* lt;                // [B, max_pages]
  const uint32_t* slt;               // scale page table; == lt when absent
  const uint32_t* cache_lengths;     // [B], the new tokens included
  int64_t page_stride, layer_offset; // bytes, as in DecodeArgs
  int64_t spage_stride, slayer_offset;   // floats, as in DecodeArgs
  int64_t num_blocks, num_scale_blocks;  // page ids at or past these are not written
  int32_t batch, q_len, max_pages, page_size;
};

hipError_t launch_append(const AppendArgs& a, int scale_groups, hipStream_t stream);

// Launch the decode kernel (with its split merge when num_splits > 1).  The
// optional events are recorded right before / after the launch.
hipError_t launch_decode(const DecodeArgs& a, int scale_groups, hipStream_t stream,
                         hipEvent_t main_begin = nullptr, hipEvent_t main_end = nullptr);

// Launch the decode with both contractions on the block-scaled FP8 MFMA
// (mla_decode_rf.hip; per-token scales), with its split merge.
hipError_t launch_decode_rf(const DecodeArgs& a, hipStream_t stream, hipEvent_t main_begin = nullptr,
                            hipEvent_t main_end = nullptr);

// Launch the unquantized (bf16 cache) decode kernel (with its split merge
// when num_splits > 1).  DecodeArgs as for the FP8 kernel with blocks holding
// bf16 rows (page_stride / layer_offset in bytes); scales and slt are unused.
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream, hipEvent_t main_begin = nullptr,
                              hipEvent_t main_end = nullptr);

// Merge workgroups to append to a decode grid (of 4- or 8-wave workgroups):
// sets a.dgrid and a.merge_nwb and returns the merge grid (0 when unsplit).
int plan_merge(DecodeArgs& a, int dgrid);

// The decode with a caller-given workspace (api.cpp), for other entry points.
mla_status decode_with_workspace(const void* q, const void* blocks, const float* scales,
                                 const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                                 const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                                 float softmax_scale, void* out, const mla_shape* shape, void* workspace,
                                 size_t workspace_bytes, int32_t num_splits, hipStream_t stream);
// Host checks of a decode call's arguments (pointers, sizes, ranges,
// alignment), as every FP8 decode entry point makes them before any HIP call.
mla_status check_decode_args(const void* q, const void* blocks, const float* scales,
                             const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                             const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                             float softmax_scale, const void* out, const mla_shape* shape,
                             int32_t num_splits);
// Workspace bytes of the plan for these sizes: the automatic plan (num_splits
// 0) limited to ws_limit bytes, or the explicit split count's (unlimited).
mla_status plan_workspace(const mla_shape* shape, int32_t q_len, int32_t num_splits, size_t ws_limit,
                          size_t* bytes);

hipError_t launch_resolve(const uint32_t* lt, const uint32_t* slt, const uint32_t* cache_lengths,
                          int batch, int max_pages, int page_size, int max_tokens,
                          uint32_t* page, uint32_t* slot, uint32_t* spage, hipStream_t stream);

}  // namespace mla
