// C-ABI layer: argument validation (host only, before any HIP call), the work
// plan (row groups x key splits), workspace sizing, and the launches.
#include <math.h>
#include <mutex>
#include <vector>

#include "../../include/mla_paged.h"
#include "mla_internal.h"

namespace {

using mla::kRows;
using mla::kSplitQuantum;

// Number of compute units of the current device (cached per device id).
int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

mla_status check_shape(const mla_shape* s, int32_t q_len) {
  if (!s) return MLA_ERR_NULL;
  if (s->batch <= 0 || s->num_q_heads <= 0 || s->head_dim <= 0 || s->v_dim <= 0 ||
      s->num_blocks <= 0 || s->kv_dim <= 0 || s->num_layers <= 0 || s->page_size <= 0 ||
      s->num_kv_heads <= 0 || s->num_scale_blocks <= 0 || s->scale_groups <= 0 ||
      s->max_pages <= 0)
    return MLA_ERR_SHAPE;
  if (s->head_dim % s->scale_groups != 0) return MLA_ERR_SHAPE;   // granularity must divide head_dim
  if (s->v_dim > s->head_dim) return MLA_ERR_SHAPE;
  if (q_len <= 0) return MLA_ERR_RANGE;
  if (s->head_dim != mla::kHeadDim || s->v_dim != mla::kVDim || s->num_kv_heads != 1)
    return MLA_ERR_UNSUPPORTED;
  if (s->scale_groups != 1 && s->scale_groups != 9) return MLA_ERR_UNSUPPORTED;
  if (s->page_size % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)q_len * s->num_q_heads > 65536) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)s->max_pages * s->page_size > (int64_t)1 << 30) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// Split plan.  Work units are (request, pair of row groups, key split); the number of
// splits is the smallest that gives about one workgroup per compute unit and
// keeps every split within kMaxSplitKeys, capped so that each split keeps at
// least one 128-key chunk, and limited by the workspace the caller provided.
// Batches of more than kSplitFlagPairs (request, row-group pair) units are not
// split, splits are at most kMaxSplits and (units x splits) at most
// kSplitFlagEntries (an explicit split count beyond these is refused; one
// beyond kMaxSplits is clamped).
mla_status make_plan(const mla_shape* s, int32_t q_len, int32_t want_splits, size_t ws_limit,
                     bool ws_limited, mla_plan* p) {
  const int64_t rows = (int64_t)q_len * s->num_q_heads;
  const int64_t rg = (rows + kRows - 1) / kRows;
  const int64_t max_keys = (int64_t)s->max_pages * s->page_size;
  const int64_t chunks = (max_keys + kSplitQuantum - 1) / kSplitQuantum;
  const int64_t units = (int64_t)s->batch * ((rg + 1) / 2);   // one workgroup per row-group pair
  int64_t splits;
  if (want_splits > 0) {
    splits = want_splits < chunks ? want_splits : chunks;
    if (splits > mla::kMaxSplits) splits = mla::kMaxSplits;
    // the split merge keeps completion words per (request, row-group pair)
    // and per (request, row-group pair, split)
    if (splits > 1 && (units > mla::kSplitFlagPairs || units * splits > mla::kSplitFlagEntries))
      return MLA_ERR_UNSUPPORTED;
  } else {
    const int64_t target = device_cu_count();
    splits = units >= target ? 1 : (target + units - 1) / units;
    // Many requests: their lengths usually differ, and two waves of
    // workgroups dealt largest-first (the kernels' device-side order) keep
    // the compute units busier than one wave sized for the longest request,
    // provided the splits stay long (at least kMinWaveSplitKeys keys, so
    // that per-workgroup fixed costs stay small).  With equal lengths the
    // second wave only adds those fixed costs, hence the rule is kept to
    // batches of 32 requests or more; smaller batches keep one wave.
    if (s->batch >= 32 && units < target) {
      const int64_t s2 = (2 * target + units - 1) / units;
      if ((max_keys + s2 - 1) / s2 >= mla::kMinWaveSplitKeys && s->batch <= mla::kLptMaxBatch) splits = s2;
    }
    // Long requests spread over several workgroups only while the units alone
    // would fill the device less than twice over: with more units the
    // largest-first order balances the compute units, and splitting would
    // only add partials and the merge (measured: 4 % slower on 128 requests
    // x 2048..32768 keys, q_len 4).
    const int64_t min_splits = (max_keys + mla::kMaxSplitKeys - 1) / mla::kMaxSplitKeys;
    if (splits < min_splits && units < 2 * target) splits = min_splits;
    if (splits > chunks) splits = chunks;
    // so many (request, row-group pair) units fill the device many times over
    // without splitting, and the split merge has completion words for at
    // most kSplitFlagPairs pairs and kSplitFlagEntries (pair, split) units
    if (splits > mla::kMaxSplits) splits = mla::kMaxSplits;
    if (units > mla::kSplitFlagPairs) splits = 1;
    while (splits > 1 && units * splits > mla::kSplitFlagEntries) --splits;
    if (ws_limited) {
      while (splits > 1 && mla::partial_bytes(s->batch, rg, splits) > ws_limit) --splits;
    }
  }
  if (splits < 1) splits = 1;
  const int64_t chunks_per_split = (chunks + splits - 1) / splits;
  splits = (chunks + chunks_per_split - 1) / chunks_per_split;   // drop empty tails
  const int64_t grid_units = units * splits;
  if (grid_units > ((int64_t)1 << 30)) return MLA_ERR_UNSUPPORTED;
  p->row_groups = (int32_t)rg;
  p->num_splits = (int32_t)splits;
  p->tokens_per_split = (int32_t)(chunks_per_split * kSplitQuantum);
  p->grid = (int32_t)(8 * ((grid_units + 7) / 8));
  p->workspace_bytes = mla::partial_bytes(s->batch, rg, splits);
  return MLA_OK;
}

// The kernels move q, cache rows, outputs and partials in 16-byte pieces and
// scales, tables and lengths in 4-byte ones.
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shape check of an unquantized (bf16) cache: the scale fields do not apply.
mla_status check_shape_unquantized(const mla_shape* s, int32_t q_len) {
  if (!s) return MLA_ERR_NULL;
  mla_shape t = *s;
  t.num_scale_blocks = 1;
  t.scale_groups = 1;
  return check_shape(&t, q_len);
}

// Pointers, sizes, ranges and alignment of a decode call (host only).
mla_status check_args(const void* q, const void* blocks, const float* scales, const uint32_t* lookup_table,
                      const uint32_t* scales_lookup_table, const uint32_t* cache_lengths, int32_t layer_idx,
                      int32_t q_len, float softmax_scale, const void* out, const mla_shape* shape,
                      int32_t num_splits, bool unquantized) {
  if (!q || !blocks || (!unquantized && !scales) || !lookup_table || !cache_lengths || !out || !shape)
    return MLA_ERR_NULL;
  mla_status st = unquantized ? check_shape_unquantized(shape, q_len) : check_shape(shape, q_len);
  if (st != MLA_OK) return st;
  if (layer_idx < 0 || layer_idx >= shape->num_layers) return MLA_ERR_RANGE;
  if (num_splits < 0) return MLA_ERR_RANGE;
  if (!isfinite(softmax_scale) || softmax_scale <= 0.0f) return MLA_ERR_RANGE;
  if (!aligned(q, 16) || !aligned(blocks, 16) || !aligned(out, 16) ||
      (!unquantized && !aligned(scales, 4)) || !aligned(lookup_table, 4) ||
      (scales_lookup_table && !aligned(scales_lookup_table, 4)) || !aligned(cache_lengths, 4))
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// unquantized: blocks hold bf16 rows and there are no scales (scales and
// scales_lookup_table are ignored).
mla_status decode_impl(const void* q, const void* blocks, const float* scales,
                       const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                       const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                       float softmax_scale, void* out, const mla_shape* shape, void* workspace,
                       size_t workspace_bytes, int32_t num_splits, bool explicit_splits,
                       hipStream_t stream, hipEvent_t main_begin = nullptr,
                       hipEvent_t main_end = nullptr, bool unquantized = false,
                       uint64_t* dbg_offsets = nullptr, int32_t dbg_blocks = 0,
                       const uint32_t* q_offsets = nullptr, int fp8_mfma = 0) {
  mla_status st = check_args(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx,
                             q_len, softmax_scale, out, shape, num_splits, unquantized);
  if (st != MLA_OK) return st;
  if (!aligned(workspace, 16)) return MLA_ERR_UNSUPPORTED;
  if (q_offsets && !aligned(q_offsets, 4)) return MLA_ERR_UNSUPPORTED;

  mla_plan plan;
  if (explicit_splits && num_splits > 0) {
    st = make_plan(shape, q_len, num_splits, 0, false, &plan);
    if (st != MLA_OK) return st;
    if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
      return MLA_ERR_WORKSPACE;
  } else {
    const bool limited = true;
    const size_t limit = workspace ? workspace_bytes : 0;
    st = make_plan(shape, q_len, 0, limit, limited, &plan);
    if (st != MLA_OK) return st;
  }

  mla::DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.q_offsets = q_offsets;
  a.blocks = (const uint8_t*)blocks;
  a.scales = unquantized ? nullptr : scales;
  a.lt = lookup_table;
  a.slt = (!unquantized && scales_lookup_table) ? scales_lookup_table : lookup_table;
  a.cache_lengths = cache_lengths;
  a.out = (uint16_t*)out;
  const size_t units = (size_t)shape->batch * plan.row_groups * plan.num_splits;
  // workspace: completion counters, then partial O, then partial lse
  a.ws_flags = plan.num_splits > 1 ? (uint32_t*)workspace : nullptr;
  a.ws_o = plan.num_splits > 1 ? (float*)((char*)workspace + mla::kFlagBytes) : nullptr;
  a.ws_lse = plan.num_splits > 1 ? a.ws_o + units * kRows * mla::kVDim : nullptr;
  const int64_t P = shape->page_size;
  const int64_t elem = unquantized ? 2 : 1;     // bytes per cached element
  a.page_stride = (int64_t)shape->kv_dim * shape->num_layers * P * shape->head_dim * elem;
  a.layer_offset = (int64_t)layer_idx * P * shape->head_dim * elem;
  if (!unquantized) {
    a.spage_stride = (int64_t)shape->kv_dim * shape->num_layers * P * shape->scale_groups;
    a.slayer_offset = (int64_t)layer_idx * P * shape->scale_groups;
  }
  a.batch = shape->batch;
  a.q_len = q_len;
  a.num_heads = shape->num_q_heads;
  a.max_pages = shape->max_pages;
  a.page_size = shape->page_size;
  a.row_groups = plan.row_groups;
  a.num_splits = plan.num_splits;
  a.tokens_per_split = plan.tokens_per_split;
  a.grid_units = (int32_t)((size_t)shape->batch * ((plan.row_groups + 1) / 2) * plan.num_splits);
  // largest key ranges first when the workgroups come in more than one wave
  a.lpt = (shape->batch > 1 && shape->batch <= mla::kLptMaxBatch &&
           (int64_t)shape->batch * plan.num_splits < 65536 && a.grid_units > device_cu_count()) ? 1 : 0;
  a.sm_log2 = softmax_scale * 1.4426950408889634f;
  if (fp8_mfma) {
    if (unquantized || shape->scale_groups != 1) return MLA_ERR_UNSUPPORTED;
    a.fp8_mfma = fp8_mfma;
  }
  if (dbg_offsets) {
    // one record per 16-key block the table width can address
    if ((int64_t)dbg_blocks * 16 < (int64_t)shape->max_pages * shape->page_size) return MLA_ERR_SHAPE;
    if (!aligned(dbg_offsets, 8)) return MLA_ERR_UNSUPPORTED;
    a.dbg_offsets = dbg_offsets;
    a.dbg_blocks = dbg_blocks;
  }

  hipError_t e = unquantized ? mla::launch_decode_bf16(a, stream, main_begin, main_end)
                             : mla::launch_decode(a, shape->scale_groups, stream, main_begin, main_end);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

namespace mla {
// The decode entry with an explicit workspace, for the entry points defined in
// other source files of the library (noalloc.hip).
mla_status decode_with_workspace(const void* q, const void* blocks, const float* scales,
                                 const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                                 const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                                 float softmax_scale, void* out, const mla_shape* shape, void* workspace,
                                 size_t workspace_bytes, int32_t num_splits, hipStream_t stream) {
  return decode_impl(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx,
                     q_len, softmax_scale, out, shape, workspace, workspace_bytes, num_splits,
                     num_splits > 0, stream);
}

mla_status check_decode_args(const void* q, const void* blocks, const float* scales,
                             const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                             const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                             float softmax_scale, const void* out, const mla_shape* shape,
                             int32_t num_splits) {
  return check_args(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx, q_len,
                    softmax_scale, out, shape, num_splits, false);
}

// Workspace bytes the plan for these sizes needs (0: unsplit), or a status.
mla_status plan_workspace(const mla_shape* shape, int32_t q_len, int32_t num_splits, size_t ws_limit,
                          size_t* bytes) {
  mla_plan p;
  mla_status st = check_shape(shape, q_len);
  if (st != MLA_OK) return st;
  if (num_splits < 0) return MLA_ERR_RANGE;
  st = make_plan(shape, q_len, num_splits, ws_limit, num_splits == 0, &p);
  if (st != MLA_OK) return st;
  *bytes = p.workspace_bytes;
  return MLA_OK;
}
}  // namespace mla

extern "C" {

mla_status mla_decode_paged_fp8(const void* q, const void* blocks, const float* scales,
                                const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                                const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                                float softmax_scale, void* out, const mla_shape* shape,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx,
                     q_len, softmax_scale, out, shape, workspace, workspace_bytes, 0, false, stream);
}

mla_status mla_decode_paged_fp8_splits(const void* q, const void* blocks, const float* scales,
                                       const uint32_t* lookup_table,
                                       const uint32_t* scales_lookup_table,
                                       const uint32_t* cache_lengths, int32_t layer_idx,
                                       int32_t q_len, float softmax_scale, void* out,
                                       const mla_shape* shape, void* workspace,
                                       size_t workspace_bytes, int32_t num_splits,
                                       hipStream_t stream) {
  return decode_impl(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx,
                     q_len, softmax_scale, out, shape, workspace, workspace_bytes, num_splits, true,
                     stream);
}

mla_status mla_decode_paged_fp8_profiled(const void* q, const void* blocks, const float* scales,
                                         const uint32_t* lookup_table,
                                         const uint32_t* scales_lookup_table,
                                         const uint32_t* cache_lengths, int32_t layer_idx,
                                         int32_t q_len, float softmax_scale, void* out,
                                         const mla_shape* shape, void* workspace,
                                         size_t workspace_bytes, int32_t num_splits,
                                         hipEvent_t main_begin, hipEvent_t main_end,
                                         hipStream_t stream) {
  return decode_impl(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx,
                     q_len, softmax_scale, out, shape, workspace, workspace_bytes, num_splits,
                     num_splits > 0, stream, main_begin, main_end);
}

mla_status mla_decode_paged_fp8_ragged(const void* q, const uint32_t* q_offsets, const void* blocks,
                                       const float* scales, const uint32_t* lookup_table,
                                       const uint32_t* scales_lookup_table, const uint32_t* cache_lengths,
                                       int32_t layer_idx, int32_t max_q_len, float softmax_scale, void* out,
                                       const mla_shape* shape, void* workspace, size_t workspace_bytes,
                                       int32_t num_splits, hipStream_t stream) {
  if (!q_offsets) return MLA_ERR_NULL;
  return decode_impl(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx,
                     max_q_len, softmax_scale, out, shape, workspace, workspace_bytes, num_splits,
                     num_splits > 0, stream, nullptr, nullptr, false, nullptr, 0, q_offsets);
}

mla_status mla_decode_paged_fp8_mfma8(const void* q, const void* blocks, const float* scales,
                                      const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                                      const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                                      float softmax_scale, void* out, const mla_shape* shape, void* workspace,
                                      size_t workspace_bytes, int32_t num_splits, hipEvent_t main_begin,
                                      hipEvent_t main_end, hipStream_t stream) {
  return decode_impl(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx,
                     q_len, softmax_scale, out, shape, workspace, workspace_bytes, num_splits,
                     num_splits > 0, stream, main_begin, main_end, false, nullptr, 0, nullptr, 1);
}

mla_status mla_decode_paged_fp8_mfma8_kv(const void* q, const void* blocks, const float* scales,
                                         const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                                         const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                                         float softmax_scale, void* out, const mla_shape* shape, void* workspace,
                                         size_t workspace_bytes, int32_t num_splits, hipEvent_t main_begin,
                                         hipEvent_t main_end, hipStream_t stream) {
  return decode_impl(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx,
                     q_len, softmax_scale, out, shape, workspace, workspace_bytes, num_splits,
                     num_splits > 0, stream, main_begin, main_end, false, nullptr, 0, nullptr, 2);
}

mla_status mla_decode_paged_fp8_block_offsets(const void* q, const void* blocks, const float* scales,
                                              const uint32_t* lookup_table,
                                              const uint32_t* scales_lookup_table,
                                              const uint32_t* cache_lengths, int32_t layer_idx,
                                              int32_t q_len, float softmax_scale, void* out,
                                              const mla_shape* shape, void* workspace,
                                              size_t workspace_bytes, int32_t num_splits,
                                              uint64_t* block_offsets, int32_t max_blocks,
                                              hipStream_t stream) {
  if (!block_offsets) return MLA_ERR_NULL;
  if (max_blocks <= 0) return MLA_ERR_SHAPE;
  return decode_impl(q, blocks, scales, lookup_table, scales_lookup_table, cache_lengths, layer_idx,
                     q_len, softmax_scale, out, shape, workspace, workspace_bytes, num_splits,
                     num_splits > 0, stream, nullptr, nullptr, false, block_offsets, max_blocks);
}

mla_status mla_decode_paged_bf16(const void* q, const void* blocks, const uint32_t* lookup_table,
                                 const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                                 float softmax_scale, void* out, const mla_shape* shape,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(q, blocks, nullptr, lookup_table, nullptr, cache_lengths, layer_idx, q_len,
                     softmax_scale, out, shape, workspace, workspace_bytes, 0, false, stream, nullptr,
                     nullptr, true);
}

mla_status mla_decode_paged_bf16_profiled(const void* q, const void* blocks,
                                          const uint32_t* lookup_table, const uint32_t* cache_lengths,
                                          int32_t layer_idx, int32_t q_len, float softmax_scale,
                                          void* out, const mla_shape* shape, void* workspace,
                                          size_t workspace_bytes, int32_t num_splits,
                                          hipEvent_t main_begin, hipEvent_t main_end,
                                          hipStream_t stream) {
  return decode_impl(q, blocks, nullptr, lookup_table, nullptr, cache_lengths, layer_idx, q_len,
                     softmax_scale, out, shape, workspace, workspace_bytes, num_splits,
                     num_splits > 0, stream, main_begin, main_end, true);
}

mla_status mla_append_kv_fp8(const void* kv_new, void* blocks, float* scales,
                             const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                             const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                             const mla_shape* shape, hipStream_t stream) {
  if (!kv_new || !blocks || !scales || !lookup_table || !cache_lengths || !shape) return MLA_ERR_NULL;
  mla_status st = check_shape(shape, q_len);
  if (st != MLA_OK) return st;
  if (layer_idx < 0 || layer_idx >= shape->num_layers) return MLA_ERR_RANGE;
  if ((int64_t)shape->batch * q_len > ((int64_t)1 << 30)) return MLA_ERR_UNSUPPORTED;
  mla::AppendArgs a{};
  a.kv_new = (const uint16_t*)kv_new;
  a.blocks = (uint8_t*)blocks;
  a.scales = scales;
  a.lt = lookup_table;
  a.slt = scales_lookup_table ? scales_lookup_table : lookup_table;
  a.cache_lengths = cache_lengths;
  const int64_t P = shape->page_size;
  a.page_stride = (int64_t)shape->kv_dim * shape->num_layers * P * shape->head_dim;
  a.layer_offset = (int64_t)layer_idx * P * shape->head_dim;
  a.spage_stride = (int64_t)shape->kv_dim * shape->num_layers * P * shape->scale_groups;
  a.slayer_offset = (int64_t)layer_idx * P * shape->scale_groups;
  a.num_blocks = shape->num_blocks;
  a.num_scale_blocks = shape->num_scale_blocks;
  a.batch = shape->batch;
  a.q_len = q_len;
  a.max_pages = shape->max_pages;
  a.page_size = shape->page_size;
  hipError_t e = mla::launch_append(a, shape->scale_groups, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_paged_fp8_plan(const mla_shape* shape, int32_t q_len, int32_t num_splits,
                                     mla_plan* plan) {
  if (!shape || !plan) return MLA_ERR_NULL;
  mla_status st = check_shape(shape, q_len);
  if (st != MLA_OK) return st;
  if (num_splits < 0) return MLA_ERR_RANGE;
  return make_plan(shape, q_len, num_splits, 0, false, plan);
}

mla_status mla_resolve_pages(const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                             const uint32_t* cache_lengths, int32_t batch, int32_t max_pages,
                             int32_t page_size, int32_t max_tokens, uint32_t* page, uint32_t* slot,
                             uint32_t* spage, hipStream_t stream) {
  if (!lookup_table || !cache_lengths || !page || !slot || !spage) return MLA_ERR_NULL;
  if (batch <= 0 || max_pages <= 0 || page_size <= 0 || max_tokens <= 0) return MLA_ERR_SHAPE;
  if (batch > 65535) return MLA_ERR_UNSUPPORTED;
  hipError_t e = mla::launch_resolve(lookup_table, scales_lookup_table ? scales_lookup_table : lookup_table,
                                     cache_lengths, batch, max_pages, page_size, max_tokens, page,
                                     slot, spage, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

const char* mla_status_string(mla_status status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer argument is NULL";
    case MLA_ERR_SHAPE: return "inconsistent or non-positive sizes";
    case MLA_ERR_RANGE: return "layer_idx, q_len, num_splits or softmax_scale out of range";
    case MLA_ERR_UNSUPPORTED: return "sizes not served by these kernels";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small for the requested split plan";
    case MLA_ERR_HIP: return "HIP runtime call or kernel launch failed";
  }
  return "unknown status";
}

int32_t mla_abi_version(void) { return MLA_PAGED_ABI_VERSION; }

}  // extern "C"
