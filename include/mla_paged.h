/*
 * mla_paged.h — C ABI of the MI355X (gfx950) paged-FP8 MLA decode library.
 *
 * The library computes multi-head latent attention (MLA) decode over a paged
 * KV cache whose latent rows are stored as FP8 E4M3FN bytes with separately
 * stored float32 scales.  The storage it reads is the one described on two
 * Modular API pages:
 *
 *   - "generic_get_paged_cache_with_scales" (Mojo function page, section
 *     "Args"): the blocks tensor [num_blocks, kv_dim, num_layers, page_size,
 *     num_heads, head_dim]; the scales tensor [num_blocks, kv_dim,
 *     num_layers, page_size, num_heads, head_dim_granularity]; the page
 *     lookup table [batch, max_pages]; per-request cache_lengths [batch];
 *     max_prompt_length (here q_len); and the optional scales lookup table
 *     [batch, max_pages] for scale pages that carry their own ids (when it
 *     is absent, scale pages resolve through the value page table).
 *   - "KVCacheScalesMHAOperand" (Mojo struct page, description and the
 *     scales_raw_ptr method): per-token K scales kept in the scales field
 *     when the quantization granularity equals the head size, as Float32.
 *
 * The attention step itself (MLA decode with a 576-deep latent key whose
 * first 512 dims are the value, FP8 KV tiles converted to a 16-bit type for
 * the tensor-core contractions) is the subject of the "KVLoad2CvtProducer"
 * page (Mojo struct page, description and "Parameters").
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major
 *     buffers with the shapes given below; the caller owns them.  The
 *     library allocates no device memory and keeps no pointer after a call
 *     returns.  The only state that outlives a call is the split completion
 *     flags at the start of a workspace, which every call returns to
 *     zero (see mla_decode_paged_fp8, workspace).
 *   - Work is enqueued asynchronously on `stream`; inputs must stay alive
 *     and unmodified until the stream has passed the call.
 *   - Arguments are validated on the host before any HIP call.  On any
 *     error nothing is launched and the outputs are untouched.
 *   - Decode entry points need q, blocks, out and the workspace 16-byte
 *     aligned and scales, tables and cache_lengths 4-byte aligned
 *     (MLA_ERR_UNSUPPORTED otherwise); device allocations are.
 *   - Device-side contract (not checked on the device): every page id read
 *     is < num_blocks (values) or < num_scale_blocks (scales); q_len <=
 *     cache_lengths[b] <= max_pages * page_size.  Table columns at or past
 *     ceil(cache_lengths[b] / page_size) are never read, so they may hold
 *     anything; so may unused slots, pages, layers and kv_dim entries.
 *   - What the C layer can and cannot check: it receives raw pointers and an
 *     mla_shape, so it validates the sizes, ranges, alignment and nullness
 *     listed per entry point, but it cannot see element types, strides or the
 *     tensors' own extents.  Element types, contiguous row-major layout, and
 *     the agreement between tensors (scales dims 1..4 == blocks dims 1..4,
 *     scales_lookup_table shape == lookup_table shape, out == [batch, q_len,
 *     num_q_heads, 512], q's second dimension == q_len) are the caller's
 *     contract; the Python binding checks them on the torch tensors before it
 *     calls.  A C caller that breaks them gets undefined results.
 */
#ifndef MLA_PAGED_H
#define MLA_PAGED_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_PAGED_ABI_VERSION 5

/* Status codes.  mla_status_string() returns a static description. */
typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer argument is NULL            */
  MLA_ERR_SHAPE = 2,       /* inconsistent or non-positive sizes             */
  MLA_ERR_RANGE = 3,       /* layer_idx / q_len / num_splits out of range    */
  MLA_ERR_UNSUPPORTED = 4, /* sizes valid but not served by these kernels    */
  MLA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required     */
  MLA_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed     */
} mla_status;

/*
 * Sizes of one call.  The tensors are contiguous row-major:
 *   q      bf16  [batch, q_len, num_q_heads, head_dim]
 *   blocks u8    [num_blocks, kv_dim, num_layers, page_size, num_kv_heads, head_dim]
 *                (OCP FP8 E4M3FN bytes; kv index 0 and kv head 0 are read)
 *   scales f32   [num_scale_blocks, kv_dim, num_layers, page_size, num_kv_heads,
 *                 scale_groups]   with scale_groups = head_dim / granularity
 *   lookup_table, scales_lookup_table  u32 [batch, max_pages]
 *   cache_lengths u32 [batch]
 *   out    bf16  [batch, q_len, num_q_heads, v_dim]
 * Served by the kernels: head_dim == 576, v_dim == 512, num_kv_heads == 1,
 * scale_groups in {1, 9} (granularity 576 or 64), page_size a positive
 * multiple of 16, num_q_heads * q_len <= 65536.
 */
typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t v_dim;
  int64_t num_blocks;
  int32_t kv_dim;
  int32_t num_layers;
  int32_t page_size;
  int32_t num_kv_heads;
  int64_t num_scale_blocks;
  int32_t scale_groups;
  int32_t max_pages;
} mla_shape;

/* Work decomposition chosen for a call (see mla_decode_paged_fp8_plan). */
typedef struct {
  int32_t row_groups;        /* ceil(q_len * num_q_heads / 32)                     */
  int32_t num_splits;        /* key-range splits per (request, row group)          */
  int32_t tokens_per_split;  /* keys per split, a multiple of 128                  */
  int32_t grid;              /* decode workgroups in request order; with more
                                workgroups than compute units (batch <= 256) the
                                kernels deal (request, split) key ranges largest
                                first and may launch up to 8 * ceil(q_len * heads / 64)
                                more, which exit at once.  With num_splits > 1 the
                                same launch adds the split-merge workgroups      */
  size_t workspace_bytes;    /* split flags (288 KiB) + partials; 0 when
                                num_splits == 1                                  */
} mla_plan;

/*
 * mla_decode_paged_fp8 — attention output of every query row over its
 * request's paged FP8 cache.
 *
 * For request b, query position i < q_len and head h:
 *   K_j[d] = e4m3fn(blocks[LT[b, j/P], 0, layer_idx, j%P, 0, d])
 *            * scales[SLT[b, j/P], 0, layer_idx, j%P, 0, d / granularity]
 *   (SLT = scales_lookup_table when non-NULL, else lookup_table)
 *   s_j    = softmax_scale * sum_{d<576} q[b,i,h,d] * K_j[d]
 *   out[b,i,h,:] = bf16( sum_j softmax(s)_j * K_j[0:512] ),
 * over keys j <= cache_lengths[b] - q_len + i (the q_len newest cached
 * tokens are the queries themselves, causal among each other).  A row with
 * no visible key yields zeros.
 *
 * workspace: device buffer for a split plan, or NULL.  With NULL (or too
 * small to hold any split plan) the call runs unsplit, which is always
 * correct.  Use mla_decode_paged_fp8_plan() to learn the size that the
 * automatic plan wants.  Layout: 288 KiB of split completion flags, then
 * the fp32 partials.  The flags must be ZERO before a buffer's first use
 * as a workspace (e.g. hipMemset once after allocating it); every call that
 * splits returns them to zero, so the same workspace serves any later call,
 * of any shape, with no clearing in between (also under graph replay).
 * Calls that share a workspace must not overlap in time (one stream, or
 * caller-side ordering); a workspace whose flags are not zero makes the
 * split merge wait (bounded, about half a second) and write NaN rows.
 * Split plans serve at most 8192 (request, row-group pair) units (larger
 * batches run unsplit), at most 4096 splits, and at most 65536 (pair,
 * split) units (the automatic plan takes fewer splits).  q values must
 * satisfy |q| <= 65504.  Scales must be finite and non-negative, at most
 * 255 with 64-wide groups (P' = f16(p * s) with p <= 2^8) and at most 2^15
 * with per-token scales (the lazy threshold keeps p * s below 2^15); larger
 * scales overflow P' to inf.
 */
mla_status mla_decode_paged_fp8(const void* q, const void* blocks, const float* scales,
                                const uint32_t* lookup_table,
                                const uint32_t* scales_lookup_table, /* nullable */
                                const uint32_t* cache_lengths, int32_t layer_idx,
                                int32_t q_len, float softmax_scale, void* out,
                                const mla_shape* shape, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Same as mla_decode_paged_fp8 with an explicit split count (0 = automatic).
 * An explicit count needs a workspace of at least plan.workspace_bytes
 * (MLA_ERR_WORKSPACE otherwise); num_splits is clamped to the number of
 * 128-key chunks of max_pages * page_size and to 4096.  A count > 1 for more
 * than 8192 (request, row-group pair) units, or whose (pair, split) units
 * exceed 65536, is refused with MLA_ERR_UNSUPPORTED. */
mla_status mla_decode_paged_fp8_splits(const void* q, const void* blocks, const float* scales,
                                       const uint32_t* lookup_table,
                                       const uint32_t* scales_lookup_table,
                                       const uint32_t* cache_lengths, int32_t layer_idx,
                                       int32_t q_len, float softmax_scale, void* out,
                                       const mla_shape* shape, void* workspace,
                                       size_t workspace_bytes, int32_t num_splits,
                                       hipStream_t stream);

/* Same as mla_decode_paged_fp8_splits, and additionally times the decode
 * launch (the one kernel, its split merge included): when both `main_begin` and `main_end`
 * (caller-created HIP events) are given, the kernel is launched with
 * hipExtLaunchKernel so that the events carry its own start and end
 * timestamps; when only one is given it is recorded on `stream` right before
 * (begin) or after (end) the kernel.  NULL events are ignored.  For callers
 * that time the main kernel on its own. */
mla_status mla_decode_paged_fp8_profiled(const void* q, const void* blocks, const float* scales,
                                         const uint32_t* lookup_table,
                                         const uint32_t* scales_lookup_table,
                                         const uint32_t* cache_lengths, int32_t layer_idx,
                                         int32_t q_len, float softmax_scale, void* out,
                                         const mla_shape* shape, void* workspace,
                                         size_t workspace_bytes, int32_t num_splits,
                                         hipEvent_t main_begin, hipEvent_t main_end,
                                         hipStream_t stream);

/*
 * mla_decode_paged_fp8_mfma8 — mla_decode_paged_fp8_profiled with the value
 * contraction (P' V) on the block-scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_
 * f8f6f4) with the key scales folded into P' ("KVLoad2CvtProducer" page,
 * Parameters: FP8 KV tiles): the V rows enter as their E4M3 codes, and
 * P' = p * key scale as two
 * E4M3 parts per element (P' = 2^e (hi + 2^-4 lo), e per query row and 32-key
 * tile, applied through the MFMA's E8M0 operand scales).  The key
 * contraction stays exact (bf16 MFMA on the widened codes).  Per-token
 * scales only (scale_groups == 1): MLA_ERR_UNSUPPORTED otherwise.  A LOSSY
 * mode: P' in two E4M3 parts keeps about 8 significant bits, so most outputs
 * are as accurate as mla_decode_paged_fp8's but some land two bf16 ulps from
 * the exact result (measured: max normalized error 1.17e-2 on one of three
 * seeds of 32 requests x 128 heads with up to 1,500 keys; mean error 2.7x
 * the default path's); a separate, opt-in entry point.  Arguments, plan,
 * workspace, events and errors as for mla_decode_paged_fp8_profiled.
 */
mla_status mla_decode_paged_fp8_mfma8(const void* q, const void* blocks, const float* scales,
                                      const uint32_t* lookup_table,
                                      const uint32_t* scales_lookup_table, /* nullable */
                                      const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                                      float softmax_scale, void* out, const mla_shape* shape,
                                      void* workspace, size_t workspace_bytes, int32_t num_splits,
                                      hipEvent_t main_begin, hipEvent_t main_end, hipStream_t stream);

/*
 * mla_decode_paged_fp8_mfma8_kv — mla_decode_paged_fp8_mfma8 with the key
 * contraction (S = q K^T) on the block-scaled FP8 MFMA too (v_mfma_scale_f32_
 * 16x16x128_f8f6f4; "KVLoad2CvtProducer" page, Parameters: FP8 KV tiles, with
 * no widening stage): the key rows enter as their E4M3 codes, q (bf16) as two
 * E4M3 parts per element with one power-of-two factor pair per query row
 * (q = 2^a (hi + 2^-t lo)), the key scales multiply the fp32 score columns,
 * and P' is split as in mla_decode_paged_fp8_mfma8 (here with one exponent
 * per query row, step of 64 keys and half of the step's keys).  Per-token
 * scales only (scale_groups == 1): MLA_ERR_UNSUPPORTED otherwise.  A LOSSY
 * mode: the FP8 MFMA's accumulation of the key contraction adds up to about
 * one bf16 ulp to the output beyond the other entry points' error (measured
 * up to two bf16 ulps against the exact result at |O| ~ 1.4), so it does not
 * meet their accuracy on every input.  Arguments, plan, workspace, events
 * and errors as for mla_decode_paged_fp8_profiled.
 */
mla_status mla_decode_paged_fp8_mfma8_kv(const void* q, const void* blocks, const float* scales,
                                         const uint32_t* lookup_table,
                                         const uint32_t* scales_lookup_table, /* nullable */
                                         const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                                         float softmax_scale, void* out, const mla_shape* shape,
                                         void* workspace, size_t workspace_bytes, int32_t num_splits,
                                         hipEvent_t main_begin, hipEvent_t main_end, hipStream_t stream);

/*
 * mla_decode_paged_fp8_ragged — mla_decode_paged_fp8_splits for requests with
 * their own query counts ("generic_get_paged_cache_with_scales" page, Args:
 * max_prompt_length is the batch's largest query length; "KVCacheScalesMHA-
 * Operand" page, create_ragged_tma_tile: ragged query rows).  The queries are
 * packed request after request:
 *   q          bf16 [T, num_q_heads, 576], T = q_offsets[batch]
 *   q_offsets  device uint32 [batch + 1], q_offsets[0] = 0, non-decreasing:
 *              request b owns q rows q_offsets[b] .. q_offsets[b + 1] - 1, its
 *              n_b = q_offsets[b + 1] - q_offsets[b] new tokens (0 allowed: no
 *              output rows; n_b <= max_q_len)
 *   max_q_len  the largest n_b (the plan is sized for it, as for q_len)
 *   out        bf16 [T, num_q_heads, 512] (written for every packed row)
 * Query i of request b sees keys j <= cache_lengths[b] - n_b + i (each request
 * causal among its own new tokens).  The other arguments, the plan
 * (mla_decode_paged_fp8_plan with q_len = max_q_len), the workspace, split
 * counts and errors are those of mla_decode_paged_fp8_splits; MLA_ERR_NULL
 * when q_offsets is NULL, MLA_ERR_UNSUPPORTED when it is not 4-byte aligned.
 * The offsets are read on the device only: offsets that break the contract
 * above give undefined results.
 */
mla_status mla_decode_paged_fp8_ragged(const void* q, const uint32_t* q_offsets, const void* blocks,
                                       const float* scales, const uint32_t* lookup_table,
                                       const uint32_t* scales_lookup_table, /* nullable */
                                       const uint32_t* cache_lengths, int32_t layer_idx,
                                       int32_t max_q_len, float softmax_scale, void* out,
                                       const mla_shape* shape, void* workspace,
                                       size_t workspace_bytes, int32_t num_splits,
                                       hipStream_t stream);

/*
 * mla_decode_paged_fp8_block_offsets — debug variant of
 * mla_decode_paged_fp8_splits that also reports the page resolution the
 * decode kernel itself computed for its loads ("generic_get_paged_cache_with_
 * scales" page, "Args": lookup_table, scales_lookup_table).  The decode runs
 * exactly as in mla_decode_paged_fp8_splits (same plan, same output); in
 * addition, for every 16-key block k (keys 16k .. 16k+15) of request b that
 * the kernel loads, it writes
 *   block_offsets[b, k, 0] = byte offset of the block's first row,
 *       LT[b, 16k / P] * page_stride + (16k % P) * head_dim
 *   block_offsets[b, k, 1] = float offset of its first scale row,
 *       SLT[b, 16k / P] * spage_stride + (16k % P) * scale_groups
 * both counted from element (page 0, kv 0, layer_idx, slot 0, head 0, 0) of
 * blocks / scales, with page_stride = kv_dim * num_layers * page_size *
 * head_dim and spage_stride = kv_dim * num_layers * page_size * scale_groups.
 * A block never straddles a page (page_size is a multiple of 16), so these
 * two numbers fix the page, slot and scale page of all its 16 keys.  Blocks
 * at or past ceil(L_b / 16) are not written.
 *   block_offsets  device u64 [batch, max_blocks, 2] (written), 8-byte aligned
 *   max_blocks     >= ceil(max_pages * page_size / 16), else MLA_ERR_SHAPE
 * Other arguments, errors and ownership as for mla_decode_paged_fp8_splits;
 * MLA_ERR_NULL when block_offsets is NULL.  For tests that check the index
 * work bit for bit; not for production calls.
 */
mla_status mla_decode_paged_fp8_block_offsets(const void* q, const void* blocks, const float* scales,
                                              const uint32_t* lookup_table,
                                              const uint32_t* scales_lookup_table,
                                              const uint32_t* cache_lengths, int32_t layer_idx,
                                              int32_t q_len, float softmax_scale, void* out,
                                              const mla_shape* shape, void* workspace,
                                              size_t workspace_bytes, int32_t num_splits,
                                              uint64_t* block_offsets, int32_t max_blocks,
                                              hipStream_t stream);

/*
 * mla_decode_paged_fp8_noalloc — mla_decode_paged_fp8 for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and result as
 * mla_decode_paged_fp8_splits without the workspace: the split partials go to
 * a device array inside the library, mla_noalloc_scratch_bytes() bytes
 * (64 MiB) per GPU, resolved on the first call on each device and held until
 * the process ends.  The call itself allocates nothing (no hipMalloc, hipFree
 * or allocating library routine).
 *   num_splits  0: the automatic plan, limited to what the scratch holds
 *               (fewer splits, or none, for very large batches); > 0: that
 *               split count, rejected with MLA_ERR_WORKSPACE when its
 *               partials (mla_decode_paged_fp8_plan's workspace_bytes)
 *               exceed the scratch.
 * Every call on one GPU uses that GPU's one scratch array: calls that overlap
 * in time on the same GPU (different streams, or host threads) race and must
 * be serialized by the caller.  The scratch needs no clearing: its split
 * flags start at zero (the array is zero-initialized when the library is
 * loaded) and every call returns them to zero, and a call writes every
 * partial it reads.  Errors as for mla_decode_paged_fp8_splits, all
 * checked on the host before any HIP call; MLA_ERR_HIP when the scratch's
 * device address cannot be obtained.
 */
mla_status mla_decode_paged_fp8_noalloc(const void* q, const void* blocks, const float* scales,
                                        const uint32_t* lookup_table,
                                        const uint32_t* scales_lookup_table,
                                        const uint32_t* cache_lengths, int32_t layer_idx,
                                        int32_t q_len, float softmax_scale, void* out,
                                        const mla_shape* shape, int32_t num_splits,
                                        hipStream_t stream);

/* Bytes of the per-GPU split scratch of mla_decode_paged_fp8_noalloc. */
size_t mla_noalloc_scratch_bytes(void);

/*
 * mla_decode_paged_bf16 — the same attention over an unquantized paged cache.
 *
 * Quantization is a property of the cache type ("KVCacheScalesMHAOperand"
 * page, the quantization_enabled alias); without it the latent rows are kept
 * as they are, in the blocks tensor of "generic_get_paged_cache_with_scales"
 * (section "Args"), here as bf16, and there are no scales:
 *   K_j[d] = blocks[LT[b, j/P], 0, layer_idx, j%P, 0, d]
 * and everything else (scores over the 576-deep row, V = K_j[0:512], the
 * causal rule for q_len > 1, empty rows -> zeros) is as for
 * mla_decode_paged_fp8.
 *
 *   q        bf16 [batch, q_len, num_q_heads, 576] (device, read)
 *   blocks   bf16 [num_blocks, kv_dim, num_layers, page_size, 1, 576] (device, read)
 *   lookup_table u32 [batch, max_pages], cache_lengths u32 [batch] (device, read)
 *   out      bf16 [batch, q_len, num_q_heads, 512] (device, written)
 *   shape    as for mla_decode_paged_fp8; num_scale_blocks and scale_groups
 *            are not used (any value)
 *   workspace / workspace_bytes: split partials, as for mla_decode_paged_fp8;
 *            the plan (and so the size) is the one mla_decode_paged_fp8_plan
 *            reports for the same shape and q_len.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_RANGE, MLA_ERR_UNSUPPORTED,
 * MLA_ERR_HIP, as for mla_decode_paged_fp8.  The probabilities enter the
 * value contraction as a sum of two bf16 numbers (about 16 significant bits).
 */
mla_status mla_decode_paged_bf16(const void* q, const void* blocks, const uint32_t* lookup_table,
                                 const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                                 float softmax_scale, void* out, const mla_shape* shape,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* mla_decode_paged_bf16 with an explicit split count (0 = automatic; an
 * explicit count needs plan.workspace_bytes of workspace) and the optional
 * kernel-timing events of mla_decode_paged_fp8_profiled (NULL = none). */
mla_status mla_decode_paged_bf16_profiled(const void* q, const void* blocks,
                                          const uint32_t* lookup_table, const uint32_t* cache_lengths,
                                          int32_t layer_idx, int32_t q_len, float softmax_scale,
                                          void* out, const mla_shape* shape, void* workspace,
                                          size_t workspace_bytes, int32_t num_splits,
                                          hipEvent_t main_begin, hipEvent_t main_end,
                                          hipStream_t stream);

/*
 * mla_append_kv_fp8 — write the latent rows of the q_len new tokens of every
 * request into the paged FP8 cache, quantised; the step before a decode call.
 * Storage as on the "generic_get_paged_cache_with_scales" page (section
 * "Args"), scale type and granularity as on the "KVCacheScalesMHAOperand"
 * page: new row i of request b is token t = cache_lengths[b] - q_len + i
 * (cache_lengths already count the new tokens, as for decode); its codes go
 * to blocks[LT[b, t / P], 0, layer_idx, t % P, 0, :] and its scales to
 * scales[SLT[b, t / P], 0, layer_idx, t % P, 0, :] (SLT = LT when NULL).
 *
 * Quantisation per granularity group (576 / scale_groups elements): s =
 * amax / 448 in float32 (correctly rounded), code = the E4M3FN value nearest
 * to clip(x / s, -448, 448) with the division correctly rounded in float32,
 * ties to the even code, the sign bit from x / s; a group whose amax is 0
 * gets s = 0 and codes 0x00.
 *
 *   kv_new        bf16 [B, q_len, 576] (device, read)
 *   blocks        E4M3FN bytes [num_blocks, kv_dim, num_layers, P, 1, 576] (written in place)
 *   scales        float32 [num_scale_blocks, kv_dim, num_layers, P, 1, scale_groups] (written in place)
 *   lookup_table, scales_lookup_table (or NULL), cache_lengths: as for decode
 *   layer_idx     layer written, 0 <= layer_idx < num_layers
 *   q_len         new tokens per request, >= 1
 *   shape         the same shape description decode takes (num_q_heads is not used but must be > 0)
 *
 * Rows with t < 0 or t >= max_pages * page_size, and rows whose page id is
 * >= num_blocks or whose scale page id is >= num_scale_blocks, are not
 * written.  Only the row's 576 code bytes and scale_groups scales are
 * written; everything else is left as it was.  Non-finite inputs are outside
 * the contract.  Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_RANGE,
 * MLA_ERR_UNSUPPORTED (as for decode), MLA_ERR_HIP (launch failed).
 */
mla_status mla_append_kv_fp8(const void* kv_new, void* blocks, float* scales,
                             const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                             const uint32_t* cache_lengths, int32_t layer_idx, int32_t q_len,
                             const mla_shape* shape, hipStream_t stream);

/* The decomposition a call with these sizes would use (host only, no HIP call
 * except a cached device-property query).  num_splits = 0 asks for the
 * automatic plan with an unlimited workspace. */
mla_status mla_decode_paged_fp8_plan(const mla_shape* shape, int32_t q_len,
                                     int32_t num_splits, mla_plan* plan);

/*
 * mla_resolve_pages — per-token view of page resolution by a small debug
 * kernel of its own (generic_get_paged_cache_with_scales page, "Args":
 * lookup_table and scales_lookup_table).  It does not run the decode
 * kernel's addressing code; mla_decode_paged_fp8_block_offsets reports that.
 * For b < batch and t < max_tokens writes
 *   page[b, t]  = LT[b, t / page_size]   slot[b, t] = t % page_size
 *   spage[b, t] = SLT[b, t / page_size]  (SLT = LT when NULL)
 * for t < min(cache_lengths[b], max_pages * page_size), and 0xFFFFFFFF in all
 * three otherwise.  Outputs are device u32 [batch, max_tokens].
 */
mla_status mla_resolve_pages(const uint32_t* lookup_table, const uint32_t* scales_lookup_table,
                             const uint32_t* cache_lengths, int32_t batch, int32_t max_pages,
                             int32_t page_size, int32_t max_tokens, uint32_t* page,
                             uint32_t* slot, uint32_t* spage, hipStream_t stream);

/* Static, human-readable description of a status code. */
const char* mla_status_string(mla_status status);

/* MLA_PAGED_ABI_VERSION of the built library. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_H */
