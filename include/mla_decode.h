/*
 * mla_decode.h — C ABI of the MI355X (gfx950) MLA paged-KV decode library.
 *
 * Operation (what every entry point computes): Multi-head Latent Attention
 * decode over a paged latent KV cache.
 *   - A cache row is 576 elements: a 512-wide latent, which is also the value
 *     vector V, followed by a 64-wide RoPE part (tokenspeed-mla package page,
 *     "Quickstart": kv_lora_rank = 512, qk_rope_head_dim = 64).
 *   - Sequence b's key j is row (j % page_size) of page
 *     block_table[b * max_pages + j / page_size] (TokenSpeed MLA article,
 *     section 6: kv_cache [num_pages, page_size, D_total] with block_tables).
 *   - Queries are [batch, q_len, num_heads, 576]; token t of q_len attends to
 *     keys j < seq_lens[b] - q_len + t + 1 (causal across the new tokens, the
 *     sequence length counting them; a row with no visible key gets O = 0 and
 *     LSE = -inf).
 *   - score = softmax_scale * (q_scale * q) . (kv_scale * k) over all 576
 *     dims; O = softmax(score) @ V (first 512 dims), written as bf16;
 *     LSE = natural log of sum exp(score), fp32.
 *   - Work is split along the KV sequence into partial (O, LSE) pieces that a
 *     second kernel merges by LSE weighting (article, section 2); query
 *     tokens are folded into the head dimension, F = the largest divisor of
 *     q_len with num_heads * F <= 128 (article, section 3).
 *
 * Conventions for every entry point:
 *   - Return 0 (MLA_OK) or a negative mla_status; mla_last_error() then holds
 *     a message for the calling thread.  Arguments are validated on the host
 *     before anything is enqueued: a failed call enqueues nothing.
 *   - Pointers documented "device" are HIP device pointers; the library never
 *     reads device memory on the host, never allocates or frees memory and
 *     never synchronises: calls enqueue on `stream` (a hipStream_t, NULL for
 *     the default stream) and return.  Faults inside kernels surface at the
 *     caller's next synchronisation.  No memset is enqueued, so calls may be
 *     captured into a HIP graph.
 *   - The caller owns every buffer.  Calls that share a workspace on streams
 *     that run concurrently race on it.
 *   - Thread-safe: the per-shape plan cache is guarded by a mutex.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_VERSION 100 /* 1.0.0 */

#define MLA_D_QK 576 /* latent 512 + rope 64 */
#define MLA_D_V 512
#define MLA_KV_LORA_RANK 512
#define MLA_QK_ROPE_HEAD_DIM 64

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_DTYPE = -2,       /* dtype code not accepted */
  MLA_ERR_SHAPE = -3,       /* a size is out of range or inconsistent */
  MLA_ERR_ALIGN = -4,       /* a device pointer is not aligned as required */
  MLA_ERR_WORKSPACE = -5,   /* workspace NULL, too small, misaligned, or planned for another shape */
  MLA_ERR_UNSUPPORTED = -6, /* valid but not implemented */
  MLA_ERR_HIP = -7,         /* a HIP runtime call failed (message names it) */
  MLA_ERR_DEVICE = -8,      /* no usable HIP device */
  MLA_ERR_STRIDE = -9       /* a tensor descriptor's strides are not the layout the kernels read */
} mla_status;

typedef enum mla_dtype {
  MLA_DTYPE_BF16 = 1,     /* bfloat16, stored as 16-bit patterns */
  MLA_DTYPE_FP8_E4M3 = 2, /* OCP FP8 E4M3 (e4m3fn): bias 7, no inf, S.1111.111 = NaN, max 448 */
  MLA_DTYPE_FP16 = 3,     /* IEEE binary16 (tokenspeed-mla package page: FP16 / BF16 / FP8 decode inputs) */
  MLA_DTYPE_BF16_Q_FP8_KV = 4 /* bf16 q over an OCP FP8 E4M3 kv_cache (the same package page's
                                 FP8 decode, with queries kept in bf16) */
} mla_dtype;

/* Sizes of one decode call.  All fields are element counts. */
typedef struct mla_shape {
  int32_t batch;       /* B >= 0 sequences */
  int32_t q_len;       /* new query tokens per sequence, >= 1 */
  int32_t num_heads;   /* H >= 1 query heads sharing the one latent KV head */
  int32_t num_pages;   /* pages in kv_cache, >= 1 */
  int32_t page_size;   /* rows per page: a power of two, 16 <= page_size <= 65536 */
  int32_t max_pages;   /* entries per block_table row (its row stride), >= 1 */
  int32_t max_seq_len; /* the length the workspace was planned for (upper bound of seq_lens);
                          0 <= max_seq_len <= max_pages * page_size */
  int32_t dtype;       /* mla_dtype of q and kv_cache (both the same, except MLA_DTYPE_BF16_Q_FP8_KV) */
} mla_shape;

/*
 * Plan a decode shape: the number of KV splits and the workspace size.
 *
 * The split count and workspace are derived from (batch, q_len, num_heads,
 * max_seq_len) and the current device's compute-unit count and cached per
 * shape, so callers never tune them (article, section 2: split_kv and the
 * workspace size are derived at run time from batch size, q_len and
 * max_seq_len, and cached).  num_splits is the number of KV slices that
 * each workgroup row's work (one query group of F folded tokens and up to 128
 * of its rows, over every sequence of the batch) is cut into; workspace_bytes
 * is what mla_decode needs for that shape (0 when no merge is needed).
 *
 * Inputs are host integers; outputs are host pointers (must be non-NULL).
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (batch < 0, q_len < 1, num_heads < 1,
 * max_seq_len < 0), MLA_ERR_DEVICE / MLA_ERR_HIP when the device cannot be
 * queried.
 */
int mla_get_split_kv_and_workspace(int32_t batch, int32_t q_len, int32_t num_heads, int32_t max_seq_len,
                                   int32_t* num_splits, size_t* workspace_bytes);

/*
 * MLA decode (the operation described at the top of this file).
 *
 *   shape       host pointer to the call's sizes.
 *   q           device, [batch, q_len, num_heads, 576] of shape->dtype (bf16 for
 *               MLA_DTYPE_BF16_Q_FP8_KV), contiguous, 16-byte aligned.
 *   kv_cache    device, [num_pages, page_size, 576] of shape->dtype (E4M3 for
 *               MLA_DTYPE_BF16_Q_FP8_KV), contiguous, 16-byte aligned.
 *   block_table device int32, [batch, max_pages] row-major.  The first
 *               ceil(seq_lens[b] / page_size) entries of row b must be page
 *               indices in [0, num_pages); later entries are never read.
 *               Out-of-range entries are clamped into range (no out-of-bounds
 *               access; results for that sequence are then unspecified).
 *   seq_lens    device int32 [batch], each >= 0 (keys in the cache for that
 *               sequence, including the q_len new tokens).  Values above
 *               max_seq_len are still computed correctly (less balanced).
 *   softmax_scale, q_scale, kv_scale
 *               host floats; dequantised value = stored value * scale (pass
 *               1.0 for bf16 and fp16 data).  The scores are formed exactly
 *               from the stored values (bf16 x E4M3 products are exact in
 *               the fp32 accumulation's inputs); P is rounded to bf16 for the
 *               PV product except in the all-FP8 path, where it is E4M3 with a
 *               per-row power-of-two scale.
 *   out         device bf16 [batch, q_len, num_heads, 512], contiguous, 16-byte aligned.
 *   lse         device fp32 [batch, q_len, num_heads] or NULL to skip.
 *   workspace   device scratch of workspace_bytes bytes, 256-byte aligned, at
 *               least the size mla_get_split_kv_and_workspace returns for
 *               (batch, q_len, num_heads, max_seq_len); may be NULL when that
 *               size is 0.  Its contents need no initialisation.
 *   stream      hipStream_t or NULL.
 *
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DTYPE, MLA_ERR_ALIGN, MLA_ERR_WORKSPACE, MLA_ERR_DEVICE, MLA_ERR_HIP
 * (kernel launch failed).  batch == 0 returns MLA_OK and enqueues nothing.
 */
int mla_decode(const mla_shape* shape, const void* q, const void* kv_cache, const int32_t* block_table,
               const int32_t* seq_lens, float softmax_scale, float q_scale, float kv_scale, void* out, float* lse,
               void* workspace, size_t workspace_bytes, void* stream);

/* Knobs of mla_decode_ex, for tests and tuning.  Zero-initialise, then set. */
typedef struct mla_options {
  int32_t num_splits;   /* > 0: use this many KV slices instead of the planned count */
  int32_t no_fold;      /* != 0: do not fold query tokens into heads (F = 1) */
  int32_t partial_fp32; /* != 0: keep the split partial outputs in fp32 (default: bf16 for E4M3
                           and bf16 caches, fp32 for fp16 caches) */
  int32_t stages;       /* 0: both kernels; 1: only the split-KV kernel; 2: only the merge kernel
                           (re-merging the partials a previous call with the same arguments left in
                           the workspace).  1 and 2 exist to time each kernel back to back. */
  int32_t window;       /* > 0: sliding-window mask.  Token t of a sequence sees only its last
                           `window` visible keys, [max(0, n_t - window), n_t) with
                           n_t = clamp(L - q_len + t + 1, 0, L); tiles before the earliest
                           such key are never read.  0: the plain causal mask.  (TokenSpeed
                           MLA article, section 6: a sliding-window mask among the decode
                           tests; the convention is this library's reading.)  < 0:
                           MLA_ERR_SHAPE.  Plan the workspace with the same options. */
  int32_t kernel;       /* E4M3 inputs: 1 the four-wave split-KV kernel, 2 the twelve-wave
                           role-specialised one; 0 the default: the four-wave kernel when
                           page_size is at least 64 (whole 64-key tiles per page) and no window
                           is set, the twelve-wave kernel otherwise.  Sequences of at most 8,192 keys take a second P
                           term (E2M1 codes of E4M3's rounding residual) in the twelve-wave
                           kernel and in the default four-wave one; a four-wave kernel forced
                           onto other pages or a window runs without it.  Other dtypes ignore
                           the field.  Other values: MLA_ERR_SHAPE */
  int32_t merge;        /* rows merged from many slices (more than 16 per row on average): 0 the
                           wide merge (a wave per quarter row, a whole chunk of slices in flight;
                           the default), 1 a workgroup per row (kept for comparison); 2 the
                           per-wave merge (a wave per row), which rows over at most 16 slices on
                           average always take.  Other values: MLA_ERR_SHAPE */
  int32_t reserved[1];
  void* split_event;    /* hipEvent_t or NULL: recorded on `stream` after the split-KV kernel
                           and before the merge kernel, so callers can time each kernel */
} mla_options;

/*
 * mla_decode with explicit options.  The workspace must be sized with
 * mla_workspace_bytes_ex for the same options.  Results equal mla_decode's
 * up to floating-point summation order (the fold factor only re-indexes rows;
 * the split count only changes where the LSE merge happens).
 */
int mla_decode_ex(const mla_shape* shape, const void* q, const void* kv_cache, const int32_t* block_table,
                  const int32_t* seq_lens, float softmax_scale, float q_scale, float kv_scale, void* out,
                  float* lse, void* workspace, size_t workspace_bytes, void* stream, const mla_options* options);

/*
 * Ragged batch: sequence b has its own number of new query tokens,
 * q_len_b = cu_seqlens_q[b+1] - cu_seqlens_q[b], for example a chunked or
 * ragged varlen prefill over the paged latent cache (tokenspeed-mla package
 * page and TokenSpeed MLA article, section 1: the varlen ragged prefill
 * without padding).  Token t of sequence b attends to keys
 * j < seq_lens[b] - q_len_b + t + 1, the rule of mla_decode with q_len_b in
 * place of q_len; everything else is as for mla_decode_ex.
 *
 *   shape->q_len    the largest q_len_b (it sizes the plan, the fold and the
 *                   workspace: plan with mla_workspace_bytes_ex(batch, max q_len_b, ...)).
 *   q               device, [total_q, num_heads, 576]: the new tokens of every
 *                   sequence, sequence b's at rows [cu_seqlens_q[b], cu_seqlens_q[b+1]).
 *   cu_seqlens_q    device int32 [batch + 1], non-decreasing, cu_seqlens_q[0] = 0,
 *                   cu_seqlens_q[batch] = total_q.  Values out of range are clamped into
 *                   [0, total_q] and counts above shape->q_len are cut to it: no access
 *                   leaves q, out or lse, but results are then unspecified.
 *   total_q         host int32, rows of q / out / lse (>= 0; 0 enqueues nothing).
 *   out, lse        device, [total_q, num_heads, 512] bf16 and [total_q, num_heads] fp32.
 * Errors: as mla_decode_ex; MLA_ERR_NULL for a NULL cu_seqlens_q, MLA_ERR_SHAPE for
 * total_q < 0, MLA_ERR_ALIGN for a cu_seqlens_q not 4-byte aligned.
 */
int mla_decode_varlen(const mla_shape* shape, const void* q, const int32_t* cu_seqlens_q, int32_t total_q,
                      const void* kv_cache, const int32_t* block_table, const int32_t* seq_lens, float softmax_scale,
                      float q_scale, float kv_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream, const mla_options* options);

/*
 * Tensor-descriptor form of mla_decode_ex, for C callers that hold strided
 * views: every tensor carries its element type, shape and strides, and the
 * library checks them against the layouts the kernels read before anything
 * is enqueued.  The operation, ownership, stream and error conventions are
 * those of mla_decode (top of this file); the argument list is the decode
 * call of the TokenSpeed MLA article, section 6 (query, kv_cache,
 * block_tables, cache_seqlens, softmax_scale, output / LSE, workspace).
 *
 * mla_tensor: data is a device pointer; dtype an mla_elem; ndim the number of
 * dimensions used (<= 4); shape and stride (in elements, as torch reports
 * them) of each dimension.  A dimension of extent 1 may have any stride.
 *
 *   q           ndim 4, [batch, q_len, num_heads, 576], bf16 / fp16 / E4M3, contiguous.
 *   kv_cache    ndim 3, [num_pages, page_size, 576], contiguous; its element type with
 *               q's selects the mla_dtype (equal, or bf16 q over an E4M3 cache).
 *   block_table ndim 2, int32 [batch, max_pages], packed rows (stride {max_pages, 1}).
 *   seq_lens    ndim 1, int32 [batch], unit stride.
 *   out         ndim 4, bf16 [batch, q_len, num_heads, 512], contiguous.
 *   lse         NULL, or ndim 3, fp32 [batch, q_len, num_heads], contiguous.
 *   workspace   host descriptor (required): data / bytes as mla_decode's workspace,
 *               max_seq_len the bound the plan was made for (0 <= max_seq_len <=
 *               max_pages * page_size), num_splits the plan's split count or 0 (not
 *               checked); a non-zero value other than the plan's is MLA_ERR_WORKSPACE.
 *   options     as mla_decode_ex (NULL = defaults).
 *
 * Errors: MLA_ERR_NULL (a NULL descriptor or data pointer), MLA_ERR_DTYPE (element types),
 * MLA_ERR_SHAPE (ndim, extents that disagree between tensors), MLA_ERR_STRIDE (strides),
 * then every error of mla_decode_ex.
 */
typedef enum mla_elem {
  MLA_ELEM_BF16 = 1,
  MLA_ELEM_FP8_E4M3 = 2,
  MLA_ELEM_FP16 = 3,
  MLA_ELEM_FP32 = 4,
  MLA_ELEM_INT32 = 5
} mla_elem;

typedef struct mla_tensor {
  void* data;
  int32_t dtype; /* mla_elem */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} mla_tensor;

typedef struct mla_workspace {
  void* data;
  size_t bytes;
  int32_t num_splits;
  int32_t max_seq_len;
} mla_workspace;

int mla_decode_tensors(const mla_tensor* q, const mla_tensor* kv_cache, const mla_tensor* block_table,
                       const mla_tensor* seq_lens, float softmax_scale, float q_scale, float kv_scale,
                       const mla_tensor* out, const mla_tensor* lse, const mla_workspace* workspace, void* stream,
                       const mla_options* options);

/*
 * mla_decode_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace is a file-scope device
 * array of 160 MiB inside the library (one copy per GPU, held until the process
 * ends; its address is looked up once per device, on that device's first call).
 * The call allocates and frees nothing.  Inputs, outputs, sizes, options and
 * errors are those of mla_decode_ex; in addition, a shape whose plan needs
 * more than 160 MiB (mla_workspace_bytes_ex) fails with MLA_ERR_WORKSPACE
 * before anything is enqueued.  The array needs no clearing: nothing in it
 * carries over from one call to the next.  Every call on one GPU uses the
 * same array, so calls that overlap on one GPU (concurrent streams, or
 * threads) race on it; calls on one stream are ordered and safe.
 */
int mla_decode_static(const mla_shape* shape, const void* q, const void* kv_cache, const int32_t* block_table,
                      const int32_t* seq_lens, float softmax_scale, float q_scale, float kv_scale, void* out,
                      float* lse, void* stream, const mla_options* options);

/* Workspace size and split count for mla_decode_ex with `options` (NULL = defaults). */
int mla_workspace_bytes_ex(int32_t batch, int32_t q_len, int32_t num_heads, int32_t max_seq_len,
                           const mla_options* options, int32_t* num_splits, size_t* workspace_bytes);

/*
 * Host-only planning for an explicit compute-unit count (no device query), so
 * the split heuristic can be checked without a GPU.  fold_factor receives F.
 */
int mla_plan_for_cus(int32_t batch, int32_t q_len, int32_t num_heads, int32_t max_seq_len, int32_t num_cus,
                     const mla_options* options, int32_t* num_splits, int32_t* fold_factor,
                     size_t* workspace_bytes);

/*
 * Fused K/V pack + FP8 quantise: the step that writes decode's cache rows.
 * Row t of the output is e4m3(latent[t, 0:512] / kv_scale) ||
 * e4m3(rope[t, 0:64] / kv_scale), round-to-nearest-even with saturation to
 * +-448 (NaN stays NaN).  It replaces a separate concatenation and cast
 * (tokenspeed-mla package page, "What it is": the fused K/V packing and FP8
 * quantisation kernel; TokenSpeed MLA article, section 1, kernel table).
 *
 *   latent        device bf16 [num_tokens, 512], row stride latent_stride elements (>= 512), 16-byte aligned rows.
 *   rope          device bf16 [num_tokens, 64],  row stride rope_stride elements (>= 64), 16-byte aligned rows.
 *   slot_mapping  device int64 [num_tokens] or NULL.  NULL: token t goes to
 *                 row t of out.  Otherwise to row slot_mapping[t] of out;
 *                 negative slots are skipped; slots >= out_rows are skipped.
 *   out           device uint8 [out_rows, 576] (e.g. a paged cache viewed as rows), 16-byte aligned.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ALIGN, MLA_ERR_HIP.
 */
int mla_kv_pack_quantize_fp8(const void* latent, int64_t latent_stride, const void* rope, int64_t rope_stride,
                             const int64_t* slot_mapping, int32_t num_tokens, float kv_scale, void* out,
                             int64_t out_rows, void* stream);

/* Message for the calling thread's last non-zero return ("" if none). */
const char* mla_last_error(void);

/* MLA_VERSION of the built library. */
int mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
