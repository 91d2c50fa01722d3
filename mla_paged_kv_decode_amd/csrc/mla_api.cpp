// Host runtime of the MLA decode library: argument validation, the cached
// per-shape plan (fold factor, KV slices, workspace layout) and kernel
// dispatch.  Implements the C ABI declared in include/mla_decode.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "mla_decode.h"
#include "mla_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MLA_OK;
}

// At least one 64-key unit per KV slice.  A workgroup's fixed latency chain
// (sequence lengths, block table, first tiles, epilogue) is about 12 us, so a
// small batch is faster spread one unit per slice plus the merge (256 keys of
// bf16: 22 us) than run as fewer, longer slices (28 us as one slice).
constexpr int kMinUnitsPerSlice = 1;
// Above this many workgroup rows (query groups x row tiles) the rows' work can
// differ widely: the query groups of a ragged batch hold tokens of different
// sequences, and causal groups of a long query see different key counts.
// Such launches take about kDynamicWaves workgroups per compute unit and at
// least two slices per row, so the hardware dispatcher evens out the rows and
// no row's whole work lands on one CU.  More slices per row cost partial-output
// traffic: 4 workgroups per CU was 8% slower than 2 on a ragged FP8 prefill.
constexpr int kManyRows = 32;
constexpr int kDynamicWaves = 2;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int F, H_eff, q_len_eff, m_tiles, U, G, xcd_map, u_major;
  size_t rows_per_b;
  size_t off_part_o, off_part_lse, off_meta, bytes;
};

// Largest F with q_len % F == 0 and H * F <= 128 (TokenSpeed MLA article,
// section 3: query-token folding into the head dimension).
int fold_factor(int q_len, int H, bool no_fold) {
  int best = 1;
  if (no_fold) return 1;
  for (int F = 1; F <= q_len; ++F)
    if (q_len % F == 0 && (long long)H * F <= mla::kTileM) best = F;
  return best;
}

// Split heuristic: one workgroup per compute unit (each holds a 147 KiB LDS
// ring and 512 VGPRs per lane), each workgroup row's KV work cut into G equal
// slices, none smaller than kMinUnitsPerSlice units; with more than kManyRows
// rows, about kDynamicWaves workgroups per compute unit instead (at least two
// slices per row).  G is a
// multiple of 8 when >= 8 so every XCD gets the same number of slices.
Plan make_plan(int B, int q_len, int H, int max_seq_len, int num_cus, const mla_options* opt) {
  Plan pl{};
  pl.F = fold_factor(q_len, H, opt && opt->no_fold);
  pl.H_eff = H * pl.F;
  pl.q_len_eff = q_len / pl.F;
  pl.m_tiles = (pl.H_eff + mla::kTileM - 1) / mla::kTileM;
  pl.U = pl.q_len_eff * pl.m_tiles;
  long long units_per_seq = max_seq_len > 0 ? (max_seq_len + mla::kPlanUnitKeys - 1) / mla::kPlanUnitKeys : 1;
  if (opt && opt->window > 0) {
    // a window reads at most window + q_len - 1 keys per sequence, from a unit-aligned start
    const long long w_units = ((long long)opt->window + q_len - 1 + mla::kPlanUnitKeys - 1) / mla::kPlanUnitKeys + 1;
    if (w_units < units_per_seq) units_per_seq = w_units;
  }
  const long long units_max = (long long)B * units_per_seq;
  int G;
  if (opt && opt->num_splits > 0) {
    G = opt->num_splits;
  } else {
    if (pl.U > kManyRows) {
      G = (kDynamicWaves * num_cus + pl.U - 1) / pl.U;
      if (G < 2) G = 2;
    } else {
      G = num_cus / pl.U;
    }
    if (G < 1) G = 1;
    long long cap = (units_max + kMinUnitsPerSlice - 1) / kMinUnitsPerSlice;
    if (cap < 1) cap = 1;
    if (G > cap) G = (int)cap;
    if (G >= 8) G -= G % 8;
  }
  pl.G = G;
  pl.xcd_map = (pl.U == 1 || G % 8 == 0) ? 1 : 0;
  pl.u_major = pl.U > kManyRows ? 1 : 0;
  pl.rows_per_b = (size_t)q_len * H;
  if (G <= 1) {
    pl.bytes = 0;
    pl.off_part_o = pl.off_part_lse = pl.off_meta = 0;
  } else {
    // partial outputs are sized for fp32 (the plan carries no dtype; E4M3 and bf16
    // caches write bf16 partials into the first half of the region)
    const size_t slots = (size_t)G + (size_t)B;
    const size_t esz = 4;
    pl.off_part_o = 0;
    pl.off_part_lse = align_up(slots * pl.rows_per_b * mla::kDv * esz);
    pl.off_meta = pl.off_part_lse + align_up(slots * pl.rows_per_b * sizeof(float));
    // per workgroup row: [B][2] slice ranges, then the rows' total units T
    pl.bytes = pl.off_meta + align_up((size_t)pl.U * B * 2 * sizeof(int32_t) + (size_t)pl.U * sizeof(int64_t));
  }
  return pl;
}

std::mutex g_mu;
std::map<int, int> g_cus;  // device -> compute units (0 = not gfx950)
std::map<std::tuple<int, int, int, int, int, int, int, int, int, int>, Plan> g_plans;

int device_cus(int* dev_out, int* cus_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_cus.find(dev);
    if (it != g_cus.end()) {
      if (it->second <= 0) return fail(MLA_ERR_DEVICE, "device %d is not a gfx950 GPU", dev);
      *dev_out = dev;
      *cus_out = it->second;
      return MLA_OK;
    }
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(MLA_ERR_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
  const bool is950 = std::string(prop.gcnArchName).rfind("gfx950", 0) == 0;
  const int cus = is950 ? prop.multiProcessorCount : 0;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_cus[dev] = cus;
  }
  if (cus <= 0) return fail(MLA_ERR_DEVICE, "device %d (%s) is not a gfx950 GPU", dev, prop.gcnArchName);
  *dev_out = dev;
  *cus_out = cus;
  return MLA_OK;
}

int check_plan_args(int B, int q_len, int H, int max_seq_len) {
  if (B < 0) return fail(MLA_ERR_SHAPE, "batch must be >= 0 (got %d)", B);
  if (q_len < 1) return fail(MLA_ERR_SHAPE, "q_len must be >= 1 (got %d)", q_len);
  if (H < 1) return fail(MLA_ERR_SHAPE, "num_heads must be >= 1 (got %d)", H);
  if (max_seq_len < 0) return fail(MLA_ERR_SHAPE, "max_seq_len must be >= 0 (got %d)", max_seq_len);
  if ((long long)q_len * H > (1 << 20)) return fail(MLA_ERR_SHAPE, "q_len * num_heads too large");
  return MLA_OK;
}

int cached_plan(int dev, int cus, int B, int q_len, int H, int max_seq_len, const mla_options* opt, Plan* out) {
  const auto key = std::make_tuple(dev, B, q_len, H, max_seq_len, opt ? opt->num_splits : 0, opt ? opt->no_fold : 0,
                                   opt ? opt->partial_fp32 : 0, cus, opt ? opt->window : 0);
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_plans.find(key);
  if (it == g_plans.end()) it = g_plans.emplace(key, make_plan(B, q_len, H, max_seq_len, cus, opt)).first;
  *out = it->second;
  return MLA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int decode_impl(const mla_shape* s, const void* q, const void* kv, const int32_t* bt, const int32_t* seq_lens,
                float softmax_scale, float q_scale, float kv_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                void* stream, const mla_options* opt,
                const int32_t* cu_q = nullptr, int32_t total_q = 0, bool static_ws = false) {
  if (opt && (opt->stages < 0 || opt->stages > 2)) return fail(MLA_ERR_SHAPE, "options.stages must be 0, 1 or 2");
  if (opt && opt->window < 0) return fail(MLA_ERR_SHAPE, "options.window must be >= 0 (got %d)", opt->window);
  if (opt && (opt->kernel < 0 || opt->kernel > 2)) return fail(MLA_ERR_SHAPE, "options.kernel must be 0, 1 or 2");
  if (opt && (opt->merge < 0 || opt->merge > 2)) return fail(MLA_ERR_SHAPE, "options.merge must be 0, 1 or 2");
  if (!s) return fail(MLA_ERR_NULL, "shape is NULL");
  if (s->dtype != MLA_DTYPE_BF16 && s->dtype != MLA_DTYPE_FP8_E4M3 && s->dtype != MLA_DTYPE_FP16 &&
      s->dtype != MLA_DTYPE_BF16_Q_FP8_KV)
    return fail(MLA_ERR_DTYPE,
                "dtype %d is not MLA_DTYPE_BF16, MLA_DTYPE_FP16, MLA_DTYPE_FP8_E4M3 or MLA_DTYPE_BF16_Q_FP8_KV",
                s->dtype);
  int rc = check_plan_args(s->batch, s->q_len, s->num_heads, s->max_seq_len);
  if (rc) return rc;
  if (s->num_pages < 1) return fail(MLA_ERR_SHAPE, "num_pages must be >= 1 (got %d)", s->num_pages);
  if (s->max_pages < 1) return fail(MLA_ERR_SHAPE, "max_pages must be >= 1 (got %d)", s->max_pages);
  if (s->page_size < 16 || s->page_size > 65536 || (s->page_size & (s->page_size - 1)))
    return fail(MLA_ERR_SHAPE, "page_size must be a power of two in [16, 65536] (got %d)", s->page_size);
  if ((long long)s->max_seq_len > (long long)s->max_pages * s->page_size)
    return fail(MLA_ERR_SHAPE, "max_seq_len %d exceeds max_pages * page_size", s->max_seq_len);
  if ((long long)s->max_pages * s->page_size > (1LL << 31) - 1)
    return fail(MLA_ERR_SHAPE, "max_pages * page_size must fit in int32");
  if (!isfinite(softmax_scale) || !isfinite(q_scale) || !isfinite(kv_scale))
    return fail(MLA_ERR_SHAPE, "scales must be finite");
  if (!((double)softmax_scale * q_scale * kv_scale > 0.0))
    return fail(MLA_ERR_SHAPE, "softmax_scale * q_scale * kv_scale must be positive");
  if (s->batch == 0) return ok();
  if (cu_q != nullptr) {  // a ragged batch
    if (total_q < 0) return fail(MLA_ERR_SHAPE, "total_q must be >= 0 (got %d)", total_q);
    if (!aligned(cu_q, 4)) return fail(MLA_ERR_ALIGN, "cu_seqlens_q must be 4-byte aligned");
    if (total_q == 0) return ok();  // no new token anywhere
  }
  if (!q || !kv || !bt || !seq_lens || !out)
    return fail(MLA_ERR_NULL, "q, kv_cache, block_table, seq_lens and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16))
    return fail(MLA_ERR_ALIGN, "q, kv_cache and out must be 16-byte aligned");
  if (!aligned(bt, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
    return fail(MLA_ERR_ALIGN, "block_table, seq_lens and lse must be 4-byte aligned");

  int dev = 0, cus = 0;
  rc = device_cus(&dev, &cus);
  if (rc) return rc;
  Plan pl;
  cached_plan(dev, cus, s->batch, s->q_len, s->num_heads, s->max_seq_len, opt, &pl);
  if (static_ws) {
    if (pl.bytes > mla::kStaticScratchBytes)
      return fail(MLA_ERR_WORKSPACE,
                  "this shape needs a %zu-byte workspace, more than the %zu-byte static scratch of mla_decode_static",
                  pl.bytes, mla::kStaticScratchBytes);
    hipError_t e = mla::static_scratch(&ws);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    ws_bytes = mla::kStaticScratchBytes;
  }
  if (pl.bytes > 0) {
    if (!ws) return fail(MLA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", pl.bytes);
    if (!aligned(ws, kAlign)) return fail(MLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < pl.bytes)
      return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes this shape needs", ws_bytes,
                  pl.bytes);
  }

  const int dt = s->dtype == MLA_DTYPE_FP8_E4M3      ? mla::kFp8
                 : s->dtype == MLA_DTYPE_FP16         ? mla::kFp16
                 : s->dtype == MLA_DTYPE_BF16_Q_FP8_KV ? mla::kMixed
                                                      : mla::kBf16;
  int shift = 0;
  while ((1 << shift) < s->page_size) ++shift;
  mla::PartialParams p{};
  p.q = (const uint8_t*)q;
  p.kv = (const uint8_t*)kv;
  p.block_table = bt;
  p.seq_lens = seq_lens;
  p.out = (uint16_t*)out;
  p.lse = lse;
  uint8_t* wsb = (uint8_t*)ws;
  p.part_o = pl.bytes ? wsb + pl.off_part_o : nullptr;
  p.part_lse = pl.bytes ? (float*)(wsb + pl.off_part_lse) : nullptr;
  p.meta = pl.bytes ? (int32_t*)(wsb + pl.off_meta) : nullptr;
  p.B = s->batch;
  p.q_len = s->q_len;
  p.H = s->num_heads;
  p.F = pl.F;
  p.H_eff = pl.H_eff;
  p.q_len_eff = pl.q_len_eff;
  p.m_tiles = pl.m_tiles;
  p.U = pl.U;
  p.G = pl.G;
  p.xcd_map = pl.xcd_map;
  p.u_major = pl.u_major;
  p.page_size = s->page_size;
  p.page_shift = shift;
  p.max_pages = s->max_pages;
  p.num_pages = s->num_pages;
  p.s_scale_log2 = (float)((double)softmax_scale * (double)q_scale * (double)kv_scale * 1.4426950408889634074);
  p.v_scale = kv_scale;
  // Partial outputs: bf16 for E4M3 and bf16 caches (the partials' round trip is the step's largest
  // overhead after the KV stream; rounding each slice's O to bf16 moves the merged row by at most
  // 2^-9 of sum_j w_j |v_j|), fp32 for fp16 caches (their V values are not bf16 values: a single
  // key's V must come back as stored).
  const bool bf16_part = dt == mla::kFp8 || dt == mla::kMixed || dt == mla::kBf16;
  p.part_bf16 = (!(opt && opt->partial_fp32) && bf16_part) ? 1 : 0;
  p.window = opt ? opt->window : 0;
  p.cu_q = cu_q;
  p.total_q = total_q;
  p.kernel = opt ? opt->kernel : 0;
  const int tile = (dt == mla::kFp8 || dt == mla::kMixed) ? 64 : 32;  // keys per LDS tile
  hipStream_t st = (hipStream_t)stream;
  const int stages = opt ? opt->stages : 0;
  hipError_t e = hipSuccess;
  if (stages != 2) {
    e = mla::launch_partial(p, dt, s->page_size >= tile, st);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "split-KV partial kernel launch failed: %s", hipGetErrorString(e));
  }
  if (opt && opt->split_event) {
    e = hipEventRecord((hipEvent_t)opt->split_event, st);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipEventRecord(split_event) failed: %s", hipGetErrorString(e));
  }
  if (pl.G > 1 && stages != 1) {
    mla::CombineParams c{};
    c.part_o = p.part_o;
    c.part_lse = p.part_lse;
    c.meta = p.meta;
    c.out = p.out;
    c.lse = lse;
    c.B = s->batch;
    c.rows_per_b = (int)pl.rows_per_b;
    c.G = pl.G;
    c.part_bf16 = p.part_bf16;
    c.H = s->num_heads;
    c.q_len = s->q_len;
    c.F = pl.F;
    c.q_len_eff = pl.q_len_eff;
    c.U = pl.U;
    c.cu_q = cu_q;
    c.total_q = total_q;
    c.merge_kernel = opt ? opt->merge : 0;
    e = mla::launch_combine(c, st);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

int mla_plan_for_cus(int32_t batch, int32_t q_len, int32_t num_heads, int32_t max_seq_len, int32_t num_cus,
                     const mla_options* options, int32_t* num_splits, int32_t* fold, size_t* workspace_bytes) {
  if (!num_splits || !workspace_bytes || !fold) return fail(MLA_ERR_NULL, "output pointers must be non-NULL");
  int rc = check_plan_args(batch, q_len, num_heads, max_seq_len);
  if (rc) return rc;
  if (options && options->window < 0) return fail(MLA_ERR_SHAPE, "options.window must be >= 0 (got %d)", options->window);
  if (num_cus < 1) return fail(MLA_ERR_SHAPE, "num_cus must be >= 1");
  const Plan pl = make_plan(batch, q_len, num_heads, max_seq_len, num_cus, options);
  *num_splits = pl.G;
  *fold = pl.F;
  *workspace_bytes = pl.bytes;
  return ok();
}

int mla_workspace_bytes_ex(int32_t batch, int32_t q_len, int32_t num_heads, int32_t max_seq_len,
                           const mla_options* options, int32_t* num_splits, size_t* workspace_bytes) {
  if (!num_splits || !workspace_bytes) return fail(MLA_ERR_NULL, "output pointers must be non-NULL");
  int rc = check_plan_args(batch, q_len, num_heads, max_seq_len);
  if (rc) return rc;
  if (options && options->window < 0) return fail(MLA_ERR_SHAPE, "options.window must be >= 0 (got %d)", options->window);
  int dev = 0, cus = 0;
  rc = device_cus(&dev, &cus);
  if (rc) return rc;
  Plan pl;
  cached_plan(dev, cus, batch, q_len, num_heads, max_seq_len, options, &pl);
  *num_splits = pl.G;
  *workspace_bytes = pl.bytes;
  return ok();
}

int mla_get_split_kv_and_workspace(int32_t batch, int32_t q_len, int32_t num_heads, int32_t max_seq_len,
                                   int32_t* num_splits, size_t* workspace_bytes) {
  return mla_workspace_bytes_ex(batch, q_len, num_heads, max_seq_len, nullptr, num_splits, workspace_bytes);
}

int mla_decode(const mla_shape* shape, const void* q, const void* kv_cache, const int32_t* block_table,
               const int32_t* seq_lens, float softmax_scale, float q_scale, float kv_scale, void* out, float* lse,
               void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(shape, q, kv_cache, block_table, seq_lens, softmax_scale, q_scale, kv_scale, out, lse, workspace,
                     workspace_bytes, stream, nullptr);
}

int mla_decode_ex(const mla_shape* shape, const void* q, const void* kv_cache, const int32_t* block_table,
                  const int32_t* seq_lens, float softmax_scale, float q_scale, float kv_scale, void* out, float* lse,
                  void* workspace, size_t workspace_bytes, void* stream, const mla_options* options) {
  return decode_impl(shape, q, kv_cache, block_table, seq_lens, softmax_scale, q_scale, kv_scale, out, lse, workspace,
                     workspace_bytes, stream, options);
}

int mla_decode_varlen(const mla_shape* shape, const void* q, const int32_t* cu_seqlens_q, int32_t total_q,
                      const void* kv_cache, const int32_t* block_table, const int32_t* seq_lens, float softmax_scale,
                      float q_scale, float kv_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream, const mla_options* options) {
  if (!cu_seqlens_q) return fail(MLA_ERR_NULL, "cu_seqlens_q is NULL");
  return decode_impl(shape, q, kv_cache, block_table, seq_lens, softmax_scale, q_scale, kv_scale, out, lse, workspace,
                     workspace_bytes, stream, options, cu_seqlens_q, total_q);
}

int mla_kv_pack_quantize_fp8(const void* latent, int64_t latent_stride, const void* rope, int64_t rope_stride,
                             const int64_t* slot_mapping, int32_t num_tokens, float kv_scale, void* out,
                             int64_t out_rows, void* stream) {
  if (num_tokens < 0) return fail(MLA_ERR_SHAPE, "num_tokens must be >= 0");
  if (latent_stride < MLA_D_V || rope_stride < MLA_QK_ROPE_HEAD_DIM)
    return fail(MLA_ERR_SHAPE, "latent_stride must be >= 512 and rope_stride >= 64");
  if (latent_stride % 8 || rope_stride % 8) return fail(MLA_ERR_ALIGN, "row strides must be multiples of 8 elements");
  if (out_rows < 0) return fail(MLA_ERR_SHAPE, "out_rows must be >= 0");
  if (!(kv_scale > 0.f) || !isfinite(kv_scale)) return fail(MLA_ERR_SHAPE, "kv_scale must be finite and > 0");
  if (slot_mapping == nullptr && out_rows < num_tokens)
    return fail(MLA_ERR_SHAPE, "out_rows must be >= num_tokens without a slot mapping");
  if (num_tokens == 0) return ok();
  if (!latent || !rope || !out) return fail(MLA_ERR_NULL, "latent, rope and out must be non-NULL");
  if (!aligned(latent, 16) || !aligned(rope, 16) || !aligned(out, 16) || (slot_mapping && !aligned(slot_mapping, 8)))
    return fail(MLA_ERR_ALIGN, "latent, rope and out must be 16-byte aligned, slot_mapping 8-byte aligned");
  mla::PackParams p{};
  p.latent = (const uint16_t*)latent;
  p.rope = (const uint16_t*)rope;
  p.slot_mapping = slot_mapping;
  p.out = (uint8_t*)out;
  p.latent_stride = latent_stride;
  p.rope_stride = rope_stride;
  p.out_rows = out_rows;
  p.num_tokens = num_tokens;
  p.scale = kv_scale;
  hipError_t e = mla::launch_pack_fp8(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "pack kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int mla_decode_static(const mla_shape* shape, const void* q, const void* kv_cache, const int32_t* block_table,
                      const int32_t* seq_lens, float softmax_scale, float q_scale, float kv_scale, void* out,
                      float* lse, void* stream, const mla_options* options) {
  return decode_impl(shape, q, kv_cache, block_table, seq_lens, softmax_scale, q_scale, kv_scale, out, lse, nullptr, 0,
                     stream, options, nullptr, 0, true);
}

// Tensor-descriptor form: every descriptor is checked against the layout the
// kernels read (element type, extents, strides), then the call is mla_decode_ex's.
int mla_decode_tensors(const mla_tensor* q, const mla_tensor* kv_cache, const mla_tensor* block_table,
                       const mla_tensor* seq_lens, float softmax_scale, float q_scale, float kv_scale,
                       const mla_tensor* out, const mla_tensor* lse, const mla_workspace* workspace, void* stream,
                       const mla_options* options) {
  if (!q || !kv_cache || !block_table || !seq_lens || !out || !workspace)
    return fail(MLA_ERR_NULL, "q, kv_cache, block_table, seq_lens, out and workspace descriptors must be non-NULL");
  struct Named {
    const mla_tensor* t;
    const char* name;
    int ndim;
  };
  const Named all[] = {{q, "q", 4}, {kv_cache, "kv_cache", 3}, {block_table, "block_table", 2},
                       {seq_lens, "seq_lens", 1}, {out, "out", 4}, {lse, "lse", 3}};
  for (const Named& n : all) {
    if (!n.t) continue;
    if (n.t->ndim != n.ndim) return fail(MLA_ERR_SHAPE, "%s must have %d dimensions (got %d)", n.name, n.ndim, n.t->ndim);
    for (int d = 0; d < n.ndim; ++d)
      if (n.t->shape[d] < 0 || n.t->shape[d] > INT32_MAX)
        return fail(MLA_ERR_SHAPE, "%s extent %d out of range (%lld)", n.name, d, (long long)n.t->shape[d]);
  }
  // element types
  const int qt = q->dtype, kt = kv_cache->dtype;
  int dtype;
  if (qt == kt && (qt == MLA_ELEM_BF16 || qt == MLA_ELEM_FP16 || qt == MLA_ELEM_FP8_E4M3)) {
    dtype = qt == MLA_ELEM_BF16 ? MLA_DTYPE_BF16 : qt == MLA_ELEM_FP16 ? MLA_DTYPE_FP16 : MLA_DTYPE_FP8_E4M3;
  } else if (qt == MLA_ELEM_BF16 && kt == MLA_ELEM_FP8_E4M3) {
    dtype = MLA_DTYPE_BF16_Q_FP8_KV;
  } else {
    return fail(MLA_ERR_DTYPE, "q / kv_cache element types %d / %d are not a supported pair", qt, kt);
  }
  if (block_table->dtype != MLA_ELEM_INT32 || seq_lens->dtype != MLA_ELEM_INT32)
    return fail(MLA_ERR_DTYPE, "block_table and seq_lens must be int32");
  if (out->dtype != MLA_ELEM_BF16) return fail(MLA_ERR_DTYPE, "out must be bf16");
  if (lse && lse->dtype != MLA_ELEM_FP32) return fail(MLA_ERR_DTYPE, "lse must be fp32");
  // extents
  const int64_t B = q->shape[0], QL = q->shape[1], H = q->shape[2];
  if (q->shape[3] != MLA_D_QK || kv_cache->shape[2] != MLA_D_QK)
    return fail(MLA_ERR_SHAPE, "q and kv_cache rows must be %d wide", MLA_D_QK);
  if (block_table->shape[0] != B || seq_lens->shape[0] != B)
    return fail(MLA_ERR_SHAPE, "block_table must have batch rows and seq_lens batch entries (batch = %lld)",
                (long long)B);
  if (out->shape[0] != B || out->shape[1] != QL || out->shape[2] != H || out->shape[3] != MLA_D_V)
    return fail(MLA_ERR_SHAPE, "out must be [batch, q_len, num_heads, %d]", MLA_D_V);
  if (lse && (lse->shape[0] != B || lse->shape[1] != QL || lse->shape[2] != H))
    return fail(MLA_ERR_SHAPE, "lse must be [batch, q_len, num_heads]");
  // strides: packed row-major everywhere; a dimension of extent 1 may carry any stride
  auto packed = [](const mla_tensor* t) {
    int64_t want = 1;
    for (int d = t->ndim - 1; d >= 0; --d) {
      if (t->shape[d] != 1 && t->stride[d] != want) return false;
      want *= t->shape[d];
    }
    return true;
  };
  for (const Named& n : all)
    if (n.t && !packed(n.t))
      return fail(MLA_ERR_STRIDE, "%s must be packed row-major (its strides are not)", n.name);
  if (!q->data || !kv_cache->data || !block_table->data || !seq_lens->data || !out->data || (lse && !lse->data))
    return fail(MLA_ERR_NULL, "a tensor descriptor has a NULL data pointer");
  mla_shape s{};
  s.batch = (int32_t)B;
  s.q_len = (int32_t)QL;
  s.num_heads = (int32_t)H;
  s.num_pages = (int32_t)kv_cache->shape[0];
  s.page_size = (int32_t)kv_cache->shape[1];
  s.max_pages = (int32_t)block_table->shape[1];
  s.max_seq_len = workspace->max_seq_len;
  s.dtype = dtype;
  if (workspace->num_splits != 0 && s.batch > 0) {
    int rc = check_plan_args(s.batch, s.q_len, s.num_heads, s.max_seq_len);
    if (rc) return rc;
    int dev = 0, cus = 0;
    rc = device_cus(&dev, &cus);
    if (rc) return rc;
    Plan pl;
    cached_plan(dev, cus, s.batch, s.q_len, s.num_heads, s.max_seq_len, options, &pl);
    if (pl.G != workspace->num_splits)
      return fail(MLA_ERR_WORKSPACE, "workspace was planned for %d splits, this shape plans %d", workspace->num_splits,
                  pl.G);
  }
  return decode_impl(&s, q->data, kv_cache->data, (const int32_t*)block_table->data, (const int32_t*)seq_lens->data,
                     softmax_scale, q_scale, kv_scale, out->data, lse ? (float*)lse->data : nullptr, workspace->data,
                     workspace->bytes, stream, options);
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

int mla_version(void) { return MLA_VERSION; }

}  // extern "C"
