// Internal interfaces between the host runtime (mla_api.cpp) and the gfx950
// kernels (mla_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kTileM = 128;     // folded query rows per workgroup (4 waves x 32 rows)
// Keys per work unit of the host's plan: the smallest LDS tile (32 bf16 / fp16
// keys), since the plan does not know the dtype.  Each kernel partitions in its
// own tile (64 keys for E4M3 tiles, whose small batches may then leave some of
// the planned slices empty: they write nothing and the merge skips them).
constexpr int kPlanUnitKeys = 32;
constexpr int kStages = 4;      // LDS ring of KV tiles
constexpr int kStageBytes = 36864;  // 64 fp8 rows or 32 bf16 rows of 576 elements
constexpr int kThreads = 256;

// kMixed: bf16 q over an OCP E4M3 cache
enum KernelDtype { kBf16 = 1, kFp8 = 2, kFp16 = 3, kMixed = 4 };

// Everything the split-KV partial kernel needs.  Passed by value.
struct PartialParams {
  const uint8_t* q;          // [B, q_len, H, 576] elements
  const uint8_t* kv;         // [num_pages, page_size, 576] elements
  const int32_t* block_table;  // [B, max_pages]
  const int32_t* seq_lens;   // [B]
  uint16_t* out;             // bf16 [B, q_len, H, 512]
  float* lse;                // [B, q_len, H] or nullptr
  void* part_o;              // [G + B][q_len * H][512] fp32 or bf16
  float* part_lse;           // [G + B][q_len * H]
  int32_t* meta;             // [U][B][2]: first and last KV slice of workgroup row u touching sequence b; then int64 C[U]
  int32_t B, q_len, H, F, H_eff, q_len_eff, m_tiles, U, G;
  int32_t xcd_map;           // 1: slices are dealt to the XCDs in turn, each slice's workgroups on one XCD
  int32_t u_major;           // 1: workgroup ids run over the slices of one query group first (many groups)
  int32_t page_size, page_shift, max_pages, num_pages;
  float s_scale_log2;        // softmax_scale * q_scale * kv_scale * log2(e)
  float v_scale;             // kv_scale (V dequantisation)
  int32_t part_bf16;
  int32_t window;            // sliding window in keys (0: none)
  const int32_t* cu_q;       // ragged batch: [B+1] cumulative new-token counts (device), or nullptr
  int32_t total_q;           // ragged batch: token rows of q / out
  int32_t kernel;            // E4M3: 1 the four-wave kernel, 2 the role-specialised kernel, 0 the default (see launch_partial)
  // Work partition in cost units of a quarter tile: a tile costs 4, or lo_cost in E4M3 sequences
  // that take the second P term (set per kernel at launch)
  int32_t lo_cost;
};

struct CombineParams {
  const void* part_o;
  const float* part_lse;
  const int32_t* meta;
  uint16_t* out;
  float* lse;
  int32_t B, rows_per_b, G;
  int32_t part_bf16;
  int32_t H, q_len;           // heads and the (largest) query count of a sequence
  int32_t F, q_len_eff, U;    // fold factor, query groups, workgroup rows (meta is [U][B][2], then int64 T[U])
  const int32_t* cu_q;        // ragged batch: [B+1] cumulative new-token counts, or nullptr
  int32_t total_q;
  int32_t merge_kernel;       // rows over many slices: 0 the wide merge (a wave per row quarter), 1 a workgroup per row, 2 a wave per row
};

struct PackParams {
  const uint16_t* latent;
  const uint16_t* rope;
  const int64_t* slot_mapping;
  uint8_t* out;
  int64_t latent_stride, rope_stride, out_rows;
  int32_t num_tokens;
  float scale;  // kv_scale: stored code = e4m3(x / scale)
};

// Launchers (defined in mla_kernels.hip).  Return the launch's hipError_t.
hipError_t launch_partial(const PartialParams& p, int dtype, bool fast_pages, hipStream_t stream);
// The merge runs one wave per output row when sequences span at most 16 slices
// on average (G <= 16 B: one chunk of the per-wave merge's loads), and spreads a
// row over a workgroup otherwise.
inline bool combine_per_wave(int B, int G) { return (long long)G <= 16LL * B; }
// The 16-bit kernels spread PV over all four waves (the fp8 layout: P through
// LDS, one more barrier per 32 keys) when a workgroup's 128 rows are not all
// filled, i.e. fewer than 128 folded rows: otherwise the waves holding rows
// would do all of PV.  With every row block filled the own-rows layout is faster.
inline bool cross_wave_pv(int H_eff) { return H_eff < 128; }
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
// mla_decode_static's workspace: a file-scope device array of this many bytes
// (enough for the plans of every decode workload benchmarked here, the largest
// being 128.3 MiB); static_scratch() returns the current device's copy, looked
// up once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t(160) << 20;
hipError_t static_scratch(void** ptr);
hipError_t launch_pack_fp8(const PackParams& p, hipStream_t stream);

}  // namespace mla
