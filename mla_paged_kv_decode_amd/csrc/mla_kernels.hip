// gfx950 (MI355X, CDNA4) kernels for MLA decode over a paged latent KV cache.
//
//  * mla_split_kv_partial: one workgroup = 4 waves = 128 folded query rows of
//    one (sequence, query group) and one contiguous slice of the batch's KV
//    work.  KV tiles (36,864 bytes: 64 E4M3 rows or 32 bf16 / fp16 rows of
//    576 elements) stream HBM -> LDS through a 4-deep ring filled by direct
//    global->LDS loads; scores S^T = K Q^T and the output O^T = V^T P^T run on
//    MFMA (32x32x64 f8f6f4, or 32x32x16 bf16 / f16; bf16 q over an E4M3 cache
//    widens its K and V operands to bf16 after the LDS read), V^T being read
//    from the same LDS tile with the transposing LDS reads.  Softmax in base 2
//    relative to a per-row reference fixed at the row's first visible tile (a
//    segment is recomputed in the rare case a row max outgrows it); the FP8
//    probabilities carry a per-row power-of-two block scale through the MFMA's
//    scale operand; O is normalised by the sum of the rounded probabilities (the
//    weights the PV product used), the LSE by the exact sum.  Writes the final bf16 O / fp32
//    LSE when the slice holds the whole sequence, else a partial (O, LSE).
//    (Split-KV partial kernel: TokenSpeed MLA article, section 2; query-token
//    folding: section 3.)
//  * mla_combine: LSE-weighted merge of the partials of every sequence that
//    spans several slices (article, section 2, the second, reduction kernel).
//  * mla_kv_pack_fp8: latent || rope -> E4M3 rows (tokenspeed-mla package
//    page, fused K/V pack + FP8 quantisation).
#include <math.h>

#include <map>
#include <mutex>
#include <type_traits>

#include "mla_internal.h"

// Workspace of mla_decode_static (callers that cannot allocate): one copy per
// GPU, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it only stands in for the symbol); it uses the
// device address that static_scratch() looks up per device.
static __device__ __align__(256) uint8_t scratch[mla::kStaticScratchBytes];

namespace mla {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_t;
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(4))) const int32_t cint_t;

constexpr float kTau = 32.0f;  // recompute the segment only when a row max grows past the reference by more (log2 units)
// fp16 P must stay below 65504, so its rows are recomputed once their max grows by more than 2^15
template <int DT>
constexpr float kTauOf = DT == kFp16 ? 15.0f : kTau;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kDmaPerWave = kStageBytes / 1024 / 4;  // 9 one-KiB LDS writes per wave per tile
// Epilogue staging: per wave 32 rows of 256 columns; row pitches padded by 8
// (bf16) / 16 (fp32) bytes so column-wise writes of 32 rows hit distinct banks.
constexpr int kEpiRowB16 = 256 * 2 + 8;
constexpr int kEpiRowF32 = 256 * 4 + 16;
constexpr int kEpiWaveBytes = 32 * kEpiRowF32;
static_assert(4 * kEpiWaveBytes <= kStages * kStageBytes, "epilogue staging must fit in the KV ring");
// 1 KiB LDS scratch after the ring: destination of the loads of dummy tiles
constexpr int kDummyOffset = kStages * kStageBytes;
// P exchange of the cross-wave PV layout (fp8 path, and 16-bit kernels with
// rows missing): P of the four row blocks (B-operand layout, 2 KiB each) and,
// for fp8, their per-row MFMA scales (one dword per lane, wave-major so that
// every access is conflict-free), shared by all waves
constexpr int kPOffset = kDummyOffset + 1024;
constexpr int kPScaleOffset = kPOffset + 4 * 2048;
// block-table entries of the current segment, kBtEntries at a time
constexpr int kBtOffset = kPScaleOffset + 1024;
constexpr int kBtEntries = 256;
constexpr int kLdsBytes = kBtOffset + 4 * kBtEntries;
static_assert(kBtEntries == kThreads, "one block-table entry per thread per refill");
// fp8 epilogue staging: 128 rows, pitch 1 KiB + 16 bytes
constexpr int kEpiPitch = 1024 + 16;
static_assert(kTileM * kEpiPitch <= kStages * kStageBytes, "epilogue staging must fit in the KV ring");

template <int DT>
struct Traits;
template <>
struct Traits<kFp8> {
  static constexpr int kTile = 64;        // keys per LDS tile
  static constexpr int kRowBytes = 576;   // bytes per cache row
  static constexpr int kChunks = 36;      // 16-byte chunks per row
};
template <>
struct Traits<kBf16> {
  static constexpr int kTile = 32;
  static constexpr int kRowBytes = 1152;
  static constexpr int kChunks = 72;
};
template <>
struct Traits<kFp16> : Traits<kBf16> {};  // same 2-byte rows and tiles
template <>
struct Traits<kMixed> : Traits<kFp8> {};  // E4M3 cache rows and tiles

// LDS layout of a tile: row r, 16-byte chunk c lives at chunk slot
// r * kChunks + (c ^ swz(r)).  The XOR keeps every access pattern of the
// kernel (row-wise K reads, 8/4-row transposing V reads, 1 KiB DMA writes)
// free of bank conflicts on the 64-bank LDS.
template <int DT>
__device__ __forceinline__ int swz(int r) {
  if constexpr (DT == kFp8 || DT == kMixed) {
    return (r >> 2) & 3;
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}

__device__ __forceinline__ uint32_t lds_addr(const lds_t* p) { return (uint32_t)(uintptr_t)p; }

// Direct global -> LDS copy of 16 bytes per lane; the wave's 64 lanes fill
// 1 KiB of LDS starting at m0.  Issued through inline asm so that the
// compiler neither waits on it nor reorders LDS accesses around it (memory
// clobber); completion is tracked by hand with vmcnt.
// (an SALU write of M0 needs one wait state before a load that writes LDS)
__device__ __forceinline__ void dma16_sbase(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_vaddr(const void* vaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(vaddr), "s"(m0) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight,
// then barrier the workgroup.  One asm statement: nothing moves across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_tile_barrier(int younger_tiles) {
  // younger_tiles DMA tiles (kDmaPerWave loads each) may stay in flight.
  if (younger_tiles >= 2) {
    wait_vm_barrier<2 * kDmaPerWave>();
  } else if (younger_tiles == 1) {
    wait_vm_barrier<kDmaPerWave>();
  } else {
    wait_vm_barrier<0>();
  }
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


// Score MFMAs are issued through asm so that their accumulators stay in
// VGPRs: the compiler otherwise selects the AGPR form for every MFMA of the
// kernel, and the 256 AGPRs are exactly the 32x512 fp32 output accumulator.
// The compiler does not model hazards of asm MFMAs and takes their results as
// written when the asm issues, while the hardware writes them some 64 cycles
// later.  The last MFMA of a chain therefore carries the wait states that must
// pass before anything (a VALU use, or a copy the register allocator may
// insert) reads the accumulator, inside the same asm statement.  The fp8 score
// MFMAs read only LDS-loaded, global-loaded and MFMA-written registers, so they
// need no wait states before them; the bf16 ones take operands the compiler
// may assemble with VALU moves, hence their leading s_nop.
__device__ __forceinline__ void qk_mfma_f8(v16f& acc, const v8i& a, const v8i& b, bool last) {
  if (last) {
    asm volatile(
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 7"
        : "+v"(acc)
        : "v"(a), "v"(b), "v"(127));
  } else {
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+v"(acc)
                 : "v"(a), "v"(b), "v"(127));
  }
}
// first MFMA of a chain: accumulator input is zero.  The output is early-clobber:
// a multi-pass MFMA must not write registers that hold its own A or B operand.
__device__ __forceinline__ void qk_mfma_f8_first(v16f& acc, const v8i& a, const v8i& b) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0]"
               : "=&v"(acc)
               : "v"(a), "v"(b), "v"(127));
}
template <int DT>
__device__ __forceinline__ void qk_mfma_h16(v16f& acc, const v4i& a, const v4i& b, bool last) {
  if constexpr (DT == kFp16) {
    if (last) {
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                   : "+v"(acc)
                   : "v"(a), "v"(b));
    } else {
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
    }
  } else {
    if (last) {
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                   : "+v"(acc)
                   : "v"(a), "v"(b));
    } else {
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
    }
  }
}
// MFMA with its accumulator in VGPRs, through asm (the role-specialised FP8
// kernel keeps every value in VGPRs, so that its two roles share one register
// budget).  The compiler models neither its latency nor its hazards: a
// VALU-written operand needs two wait states before it (lead), and the caller
// pads with s_nop (mfma_drain) after the last MFMA before the accumulators are
// read or rewritten by anything but another MFMA.
__device__ __forceinline__ void mfma_f8_v(v16f& acc, const v8i& a, const v8i& b, int scale_b, bool lead) {
  if (lead) {
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+v"(acc)
                 : "v"(a), "v"(b), "v"(127), "v"(scale_b));
  } else {
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+v"(acc)
                 : "v"(a), "v"(b), "v"(127), "v"(scale_b));
  }
}
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Scheduling fences.  The instruction selector places pure arithmetic next to
// its uses, regardless of where the source puts it; routing a slot's inputs
// and outputs through empty volatile asm statements pins that work between
// the MFMAs it is meant to overlap.
template <typename T>
__device__ __forceinline__ void fence_v(T& x) {
  asm volatile("" : "+v"(x));
}
// max / sum of a value with the one held 32 lanes away (v_permlane32_swap)
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Keep a 16-float accumulator block in AGPRs: values defined by VALU code
// (zero-init, the reset before a recomputation) are moved there so the loop-carried output tile never
// gets a VGPR copy.
__device__ __forceinline__ void pin_agpr(v16f& x) { asm volatile("" : "+a"(x)); }

// This lane's index (0..63), recomputed where it is used: an opaque instruction pair that the
// compiler cannot hoist, so no register holds the lane id across a segment loop (in the kernels
// that use all 512 registers such a value spills).
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Work units of the KV partition are one LDS tile of the kernel: UK = 64 keys
// (E4M3 tiles) or 32 (16-bit tiles).  A sequence has at least one unit.
template <int UK>
__device__ __forceinline__ int units_of(int L) { return L > 0 ? (L + UK - 1) / UK : 1; }
// First key any query token of a sequence of length L can see, rounded down
// to a unit: 0 without a sliding window, else the earliest window start
// (token 0's, n_0 - window) rounded down.  A query group's work is the units
// from there to the last key it sees; tiles before it are never read.
template <int UK>
__device__ __forceinline__ int seq_key0(int L, int q_len, int window) {
  if (window <= 0) return 0;
  const long long lo = (long long)L - q_len + 1 - window;
  return lo > 0 ? (int)(lo & ~(long long)(UK - 1)) : 0;
}

// Butterfly reduction over the 64 lanes with no lane-index registers: v_permlane32_swap pairs
// lane i with lane i ^ 32, then ds_swizzle in bit-mask mode (and-mask 31, xor-mask k) pairs each
// lane with lane i ^ k inside its half, for k = 16, 8, 4, 2, 1.  Every lane ends with the result.
// (A shuffle by lane index would keep six loop-invariant index registers live, and spill them.)
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  int x = __builtin_bit_cast(int, v);
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);  // {own, partner} in some order
  v = op(__builtin_bit_cast(T, (int)r[0]), __builtin_bit_cast(T, (int)r[1]));
#pragma unroll
  for (int k = 16; k > 0; k >>= 1) {
    x = __builtin_bit_cast(int, v);
    int y;
    switch (k) {  // the swizzle pattern is an immediate
      case 16: y = __builtin_amdgcn_ds_swizzle(x, (16 << 10) | 31); break;
      case 8: y = __builtin_amdgcn_ds_swizzle(x, (8 << 10) | 31); break;
      case 4: y = __builtin_amdgcn_ds_swizzle(x, (4 << 10) | 31); break;
      case 2: y = __builtin_amdgcn_ds_swizzle(x, (2 << 10) | 31); break;
      default: y = __builtin_amdgcn_ds_swizzle(x, (1 << 10) | 31); break;
    }
    v = op(v, __builtin_bit_cast(T, y));
  }
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ int wave_min_i32(int v) {
  return wave_reduce(v, [](int a, int b) { return min(a, b); });
}
__device__ __forceinline__ int wave_max_i32(int v) {
  return wave_reduce(v, [](int a, int b) { return max(a, b); });
}
// Inclusive prefix sum over the 64 lanes of a wave, on DPP moves (no LDS
// traffic): shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then the
// last lane of rows 0 and 2 is added into rows 1 and 3, and the last lane of
// row 1 into rows 2 and 3.  64-bit values move as two 32-bit halves.
template <int CTRL, int ROWS>
__device__ __forceinline__ long long dpp_move_ll(long long v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(v & 0xffffffffll), CTRL, ROWS, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, ROWS, 0xf, true);
  return (long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ long long wave_incl_scan_ll(long long v) {
  v += dpp_move_ll<0x111, 0xf>(v);  // row_shr:1
  v += dpp_move_ll<0x112, 0xf>(v);  // row_shr:2
  v += dpp_move_ll<0x114, 0xf>(v);  // row_shr:4
  v += dpp_move_ll<0x118, 0xf>(v);  // row_shr:8
  v += dpp_move_ll<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move_ll<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
__device__ __forceinline__ long long readlane_ll(long long v, int l) {
  const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffffll), l);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
  return (long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}

// two probabilities in the PV operand format (bf16 or fp16, round to nearest even)
// (one v_cvt_pk_{bf16,f16}_f32; a lands in the low half)
template <int DT>
__device__ __forceinline__ uint32_t pack_p16x2(float a, float b) {
  if constexpr (DT == kFp16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2h));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
  }
}
// The two probabilities of a packed word as the PV product sees them, summed in fp32.
template <int DT>
__device__ __forceinline__ float sum_p16x2(uint32_t w) {
  if constexpr (DT == kFp16) {
    const v2f f = __builtin_convertvector(__builtin_bit_cast(v2h, w), v2f);
    return f[0] + f[1];
  } else {
    return __builtin_bit_cast(float, w << 16) + __builtin_bit_cast(float, w & 0xffff0000u);
  }
}
template <int DT>
__device__ __forceinline__ v16f pv_mfma_h16(const v4i& v, const v4i& pw, const v16f& acc) {
  if constexpr (DT == kFp16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, v), __builtin_bit_cast(v8h, pw), acc, 0, 0,
                                                  0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, v), __builtin_bit_cast(v8bf, pw), acc, 0,
                                                   0, 0);
  }
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}
// eight E4M3 codes (in byte order) -> eight bf16 values, exactly (every E4M3
// value is a bf16 value)
__device__ __forceinline__ v4i widen_e4m3_bf16(const v2i& x) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true);
  return v4i{__builtin_bit_cast(int, a), __builtin_bit_cast(int, b), __builtin_bit_cast(int, c),
             __builtin_bit_cast(int, d)};
}

// Epilogue stores: the final O of a sequence held by one slice goes out
// non-temporal (no dirty lines left for the kernel-end writeback); a split
// partial uses an ordinary store, so the merge that follows finds it in cache.
__device__ __forceinline__ void store_out(const v4i& v, v4i* dst, bool final_out) {
  if (final_out) {
    __builtin_nontemporal_store(v, dst);
  } else {
    *dst = v;
  }
}

// ---------------------------------------------------------------------------
// Balanced partition of one workgroup row's KV work (a query group g, one row
// tile): sequence b owns group_units(b, g) consecutive units (one LDS tile
// each); slice w of G covers units [w*T/G, (w+1)*T/G) of the row's total T.
// Every (slice, sequence) intersection is one segment; its partial lives in
// workspace slot w + b (unique along the monotone staircase of segments).
// ---------------------------------------------------------------------------
// Slice w of a row whose work costs C starts at position w C / G; position x lies in slice
// slice_of_unit(x, C, G).
__device__ __forceinline__ long long slice_start(long long w, long long T, int G) { return (w * T) / G; }
__device__ __forceinline__ int slice_of_unit(long long u, long long T, int G) {
  return (int)(((u + 1) * (long long)G - 1) / T);
}

struct SegmentCtx {
  int b, u0, u1, slot;
  bool single;
  int L, qlen, tok0;  // sequence b: keys (clamped at 0), new tokens, first token row (seq_tokens)
};

// ---------------------------------------------------------------------------
// One segment: rows of (b, group g, m-tile mt) against keys [64*u0, 64*u1).
//
// Softmax bookkeeping: each row's probabilities are taken relative to a
// reference m_ref fixed at the row's first tile with a visible key, so the
// output accumulators are only ever touched by MFMA (no rescale in the loop).
// If a later tile's row max exceeds m_ref by more than kTauOf<DT> (log2 units), the
// result could overflow: the workgroup then recomputes the segment with
// m_ref set to the exact row maxima seen in the first pass.
// ---------------------------------------------------------------------------
// New query tokens of sequence b, and the index of its first one among q's and
// out's token rows: q_len each in a uniform batch ([B, q_len, H, ...]), or each
// sequence's own count from cumulative offsets in a ragged one ([total_q, H,
// ...]).  Offsets are clamped so that every read stays inside the q tensor.
__device__ __forceinline__ void seq_tokens(const PartialParams& p, int b, int& qlen_b, int& tok0) {
  if (p.cu_q == nullptr) {
    qlen_b = p.q_len;
    tok0 = b * p.q_len;
  } else {
    cint_t* cu = (cint_t*)p.cu_q;
    const int c0 = min(max(cu[b], 0), p.total_q);
    const int c1 = min(max(cu[b + 1], c0), p.total_q);
    tok0 = c0;
    qlen_b = min(c1 - c0, p.q_len);
  }
}

// Units of query group g of sequence b: from the sequence's first unit to the
// last key the group's last token sees.  A group holding no token of the
// sequence (a ragged batch's shorter sequences) keeps one empty unit, so every
// (group, sequence) pair has at least one.
template <int UK>
__device__ __forceinline__ int group_units_of(const PartialParams& p, int L, int qlen_b, int g, int window) {
  const int gF = g * p.F;
  if (qlen_b <= gF) return 1;
  const int n_gmax = min(max(L - qlen_b + gF + p.F, 0), L);
  return units_of<UK>(n_gmax - seq_key0<UK>(L, qlen_b, window));
}

// Sequences of at most this many keys take the second P term.  The E4M3 rounding of P moves a
// row's output by up to ~2^-4 of the weight its few largest keys carry; over many keys the
// weights spread and the per-key errors average out.  Measured with the single term, beyond the
// output's bf16 rounding: up to 4.9e-2 in sequences below this length, at most 2.2e-2 above it.
constexpr int kLoKeys = 8192;

// XPV (16-bit paths): the fp8 path's cross-wave PV layout instead of the own-rows one.
// LO (E4M3): P goes out in two terms, E4M3 codes and E2M1 codes of their rounding residuals.
template <int DT, bool FAST, bool WIN, bool XPV, bool LO = false>
__device__ __forceinline__ void run_segment(const PartialParams& p, lds_t* smem, int* s_flag, const SegmentCtx& sg,
                                            int g, int mt, int wave, int lane) {
  using TR = Traits<DT>;
  constexpr int TILE = TR::kTile;
  constexpr int RB = TR::kRowBytes;
  constexpr int CH = TR::kChunks;
  constexpr int ESZ = (DT == kFp8) ? 1 : 2;

  // Opaque copies of the lane and wave ids: everything derived from them is
  // computed inside this segment instead of being hoisted above the caller's
  // segment loop, where it would stay live (and spill) across the whole kernel.
  asm volatile("" : "+v"(lane));
  asm volatile("" : "+s"(wave));
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int L = sg.L, qlen_b = sg.qlen, tok0 = sg.tok0;
  const int gF = g * p.F;
  // folded rows that hold a token of this sequence (fewer than H_eff only in the
  // last query group of a ragged batch's shorter sequences; none past its end)
  const int rows_valid = min(p.H_eff, max(qlen_b - gF, 0) * p.H);
  if (rows_valid <= mt * kTileM) return;  // a ragged batch's query group past this sequence's tokens
  // keys visible to the last token of this query group
  const int n_gmax = min(max(L - qlen_b + gF + p.F, 0), L);
  const int window = WIN ? p.window : 0;  // sliding window (kernels built without one fold it away)
  const int kbase = seq_key0<TILE>(L, qlen_b, window);  // unit 0 of the sequence starts here
  const int k0 = kbase + sg.u0 * TILE;
  const int k1 = min(kbase + sg.u1 * TILE, n_gmax);

  // this lane's query row (row n of the wave's 32)
  const int r = 32 * wave + n;
  const int m = mt * kTileM + r;
  const bool row_valid = m < rows_valid;
  int h_div = p.H;
  asm volatile("" : "+s"(h_div));  // (the division's reciprocal is then not hoisted above the segment loop)
  const int fold = row_valid ? m / h_div : 0;
  const int t_tok = gF + fold;
  const int n_row = row_valid ? min(max(L - qlen_b + t_tok + 1, 0), L) : 0;
  const int lim = min(n_row, k1);  // keys [max(k0, lo), lim) are visible to this row
  const int lo = window > 0 ? max(n_row - window, 0) : 0;  // sliding-window start
  // Masking bound of this row, (key - lo) unsigned >= vis for masked keys: below
  // lo or at/after lim.  With a window it is rebuilt where a tile is masked, so
  // that at most one per-row value stays live across the loop for it: an opaque
  // copy of n_row (fp8), or none (16-bit paths, whose registers are fuller: n_row
  // is recomputed from the lane id and uniform values).
  auto mask_bounds = [&](int& lo_m, uint32_t& vis_m) {
    if constexpr (WIN) {
      int nr;
      if constexpr (DT == kFp8) {
        nr = n_row;
        asm volatile("" : "+v"(nr));
      } else {
        int ln = lane, hh_ = p.H;
        asm volatile("" : "+v"(ln), "+s"(hh_));  // nothing of the division is hoisted out of the loop
        const int m_ = mt * kTileM + 32 * wave + (ln & 31);
        nr = m_ < rows_valid ? min(max(L - qlen_b + gF + m_ / hh_ + 1, 0), L) : 0;
      }
      lo_m = window > 0 ? max(nr - window, 0) : 0;
      vis_m = (uint32_t)max(min(nr, k1) - lo_m, 0);
    } else {
      lo_m = 0;
      vis_m = (uint32_t)lim;
    }
  };
  const size_t rows_per_b = (size_t)p.q_len * p.H;  // rows of a sequence's workspace slot
  const size_t out_row0 = (size_t)tok0 * p.H;       // the sequence's first row of out / lse
  const bool wave_active = (mt * kTileM + 32 * wave) < rows_valid;

  // ---- Q rows into registers, laid out as the B operand of S^T = K Q^T ----
  // (invalid rows read row 0 of the group and are zeroed: no divergent branches)
  // fp8 Q takes the direct-to-LDS path at the start of the tile pipeline below;
  // bf16 Q (twice the bytes: the whole ring) is loaded here.
  constexpr int QSTEPS = (DT == kFp8) ? 9 : 36;
  v8i qreg[QSTEPS];
  if constexpr (DT != kFp8) {
    const size_t qrow_idx = ((size_t)tok0 + gF) * p.H + (size_t)(row_valid ? m : 0);
    const uint8_t* qrow = p.q + qrow_idx * kDqk * ESZ;
    const int keep = row_valid ? -1 : 0;
#pragma unroll
    for (int c = 0; c < QSTEPS; ++c) {
      // (bf16 q over an E4M3 cache: step c holds dims 32(c/2) + 16hh + 8(c%2) + [0, 8), the order
      // in which that kernel reads its K operands, 16 bytes per pair of steps)
      const int d0 = DT == kMixed ? 32 * (c >> 1) + 16 * hh + 8 * (c & 1) : 16 * c + 8 * hh;
      const v4i x = *(const v4i*)(qrow + 2 * d0) & keep;
      qreg[c] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    }
    // Q must be in registers before the KV ring starts: the compiler cannot see the
    // asynchronous LDS loads, so its own wait for Q would otherwise drain the ring.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0), expcnt/lgkmcnt unconstrained
  }

  v16f o[16];
  float m_ref = -INFINITY;  // reference the accumulators are relative to (log2 units)
  float l_acc = 0.f;        // this lane's share of sum exp2(s - m_ref)
  float l_acc_r = 0.f;      // the same over P as rounded for the PV MFMA (E4M3): normalises O
  // 16-bit P keeps that rounded sum in LDS instead (one slot per lane, in the E4M3 P-scale
  // area these kernels leave unused): the register-bound loop holds no second sum
  typedef __attribute__((address_space(3))) float lds_f32;
  auto lr_slot = [&]() { return (lds_f32*)(smem + kPScaleOffset + 256 * wave + 4 * lane); };
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    o[i] = v16f{0};
    pin_agpr(o[i]);
  }

  if (k1 > k0) {
    const int ntiles = (k1 - k0 + TILE - 1) / TILE;
    const int pmask = p.page_size - 1;
    cint_t* bt = (cint_t*)p.block_table + (size_t)sg.b * p.max_pages;
    // last block_table entry this segment may read (never past the row, even for bad seq_lens)
    const int plast = min((k1 - 1) >> p.page_shift, p.max_pages - 1);
    const uint32_t smem_base = lds_addr(smem);

    // Per-lane DMA geometry: wave instruction kk writes LDS chunk slots
    // [64*(wave+4kk), +64); lane -> slot -> (row, source chunk), kept packed
    // as row << 16 | (row*RB + chunk*16) (that byte offset is below 2^16).
    // The nine values stay in registers, except in the cross-wave 16-bit kernels
    // (twice the Q registers, plus the P exchange) and the bf16-q / E4M3 ones
    // (widening temporaries), which recompute each one where the load is issued.
    constexpr bool kGeoRegs = DT == kFp8 || (!XPV && DT != kMixed);
    auto dma_geo = [&](int kk) -> uint32_t {
      int ln = lane;
      if constexpr (!kGeoRegs) asm volatile("" : "+v"(ln));
      const int slot = 64 * (wave + 4 * kk) + ln;
      const int row = slot / CH;
      const int col = ((slot - row * CH) ^ swz<DT>(row)) * 16;
      return ((uint32_t)row << 16) | (uint32_t)(row * RB + col);
    };
    uint32_t dgeo[kDmaPerWave];
#pragma unroll
    for (int kk = 0; kk < kDmaPerWave; ++kk) dgeo[kk] = kGeoRegs ? dma_geo(kk) : 0u;

    // fp8: the segment's block-table entries are staged in LDS (kBtEntries at
    // a time, refilled when the tiles run past them) and read from there one
    // tile ahead.  A scalar load in the loop would make the next wait for LDS
    // data wait for the scalar load as well (they share a counter and the
    // scalar one completes out of order).  The bf16 path keeps scalar loads:
    // its 144 Q registers leave no VGPR for the staged entry, and a spill
    // reload in the loop would wait for every load in flight.
    typedef __attribute__((address_space(3))) int lds_i32;
    int bt_base = 0;
    auto bt_fill = [&](int first) {
      bt_base = first;
      const int v = bt[min(first + 64 * wave + lane, plast)];
      lds_barrier();  // every wave is done with the previous entries
      *(lds_i32*)(smem + kBtOffset + 4 * (64 * wave + lane)) = v;
      lds_barrier();
    };
    auto page_raw = [&](int pidx) -> int {
      if constexpr (DT == kFp8) {
        return *(const lds_i32*)(smem + kBtOffset + 4 * (min(pidx, plast) - bt_base));
      } else {
        return bt[min(pidx, plast)];
      }
    };
    auto clamp_page = [&](int pg) -> int {
      return min(max(__builtin_amdgcn_readfirstlane(pg), 0), p.num_pages - 1);
    };

    // Scalar state of the tile whose loads are being issued.  Block-table
    // entries are read one tile ahead, so the scalar-load wait lands at the
    // top of an iteration rather than inside an MFMA chain.  A tile index past
    // the segment sets up a dummy tile: its loads re-read row 0 of the last
    // real tile (an L2 hit) into a 1 KiB scratch area of LDS, which keeps the
    // number of loads per iteration, and hence every vmcnt wait, uniform.
    const uint8_t* d_base = p.kv;
    uint32_t d_m0 = smem_base, d_step = 1024;
    int d_nvalid = 0, d_key0 = k0, d_pidx0 = 0;
    int d_pg0 = 0, d_pg1 = 0, d_pg2 = 0, d_pg3 = 0;
    int pf0 = 0, pf1 = 0, pf2 = 0, pf3 = 0;
    auto prefetch_pages = [&](int tt) {
      const int pidx0 = (k0 + tt * TILE) >> p.page_shift;
      // refill at fixed tile counts (a test of bt_base here would make the DMA
      // addresses look divergent to the compiler): a tile needs at most one
      // entry when pages are at least a tile long, at most four otherwise
      constexpr int kFillTiles = FAST ? kBtEntries : (kBtEntries - 3) / 4;
      if constexpr (DT == kFp8) {
        if (tt > 0 && tt % kFillTiles == 0) bt_fill(pidx0);
      }
      pf0 = page_raw(pidx0);
      if constexpr (!FAST) {
        pf1 = page_raw(pidx0 + 1);
        pf2 = page_raw(pidx0 + 2);
        pf3 = page_raw(pidx0 + 3);
      }
    };
    auto dma_setup = [&](int tt) {
      if (tt < ntiles) {
        const int key0 = k0 + tt * TILE;
        d_m0 = smem_base + (uint32_t)((tt % kStages) * kStageBytes);
        d_step = 1024;
        d_nvalid = min(TILE, k1 - key0);
        d_key0 = key0;
        d_pidx0 = key0 >> p.page_shift;
        if constexpr (FAST) {
          d_base = p.kv + ((size_t)clamp_page(pf0) * p.page_size + (key0 & pmask)) * RB;
        } else {
          d_pg0 = clamp_page(pf0);
          d_pg1 = clamp_page(pf1);
          d_pg2 = clamp_page(pf2);
          d_pg3 = clamp_page(pf3);
        }
        if (tt + 1 < ntiles) prefetch_pages(tt + 1);
      } else {
        d_m0 = smem_base + (uint32_t)kDummyOffset;
        d_step = 0;
        d_nvalid = 0;
      }
    };
    // load kk (of kDmaPerWave) of this wave for the tile set up last
    auto dma_issue = [&](int kk) {
      const uint32_t g = kGeoRegs ? dgeo[kk] : dma_geo(kk);
      const int row = (int)(g >> 16);
      const uint32_t off = g & 0xffffu;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(d_m0 + d_step * (uint32_t)(wave + 4 * kk));
      // Tiles of pages at least a tile long (and every fp8 tile) are loaded whole and
      // their rows past the segment's last key are zeroed in LDS afterwards (zero_tail);
      // 16-bit tiles over shorter pages re-read row 0 there (the next page may not exist).
      constexpr bool kClampRows = DT != kFp8 && !FAST;
      if constexpr (FAST) {
        // page_size >= TILE: the tile is TILE consecutive rows of one page
        const uint32_t voff = (!kClampRows || row < d_nvalid) ? off : off - (uint32_t)(row * RB);
        dma16_sbase(voff, d_base, m0);
      } else {
        // page_size < TILE: up to four pages per tile
        const int key = d_key0 + ((!kClampRows || row < d_nvalid) ? row : 0);
        const int rel = (key >> p.page_shift) - d_pidx0;
        // readfirstlane (a no-op on these uniform values) keeps the per-lane select
        // a select of values: a select of loads would be folded into a load through
        // a selected address, which pins the captured variables in private memory
        const int g0 = __builtin_amdgcn_readfirstlane(d_pg0), g1 = __builtin_amdgcn_readfirstlane(d_pg1);
        const int g2 = __builtin_amdgcn_readfirstlane(d_pg2), g3 = __builtin_amdgcn_readfirstlane(d_pg3);
        const int pg = rel == 0 ? g0 : rel == 1 ? g1 : rel == 2 ? g2 : g3;
        const uint8_t* src = p.kv + ((size_t)pg * p.page_size + (key & pmask)) * RB + (off - (uint32_t)(row * RB));
        dma16_vaddr(src, m0);
      }
    };
    auto issue_tile = [&](int tt) {
      dma_setup(tt);
#pragma unroll
      for (int kk = 0; kk < kDmaPerWave; ++kk) dma_issue(kk);
    };

    // smallest visible limit and largest window start over the wave's rows:
    // tiles inside [lo_max, lim_min) need no mask
    const int lim_min = wave_min_i32(lim), lo_max = wave_max_i32(lo);
    auto tile_needs_mask = [&](int key0) { return key0 + TILE > lim_min || key0 < lo_max; };

    // per-lane LDS read geometry
    int kaddr[4];
    int vaddr[4];
    if constexpr (DT == kFp8) {
      const int sw = (n >> 2) & 3;
      kaddr[0] = n * RB + (((2 * hh) ^ sw) * 16);
      kaddr[1] = n * RB + (((2 * hh + 1) ^ sw) * 16);
      kaddr[2] = kaddr[3] = 0;
      // transposing V reads: source-lane roles inside each 16-lane group
      const int grp = lane >> 4, hs = grp >> 1, dsub = grp & 1, uu = lane & 15, rr = uu >> 1, c8 = uu & 1;
      const int kbase = 8 * (rr >> 2) + 4 * hs + (rr & 3);
      const int s8 = (2 * (rr >> 2) + hs) & 3;
      vaddr[0] = kbase * RB + (((0 + dsub) ^ s8) * 16) + 8 * c8;
      vaddr[1] = kbase * RB + (((2 + dsub) ^ s8) * 16) + 8 * c8;
      vaddr[2] = vaddr[3] = 0;
    } else if constexpr (DT == kMixed) {
      // K: sixteen E4M3 codes of key row n per pair j of 16-dim steps, dims [32j + 16hh, +16)
      // (16-byte chunk 2j + hh: slot hh of its group of four for even j, 2 + hh for odd j);
      // V: the transposing 8-bit reads of the fp8 path, one read per operand
      const int sw = (n >> 2) & 3;
      kaddr[0] = n * RB + ((hh ^ sw) * 16);
      kaddr[1] = n * RB + (((2 + hh) ^ sw) * 16);
      kaddr[2] = kaddr[3] = 0;
      const int grp = lane >> 4, hs = grp >> 1, dsub = grp & 1, uu = lane & 15, rr = uu >> 1, c8 = uu & 1;
      const int kbase = 8 * (rr >> 2) + 4 * hs + (rr & 3);
      const int s8 = (2 * (rr >> 2) + hs) & 3;
      // (cross-wave PV: + this wave's 128 latent dims, 4 blocks of 32 dims, 2 chunks of 16 bytes each)
      vaddr[0] = kbase * RB + (((0 + dsub) ^ s8) * 16) + 8 * c8 + (XPV ? 128 * wave : 0);
      vaddr[1] = kbase * RB + (((2 + dsub) ^ s8) * 16) + 8 * c8 + (XPV ? 128 * wave : 0);
      vaddr[2] = vaddr[3] = 0;
    } else {
      const int sw = swz<DT>(n);
#pragma unroll
      for (int x = 0; x < 4; ++x) kaddr[x] = n * RB + (((2 * x + hh) ^ sw) * 16);
      const int grp = lane >> 4, hs = grp >> 1, dsub = grp & 1, uu = lane & 15, rr = uu >> 2, c4 = uu & 3;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int sv = ((rr >> 1) << 2) | ((2 * v + hs) & 3);
        const int krow = 8 * v + 4 * hs + rr;
#pragma unroll
        for (int x = 0; x < 2; ++x)  // (cross-wave PV: + this wave's 128 latent dims)
          vaddr[2 * v + x] = krow * RB + (((4 * x + 2 * dsub + (c4 >> 1)) ^ sv) * 16) + 8 * (c4 & 1) + (XPV ? 256 * wave : 0);
      }
    }

    float m_init = -INFINITY;
#pragma unroll 1
    for (int attempt = 0; attempt < 2; ++attempt) {
      float m_seen = -INFINITY;
      bool ovf = false;
      m_ref = m_init;
      l_acc = 0.f;
      l_acc_r = 0.f;
      if constexpr (DT != kFp8) *lr_slot() = 0.f;
      if (attempt > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          o[i] = v16f{0};
          pin_agpr(o[i]);
        }
      }
      // all waves are done with the previous use of the LDS ring (bt_fill starts with a barrier)
      if constexpr (DT == kFp8) {
        bt_fill(k0 >> p.page_shift);
      } else {
        lds_barrier();
      }
      prefetch_pages(0);

      if constexpr (DT == kFp8) {
        // Software pipeline, iteration t (one 64-key tile):
        //   wait for tile t; set up the loads of tile t+2;
        //   score MFMAs of tile t, interleaved with the loads of tile t+2 and
        //     the second half of tile t-1's softmax (keys 32..63);
        //   PV MFMAs of tile t-1, interleaved with the first half of tile t's
        //     softmax (row max, scale, keys 0..31).
        // Ring stages in use during iteration t: t-1 (PV), t (scores), t+1 and
        // t+2 (loads in flight).  LDS operands are read three MFMAs ahead.
        auto kread = [&](const lds_t* st, int c, int kb) -> v8i {
          const v4i x = *(const lds_v4i*)(st + kaddr[0] + 64 * c + 32 * RB * kb);
          const v4i y = *(const lds_v4i*)(st + kaddr[1] + 64 * c + 32 * RB * kb);
          return v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        };
        auto vread = [&](const lds_t* st, int db) -> v8i {
          const int base = vaddr[db & 1] + 64 * (db >> 1);
          const v2i r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base));
          const v2i r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base + 16 * RB));
          const v2i r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base + 32 * RB));
          const v2i r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base + 48 * RB));
          return v8i{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
        };
        v16f s0, s1;            // scores of the tile passing through the score MFMAs
        v16f hb;                // keys 32..63 of the previous tile's scores
        int pa[4], pb[4];       // fp8 P words: keys 0..31 and 32..63
        // (LO) E2M1 codes of half the E4M3 rounding residual of each P element: nibble k of
        // la / lb belongs to byte k of pa / pb
        int la[2] = {0, 0}, lb[2] = {0, 0};
        float pe_off = 0.f;     // exp2 offset of the tile whose P is being built
        int pe_e = 0;           // its power-of-two scale
        float lsum = 0.f, lsum_r = 0.f, mx_raw = -INFINITY, p_hold = 0.f;
        int w_hold = 0;

        // softmax, first half (PV slots 0..15): row max over the tile (tree, two
        // slots), reference and scale (two slots), then P of keys 0..31 (two
        // elements per slot in slots 4..7, one in slots 8..15)
        float mx0 = -INFINITY;
        auto max16 = [&](const v16f& x) -> float {
          const float a0 = fmaxf(fmaxf(x[0], x[1]), x[2]), a1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
          const float a2 = fmaxf(fmaxf(x[6], x[7]), x[8]), a3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
          const float a4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
          return fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), x[15]));
        };
        // The exponentials run as a three-stage pipeline across MFMA slots
        // (fma in one slot, exp2 in the next, sum and fp8 pack in the one after),
        // so the VALU work inside a slot has no dependency chain to wait on.
        float ya[2], yb[2], qa[2], qb[2];  // pair stages: fma results, exp2 results
        // Returns the sum of the two values as rounded to E4M3: O is normalised by the sum of
        // the weights the PV product used, so they sum to one (a row that sees one key returns
        // that key's V exactly); the LSE keeps the exact sum.
        auto pack_pair = [&](float p0, float p1, int pair, int* words, int* lo) -> float {
          // pair j holds elements 2j, 2j+1: even pairs fill the low half of word j/2, odd pairs the high
          v2f r;
          if ((pair & 1) == 0) {
            w_hold = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
            fence_v(w_hold);
            r = __builtin_amdgcn_cvt_pk_f32_fp8(w_hold, false);
          } else {
            words[pair >> 1] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, w_hold, true);
            fence_v(words[pair >> 1]);
            r = __builtin_amdgcn_cvt_pk_f32_fp8(words[pair >> 1], true);
          }
          if constexpr (LO) {
            // the residuals as E2M1 codes of half their value (every p is at most 256 here, so a
            // residual is at most 8) into byte pair % 4 of lo word pair / 4 (byte selects must be
            // literal constants)
            const float d0 = p0 - r[0], d1 = p1 - r[1];
            uint32_t lw = (uint32_t)lo[pair >> 2];
            switch (pair & 3) {
              case 0: lw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lw, d0, d1, 2.f, 0); break;
              case 1: lw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lw, d0, d1, 2.f, 1); break;
              case 2: lw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lw, d0, d1, 2.f, 2); break;
              default: lw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lw, d0, d1, 2.f, 3); break;
            }
            lo[pair >> 2] = (int)lw;
          }
          return r[0] + r[1];
        };
        auto part_a = [&](int slot, int key0, bool need_mask) {
          if (slot == 0) {
            if (need_mask) {
              int lo_m;
              uint32_t vis_m;
              mask_bounds(lo_m, vis_m);
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = key0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                if ((uint32_t)(key - lo_m) >= vis_m) s0[r] = -INFINITY;
                if ((uint32_t)(key + 32 - lo_m) >= vis_m) s1[r] = -INFINITY;
              }
            }
            fence_v(s0);
            mx0 = max16(s0);
            fence_v(mx0);
          } else if (slot == 1) {
            fence_v(s1);
            mx_raw = fmaxf(mx0, max16(s1));
            fence_v(mx_raw);
          } else if (slot == 2) {
            const float mx = mx_raw * p.s_scale_log2;  // lane max, log2 units
            mx_raw = xor32_max(mx);                     // row max of the tile
            m_seen = fmaxf(m_seen, mx_raw);
            if (m_ref == -INFINITY) m_ref = mx_raw;
            ovf = ovf || (mx_raw > m_ref + kTau);
            fence_v(mx_raw);
            fence_v(m_seen);
            fence_v(m_ref);
          } else if (slot == 3) {
            const float rm = mx_raw;
            const float mref = m_ref > -INFINITY ? m_ref : 0.f;
            // power-of-two block scale per query row: the row's largest p of this tile lands
            // in (128, 256].  The MFMA's 32-element scale blocks of a column interleave both
            // lane halves (bytes 0-15 of lanes n and n+32 take lane n's scale, bytes 16-31
            // take lane n+32's), so both halves of a row must carry the same scale.
            int e = 0;
            if (rm > -INFINITY) e = 8 - (int)ceilf(rm - mref);
            e = min(max(e, -120), 120);
            pe_e = e;
            pe_off = mref - (float)e;
            lsum = 0.f;
            lsum_r = 0.f;
            fence_v(pe_off);
            fence_v(pe_e);
          } else if (slot >= 4 && slot < 14) {
            // P of keys 0..31 (elements of s0) in pairs: slot 4+t sums/packs pair t-2,
            // exponentiates pair t-1 and scales pair t
            const int t = slot - 4;
            fence_v(s0);
            if (t >= 2) {
              const int j = t - 2;
              lsum += qa[j & 1] + qb[j & 1];
              lsum_r += pack_pair(qa[j & 1], qb[j & 1], j, pa, la);
              fence_v(lsum);
              fence_v(lsum_r);
            }
            if (t >= 1 && t <= 8) {
              const int j = t - 1;
              qa[j & 1] = __builtin_amdgcn_exp2f(ya[j & 1]);
              qb[j & 1] = __builtin_amdgcn_exp2f(yb[j & 1]);
              fence_v(qa[j & 1]);
              fence_v(qb[j & 1]);
            }
            if (t <= 7) {
              ya[t & 1] = __builtin_fmaf(s0[2 * t], p.s_scale_log2, -pe_off);
              yb[t & 1] = __builtin_fmaf(s0[2 * t + 1], p.s_scale_log2, -pe_off);
              fence_v(ya[t & 1]);
              fence_v(yb[t & 1]);
            }
          }
        };
        // softmax, second half (score slots 0..17): P of keys 32..63 (from hb), one
        // element per slot through the same three stages, then the row sum
        auto part_b = [&](int slot) {
          fence_v(hb);  // (in place: no copy)
          if (slot >= 2) {
            const int k = slot - 2;  // sum and pack element k (the rounded sum pair by pair)
            lsum += qa[k & 1];
            fence_v(lsum);
            if ((k & 1) == 0) {
              p_hold = qa[k & 1];
              fence_v(p_hold);
            } else {
              lsum_r += pack_pair(p_hold, qa[k & 1], k >> 1, pb, lb);
              fence_v(lsum_r);
            }
          }
          if (slot >= 1 && slot <= 16) {
            const int k = slot - 1;
            qa[k & 1] = __builtin_amdgcn_exp2f(ya[k & 1]);
            fence_v(qa[k & 1]);
          }
          if (slot <= 15) {
            ya[slot & 1] = __builtin_fmaf(hb[slot], p.s_scale_log2, -pe_off);
            fence_v(ya[slot & 1]);
          }
          if (slot == 17) {
            l_acc += __builtin_ldexpf(lsum, -pe_e);
            l_acc_r += __builtin_ldexpf(lsum_r, -pe_e);
            fence_v(l_acc);
            fence_v(l_acc_r);
          }
        };
        // S^T = K Q^T for one tile: two 32-key blocks, K = 576 in 9 steps of 64
        auto qk_chain = [&](const lds_t* st, bool with_b) {
          if constexpr (!FAST) {
#pragma unroll
            for (int kk = 0; kk < kDmaPerWave; ++kk) dma_issue(kk);
          }
          v8i kb[4];
          kb[0] = kread(st, 0, 0);
          kb[1] = kread(st, 0, 1);
          kb[2] = kread(st, 1, 0);
#pragma unroll
          for (int i = 0; i < 18; ++i) {
            if (i + 3 < 18) kb[(i + 3) & 3] = kread(st, (i + 3) >> 1, (i + 3) & 1);
            if (i & 1) {
              if (i == 1) {
                qk_mfma_f8_first(s1, kb[i & 3], qreg[i >> 1]);
              } else {
                qk_mfma_f8(s1, kb[i & 3], qreg[i >> 1], i == 17);
              }
              if constexpr (FAST) dma_issue(i >> 1);
            } else {
              if (i == 0) {
                qk_mfma_f8_first(s0, kb[i & 3], qreg[i >> 1]);
              } else {
                qk_mfma_f8(s0, kb[i & 3], qreg[i >> 1], i == 16);
              }
            }
            if (with_b) part_b(i);
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        // this wave's P (its 32 rows, B-operand layout) and per-row scale into LDS
        // (LO) The second term of a tile's P goes into the rope columns of the tile's own stage
        // (bytes 512..575 of its 64 rows): every wave is past the tile's scores, and the stage is
        // not reloaded before the tile's PV.  Entry 64 w + lane (16 bytes) sits at row entry / 4,
        // bytes 512 + 16 (entry % 4).
        auto lo_entry = [&](const lds_t* st, int e) -> const lds_t* { return st + (e >> 2) * RB + 512 + 16 * (e & 3); };
        auto p_publish = [&](const lds_t* st) {
          lds_t* pw = smem + kPOffset + wave * 2048;
          *(lds_v4i*)(pw + 16 * lane) = v4i{pa[0], pa[1], pa[2], pa[3]};
          *(lds_v4i*)(pw + 1024 + 16 * lane) = v4i{pb[0], pb[1], pb[2], pb[3]};
          *(__attribute__((address_space(3))) int*)(smem + kPScaleOffset + 256 * wave + 4 * lane) = 127 - pe_e;
          if constexpr (LO) *(lds_v4i*)lo_entry(st, 64 * wave + lane) = v4i{la[0], la[1], lb[0], lb[1]};
        };
        // O^T += V^T P^T for this wave's 128 latent dims (4 blocks of 32) and all
        // four row blocks: each transposed V read feeds four MFMAs.  Accumulator
        // o[4j + rr] holds latent block j of row block (wave + rr) & 3 (rr = 0 is
        // this wave's own rows, whose P is still in registers).  The first two V
        // blocks are read before the P barrier (their stage landed long ago).
        v8i vb[2];
        auto pv_prefetch = [&](const lds_t* st) {
          vb[0] = vread(st, 4 * wave);
          vb[1] = vread(st, 4 * wave + 1);
        };
        auto stage = [&](int t) -> const lds_t* { return smem + (t % kStages) * kStageBytes; };
        // The segment's last tile was loaded whole: rows past its last key hold
        // whatever follows in the page (possibly NaN).  Their scores are masked,
        // but 0 * NaN would still reach O through the PV MFMA, so zero them.
        auto zero_tail = [&](int t) {
          const int nvalid = k1 - (k0 + t * TILE);
          if (nvalid < TILE) {
            lds_t* z = smem + (t % kStages) * kStageBytes + nvalid * RB;
            const int nchunks = (TILE - nvalid) * (RB / 16);
            for (int i = 64 * wave + lane; i < nchunks; i += kThreads) *(lds_v4i*)(z + 16 * i) = v4i{0, 0, 0, 0};
            lds_barrier();
          }
        };
        auto pv_chain = [&](const lds_t* st, bool with_a, int key0, bool need_mask) {
          v8i pt[4];
          int psc[4];
          pt[0] = v8i{pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
          psc[0] = 127 - pe_e;
#pragma unroll
          for (int rr = 1; rr < 4; ++rr) {
            const int r = (wave + rr) & 3;
            const v4i x = *(const lds_v4i*)(smem + kPOffset + r * 2048 + 16 * lane);
            const v4i y = *(const lds_v4i*)(smem + kPOffset + r * 2048 + 1024 + 16 * lane);
            pt[rr] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
            psc[rr] = *(const __attribute__((address_space(3))) int*)(smem + kPScaleOffset + 256 * r + 4 * lane);
          }
          // MFMA order (as 4j + rr): both own-row MFMAs of latent blocks 0 and 1
          // first, so the other waves' P has two MFMAs to arrive from LDS; V
          // blocks 0 and 1 were read before the barrier, blocks 2 and 3 are
          // read into the freed registers four MFMAs before their first use.
          constexpr int kOrder[16] = {0, 4, 1, 2, 3, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15};
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const int idx = kOrder[k], j = idx >> 2, rr = idx & 3;
            fence_v(vb[j & 1]);
            o[idx] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb[j & 1], pt[rr], o[idx], 0, 0, 0, 127, 0,
                                                                     psc[rr]);
            pin_agpr(o[idx]);
            if (with_a) part_a(k, key0, need_mask);
            if (k == 4) vb[0] = vread(st, 4 * wave + 2);
            if (k == 7) vb[1] = vread(st, 4 * wave + 3);
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (LO) {
            // The residual term: B in E2M1 (blgp 4) at twice the E4M3 term's scale, latent blocks
            // 2 and 3 (in vb) and then 0 and 1, each row block's operand read where it is used.
            // The E2M1 operand of a column: lane half h takes bytes 8h..8h+7 of the entries of
            // lanes n and n + 32 (its K-slots are those of E4M3 bytes 16h..16h+15 of both halves).
            const int hb = 8 * (lane >> 5), ln = lane & 31;
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
              const int j0 = jp == 0 ? 2 : 0;
              if (jp == 1) {
                vb[0] = vread(st, 4 * wave);
                vb[1] = vread(st, 4 * wave + 1);
              }
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int r = (wave + rr) & 3;
                const v2i l0 = *(const lds_v2i*)(lo_entry(st, 64 * r + ln) + hb);
                const v2i l1 = *(const lds_v2i*)(lo_entry(st, 64 * r + 32 + ln) + hb);
                const v8i pl = v8i{l0[0], l0[1], l1[0], l1[1], 0, 0, 0, 0};
                o[4 * j0 + rr] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb[0], pl, o[4 * j0 + rr], 0, 4, 0,
                                                                                127, 0, psc[rr] + 1);
                o[4 * j0 + 4 + rr] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    vb[1], pl, o[4 * j0 + 4 + rr], 0, 4, 0, 127, 0, psc[rr] + 1);
                pin_agpr(o[4 * j0 + rr]);
                pin_agpr(o[4 * j0 + 4 + rr]);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        };

        // Q: each wave's 32 rows (18 KiB, one contiguous block of the folded
        // query) are copied straight into ring stages 2-3, which stay free
        // until tile 2 is issued, so their latency overlaps that of tiles 0-1.
        // Rows are laid out as the KV tiles are: 16-byte chunks XOR-swizzled
        // by (row / 4) % 4 inside each group of four, so that the reads of one
        // chunk column by sixteen consecutive rows meet sixteen bank groups
        // (unswizzled, 576-byte rows put them on four).  The swizzle is made
        // on the source side: LDS chunk p of row r takes chunk p ^ ((r/4)%4).
        constexpr int kQDma = 32 * kDqk / 1024;  // 18 one-KiB loads per wave
        {
          const uint8_t* qblk = p.q + ((size_t)tok0 + gF) * p.H * kDqk;
          const uint32_t qlds = smem_base + (uint32_t)(2 * kStageBytes + wave * 32 * kDqk);
          int qlane = lane;
          asm volatile("" : "+v"(qlane));  // addresses computed here, not kept live from the segment start
#pragma unroll
          for (int kk = 0; kk < kQDma; ++kk) {
            const int o = 1024 * kk + 16 * qlane;
            const int qn = o / kDqk;
            const int pc = (o - qn * kDqk) >> 4;                  // LDS chunk of row qn
            const int lc = (pc & ~3) | ((pc & 3) ^ ((qn >> 2) & 3));  // source chunk
            const int mrow = mt * kTileM + 32 * wave + qn;
            const int src_row = mrow < rows_valid ? mrow : 0;
            dma16_vaddr(qblk + (size_t)src_row * kDqk + 16 * lc,
                        __builtin_amdgcn_readfirstlane(qlds + 1024u * (uint32_t)kk));
          }
        }
        // Every wave takes part in every tile: rows past H_eff score against
        // zero queries and are never stored.
        issue_tile(0);
        issue_tile(1);  // a dummy tile when the segment has one tile
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kDmaPerWave) : "memory");  // this wave's Q has landed
        {
          // logical chunks 4c + 2hh and 4c + 2hh + 1 of row n sit at the 32-byte pair
          // 4c + ((2hh ^ sw) & 2), in swapped order when sw = (n / 4) % 4 is odd
          const int qsw = (n >> 2) & 3;
          const lds_t* qs = smem + 2 * kStageBytes + wave * 32 * kDqk + n * kDqk + (((2 * hh) ^ qsw) & 2) * 16;
          const bool qswap = (qsw & 1) != 0;
          const int keep = row_valid ? -1 : 0;
#pragma unroll
          for (int c = 0; c < QSTEPS; ++c) {
            const v4i y0 = *(const lds_v4i*)(qs + 64 * c);
            const v4i y1 = *(const lds_v4i*)(qs + 64 * c + 16);
            const v4i x0 = (qswap ? y1 : y0) & keep;
            const v4i x1 = (qswap ? y0 : y1) & keep;
            qreg[c] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          }
        }
        // tile 0 has landed and every wave holds its Q: stages 2-3 may be refilled
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaPerWave) : "memory");
        if (ntiles == 1) zero_tail(0);
        dma_setup(2);
        qk_chain(stage(0), false);
        {
          const bool nm = tile_needs_mask(k0);
#pragma unroll
          for (int slot = 0; slot < 16; ++slot) part_a(slot, k0, nm);
        }
        for (int t = 1; t < ntiles; ++t) {
          wait_vm_barrier<kDmaPerWave>();  // tile t has landed; every wave is done with iteration t-1
          if (t == ntiles - 1) zero_tail(t);
          dma_setup(t + 2);
          hb = s1;
          qk_chain(stage(t), true);  // also finishes the softmax of tile t-1
          p_publish(stage(t - 1));
          pv_prefetch(stage(t - 1));
          lds_barrier();  // P of tile t-1 from all waves is visible
          const int key0 = k0 + t * TILE;
          pv_chain(stage(t - 1), true, key0, tile_needs_mask(key0));
        }
        hb = s1;
#pragma unroll
        for (int slot = 0; slot < 18; ++slot) part_b(slot);
        p_publish(stage(ntiles - 1));
        pv_prefetch(stage(ntiles - 1));
        lds_barrier();
        pv_chain(stage(ntiles - 1), false, 0, false);
        // the dummy loads of the last two iterations must land before LDS is reused
        wait_vm_barrier<0>();
      } else {
        // ------- bf16 / fp16 (and bf16 q over E4M3 tiles): one 32x32 score block per 32 keys -------
        // A 64-key E4M3 tile is processed as two 32-key halves; its K and V
        // operands are widened to bf16 in registers after the LDS read.
        constexpr int CT = 32;               // keys per score block
        constexpr int HALVES = TILE / CT;    // score blocks per LDS tile
        constexpr int CDT = DT == kMixed ? kBf16 : DT;  // MFMA operand type
        // Over pages of at least a tile the segment's last tile is loaded whole: rows past its last
        // key hold whatever follows in the page (possibly NaN).  Their P is zero, but 0 * NaN would
        // still reach O through the PV MFMA, so they are zeroed once the tile has landed.
        auto zero_tail16 = [&](int t) {
          if constexpr (FAST) {
            const int nvalid = k1 - (k0 + t * TILE);
            if (nvalid < TILE) {
              lds_t* z = smem + (t % kStages) * kStageBytes + nvalid * RB;
              const int nchunks = (TILE - nvalid) * (RB / 16);
              for (int i = 64 * wave + lane_id_here(); i < nchunks; i += kThreads)
                *(lds_v4i*)(z + 16 * i) = v4i{0, 0, 0, 0};
              lds_barrier();
            }
          }
        };
        issue_tile(0);
        if (1 < ntiles) issue_tile(1);
        // raw operands: bf16 / fp16 are MFMA-ready (v4i), E4M3 is widened first (v2i)
        using raw_t = std::conditional_t<DT == kMixed, v2i, v4i>;
        auto kread = [&](const lds_t* st, int c) -> v4i {
          if constexpr (DT == kMixed) {
            // the 16 codes of step pair c (steps 2c and 2c+1)
            return *(const lds_v4i*)(st + kaddr[c & 1] + 64 * (c >> 1));
          } else {
            return *(const lds_v4i*)(st + kaddr[c & 3] + 128 * (c >> 2));
          }
        };
        auto vread = [&](const lds_t* st, int db, int u) -> raw_t {
          if constexpr (DT == kMixed) {
            return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + vaddr[db & 1] + 64 * (db >> 1) + 16 * RB * u));
          } else {
            const int x = db & 1;
            const int base0 = vaddr[x] + 128 * (db >> 1) + 16 * RB * u;
            const int base1 = vaddr[2 + x] + 128 * (db >> 1) + 16 * RB * u;
            const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(st + base0));
            const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(st + base1));
            const v2i r0i = __builtin_bit_cast(v2i, r0), r1i = __builtin_bit_cast(v2i, r1);
            return v4i{r0i[0], r0i[1], r1i[0], r1i[1]};
          }
        };
        auto ready = [&](const raw_t& x) -> v4i {
          if constexpr (DT == kMixed) {
            return widen_e4m3_bf16(x);
          } else {
            return x;
          }
        };
        // LDS operands are read several MFMAs ahead (K four, V two blocks): one
        // 16-bit MFMA (32 cycles) is shorter than the latency of an LDS read.
        // Widened operands are produced one MFMA ahead, in the previous one's shadow.
        constexpr int kAhead = 4, kVAhead = 2;
        auto qk = [&](const lds_t* st, v16f& s) {
          s = v16f{0};
          if constexpr (DT == kMixed) {
            // One 16-byte read per lane and pair of steps (two pairs ahead), its halves widened
            // one MFMA ahead.  Over 576-byte rows, 8-byte reads of one step put rows n and
            // n + 16 on the same banks; 16-byte reads of 16 consecutive rows cover each bank once.
            constexpr int kP = kAhead / 2;
            v4i a[kP];
#pragma unroll
            for (int j = 0; j < kP; ++j) a[j] = kread(st, j);
            v4i cur = widen_e4m3_bf16(v2i{a[0][0], a[0][1]});
#pragma unroll
            for (int c = 0; c < 36; ++c) {
              const v4i qb = v4i{qreg[c][0], qreg[c][1], qreg[c][2], qreg[c][3]};
              qk_mfma_h16<CDT>(s, cur, qb, c == 35);
              const int j = c >> 1;
              if ((c & 1) == 0) {
                cur = widen_e4m3_bf16(v2i{a[j % kP][2], a[j % kP][3]});
              } else {
                if (j + kP < 18) a[j % kP] = kread(st, j + kP);
                if (c + 1 < 36) cur = widen_e4m3_bf16(v2i{a[(j + 1) % kP][0], a[(j + 1) % kP][1]});
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
            raw_t a[kAhead];
#pragma unroll
            for (int c = 0; c < kAhead; ++c) a[c] = kread(st, c);
            v4i cur = ready(a[0]);
#pragma unroll
            for (int c = 0; c < 36; ++c) {
              const v4i qb = v4i{qreg[c][0], qreg[c][1], qreg[c][2], qreg[c][3]};
              qk_mfma_h16<CDT>(s, cur, qb, c == 35);
              if (c + kAhead < 36) a[c % kAhead] = kread(st, c + kAhead);
              if (c + 1 < 36) cur = ready(a[(c + 1) % kAhead]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        };
        float mx_raw = -INFINITY, mref = 0.f, lsum = 0.f;
        v4i pb[2];
        v16f sc;
        auto sm_chunk = [&](int i, int key0, bool need_mask) {
          if (i == 0) {
            mx_raw = -INFINITY;
            lsum = 0.f;
            if (need_mask) {
              int lo_m;
              uint32_t vis_m;
              mask_bounds(lo_m, vis_m);
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = key0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                if ((uint32_t)(key - lo_m) >= vis_m) sc[r] = -INFINITY;
              }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) mx_raw = fmaxf(mx_raw, sc[r]);
          } else if (i == 1) {
            const float mx = mx_raw * p.s_scale_log2;
            const float rm = xor32_max(mx);
            m_seen = fmaxf(m_seen, rm);
            if (m_ref == -INFINITY) m_ref = rm;
            ovf = ovf || (rm > m_ref + kTauOf<DT>);
            mref = m_ref > -INFINITY ? m_ref : 0.f;
          } else if (i >= 2 && i < 6) {
            // four probabilities, packed at once into the P operand (word 2(g4&1) of pb[g4>>1])
            const int g4 = i - 2;
            float pv4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              pv4[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * g4 + j], p.s_scale_log2, -mref));
              lsum += pv4[j];
            }
            pb[g4 >> 1][2 * (g4 & 1)] = (int)pack_p16x2<CDT>(pv4[0], pv4[1]);
            pb[g4 >> 1][2 * (g4 & 1) + 1] = (int)pack_p16x2<CDT>(pv4[2], pv4[3]);
          } else if (i == 7) {
            l_acc += lsum;
            // the sum of P as rounded into the operand words (summed once they are all packed, so
            // no second running sum is held across the chunks)
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              r0 += sum_p16x2<CDT>((uint32_t)pb[0][w]);
              r1 += sum_p16x2<CDT>((uint32_t)pb[1][w]);
            }
            __hip_atomic_fetch_add(lr_slot(), r0 + r1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        };
        if constexpr (XPV) {
        // PV across the waves, as in the fp8 path: wave w accumulates O^T for latent dims
        // [128w, 128w+128) of all 128 rows (accumulator 4j + rr: dim block j, row block
        // rr), so each transposed V read feeds up to four MFMAs.  The row blocks' P
        // operands (B layout, 1 KiB per 16-key step) pass through LDS.
        const int nrb = min(4, (rows_valid - mt * kTileM + 31) / 32);  // row blocks holding rows
        auto publish_p = [&](const v4i& p0, const v4i& p1) {
          *(lds_v4i*)(smem + kPOffset + 2048 * wave + 16 * lane) = p0;
          *(lds_v4i*)(smem + kPOffset + 2048 * wave + 1024 + 16 * lane) = p1;
        };
        // Four phases per block (16-key step u, row-block pair h): the phase's two P
        // operands stay in registers while the wave's four V operands stream past (V is
        // read twice per block).  The next phase's P operands and first V operand are
        // read during the current phase, so no phase starts on an LDS wait.
        auto pread = [&](int u, int rb) -> v4i {
          return *(const lds_v4i*)(smem + kPOffset + 2048 * rb + 1024 * u + 16 * lane);
        };
        auto pv = [&](const lds_t* st, bool with_sm, int key0, bool need_mask) {
          v4i pk[2] = {pread(0, 0), pread(0, 1)};
          raw_t an = vread(st, 0, 0);  // vaddr already points at this wave's 128 dims
#pragma unroll
          for (int ph = 0; ph < 4; ++ph) {
            const int u = ph >> 1, h = ph & 1;
            v4i pn[2] = {pk[0], pk[1]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const v4i a = ready(an);
              if (j < 3) {
                an = vread(st, j + 1, u);
              } else if (ph < 3) {
                an = vread(st, 0, (ph + 1) >> 1);
              }
              if (j == 1 && ph < 3) {
                const int un = (ph + 1) >> 1, hn = (ph + 1) & 1;
                pn[0] = pread(un, 2 * hn);
                pn[1] = pread(un, 2 * hn + 1);
              }
#pragma unroll
              for (int r2 = 0; r2 < 2; ++r2) {
                const int rr = 2 * h + r2;
                if (rr < nrb) o[4 * j + rr] = pv_mfma_h16<CDT>(a, pk[r2], o[4 * j + rr]);
              }
              if (with_sm && (j & 1) == 0) sm_chunk(2 * ph + (j >> 1), key0, need_mask);  // one every two steps
              __builtin_amdgcn_sched_barrier(0);
            }
            pk[0] = pn[0];
            pk[1] = pn[1];
          }
        };
        // score block v covers keys [k0 + 32v, +32) of LDS tile v / HALVES
        auto block_base = [&](int v) -> const lds_t* {
          return smem + ((v / HALVES) % kStages) * kStageBytes + (v % HALVES) * CT * RB;
        };
        auto block_needs_mask = [&](int key0) { return key0 + CT > lim_min || key0 < lo_max; };
        const int nblocks = (k1 - k0 + CT - 1) / CT;

        // Block v: [barrier] publish P(v-1); scores of v; [barrier] PV of v-1 with the
        // softmax of v in its first MFMA slots.  The barrier before the publication
        // keeps it from overwriting P(v-2) while a wave still reads it.
        wait_tile_barrier(min(1, ntiles - 1));
        if (ntiles == 1) zero_tail16(0);
        if (2 < ntiles) issue_tile(2);
        v4i pp0 = v4i{0, 0, 0, 0}, pp1 = v4i{0, 0, 0, 0};
        if (wave_active) {
          qk(smem, sc);
          const bool nm = block_needs_mask(k0);
#pragma unroll
          for (int i = 0; i < 8; ++i) sm_chunk(i, k0, nm);
          pp0 = pb[0];
          pp1 = pb[1];
        }
        for (int v = 1; v < nblocks; ++v) {
          if (v % HALVES == 0) {
            const int tt = v / HALVES;
            wait_tile_barrier(min(1, ntiles - 1 - tt));
            if (tt == ntiles - 1) zero_tail16(tt);
            if (tt + 2 < ntiles) issue_tile(tt + 2);
          } else {
            lds_barrier();
          }
          if (wave_active) publish_p(pp0, pp1);
          const int key0 = k0 + v * CT;
          if (wave_active) qk(block_base(v), sc);
          lds_barrier();
          pv(block_base(v - 1), wave_active, key0, block_needs_mask(key0));
          if (wave_active) {
            pp0 = pb[0];
            pp1 = pb[1];
          }
        }
        lds_barrier();
        if (wave_active) publish_p(pp0, pp1);
        lds_barrier();
        pv(block_base(nblocks - 1), false, 0, false);
              } else {
        // Own-rows layout: each wave accumulates O^T for its 32 rows x all 512 latent
        // dims, so no P exchange and no extra barrier (faster when all four row
        // blocks hold rows).
        auto pv = [&](const lds_t* st, const v4i& p0, const v4i& p1, bool with_sm, int key0, bool need_mask) {
          raw_t vt[kVAhead][2];
#pragma unroll
          for (int db = 0; db < kVAhead; ++db) {
            vt[db][0] = vread(st, db, 0);
            vt[db][1] = vread(st, db, 1);
          }
          v4i w0 = ready(vt[0][0]), w1 = ready(vt[0][1]);
#pragma unroll
          for (int db = 0; db < 16; ++db) {
            const int sl = db % kVAhead;
            o[db] = pv_mfma_h16<CDT>(w0, p0, o[db]);
            o[db] = pv_mfma_h16<CDT>(w1, p1, o[db]);
            if constexpr (DT == kMixed) __builtin_amdgcn_sched_barrier(0);
            if (db + kVAhead < 16) {
              vt[sl][0] = vread(st, db + kVAhead, 0);
              vt[sl][1] = vread(st, db + kVAhead, 1);
            }
            if (db + 1 < 16) {
              w0 = ready(vt[(db + 1) % kVAhead][0]);
              w1 = ready(vt[(db + 1) % kVAhead][1]);
            }
            if (with_sm && db < 8) sm_chunk(db, key0, need_mask);
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        // score block v covers keys [k0 + 32v, +32) of LDS tile v / HALVES
        auto block_base = [&](int v) -> const lds_t* {
          return smem + ((v / HALVES) % kStages) * kStageBytes + (v % HALVES) * CT * RB;
        };
        auto block_needs_mask = [&](int key0) { return key0 + CT > lim_min || key0 < lo_max; };
        const int nblocks = (k1 - k0 + CT - 1) / CT;

        wait_tile_barrier(min(1, ntiles - 1));
        if (ntiles == 1) zero_tail16(0);
        if (2 < ntiles) issue_tile(2);
        v4i pp0 = v4i{0, 0, 0, 0}, pp1 = v4i{0, 0, 0, 0};
        if (wave_active) {
          qk(smem, sc);
          const bool nm = block_needs_mask(k0);
#pragma unroll
          for (int i = 0; i < 8; ++i) sm_chunk(i, k0, nm);
          pp0 = pb[0];
          pp1 = pb[1];
        }
        for (int v = 1; v < nblocks; ++v) {
          if (v % HALVES == 0) {
            const int tt = v / HALVES;
            wait_tile_barrier(min(1, ntiles - 1 - tt));
            if (tt == ntiles - 1) zero_tail16(tt);
            if (tt + 2 < ntiles) issue_tile(tt + 2);
          }
          if (!wave_active) continue;
          const int key0 = k0 + v * CT;
          qk(block_base(v), sc);
          pv(block_base(v - 1), pp0, pp1, true, key0, block_needs_mask(key0));
          pp0 = pb[0];
          pp1 = pb[1];
        }
        if (wave_active) pv(block_base(nblocks - 1), pp0, pp1, false, 0, false);
              }
      }
      // did any row of the workgroup outgrow its reference?  Segments of at most 128 keys are also
      // redone when any row's max came after its first tile: a row with few keys gives most of its
      // weight to a handful of them, and with the row max as reference the largest p is exactly 1
      // (E4M3: a power of two), so only the smaller weights carry the rounding of P.
      if (attempt == 0 && ntiles * TILE <= 128) ovf = ovf || (m_seen > m_ref);
      const bool wave_ovf = __builtin_amdgcn_ballot_w64(ovf) != 0;
      if (lane == 0) s_flag[wave] = wave_ovf ? 1 : 0;
      lds_barrier();
      const bool redo = (s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3]) != 0;
      if (!redo) break;
      m_init = m_seen;
    }
  }

  // ---- epilogue: normalise, write final or partial ----
  if constexpr (DT == kFp8 || XPV) {
    // Wave w holds O^T for latent dims [128w, 128w+128) of all 128 rows; the
    // row owners publish 1/l, then the whole 128x512 tile is staged in LDS and
    // written row-contiguous (whole 128-byte lines per store; see store_out for
    // the cache policy of final outputs and partials).
    asm volatile("" : "+v"(lane));
    const int ne = lane & 31, he = lane >> 5;
    const float l_tot = xor32_sum(l_acc);
    const bool has = l_tot > 0.f;
    // O is normalised by the sum of the weights the PV product used (P as rounded to its
    // operand type), the LSE by the exact sum; with the second E4M3 term the weights are P up to
    // E2M1's rounding of the residual, and the exact sum normalises O as well
    const float l_norm = DT == kFp8 ? (LO ? l_tot : xor32_sum(l_acc_r)) : xor32_sum(*lr_slot());
    const float inv = has && l_norm > 0.f ? p.v_scale / l_norm : 0.f;
    const float lse_v = has ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
    lds_f32* s_inv = (lds_f32*)(smem + kPOffset);
    lds_barrier();  // every wave is done with the KV ring and the P buffer
    if (he == 0) s_inv[32 * wave + ne] = inv;
    lds_barrier();
    // accumulator rr of every latent block holds row block (wave + rr) & 3 (fp8) or rr
    auto rowblk = [&](int rr) { return DT == kFp8 ? (wave + rr) & 3 : rr; };
    float invr[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) invr[rr] = s_inv[32 * rowblk(rr) + ne];
    const bool f32out = !sg.single && !p.part_bf16;
    const int row0 = mt * kTileM;
    if (!f32out) {
      uint16_t* dst = sg.single ? p.out + out_row0 * kDv
                                : (uint16_t*)p.part_o + (size_t)sg.slot * rows_per_b * kDv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int row = 32 * rowblk(rr) + ne, col = 128 * wave + 32 * j + 8 * gq + 4 * he;
            const v16f& acc = o[4 * j + rr];
            const v2i w = v2i{(int)pack_bf16x2(acc[4 * gq + 0] * invr[rr], acc[4 * gq + 1] * invr[rr]),
                              (int)pack_bf16x2(acc[4 * gq + 2] * invr[rr], acc[4 * gq + 3] * invr[rr])};
            *(lds_v2i*)(smem + row * kEpiPitch + 2 * col) = w;
          }
        }
      }
      lds_barrier();
#pragma unroll 4
      for (int k = 0; k < 32; ++k) {
        const int row = 32 * wave + k;
        const v4i v = *(const lds_v4i*)(smem + row * kEpiPitch + 16 * lane);
        const int m_r = row0 + row;
        if (m_r < rows_valid) {
          const size_t rowb = (size_t)gF * p.H + (size_t)m_r;
          store_out(v, (v4i*)(dst + rowb * kDv + 8 * lane), sg.single);
        }
      }
    } else {
      float* dst = (float*)p.part_o + (size_t)sg.slot * rows_per_b * kDv;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if ((wave >> 1) == h) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
              for (int gq = 0; gq < 4; ++gq) {
                const int row = 32 * rowblk(rr) + ne, col = 128 * (wave & 1) + 32 * j + 8 * gq + 4 * he;
                const v16f& acc = o[4 * j + rr];
                *(__attribute__((address_space(3))) v4f*)(smem + row * kEpiPitch + 4 * col) =
                    v4f{acc[4 * gq + 0] * invr[rr], acc[4 * gq + 1] * invr[rr], acc[4 * gq + 2] * invr[rr],
                        acc[4 * gq + 3] * invr[rr]};
              }
            }
          }
        }
        lds_barrier();
#pragma unroll 4
        for (int k = 0; k < 32; ++k) {
          const int row = 32 * wave + k;
          const v4f v = *(const __attribute__((address_space(3))) v4f*)(smem + row * kEpiPitch + 16 * lane);
          const int m_r = row0 + row;
          if (m_r < rows_valid) {
            const size_t rowb = (size_t)gF * p.H + (size_t)m_r;
            *(v4f*)(dst + rowb * kDv + 256 * h + 4 * lane) = v;  // a partial: the merge reads it next
          }
        }
        lds_barrier();
      }
    }
    const int m_l = row0 + 32 * wave + ne;
    if (m_l < rows_valid && he == 0) {
      const size_t rowb = (size_t)gF * p.H + (size_t)m_l;
      if (sg.single) {
        if (p.lse != nullptr) p.lse[out_row0 + rowb] = lse_v;
      } else {
        p.part_lse[(size_t)sg.slot * rows_per_b + rowb] = lse_v;
      }
    }
    } else {
  // Each wave moves its 32x512 tile through its own LDS region in two passes
  // of 256 columns: accumulators are scaled by 1/l and converted to the
  // output type on the way in (rows padded so the column-wise writes hit
  // distinct banks), then read back row-contiguous so that every store
  // instruction writes whole 128-byte lines.
  asm volatile("" : "+v"(lane));  // epilogue addressing is computed here, after the loop
  const int ne = lane & 31, he = lane >> 5;
  const float l_tot = xor32_sum(l_acc);
  const bool has = l_tot > 0.f;
  const float l_norm = xor32_sum(*lr_slot());  // the rounded P's sum, as in the other epilogue
  const float inv = has && l_norm > 0.f ? p.v_scale / l_norm : 0.f;
  const float lse_v = has ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  const bool f32out = !sg.single && !p.part_bf16;
  const int wrow0 = mt * kTileM + 32 * wave;  // first row of this wave
  lds_barrier();  // every wave is done with the KV ring
  lds_t* wl = smem + wave * kEpiWaveBytes;
  if (!f32out) {
    uint16_t* dst = sg.single ? p.out + out_row0 * kDv
                              : (uint16_t*)p.part_o + (size_t)sg.slot * rows_per_b * kDv;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int dbl = 0; dbl < 8; ++dbl) {
        const int db = 8 * pass + dbl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = 32 * dbl + 8 * i + 4 * he;
          const v2i w = v2i{(int)pack_bf16x2(o[db][4 * i + 0] * inv, o[db][4 * i + 1] * inv),
                            (int)pack_bf16x2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv)};
          *(lds_v2i*)(wl + ne * kEpiRowB16 + 2 * col) = w;
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int r = 2 * k + (lane >> 5), ch = lane & 31;
        const v4i v = *(const lds_v4i*)(wl + r * kEpiRowB16 + 16 * ch);
        const int m_r = wrow0 + r;
        if (m_r < rows_valid) {
          const size_t rowb = (size_t)gF * p.H + (size_t)m_r;
          store_out(v, (v4i*)(dst + rowb * kDv + 256 * pass + 8 * ch), sg.single);
        }
      }
    }
  } else {
    float* dst = (float*)p.part_o + (size_t)sg.slot * rows_per_b * kDv;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int dbl = 0; dbl < 8; ++dbl) {
        const int db = 8 * pass + dbl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = 32 * dbl + 8 * i + 4 * he;
          *(__attribute__((address_space(3))) v4f*)(wl + ne * kEpiRowF32 + 4 * col) =
              v4f{o[db][4 * i + 0] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv};
        }
      }
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const v4f v = *(const __attribute__((address_space(3))) v4f*)(wl + r * kEpiRowF32 + 16 * lane);
        const int m_r = wrow0 + r;
        if (m_r < rows_valid) {
          const size_t rowb = (size_t)gF * p.H + (size_t)m_r;
          *(v4f*)(dst + rowb * kDv + 256 * pass + 4 * lane) = v;  // a partial: the merge reads it next
        }
      }
    }
  }
  const int m_l = wrow0 + ne;
  if (m_l < rows_valid && he == 0) {
    const size_t rowb = (size_t)gF * p.H + (size_t)m_l;
    if (sg.single) {
      if (p.lse != nullptr) p.lse[out_row0 + rowb] = lse_v;
    } else {
      p.part_lse[(size_t)sg.slot * rows_per_b + rowb] = lse_v;
    }
  }
  }
}

// ---------------------------------------------------------------------------
// FP8 split-KV segment with specialised waves: twelve waves, three per SIMD
// (168 registers each, all VGPRs).
//   score waves 0-3, one per SIMD: row block sr = wave (32 query rows) against
//     the whole 64-key tile: 18 MFMAs (two 32-key blocks x 9 K-steps of 64),
//     then the softmax; their Q block lives in 72 VGPRs.  Each owns its rows'
//     softmax state: a reference m_ref fixed at the row's first visible tile,
//     P scaled per tile so its largest value lands in (128, 256], the scale
//     2^-e handed to the PV MFMA as its E8M0 block scale, the exact row sums.
//     P goes out in two terms: E4M3 codes, and E2M1 codes of their rounding
//     residuals (used for sequences of at most kLoKeys keys).
//   PV waves 4-11: O^T for latent dims [64 pw, 64 pw + 64), pw = wave - 4, and
//     all 128 rows: 8 MFMAs (2 dim blocks x 4 row blocks) per tile, 8 more for
//     the second P term, their output block in 128 VGPRs; waves 4-7 also issue
//     the tile loads.
// Per tile t, phase A: the DMA waves issue tile t+2 into the stage of tile t-2;
// the score waves run the scores and softmax of tile t (at raised priority while
// their MFMAs issue), the PV waves the PV of tile t-1, so the score waves'
// softmax overlaps the PV MFMAs on every SIMD.  [barrier]  Phase B: the score
// waves publish P(t), its scales and the rows' rescale factors.  [barrier, tile
// t+1 landed]  Two tiles stay in flight.  A row whose max outgrows its reference
// by more than kTau moves the reference (one pass, no recomputation): the score
// wave scales its row sums by 2^(old - new) and publishes that factor, the PV
// waves scale the row's output accumulators by it before adding the tile.
// ---------------------------------------------------------------------------
constexpr int kThreadsR = 768;
constexpr int kRDummy = kStages * kStageBytes;  // 1 KiB: destination of dummy-tile loads
constexpr int kRP = kRDummy + 1024;              // P codes: [row block 4][half 2][lane 64][16 bytes]
constexpr int kRScale = kRP + 8192;              // E8M0 scale codes: [row block 4][lane 64] int32
constexpr int kRResc = kRScale + 1024;           // per-row rescale factor of the tile: [row block 4][row 32] fp32
constexpr int kRBt = kRResc + 512;                // block-table entries of the segment
constexpr int kRLdsBytes = kRBt + 4 * kBtEntries;
static_assert(kRLdsBytes <= 160 * 1024, "LDS budget of one workgroup");

// SCORE: the code of the score waves (true) or of the PV waves (false).  The two
// are separate instantiations, called from separate branches of the kernel, so
// that a wave's registers hold only its own role's state; both run the same
// sequence of workgroup barriers.
template <bool FAST, bool WIN, bool SCORE>
__device__ __forceinline__ void run_segment_roles(const PartialParams& p, lds_t* smem, const SegmentCtx& sg, int g,
                                                  int mt, int wave, int lane) {
  constexpr int TILE = 64;
  constexpr int RB = 576;
  constexpr int CH = 36;
  typedef __attribute__((address_space(3))) int lds_i32;
  typedef __attribute__((address_space(3))) float lds_f32;

  asm volatile("" : "+v"(lane));
  asm volatile("" : "+s"(wave));
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int sr = wave & 3;                         // score role: row block
  const int pw = wave - 4;                         // PV role: latent dims [64 pw, +64)
  const bool dma_wave = !SCORE && wave < 8;        // issue the tile loads (PV waves 4-7)
  const int dw = wave - 4;                         // their index
  const int L = sg.L, qlen_b = sg.qlen, tok0 = sg.tok0;
  const int gF = g * p.F;
  const int rows_valid = min(p.H_eff, max(qlen_b - gF, 0) * p.H);
  if (rows_valid <= mt * kTileM) return;
  const int n_gmax = min(max(L - qlen_b + gF + p.F, 0), L);
  const int window = WIN ? p.window : 0;
  const int kbase = seq_key0<TILE>(L, qlen_b, window);
  const bool lo_seg = L <= kLoKeys;
  const int k0 = kbase + sg.u0 * TILE;
  const int k1 = min(kbase + sg.u1 * TILE, n_gmax);

  // the score wave's row (row n of block sr)
  const int m = mt * kTileM + 32 * sr + n;
  const bool row_valid = m < rows_valid;
  const int n_row = row_valid ? min(max(L - qlen_b + gF + m / p.H + 1, 0), L) : 0;
  const int lim = min(n_row, k1);
  const int lo = window > 0 ? max(n_row - window, 0) : 0;
  auto mask_bounds = [&](int& lo_m, uint32_t& vis_m) {
    if constexpr (WIN) {
      int nr = n_row;
      asm volatile("" : "+v"(nr));
      lo_m = window > 0 ? max(nr - window, 0) : 0;
      vis_m = (uint32_t)max(min(nr, k1) - lo_m, 0);
    } else {
      lo_m = 0;
      vis_m = (uint32_t)lim;
    }
  };
  const size_t rows_per_b = (size_t)p.q_len * p.H;
  const size_t out_row0 = (size_t)tok0 * p.H;

  v8i qreg[SCORE ? 9 : 1];  // score waves: Q of the row block (B operand, K-steps of 64)
  v16f o[SCORE ? 1 : 8];     // PV waves: o[4 j + rb] = dims 64 pw + 32 j .. + 31 of row block rb
  float m_ref = -INFINITY;
  float l_acc = 0.f;
  if constexpr (!SCORE) {
    // zeros made here (opaque): a hoisted constant block would be kept, or spilled, across segments
    float z = 0.f;
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = v16f{z, z, z, z, z, z, z, z, z, z, z, z, z, z, z, z};
  }

  if (k1 > k0) {
    const int ntiles = (k1 - k0 + TILE - 1) / TILE;
    const int pmask = p.page_size - 1;
    cint_t* bt = (cint_t*)p.block_table + (size_t)sg.b * p.max_pages;
    const int plast = min((k1 - 1) >> p.page_shift, p.max_pages - 1);
    const uint32_t smem_base = lds_addr(smem);

    int bt_base = 0;
    auto bt_fill = [&](int first) {
      bt_base = first;
      int v = 0;
      if (dma_wave) v = bt[min(first + 64 * dw + lane, plast)];
      lds_barrier();
      if (dma_wave) *(lds_i32*)(smem + kRBt + 4 * (64 * dw + lane)) = v;
      lds_barrier();
    };
    // (uniform: kept in scalar registers from the start)
    auto page_raw = [&](int pidx) -> int {
      return __builtin_amdgcn_readfirstlane(*(const lds_i32*)(smem + kRBt + 4 * (min(pidx, plast) - bt_base)));
    };
    auto clamp_page = [&](int pg) -> int { return min(max(__builtin_amdgcn_readfirstlane(pg), 0), p.num_pages - 1); };
    const uint8_t* d_base = p.kv;
    uint32_t d_m0 = smem_base, d_step = 1024;
    int d_key0 = k0, d_pidx0 = 0;
    int d_pg0 = 0, d_pg1 = 0, d_pg2 = 0, d_pg3 = 0;
    int pf0 = 0, pf1 = 0, pf2 = 0, pf3 = 0;
    // every wave takes part in the block-table refills (workgroup barriers); only the DMA waves
    // look up pages and set up loads
    auto prefetch_pages = [&](int tt) {
      const int pidx0 = (k0 + tt * TILE) >> p.page_shift;
      constexpr int kFillTiles = FAST ? kBtEntries : (kBtEntries - 3) / 4;
      if (tt > 0 && tt % kFillTiles == 0) bt_fill(pidx0);
      if (!dma_wave) return;
      pf0 = page_raw(pidx0);
      if constexpr (!FAST) {
        pf1 = page_raw(pidx0 + 1);
        pf2 = page_raw(pidx0 + 2);
        pf3 = page_raw(pidx0 + 3);
      }
    };
    auto dma_setup = [&](int tt) {
      if (tt < ntiles) {
        if (dma_wave) {
          const int key0 = k0 + tt * TILE;
          d_m0 = smem_base + (uint32_t)((tt % kStages) * kStageBytes);
          d_step = 1024;
          d_key0 = key0;
          d_pidx0 = key0 >> p.page_shift;
          if constexpr (FAST) {
            d_base = p.kv + ((size_t)clamp_page(pf0) * p.page_size + (key0 & pmask)) * RB;
          } else {
            d_pg0 = clamp_page(pf0);
            d_pg1 = clamp_page(pf1);
            d_pg2 = clamp_page(pf2);
            d_pg3 = clamp_page(pf3);
          }
        }
        if (tt + 1 < ntiles) prefetch_pages(tt + 1);
      } else {
        d_m0 = smem_base + (uint32_t)kRDummy;
        d_step = 0;
      }
    };
    auto dma_issue = [&](int kk) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int slot = 64 * (dw + 4 * kk) + ln;
      const int row = slot / CH;
      const uint32_t off = (uint32_t)(row * RB + ((slot - row * CH) ^ swz<kFp8>(row)) * 16);
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(d_m0 + d_step * (uint32_t)(dw + 4 * kk));
      if constexpr (FAST) {
        dma16_sbase(off, d_base, m0);
      } else {
        const int key = d_key0 + row;
        const int rel = (key >> p.page_shift) - d_pidx0;
        const int g0 = __builtin_amdgcn_readfirstlane(d_pg0), g1 = __builtin_amdgcn_readfirstlane(d_pg1);
        const int g2 = __builtin_amdgcn_readfirstlane(d_pg2), g3 = __builtin_amdgcn_readfirstlane(d_pg3);
        const int pg = rel == 0 ? g0 : rel == 1 ? g1 : rel == 2 ? g2 : g3;
        const uint8_t* src = p.kv + ((size_t)pg * p.page_size + (key & pmask)) * RB + (off - (uint32_t)(row * RB));
        dma16_vaddr(src, m0);
      }
    };
    auto issue_tile = [&](int tt) {
      dma_setup(tt);
      if (dma_wave) {
#pragma unroll
        for (int kk = 0; kk < kDmaPerWave; ++kk) dma_issue(kk);
      }
    };
    // Phase A is split at the end of the score MFMAs: the PV waves read their V operands, then
    // wait here, so that their MFMAs run beside the softmax instead of stretching the score
    // chain (the MFMA pipe is shared, and an issued MFMA is not preempted).  No wait on memory.
    auto mid_barrier = [&]() { __builtin_amdgcn_s_barrier(); };
    // the DMA waves wait for their loads of the next tile (the younger tile stays in flight),
    // every wave for its LDS writes; then the barrier
    auto wait_next = [&]() {
      if (dma_wave) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaPerWave) : "memory");
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    };
    auto stage = [&](int t) -> const lds_t* { return smem + (t % kStages) * kStageBytes; };
    auto zero_tail = [&](int t) {
      const int nvalid = k1 - (k0 + t * TILE);
      if (nvalid < TILE) {
        lds_t* z = smem + (t % kStages) * kStageBytes + nvalid * RB;
        const int nchunks = (TILE - nvalid) * (RB / 16);
        int zr = 0;
        asm volatile("" : "+v"(zr));  // (a hoisted zero vector would be kept across the loop)
        for (int i = 64 * wave + lane; i < nchunks; i += kThreadsR) *(lds_v4i*)(z + 16 * i) = v4i{zr, zr, zr, zr};
        lds_barrier();
      }
    };

    // score waves: keys inside [lo_max, lim_min) of every row need no mask
    int lim_min = lim, lo_max = lo;
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) {
      lim_min = min(lim_min, __shfl_xor(lim_min, o2, 64));
      lo_max = max(lo_max, __shfl_xor(lo_max, o2, 64));
    }
    lim_min = __builtin_amdgcn_readfirstlane(lim_min);
    lo_max = __builtin_amdgcn_readfirstlane(lo_max);
    auto tile_needs_mask = [&](int key0) { return key0 + TILE > lim_min || key0 < lo_max; };

    {
      bt_fill(k0 >> p.page_shift);  // (its first barrier: the previous use of LDS is over)
      prefetch_pages(0);

      // ---------------- score role ----------------
      v16f s0, s1;
      int pa[4], pb[4];
      // second term of P: the E4M3 rounding residual of every element, as E2M1 codes of half
      // its value (nibble k = K-slot k of the E4M3 operand: la = keys of s0, lb = keys of s1)
      int la[2], lb[2];
      int sc_code = 127;
      float resc = 1.f;  // this tile's reference change of the row (1: none)
      auto qk = [&](const lds_t* st) {
        int ka = (32 * 0 + n) * RB + (((2 * hh) ^ ((n >> 2) & 3)) * 16);
        asm volatile("" : "+v"(ka));
        auto kread = [&](int c, int kb) -> v8i {
          const int a0 = ka + 32 * RB * kb;
          const v4i x = *(const lds_v4i*)(st + a0 + 64 * c);
          const v4i y = *(const lds_v4i*)(st + (a0 ^ 16) + 64 * c);
          return v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        };
        v8i kb[3];
        kb[0] = kread(0, 0);
        kb[1] = kread(0, 1);
#pragma unroll
        for (int i = 0; i < 18; ++i) {
          if (i + 2 < 18) kb[(i + 2) % 3] = kread((i + 2) >> 1, (i + 2) & 1);
          if (i & 1) {
            if (i == 1) qk_mfma_f8_first(s1, kb[i % 3], qreg[i >> 1]);
            else qk_mfma_f8(s1, kb[i % 3], qreg[i >> 1], i == 17);
          } else {
            if (i == 0) qk_mfma_f8_first(s0, kb[i % 3], qreg[i >> 1]);
            else qk_mfma_f8(s0, kb[i % 3], qreg[i >> 1], i == 16);
          }
        }
      };
      auto softmax = [&](int key0, bool need_mask) {
        if (need_mask) {
          int lo_m;
          uint32_t vis_m;
          mask_bounds(lo_m, vis_m);
          int kb = 4 * hh;
          asm volatile("" : "+v"(kb));
          kb += key0 - lo_m;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if ((uint32_t)(kb + 8 * (r >> 2) + (r & 3)) >= vis_m) s0[r] = -INFINITY;
            if ((uint32_t)(kb + 32 + 8 * (r >> 2) + (r & 3)) >= vis_m) s1[r] = -INFINITY;
          }
        }
        // row max over the lane's 32 scores: a three-input max tree (fmaxf would first quiet every
        // score, the MFMA results being opaque to the compiler)
        auto max3 = [](float a, float b, float c) -> float {
          float r;
          asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
          return r;
        };
        float m9[11];
#pragma unroll
        for (int i = 0; i < 5; ++i) m9[i] = max3(s0[3 * i], s0[3 * i + 1], s0[3 * i + 2]);
#pragma unroll
        for (int i = 0; i < 5; ++i) m9[5 + i] = max3(s1[3 * i], s1[3 * i + 1], s1[3 * i + 2]);
        m9[10] = max3(s0[15], s1[15], m9[9]);
        const float mx = max3(max3(m9[0], m9[1], m9[2]), max3(m9[3], m9[4], m9[5]), max3(m9[6], m9[7], m9[8]));
        const float mxx = max3(mx, m9[10], m9[10]);
        const float rm = xor32_max(mxx * p.s_scale_log2);  // row max of the tile, log2 units
        // The reference is fixed at the row's first visible tile and moves only when a tile's
        // max outgrows it by more than kTau: then everything accumulated so far is scaled by
        // 2^(old - new) (the row sums here, the output accumulators by the PV waves).
        resc = 1.f;
        if (m_ref == -INFINITY) {
          m_ref = rm;
        } else if (rm > m_ref + kTau) {
          resc = __builtin_amdgcn_exp2f(m_ref - rm);
          m_ref = rm;
          l_acc *= resc;
        }
        const float mref = m_ref > -INFINITY ? m_ref : 0.f;
        int e = 0;
        if (rm > -INFINITY) e = 8 - (int)ceilf(rm - mref);
        e = min(max(e, -120), 120);
        const float off = mref - (float)e;
        float lsum = 0.f;
        // Four probabilities: the E4M3 codes (returned) and the E2M1 codes of their residuals, written
        // into bytes 2 (w2 & 1) and 2 (w2 & 1) + 1 of `lo`.  Every p is at most 256 here, so a
        // residual is at most 8 (half an E4M3 step in [128, 256]) and half of it fits E2M1's range;
        // with the second term each p is off by at most 2^-7 of its own binade.  O is normalised by
        // the exact sum: the two terms differ from it by less than that.
        auto four = [&](const v16f& sv, int w2, int& lo, auto with_lo) -> int {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * w2 + 0], p.s_scale_log2, -off));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * w2 + 1], p.s_scale_log2, -off));
          const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * w2 + 2], p.s_scale_log2, -off));
          const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * w2 + 3], p.s_scale_log2, -off));
          int wv = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
          wv = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, wv, true);
          lsum += (e0 + e1) + (e2 + e3);
          if constexpr (!decltype(with_lo)::value) return wv;
          const v2f r0 = __builtin_amdgcn_cvt_pk_f32_fp8(wv, false);
          const v2f r1 = __builtin_amdgcn_cvt_pk_f32_fp8(wv, true);
          // (the conversion divides by its scale: codes of d / 2)
          uint32_t lw = (uint32_t)lo;
          if ((w2 & 1) == 0) {  // (byte selects must be literal constants)
            lw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lw, e0 - r0[0], e1 - r0[1], 2.f, 0);
            lw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lw, e2 - r1[0], e3 - r1[1], 2.f, 1);
          } else {
            lw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lw, e0 - r0[0], e1 - r0[1], 2.f, 2);
            lw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lw, e2 - r1[0], e3 - r1[1], 2.f, 3);
          }
          lo = (int)lw;
          return wv;
        };
        la[0] = la[1] = lb[0] = lb[1] = 0;
        if (lo_seg) {
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            pa[w2] = four(s0, w2, la[w2 >> 1], std::true_type{});
            pb[w2] = four(s1, w2, lb[w2 >> 1], std::true_type{});
          }
        } else {
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            pa[w2] = four(s0, w2, la[w2 >> 1], std::false_type{});
            pb[w2] = four(s1, w2, lb[w2 >> 1], std::false_type{});
          }
        }
        l_acc += __builtin_ldexpf(lsum, -e);
        sc_code = (127 - e) | (lo_seg ? 0x100 : 0);  // bit 8: the PV waves add the second term
      };
      // The second term of P(t) goes into the rope columns of tile t's own stage (bytes 512..575 of
      // its 64 rows): the score waves are done with them once the barrier after the scores has
      // passed, and the stage is not reloaded before the PV of tile t has read them.  Entry
      // 64 rb + lane (16 bytes) sits at row entry / 4, bytes 512 + 16 (entry % 4).
      auto lo_entry = [&](const lds_t* st, int e) -> const lds_t* { return st + (e >> 2) * RB + 512 + 16 * (e & 3); };
      auto publish = [&](int t) {
        *(lds_v4i*)lo_entry(stage(t), 64 * sr + lane) = v4i{la[0], la[1], lb[0], lb[1]};
        *(lds_v4i*)(smem + kRP + 2048 * sr + 16 * lane) = v4i{pa[0], pa[1], pa[2], pa[3]};
        *(lds_v4i*)(smem + kRP + 2048 * sr + 1024 + 16 * lane) = v4i{pb[0], pb[1], pb[2], pb[3]};
        *(lds_i32*)(smem + kRScale + 256 * sr + 4 * lane) = sc_code;
        if (hh == 0) *(lds_f32*)(smem + kRResc + 128 * sr + 4 * n) = resc;
      };
      auto score_tile = [&](int t) {
        const int key0 = k0 + t * TILE;
        __builtin_amdgcn_s_setprio(2);  // the score chain is the tile's critical path
        qk(stage(t));
        __builtin_amdgcn_s_setprio(0);
        mid_barrier();
        softmax(key0, tile_needs_mask(key0));
      };

      // ---------------- PV role ----------------
      int vaddr0;
      {
        const int grp = lane >> 4, hs = grp >> 1, dsub = grp & 1, uu = lane & 15, rr = uu >> 1, c8 = uu & 1;
        const int kbr = 8 * (rr >> 2) + 4 * hs + (rr & 3);
        const int s8 = (2 * (rr >> 2) + hs) & 3;
        vaddr0 = kbr * RB + ((dsub ^ s8) * 16) + 8 * c8;  // chunk pair partner: ^ 32
      }
      // with_dma: the DMA waves issue the loads set up last (dma_setup) between the row blocks,
      // three, two, two and two, so that they share the SIMD with the MFMAs instead of queueing
      // ahead of them
      auto pv_tile = [&](int t, bool with_dma) {
        const lds_t* st = stage(t);
        int va = vaddr0 + 64 * pw;
        asm volatile("" : "+v"(va));
        auto vread = [&](int base) -> v8i {
          const v2i r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base));
          const v2i r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base + 16 * RB));
          const v2i r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base + 32 * RB));
          const v2i r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base + 48 * RB));
          return v8i{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
        };
        // rows whose reference moved with this tile: rescale what they hold first
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const float f = *(const lds_f32*)(smem + kRResc + 128 * rb + 4 * (lane & 31));
          if (__builtin_amdgcn_ballot_w64(f != 1.f) != 0) {
            o[rb] *= f;
            o[4 + rb] *= f;
          }
        }
        const v8i v0 = vread(va), v1 = vread(va ^ 32);
        mid_barrier();
        // The four row blocks' P stream past the two V operands, one at a time: each read's
        // address is made opaque where it is used, so that the reads are neither merged nor
        // hoisted together (32 more live registers than the budget allows).
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          int pa_ = 16 * lane;
          asm volatile("" : "+v"(pa_));
          const v4i x = *(const lds_v4i*)(smem + kRP + 2048 * rb + pa_);
          const v4i y = *(const lds_v4i*)(smem + kRP + 2048 * rb + 1024 + pa_);
          const int scw = *(const lds_i32*)(smem + kRScale + 256 * rb + (pa_ >> 2));
          const int scb = scw & 0xff;
          const v8i pr = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
          o[rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v0, pr, o[rb], 0, 0, 0, 127, 0, scb);
          o[4 + rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v1, pr, o[4 + rb], 0, 0, 0, 127, 0, scb);
          if (__builtin_amdgcn_readfirstlane(scw) & 0x100) {
            // The residual term: B in E2M1 (blgp 4), twice the E4M3 term's scale.  The E2M1 operand
            // of a column: lane half h takes bytes 8h..8h+7 of the entries of lanes n and n + 32
            // (its K-slots are those of E4M3 bytes 16h..16h+15 of both lane halves).
            const int hb = 8 * (lane >> 5), ln = lane & 31;
            const v2i l0 = *(const lds_v2i*)(lo_entry(st, 64 * rb + ln) + hb);
            const v2i l1 = *(const lds_v2i*)(lo_entry(st, 64 * rb + 32 + ln) + hb);
            const v8i pl = v8i{l0[0], l0[1], l1[0], l1[1], 0, 0, 0, 0};
            o[rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v0, pl, o[rb], 0, 4, 0, 127, 0, scb + 1);
            o[4 + rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v1, pl, o[4 + rb], 0, 4, 0, 127, 0, scb + 1);
          }
          // The MFMAs stay in the tile (left alone, the compiler sinks them past the barrier that
          // follows, keeping every P operand live across it): the previous row block's results
          // are pinned here, one block late, so the pin finds them complete instead of waiting
          // for the MFMAs just issued.
          if (rb > 0) asm volatile("" : "+v"(o[rb - 1]), "+v"(o[3 + rb]));
          if (with_dma && dma_wave) {
            static_assert(kDmaPerWave == 9, "loads per row block below");
            if (rb == 0) {
              dma_issue(0);
              dma_issue(1);
              dma_issue(2);
            } else {
              dma_issue(2 * rb + 1);
              dma_issue(2 * rb + 2);
            }
          }
        }
        asm volatile("" : "+v"(o[3]), "+v"(o[7]));
      };

      // ---- prologue: Q through ring stages 2-3, tiles 0 and 1 ----
      constexpr int kQDma = 32 * kDqk / 1024;  // 18 one-KiB loads per DMA wave (one row block)
      if (dma_wave) {
        const uint8_t* qblk = p.q + ((size_t)tok0 + gF) * p.H * kDqk;
        const uint32_t qlds = smem_base + (uint32_t)(2 * kStageBytes + dw * 32 * kDqk);
        int qlane = lane;
        asm volatile("" : "+v"(qlane));
#pragma unroll
        for (int kk = 0; kk < kQDma; ++kk) {
          const int o_ = 1024 * kk + 16 * qlane;
          const int qn = o_ / kDqk;
          const int mrow = mt * kTileM + 32 * dw + qn;
          const int src_row = mrow < rows_valid ? mrow : 0;
          dma16_vaddr(qblk + (size_t)src_row * kDqk + (o_ - qn * kDqk),
                      __builtin_amdgcn_readfirstlane(qlds + 1024u * (uint32_t)kk));
        }
      }
      issue_tile(0);
      issue_tile(1);
      if (dma_wave) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kDmaPerWave) : "memory");  // Q has landed
      lds_barrier();
      if constexpr (SCORE) {
        const lds_t* qs = smem + 2 * kStageBytes + sr * 32 * kDqk + n * kDqk + 32 * hh;
        const int keep = row_valid ? -1 : 0;
#pragma unroll
        for (int c = 0; c < 9; ++c) {
          const v4i x0 = *(const lds_v4i*)(qs + 64 * c) & keep;
          const v4i x1 = *(const lds_v4i*)(qs + 64 * c + 16) & keep;
          qreg[c] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        }
      }
      // tile 0 has landed and every score wave holds its Q: stages 2-3 may be refilled
      if (dma_wave) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaPerWave) : "memory");
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
      if (ntiles == 1) zero_tail(0);
      issue_tile(2);
      if constexpr (SCORE) {
        score_tile(0);
      } else {
        mid_barrier();
      }
      lds_barrier();
      if constexpr (SCORE) publish(0);
      wait_next();  // P(0) visible, tile 1 landed

      for (int t = 1; t < ntiles; ++t) {
        if (t == ntiles - 1) zero_tail(t);
        // Tile t+2 goes into the stage of tile t-2, free since the PV of t-2 (the last iteration):
        // the DMA waves issue it during their PV work, off the score waves' path.
        // (pages shorter than a tile take four page registers: their loads go out at once, here)
        if constexpr (FAST) {
          dma_setup(t + 2);
        } else {
          issue_tile(t + 2);
        }
        if constexpr (SCORE) {
          score_tile(t);
        } else {
          pv_tile(t - 1, FAST);
        }
        lds_barrier();  // PV of tile t-1 is done: the P buffer is free
        if constexpr (SCORE) publish(t);
        wait_next();  // P(t) visible, tile t+1 landed
      }
      if constexpr (SCORE) {
        mid_barrier();
      } else {
        pv_tile(ntiles - 1, false);
      }
      // the dummy loads must land before LDS is reused
      if (dma_wave) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    }
  }

  // ---- epilogue: the score waves publish 1/l and write the LSE; the PV waves stage O ----
  asm volatile("" : "+v"(lane));
  const int ne = lane & 31, he = lane >> 5;
  lds_f32* s_inv = (lds_f32*)(smem + kRScale);
  lds_barrier();  // every wave is done with the ring, P and the scales
  const int row0 = mt * kTileM;
  if constexpr (SCORE) {
    const float l_tot = xor32_sum(l_acc);
    const bool has = l_tot > 0.f;
    const float inv = has ? p.v_scale / l_tot : 0.f;
    const float lse_v = has ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
    if (he == 0) s_inv[32 * sr + ne] = inv;
    const int m_l = row0 + 32 * sr + ne;
    if (he == 0 && m_l < rows_valid) {
      const size_t rowb = (size_t)gF * p.H + (size_t)m_l;
      if (sg.single) {
        if (p.lse != nullptr) p.lse[out_row0 + rowb] = lse_v;
      } else {
        p.part_lse[(size_t)sg.slot * rows_per_b + rowb] = lse_v;
      }
    }
  }
  lds_barrier();
  float invr[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) invr[rb] = s_inv[32 * rb + ne];
  const bool f32out = !sg.single && !p.part_bf16;
  if (!f32out) {
    uint16_t* dst = sg.single ? p.out + out_row0 * kDv : (uint16_t*)p.part_o + (size_t)sg.slot * rows_per_b * kDv;
    if constexpr (!SCORE) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int row = 32 * rb + ne, col = 64 * pw + 32 * j + 8 * gq + 4 * he;
            const v16f& acc = o[4 * j + rb];
            const v2i wv = v2i{(int)pack_bf16x2(acc[4 * gq + 0] * invr[rb], acc[4 * gq + 1] * invr[rb]),
                               (int)pack_bf16x2(acc[4 * gq + 2] * invr[rb], acc[4 * gq + 3] * invr[rb])};
            *(lds_v2i*)(smem + row * kEpiPitch + 2 * col) = wv;
          }
        }
      }
    }
    lds_barrier();
    if constexpr (!SCORE) {
#pragma unroll 4
      for (int k = 0; k < 16; ++k) {
        const int row = 16 * pw + k;
        const v4i v = *(const lds_v4i*)(smem + row * kEpiPitch + 16 * lane);
        const int m_r = row0 + row;
        if (m_r < rows_valid) {
          const size_t rowb = (size_t)gF * p.H + (size_t)m_r;
          store_out(v, (v4i*)(dst + rowb * kDv + 8 * lane), sg.single);
        }
      }
    }
  } else {
    float* dst = (float*)p.part_o + (size_t)sg.slot * rows_per_b * kDv;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (!SCORE && (pw >> 2) == h) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int row = 32 * rb + ne, col = 64 * (pw & 3) + 32 * j + 8 * gq + 4 * he;
              const v16f& acc = o[4 * j + rb];
              *(__attribute__((address_space(3))) v4f*)(smem + row * kEpiPitch + 4 * col) =
                  v4f{acc[4 * gq + 0] * invr[rb], acc[4 * gq + 1] * invr[rb], acc[4 * gq + 2] * invr[rb],
                      acc[4 * gq + 3] * invr[rb]};
            }
          }
        }
      }
      lds_barrier();
      if constexpr (!SCORE) {
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
          const int row = 16 * pw + k;
          const v4f v = *(const __attribute__((address_space(3))) v4f*)(smem + row * kEpiPitch + 16 * lane);
          const int m_r = row0 + row;
          if (m_r < rows_valid) {
            const size_t rowb = (size_t)gF * p.H + (size_t)m_r;
            *(v4f*)(dst + rowb * kDv + 256 * h + 4 * lane) = v;
          }
        }
      }
      lds_barrier();
    }
  }
}

// The workgroup's slice of its row's work, segment by segment: finds the row's
// total work T and the slice's first sequence, records the merge metadata, and
// calls seg(sg, g, mt) for each (slice, sequence) segment in order.  Uniform
// across the workgroup (every wave computes the same answer).
// KEEP: lanes keep the sequences' values across the segments (kernels with registers to spare).
// OPQ: divisors and stored values of the segment loop are made opaque inside it, so that the
// compiler computes their vector copies there instead of keeping them across the loop (the
// four-wave kernels, whose registers are full; the twelve-wave kernel keeps them).
template <int UK, bool WIN, bool KEEP, bool OPQ, typename SegFn>
__device__ __forceinline__ void for_each_segment(const PartialParams& p, int wave, int lane, SegFn&& seg) {
  int w, u;
  if (p.xcd_map) {
    // slices are dealt to the 8 XCDs in turn.  Few rows: the U workgroups of one
    // slice are consecutive dispatches of one XCD (they read the same keys).
    // Many rows: the G slices of one row are dispatched together, row by row.
    const int bid = blockIdx.x, xcd = bid & 7, idx = bid >> 3;
    int sl;
    if (p.u_major) {
      const int gx = p.G >> 3;  // slices per XCD
      u = idx / gx;
      sl = idx - u * gx;
    } else {
      sl = idx / p.U;
      u = idx - sl * p.U;
    }
    w = sl * 8 + xcd;
  } else if (p.u_major) {
    u = blockIdx.x / p.G;
    w = blockIdx.x - u * p.G;
  } else {
    w = blockIdx.x / p.U;
    u = blockIdx.x - w * p.U;
  }
  if (u >= p.U) return;
  if (w >= p.G) return;
  const int g = u % p.q_len_eff;
  const int mt = u / p.q_len_eff;

  // ---- the row's work in cost units, and the slice's first sequence ----
  // Sequence b of this row holds n_b units (tiles).  It costs c_b per unit: 4, or p.lo_cost for
  // an E4M3 sequence that takes the second P term.  The slices cut the row's total cost C evenly,
  // and unit i of b belongs to the slice holding its position S_b + c_b i (S_b: the cost of the
  // sequences before b), so slices full of costlier units get fewer of them.
  // Every wave computes the same answer on its own (no LDS, no barrier): lane i sums the costs of
  // sequences [i*kper, (i+1)*kper), one wave-wide prefix sum gives C and each lane's first
  // position, and the lane whose range holds the slice's start is found by ballot.
  const int kper = (p.B + 63) >> 6;
  const int bl0 = min(lane * kper, p.B), bl1 = min(bl0 + kper, p.B);
  const int window = WIN ? p.window : 0;
  struct SeqV {
    int L, qlen, tok0, n, c;
  };
  auto load_seq = [&](int bb) -> SeqV {
    SeqV v;
    seq_tokens(p, bb, v.qlen, v.tok0);
    v.L = max(((cint_t*)p.seq_lens)[bb], 0);
    v.n = group_units_of<UK>(p, v.L, v.qlen, g, window);
    v.c = p.lo_cost != 4 && v.L <= kLoKeys ? p.lo_cost : 4;
    return v;
  };
  // With KEEP and at most 64 sequences lane b keeps sequence b's values, and the walks below read
  // them with readlane instead of waiting on memory again (each dependent load costs a memory
  // latency); kernels without registers to spare do not keep them.
  SeqV mine = {0, 0, 0, 0, 4};
  long long own = 0;
  for (int bb = bl0; bb < bl1; ++bb) {
    const SeqV v = load_seq(bb);
    own += (long long)v.c * v.n;
    mine = v;
  }
  auto seq_of = [&](int bb) -> SeqV {
    if (!KEEP || kper != 1) return load_seq(bb);
    SeqV v;
    v.L = __builtin_amdgcn_readlane(mine.L, bb);
    v.qlen = __builtin_amdgcn_readlane(mine.qlen, bb);
    v.tok0 = __builtin_amdgcn_readlane(mine.tok0, bb);
    v.n = __builtin_amdgcn_readlane(mine.n, bb);
    v.c = __builtin_amdgcn_readlane(mine.c, bb);
    return v;
  };
  const long long incl = wave_incl_scan_ll(own);
  const long long C = readlane_ll(incl, 63);
  int32_t* meta_u = p.meta != nullptr ? p.meta + 2 * (size_t)u * p.B : nullptr;
  if (w == 0 && wave == 0 && lane == 0 && meta_u != nullptr) ((long long*)(p.meta + 2 * (size_t)p.U * p.B))[u] = C;
  const long long a = slice_start(w, C, p.G), e = slice_start(w + 1, C, p.G);
  const long long excl = incl - own;
  // every sequence costs at least one unit, so a < C lies in exactly one non-empty lane range
  const unsigned long long hit = __builtin_amdgcn_ballot_w64(own > 0 && excl <= a && a < incl);
  if (hit == 0) return;  // past the last sequence
  const int hl = (int)__builtin_ctzll(hit);
  long long S = readlane_ll(excl, hl);
  int b = hl * kper;
  while (b + 1 < p.B) {
    const SeqV v = seq_of(b);
    const long long cb = (long long)v.c * v.n;
    if (a < S + cb) break;
    S += cb;
    ++b;
  }

  // ---- segments of this slice ----
  // The merge reads the slots of slices [first, last] of each sequence: every slice in that
  // range runs a segment of the sequence, an empty one (it writes O = 0, LSE = -inf) when no
  // unit's position falls inside the slice.
  while (b < p.B) {
    const SeqV v = seq_of(b);
    const int nb = v.n, cu = v.c;
    const long long first = S, last = first + (long long)cu * (nb - 1);
    if (first >= e) break;
    if (last >= a) {
      long long cuq = cu, Cq = C;
      if constexpr (OPQ) asm volatile("" : "+s"(cuq), "+s"(Cq));  // (no division reciprocal is hoisted out of this loop)
      const int u0 = a <= first ? 0 : (int)((a - first + cuq - 1) / cuq);
      const int u1 = max(u0, min(nb, (int)((e - first + cuq - 1) / cuq)));
      SegmentCtx sg;
      sg.b = b;
      sg.u0 = u0;
      sg.u1 = u1;
      sg.single = (u0 == 0 && u1 == nb);
      sg.slot = w + b;
      sg.L = v.L;
      sg.qlen = v.qlen;
      sg.tok0 = v.tok0;
      if (meta_u != nullptr && u0 == 0 && wave == 0 && lane_id_here() == 0) {
        int wv = w;
        if constexpr (OPQ) asm volatile("" : "+s"(wv));  // (a vector copy of w made above the loop would stay live, and spill)
        meta_u[2 * b] = wv;
        meta_u[2 * b + 1] = slice_of_unit(last, Cq, p.G);
      }
      seg(sg, g, mt);
    }
    S += (long long)cu * nb;
    ++b;
  }
}

template <int DT, bool FAST, bool WIN, bool XPV>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_split_kv_partial(PartialParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[kLdsBytes];
  __shared__ int s_flag[4];
  lds_t* smem = (lds_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps LDS bases in SGPRs
  // (only the default E4M3 instantiation: the others have no register to keep them in, and in the
  // 16-bit kernels the values held across their segments cost more than the loads they save)
  constexpr bool kKeep = DT == kFp8 && FAST && !WIN;
  // Fetch the parameters the slice walk needs together with those of the block mapping: the
  // compiler would otherwise load them only after the mapping's early exits, a second kernel-
  // argument round trip before the sequence lengths can be requested.
  asm volatile("" ::"s"(p.seq_lens), "s"(p.meta), "s"(p.B), "s"(p.q_len), "s"(p.F), "s"(p.q_len_eff),
               "s"(p.lo_cost), "s"(p.cu_q));
  for_each_segment<Traits<DT>::kTile, WIN, kKeep, true>(p, wave, lane, [&](const SegmentCtx& sg, int g, int mt) {
    if constexpr (DT == kFp8 && FAST && !WIN) {
      // two copies of the segment code, so that the second P term costs the long sequences nothing
      if (sg.L <= kLoKeys) {
        run_segment<DT, FAST, WIN, XPV, true>(p, smem, s_flag, sg, g, mt, wave, lane_id_here());
      } else {
        run_segment<DT, FAST, WIN, XPV, false>(p, smem, s_flag, sg, g, mt, wave, lane_id_here());
      }
    } else {
      run_segment<DT, FAST, WIN, XPV>(p, smem, s_flag, sg, g, mt, wave, lane_id_here());
    }
  });
}

template <bool FAST, bool WIN>
__global__ void __launch_bounds__(kThreadsR) __attribute__((amdgpu_waves_per_eu(3, 3)))
mla_split_kv_fp8_roles(PartialParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[kRLdsBytes];
  lds_t* smem = (lds_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // two instantiations in separate branches: a wave's registers hold only its role's state
  if (wave < 4) {
    for_each_segment<64, WIN, false, false>(p, wave, lane, [&](const SegmentCtx& sg, int g, int mt) {
      run_segment_roles<FAST, WIN, true>(p, smem, sg, g, mt, wave, lane);
    });
  } else {
    for_each_segment<64, WIN, false, false>(p, wave, lane, [&](const SegmentCtx& sg, int g, int mt) {
      run_segment_roles<FAST, WIN, false>(p, smem, sg, g, mt, wave, lane);
    });
  }
}

// Row `row` of sequence b's workspace slot -> its row of out / lse.  In a ragged
// batch the rows past the sequence's tokens hold nothing (false); the offsets are
// clamped exactly as the split-KV kernel clamps them.
__device__ __forceinline__ bool merge_out_row(const CombineParams& p, int b, int row, size_t& orow) {
  if (p.cu_q == nullptr) {
    orow = (size_t)b * p.rows_per_b + row;
    return true;
  }
  cint_t* cu = (cint_t*)p.cu_q;
  const int c0 = min(max(cu[b], 0), p.total_q);
  const int c1 = min(max(cu[b + 1], c0), p.total_q);
  if (row >= min(c1 - c0, p.q_len) * p.H) return false;
  orow = (size_t)c0 * p.H + row;
  return true;
}

// The slices [w0, w1] holding partials of row `row` of sequence b: those of the
// workgroup row (query group, row tile) the row belongs to.
__device__ __forceinline__ void merge_slices(const CombineParams& p, int b, int row, int& w0, int& w1) {
  const int t = row / p.H, h = row - t * p.H;
  const int g = t / p.F, f = t - g * p.F;
  const int u = ((f * p.H + h) / kTileM) * p.q_len_eff + g;
  const int32_t* m = p.meta + 2 * ((size_t)u * p.B + b);
  w0 = max(m[0], 0);
  w1 = min(m[1], p.G - 1);
}

// ---------------------------------------------------------------------------
// Merge: one workgroup per output row.  The slice weights exp(lse_s - LSE)
// are computed once per row into LDS (256 slices at a time); each of the four
// waves then sums 128 of the 512 latent columns (two per lane), with sixteen
// slices' loads in flight.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) mla_combine(CombineParams p) {
  __shared__ float s_w[256];
  __shared__ float s_red[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const long long grow = (long long)blockIdx.x;
  if (grow >= (long long)p.B * p.rows_per_b) return;
  const int b = (int)(grow / p.rows_per_b);
  const int row = (int)(grow - (long long)b * p.rows_per_b);
  size_t orow;
  if (!merge_out_row(p, b, row, orow)) return;
  int w0, w1;
  merge_slices(p, b, row, w0, w1);
  if (w0 >= w1) return;  // single slice: written by the partial kernel
  // (a slice without units of the sequence ran an empty segment: LSE -inf, O = 0)
  auto lse_of = [&](int s) -> float { return p.part_lse[(size_t)(s + b) * p.rows_per_b + row]; };
  const int n = w1 - w0 + 1;
  // LSE over the slices (each thread keeps the lse values of its slices)
  float my[4];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 256 * k;
    my[k] = i < n ? lse_of(w0 + i) : -INFINITY;
    mx = fmaxf(mx, my[k]);
  }
  for (int i = tid + 1024; i < n; i += 256) mx = fmaxf(mx, lse_of(w0 + i));
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  float sum = 0.f;
  if (mx > -INFINITY) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sum += expf(my[k] - mx);
    for (int i = tid + 1024; i < n; i += 256) sum += expf(lse_of(w0 + i) - mx);
  }
  sum = wave_sum(sum);
  if (lane == 0) s_red[wave] = sum;
  __syncthreads();
  sum = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  const float lse_out = mx > -INFINITY ? mx + logf(sum) : -INFINITY;

  const int d = 128 * wave + 2 * lane;
  float acc0 = 0.f, acc1 = 0.f;
  const size_t st_rows = (size_t)p.rows_per_b * kDv;  // elements between consecutive slots
  const size_t base = ((size_t)(w0 + b) * p.rows_per_b + row) * kDv + d;
  for (int c0 = 0; c0 < n && mx > -INFINITY; c0 += 256) {
    const int cn = min(256, n - c0);
    __syncthreads();
    if (tid < cn) s_w[tid] = expf((c0 + tid < 1024 ? my[(c0 + tid) >> 8] : lse_of(w0 + c0 + tid)) - lse_out);
    __syncthreads();
    if (p.part_bf16) {
      const uint16_t* src = (const uint16_t*)p.part_o + base + (size_t)c0 * st_rows;
#pragma unroll 16
      for (int i = 0; i < cn; ++i) {
        const float wgt = s_w[i];
        const uint32_t x = *(const uint32_t*)(src + (size_t)i * st_rows);
        // slots of empty slices hold stale bytes: select, never multiply them by 0
        acc0 += wgt > 0.f ? wgt * __builtin_bit_cast(float, x << 16) : 0.f;
        acc1 += wgt > 0.f ? wgt * __builtin_bit_cast(float, x & 0xffff0000u) : 0.f;
      }
    } else {
      const float* src = (const float*)p.part_o + base + (size_t)c0 * st_rows;
#pragma unroll 16
      for (int i = 0; i < cn; ++i) {
        const float wgt = s_w[i];
        const float2 x = *(const float2*)(src + (size_t)i * st_rows);
        acc0 += wgt > 0.f ? wgt * x.x : 0.f;
        acc1 += wgt > 0.f ? wgt * x.y : 0.f;
      }
    }
  }
  *(uint32_t*)(p.out + orow * kDv + d) = pack_bf16x2(acc0, acc1);
  if (p.lse != nullptr && tid == 0) p.lse[orow] = lse_out;
}

// ---------------------------------------------------------------------------
// Merge for rows spread over many slices: one wave per (output row, quarter of
// the 512 latent dims), four waves (one row) per workgroup, no barriers.  A
// load instruction covers 16 bytes of a lane for SPI slices at once (the
// quarter is 16 lanes of bf16 or 32 lanes of fp32), so 16 instructions keep a
// whole chunk of 16 SPI slices in flight (16 KiB per wave).  Each lane then sums
// its slices' values, weighted by exp(lse_s - LSE) (broadcast from the lane
// that computed them), and the lane groups holding the same dims combine by
// shuffles.  Empty slices' stale bytes are selected away, never multiplied.
// ---------------------------------------------------------------------------
template <bool BF16P>
__global__ void __launch_bounds__(256) mla_combine_wide(CombineParams p) {
  constexpr int LPS = BF16P ? 16 : 32;  // lanes covering one slice's quarter row (16 bytes each)
  constexpr int SPI = 64 / LPS;         // slices per load instruction
  constexpr int CS = 16 * SPI;          // slices per chunk (16 loads in flight)
  const int lane = threadIdx.x & 63;
  const int quarter = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long grow = (long long)blockIdx.x;
  if (grow >= (long long)p.B * p.rows_per_b) return;
  const int b = (int)(grow / p.rows_per_b);
  const int row = (int)(grow - (long long)b * p.rows_per_b);
  size_t orow;
  if (!merge_out_row(p, b, row, orow)) return;
  int w0, w1;
  merge_slices(p, b, row, w0, w1);
  if (w0 >= w1) return;  // single slice: written by the partial kernel
  const int n = w1 - w0 + 1;
  // (a slice without units of the sequence ran an empty segment: LSE -inf, O = 0)
  auto lse_of = [&](int s) -> float { return p.part_lse[(size_t)(s + b) * p.rows_per_b + row]; };
  const int grp = lane / LPS, sub = lane - grp * LPS;  // this lane: slice grp of each SPI, 16 bytes sub
  const size_t slot_elems = (size_t)p.rows_per_b * kDv;  // elements between consecutive slots
  const size_t base = ((size_t)(w0 + b) * p.rows_per_b + row) * kDv + 128 * quarter + (BF16P ? 8 : 4) * sub;
  auto load_chunk = [&](int c0, int cn, v4i* x) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int sl = SPI * i + grp;  // slice of the chunk this lane loads with instruction i
      if (sl < cn) {
        if constexpr (BF16P) {
          x[i] = *(const v4i*)((const uint16_t*)p.part_o + base + (size_t)(c0 + sl) * slot_elems);
        } else {
          x[i] = *(const v4i*)((const float*)p.part_o + base + (size_t)(c0 + sl) * slot_elems);
        }
      }
    }
  };
  // requests: the LSEs of the first 64 slices (one per lane) and the first chunk's partials,
  // before any of the LSE arithmetic
  const float l0 = lane < n ? lse_of(w0 + lane) : -INFINITY;
  v4i x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = v4i{0, 0, 0, 0};
  load_chunk(0, min(CS, n), x);
  float mx = l0;
  for (int i = lane + 64; i < n; i += 64) mx = fmaxf(mx, lse_of(w0 + i));
  mx = wave_max(mx);
  float sum = 0.f;
  if (mx > -INFINITY) {
    sum = expf(l0 - mx);  // 0 on lanes past n
    for (int i = lane + 64; i < n; i += 64) sum += expf(lse_of(w0 + i) - mx);
  }
  sum = wave_sum(sum);
  const float lse_out = mx > -INFINITY ? mx + logf(sum) : -INFINITY;

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (mx > -INFINITY) {
    for (int c0 = 0; c0 < n; c0 += CS) {
      const int cn = min(CS, n - c0);
      // slice weights of the chunk, one per lane (lanes past the chunk: 0)
      const float wl = lane < cn ? expf((c0 == 0 ? l0 : lse_of(w0 + c0 + lane)) - lse_out) : 0.f;
      if (c0 > 0) load_chunk(c0, cn, x);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int sl = SPI * i + grp;
        const float wgt = __shfl(wl, sl < 64 ? sl : 0, 64);
        const bool use = sl < cn && wgt > 0.f;
        if constexpr (BF16P) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t u = (uint32_t)x[i][e];
            acc[2 * e] += use ? wgt * __builtin_bit_cast(float, u << 16) : 0.f;
            acc[2 * e + 1] += use ? wgt * __builtin_bit_cast(float, u & 0xffff0000u) : 0.f;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // (through a scalar: a bit cast of the vector element itself read element 0 every time)
            const int xe = x[i][e];
            acc[e] += use ? wgt * __builtin_bit_cast(float, xe) : 0.f;
          }
        }
      }
    }
  }
  // lanes sub, sub + LPS, ... hold the same dims: sum across the lane groups (lane ^ 16 by
  // ds_swizzle inside each half, lane ^ 32 by v_permlane32_swap)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (BF16P || e < 4) {
      if constexpr (LPS == 16)
        acc[e] += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, acc[e]), (16 << 10) | 31));
      acc[e] = xor32_sum(acc[e]);
    }
  }
  if (lane < LPS) {
    if constexpr (BF16P) {
      const v4i packed = v4i{(int)pack_bf16x2(acc[0], acc[1]), (int)pack_bf16x2(acc[2], acc[3]),
                             (int)pack_bf16x2(acc[4], acc[5]), (int)pack_bf16x2(acc[6], acc[7])};
      *(v4i*)(p.out + orow * kDv + 128 * quarter + 8 * sub) = packed;
    } else {
      const v2i packed = v2i{(int)pack_bf16x2(acc[0], acc[1]), (int)pack_bf16x2(acc[2], acc[3])};
      *(v2i*)(p.out + orow * kDv + 128 * quarter + 4 * sub) = packed;
    }
  }
  if (p.lse != nullptr && quarter == 0 && lane == 0) p.lse[orow] = lse_out;
}

// ---------------------------------------------------------------------------
// Merge, one wave per output row (four rows per workgroup, no barriers): for
// batches whose sequences span few slices, where a whole workgroup per row
// would mostly wait.  Lane l owns latent dims [8l, 8l+8).  The row's first
// chunk of partial rows (16 slices of bf16, 8 of fp32) is requested together
// with the slice LSEs, before any of the LSE arithmetic, so a row that spans at
// most one chunk costs two memory round trips (the slice range, then LSEs and
// partials together).  Slice weights are computed by the lane of the slice and
// broadcast with readlane.
// ---------------------------------------------------------------------------
template <bool BF16P, int K>
__global__ void __launch_bounds__(256) mla_combine_rows(CombineParams p) {
  // K slices per chunk: K x 16 bytes of bf16 partials per lane, or K x 32 bytes of fp32
  const int lane = threadIdx.x & 63;
  // wave-uniform: the row, its slice range and T are then scalar values
  const long long grow = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (grow >= (long long)p.B * p.rows_per_b) return;
  const int b = (int)(grow / p.rows_per_b);
  const int row = (int)(grow - (long long)b * p.rows_per_b);
  size_t orow;
  if (!merge_out_row(p, b, row, orow)) return;
  int w0, w1;
  merge_slices(p, b, row, w0, w1);
  if (w0 >= w1) return;  // single slice: written by the partial kernel
  const int n = w1 - w0 + 1;
  // (a slice without units of the sequence ran an empty segment: LSE -inf, O = 0)
  auto lse_of = [&](int s) -> float { return p.part_lse[(size_t)(s + b) * p.rows_per_b + row]; };
  const size_t st_bytes = (size_t)p.rows_per_b * kDv * (BF16P ? 2 : 4);  // bytes between consecutive slots
  const uint8_t* src0 =
      (const uint8_t*)p.part_o + ((size_t)(w0 + b) * p.rows_per_b + row) * kDv * (BF16P ? 2 : 4) +
      (BF16P ? 16 : 32) * lane;
  // requests: the LSEs of the first 64 slices (one per lane) and the first chunk's partial rows
  const float l0 = lane < n ? lse_of(w0 + lane) : -INFINITY;
  using V = std::conditional_t<BF16P, v4i, v4f>;
  V x[K], y[K];  // y: the second 16 bytes of fp32 partials
#pragma unroll
  for (int j = 0; j < K; ++j) {
    x[j] = V{0, 0, 0, 0};
    y[j] = V{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (j < n) {
      const V* a = (const V*)(src0 + (size_t)j * st_bytes);
      x[j] = a[0];
      if constexpr (!BF16P) y[j] = a[1];
    }
  }
  float mx = l0;
  for (int i = lane + 64; i < n; i += 64) mx = fmaxf(mx, lse_of(w0 + i));
  mx = wave_max(mx);
  float sum = 0.f;
  if (mx > -INFINITY) {
    sum = expf(l0 - mx);  // 0 on lanes past n
    for (int i = lane + 64; i < n; i += 64) sum += expf(lse_of(w0 + i) - mx);
  }
  sum = wave_sum(sum);
  const float lse_out = mx > -INFINITY ? mx + logf(sum) : -INFINITY;

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (mx > -INFINITY) {
    for (int c0 = 0; c0 < n; c0 += 64) {
      const int cn = min(64, n - c0);
      const float wl = lane < cn ? expf((c0 == 0 ? l0 : lse_of(w0 + c0 + lane)) - lse_out) : 0.f;
      for (int i = 0; i < cn; i += K) {
        if (c0 + i > 0) {
#pragma unroll
          for (int j = 0; j < K; ++j) {
            if (i + j < cn) {
              const V* a = (const V*)(src0 + (size_t)(c0 + i + j) * st_bytes);
              x[j] = a[0];
              if constexpr (!BF16P) y[j] = a[1];
            }
          }
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
          // slots of empty slices hold stale bytes: select, never multiply them by 0
          const float wgt =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), min(i + j, 63)));
          const bool use = i + j < cn && wgt > 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (BF16P) {
              const uint32_t u = (uint32_t)x[j][e];
              acc[2 * e] += use ? wgt * __builtin_bit_cast(float, u << 16) : 0.f;
              acc[2 * e + 1] += use ? wgt * __builtin_bit_cast(float, u & 0xffff0000u) : 0.f;
            } else {
              acc[e] += use ? wgt * x[j][e] : 0.f;
              acc[4 + e] += use ? wgt * y[j][e] : 0.f;
            }
          }
        }
      }
    }
  }
  const v4i packed = v4i{(int)pack_bf16x2(acc[0], acc[1]), (int)pack_bf16x2(acc[2], acc[3]),
                         (int)pack_bf16x2(acc[4], acc[5]), (int)pack_bf16x2(acc[6], acc[7])};
  *(v4i*)(p.out + orow * kDv + 8 * lane) = packed;
  if (p.lse != nullptr && lane == 0) p.lse[orow] = lse_out;
}

// ---------------------------------------------------------------------------
// Pack + quantise: one thread per 16 elements of a 576-wide output row, 36
// threads per token, 7 tokens per 256-thread workgroup (index math in 32 bits).
// ---------------------------------------------------------------------------
constexpr int kPackThreadsPerToken = kDqk / 16;                   // 36
constexpr int kPackTokensPerBlock = 256 / kPackThreadsPerToken;  // 7

__device__ __forceinline__ float quant_in(uint32_t bits16, float scale) {
  const float x = __builtin_bit_cast(float, bits16 << 16) / scale;
  if (x != x) return x;
  return fminf(fmaxf(x, -448.f), 448.f);
}

// four inputs -> four E4M3 codes (round to nearest even; NaN -> the canonical 0x7F)
__device__ __forceinline__ uint32_t pack4_e4m3(const float* f) {
  int wv = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  wv = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], wv, true);
  uint32_t u = (uint32_t)wv;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (f[j] != f[j]) u = (u & ~(0xffu << (8 * j))) | (0x7fu << (8 * j));
  return u;
}

__global__ void __launch_bounds__(256) mla_kv_pack_fp8(PackParams p) {
  const int tid = threadIdx.x;
  const int lt = tid / kPackThreadsPerToken;
  if (lt >= kPackTokensPerBlock) return;
  const int grp = tid - lt * kPackThreadsPerToken;  // 16-element group: 0..31 latent, 32..35 rope
  const long long t = (long long)blockIdx.x * kPackTokensPerBlock + lt;
  if (t >= p.num_tokens) return;
  long long dst = t;
  if (p.slot_mapping != nullptr) dst = p.slot_mapping[t];
  if (dst < 0 || dst >= p.out_rows) return;
  const uint16_t* src = grp < 32 ? p.latent + (size_t)t * p.latent_stride + 16 * grp
                                 : p.rope + (size_t)t * p.rope_stride + 16 * (grp - 32);
  const uint4 x0 = *(const uint4*)src;
  const uint4 x1 = *(const uint4*)(src + 8);
  const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  float f[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f[2 * j] = quant_in(xs[j] & 0xffffu, p.scale);
    f[2 * j + 1] = quant_in(xs[j] >> 16, p.scale);
  }
  *(uint4*)(p.out + (size_t)dst * kDqk + 16 * grp) =
      make_uint4(pack4_e4m3(f), pack4_e4m3(f + 4), pack4_e4m3(f + 8), pack4_e4m3(f + 12));
}

}  // namespace

template <bool FAST>
void launch_fp8_roles(const PartialParams& p, bool win, dim3 grid, hipStream_t stream) {
  if (win) hipLaunchKernelGGL((mla_split_kv_fp8_roles<FAST, true>), grid, dim3(kThreadsR), 0, stream, p);
  else hipLaunchKernelGGL((mla_split_kv_fp8_roles<FAST, false>), grid, dim3(kThreadsR), 0, stream, p);
}

template <int DT, bool XPV>
void launch_partial_dt(const PartialParams& p, bool fast_pages, bool win, dim3 grid, dim3 block, hipStream_t stream) {
  if (fast_pages) {
    if (win) hipLaunchKernelGGL((mla_split_kv_partial<DT, true, true, XPV>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((mla_split_kv_partial<DT, true, false, XPV>), grid, block, 0, stream, p);
  } else {
    if (win) hipLaunchKernelGGL((mla_split_kv_partial<DT, false, true, XPV>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((mla_split_kv_partial<DT, false, false, XPV>), grid, block, 0, stream, p);
  }
}
template <int DT>
void launch_partial_16(const PartialParams& p, bool fast_pages, bool win, dim3 grid, dim3 block, hipStream_t stream) {
  if (cross_wave_pv(p.H_eff)) launch_partial_dt<DT, true>(p, fast_pages, win, grid, block, stream);
  else launch_partial_dt<DT, false>(p, fast_pages, win, grid, block, stream);
}

hipError_t launch_partial(const PartialParams& p_in, int dtype, bool fast_pages, hipStream_t stream) {
  const dim3 grid((unsigned)(p_in.G * p_in.U)), block(kThreads);
  // Cost model of the work partition (quarter tiles): a tile with the second P term costs about
  // 1.25 tiles in the twelve-wave kernel and 1.5 in the four-wave one.
  PartialParams p = p_in;
  // kernels without a sliding window are separate instantiations, so the
  // window's per-row state costs them no registers
  const bool win = p.window > 0;
  // E4M3 default: the four-wave kernel on whole-tile pages without a window (the instantiation with
  // the second P term), the twelve-wave kernel elsewhere
  const int fp8_kernel = p.kernel != 0 ? p.kernel : (fast_pages && !win ? 1 : 2);
  const bool lo_terms = dtype == kFp8 && (fp8_kernel == 2 || (fast_pages && !win));
  p.lo_cost = !lo_terms ? 4 : fp8_kernel == 2 ? 5 : 6;
  switch (dtype) {
    case kFp8:
      if (fp8_kernel == 1) {
        launch_partial_dt<kFp8, true>(p, fast_pages, win, grid, block, stream);  // the four-wave kernel
      } else if (fast_pages) {
        launch_fp8_roles<true>(p, win, grid, stream);
      } else {
        launch_fp8_roles<false>(p, win, grid, stream);
      }
      break;
    case kFp16: launch_partial_16<kFp16>(p, fast_pages, win, grid, block, stream); break;
    case kMixed: launch_partial_16<kMixed>(p, fast_pages, win, grid, block, stream); break;
    default: launch_partial_16<kBf16>(p, fast_pages, win, grid, block, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.rows_per_b;
  if (p.merge_kernel == 2 || combine_per_wave(p.B, p.G)) {
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    // chunk size: about a row's slices (G / B + 1 on average), fewer registers for fewer slices
    const long long G = p.G, B = p.B;
    if (p.part_bf16 && G >= 7 * B) hipLaunchKernelGGL((mla_combine_rows<true, 16>), grid, block, 0, stream, p);
    else if (p.part_bf16 && G >= 2 * B) hipLaunchKernelGGL((mla_combine_rows<true, 8>), grid, block, 0, stream, p);
    else if (p.part_bf16) hipLaunchKernelGGL((mla_combine_rows<true, 4>), grid, block, 0, stream, p);
    else if (G >= 2 * B) hipLaunchKernelGGL((mla_combine_rows<false, 8>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((mla_combine_rows<false, 4>), grid, block, 0, stream, p);
  } else if (p.merge_kernel == 1) {
    const dim3 grid((unsigned)rows), block(256);
    hipLaunchKernelGGL(mla_combine, grid, block, 0, stream, p);
  } else {
    const dim3 grid((unsigned)rows), block(256);
    if (p.part_bf16) hipLaunchKernelGGL(mla_combine_wide<true>, grid, block, 0, stream, p);
    else hipLaunchKernelGGL(mla_combine_wide<false>, grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;  // device -> address of that device's copy of `scratch`
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current: its own copy
    if (e != hipSuccess) return e;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

hipError_t launch_pack_fp8(const PackParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.num_tokens + kPackTokensPerBlock - 1) / kPackTokensPerBlock)), block(256);
  hipLaunchKernelGGL(mla_kv_pack_fp8, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
