// gfx950 (MI355X, CDNA4) kernels for MLA decode over a paged latent KV cache.
//
//  * mla_split_kv_partial: one workgroup = 4 waves = 128 folded query rows of
//    one (sequence, query group) and one contiguous slice of the batch's KV
//    work.  KV tiles (36,864 bytes: 64 fp8 rows or 32 bf16 rows of 576
//    elements) stream HBM -> LDS through a 4-deep ring filled by direct
//    global->LDS loads; scores S^T = K Q^T and the output O^T = V^T P^T run on
//    MFMA (32x32x64 f8f6f4 or 32x32x16 bf16), V^T being read from the same
//    LDS tile with the transposing LDS reads.  Online softmax in base 2 with a
//    lazy rescale; the FP8 probabilities carry a per-lane power-of-two block
//    scale through the MFMA's scale operand.  Writes the final bf16 O / fp32
//    LSE when the slice holds the whole sequence, else a partial (O, LSE).
//    (Split-KV partial kernel: TokenSpeed MLA article, section 2; query-token
//    folding: section 3.)
//  * mla_combine: LSE-weighted merge of the partials of every sequence that
//    spans several slices (article, section 2, the second, reduction kernel).
//  * mla_kv_pack_fp8: latent || rope -> E4M3 rows (tokenspeed-mla package
//    page, fused K/V pack + FP8 quantisation).
#include <math.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_t;
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(4))) const int32_t cint_t;

constexpr float kTau = 32.0f;  // rescale the accumulators only when a row max grows by more (log2 units)
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kDmaPerWave = kStageBytes / 1024 / 4;  // 9 one-KiB LDS writes per wave per tile

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

// LDS layout of a tile: row r, 16-byte chunk c lives at chunk slot
// r * kChunks + (c ^ swz(r)).  The XOR keeps every access pattern of the
// kernel (row-wise K reads, 8/4-row transposing V reads, 1 KiB DMA writes)
// free of bank conflicts on the 64-bank LDS.
template <int DT>
__device__ __forceinline__ int swz(int r) {
  if constexpr (DT == kFp8) {
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
__device__ __forceinline__ void dma16_sbase(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma16_vaddr(const void* vaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(vaddr), "s"(m0) : "memory", "m0");
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
// The compiler does not model hazards of asm MFMAs, so each one starts with
// a short s_nop (VALU-written operands) and the chain ends with qk_fence()
// before any VALU reads the accumulators.
__device__ __forceinline__ void qk_mfma_f8(v16f& acc, const v8i& a, const v8i& b, int sc) {
  asm("s_nop 2\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
      : "+v"(acc)
      : "v"(a), "v"(b), "v"(sc));
}
__device__ __forceinline__ void qk_mfma_bf16(v16f& acc, const v4i& a, const v4i& b) {
  asm("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_fence(v16f& a) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a)); }
__device__ __forceinline__ void qk_fence(v16f& a, v16f& b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}

// Keep a 16-float accumulator block in AGPRs: values defined by VALU code
// (zero-init, rescale) are moved there so the loop-carried output tile never
// gets a VGPR copy.
__device__ __forceinline__ void pin_agpr(v16f& x) { asm volatile("" : "+a"(x)); }

__device__ __forceinline__ int units_of(int L) { return L > 0 ? (L >> 6) + ((L & 63) != 0) : 1; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// ---------------------------------------------------------------------------
// Balanced partition of the batch's KV work: sequence b owns units_of(L_b)
// consecutive 64-key units; slice w of G covers units [w*T/G, (w+1)*T/G).
// Every (slice, sequence) intersection is one segment; its partial lives in
// workspace slot w + b (unique along the monotone staircase of segments).
// ---------------------------------------------------------------------------
__device__ __forceinline__ long long slice_start(long long w, long long T, int G) { return (w * T) / G; }
__device__ __forceinline__ int slice_of_unit(long long u, long long T, int G) {
  return (int)(((u + 1) * (long long)G - 1) / T);
}

struct SegmentCtx {
  int b, u0, u1, slot;
  bool single;
};

// ---------------------------------------------------------------------------
// One segment: rows of (b, group g, m-tile mt) against keys [64*u0, 64*u1).
//
// Softmax bookkeeping: each row's probabilities are taken relative to a
// reference m_ref fixed at the row's first tile with a visible key, so the
// output accumulators are only ever touched by MFMA (no rescale in the loop).
// If a later tile's row max exceeds m_ref by more than kTau (log2 units), the
// result could overflow: the workgroup then recomputes the segment with
// m_ref set to the exact row maxima seen in the first pass.
// ---------------------------------------------------------------------------
template <int DT, bool FAST>
__device__ __forceinline__ void run_segment(const PartialParams& p, lds_t* smem, int* s_flag, const SegmentCtx& sg,
                                            int g, int mt, int wave, int lane) {
  using TR = Traits<DT>;
  constexpr int TILE = TR::kTile;
  constexpr int RB = TR::kRowBytes;
  constexpr int CH = TR::kChunks;
  constexpr int ESZ = (DT == kFp8) ? 1 : 2;

  const int n = lane & 31;
  const int hh = lane >> 5;
  cint_t* seq_lens = (cint_t*)p.seq_lens;
  const int L = max(seq_lens[sg.b], 0);
  const int gF = g * p.F;
  // keys visible to the last token of this query group
  const int n_gmax = min(max(L - p.q_len + gF + p.F, 0), L);
  const int k0 = sg.u0 * kUnitKeys;
  const int k1 = min(sg.u1 * kUnitKeys, n_gmax);

  // this lane's query row (row n of the wave's 32)
  const int r = 32 * wave + n;
  const int m = mt * kTileM + r;
  const bool row_valid = m < p.H_eff;
  const int fold = row_valid ? m / p.H : 0;
  const int t_tok = gF + fold;
  const int n_row = row_valid ? min(max(L - p.q_len + t_tok + 1, 0), L) : 0;
  const int lim = min(n_row, k1);  // keys [k0, lim) are visible to this row
  const size_t rows_per_b = (size_t)p.q_len * p.H;
  const bool wave_active = (mt * kTileM + 32 * wave) < p.H_eff;

  // ---- Q rows into registers, laid out as the B operand of S^T = K Q^T ----
  // (invalid rows read row 0 of the group and are zeroed: no divergent branches)
  constexpr int QSTEPS = (DT == kFp8) ? 9 : 36;
  v8i qreg[QSTEPS];
  {
    const size_t qrow_idx = ((size_t)sg.b * p.q_len + gF) * p.H + (size_t)(row_valid ? m : 0);
    const uint8_t* qrow = p.q + qrow_idx * kDqk * ESZ;
    const int keep = row_valid ? -1 : 0;
#pragma unroll
    for (int c = 0; c < QSTEPS; ++c) {
      if constexpr (DT == kFp8) {
        const v4i* src = (const v4i*)(qrow + 64 * c + 32 * hh);
        const v4i x0 = src[0] & keep, x1 = src[1] & keep;
        qreg[c] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      } else {
        const v4i x = *(const v4i*)(qrow + 2 * (16 * c + 8 * hh)) & keep;
        qreg[c] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
      }
    }
  }

  v16f o[16];
  float m_ref = -INFINITY;  // reference the accumulators are relative to (log2 units)
  float l_acc = 0.f;        // this lane's share of sum exp2(s - m_ref)
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
    // [64*(wave+4kk), +64); lane -> slot -> (row, source chunk).  The nine
    // byte offsets row*RB + chunk*16 (< 2^16) are kept as packed halves.
    auto dma_row = [&](int kk) -> int { return (64 * (wave + 4 * kk) + lane) / CH; };
    auto dma_col = [&](int kk) -> int {
      const int slot = 64 * (wave + 4 * kk) + lane;
      const int row = slot / CH;
      return ((slot - row * CH) ^ swz<DT>(row)) * 16;
    };
    uint32_t dofs[(kDmaPerWave + 1) / 2];
#pragma unroll
    for (int i = 0; i < (kDmaPerWave + 1) / 2; ++i) {
      const uint32_t lo = (uint32_t)(dma_row(2 * i) * RB + dma_col(2 * i));
      const uint32_t hi = (2 * i + 1 < kDmaPerWave) ? (uint32_t)(dma_row(2 * i + 1) * RB + dma_col(2 * i + 1)) : 0u;
      dofs[i] = lo | (hi << 16);
    }

    auto page_of = [&](int pidx) -> int {
      int pg = bt[min(pidx, plast)];
      return min(max(pg, 0), p.num_pages - 1);
    };

    // Issue the DMA of tile `tt` (segment-relative) into its ring stage.
    auto issue_tile = [&](int tt) {
      const int key0 = k0 + tt * TILE;
      const uint32_t m0_stage = smem_base + (uint32_t)((tt % kStages) * kStageBytes);
      const bool tail = key0 + TILE > k1;
      if constexpr (FAST) {
        // page_size >= TILE: the tile is TILE consecutive rows of one page
        const int pg = page_of(key0 >> p.page_shift);
        const int rip = key0 & pmask;
        const uint8_t* sbase = p.kv + ((size_t)pg * p.page_size + rip) * RB;
        if (!tail) {
#pragma unroll
          for (int kk = 0; kk < kDmaPerWave; ++kk) {
            const uint32_t off = (dofs[kk >> 1] >> (16 * (kk & 1))) & 0xffffu;
            const uint32_t m0 = m0_stage + (uint32_t)(1024 * (wave + 4 * kk));
            dma16_sbase(off, sbase, __builtin_amdgcn_readfirstlane(m0));
          }
        } else {
          // rows past the segment's last key re-read row 0 (finite data, masked later)
#pragma unroll
          for (int kk = 0; kk < kDmaPerWave; ++kk) {
            const int row = dma_row(kk);
            const uint32_t off = (uint32_t)((key0 + row >= k1 ? 0 : row * RB) + dma_col(kk));
            const uint32_t m0 = m0_stage + (uint32_t)(1024 * (wave + 4 * kk));
            dma16_sbase(off, sbase, __builtin_amdgcn_readfirstlane(m0));
          }
        }
      } else {
        // page_size < TILE: up to four pages per tile
        const int pidx0 = key0 >> p.page_shift;
        const int pg0 = page_of(pidx0), pg1 = page_of(pidx0 + 1), pg2 = page_of(pidx0 + 2), pg3 = page_of(pidx0 + 3);
#pragma unroll
        for (int kk = 0; kk < kDmaPerWave; ++kk) {
          int key = key0 + dma_row(kk);
          if (key >= k1) key = key0;
          const int rel = (key >> p.page_shift) - pidx0;
          const int pg = rel == 0 ? pg0 : rel == 1 ? pg1 : rel == 2 ? pg2 : pg3;
          const uint8_t* src = p.kv + ((size_t)pg * p.page_size + (key & pmask)) * RB + dma_col(kk);
          const uint32_t m0 = m0_stage + (uint32_t)(1024 * (wave + 4 * kk));
          dma16_vaddr(src, __builtin_amdgcn_readfirstlane(m0));
        }
      }
    };

    // smallest visible limit over the wave's rows: tiles below it need no mask
    int lim_min = lim;
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) lim_min = min(lim_min, __shfl_xor(lim_min, o2, 64));

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
    } else {
      const int sw = swz<kBf16>(n);
#pragma unroll
      for (int x = 0; x < 4; ++x) kaddr[x] = n * RB + (((2 * x + hh) ^ sw) * 16);
      const int grp = lane >> 4, hs = grp >> 1, dsub = grp & 1, uu = lane & 15, rr = uu >> 2, c4 = uu & 3;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int sv = ((rr >> 1) << 2) | ((2 * v + hs) & 3);
        const int krow = 8 * v + 4 * hs + rr;
#pragma unroll
        for (int x = 0; x < 2; ++x)
          vaddr[2 * v + x] = krow * RB + (((4 * x + 2 * dsub + (c4 >> 1)) ^ sv) * 16) + 8 * (c4 & 1);
      }
    }

    float m_init = -INFINITY;
#pragma unroll 1
    for (int attempt = 0; attempt < 2; ++attempt) {
      float m_seen = -INFINITY;
      bool ovf = false;
      m_ref = m_init;
      l_acc = 0.f;
      if (attempt > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          o[i] = v16f{0};
          pin_agpr(o[i]);
        }
      }
      // all waves are done with the previous use of the LDS ring
      lds_barrier();
#pragma unroll
      for (int s = 0; s < kStages - 1; ++s)
        if (s < ntiles) issue_tile(s);

      for (int tt = 0; tt < ntiles; ++tt) {
        wait_tile_barrier(min(kStages - 2, ntiles - 1 - tt));
        if (tt + kStages - 1 < ntiles) issue_tile(tt + kStages - 1);
        if (!wave_active) continue;

        const lds_t* st = smem + (tt % kStages) * kStageBytes;
        const int key0 = k0 + tt * TILE;
        const bool need_mask = key0 + TILE > lim_min;

        if constexpr (DT == kFp8) {
          // ---- S^T = K Q^T : two 32-key blocks, K = 576 in 9 steps of 64 ----
          // one step of LDS reads in flight ahead of the MFMAs
          auto kread = [&](int c, int kb) -> v8i {
            const v4i x = *(const lds_v4i*)(st + kaddr[0] + 64 * c + 32 * RB * kb);
            const v4i y = *(const lds_v4i*)(st + kaddr[1] + 64 * c + 32 * RB * kb);
            return v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
          };
          v16f s0 = v16f{0}, s1 = v16f{0};
          v8i a0 = kread(0, 0), a1 = kread(0, 1);
#pragma unroll
          for (int c = 0; c < 9; ++c) {
            v8i n0 = a0, n1 = a1;
            if (c + 1 < 9) {
              n0 = kread(c + 1, 0);
              n1 = kread(c + 1, 1);
            }
            qk_mfma_f8(s0, a0, qreg[c], 127);
            qk_mfma_f8(s1, a1, qreg[c], 127);
            __builtin_amdgcn_sched_barrier(0);
            a0 = n0;
            a1 = n1;
          }
          qk_fence(s0, s1);
          // ---- mask, softmax numerators (base 2) ----
          if (need_mask) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = key0 + 8 * (i >> 2) + 4 * hh + (i & 3);
              if (key >= lim) s0[i] = -INFINITY;
              if (key + 32 >= lim) s1[i] = -INFINITY;
            }
          }
          float mx_raw = fmaxf(s0[0], s1[0]);
#pragma unroll
          for (int i = 1; i < 16; ++i) mx_raw = fmaxf(mx_raw, fmaxf(s0[i], s1[i]));
          const float mx = mx_raw * p.s_scale_log2;  // lane max, log2 units
          const float rm = fmaxf(mx, __shfl_xor(mx, 32, 64));
          m_seen = fmaxf(m_seen, rm);
          if (m_ref == -INFINITY) m_ref = rm;
          ovf = ovf || (rm > m_ref + kTau);
          const float mref = m_ref > -INFINITY ? m_ref : 0.f;
          // power-of-two block scale per query row: the row's largest p of this tile lands in
          // (128, 256].  The MFMA's 32-element scale blocks of a column interleave both lane
          // halves (bytes 0-15 of lanes n and n+32 take lane n's scale, bytes 16-31 take lane
          // n+32's), so both halves of a row must carry the same scale.
          int e = 0;
          if (rm > -INFINITY) e = 8 - (int)ceilf(rm - mref);
          e = min(max(e, -120), 120);
          const float off = mref - (float)e;
          float lsum = 0.f;
          int pk[8];
#pragma unroll
          for (int w4 = 0; w4 < 8; ++w4) {
            const v16f& sx = (w4 < 4) ? s0 : s1;
            float pv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[4 * (w4 & 3) + j], p.s_scale_log2, -off));
              lsum += pv[j];
            }
            int wv = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
            wv = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], wv, true);
            pk[w4] = wv;
          }
          l_acc += __builtin_ldexpf(lsum, -e);
          const v8i pt = v8i{pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};
          const int pscale = 127 - e;
          // ---- O^T += V^T P^T over 16 blocks of 32 latent dims ----
          auto vread = [&](int db) -> v8i {
            const int base = vaddr[db & 1] + 64 * (db >> 1);
            const v2i r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base));
            const v2i r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base + 16 * RB));
            const v2i r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base + 32 * RB));
            const v2i r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + base + 48 * RB));
            return v8i{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
          };
          __builtin_amdgcn_sched_barrier(0);
          v8i vt = vread(0);
#pragma unroll
          for (int db = 0; db < 16; ++db) {
            v8i vn = vt;
            if (db + 1 < 16) vn = vread(db + 1);
            o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vt, pt, o[db], 0, 0, 0, 127, 0, pscale);
            __builtin_amdgcn_sched_barrier(0);
            vt = vn;
          }
        } else {
          // ---- bf16: S^T for one 32-key block, K = 576 in 36 steps of 16 ----
          auto kread = [&](int c) -> v4i { return *(const lds_v4i*)(st + kaddr[c & 3] + 128 * (c >> 2)); };
          v16f s0 = v16f{0};
          v4i a = kread(0);
#pragma unroll
          for (int c = 0; c < 36; ++c) {
            v4i an = a;
            if (c + 1 < 36) an = kread(c + 1);
            const v4i qb = v4i{qreg[c][0], qreg[c][1], qreg[c][2], qreg[c][3]};
            qk_mfma_bf16(s0, a, qb);
            __builtin_amdgcn_sched_barrier(0);
            a = an;
          }
          qk_fence(s0);
          if (need_mask) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = key0 + 8 * (i >> 2) + 4 * hh + (i & 3);
              if (key >= lim) s0[i] = -INFINITY;
            }
          }
          float mx_raw = s0[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx_raw = fmaxf(mx_raw, s0[i]);
          const float mx = mx_raw * p.s_scale_log2;
          const float rm = fmaxf(mx, __shfl_xor(mx, 32, 64));
          m_seen = fmaxf(m_seen, rm);
          if (m_ref == -INFINITY) m_ref = rm;
          ovf = ovf || (rm > m_ref + kTau);
          const float mref = m_ref > -INFINITY ? m_ref : 0.f;
          float pv[16];
          float lsum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], p.s_scale_log2, -mref));
            lsum += pv[i];
          }
          l_acc += lsum;
          v8bf pbf[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const v4i pb = v4i{(int)pack_bf16x2(pv[8 * u + 0], pv[8 * u + 1]), (int)pack_bf16x2(pv[8 * u + 2], pv[8 * u + 3]),
                               (int)pack_bf16x2(pv[8 * u + 4], pv[8 * u + 5]), (int)pack_bf16x2(pv[8 * u + 6], pv[8 * u + 7])};
            pbf[u] = __builtin_bit_cast(v8bf, pb);
          }
          auto vread = [&](int db, int u) -> v4i {
            const int x = db & 1;
            const int base0 = vaddr[x] + 128 * (db >> 1) + 16 * RB * u;
            const int base1 = vaddr[2 + x] + 128 * (db >> 1) + 16 * RB * u;
            const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(st + base0));
            const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(st + base1));
            const v2i r0i = __builtin_bit_cast(v2i, r0), r1i = __builtin_bit_cast(v2i, r1);
            return v4i{r0i[0], r0i[1], r1i[0], r1i[1]};
          };
          __builtin_amdgcn_sched_barrier(0);
          v4i vt0 = vread(0, 0), vt1 = vread(0, 1);
#pragma unroll
          for (int db = 0; db < 16; ++db) {
            v4i vn0 = vt0, vn1 = vt1;
            if (db + 1 < 16) {
              vn0 = vread(db + 1, 0);
              vn1 = vread(db + 1, 1);
            }
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, vt0), pbf[0], o[db], 0, 0, 0);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, vt1), pbf[1], o[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            vt0 = vn0;
            vt1 = vn1;
          }
        }
      }
      // did any row of the workgroup outgrow its reference?
      const bool wave_ovf = __builtin_amdgcn_ballot_w64(ovf) != 0;
      if (lane == 0) s_flag[wave] = wave_ovf ? 1 : 0;
      lds_barrier();
      const bool redo = (s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3]) != 0;
      if (!redo) break;
      m_init = m_seen;
    }
  }

  // ---- epilogue: normalise, write final or partial ----
  // The 32x512 accumulator tile of each wave goes through LDS in four
  // 128-column passes (stored straight from the accumulator registers), then
  // every lane writes 64 contiguous columns of one row.
  const float l_tot = l_acc + __shfl_xor(l_acc, 32, 64);
  const bool has = l_tot > 0.f;
  const float inv = has ? p.v_scale / l_tot : 0.f;
  const float lse_v = has ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  const int rr = lane >> 1, hf = lane & 1;  // read-back role: row rr, columns [64*hf, +64) of the pass
  const float inv_r = __shfl(inv, rr, 64);
  const float lse_r = __shfl(lse_v, rr, 64);
  const int m_r = mt * kTileM + 32 * wave + rr;
  const bool valid_r = m_r < p.H_eff;
  const size_t rowb_r = (size_t)gF * p.H + (size_t)m_r;
  lds_barrier();  // every wave is done with the KV ring
  lds_t* wl = smem + wave * 16384;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
    for (int dbl = 0; dbl < 4; ++dbl) {
      const int db = 4 * pass + dbl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dl = 32 * dbl + 8 * i + 4 * hh;
        *(__attribute__((address_space(3))) v4f*)(wl + (n * 128 + dl) * 4) =
            v4f{o[db][4 * i + 0], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]};
      }
    }
    float v[64];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const v4f x = *(const __attribute__((address_space(3))) v4f*)(wl + (rr * 128 + 64 * hf + 4 * k) * 4);
      v[4 * k + 0] = x[0] * inv_r;
      v[4 * k + 1] = x[1] * inv_r;
      v[4 * k + 2] = x[2] * inv_r;
      v[4 * k + 3] = x[3] * inv_r;
    }
    if (valid_r) {
      const int d0 = 128 * pass + 64 * hf;
      if (sg.single) {
        uint16_t* orow = p.out + ((size_t)sg.b * rows_per_b + rowb_r) * kDv + d0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uint4 w;
          w.x = pack_bf16x2(v[8 * k + 0], v[8 * k + 1]);
          w.y = pack_bf16x2(v[8 * k + 2], v[8 * k + 3]);
          w.z = pack_bf16x2(v[8 * k + 4], v[8 * k + 5]);
          w.w = pack_bf16x2(v[8 * k + 6], v[8 * k + 7]);
          *(uint4*)(orow + 8 * k) = w;
        }
      } else if (p.part_bf16) {
        uint16_t* orow = (uint16_t*)p.part_o + ((size_t)sg.slot * rows_per_b + rowb_r) * kDv + d0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uint4 w;
          w.x = pack_bf16x2(v[8 * k + 0], v[8 * k + 1]);
          w.y = pack_bf16x2(v[8 * k + 2], v[8 * k + 3]);
          w.z = pack_bf16x2(v[8 * k + 4], v[8 * k + 5]);
          w.w = pack_bf16x2(v[8 * k + 6], v[8 * k + 7]);
          *(uint4*)(orow + 8 * k) = w;
        }
      } else {
        float* orow = (float*)p.part_o + ((size_t)sg.slot * rows_per_b + rowb_r) * kDv + d0;
#pragma unroll
        for (int k = 0; k < 16; ++k) *(v4f*)(orow + 4 * k) = v4f{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
      }
    }
  }
  if (valid_r && hf == 0) {
    if (sg.single) {
      if (p.lse != nullptr) p.lse[(size_t)sg.b * rows_per_b + rowb_r] = lse_r;
    } else {
      p.part_lse[(size_t)sg.slot * rows_per_b + rowb_r] = lse_r;
    }
  }
}

template <int DT, bool FAST>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_split_kv_partial(PartialParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[kStages * kStageBytes];
  __shared__ long long s_red[4];
  __shared__ long long s_found[2];
  __shared__ int s_flag[4];
  lds_t* smem = (lds_t*)smem_raw;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int w, u;
  if (p.xcd_map) {
    // the U workgroups of one slice are consecutive dispatches of one XCD
    const int bid = blockIdx.x, xcd = bid & 7, idx = bid >> 3;
    const int sl = idx / p.U;
    u = idx - sl * p.U;
    w = sl * 8 + xcd;
  } else {
    w = blockIdx.x / p.U;
    u = blockIdx.x - w * p.U;
  }
  if (w >= p.G) return;
  const int g = u % p.q_len_eff;
  const int mt = u / p.q_len_eff;

  // ---- total work T (units) ----
  long long local = 0;
  for (int b = tid; b < p.B; b += kThreads) local += units_of(p.seq_lens[b]);
  local = wave_sum_ll(local);
  if (lane == 0) s_red[wave] = local;
  __syncthreads();
  const long long T = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  // the merge needs T to recognise empty slices (they write no partials)
  if (blockIdx.x == 0 && tid == 0 && p.meta != nullptr) *(long long*)(p.meta + 2 * p.B) = T;
  const long long t0 = slice_start(w, T, p.G), t1 = slice_start(w + 1, T, p.G);
  if (t0 >= t1) return;
  __syncthreads();

  // ---- first sequence of the slice: chunked block scan over sequences ----
  long long base = 0;
  if (tid == 0) s_found[0] = -1;
  for (int start = 0; start < p.B; start += kThreads) {
    const int b = start + tid;
    const long long nb = b < p.B ? units_of(p.seq_lens[b]) : 0;
    long long incl = nb;
#pragma unroll
    for (int o2 = 1; o2 < 64; o2 <<= 1) {
      const long long y = __shfl_up(incl, o2, 64);
      if (lane >= o2) incl += y;
    }
    __syncthreads();
    if (lane == 63) s_red[wave] = incl;
    __syncthreads();
    long long woff = 0;
    for (int k = 0; k < wave; ++k) woff += s_red[k];
    const long long P = base + woff + incl - nb;
    if (b < p.B && P <= t0 && t0 < P + nb) {
      s_found[0] = b;
      s_found[1] = P;
    }
    base += s_red[0] + s_red[1] + s_red[2] + s_red[3];
    __syncthreads();
    if (s_found[0] >= 0) break;
  }
  int b = (int)s_found[0];
  long long P = s_found[1];

  // ---- segments of this slice ----
  long long cur = t0;
  cint_t* seq_lens = (cint_t*)p.seq_lens;
  while (cur < t1 && b < p.B) {
    const int nb = units_of(seq_lens[b]);
    const long long seg_end = min(t1, P + nb);
    SegmentCtx sg;
    sg.b = b;
    sg.u0 = (int)(cur - P);
    sg.u1 = (int)(seg_end - P);
    sg.single = (sg.u0 == 0 && sg.u1 == nb);
    sg.slot = w + b;
    if (p.meta != nullptr && sg.u0 == 0 && u == 0 && tid == 0) {
      p.meta[2 * b] = w;
      p.meta[2 * b + 1] = slice_of_unit(P + nb - 1, T, p.G);
    }
    run_segment<DT, FAST>(p, smem, s_flag, sg, g, mt, wave, lane);
    cur = seg_end;
    P += nb;
    ++b;
  }
}

// ---------------------------------------------------------------------------
// Merge: one wave per output row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) mla_combine(CombineParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long grow = (long long)blockIdx.x * 4 + wave;
  if (grow >= (long long)p.B * p.rows_per_b) return;
  const int b = (int)(grow / p.rows_per_b);
  const int row = (int)(grow - (long long)b * p.rows_per_b);
  const int w0 = max(p.meta[2 * b], 0), w1 = min(p.meta[2 * b + 1], p.G - 1);
  if (w0 >= w1) return;  // single slice: written by the partial kernel
  // slices of the range that hold no work (more slices than units) wrote nothing
  const long long T = *(const long long*)(p.meta + 2 * p.B);
  auto empty = [&](int s) { return slice_start(s, T, p.G) == slice_start(s + 1, T, p.G); };

  float mx = -INFINITY;
  for (int s = w0 + lane; s <= w1; s += 64)
    if (!empty(s)) mx = fmaxf(mx, p.part_lse[(size_t)(s + b) * p.rows_per_b + row]);
  mx = wave_max(mx);
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float lse_out = -INFINITY;
  if (mx > -INFINITY) {
    float sum = 0.f;
    for (int s = w0 + lane; s <= w1; s += 64)
      if (!empty(s)) sum += expf(p.part_lse[(size_t)(s + b) * p.rows_per_b + row] - mx);
    sum = wave_sum(sum);
    lse_out = mx + logf(sum);
    for (int s = w0; s <= w1; ++s) {
      if (empty(s)) continue;
      const size_t prow = (size_t)(s + b) * p.rows_per_b + row;
      const float wgt = expf(p.part_lse[prow] - lse_out);
      if (p.part_bf16) {
        const uint4 x = *(const uint4*)((const uint16_t*)p.part_o + prow * kDv + 8 * lane);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] += wgt * __builtin_bit_cast(float, xs[j] << 16);
          v[2 * j + 1] += wgt * __builtin_bit_cast(float, xs[j] & 0xffff0000u);
        }
      } else {
        const v4f* src = (const v4f*)((const float*)p.part_o + prow * kDv + 8 * lane);
        const v4f x0 = src[0], x1 = src[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] += wgt * x0[j];
          v[4 + j] += wgt * x1[j];
        }
      }
    }
  }
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]);
  w.w = pack_bf16x2(v[6], v[7]);
  *(uint4*)(p.out + ((size_t)b * p.rows_per_b + row) * kDv + 8 * lane) = w;
  if (p.lse != nullptr && lane == 0) p.lse[(size_t)b * p.rows_per_b + row] = lse_out;
}

// ---------------------------------------------------------------------------
// Pack + quantise: one thread per 8 elements of a 576-wide output row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float quant_in(uint32_t bits16, float scale) {
  const float x = __builtin_bit_cast(float, bits16 << 16) / scale;
  if (x != x) return x;
  return fminf(fmaxf(x, -448.f), 448.f);
}

__global__ void __launch_bounds__(256) mla_kv_pack_fp8(PackParams p) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)p.num_tokens * 72;
  if (gid >= total) return;
  const int t = (int)(gid / 72);
  const int grp = (int)(gid - (long long)t * 72);
  long long dst = t;
  if (p.slot_mapping != nullptr) dst = p.slot_mapping[t];
  if (dst < 0 || dst >= p.out_rows) return;
  uint4 x;
  if (grp < 64) {
    x = *(const uint4*)(p.latent + (size_t)t * p.latent_stride + 8 * grp);
  } else {
    x = *(const uint4*)(p.rope + (size_t)t * p.rope_stride + 8 * (grp - 64));
  }
  const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = quant_in(xs[j] & 0xffffu, p.scale);
    f[2 * j + 1] = quant_in(xs[j] >> 16, p.scale);
  }
  uint32_t outw[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int wv = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * h + 0], f[4 * h + 1], 0, false);
    wv = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * h + 2], f[4 * h + 3], wv, true);
    uint32_t u = (uint32_t)wv;
    // canonical NaN code 0x7F (the convert may set the sign bit)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (f[4 * h + j] != f[4 * h + j]) u = (u & ~(0xffu << (8 * j))) | (0x7fu << (8 * j));
    outw[h] = u;
  }
  *(uint2*)(p.out + (size_t)dst * kDqk + 8 * grp) = make_uint2(outw[0], outw[1]);
}

}  // namespace

hipError_t launch_partial(const PartialParams& p, int dtype, bool fast_pages, hipStream_t stream) {
  const dim3 grid((unsigned)(p.G * p.U)), block(kThreads);
  if (dtype == kFp8) {
    if (fast_pages)
      hipLaunchKernelGGL((mla_split_kv_partial<kFp8, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((mla_split_kv_partial<kFp8, false>), grid, block, 0, stream, p);
  } else {
    if (fast_pages)
      hipLaunchKernelGGL((mla_split_kv_partial<kBf16, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((mla_split_kv_partial<kBf16, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.rows_per_b;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  hipLaunchKernelGGL(mla_combine, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(const PackParams& p, hipStream_t stream) {
  const long long total = (long long)p.num_tokens * 72;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  hipLaunchKernelGGL(mla_kv_pack_fp8, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
