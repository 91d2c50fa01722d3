// HBM -> LDS streaming probe for gfx950 (a measurement helper, not part of the decode path).
//
// It moves a buffer into LDS through the split-KV kernel's own load path -- global_load_lds_dwordx4,
// one KiB per wave instruction, 36,864-byte tiles (64 E4M3 rows of 576), two tiles in flight per
// wave, one 256-thread workgroup per compute unit holding a 4-tile LDS ring -- and does nothing
// else, so its rate is what that path can reach on the GPU it runs on: the reference bench.py
// reports the split-KV kernel's bandwidth against, beside the 8 TB/s of the specification.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kTileBytes = 36864;  // one KV tile: 36 one-KiB loads, 9 per wave
constexpr int kLoadsPerWave = kTileBytes / 1024 / 4;
constexpr int kRing = 4;

__global__ void __launch_bounds__(256) stream_probe_kernel(const uint8_t* src, long long ntiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kTileBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
  int k = 0;  // tiles this workgroup has issued
  for (long long t = blockIdx.x; t < ntiles; t += gridDim.x, ++k) {
    const uint8_t* tile = src + t * kTileBytes;
    const uint32_t stage = base + (uint32_t)((k % kRing) * kTileBytes);
#pragma unroll
    for (int kk = 0; kk < kLoadsPerWave; ++kk) {
      const int slot = wave + 4 * kk;  // this wave's kk-th KiB of the tile
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + 1024u * (uint32_t)slot);
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   ::"v"(tile + 1024 * slot + 16 * lane), "s"(m0) : "memory", "m0");
    }
    // at most two tiles of this wave in flight: the ring stage issued next is then free
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kLoadsPerWave) : "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

// Streams the first floor(bytes / 36864) tiles of `src` (device memory, caller-owned) into LDS
// with `workgroups` workgroups (0: one per compute unit) on `stream` (hipStream_t or NULL).
// Returns 0, or -1 if an argument is invalid, -2 if the launch fails.  Asynchronous.
extern "C" int mla_stream_probe(const void* src, long long bytes, int workgroups, void* stream) {
  if (src == nullptr || bytes < kTileBytes || workgroups < 0) return -1;
  if (workgroups == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -2;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -2;
    workgroups = cus;
  }
  const long long ntiles = bytes / kTileBytes;
  hipLaunchKernelGGL(stream_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const uint8_t*)src, ntiles);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
