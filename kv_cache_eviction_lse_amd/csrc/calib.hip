// Measured ceilings for the benchmark (libkvscore_calib.so; not part of the
// scoring library's C ABI, which include/kvscore.h declares):
//   kvs_calib_copy  a plain device copy of n bytes with 16-byte non-temporal
//                   loads and stores, the form the eviction's row copy uses:
//                   the bandwidth ceiling for the eviction's bytes;
//   kvs_calib_mfma  v_mfma_f32_32x32x16_bf16 chains and nothing else, 4-wave
//                   workgroups at 3 per CU (the LSE pass's occupancy): the
//                   matrix-core ceiling; lane 0 of workgroup 0 also reads the
//                   shader clock counter and the 100 MHz real-time counter at
//                   its start and end, which gives the clock under that load.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

#define KVS_CALIB_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int CP_THREADS = 256;
constexpr int CP_UNROLL = 4;  // 16-byte pieces in flight per thread

__global__ __launch_bounds__(CP_THREADS) void calib_copy(const kvs::u32x4* src, kvs::u32x4* dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * CP_THREADS * CP_UNROLL;
  for (int64_t i0 = (int64_t)blockIdx.x * CP_THREADS * CP_UNROLL + threadIdx.x; i0 < n16; i0 += stride) {
    kvs::u32x4 v[CP_UNROLL];
#pragma unroll
    for (int u = 0; u < CP_UNROLL; ++u) {
      const int64_t i = i0 + (int64_t)u * CP_THREADS;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < CP_UNROLL; ++u) {
      const int64_t i = i0 + (int64_t)u * CP_THREADS;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

constexpr int MF_WAVES = 4;

// Each wave runs two independent chains of `iters` x 8 MFMAs (as the LSE
// pass's two query subtiles over the 8 k-steps of a 128-wide key tile).
__global__ __launch_bounds__(MF_WAVES * 64, 3) void calib_mfma(int iters, float* sink, uint64_t* clocks) {
  const int lane = threadIdx.x & 63;
  kvs::bf16x8 a[8], b0[8], b1[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    kvs::u32x4 v = {(uint32_t)(lane + s), (uint32_t)(3 * lane + s), 0x3f803f80u, 0x3c003c00u};
    kvs::pin(v);
    a[s] = kvs::as_bf16x8(v);
    b0[s] = kvs::as_bf16x8(kvs::u32x4{0x3f803f80u, (uint32_t)lane, 0u, 1u});
    b1[s] = kvs::as_bf16x8(kvs::u32x4{0x3f003f00u, 0u, (uint32_t)s, 2u});
  }
  uint64_t t0 = 0, r0 = 0;
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  kvs::f32x16 c0 = {}, c1 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      c0 = kvs::mfma32(a[s], b0[s], c0);
      c1 = kvs::mfma32(a[s], b1[s], c1);
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc += c0[r] + c1[r];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;  // keeps the chains live
  if (timer) {
    uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    uint64_t v0 = t1 - t0, v1 = r1 - r0;
    asm volatile("" : "+v"(v0), "+v"(v1));  // stored from vector registers
    clocks[0] = v0;
    clocks[1] = v1;
  }
}

}  // namespace

// Copies n bytes (a multiple of 16; both pointers 16-byte aligned) on `stream`.
KVS_CALIB_API int kvs_calib_copy(const void* src, void* dst, size_t n, void* stream) {
  if (!src || !dst || (n & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return 1;
  const int64_t n16 = (int64_t)(n / 16);
  if (n16 == 0) return 0;
  const int64_t per_block = (int64_t)CP_THREADS * CP_UNROLL;
  int64_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(calib_copy, dim3((unsigned)blocks), dim3(CP_THREADS), 0, static_cast<hipStream_t>(stream),
                     static_cast<const kvs::u32x4*>(src), static_cast<kvs::u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Runs `blocks` workgroups of 4 waves, each wave 2 x 8 x iters MFMAs of
// 32x32x16 (32768 flops each); sink: blocks * 256 floats; clocks: 2 uint64
// (shader clock cycles and 100 MHz ticks over workgroup 0's run), device.
KVS_CALIB_API int kvs_calib_mfma(int iters, int blocks, float* sink, uint64_t* clocks, void* stream) {
  if (iters < 1 || blocks < 1 || !sink || !clocks) return 1;
  hipLaunchKernelGGL(calib_mfma, dim3(blocks), dim3(MF_WAVES * 64), 0, static_cast<hipStream_t>(stream), iters, sink,
                     clocks);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
