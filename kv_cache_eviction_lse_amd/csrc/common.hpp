// Device-side building blocks shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] * B[16x32].
// Operands, lane l = 0..63, half = l / 32:
//   A: row l % 32, k = 8*half .. 8*half+7      B: col l % 32, same k range
//   C: col l % 32, rows 8*(r/4) + 4*half + (r%4) for register r = 0..15
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in register r by a lane of half `half`.
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte global load / store of raw bits.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Buffer resource over `bytes` bytes from `base` (gfx9 raw buffer: stride 0,
// word 3 = 0x00020000). A buffer load whose offset falls at or past `bytes`
// returns zero instead of touching memory, so a tile resource that covers
// only the rows that exist needs no clamped row indices. `base` and `bytes`
// must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Make a loaded value opaque to the optimiser: it then stays in registers
// instead of being re-loaded (rematerialised) where it is used in a loop.
__device__ __forceinline__ void pin(u32x4& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

}  // namespace kvs
