// Value norms ||W_O v_i|| per KV head and key: the weight the KVzip+ score
// puts on a_ji ("KVzap: Fast, Adaptive, and Faithful KV Cache Pruning", §3.2,
// Eq. 3 and its variable table). W_O is [d_model, Hkv * D]; head h's values
// meet its column block [h*D, (h+1)*D).
//
// Y^T = W_h V^T on v_mfma_f32_32x32x16_bf16, output features as rows and keys
// as columns, reduced to sum_f y_f^2 in registers (products of bf16 values are
// exact; accumulation is fp32):
//   * a workgroup owns NW * NT * 32 keys of one KV head; each wave keeps its
//     NT * 32 value rows in VGPRs as B operands for the whole kernel;
//   * W_h streams past in tiles of 128 output features through a
//     double-buffered LDS stage shared by the waves;
//   * a lane holds one key column and 16 feature rows of each 32 x 32 block,
//     so the sum of squares is in-register; the two half-waves are added once
//     at the end, then one square root per key.
//   * the head dimension is read in the permuted order of the score pass
//     (lane half h takes elements [h*D/2, h*D/2 + D/2)) on both operands.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace kvs {
namespace {

struct VnParams {
  const uint16_t* V;
  const uint16_t* W;
  float* out;
  int64_t v_hs, v_ts, w_rs;
  int64_t n;        // keys per head
  int d_model;
  int Hkv;
};

constexpr int VN_NW = 8, VN_NT = 2, VN_RT = 4;

template <int D>
__global__ __launch_bounds__(VN_NW * WAVE) void vnorm_kernel(VnParams p) {
  constexpr int NW = VN_NW, NT = VN_NT, RT = VN_RT;
  constexpr int TR = RT * 32;                  // features per tile
  constexpr int STEPS = D / 16;
  constexpr int LDS_STRIDE = D * 2 + 16;       // padded feature rows
  constexpr int NTHREADS = NW * WAVE;
  constexpr int CHUNKS = TR * D / 8;
  constexpr int CPR = D / 8;
  constexpr int CPT = CHUNKS / NTHREADS;
  static_assert(CHUNKS % NTHREADS == 0, "tile pieces must split evenly over the threads");
  constexpr int BK = NW * NT * 32;

  __shared__ __attribute__((aligned(16))) char s_w[2][TR * LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const int h = blockIdx.x % p.Hkv;
  const int kb = blockIdx.x / p.Hkv;
  const int64_t wave_key0 = (int64_t)kb * BK + (int64_t)wave * NT * 32;

  // resident values (B operands); keys past the end load the last key and are never written
  bf16x8 vreg[NT][STEPS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int64_t key = wave_key0 + 32 * t + col;
    key = key < p.n ? key : p.n - 1;
    const uint16_t* vp = p.V + (int64_t)h * p.v_hs + key * p.v_ts + half * (D / 2);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      u32x4 v = ld16(vp + 8 * s);
      pin(v);
      vreg[t][s] = as_bf16x8(v);
    }
  }

  // W_h tiles: rows f0 .. f0+63 of the column block; rows past d_model read zero
  int voff[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = tid + c * NTHREADS;
    voff[c] = (int)((idx / CPR) * p.w_rs * 2 + (idx % CPR) * 16);
  }
  const uint16_t* wbase = p.W + (int64_t)h * D;
  u32x4 pre[CPT];
  auto load_tile = [&](int ft) {
    const int f0 = ft * TR;
    const int rows = min(p.d_model - f0, TR);
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(wbase + (int64_t)f0 * p.w_rs, rows * (int)p.w_rs * 2);
#pragma unroll
    for (int c = 0; c < CPT; ++c) pre[c] = buf_ld16(r, voff[c]);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NTHREADS;
      *reinterpret_cast<u32x4*>(&s_w[buf][(idx / CPR) * LDS_STRIDE + (idx % CPR) * 16]) = pre[c];
    }
  };

  float sq[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) sq[t] = 0.f;

  const int n_tiles = (p.d_model + TR - 1) / TR;
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int ft = 0; ft < n_tiles; ++ft) {
    const int cur = ft & 1;
    if (ft + 1 < n_tiles) load_tile(ft + 1);
#pragma unroll
    for (int rs = 0; rs < RT; ++rs) {
      if (rs) __builtin_amdgcn_sched_barrier(0);
      bf16x8 a[STEPS];
      const char* wrow = &s_w[cur][(rs * 32 + col) * LDS_STRIDE + half * D];
#pragma unroll
      for (int s = 0; s < STEPS; ++s) a[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(wrow + 16 * s));
#pragma unroll
      for (int st = 0; st < NT; ++st) {
        f32x16 y = mfma32(a[0], vreg[st][0], f32x16{});
#pragma unroll
        for (int s = 1; s < STEPS; ++s) y = mfma32(a[s], vreg[st][s], y);
        float acc = sq[st];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc = __builtin_fmaf(y[r], y[r], acc);
        sq[st] = acc;
      }
    }
    if (ft + 1 < n_tiles) store_tile(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int st = 0; st < NT; ++st) {
    const float tot = sq[st] + __shfl_xor(sq[st], 32);
    const int64_t key = wave_key0 + 32 * st + col;
    if (half == 0 && key < p.n) p.out[(int64_t)h * p.n + key] = sqrtf(tot);
  }
}

template <int D>
hipError_t run(const VnParams& p, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((vnorm_kernel<D>), dim3(nblocks), dim3(VN_NW * WAVE), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vnorm(const kvs_vnorm_desc& d, const uint16_t* V, const uint16_t* W_O, float* vnorm,
                        hipStream_t s) {
  if (d.n_tok == 0) return hipSuccess;
  VnParams p{};
  p.V = V; p.W = W_O; p.out = vnorm;
  p.v_hs = d.v_head_stride; p.v_ts = d.v_tok_stride; p.w_rs = d.wo_row_stride;
  p.n = d.n_tok; p.d_model = d.d_model; p.Hkv = d.n_kvheads;
  constexpr int BK = VN_NW * VN_NT * 32;
  const int64_t nblocks = ((d.n_tok + BK - 1) / BK) * d.n_kvheads;
  if (d.head_dim == 128) return run<128>(p, (int)nblocks, s);
  return run<64>(p, (int)nblocks, s);
}

}  // namespace kvs
