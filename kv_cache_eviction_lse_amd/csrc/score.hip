// Transposed score pass: per-key reductions of exp(scale*q.k - lse_j) over
// query rows, without an attention map.
//
// max mode (KVzip Eq. 1 / KVzip+ Eq. 3 of "KVzap: Fast, Adaptive, and
// Faithful KV Cache Pruning", §3.1-§3.2): s_i = vnorm_i * max_{g,j}
//   exp(scale*q_j^g.k_i - lse_j^g - ln hnorm_j), every context key visible to
//   every repeat query.
// sum mode (KVpop future-attention target, "[논문리뷰] KVpop ..." §1):
//   t_i = vnorm_i * sum_{g} sum_{j >= i + w} exp(scale*q_j^g.k_i - lse_j^g - ln hnorm_j).
//
// Layout of the work:
//   * a workgroup owns BK = NWAVES * NT * 32 consecutive keys of one KV head;
//     each wave keeps its NT*32 keys in VGPRs as MFMA B operands for the whole
//     kernel (the key tile never leaves the chip);
//   * the group's query rows stream past in tiles of 32 through a
//     double-buffered LDS stage, shared by all waves of the workgroup;
//   * S = Q_tile * K^T on v_mfma_f32_32x32x16_bf16 with queries as rows, so a
//     lane holds one key column and 16 query rows: the reduction over queries
//     is in-register, and the two half-waves are combined once at the end;
//   * the per-row bias -(lse_j + ln hnorm_j)/scale is the accumulator's
//     initial value, so the MFMA result is already the shifted logit / scale.
//     max mode then needs only a running max per lane and one exp per key;
//     sum mode takes one exp2 per pair.
//   * the head dimension is read in a permuted order (lane half h takes
//     elements [h*D/2, h*D/2 + D/2) in steps of 8) on both operands; a dot
//     product does not depend on the order of its terms.
#include "common.hpp"
#include "internal.hpp"

namespace kvs {
namespace {

struct ScoreParams {
  const uint16_t* Q;
  const uint16_t* K;
  const float* lse;
  const float* vnorm;
  const float* hnorm;
  float* out;
  int64_t q_hs, q_ts, k_hs, k_ts;
  int64_t n_keys;  // context keys (max) or T (sum)
  int64_t n_q;     // queries per query head (max) or T (sum)
  int64_t window;  // sum mode
  int Hkv, G;
  int n_kblocks;   // key blocks per KV head
  int nsplit;      // max mode: query-row splits per key block
  int use_atomic;  // max mode: combine with atomicMax on the score bits
  float scale;
};

template <int D>
struct Tile {
  static constexpr int STEPS = D / 16;           // k-steps of 16 per MFMA chain
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int LDS_STRIDE = ROW_BYTES + 16;  // pad: 16 rows hit distinct banks
  static constexpr int CHUNKS = 32 * D / 8;      // 16-byte pieces per 32-row tile
  static constexpr int BYTES = 32 * LDS_STRIDE;
};

template <int D, int NWAVES, int NT, bool SUM>
__global__ __launch_bounds__(NWAVES * WAVE) void score_kernel(ScoreParams p) {
  using T = Tile<D>;
  constexpr int NTHREADS = NWAVES * WAVE;
  constexpr int BK = NWAVES * NT * 32;
  constexpr int CPT = (T::CHUNKS + NTHREADS - 1) / NTHREADS;  // 16-B chunks per thread per tile
  constexpr int CHUNKS_PER_ROW = D / 8;

  __shared__ __attribute__((aligned(16))) char s_q[2][T::BYTES];
  __shared__ __attribute__((aligned(16))) float s_bias[2][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int b = blockIdx.x;
  const int h = b % p.Hkv;
  const int rest = b / p.Hkv;
  const float inv_scale = 1.0f / p.scale;
  const float c2 = p.scale * LOG2E;

  // work items: max mode -> one key block and one query split;
  // sum mode -> a pair of key blocks (kb, n_kblocks-1-kb), balancing the triangle.
  int kb_list[2];
  int n_items = 1;
  int split = 0;
  if (SUM) {
    kb_list[0] = rest;
    kb_list[1] = p.n_kblocks - 1 - rest;
    n_items = (kb_list[1] != kb_list[0]) ? 2 : 1;
  } else {
    kb_list[0] = rest % p.n_kblocks;
    split = rest / p.n_kblocks;
  }

  for (int item = 0; item < n_items; ++item) {
    const int kb = kb_list[item];
    const int64_t key0 = (int64_t)kb * BK;
    const int64_t wave_key0 = key0 + (int64_t)wave * NT * 32;

    // ---- resident keys: B operands (col = key, k-range per half, permuted D)
    bf16x8 kreg[NT][T::STEPS];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t key = wave_key0 + 32 * t + col;
      const bool ok = key < p.n_keys;
      const uint16_t* kp = p.K + (int64_t)h * p.k_hs + (ok ? key : 0) * p.k_ts + half * (D / 2);
#pragma unroll
      for (int s = 0; s < T::STEPS; ++s) {
        u32x4 v = ok ? ld16(kp + 8 * s) : u32x4{0, 0, 0, 0};
        kreg[t][s] = as_bf16x8(v);
      }
    }

    // ---- the row space this item visits, in tiles of 32 rows
    // max: rows r in [0, G*n_q): g = r / n_q, j = r % n_q; split s takes an even share.
    // sum: per group head, j-tiles aligned to 32 from the first row any key of the
    //      block can count (j >= key0 + window) to T.
    int64_t t_begin, t_end, jt_first = 0, tiles_per_g = 0;
    if (SUM) {
      const int64_t j_lo = key0 + p.window;
      if (j_lo >= p.n_q) {
        tiles_per_g = 0;
      } else {
        jt_first = j_lo / 32;
        tiles_per_g = (p.n_q + 31) / 32 - jt_first;
      }
      t_begin = 0;
      t_end = tiles_per_g * p.G;
    } else {
      const int64_t n_tiles = ((int64_t)p.G * p.n_q + 31) / 32;
      t_begin = n_tiles * split / p.nsplit;
      t_end = n_tiles * (split + 1) / p.nsplit;
    }

    // row rr of tile t -> (query head g, query j); valid = j inside the sequence
    auto row_of = [&](int64_t t, int rr, int& g, int64_t& j) -> bool {
      if (SUM) {
        const int64_t gl = t / tiles_per_g;
        j = (jt_first + t % tiles_per_g) * 32 + rr;
        g = h * p.G + (int)gl;
        return j < p.n_q;
      } else {
        const int64_t r = t * 32 + rr;
        const int64_t gl = r / p.n_q;
        j = r - gl * p.n_q;
        g = h * p.G + (int)gl;
        return gl < p.G;
      }
    };

    u32x4 pre[CPT];
    float pre_bias = 0.f;
    auto load_tile = [&](int64_t t) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + c * NTHREADS;
        pre[c] = u32x4{0, 0, 0, 0};
        if (idx < T::CHUNKS) {
          const int rr = idx / CHUNKS_PER_ROW, part = idx % CHUNKS_PER_ROW;
          int g;
          int64_t j;
          if (row_of(t, rr, g, j))
            pre[c] = ld16(p.Q + (int64_t)g * p.q_hs + j * p.q_ts + part * 8);
        }
      }
      if (tid < 32) {
        int g;
        int64_t j;
        if (row_of(t, tid, g, j)) {
          const float hn = p.hnorm ? p.hnorm[j] : 1.0f;
          pre_bias = -(p.lse[(int64_t)g * p.n_q + j] + __logf(hn)) * inv_scale;
        } else {
          pre_bias = -INFINITY;
        }
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + c * NTHREADS;
        if (idx < T::CHUNKS) {
          const int rr = idx / CHUNKS_PER_ROW, part = idx % CHUNKS_PER_ROW;
          *reinterpret_cast<u32x4*>(&s_q[buf][rr * T::LDS_STRIDE + part * 16]) = pre[c];
        }
      }
      if (tid < 32) s_bias[buf][tid] = pre_bias;
    };

    float red[NT];  // max: running max of the shifted logit / scale; sum: running sum
#pragma unroll
    for (int t = 0; t < NT; ++t) red[t] = SUM ? 0.f : -INFINITY;

    if (t_begin < t_end) {
      load_tile(t_begin);
      store_tile(0);
    }
    __syncthreads();

    for (int64_t t = t_begin; t < t_end; ++t) {
      const int cur = (int)((t - t_begin) & 1);
      if (t + 1 < t_end) load_tile(t + 1);

      // A operands (query rows) and the bias column for this lane's 16 rows
      bf16x8 a[T::STEPS];
      const char* qrow = &s_q[cur][col * T::LDS_STRIDE + half * (D / 2) * 2];
#pragma unroll
      for (int s = 0; s < T::STEPS; ++s) a[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * s));
      f32x16 bias;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&s_bias[cur][8 * q + 4 * half]);
        bias[4 * q + 0] = v.x;
        bias[4 * q + 1] = v.y;
        bias[4 * q + 2] = v.z;
        bias[4 * q + 3] = v.w;
      }

      if (SUM) {
        // rows j = jt + acc_row(r, half); this wave's keys i = wave_key0 + 32*t + col
        const int64_t jt = (jt_first + t % tiles_per_g) * 32;
#pragma unroll
        for (int st = 0; st < NT; ++st) {
          const int64_t ib = wave_key0 + 32 * st;
          if (jt + 31 < ib + p.window) continue;  // every pair still inside the window
          f32x16 acc = bias;
#pragma unroll
          for (int s = 0; s < T::STEPS; ++s) acc = mfma32(a[s], kreg[st][s], acc);
          float sum = 0.f;
          if (jt >= ib + 31 + p.window) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += fast_exp2(acc[r] * c2);
          } else {
            // diagonal band: keep pairs with j - i >= window
            const int64_t base = jt - ib - p.window - col + 4 * half;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = fast_exp2(acc[r] * c2);
              sum += (base + 8 * (r >> 2) + (r & 3) >= 0) ? e : 0.f;
            }
          }
          red[st] += sum;
        }
      } else {
#pragma unroll
        for (int st = 0; st < NT; ++st) {
          f32x16 acc = bias;
#pragma unroll
          for (int s = 0; s < T::STEPS; ++s) acc = mfma32(a[s], kreg[st][s], acc);
          float m = red[st];
#pragma unroll
          for (int r = 0; r < 16; r += 2) m = max3(m, acc[r], acc[r + 1]);
          red[st] = m;
        }
      }

      if (t + 1 < t_end) store_tile(cur ^ 1);
      __syncthreads();
    }

    // ---- combine the two half-waves and write one value per key
#pragma unroll
    for (int st = 0; st < NT; ++st) {
      const float other = __shfl_xor(red[st], 32);
      const float v = SUM ? red[st] + other : fmaxf(red[st], other);
      const int64_t key = wave_key0 + 32 * st + col;
      if (half == 0 && key < p.n_keys) {
        const float vn = p.vnorm ? p.vnorm[(int64_t)h * p.n_keys + key] : 1.0f;
        float* dst = p.out + (int64_t)h * p.n_keys + key;
        if (SUM) {
          *dst = v * vn;
        } else {
          float val = __expf(p.scale * v) * vn;
          if (!(val > 0.f)) val = 0.f;  // -0, NaN -> +0 so the bit pattern orders like the value
          if (p.use_atomic)
            atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(val));
          else
            *dst = val;
        }
      }
    }
    __syncthreads();  // the LDS stage is reused by the next item
  }
}

__global__ void fill_zero(float* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

constexpr int MAX_WAVES = 8, MAX_NT = 2;
constexpr int SUM_WAVES = 8, SUM_NT = 2;

template <int D, int NWAVES, int NT, bool SUM>
hipError_t run(const ScoreParams& p, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((score_kernel<D, NWAVES, NT, SUM>), dim3(nblocks), dim3(NWAVES * WAVE), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_max(const kvs_attn_desc& d, const uint16_t* Q, const uint16_t* K, const float* lse,
                            const float* vnorm, const float* hnorm, float* scores, int accumulate,
                            int num_cus, hipStream_t s) {
  const int64_t n_keys = d.n_ctx;
  if (n_keys == 0) return hipSuccess;
  ScoreParams p{};
  p.Q = Q; p.K = K; p.lse = lse; p.vnorm = vnorm; p.hnorm = hnorm; p.out = scores;
  p.q_hs = d.q_head_stride; p.q_ts = d.q_tok_stride; p.k_hs = d.k_head_stride; p.k_ts = d.k_tok_stride;
  p.n_keys = n_keys; p.n_q = d.n_q; p.window = 0;
  p.Hkv = d.n_kvheads; p.G = d.n_qheads / d.n_kvheads; p.scale = d.scale;
  constexpr int BK = MAX_WAVES * MAX_NT * 32;
  p.n_kblocks = (int)((n_keys + BK - 1) / BK);
  const int64_t base = (int64_t)p.n_kblocks * p.Hkv;
  const int64_t n_tiles = ((int64_t)p.G * d.n_q + 31) / 32;
  // enough workgroups to cover every CU twice; never split below 4 row tiles
  int64_t nsplit = (2 * (int64_t)num_cus + base - 1) / base;
  nsplit = nsplit < 1 ? 1 : nsplit;
  const int64_t max_split = n_tiles / 4 > 1 ? n_tiles / 4 : 1;
  nsplit = nsplit > max_split ? max_split : nsplit;
  p.nsplit = (int)nsplit;
  p.use_atomic = (accumulate || nsplit > 1) ? 1 : 0;
  if (!accumulate && nsplit > 1) {
    const int64_t n = (int64_t)p.Hkv * n_keys;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)), dim3(256), 0,
                       s, scores, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nblocks = (int)(base * nsplit);
  if (d.head_dim == 128) return run<128, MAX_WAVES, MAX_NT, false>(p, nblocks, s);
  return run<64, MAX_WAVES, MAX_NT, false>(p, nblocks, s);
}

hipError_t launch_score_sum(const kvs_attn_desc& d, const uint16_t* Q, const uint16_t* K, const float* lse,
                            int64_t window, const float* vnorm, const float* hnorm, float* target,
                            hipStream_t s) {
  const int64_t T = d.n_ctx;
  if (T == 0) return hipSuccess;
  ScoreParams p{};
  p.Q = Q; p.K = K; p.lse = lse; p.vnorm = vnorm; p.hnorm = hnorm; p.out = target;
  p.q_hs = d.q_head_stride; p.q_ts = d.q_tok_stride; p.k_hs = d.k_head_stride; p.k_ts = d.k_tok_stride;
  p.n_keys = T; p.n_q = T; p.window = window;
  p.Hkv = d.n_kvheads; p.G = d.n_qheads / d.n_kvheads; p.scale = d.scale;
  constexpr int BK = SUM_WAVES * SUM_NT * 32;
  p.n_kblocks = (int)((T + BK - 1) / BK);
  p.nsplit = 1;
  p.use_atomic = 0;
  const int npairs = (p.n_kblocks + 1) / 2;
  const int nblocks = npairs * p.Hkv;
  if (d.head_dim == 128) return run<128, SUM_WAVES, SUM_NT, true>(p, nblocks, s);
  return run<64, SUM_WAVES, SUM_NT, true>(p, nblocks, s);
}

}  // namespace kvs
