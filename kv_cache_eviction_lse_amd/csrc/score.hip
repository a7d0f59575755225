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
//   * a workgroup owns BK = NW * NT * 32 consecutive keys of one KV head;
//     each wave keeps its NT*32 keys in VGPRs as MFMA B operands for the whole
//     kernel (the key tile never leaves the chip);
//   * the group's query rows stream past in tiles of TR rows through a
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
#include <cmath>

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
  int nsplit;      // query-row splits per key block (max) or per key-block pair (sum, at most 2)
  int use_atomic;  // combine splits: atomicMax on the score bits (max), atomicAdd (sum)
  float scale;
};

template <int D, int TR>
struct QTile {
  static constexpr int STEPS = D / 16;               // k-steps of 16 per MFMA chain
  static constexpr int LDS_STRIDE = D * 2 + 16;      // pad: 16 consecutive rows hit distinct banks
  static constexpr int CHUNKS = TR * D / 8;          // 16-byte pieces per tile
  static constexpr int CHUNKS_PER_ROW = D / 8;
  static constexpr int BYTES = TR * LDS_STRIDE;
};

// NW waves per workgroup, NT key subtiles (of 32) per wave, RT row subtiles
// (of 32) per streamed query tile.
template <int D, int NW, int NT, int RT, bool SUM>
__global__ __launch_bounds__(NW * WAVE) void score_kernel(ScoreParams p) {
  constexpr int TR = RT * 32;
  using T = QTile<D, TR>;
  constexpr int NTHREADS = NW * WAVE;
  constexpr int BK = NW * NT * 32;
  static_assert(T::CHUNKS % NTHREADS == 0, "tile chunks must split evenly over the threads");
  constexpr int CPT = T::CHUNKS / NTHREADS;

  __shared__ __attribute__((aligned(16))) char s_q[2][T::BYTES];
  __shared__ __attribute__((aligned(16))) float s_bias[2][TR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int half = lane >> 5;
  const int col = lane & 31;

  const int b = blockIdx.x;
  const int h = b % p.Hkv;
  const int rest = b / p.Hkv;
  const float inv_scale = 1.0f / p.scale;
  const float c2 = p.scale * LOG2E;
  const int n_q = (int)p.n_q;

  // work items: max mode -> one key block and one query split;
  // sum mode -> a pair of key blocks (kb, n_kblocks-1-kb), balancing the
  // triangle, and one query split of each.
  int kb_list[2];
  int n_items = 1;
  int split = 0;
  if (SUM) {
    const int npairs = (p.n_kblocks + 1) / 2;
    const int pair = rest % npairs;
    split = rest / npairs;
    kb_list[0] = pair;
    kb_list[1] = p.n_kblocks - 1 - pair;
    n_items = (kb_list[1] != kb_list[0]) ? 2 : 1;
  } else {
    kb_list[0] = rest % p.n_kblocks;
    split = rest / p.n_kblocks;
  }

  // this thread's byte offsets within a query tile (rows of q_ts elements)
  int voff[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = tid + c * NTHREADS;
    const int rr = idx / T::CHUNKS_PER_ROW, part = idx % T::CHUNKS_PER_ROW;
    voff[c] = (int)(rr * p.q_ts * 2 + part * 16);
  }

  for (int item = 0; item < n_items; ++item) {
    const int kb = kb_list[item];
    const int64_t key0 = (int64_t)kb * BK;
    const int64_t wave_key0 = key0 + (int64_t)wave * NT * 32;

    // ---- resident keys: B operands (col = key, k-range per half, permuted D).
    // Keys past the end load the last key instead; their results are never written.
    bf16x8 kreg[NT][T::STEPS];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      int64_t key = wave_key0 + 32 * t + col;
      key = key < p.n_keys ? key : p.n_keys - 1;
      const uint16_t* kp = p.K + (int64_t)h * p.k_hs + key * p.k_ts + half * (D / 2);
#pragma unroll
      for (int s = 0; s < T::STEPS; ++s) {
        u32x4 v = ld16(kp + 8 * s);
        pin(v);
        kreg[t][s] = as_bf16x8(v);
      }
    }

    // ---- the query tiles this item visits: (group head gl, row tile jt),
    // head-major. Rows of tile jt are jt*TR .. jt*TR+TR-1 of that head.
    //   max: every row tile of every group head, split s takes an even share;
    //   sum: per group head, the row tiles from the first row any key of the
    //        block can count (j >= key0 + window) to the end.
    // Split s of nsplit takes an even share of that list.
    const int n_jt_all = (n_q + TR - 1) / TR;
    int jt_start = 0;
    const int jt_end = n_jt_all;
    if (SUM) {
      const int64_t j_lo = key0 + p.window;
      jt_start = j_lo < p.n_q ? (int)(j_lo / TR) : n_jt_all;
    }
    const int n_jt = jt_end - jt_start;
    const int total = n_jt * p.G;
    const int t0 = (int)((int64_t)total * split / p.nsplit);
    const int t1 = (int)((int64_t)total * (split + 1) / p.nsplit);
    const int t_count = t1 - t0;
    int gl = n_jt ? t0 / n_jt : 0;
    int jt = jt_start + (n_jt ? t0 - gl * n_jt : 0);

    // Prefetch registers: raw Q pieces, and for the first TR threads the raw
    // lse and hnorm of one row. A tile is read through buffer resources that
    // start at its first row and cover only the rows that exist, so rows past
    // the end read as zero and a thread's byte offsets are fixed (token
    // strides are at most 2^22 elements: a 128-row tile spans at most 2^30 bytes).
    // Loads are unconditional and the bias arithmetic waits until the store,
    // so issuing a prefetch never stalls the wave. Rows past the end get bias
    // -inf: they never win a max and add exp2(-inf) = 0 to a sum.
    u32x4 pre[CPT];
    float pre_lse = 0.f, pre_hn = 1.f;
    bool pre_ok = false;
    auto load_tile = [&](int tgl, int tjt) {
      const int g = h * p.G + tgl;
      const int j0 = tjt * TR;
      const int rows = min(n_q - j0, TR);
      const __amdgpu_buffer_rsrc_t rq =
          tile_rsrc(p.Q + (int64_t)g * p.q_hs + (int64_t)j0 * p.q_ts, rows * (int)p.q_ts * 2);
#pragma unroll
      for (int c = 0; c < CPT; ++c) pre[c] = buf_ld16(rq, voff[c]);
      if (tid < TR) {
        pre_ok = tid < rows;
        const __amdgpu_buffer_rsrc_t rl = tile_rsrc(p.lse + (int64_t)g * p.n_q + j0, rows * 4);
        pre_lse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, tid * 4, 0, 0));
        if (p.hnorm) {
          const __amdgpu_buffer_rsrc_t rh = tile_rsrc(p.hnorm + j0, rows * 4);
          pre_hn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rh, tid * 4, 0, 0));
        }
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + c * NTHREADS;
        const int rr = idx / T::CHUNKS_PER_ROW, part = idx % T::CHUNKS_PER_ROW;
        *reinterpret_cast<u32x4*>(&s_q[buf][rr * T::LDS_STRIDE + part * 16]) = pre[c];
      }
      if (tid < TR) s_bias[buf][tid] = pre_ok ? -(pre_lse + __logf(pre_hn)) * inv_scale : -INFINITY;
    };
    auto advance = [&](int& tgl, int& tjt) {
      if (++tjt == jt_end) {
        tjt = jt_start;
        ++tgl;
      }
    };

    float red[NT];  // max: running max of the shifted logit / scale; sum: running sum
#pragma unroll
    for (int t = 0; t < NT; ++t) red[t] = SUM ? 0.f : -INFINITY;

    if (t_count > 0) {
      load_tile(gl, jt);
      store_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < t_count; ++t) {
      const int cur = t & 1;
      const int cur_jt = jt;
      int ngl = gl, njt = jt;
      advance(ngl, njt);
      if (t + 1 < t_count) load_tile(ngl, njt);

#pragma unroll
      for (int rs = 0; rs < RT; ++rs) {
        // keep each row subtile's operands to itself (bounds register pressure)
        if (rs) __builtin_amdgcn_sched_barrier(0);
        // A operands (query rows rs*32 + col) and the bias of this lane's 16 rows
        bf16x8 a[T::STEPS];
        const char* qrow = &s_q[cur][(rs * 32 + col) * T::LDS_STRIDE + half * D];
#pragma unroll
        for (int s = 0; s < T::STEPS; ++s) a[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * s));
        f32x16 bias;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(&s_bias[cur][rs * 32 + 8 * q + 4 * half]);
          bias[4 * q + 0] = v.x;
          bias[4 * q + 1] = v.y;
          bias[4 * q + 2] = v.z;
          bias[4 * q + 3] = v.w;
        }

        if (SUM) {
          // rows j = jt0 + acc_row(r, half); this wave's keys i = wave_key0 + 32*st + col
          const int64_t jt0 = (int64_t)cur_jt * TR + 32 * rs;
#pragma unroll
          for (int st = 0; st < NT; ++st) {
            const int64_t ib = wave_key0 + 32 * st;
            if (jt0 + 31 < ib + p.window) continue;  // every pair still inside the window
            f32x16 acc = bias;
#pragma unroll
            for (int s = 0; s < T::STEPS; ++s) acc = mfma32(a[s], kreg[st][s], acc);
            // the exponentials at raised wave priority (as in the LSE pass)
            __builtin_amdgcn_s_setprio(1);
            float sum = 0.f;
            if (jt0 >= ib + 31 + p.window) {
#pragma unroll
              for (int r = 0; r < 16; ++r) sum += fast_exp2(acc[r] * c2);
            } else {
              // diagonal band: keep pairs with j - i >= window
              const int base = (int)(jt0 - ib - p.window) - col + 4 * half;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(acc[r] * c2);
                sum += (base + 8 * (r >> 2) + (r & 3) >= 0) ? e : 0.f;
              }
            }
            red[st] += sum;
            __builtin_amdgcn_s_setprio(0);
          }
        } else {
#pragma unroll
          for (int st = 0; st < NT; ++st) {
            // two accumulator chains in flight at a time
            if (st && (st & 1) == 0) __builtin_amdgcn_sched_barrier(0);
            f32x16 acc = bias;
#pragma unroll
            for (int s = 0; s < T::STEPS; ++s) acc = mfma32(a[s], kreg[st][s], acc);
            float m = red[st];
#pragma unroll
            for (int r = 0; r < 16; r += 2) m = max3(m, acc[r], acc[r + 1]);
            red[st] = m;
          }
        }
      }

      if (t + 1 < t_count) store_tile(cur ^ 1);
      __syncthreads();
      gl = ngl;
      jt = njt;
    }

    // ---- combine the two half-waves and write one value per key. The lane
    // index is taken afresh here, so no per-lane key index computed before the
    // loop has to stay in registers across it.
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
    for (int st = 0; st < NT; ++st) {
      const float other = __shfl_xor(red[st], 32);
      const float v = SUM ? red[st] + other : fmaxf(red[st], other);
      const int64_t key = wave_key0 + 32 * st + (lane_e & 31);
      if (lane_e < 32 && key < p.n_keys) {
        const float vn = p.vnorm ? p.vnorm[(int64_t)h * p.n_keys + key] : 1.0f;
        float* dst = p.out + (int64_t)h * p.n_keys + key;
        if (SUM) {
          // two splits at most: (0 + x) + y == (0 + y) + x, so the sum is deterministic
          if (p.use_atomic)
            atomicAdd(dst, v * vn);
          else
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

// max mode: 8 waves x 2 key subtiles = 512 keys per workgroup, 128-row query
// tiles. Long contexts (at least LONG_ROUNDS rounds of workgroups of the
// long form): 8 waves x 3 key subtiles = 768 keys per workgroup and 64-row
// query tiles (the extra resident keys leave room for 64 rows only), so each
// query row read from LDS feeds 3 MFMA chains instead of 2. Measured: the
// 120k layer's pass 102.6-102.9 ms against 107.5-108.4 ms; on the 32k layer
// 344 workgroups of 768 keys leave a ragged last round, and the two forms
// measure within 1 % of each other there.
constexpr int MAX_NW = 8, MAX_NT = 2, MAX_RT = 4;
constexpr int LONG_NT = 3, LONG_RT = 2;
constexpr int LONG_ROUNDS = 4;
// sum mode: 8 waves x 2 key subtiles = 512 keys per workgroup, 64-row query tiles
constexpr int SUM_NW = 8, SUM_NT = 2, SUM_RT = 4;

template <int D, int NW, int NT, int RT, bool SUM>
hipError_t run(const ScoreParams& p, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((score_kernel<D, NW, NT, RT, SUM>), dim3(nblocks), dim3(NW * WAVE), 0, s, p);
  return hipGetLastError();
}

// Query-row splits per key block: enough workgroups to fill every CU twice
// when there are few key blocks; otherwise the split (1..4) whose last round
// of workgroups is fullest.
int choose_splits(int64_t base, int64_t n_tiles, int num_cus) {
  const int64_t max_split = n_tiles / 2 > 1 ? n_tiles / 2 : 1;
  if (base < num_cus) {
    int64_t ns = (2 * (int64_t)num_cus + base - 1) / base;
    return (int)(ns < max_split ? ns : max_split);
  }
  int best = 1;
  double best_eff = 0.0;
  for (int ns = 1; ns <= 4 && ns <= max_split; ++ns) {
    const double blocks = (double)base * ns;
    const double rounds = std::ceil(blocks / num_cus);
    const double eff = blocks / (rounds * num_cus);
    if (eff > best_eff + 0.02) {
      best_eff = eff;
      best = ns;
    }
  }
  return best;
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
  constexpr int BK_LONG = MAX_NW * LONG_NT * 32;
  const bool long_form = ((n_keys + BK_LONG - 1) / BK_LONG) * p.Hkv >= (int64_t)LONG_ROUNDS * num_cus;
  const int BK = MAX_NW * (long_form ? LONG_NT : MAX_NT) * 32;
  const int TR = (long_form ? LONG_RT : MAX_RT) * 32;
  p.n_kblocks = (int)((n_keys + BK - 1) / BK);
  const int64_t base = (int64_t)p.n_kblocks * p.Hkv;
  const int64_t n_tiles = (int64_t)p.G * ((d.n_q + TR - 1) / TR);
  const int nsplit = choose_splits(base, n_tiles, num_cus);
  p.nsplit = nsplit;
  p.use_atomic = (accumulate || nsplit > 1) ? 1 : 0;
  if (!accumulate && nsplit > 1) {
    const int64_t n = (int64_t)p.Hkv * n_keys;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)), dim3(256), 0,
                       s, scores, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nblocks = (int)(base * nsplit);
  if (long_form) {
    if (d.head_dim == 128) return run<128, MAX_NW, LONG_NT, LONG_RT, false>(p, nblocks, s);
    return run<64, MAX_NW, LONG_NT, LONG_RT, false>(p, nblocks, s);
  }
  if (d.head_dim == 128) return run<128, MAX_NW, MAX_NT, MAX_RT, false>(p, nblocks, s);
  return run<64, MAX_NW, MAX_NT, MAX_RT, false>(p, nblocks, s);
}

hipError_t launch_score_sum(const kvs_attn_desc& d, const uint16_t* Q, const uint16_t* K, const float* lse,
                            int64_t window, const float* vnorm, const float* hnorm, float* target,
                            int num_cus, hipStream_t s) {
  const int64_t T = d.n_ctx;
  if (T == 0) return hipSuccess;
  ScoreParams p{};
  p.Q = Q; p.K = K; p.lse = lse; p.vnorm = vnorm; p.hnorm = hnorm; p.out = target;
  p.q_hs = d.q_head_stride; p.q_ts = d.q_tok_stride; p.k_hs = d.k_head_stride; p.k_ts = d.k_tok_stride;
  // Keys with i + window >= T get 0 whatever the window, so a window past T
  // is the same as T; clamping keeps key0 + window (the first row a key block
  // counts) from overflowing for sentinel windows near INT64_MAX.
  p.n_keys = T; p.n_q = T; p.window = window < T ? window : T;
  p.Hkv = d.n_kvheads; p.G = d.n_qheads / d.n_kvheads; p.scale = d.scale;
  constexpr int BK = SUM_NW * SUM_NT * 32;
  p.n_kblocks = (int)((T + BK - 1) / BK);
  const int npairs = (p.n_kblocks + 1) / 2;
  // Fewer key-block pairs than CUs: split each pair's query rows in two and
  // add the halves atomically into a zeroed target. Two addends onto zero
  // round the same in either order, which keeps the result deterministic;
  // more splits would not.
  p.nsplit = ((int64_t)npairs * p.Hkv < num_cus && d.n_q >= 2 * SUM_RT * 32) ? 2 : 1;
  p.use_atomic = p.nsplit > 1;
  if (p.use_atomic) {
    const int64_t n = (int64_t)p.Hkv * T;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)), dim3(256), 0,
                       s, target, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nblocks = npairs * p.Hkv * p.nsplit;
  if (d.head_dim == 128) return run<128, SUM_NW, SUM_NT, SUM_RT, true>(p, nblocks, s);
  return run<64, SUM_NW, SUM_NT, SUM_RT, true>(p, nblocks, s);
}

}  // namespace kvs
