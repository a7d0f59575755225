// Decode attention over the compacted per-head cache that kv_evict writes:
// query head g (KV head h = g / G) attends to rows head_offsets[h] ..
// head_offsets[h+1]-1 of K_cache / V_cache ([rows, D], head after head, as
// Algorithm 1 of "KVzap: Fast, Adaptive, and Faithful KV Cache Pruning"
// returns keys[indices], values[indices]). Every KV head keeps its own number
// of rows; the pages name that non-uniform cache as what a variable-length
// kernel has to serve before pruning saves time or memory ("Limitation 3",
// FAQ "Q4"). Output: o_j = sum_r a_jr v_r and LSE_j per decode query.
//
// The work is HBM-bound (each kept K and V row is read once per call), so it
// is split by rows, flash-decoding style:
//   * decode_partial: a wave owns a chunk of WR consecutive rows of one
//     head and 4 or 8 of the head's query vectors (G heads x n_q tokens;
//     4 when the head has at most 4). A row is read by D/8 lanes, 16 bytes
//     each (coalesced); 32 rows at a time are staged in LDS and multiplied
//     with the queries on the matrix cores (S = K Q^T, 32 keys x 32 query
//     columns, of which the wave's queries are used); the scores go to
//     LDS. The chunk max and p = exp2(s - m) are then
//     computed once per (row, query) in LDS, with l = sum p; the value rows
//     are read and o += p v in fp32 (the lanes of a row own 8 dimensions
//     each). The row groups of a wave are added with shuffles and the wave
//     writes one partial (m, l, o) per query to the workspace.
//   * decode_combine: one workgroup per decode query and slice of 16 output
//     dimensions merges its head's partials (one chunk per thread at a time,
//     then a block reduction of the max and the rescaled sums, in a fixed
//     order) and writes that slice of O (bf16), and the LSE.
//   Scores are kept in the exp2 domain (scaled by scale * log2 e after the product).
//   Offsets are clamped to [0, capacity] and made monotone, so no offset
//   can send a read outside the cache. With a head stride S (the per-head
//   regions of the streaming cache) head h's rows are [h*S, h*S + len_h),
//   len_h clamped to [0, S]. Both kernels find their heads' rows with one
//   offset load per lane, 64 heads at a time.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace kvs {
namespace {

constexpr int DC_WAVES = 4;
constexpr int DC_THREADS = DC_WAVES * WAVE;
// Rows per wave chunk: the longest of 128, 64 and 32 that still gives at
// least WAVES_WANTED chunks for a cache of `capacity` rows (about 1.5 waves
// per SIMD). Longer chunks mean fewer partials to merge and fewer waves
// paying the per-wave start-up; enough waves keep the rows in flight.
// Measured with the scores on the matrix cores (us, 4 / 8 queries per
// wave): 244,110 rows 31.4 with 128-row chunks, 35.0 with 64, 42.1 with 32;
// 241,024 rows (8 queries) 36.0 / 44.4 / 51.8; 65,536 rows 24.7 / 20.5 /
// 20.4 (8 queries: 29.5 / 23.4 / 22.7); 16,752 rows 24.5 / 20.7 / 20.7.
constexpr int64_t WAVES_WANTED = 1536;
constexpr int queries_per_wave(int G, int n_q) { return G * n_q <= 4 ? 4 : 8; }
constexpr int wrows_for(int64_t capacity) {
  return capacity >= 128 * WAVES_WANTED ? 128 : (capacity >= 64 * WAVES_WANTED ? 64 : 32);
}

// Orders this wave's LDS writes before its later LDS reads by other lanes:
// wait until the wave's LDS operations have completed (lgkmcnt 0), and keep
// the compiler from moving LDS accesses across the point. Each wave of
// decode_partial works in an LDS area of its own, so no workgroup barrier is
// needed (and none would be safe where the waves' loop counts differ).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt and expcnt unconstrained, lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Floats per partial record: m, l, two pad words, then o[D] at a 16-byte offset.
constexpr int REC(int D) { return D + 4; }

struct DecParams {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const int64_t* offs;
  uint16_t* O;
  float* lse;
  float* part;  // [n_wchunks_max][G * n_q][REC(D)]: m, l, two pad words, o (16-byte aligned)
  int64_t q_hs, q_ts;
  int64_t capacity;
  int64_t S;  // head stride in rows (strided heads), 0 for offsets
  int wr;     // rows per wave chunk
  int Hkv, G, n_q, nqg, n_wc_max;
  float c2;  // scale * log2 e
};

// Row ranges and chunk numbering of the heads, 64 heads at a time across the
// lanes of a wave (every lane loads one head's offset at once, instead of a
// chain of dependent loads per head). Lane l describes head k0 + l: its rows
// [lo, hi) and its chunks [c0, c0 + nc) in the global chunk numbering.
// Offsets are clamped to [0, capacity] and made non-decreasing (a running
// max), so no offset can send a read outside the cache; with a head stride S
// head k's rows are [k*S, k*S + len_k), len_k clamped to [0, S]. `carry` is
// the running max so far (start: head 0's clamped first offset) and `cum` the
// chunks of the heads before k0; both are advanced past the 64 heads.
struct HeadLane {
  int64_t lo, hi;
  int c0, nc;
};

__device__ __forceinline__ int64_t clamp_to(int64_t v, int64_t hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

__device__ __forceinline__ HeadLane head_lanes(const DecParams& p, int k0, int64_t& carry, int& cum) {
  const int lane = threadIdx.x & 63;
  const int k = k0 + lane;
  const bool valid = k < p.Hkv;
  HeadLane r;
  if (p.S > 0) {
    r.lo = (int64_t)k * p.S;
    r.hi = r.lo + (valid ? clamp_to(p.offs[k], p.S) : 0);
  } else {
    int64_t e = valid ? clamp_to(p.offs[k + 1], p.capacity) : 0;  // this head's end before the running max
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(e, o);
      if (lane >= o) e = e > y ? e : y;
    }
    r.hi = e > carry ? e : carry;
    const int64_t prev = __shfl_up(r.hi, 1);
    r.lo = lane == 0 ? carry : prev;
  }
  r.nc = valid ? (int)((r.hi - r.lo + p.wr - 1) / p.wr) : 0;
  int incl = r.nc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  r.c0 = cum + incl - r.nc;
  cum += __shfl(incl, 63);
  carry = __shfl(r.hi, 63);
  return r;
}

__device__ __forceinline__ int64_t first_offset(const DecParams& p) {
  return p.S > 0 ? 0 : clamp_to(p.offs[0], p.capacity);
}

// Head and rows of global wave chunk wc (wave-uniform; all lanes call it);
// false past the last chunk.
__device__ bool find_chunk(const DecParams& p, int wc, int& h, int64_t& r0, int64_t& r1) {
  int64_t carry = first_offset(p);
  int cum = 0;
  for (int k0 = 0; k0 < p.Hkv; k0 += WAVE) {
    const HeadLane r = head_lanes(p, k0, carry, cum);
    const uint64_t hit = __ballot(k0 + (int)(threadIdx.x & 63) < p.Hkv && wc >= r.c0 && wc < r.c0 + r.nc);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      h = k0 + src;
      const int64_t lo = __shfl(r.lo, src), hi = __shfl(r.hi, src);
      r0 = lo + (int64_t)(wc - __shfl(r.c0, src)) * p.wr;
      r1 = min(r0 + p.wr, hi);
      return true;
    }
  }
  return false;
}

// Chunks [wc0, wc0 + nwc) of head h (wave-uniform; all lanes call it).
__device__ void head_chunks(const DecParams& p, int h, int& wc0, int& nwc) {
  int64_t carry = first_offset(p);
  int cum = 0;
  for (int k0 = 0; k0 <= h; k0 += WAVE) {
    const HeadLane r = head_lanes(p, k0, carry, cum);
    if (h < k0 + WAVE) {
      wc0 = __shfl(r.c0, h - k0);
      nwc = __shfl(r.nc, h - k0);
      return;
    }
  }
}

template <int D, int QG, int WR>
__global__ __launch_bounds__(DC_THREADS) void decode_partial(DecParams p) {
  constexpr int LPR = D / 8;            // lanes per row
  constexpr int GPW = WAVE / LPR;       // row groups per wave
  constexpr int UNROLL = 8;             // value rows per group in flight per batch
  constexpr int BATCH = 32;             // key rows per batch: one MFMA row block
  constexpr int KUNROLL = BATCH / GPW;  // key rows per group per batch
  constexpr int LPQ = WAVE / QG;        // lanes per query in the softmax phase
  constexpr int STEPS = D / 16;         // k-steps of the score MFMA chain
  constexpr int KSTRIDE = D * 2 + 16;   // padded rows of the key staging area, bytes
  static_assert(KUNROLL * GPW == BATCH, "whole row groups per key batch");
  __shared__ __attribute__((aligned(16))) float s_score[DC_WAVES][WR][QG];
  __shared__ __attribute__((aligned(16))) char s_k[DC_WAVES][BATCH * KSTRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane % LPR, grp = lane / LPR;
  const int wc = blockIdx.x * DC_WAVES + wave;
  const int qg = blockIdx.y;
  int h = 0;
  int64_t r0 = 0, r1 = 0;
  // waves past the last chunk do no work (nr = 0)
  const bool active = find_chunk(p, wc, h, r0, r1);
  const int nr = active ? (int)(r1 - r0) : 0;
  const int nq_head = p.G * p.n_q;

  // this wave's queries as MFMA B operands: lane l holds query f = qg*QG +
  // (l % 32) (zero when absent, or when l % 32 >= QG), head dimensions in the
  // permuted order [half*D/2 + 8s, +8) of step s (the key rows use the same)
  const int col = lane & 31, half = lane >> 5;
  bf16x8 qb[STEPS];
  {
    const int f = qg * QG + col;
    const bool has = col < QG && f < nq_head;
    const int g = h * p.G + (has ? f / p.n_q : 0), tok = has ? f % p.n_q : 0;
    const uint16_t* qp = p.Q + (int64_t)g * p.q_hs + (int64_t)tok * p.q_ts + half * (D / 2);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      u32x4 w = has ? ld16(qp + 8 * s) : u32x4{};
      qb[s] = as_bf16x8(w);
    }
  }

  // ---- scores, 32 rows per batch: coalesced row loads (D/8 lanes per row,
  // 16 bytes each) are staged in this wave's LDS area, read back as the A
  // operands of S = K_batch Q^T (keys as rows, queries as columns), and each
  // lane's 16 scores (query col, rows acc_row(r, half)) go to s_score,
  // scaled to the exp2 domain. Staging is ordered within the wave (no
  // workgroup barrier: each wave has its own area).
  char* const stage = s_k[wave];
  const uint16_t* Kb = p.K + r0 * D + 8 * li;
  for (int b0 = 0; b0 < nr; b0 += BATCH) {
    u32x4 kv[KUNROLL];
#pragma unroll
    for (int u = 0; u < KUNROLL; ++u) {
      const int rr = b0 + u * GPW + grp;
      kv[u] = rr < nr ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kb + (int64_t)rr * D)) : u32x4{};
    }
#pragma unroll
    for (int u = 0; u < KUNROLL; ++u)
      *reinterpret_cast<u32x4*>(stage + (u * GPW + grp) * KSTRIDE + li * 16) = kv[u];
    wave_lds_sync();
    bf16x8 a[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
      a[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(stage + col * KSTRIDE + half * D + 16 * s));
    f32x16 acc = mfma32(a[0], qb[0], f32x16{});
#pragma unroll
    for (int s = 1; s < STEPS; ++s) acc = mfma32(a[s], qb[s], acc);
    if (col < QG) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = b0 + acc_row(r, half);
        if (rr < nr) s_score[wave][rr][col] = acc[r] * p.c2;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // the first batch of value rows does not depend on the scores: issue it now
  const uint16_t* Vb = p.V + r0 * D + 8 * li;
  u32x4 vpre[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int rr = u * GPW + grp;
    vpre[u] = rr < nr ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vb + (int64_t)rr * D)) : u32x4{};
  }
  wave_lds_sync();  // scores visible to the wave's other lanes

  // ---- softmax of the chunk, once per (row, query): lane handles query
  // lane / LPQ and rows lane % LPQ + LPQ*k; the scores become p = exp2(s - m)
  // in place, and l = sum p
  float m, lsum = 0.f;
  {
    const int t = lane / LPQ, j0 = lane % LPQ;
    float mx = -INFINITY;
    for (int j = j0; j < nr; j += LPQ) mx = fmaxf(mx, s_score[wave][j][t]);
#pragma unroll
    for (int msk = 1; msk < LPQ; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk));
    m = mx;
    for (int j = j0; j < nr; j += LPQ) {
      const float pr = fast_exp2(s_score[wave][j][t] - mx);
      s_score[wave][j][t] = pr;
      lsum += pr;
    }
#pragma unroll
    for (int msk = 1; msk < LPQ; msk <<= 1) lsum += __shfl_xor(lsum, msk);
  }
  wave_lds_sync();  // probabilities visible
  float mq[QG], l[QG];
#pragma unroll
  for (int t = 0; t < QG; ++t) {
    mq[t] = __shfl(m, LPQ * t);
    l[t] = __shfl(lsum, LPQ * t);
  }

  // ---- values: o[t][e] += exp2(s - m) * v for this lane's 8 dimensions
  float o[QG][8];
#pragma unroll
  for (int t = 0; t < QG; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[t][e] = 0.f;
  for (int k0 = 0; k0 * GPW < nr; k0 += UNROLL) {
    u32x4 vv[UNROLL];
    if (k0 == 0) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) vv[u] = vpre[u];
    } else {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int rr = (k0 + u) * GPW + grp;
        vv[u] = rr < nr ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vb + (int64_t)rr * D)) : u32x4{};
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int rr = (k0 + u) * GPW + grp;
      if (rr < nr) {
        float vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[2 * e] = __uint_as_float(vv[u][e] << 16);
          vf[2 * e + 1] = __uint_as_float(vv[u][e] & 0xffff0000u);
        }
        float pr[QG];
#pragma unroll
        for (int t4 = 0; t4 < QG; t4 += 4) {
          const float4 pa = *reinterpret_cast<const float4*>(&s_score[wave][rr][t4]);
          pr[t4] = pa.x;
          pr[t4 + 1] = pa.y;
          pr[t4 + 2] = pa.z;
          pr[t4 + 3] = pa.w;
        }
#pragma unroll
        for (int t = 0; t < QG; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[t][e] = __builtin_fmaf(pr[t], vf[e], o[t][e]);
      }
    }
  }

  // ---- add the row groups of the wave (lanes li, li + LPR, ...) and write the partials
#pragma unroll
  for (int msk = LPR; msk < WAVE; msk <<= 1) {
#pragma unroll
    for (int t = 0; t < QG; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[t][e] += __shfl_xor(o[t][e], msk);
  }
  if (active && grp == 0) {
#pragma unroll
    for (int t = 0; t < QG; ++t) {
      const int f = qg * QG + t;
      if (f < nq_head) {
        float* rec = p.part + ((int64_t)wc * nq_head + f) * REC(D);
        if (li == 0) {
          rec[0] = mq[t];
          rec[1] = l[t];
        }
        *reinterpret_cast<float4*>(rec + 4 + 8 * li) = make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
        *reinterpret_cast<float4*>(rec + 8 + 8 * li) = make_float4(o[t][4], o[t][5], o[t][6], o[t][7]);
      }
    }
  }
}

// Merge of a head's partials: one workgroup per (decode query, slice of
// CB_DIMS output dimensions), so a layer's few decode queries still spread
// over many CUs. Thread t takes chunks t, t + CB_THREADS, ... (every load of
// a record issued at once: m, l and the slice of o), merges them online, and
// the block then reduces (max, then rescaled sums of l and the slice) with
// wave shuffles and one LDS step, in a fixed order. Every slice reads the
// records' m and l itself and derives the same maxima and sums, so the
// slices agree on the LSE, which the first writes.
constexpr int CB_THREADS = 256;
constexpr int CB_DIMS = 16;

template <int D>
__global__ __launch_bounds__(CB_THREADS) void decode_combine(DecParams p) {
  static_assert(D % CB_DIMS == 0, "whole slices");
  constexpr int NWV = CB_THREADS / WAVE;
  constexpr int NV = CB_DIMS + 1;  // l, then the slice of o
  __shared__ float s_m[NWV];
  __shared__ float s_v[NWV][NV];
  const int g = blockIdx.x / p.n_q, tok = blockIdx.x % p.n_q;
  const int d0 = blockIdx.y * CB_DIMS;
  const int h = g / p.G;
  const int f = (g % p.G) * p.n_q + tok;
  const int nq_head = p.G * p.n_q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this head's wave chunks: [wc0, wc0 + nwc)
  int wc0 = 0, nwc = 0;
  head_chunks(p, h, wc0, nwc);
  float M = -INFINITY, v[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) v[e] = 0.f;
  for (int c = tid; c < nwc; c += CB_THREADS) {
    const float* rec = p.part + ((int64_t)(wc0 + c) * nq_head + f) * REC(D);
    const float mc = rec[0], lc = rec[1];
    float oc[CB_DIMS];
#pragma unroll
    for (int e = 0; e < CB_DIMS; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(rec + 4 + d0 + e);
      oc[e] = x.x;
      oc[e + 1] = x.y;
      oc[e + 2] = x.z;
      oc[e + 3] = x.w;
    }
    const float Mn = fmaxf(M, mc);
    const float a = fast_exp2(M - Mn), bw = fast_exp2(mc - Mn);  // M = -inf on a thread's first chunk: a = 0
    v[0] = v[0] * a + lc * bw;
#pragma unroll
    for (int e = 0; e < CB_DIMS; ++e) v[e + 1] = v[e + 1] * a + oc[e] * bw;
    M = Mn;
  }
  // block max of the offsets
  float Mt = M;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) Mt = fmaxf(Mt, __shfl_xor(Mt, o));
  if (lane == 0) s_m[wave] = Mt;
  __syncthreads();
  Mt = s_m[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) Mt = fmaxf(Mt, s_m[w]);
  // rescale to Mt (threads with no chunk count 0), then sum over the block
  const float wgt = M == -INFINITY ? 0.f : fast_exp2(M - Mt);
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    float x = v[e] * wgt;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    v[e] = x;
  }
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < NV; ++e) s_v[wave][e] = v[e];
  }
  __syncthreads();
  if (tid < CB_DIMS) {
    float Lt = s_v[0][0], ot = s_v[0][tid + 1];
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
      Lt += s_v[w][0];
      ot += s_v[w][tid + 1];
    }
    uint16_t* orow = p.O + (int64_t)g * p.q_hs + (int64_t)tok * p.q_ts;
    const float out = nwc > 0 ? ot / Lt : 0.f;
    orow[d0 + tid] = __builtin_bit_cast(uint16_t, (__bf16)out);
    if (d0 == 0 && tid == 0) p.lse[(int64_t)g * p.n_q + tok] = nwc > 0 ? (Mt + __log2f(Lt)) * LN2 : -INFINITY;
  }
}

}  // namespace

int wrows_of(const kvs_decode_desc& d) {
  return wrows_for(d.capacity);
}

int64_t decode_wave_chunks_max(const kvs_decode_desc& d) { return d.capacity / wrows_of(d) + d.n_kvheads; }

size_t decode_workspace_bytes(const kvs_decode_desc& d) {
  const int64_t nq_head = (int64_t)(d.n_qheads / d.n_kvheads) * d.n_q;
  return (size_t)decode_wave_chunks_max(d) * (size_t)nq_head * (size_t)REC(d.head_dim) * sizeof(float);
}

template <int D, int QG>
void launch_partial(const DecParams& p, dim3 grid, hipStream_t s) {
  if (p.wr == 128)
    hipLaunchKernelGGL((decode_partial<D, QG, 128>), grid, dim3(DC_THREADS), 0, s, p);
  else if (p.wr == 64)
    hipLaunchKernelGGL((decode_partial<D, QG, 64>), grid, dim3(DC_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL((decode_partial<D, QG, 32>), grid, dim3(DC_THREADS), 0, s, p);
}

hipError_t launch_decode(const kvs_decode_desc& d, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                         const int64_t* offs, uint16_t* O, float* lse, void* workspace, hipStream_t s) {
  DecParams p{};
  p.Q = Q; p.K = K; p.V = V; p.offs = offs; p.O = O; p.lse = lse;
  p.part = static_cast<float*>(workspace);
  p.q_hs = d.q_head_stride; p.q_ts = d.q_tok_stride;
  p.capacity = d.capacity;
  p.S = d.head_stride_rows;
  p.wr = wrows_of(d);
  p.Hkv = d.n_kvheads; p.G = d.n_qheads / d.n_kvheads; p.n_q = d.n_q;
  const int qg = queries_per_wave(p.G, p.n_q);
  p.nqg = (p.G * p.n_q + qg - 1) / qg;
  p.n_wc_max = (int)decode_wave_chunks_max(d);
  p.c2 = d.scale * LOG2E;
  const dim3 grid1((unsigned)((p.n_wc_max + DC_WAVES - 1) / DC_WAVES), (unsigned)p.nqg);
  const dim3 grid2((unsigned)(d.n_qheads * d.n_q), (unsigned)(d.head_dim / CB_DIMS));
  if (d.head_dim == 128) {
    if (qg == 4) launch_partial<128, 4>(p, grid1, s);
    else launch_partial<128, 8>(p, grid1, s);
    hipLaunchKernelGGL(decode_combine<128>, grid2, dim3(CB_THREADS), 0, s, p);
  } else {
    if (qg == 4) launch_partial<64, 4>(p, grid1, s);
    else launch_partial<64, 8>(p, grid1, s);
    hipLaunchKernelGGL(decode_combine<64>, grid2, dim3(CB_THREADS), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvs
