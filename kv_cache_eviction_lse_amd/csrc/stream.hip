// Threshold pruning as tokens arrive (decoding). The keep rule of "KVzap:
// Fast, Adaptive, and Faithful KV Cache Pruning" (thresholding with a sliding
// window: keep token t iff score_t >= tau or t >= T - w) re-applied at every
// sequence length T, as the page's phase-agnostic criterion asks of a pruner
// that also runs while decoding: when the token at position p arrives, the
// token at p - w leaves the window and stays only if its score passes.
//
// Cache of one layer, per KV head h a region of C rows:
//   rows [0, w)           window ring: the window token at position p in row p mod w
//   rows [w, w + kept_h)  tokens that left the window with a passing score, ascending
// so the live rows of head h are always rows [0, head_len[h]) of its region,
// head_len[h] = min(n_seen, w) + kept_h.
//
// A call, per head:
//   phase A: the tokens leaving the window in this call (from ring rows, or
//     straight from the new tokens when more than w arrive at once), in
//     position order, TILE at a time: predicate, block scan, then a copy of
//     the kept rows to the end of the kept rows (D/8 lanes per row, UNR rows
//     per thread in flight: a bulk call is bound by load latency otherwise);
//   phase B (once every ring row has been read): the new tokens that end in
//     the window are written to their ring rows, and head_len.
// A decoding step runs both phases in one workgroup per head. A bulk call
// (more than CHUNK leaving tokens) splits phase A over workgroups of CHUNK
// leaving tokens, each counting the kept tokens before its chunk from the
// scores, then runs phase B in a second launch.
#include "common.hpp"
#include "internal.hpp"

namespace kvs {
namespace {

constexpr int ST_THREADS = 512;
constexpr int TILE = ST_THREADS;  // leaving tokens decided per pass
constexpr int UNR = 4;            // rows per thread in flight in a copy
constexpr int CHUNK = 1024;       // leaving tokens per workgroup in a bulk call

struct StreamParams {
  const float* new_scores;
  const uint16_t* K_new;
  const uint16_t* V_new;
  uint16_t* K_cache;
  uint16_t* V_cache;
  int32_t* pos_cache;
  float* win_scores;
  int64_t* head_len;
  int64_t s_hs, n_hs, n_ts;
  int64_t n_seen, n_new, w, C;
  float tau;
};


// One head's view of a call: the leaving tokens are positions L0 .. L1-1
// (index t = q - L0), taken from ring rows (q < n) or from the new tokens.
template <int D>
struct HeadCall {
  int64_t n, m, w, C, L0, L1, L, kept_old;
  uint16_t* Kc;
  uint16_t* Vc;
  int32_t* pc;
  float* ws;
  const float* sn;
  const uint16_t* Kn;
  const uint16_t* Vn;
  int64_t n_ts;
  int ring0;
  float tau;

  __device__ HeadCall(const StreamParams& p, int h) {
    n = p.n_seen; m = p.n_new; w = p.w; C = p.C;
    L0 = n > w ? n - w : 0;
    L1 = n + m > w ? n + m - w : 0;
    L = L1 - L0;
    // kept rows so far, clamped so that every write stays inside the region
    // (the host checked C >= max(w, n + m))
    kept_old = p.head_len[h] - (n < w ? n : w);
    const int64_t kept_max = min(L0, C - w - L);
    kept_old = kept_old < 0 ? 0 : (kept_old > kept_max ? kept_max : kept_old);
    Kc = p.K_cache + (int64_t)h * C * D;
    Vc = p.V_cache + (int64_t)h * C * D;
    pc = p.pos_cache + (int64_t)h * C;
    ws = p.win_scores + (int64_t)h * w;
    sn = p.new_scores + (int64_t)h * p.s_hs;
    Kn = p.K_new + (int64_t)h * p.n_hs;
    Vn = p.V_new + (int64_t)h * p.n_hs;
    n_ts = p.n_ts;
    ring0 = w > 0 ? (int)(L0 % w) : 0;
    tau = p.tau;
  }
  // Ring row of a leaving ring token without a division per row: the ring
  // tokens that leave in one call are consecutive positions L0 .. n-1, fewer
  // than w, so the slot is (L0 mod w) + (q - L0), less one w at most.
  __device__ int ring_slot(int64_t q) const {
    const int sl = ring0 + (int)(q - L0);
    return sl >= w ? sl - (int)w : sl;
  }
  __device__ bool keeps(int64_t q) const {
    const float s = q < n ? ws[ring_slot(q)] : sn[q - n];
    return s >= tau;  // NaN never passes
  }
  __device__ const uint16_t* row(const uint16_t* ring, const uint16_t* fresh, int64_t q) const {
    return q < n ? ring + (int64_t)ring_slot(q) * D : fresh + (q - n) * n_ts;
  }
};

__device__ int block_sum(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) s_wave[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int k = 0; k < ST_THREADS / WAVE; ++k) t += s_wave[k];
  __syncthreads();
  return t;
}

// Kept tokens among leaving tokens t0 .. t1-1 (block-wide, every thread).
// CU_UNR score loads per thread are issued before any is tested, so a long
// count is not a chain of one load round trip per pass.
constexpr int CU_UNR = 8;
template <int D>
__device__ int64_t count_kept(const HeadCall<D>& c, int64_t t0, int64_t t1, int* s_wave) {
  int k = 0;
  int64_t t = t0 + threadIdx.x;
  for (; t + (CU_UNR - 1) * ST_THREADS < t1; t += CU_UNR * ST_THREADS) {
    bool kk[CU_UNR];
#pragma unroll
    for (int u = 0; u < CU_UNR; ++u) kk[u] = c.keeps(c.L0 + t + u * ST_THREADS);
#pragma unroll
    for (int u = 0; u < CU_UNR; ++u) k += kk[u];
  }
  for (; t < t1; t += ST_THREADS) k += c.keeps(c.L0 + t);
  return block_sum(k, s_wave);
}

// Decide leaving tokens t0 .. t1-1 TILE at a time and append the kept ones at
// kept rows `kept` onwards: positions, then K and V rows (D/8 lanes per row,
// UNR rows per thread in flight). Returns the kept count after them.
template <int D>
__device__ int64_t append_leaving(const HeadCall<D>& c, int64_t t0, int64_t t1, int64_t kept, int* s_wave,
                                  int64_t* s_pos) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int LPR = D / 8;
  constexpr int RPP = ST_THREADS / LPR;
  const int part = tid % LPR, rr = tid / LPR;
  for (int64_t tb = t0; tb < t1; tb += TILE) {
    const int64_t q = c.L0 + tb + tid;
    const bool keep = tb + tid < t1 && c.keeps(q);
    const uint64_t b = __ballot(keep);
    const int rank = __popcll(b & ((1ull << lane) - 1));
    if (lane == 0) s_wave[wave] = __popcll(b);
    __syncthreads();
    int before = 0, cnt = 0;
#pragma unroll
    for (int k = 0; k < ST_THREADS / WAVE; ++k) {
      const int x = s_wave[k];
      if (k < wave) before += x;
      cnt += x;
    }
    if (keep) {
      s_pos[before + rank] = q;
      c.pc[c.w + kept + before + rank] = (int32_t)q;
    }
    __syncthreads();
    for (int r0 = 0; r0 < cnt; r0 += UNR * RPP) {
      u32x4 kb[UNR], vb[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int r = r0 + u * RPP + rr;
        if (r < cnt) {
          const int64_t q2 = s_pos[r];
          kb[u] = ld16(c.row(c.Kc, c.Kn, q2) + 8 * part);
          vb[u] = ld16(c.row(c.Vc, c.Vn, q2) + 8 * part);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int r = r0 + u * RPP + rr;
        if (r < cnt) {
          const int64_t dst = (c.w + kept + r) * D + 8 * part;
          st16(c.Kc + dst, kb[u]);
          st16(c.Vc + dst, vb[u]);
        }
      }
    }
    kept += cnt;
    __syncthreads();  // s_wave and s_pos are reused
  }
  return kept;
}

// The new tokens that end in the window take their ring rows (call only once
// every read of a leaving ring token is done).
template <int D>
__device__ void write_ring(const HeadCall<D>& c) {
  const int tid = threadIdx.x;
  constexpr int LPR = D / 8;
  constexpr int RPP = ST_THREADS / LPR;
  const int part = tid % LPR, rr = tid / LPR;
  const int64_t nw = c.m < c.w ? c.m : c.w;  // new tokens in the window
  const int64_t first = c.n + c.m - nw;     // their first position
  const int slot0 = nw > 0 ? (int)(first % c.w) : 0;
  for (int64_t r0 = 0; r0 < nw; r0 += UNR * RPP) {
    u32x4 kb[UNR], vb[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t r = r0 + u * RPP + rr;
      if (r < nw) {
        const int64_t q = first + r;
        kb[u] = ld16(c.Kn + (q - c.n) * c.n_ts + 8 * part);
        vb[u] = ld16(c.Vn + (q - c.n) * c.n_ts + 8 * part);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t r = r0 + u * RPP + rr;
      if (r < nw) {
        const int64_t q = first + r;
        const int64_t slot = slot0 + r >= c.w ? slot0 + r - c.w : slot0 + r;
        st16(c.Kc + slot * D + 8 * part, kb[u]);
        st16(c.Vc + slot * D + 8 * part, vb[u]);
        if (part == 0) {
          c.ws[slot] = c.sn[q - c.n];
          c.pc[slot] = (int32_t)q;
        }
      }
    }
  }
}

// A call with few leaving tokens (a decoding step): one workgroup per head.
template <int D>
__global__ __launch_bounds__(ST_THREADS) void stream_append_kernel(StreamParams p) {
  __shared__ int s_wave[ST_THREADS / WAVE];
  __shared__ int64_t s_pos[TILE];
  const HeadCall<D> c(p, blockIdx.x);
  const int64_t kept = append_leaving(c, 0, c.L, c.kept_old, s_wave, s_pos);
  __syncthreads();  // every ring read (and every read of head_len) is done
  write_ring(c);
  if (threadIdx.x == 0) p.head_len[blockIdx.x] = (c.n + c.m < c.w ? c.n + c.m : c.w) + kept;
}

// A bulk call (more than CHUNK leaving tokens, window at most CHUNK): one
// workgroup per (head, chunk of CHUNK leaving tokens). Each block counts the
// kept tokens before its chunk itself (scores only, from L2), so no block
// waits for another; stream_finish_kernel then writes the ring and head_len.
template <int D>
__global__ __launch_bounds__(ST_THREADS) void stream_bulk_kernel(StreamParams p) {
  __shared__ int s_wave[ST_THREADS / WAVE];
  __shared__ int64_t s_pos[TILE];
  const HeadCall<D> c(p, blockIdx.x);
  const int64_t t0 = (int64_t)blockIdx.y * CHUNK;
  const int64_t t1 = min(c.L, t0 + CHUNK);
  const int64_t before = count_kept(c, 0, t0, s_wave);
  append_leaving(c, t0, t1, c.kept_old + before, s_wave, s_pos);
}

template <int D>
__global__ __launch_bounds__(ST_THREADS) void stream_finish_kernel(StreamParams p) {
  __shared__ int s_wave[ST_THREADS / WAVE];
  const HeadCall<D> c(p, blockIdx.x);
  const int64_t total = count_kept(c, 0, c.L, s_wave);  // (ends with a barrier: ring scores read)
  write_ring(c);
  if (threadIdx.x == 0) p.head_len[blockIdx.x] = (c.n + c.m < c.w ? c.n + c.m : c.w) + c.kept_old + total;
}

}  // namespace

hipError_t launch_stream_append(const kvs_stream_desc& d, const float* new_scores, const uint16_t* K_new,
                                const uint16_t* V_new, uint16_t* K_cache, uint16_t* V_cache, int32_t* pos_cache,
                                float* win_scores, int64_t* head_len, hipStream_t s) {
  if (d.n_new == 0) return hipSuccess;
  StreamParams p{};
  p.new_scores = new_scores; p.K_new = K_new; p.V_new = V_new;
  p.K_cache = K_cache; p.V_cache = V_cache; p.pos_cache = pos_cache;
  p.win_scores = win_scores; p.head_len = head_len;
  p.s_hs = d.score_head_stride; p.n_hs = d.new_head_stride; p.n_ts = d.new_tok_stride;
  p.n_seen = d.n_seen; p.n_new = d.n_new; p.w = d.window; p.C = d.capacity;
  p.tau = d.tau;
  const int64_t L0 = d.n_seen > d.window ? d.n_seen - d.window : 0;
  const int64_t L1 = d.n_seen + d.n_new > d.window ? d.n_seen + d.n_new - d.window : 0;
  const int64_t L = L1 - L0;
  if (L > CHUNK && d.window <= CHUNK) {
    // (ring tokens leave only in the first chunk: L0 .. n_seen-1 is fewer than w <= CHUNK tokens)
    const dim3 grid((unsigned)d.n_kvheads, (unsigned)((L + CHUNK - 1) / CHUNK));
    if (d.head_dim == 128) {
      hipLaunchKernelGGL(stream_bulk_kernel<128>, grid, dim3(ST_THREADS), 0, s, p);
      hipLaunchKernelGGL(stream_finish_kernel<128>, dim3(d.n_kvheads), dim3(ST_THREADS), 0, s, p);
    } else {
      hipLaunchKernelGGL(stream_bulk_kernel<64>, grid, dim3(ST_THREADS), 0, s, p);
      hipLaunchKernelGGL(stream_finish_kernel<64>, dim3(d.n_kvheads), dim3(ST_THREADS), 0, s, p);
    }
    return hipGetLastError();
  }
  if (d.head_dim == 128)
    hipLaunchKernelGGL(stream_append_kernel<128>, dim3(d.n_kvheads), dim3(ST_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(stream_append_kernel<64>, dim3(d.n_kvheads), dim3(ST_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvs
