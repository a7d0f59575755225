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
// One workgroup per head:
//   phase A: the tokens leaving the window in this call (from ring rows, or
//     straight from the new tokens when more than w arrive at once), in
//     position order, TILE at a time: predicate, block scan, then a copy of
//     the kept rows to the end of the kept rows (D/8 lanes per row);
//   phase B (after a barrier, so every ring row has been read): the new
//     tokens that end in the window are written to their ring rows.
#include "common.hpp"
#include "internal.hpp"

namespace kvs {
namespace {

constexpr int ST_THREADS = 256;
constexpr int TILE = ST_THREADS;  // leaving tokens decided per pass

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

// 16-byte pieces of one row: lanes part = 0 .. D/8-1
__device__ __forceinline__ void copy_row_part(uint16_t* dst, const uint16_t* src, int part) {
  st16(dst + 8 * part, ld16(src + 8 * part));
}

template <int D>
__global__ __launch_bounds__(ST_THREADS) void stream_append_kernel(StreamParams p) {
  __shared__ int s_wave[ST_THREADS / WAVE];
  __shared__ int64_t s_pos[TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x;
  const int64_t n = p.n_seen, m = p.n_new, w = p.w, C = p.C;
  const int64_t L0 = n > w ? n - w : 0;             // first leaving position
  const int64_t L1 = n + m > w ? n + m - w : 0;     // one past the last
  const int64_t L = L1 - L0;
  // kept rows so far, clamped so that every write stays inside the region
  // (the host checked C >= max(w, n + m))
  int64_t kept = p.head_len[h] - (n < w ? n : w);
  const int64_t kept_max = min(L0, C - w - L);
  kept = kept < 0 ? 0 : (kept > kept_max ? kept_max : kept);

  uint16_t* const Kc = p.K_cache + (int64_t)h * C * D;
  uint16_t* const Vc = p.V_cache + (int64_t)h * C * D;
  int32_t* const pc = p.pos_cache + (int64_t)h * C;
  float* const ws = p.win_scores + (int64_t)h * w;
  const float* const sn = p.new_scores + (int64_t)h * p.s_hs;
  const uint16_t* const Kn = p.K_new + (int64_t)h * p.n_hs;
  const uint16_t* const Vn = p.V_new + (int64_t)h * p.n_hs;
  auto src_row = [&](const uint16_t* ring, const uint16_t* fresh, int64_t q) {
    return q < n ? ring + (q % w) * D : fresh + (q - n) * p.n_ts;
  };

  constexpr int LPR = D / 8;
  constexpr int RPP = ST_THREADS / LPR;
  const int part = tid % LPR, rr = tid / LPR;

  // ---- phase A: decide the leaving tokens, append the kept ones
  for (int64_t t0 = 0; t0 < L; t0 += TILE) {
    const int64_t q = L0 + t0 + tid;
    bool keep = false;
    if (t0 + tid < L) {
      const float s = q < n ? ws[q % w] : sn[q - n];
      keep = s >= p.tau;  // NaN never passes
    }
    const uint64_t b = __ballot(keep);
    const int rank = __popcll(b & ((1ull << lane) - 1));
    if (lane == 0) s_wave[wave] = __popcll(b);
    __syncthreads();
    int before = 0, cnt = 0;
#pragma unroll
    for (int k = 0; k < ST_THREADS / WAVE; ++k) {
      const int c = s_wave[k];
      if (k < wave) before += c;
      cnt += c;
    }
    if (keep) {
      s_pos[before + rank] = q;
      pc[w + kept + before + rank] = (int32_t)q;
    }
    __syncthreads();
    for (int r = rr; r < cnt; r += RPP) {
      const int64_t q2 = s_pos[r];
      const int64_t dst = (w + kept + r) * D;
      copy_row_part(Kc + dst, src_row(Kc, Kn, q2), part);
      copy_row_part(Vc + dst, src_row(Vc, Vn, q2), part);
    }
    kept += cnt;
    __syncthreads();  // s_wave and s_pos are reused; ring rows read before phase B
  }

  // ---- phase B: the new tokens that end in the window take their ring rows
  const int64_t nw = m < w ? m : w;  // new tokens in the window
  const int64_t first = n + m - nw;  // their first position
  for (int64_t r = rr; r < nw; r += RPP) {
    const int64_t q = first + r;
    const int64_t slot = q % w;
    copy_row_part(Kc + slot * D, Kn + (q - n) * p.n_ts, part);
    copy_row_part(Vc + slot * D, Vn + (q - n) * p.n_ts, part);
    if (part == 0) {
      ws[slot] = sn[q - n];
      pc[slot] = (int32_t)q;
    }
  }
  __syncthreads();  // every wave has read head_len (phase A may have had no barrier)
  if (tid == 0) p.head_len[h] = (n + m < w ? n + m : w) + kept;
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
  if (d.head_dim == 128)
    hipLaunchKernelGGL(stream_append_kernel<128>, dim3(d.n_kvheads), dim3(ST_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(stream_append_kernel<64>, dim3(d.n_kvheads), dim3(ST_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvs
