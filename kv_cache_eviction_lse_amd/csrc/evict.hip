// Per-KV-head eviction: keep the window of the last w keys plus the top-k or
// the tau-thresholded other keys, and compact the kept K and V rows.
//
// Selection rules: the protected window and the ">= tau" comparison of the
// thresholding rule and Algorithm 1 of "KVzap: Fast, Adaptive, and Faithful KV
// Cache Pruning"; per-head top-k as in "[논문리뷰] KVpop ..." §3. Kept rows are
// written in ascending position, head after head (Algorithm 1's keys[indices],
// values[indices]).
//
// Kernels:
//   per-head top-k (or keep-all / window-only) with at most HD_MAX
//   candidates per head: evict_head, a few workgroups per head, each of
//   which selects in LDS and then writes and copies its share of the head's
//   kept rows. One launch.
//   per-head top-k with HD_MAX < candidates <= LH_MAX per head, when its
//   workspace fits: evict_lh_hist (first-digit histograms per chunk),
//   evict_lh_bin (the k-th key's first digit, per-segment counts and the
//   digit's keys listed per head), evict_long_head (workgroups per head that
//   finish the selection from the list, write and copy their rows). Three
//   launches; see the long-heads section.
//   Otherwise (thresholds, layer budgets, longer heads), one grid of blocks
//   of 1024 or 2048 keys per head (GRID_SMALL), unless noted:
//   top-k: evict_zero, then three radix-digit histogram passes over the
//     order-preserving 32-bit keys of the candidate scores (bits 31..21,
//     20..10, 9..0). Each pass re-derives, from the previous passes'
//     histograms, the prefix of the k-th largest key, so no separate "find"
//     launch is needed. After the last pass the k-th key T is exact; keys > T
//     are kept, and among keys == T the lowest positions up to the quota.
//   evict_count: per block, rows kept for sure and rows tied at T.
//   evict_scan (one block per head): block offsets and the head's total. With
//     a layer budget the k-th key and the tie quota are the layer's (one
//     histogram for all heads); the scan gives each head its share of the
//     ties, lowest heads first.
//   evict_write: predicate, tie ranks and prefix scan, kept indices; block
//     (0, 0) writes the per-head offsets. Up to FUSED_HEADS heads and
//     FUSED_ENTRIES count entries, evict_write_fused does the scan's work in
//     every block instead (no evict_scan launch).
//   evict_gather (a grid over output rows): coalesced copy of the kept K and
//     V rows, 16-byte pieces, non-temporal loads and stores.
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace kvs {
namespace {

constexpr int EV_THREADS = 256;
// Keys per thread (PER) and per block (EV_THREADS * PER) of the grid kernels:
// 8 (2048-key blocks), or 4 (1024-key blocks) for layers that would have at
// most GRID_SMALL blocks of 2048 keys, where twice the blocks measured faster
// (32k threshold layer 58.0-58.6 -> 56.3-56.5 us); on larger layers the
// write pass's reduction of every (head, block) count grows with the square
// of the blocks (120k layer budget 87 -> 103 us with 1024-key blocks).
constexpr int GRID_SMALL = 256;
__host__ __device__ constexpr int epb_of(int per) { return EV_THREADS * per; }
constexpr int NBINS = 2048;

enum Mode : int { MODE_TOPK = 0, MODE_TAU = 1, MODE_ALL = 2, MODE_WINDOW = 3 };

struct EvictParams {
  const float* scores;
  int64_t s_hs;
  const uint16_t* K;
  const uint16_t* V;
  int64_t kv_hs, kv_ts;
  int32_t* kept_idx;
  int64_t* head_offsets;
  uint16_t* K_out;
  uint16_t* V_out;
  uint32_t* hist;   // [3][Hkv][NBINS]
  int32_t* blk;     // [Hkv][nb][4]: kept-for-sure, tied, offset in head, ties before
  int32_t* state;   // [Hkv][4]: threshold key T (bits), quota
  int64_t n, n_cand, kprime;  // kprime: per head, or for the whole layer when layer != 0
  int Hkv, D, nb, mode;
  int layer;  // top-k over all heads' candidates together (one histogram, one quota)
  float tau;
  int64_t per_head;  // one-workgroup-per-head path: rows per head (known on the host there)
  int32_t rows_q, rows_r;  // per-head paths: workgroup r of a head owns rows_q + (r < rows_r) rows
  int32_t vec4;            // long-head path: scores 16-byte aligned with a head stride divisible by 4
  uint32_t* seg_above;     // long-head path: [Hkv][n_seg] keys above the first digit's bin per segment
  int32_t* lh_state;       // long-head path: [Hkv][4] first digit, rank inside its bin, keys in the bin
  uint2* lh_list;          // long-head path: [Hkv][LH_CAP] (key, position) of the bin's keys
};

// Order-preserving key: a > b as floats <=> key(a) > key(b); -0 and +0 share
// a key; NaN maps below every number.
__device__ __forceinline__ uint32_t order_key(float s) {
  if (s != s) return 0u;
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 1023u : 2047u; }

// Exclusive prefix sum over the block's NT threads (tid order); *total gets the sum.
template <int NT = EV_THREADS>
__device__ int block_exclusive_scan(int v, int* total) {
  __shared__ int s_wave[NT / WAVE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / WAVE; ++w) {
    const int t = s_wave[w];
    if (w < wave) before += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Radix-digit pass `pass` over a finished histogram: the digit (counted from
// the top) that holds the rank-th largest key, and the number of keys in
// the higher digits. Block-wide over NT threads; every thread returns the
// same values.
template <int NT = EV_THREADS>
__device__ void find_digit(const uint32_t* bins, int pass, int rank, int& digit, int& cum_out) {
  __shared__ int s_digit, s_cum;
  const int nbins = pass == 2 ? 1024 : 2048;
  const int per = nbins / NT;  // bins per thread
  const int rt = NT - 1 - (int)threadIdx.x;  // reversed: high digits first
  int mine = 0;
  for (int k = 0; k < per; ++k) mine += (int)bins[rt * per + k];
  int tot;
  const int higher = block_exclusive_scan<NT>(mine, &tot);  // keys in higher digit bins
  if (higher < rank && rank <= higher + mine) {
    int cum = higher;
    for (int k = per - 1; k >= 0; --k) {
      const int c = (int)bins[rt * per + k];
      if (cum + c >= rank) {
        s_digit = rt * per + k;
        s_cum = cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  digit = s_digit;
  cum_out = s_cum;
  __syncthreads();
}

// Walk the finished histogram passes of head h and return the prefix of the
// k-th largest candidate key, the number of candidates above that prefix's
// range, and the rank still to find inside it. Block-wide; every thread
// returns the same values.
__device__ void radix_state(const EvictParams& p, int h, int passes, uint32_t& prefix, int& above, int& rank) {
  prefix = 0;
  above = 0;
  rank = (int)p.kprime;
  for (int pass = 0; pass < passes; ++pass) {
    int digit, cum;
    find_digit(p.hist + ((int64_t)pass * p.Hkv + h) * NBINS, pass, rank, digit, cum);
    prefix |= (uint32_t)digit << digit_shift(pass);
    above += cum;
    rank -= cum;
  }
}

__global__ void evict_zero(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

template <int PASS, int PER>
__global__ __launch_bounds__(EV_THREADS) void evict_hist(EvictParams p) {
  __shared__ uint32_t s_hist[NBINS];
  const int h = blockIdx.y, b = blockIdx.x;
  for (int i = threadIdx.x; i < NBINS; i += EV_THREADS) s_hist[i] = 0u;
  const int hh = p.layer ? 0 : h;  // histogram of this head, or the layer's
  uint32_t prefix = 0;
  int above, rank;
  if (PASS > 0) radix_state(p, hh, PASS, prefix, above, rank);
  __syncthreads();
  const int hs = PASS > 0 ? digit_shift(PASS - 1) : 32;
  const int64_t i0 = (int64_t)b * epb_of(PER) + threadIdx.x * PER;
  const float* sc = p.scores + (int64_t)h * p.s_hs;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int64_t i = i0 + e;
    if (i < p.n_cand) {
      const uint32_t u = order_key(sc[i]);
      if (PASS == 0 || (u >> hs) == (prefix >> hs))
        atomicAdd(&s_hist[(u >> digit_shift(PASS)) & digit_mask(PASS)], 1u);
    }
  }
  __syncthreads();
  uint32_t* g = p.hist + ((int64_t)PASS * p.Hkv + hh) * NBINS;
  for (int i = threadIdx.x; i < NBINS; i += EV_THREADS)
    if (s_hist[i]) atomicAdd(&g[i], s_hist[i]);
}

// keep classes of key i: 2 = kept for sure, 1 = tied at T (top-k), 0 = dropped
__device__ __forceinline__ int keep_class(const EvictParams& p, int64_t i, float s, uint32_t T) {
  if (i >= p.n_cand) return 2;  // protected window
  switch (p.mode) {
    case MODE_TOPK: {
      const uint32_t u = order_key(s);
      return u > T ? 2 : (u == T ? 1 : 0);
    }
    case MODE_TAU: return s >= p.tau ? 2 : 0;
    case MODE_ALL: return 2;
    default: return 0;
  }
}

template <int PER>
__global__ __launch_bounds__(EV_THREADS) void evict_count(EvictParams p) {
  const int h = blockIdx.y, b = blockIdx.x;
  uint32_t T = 0;
  int quota = 0;
  if (p.mode == MODE_TOPK) {
    uint32_t prefix;
    int above, rank;
    radix_state(p, p.layer ? 0 : h, 3, prefix, above, rank);
    T = prefix;
    quota = (int)p.kprime - above;  // ties kept: per head, or for the layer (split by evict_scan)
  }
  if (b == 0 && threadIdx.x == 0) {
    p.state[h * 4 + 0] = (int32_t)T;
    p.state[h * 4 + 1] = quota;
  }
  const int64_t i0 = (int64_t)b * epb_of(PER) + threadIdx.x * PER;
  const float* sc = p.scores + (int64_t)h * p.s_hs;
  int sure = 0, tied = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int64_t i = i0 + e;
    if (i < p.n) {
      const int c = keep_class(p, i, i < p.n_cand ? sc[i] : 0.f, T);
      sure += c == 2;
      tied += c == 1;
    }
  }
  int tot_sure, tot_tied;
  block_exclusive_scan(sure, &tot_sure);
  block_exclusive_scan(tied, &tot_tied);
  if (threadIdx.x == 0) {
    int32_t* e = p.blk + ((int64_t)h * p.nb + b) * 4;
    e[0] = tot_sure;
    e[1] = tot_tied;
  }
}

// One block per head: scan the head's block counts into block offsets (within
// the head) and tie ranks, and store the head's total kept rows.
__global__ __launch_bounds__(EV_THREADS) void evict_scan(EvictParams p) {
  const int h = blockIdx.x;
  int quota = p.mode == MODE_TOPK ? p.state[h * 4 + 1] : 0;
  if (p.mode == MODE_TOPK && p.layer) {
    // The layer's tie quota goes to the lowest heads first: this head keeps
    // what is left after the ties of heads 0 .. h-1, at most its own ties.
    int before = 0, mine = 0;
    for (int i = threadIdx.x; i < (h + 1) * p.nb; i += EV_THREADS) {
      const int t = p.blk[(int64_t)i * 4 + 1];
      if (i < h * p.nb) before += t; else mine += t;
    }
    int tot_before, tot_mine;
    block_exclusive_scan(before, &tot_before);
    block_exclusive_scan(mine, &tot_mine);
    quota = min(max(quota - tot_before, 0), tot_mine);
  }
  int sure_base = 0, tied_base = 0;
  for (int b0 = 0; b0 < p.nb; b0 += EV_THREADS) {
    const int b = b0 + (int)threadIdx.x;
    int32_t* e = p.blk + ((int64_t)h * p.nb + (b < p.nb ? b : 0)) * 4;
    const int sure = b < p.nb ? e[0] : 0;
    const int tied = b < p.nb ? e[1] : 0;
    int ts, tt;
    const int sb = block_exclusive_scan(sure, &ts) + sure_base;
    const int tb = block_exclusive_scan(tied, &tt) + tied_base;
    if (b < p.nb) {
      e[2] = sb + min(tb, quota);
      e[3] = tb;
    }
    sure_base += ts;
    tied_base += tt;
  }
  if (threadIdx.x == 0) {
    p.state[h * 4 + 1] = quota;  // this head's share (evict_write reads it)
    p.state[h * 4 + 2] = sure_base + min(tied_base, quota);
  }
}

// first output row of head h: the totals of the heads before it
__device__ __forceinline__ int64_t head_start(const EvictParams& p, int h) {
  int64_t off = 0;
  for (int k = 0; k < h; ++k) off += p.state[k * 4 + 2];
  return off;
}

// Predicate, tie ranks, positions and the kept indices of one block of keys,
// given the block's first output row and the head's ties before the block.
template <int PER>
__device__ void write_block(const EvictParams& p, int h, int b, uint32_t T, int quota, int64_t out0,
                            int ties_before) {
  const int64_t i0 = (int64_t)b * epb_of(PER) + threadIdx.x * PER;
  const float* sc = p.scores + (int64_t)h * p.s_hs;
  int cls[PER];
  int tied = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int64_t i = i0 + k;
    cls[k] = i < p.n ? keep_class(p, i, i < p.n_cand ? sc[i] : 0.f, T) : 0;
    tied += cls[k] == 1;
  }
  int tot;
  int tie_rank = ties_before + block_exclusive_scan(tied, &tot);
  int keep = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (cls[k] == 1) {
      cls[k] = tie_rank < quota ? 2 : 0;
      ++tie_rank;
    }
    keep += cls[k] == 2;
  }
  int n_keep;
  int pos = block_exclusive_scan(keep, &n_keep);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (cls[k] == 2) p.kept_idx[out0 + pos++] = (int32_t)(i0 + k);
  }
}

// After evict_scan: block offsets and head totals are in the workspace.
// Block (0, 0) also writes the per-head offsets.
template <int PER>
__global__ __launch_bounds__(EV_THREADS) void evict_write(EvictParams p) {
  const int h = blockIdx.y, b = blockIdx.x;
  if (b == 0 && h == 0) {
    for (int k = threadIdx.x; k <= p.Hkv; k += EV_THREADS) p.head_offsets[k] = head_start(p, k);
  }
  if (p.nb == 0) return;  // no keys: only the (zero) offsets
  const int32_t* e = p.blk + ((int64_t)h * p.nb + b) * 4;
  write_block<PER>(p, h, b, (uint32_t)p.state[h * 4 + 0], p.state[h * 4 + 1], head_start(p, h) + e[2], e[3]);
}

// Scan and write in one launch, for layers with at most FUSED_HEADS heads and
// FUSED_ENTRIES (head, block) count entries: every block reduces the count
// entries itself (per-head totals in LDS, its own head's prefix before it),
// derives each head's tie quota (its own, or its share of the layer's, lowest
// heads first) and kept total, and from them its output rows.
constexpr int FUSED_HEADS = 1024;
constexpr int FUSED_ENTRIES = 8192;
constexpr int HPT = FUSED_HEADS / EV_THREADS;  // heads per thread in the head scans

template <int PER>
__global__ __launch_bounds__(EV_THREADS) void evict_write_fused(EvictParams p) {
  __shared__ int s_sure[FUSED_HEADS], s_tied[FUSED_HEADS];
  __shared__ int64_t s_start;
  __shared__ int s_quota;
  const int h = blockIdx.y, b = blockIdx.x;
  const int tid = threadIdx.x;
  for (int k = tid; k < p.Hkv; k += EV_THREADS) s_sure[k] = s_tied[k] = 0;
  __syncthreads();
  int sb = 0, tb = 0;  // this head's counts in blocks before b
  for (int i = tid; i < p.Hkv * p.nb; i += EV_THREADS) {
    const int hh = i / p.nb, bb = i - hh * p.nb;
    const int sure = p.blk[(int64_t)i * 4 + 0], tied = p.blk[(int64_t)i * 4 + 1];
    atomicAdd(&s_sure[hh], sure);
    atomicAdd(&s_tied[hh], tied);
    if (hh == h && bb < b) {
      sb += sure;
      tb += tied;
    }
  }
  int t_sb, t_tb;
  block_exclusive_scan(sb, &t_sb);
  block_exclusive_scan(tb, &t_tb);  // also orders the LDS atomics before the reads below
  // thread t owns heads [t*HPT, t*HPT + HPT): their ties before them, then quotas and totals
  int my_tied = 0;
#pragma unroll
  for (int j = 0; j < HPT; ++j) {
    const int k = tid * HPT + j;
    if (k < p.Hkv) my_tied += s_tied[k];
  }
  int tot_tied;
  int tied_before = block_exclusive_scan(my_tied, &tot_tied);
  const bool topk = p.mode == MODE_TOPK;
  int quota_h = 0, my_total = 0;
  int64_t totals[HPT];
#pragma unroll
  for (int j = 0; j < HPT; ++j) {
    const int k = tid * HPT + j;
    totals[j] = 0;
    if (k < p.Hkv) {
      int q = 0;
      if (topk) {
        q = p.state[k * 4 + 1];
        if (p.layer) q = min(max(q - tied_before, 0), s_tied[k]);
      }
      tied_before += s_tied[k];
      totals[j] = s_sure[k] + min(s_tied[k], q);
      if (k == h) quota_h = q;
      my_total += (int)totals[j];
    }
  }
  int tot_rows;
  const int my_first = block_exclusive_scan(my_total, &tot_rows);  // rows of the heads before this thread's
  // head h's first row and quota (published by the thread that owns head h),
  // and (block (0, 0)) every head's offset
  int64_t start = my_first;
#pragma unroll
  for (int j = 0; j < HPT; ++j) {
    const int k = tid * HPT + j;
    if (k < p.Hkv) {
      if (k == h) {
        s_start = start;
        s_quota = quota_h;
      }
      if (b == 0 && h == 0) p.head_offsets[k] = start;
      start += totals[j];
    }
  }
  if (b == 0 && h == 0 && tid == 0) p.head_offsets[p.Hkv] = tot_rows;
  __syncthreads();
  if (p.nb == 0) return;
  write_block<PER>(p, h, b, (uint32_t)p.state[h * 4 + 0], s_quota, s_start + t_sb + min(t_tb, s_quota), t_tb);
}

// Coalesced copy of the kept K and V rows: GROWS output rows per block of
// GT threads, D/8 lanes per row with 16 bytes each; all loads of a block's
// rows are issued before the stores. Rows past the total (known only on the
// device in threshold mode) are skipped. Small blocks (many resident per CU)
// measured fastest: 128 threads and 16 rows against 256 and 32, 64 or more.
constexpr int GROWS = 16;
constexpr int GT = 128;
constexpr int MAX_LDS_HEADS = 256;

template <int D>
__global__ __launch_bounds__(GT) void evict_gather(EvictParams p) {
  __shared__ int64_t s_off[MAX_LDS_HEADS + 1];
  const int64_t total = p.head_offsets[p.Hkv];
  const int64_t r0 = (int64_t)blockIdx.x * GROWS;
  if (r0 >= total) return;
  const bool lds_heads = p.Hkv <= MAX_LDS_HEADS;
  if (lds_heads)
    for (int k = threadIdx.x; k <= p.Hkv; k += GT) s_off[k] = p.head_offsets[k];
  __syncthreads();
  auto head_of = [&](int64_t r) {  // last h with offset[h] <= r
    int lo = 0, hi = p.Hkv - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int64_t o = lds_heads ? s_off[mid] : p.head_offsets[mid];
      if (o <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  constexpr int LPR = D / 8;
  constexpr int RPP = GT / LPR;  // rows per pass
  constexpr int PASSES = GROWS / RPP;
  static_assert(PASSES >= 1 && PASSES * RPP == GROWS, "a block's rows are whole passes");
  const int part = threadIdx.x % LPR;
  const int rr = threadIdx.x / LPR;
  u32x4 kv[PASSES], vv[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t r = r0 + i * RPP + rr;
    if (r < total) {
      const int h = head_of(r);
      const int64_t src = (int64_t)h * p.kv_hs + (int64_t)p.kept_idx[r] * p.kv_ts + part * 8;
      kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.K + src));
      vv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.V + src));
    }
  }
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t r = r0 + i * RPP + rr;
    if (r < total) {
      __builtin_nontemporal_store(kv[i], reinterpret_cast<u32x4*>(p.K_out + r * D + part * 8));
      __builtin_nontemporal_store(vv[i], reinterpret_cast<u32x4*>(p.V_out + r * D + part * 8));
    }
  }
}

// ---------------------------------------------------------------- one workgroup per head
// Per-head top-k (and keep-all / window-only) with at most HD_MAX candidates
// per head: `reps` workgroups of HD_THREADS per head each keep the head's
// order keys in LDS and radix-select the k-th key T and the tie quota there
// (the same work in every one of them: the head's scores are at most 64 KB,
// and the copies run side by side on different CUs). Per-head row counts
// are known on the host in these modes, so head h's rows start at
// h * per_head; workgroup r of a head owns output rows
// [per_head * r / reps, per_head * (r + 1) / reps): it writes their kept
// positions and copies their K and V rows, so no gather launch follows.
//
// Radix digits as in the grid path (bits 31..21, 20..10, 9..0). Scores that
// cluster in a few bins would serialise the histogram's LDS atomics on a
// few addresses, so each bin has HD_COPIES counters and lane l adds to copy
// l % HD_COPIES: at most 64 / HD_COPIES lanes of a wave meet on an address.
// Copies are stored copy-major with a stride of NBINS + 1 words, so the
// copies of one bin sit in different LDS banks (for the atomics and for the
// digit search's reads alike).
//
// The kept positions are written in ascending order by wave segments: wave
// w owns the contiguous positions [w * seg, (w + 1) * seg) and walks them
// 64 at a time, so a ballot is the keep mask of 64 consecutive positions; a
// count walk and one pass over the 16 waves' totals give each wave its
// first output row and first tie rank. A workgroup keeps the positions of
// its own candidate rows in LDS (in the histogram's space, free once T is
// known) for the copy; its window rows follow from their row numbers.
constexpr int HD_THREADS = 1024;
constexpr int HD_WAVES = HD_THREADS / WAVE;
constexpr int HD_MAX = 16384;
constexpr int HD_COPIES = 8;
constexpr int HD_UNROLL = 16;  // score loads in flight per thread
constexpr int HD_CSTRIDE = NBINS + 1;  // words between histogram copies
constexpr int HD_STEPS = HD_MAX / (HD_WAVES * WAVE);  // 64-position steps of a wave's segment
static_assert(2 * HD_STEPS <= 32, "a segment's classes fit one 32-bit word per lane");
constexpr int HD_ROWS_PER_WG = 128;    // kept rows a workgroup of a head copies (sets the workgroups per head)
constexpr int HD_MAX_REPS = 64;        // at most this many workgroups per head
constexpr int HD_CP_PASSES = 4;        // copy passes with loads in flight
static_assert(HD_CSTRIDE * HD_COPIES >= HD_MAX, "a workgroup's candidate positions live in the histogram's space");

// Number of set bits of m below this lane.
__device__ __forceinline__ int below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave: four DPP row shifts
// (1, 2, 4, 8 lanes) give the sums within each row of 16 lanes, then the
// totals of the rows before a lane's row are added from three readlanes.
__device__ __forceinline__ int wave_incl_scan(int x) {
  constexpr int ROW_SHR1 = 0x111, ROW_SHR2 = 0x112, ROW_SHR4 = 0x114, ROW_SHR8 = 0x118;
  x += __builtin_amdgcn_update_dpp(0, x, ROW_SHR1, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, ROW_SHR2, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, ROW_SHR4, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, ROW_SHR8, 0xf, 0xf, false);
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// The digit holding the rank-th largest key, from per-thread digit counts:
// thread t holds the counts of digits lo + per - 1 (c_top) and lo (c_low,
// per == 2 only), lo = (HD_THREADS - 1 - t) * per, so thread order is
// descending digit order. A wave scan plus the 16 wave totals give each
// thread the keys above its digits, and the one thread whose range holds the
// rank-th key names the digit, the keys in higher digits and the digit's own
// count (1 <= rank <= the keys counted). Block-wide; every thread returns the
// same values.
__device__ __forceinline__ void hd_find_core(int c_top, int c_low, int per, int rank, int& digit, int& above,
                                             int& count) {
  __shared__ __attribute__((aligned(16))) int s_wsum[HD_WAVES];
  __shared__ int s_digit, s_above, s_count;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lo = (HD_THREADS - 1 - tid) * per;
  const int mine = c_top + c_low;
  const int x = wave_incl_scan(mine);
  if (lane == WAVE - 1) s_wsum[wave] = x;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < HD_WAVES; ++w) before += w < wave ? s_wsum[w] : 0;
  const int incl = before + x, excl = incl - mine;
  if (excl < rank && rank <= incl) {
    const bool in_top = rank <= excl + c_top;
    s_digit = in_top ? lo + per - 1 : lo;
    s_above = in_top ? excl : excl + c_top;
    s_count = in_top ? c_top : c_low;
  }
  __syncthreads();
  digit = s_digit;
  above = s_above;
  count = s_count;
}

// hd_find_core over an LDS histogram of nbins (2048 or 1024) digits whose
// counts are summed over COPIES copies; every read of hist is done before
// the first barrier inside.
template <int COPIES>
__device__ void hd_find_digit(const uint32_t* hist, int nbins, int rank, int& digit, int& above) {
  const int per = nbins / HD_THREADS;  // 2 (2048 bins) or 1 (1024)
  auto count = [&](int b) {
    int c = 0;
#pragma unroll
    for (int k = 0; k < COPIES; ++k) c += (int)hist[k * HD_CSTRIDE + b];
    return c;
  };
  const int lo = (HD_THREADS - 1 - (int)threadIdx.x) * per;
  const int c_top = count(lo + per - 1);  // the thread's higher digit first
  const int c_low = per == 2 ? count(lo) : 0;
  int in_digit;
  hd_find_core(c_top, c_low, per, rank, digit, above, in_digit);
}

// Copy of a head's output rows [o_lo, o_hi): D / 8 lanes per row, 16-byte
// pieces, HD_CP_PASSES passes of loads issued before their stores,
// non-temporal. Rows below cand_end take their positions from s_pos (row o
// at s_pos[o - o_lo]); row o >= total is window row o - total.
template <int D>
__device__ __forceinline__ void hd_copy_rows(const EvictParams& p, int h, int o_lo, int o_hi, int cand_end,
                                             int total, const uint32_t* s_pos) {
  constexpr int LPR = D / 8;
  constexpr int RPP = HD_THREADS / LPR;
  const int tid = threadIdx.x;
  const int part = tid % LPR;
  const int rr = tid / LPR;
  const int n_cand = (int)p.n_cand;
  const int64_t out_row0 = (int64_t)h * p.per_head;
  const int64_t head_base = (int64_t)h * p.kv_hs + part * 8;
  for (int b = o_lo; b < o_hi; b += RPP * HD_CP_PASSES) {
    u32x4 kv[HD_CP_PASSES], vv[HD_CP_PASSES];
#pragma unroll
    for (int q = 0; q < HD_CP_PASSES; ++q) {
      const int o = b + q * RPP + rr;
      if (o < o_hi) {
        int64_t pos = o < cand_end ? (int64_t)s_pos[o - o_lo] : (int64_t)n_cand + (o - total);
        pos = pos < 0 ? 0 : (pos >= p.n ? p.n - 1 : pos);
        const int64_t src = head_base + pos * p.kv_ts;
        kv[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.K + src));
        vv[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.V + src));
      }
    }
#pragma unroll
    for (int q = 0; q < HD_CP_PASSES; ++q) {
      const int o = b + q * RPP + rr;
      if (o < o_hi) {
        const int64_t dst = (out_row0 + o) * D + part * 8;
        __builtin_nontemporal_store(kv[q], reinterpret_cast<u32x4*>(p.K_out + dst));
        __builtin_nontemporal_store(vv[q], reinterpret_cast<u32x4*>(p.V_out + dst));
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(HD_THREADS) void evict_head(EvictParams p, int reps) {
  __shared__ uint32_t s_key[HD_MAX];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[HD_CSTRIDE * HD_COPIES];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist12[NBINS + NBINS / 2];  // passes 2 and 3: one copy each (few keys reach them)
  __shared__ int s_cnt[HD_WAVES][2];
  const int h = blockIdx.x / reps;
  const int rep = blockIdx.x % reps;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_cand = (int)p.n_cand;
  const int copy = lane % HD_COPIES;
  const float* sc = p.scores + (int64_t)h * p.s_hs;

  uint32_t T = 0;
  int quota = 0;
  const bool topk = p.mode == MODE_TOPK;
  if (topk) {
    // order keys of the candidates into LDS: a thread's HD_UNROLL score
    // loads (all its candidates) go out first, and the histograms are cleared
    // while they are in flight
    static_assert(HD_THREADS * HD_UNROLL == HD_MAX, "one round of loads covers every candidate");
    float v[HD_UNROLL];
#pragma unroll
    for (int u = 0; u < HD_UNROLL; ++u) {
      const int i = tid + u * HD_THREADS;
      v[u] = i < n_cand ? sc[i] : 0.f;
    }
    {
      u32x4* h4 = reinterpret_cast<u32x4*>(s_hist);
      for (int i = tid; i < HD_CSTRIDE * HD_COPIES / 4; i += HD_THREADS) h4[i] = u32x4{0u, 0u, 0u, 0u};
      u32x4* g4 = reinterpret_cast<u32x4*>(s_hist12);
      for (int i = tid; i < (NBINS + NBINS / 2) / 4; i += HD_THREADS) g4[i] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();  // the clears (the score loads may still be in flight)
    // first digit straight from the registers as each load arrives
#pragma unroll
    for (int u = 0; u < HD_UNROLL; ++u) {
      const int i = tid + u * HD_THREADS;
      if (i < n_cand) {
        const uint32_t k = order_key(v[u]);
        s_key[i] = k;
        atomicAdd(&s_hist[copy * HD_CSTRIDE + (k >> 21)], 1u);
      }
    }
    uint32_t prefix = 0;
    int rank = (int)p.kprime;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int nbins = pass == 2 ? 1024 : 2048;
      __syncthreads();  // (pass 0: the key stores and the first digit's atomics)
      uint32_t* hist = pass == 0 ? s_hist : s_hist12 + (pass == 2 ? NBINS : 0);
      const int hs = digit_shift(pass > 0 ? pass - 1 : 0);  // (pass 0 accumulates nothing here)
      const int ds = digit_shift(pass);
      const uint32_t dm = digit_mask(pass);
      constexpr int RU = 4;  // LDS reads of a batch issued before its atomics
      // passes 1 and 2: the keys that share the digits found so far
      for (int i0 = tid; pass > 0 && i0 < n_cand; i0 += HD_THREADS * RU) {
        uint32_t u[RU];
#pragma unroll
        for (int k = 0; k < RU; ++k) {
          const int i = i0 + k * HD_THREADS;
          u[k] = i < n_cand ? s_key[i] : 0u;
        }
#pragma unroll
        for (int k = 0; k < RU; ++k) {
          const int i = i0 + k * HD_THREADS;
          if (i < n_cand && (u[k] >> hs) == (prefix >> hs)) atomicAdd(&hist[(u[k] >> ds) & dm], 1u);
        }
      }
      __syncthreads();
      int digit, above;
      if (pass == 0)
        hd_find_digit<HD_COPIES>(hist, nbins, rank, digit, above);
      else
        hd_find_digit<1>(hist, nbins, rank, digit, above);
      prefix |= (uint32_t)digit << ds;
      rank -= above;
    }
    T = prefix;
    quota = rank;  // keys equal to T that are kept, lowest positions first
  } else {
    __syncthreads();
  }

  // keep classes: 1 kept, 2 tied at T (top-k), 0 dropped
  const int seg = ((n_cand + HD_WAVES * WAVE - 1) / (HD_WAVES * WAVE)) * WAVE;
  const int seg_lo = wave * seg;
  const int seg_hi = min(seg_lo + seg, n_cand);
  const bool keep_all = p.mode == MODE_ALL;
  auto cls_of = [&](int i) -> int {
    if (i >= seg_hi) return 0;
    if (!topk) return keep_all ? 1 : 0;
    const uint32_t u = s_key[i];
    return u > T ? 1 : (u == T ? 2 : 0);
  };
  constexpr int WU = 2;  // 64-position steps of a walk whose reads are issued together
  // the walk's classes, 2 bits per step (a segment has at most HD_STEPS steps),
  // kept for the write walk
  uint32_t cls_bits = 0u;
  int n_keep = 0, n_tie = 0;
  for (int i0 = seg_lo, st = 0; i0 < seg_hi; i0 += WAVE * WU, st += WU) {
    int c[WU];
#pragma unroll
    for (int k = 0; k < WU; ++k) c[k] = cls_of(i0 + k * WAVE + lane);
#pragma unroll
    for (int k = 0; k < WU; ++k) {
      cls_bits |= (uint32_t)c[k] << (2 * (st + k));
      n_keep += __popcll(__ballot(c[k] == 1));
      n_tie += __popcll(__ballot(c[k] == 2));
    }
  }
  if (lane == 0) {
    s_cnt[wave][0] = n_keep;
    s_cnt[wave][1] = n_tie;
  }
  __syncthreads();
  int out_run = 0, tie_run = 0, total = 0, ties_seen = 0, my_rows = 0;
  for (int w = 0; w < HD_WAVES; ++w) {
    const int kw = s_cnt[w][0], tw = s_cnt[w][1];
    const int take = min(max(quota - ties_seen, 0), tw);
    if (w < wave) {
      out_run += kw + take;
      tie_run += tw;
    }
    if (w == wave) my_rows = kw + take;
    total += kw + take;
    ties_seen += tw;
  }
  // Kept candidate positions, ascending, then the window's rows; this
  // workgroup writes the rows [o_lo, o_hi) of the head and records its
  // candidate rows' positions in s_pos (writes are capped to the head's rows
  // whatever the counts say).
  const int per_head = (int)p.per_head;
  int32_t* out = p.kept_idx + (int64_t)h * per_head;
  const int w_rows = (int)(p.n - p.n_cand);
  const int cand_rows = per_head - w_rows;
  const int o_lo = rep * p.rows_q + min(rep, p.rows_r);
  const int o_hi = o_lo + p.rows_q + (rep < p.rows_r ? 1 : 0);
  uint32_t* s_pos = s_hist;  // the histogram's space, free after the selection (barriers since its last read)
  // only waves whose output rows meet this workgroup's candidate rows walk
  const bool my_part = out_run < min(o_hi, cand_rows) && out_run + my_rows > o_lo;  // wave-uniform
  for (int i0 = seg_lo, st = 0; my_part && i0 < seg_hi; i0 += WAVE * WU, st += WU) {
    int c[WU];
#pragma unroll
    for (int k = 0; k < WU; ++k) c[k] = (int)((cls_bits >> (2 * (st + k))) & 3u);
#pragma unroll
    for (int k = 0; k < WU; ++k) {
      const int i = i0 + k * WAVE + lane;
      const uint64_t tm = __ballot(c[k] == 2);
      bool keep = c[k] == 1;
      if (tm) keep = keep || (c[k] == 2 && tie_run + below(tm) < quota);  // (steps with no tie skip this)
      const uint64_t km = __ballot(keep);
      const int o = out_run + below(km);
      if (keep && o < cand_rows && o >= o_lo && o < o_hi) {
        out[o] = i;
        s_pos[o - o_lo] = (uint32_t)i;
      }
      out_run += __popcll(km);
      tie_run += __popcll(tm);
    }
  }
  // window row j is row total + j
  const int win_lo = max(o_lo, total), win_hi = min(o_hi, min(total + w_rows, per_head));
  for (int o = win_lo + tid; o < win_hi; o += HD_THREADS) out[o] = n_cand + (o - total);
  if (tid == 0 && rep == 0) {
    p.head_offsets[h] = (int64_t)h * per_head;
    if (h == 0) p.head_offsets[p.Hkv] = (int64_t)p.Hkv * per_head;
  }
  __syncthreads();  // s_pos complete

  hd_copy_rows<D>(p, h, o_lo, o_hi, min(total, cand_rows), total, s_pos);
}

// ---------------------------------------------------------------- long heads
// Per-head top-k with more than HD_MAX candidates per head (up to LH_MAX),
// three launches:
// evict_lh_hist: blocks of LH_CHUNK positions of a head each store the
//   histogram of their keys' first radix digit (bits 31..21) with plain
//   stores, so no workspace needs clearing.
// evict_lh_bin: the same blocks each sum their head's block histograms and
//   find the first digit of the k-th key; then, for their own positions,
//   they store per segment of LH_SEG positions the count of keys above that
//   digit's bin, and the (key, position) pairs of the keys inside it into
//   the head's list. A block's first list entry is the bin count of the
//   blocks before it, read from their histograms, so the list holds exactly
//   the bin's keys in position order of blocks, with the keys of a segment
//   adjacent. (A bin of more than LH_CAP keys is not listed.)
// evict_long_head: `reps` workgroups per head, each of which finishes the
//   selection from the list in LDS: second and third digits, then the kept
//   and tied counts per segment. (For a bin too large for the list, it reads
//   the scores for these steps instead.) A scan of the segment counts gives
//   every segment its first output row and the ties before it; the
//   workgroup walks only the segments that meet its rows [o_lo, o_hi),
//   writes their kept positions and copies the rows as evict_head does.
//   Workgroup b serves head b % Hkv: with a multiple of 8 heads the
//   workgroups of one head share an XCD and its L2.
constexpr int LH_SEG = 4 * WAVE;                // positions per segment: a 16-byte load per lane of a wave
constexpr int LH_MAX_SEGS = 2 * HD_THREADS;     // two segments per thread in the scans
constexpr int LH_MAX = LH_SEG * LH_MAX_SEGS;    // 524,288 candidates per head
constexpr int LH_CAP = 16384;                   // keys of the first digit's bin kept in LDS
constexpr int LH_CHUNK = 8 * HD_THREADS;        // positions per first-digit histogram block
constexpr int LH_SPW = LH_CHUNK / LH_SEG / HD_WAVES;  // segments per wave in evict_lh_bin
constexpr int LH_UNROLL = 4;                    // segments per wave with loads in flight (score passes)
constexpr int LH_ROWS_PER_WG = 128;             // kept rows per workgroup, before the fill cap

// Scores i .. i + 3 of a head through a buffer resource over its candidates
// (a load past them reads 0; callers mask those entries). `wide` (uniform
// over the wave: an aligned head and a segment that is not the ragged last
// one) takes one 16-byte load, else four 4-byte loads, each checked on its
// own against the resource's end. No per-lane branch: a load is never
// ordered behind another path's loads into the same registers.
__device__ __forceinline__ void lh_load(__amdgpu_buffer_rsrc_t r, int i, bool wide, float (&v)[4]) {
  if (wide) {
    const u32x4 x = buf_ld16(r, 4 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(x[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * (i + e), 0, 0));
  }
}

// grid: nch blocks per head, head-major (block h * nch + c)
__global__ __launch_bounds__(HD_THREADS) void evict_lh_hist(EvictParams p, int nch) {
  __shared__ __attribute__((aligned(16))) uint32_t s_h[HD_CSTRIDE * HD_COPIES];
  const int h = blockIdx.x / nch, c = blockIdx.x % nch;
  const int tid = threadIdx.x;
  const int copy = (tid & 63) % HD_COPIES;
  const int n_cand = (int)p.n_cand;
  const float* sc = p.scores + (int64_t)h * p.s_hs;
  constexpr int PER = LH_CHUNK / HD_THREADS;
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = c * LH_CHUNK + u * HD_THREADS + tid;
    v[u] = i < n_cand ? sc[i] : 0.f;
  }
  u32x4* h4 = reinterpret_cast<u32x4*>(s_h);
  for (int i = tid; i < HD_CSTRIDE * HD_COPIES / 4; i += HD_THREADS) h4[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = c * LH_CHUNK + u * HD_THREADS + tid;
    if (i < n_cand) atomicAdd(&s_h[copy * HD_CSTRIDE + (order_key(v[u]) >> 21)], 1u);
  }
  __syncthreads();
  const int b = 2 * tid;
  uint32_t c0 = 0, c1 = 0;
#pragma unroll
  for (int k = 0; k < HD_COPIES; ++k) {
    c0 += s_h[k * HD_CSTRIDE + b];
    c1 += s_h[k * HD_CSTRIDE + b + 1];
  }
  *reinterpret_cast<uint2*>(p.hist + ((int64_t)h * nch + c) * NBINS + b) = make_uint2(c0, c1);
}

// grid: nch blocks per head, head-major (block h * nch + c)
__global__ __launch_bounds__(HD_THREADS) void evict_lh_bin(EvictParams p, int nch) {
  __shared__ int s_wn[HD_WAVES];
  __shared__ int s_cbase;
  const int h = blockIdx.x / nch, c = blockIdx.x % nch;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_cand = (int)p.n_cand;
  const int n_seg = (n_cand + LH_SEG - 1) / LH_SEG;
  const __amdgpu_buffer_rsrc_t rs = tile_rsrc(p.scores + (int64_t)h * p.s_hs, 4 * n_cand);
  const int n_wide = p.vec4 ? (n_cand % LH_SEG == 0 ? n_seg : n_seg - 1) : 0;
  const int sg0 = c * (LH_CHUNK / LH_SEG) + wave * LH_SPW;  // this wave's first segment
  float v[LH_SPW][4];
#pragma unroll
  for (int u = 0; u < LH_SPW; ++u) {
    const int sg = sg0 + u;
    if (sg < n_seg) lh_load(rs, sg * LH_SEG + 4 * lane, sg < n_wide, v[u]);
  }
  // first digit: thread t sums digits 2 * (HD_THREADS - 1 - t) and + 1 over
  // the head's block histograms (descending digit order over the threads)
  int c_low = 0, c_top = 0, b_low = 0, b_top = 0;  // (b_*: the chunks before this one)
  {
    const uint32_t* g = p.hist + (int64_t)h * nch * NBINS + 2 * (HD_THREADS - 1 - tid);
#pragma unroll 8
    for (int cc = 0; cc < nch; ++cc) {
      const uint2 x = *reinterpret_cast<const uint2*>(g + (int64_t)cc * NBINS);
      c_low += (int)x.x;
      c_top += (int)x.y;
      b_low += cc < c ? (int)x.x : 0;
      b_top += cc < c ? (int)x.y : 0;
    }
  }
  if (tid == 0) s_cbase = 0;  // (set below by the thread that summed the k-th key's digit)
  int d0, above, n_bin;
  hd_find_core(c_top, c_low, 2, (int)p.kprime, d0, above, n_bin);  // (its barriers order the store above)
  if (c == 0 && tid == 0) {
    p.lh_state[4 * h + 0] = d0;
    p.lh_state[4 * h + 1] = (int)p.kprime - above;  // rank of the k-th key inside the bin
    p.lh_state[4 * h + 2] = n_bin;
  }
  const uint32_t d0u = (uint32_t)d0;
  uint32_t k[LH_SPW][4];
  uint64_t m[LH_SPW][4];
  int w_n = 0;  // this wave's bin keys (wave-uniform)
#pragma unroll
  for (int u = 0; u < LH_SPW; ++u) {
    const int sg = sg0 + u;
    const int i = sg * LH_SEG + 4 * lane;
    int n_above = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k[u][e] = order_key(v[u][e]);
      const bool ok = i + e < n_cand;  // (false past the last segment)
      n_above += __popcll(__ballot(ok && (k[u][e] >> 21) > d0u));
      m[u][e] = __ballot(ok && (k[u][e] >> 21) == d0u);
      w_n += __popcll(m[u][e]);
    }
    if (sg < n_seg && lane == 0) p.seg_above[(int64_t)h * n_seg + sg] = (uint32_t)n_above;
  }
  if (n_bin > LH_CAP) return;  // (block-uniform) the long-head kernel reads the scores instead
  if (lane == 0) s_wn[wave] = w_n;
  // the bin's keys in the chunks before this one: from the thread that summed d0
  const int lo = 2 * (HD_THREADS - 1 - tid);
  if (d0 == lo) s_cbase = b_low;
  if (d0 == lo + 1) s_cbase = b_top;
  __syncthreads();
  int base = s_cbase;
#pragma unroll
  for (int w = 0; w < HD_WAVES; ++w) base += w < wave ? s_wn[w] : 0;
  uint2* out = p.lh_list + (int64_t)h * LH_CAP;
#pragma unroll
  for (int u = 0; u < LH_SPW; ++u) {
    const int i = (sg0 + u) * LH_SEG + 4 * lane;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = base + below(m[u][e]);
      if (((m[u][e] >> lane) & 1u) && j >= 0 && j < LH_CAP) out[j] = make_uint2(k[u][e], (uint32_t)(i + e));
      base += __popcll(m[u][e]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(HD_THREADS) void evict_long_head(EvictParams p, int reps) {
  // the head's bin list ((key, position) pairs); after the counts, the
  // positions of this workgroup's candidate rows
  __shared__ __attribute__((aligned(16))) uint32_t s_list[2 * LH_CAP];
  __shared__ __attribute__((aligned(16))) uint32_t s_h1[NBINS + 4];  // second digit; then segment first rows [n_seg + 1]
  __shared__ __attribute__((aligned(16))) uint32_t s_h2[NBINS / 2];  // third digit
  __shared__ __attribute__((aligned(16))) uint32_t s_kt[LH_MAX_SEGS];  // per segment: kept above T | tied << 16; then ties before
  __shared__ uint16_t s_above[LH_MAX_SEGS];  // per segment: keys above the first digit's bin
  __shared__ int s_wsum[HD_WAVES], s_wsum2[HD_WAVES];
  __shared__ int s_first, s_last, s_namb;
  static_assert(LH_SEG <= 0xffff, "segment counts fit 16 bits");
  constexpr int AMB_CAP = NBINS / 2;  // keys sharing T's bits 31..10, kept in s_h1's space
  const int h = blockIdx.x % p.Hkv;
  const int rep = blockIdx.x / p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_cand = (int)p.n_cand;
  const int n_seg = (n_cand + LH_SEG - 1) / LH_SEG;
  const float* sc = p.scores + (int64_t)h * p.s_hs;
  const __amdgpu_buffer_rsrc_t rs = tile_rsrc(sc, 4 * n_cand);
  // 16-byte loads: an aligned head, every segment but a ragged last one
  const int n_wide = p.vec4 ? (n_cand % LH_SEG == 0 ? n_seg : n_seg - 1) : 0;
  const uint32_t d0u = (uint32_t)p.lh_state[4 * h + 0];
  int rank = p.lh_state[4 * h + 1];
  const int n_bin = p.lh_state[4 * h + 2];
  const bool use_list = n_bin <= LH_CAP;  // (else the score passes below)

  // Passes over the scores (a bin too large for the list) visit the
  // segments from a per-workgroup offset on, wrapping round, so that the
  // workgroups of a head do not all read the same lines at once; wave w
  // takes the w-th of every HD_WAVES segments in that order.
  const int s_off = n_seg * rep / reps;  // n_seg <= 2048 and reps < 2^17
  auto seg_at = [&](int j) { return j + s_off < n_seg ? j + s_off : j + s_off - n_seg; };

  // the segment counts' loads go out first, then the list's (one round:
  // LH_CAP = 16 * HD_THREADS) once its length is known; the clears run
  // while they are in flight
  static_assert(LH_MAX_SEGS == 2 * HD_THREADS, "two segment counts per thread");
  uint32_t ab[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int sg = tid + q * HD_THREADS;
    ab[q] = sg < n_seg ? p.seg_above[(int64_t)h * n_seg + sg] : 0u;
  }
  constexpr int LU = LH_CAP / HD_THREADS;
  uint2 le[LU];
  if (use_list) {
    const uint2* lst = p.lh_list + (int64_t)h * LH_CAP;
#pragma unroll
    for (int u = 0; u < LU; ++u) {
      const int j = tid + u * HD_THREADS;
      le[u] = j < n_bin ? lst[j] : make_uint2(0u, 0u);
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int sg = tid + q * HD_THREADS;
    if (sg < n_seg) s_above[sg] = (uint16_t)ab[q];
  }
  for (int i = tid; i < NBINS / 4; i += HD_THREADS) reinterpret_cast<u32x4*>(s_h1)[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = tid; i < NBINS / 8; i += HD_THREADS) reinterpret_cast<u32x4*>(s_h2)[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = tid; i < LH_MAX_SEGS / 4; i += HD_THREADS) reinterpret_cast<u32x4*>(s_kt)[i] = u32x4{0u, 0u, 0u, 0u};
  if (tid == 0) {
    s_first = n_seg;  // (an empty walk unless set below)
    s_last = -1;
    s_namb = 0;
  }
  __syncthreads();

  // second digit over the bin's keys; the list into LDS
  if (use_list) {
#pragma unroll
    for (int u = 0; u < LU; ++u) {
      const int j = tid + u * HD_THREADS;
      if (j < n_bin) {
        *reinterpret_cast<uint2*>(&s_list[2 * j]) = le[u];
        atomicAdd(&s_h1[(le[u].x >> 10) & 2047u], 1u);
      }
    }
  } else {
    for (int j = wave; j < n_seg; j += HD_WAVES) {
      float v[4];
      const int s = seg_at(j);
      const int i = s * LH_SEG + 4 * lane;
      lh_load(rs, i, s < n_wide, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk = order_key(v[e]);
        if (i + e < n_cand && (kk >> 21) == d0u) atomicAdd(&s_h1[(kk >> 10) & 2047u], 1u);
      }
    }
  }
  __syncthreads();
  int d1, above;
  hd_find_digit<1>(s_h1, NBINS, rank, d1, above);
  rank -= above;
  const uint32_t pre = (d0u << 21) | ((uint32_t)d1 << 10);  // the k-th key's bits 31..10

  // Third digit over the keys with those bits, and the per-segment counts
  // of kept keys (besides those above the bin) and of ties at T. From the
  // list: one pass over each thread's run of entries (a segment's keys are
  // adjacent in the list, so a thread adds once per segment it meets) counts
  // the keys above T's bits 31..10 and histograms and sets aside the keys
  // sharing them (few unless very many keys tie); those are sorted out once
  // T is known. Without the list: two passes over the scores.
  uint32_t T;
  int quota;
  const uint32_t pre10 = pre >> 10;
  if (use_list) {
    const int per = (n_bin + HD_THREADS - 1) / HD_THREADS;  // <= LU
    const int j0 = tid * per, j1 = min(j0 + per, n_bin);
    uint2* s_amb = reinterpret_cast<uint2*>(s_h1);  // free since the second digit was found
    int cur = -1;
    uint32_t acc = 0u;
#pragma unroll
    for (int q = 0; q < LU; ++q) {
      if (j0 + q < j1) {
        const uint2 e = *reinterpret_cast<const uint2*>(&s_list[2 * (j0 + q)]);
        const int sg = (int)(e.y / LH_SEG);
        if (sg != cur) {
          if (acc) atomicAdd(&s_kt[cur], acc);
          cur = sg;
          acc = 0u;
        }
        const uint32_t t10 = e.x >> 10;
        if (t10 > pre10) {
          ++acc;
        } else if (t10 == pre10) {
          atomicAdd(&s_h2[e.x & 1023u], 1u);
          const int a = atomicAdd(&s_namb, 1);
          if (a < AMB_CAP) s_amb[a] = e;
        }
      }
    }
    if (acc) atomicAdd(&s_kt[cur], acc);
    __syncthreads();
    int d2;
    hd_find_digit<1>(s_h2, NBINS / 2, rank, d2, above);
    T = pre | (uint32_t)d2;
    quota = rank - above;
    const int n_amb = s_namb;
    if (n_amb <= AMB_CAP) {
      for (int j = tid; j < n_amb; j += HD_THREADS) {
        const uint2 e = s_amb[j];
        if (e.x >= T) atomicAdd(&s_kt[e.y / LH_SEG], e.x > T ? 1u : 0x10000u);
      }
    } else {
      for (int j = j0; j < j1; ++j) {
        const uint2 e = *reinterpret_cast<const uint2*>(&s_list[2 * j]);
        if ((e.x >> 10) == pre10 && e.x >= T) atomicAdd(&s_kt[e.y / LH_SEG], e.x > T ? 1u : 0x10000u);
      }
    }
  } else {
    for (int j = wave; j < n_seg; j += HD_WAVES) {
      float v[4];
      const int s = seg_at(j);
      const int i = s * LH_SEG + 4 * lane;
      lh_load(rs, i, s < n_wide, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk = order_key(v[e]);
        if (i + e < n_cand && (kk >> 10) == pre10) atomicAdd(&s_h2[kk & 1023u], 1u);
      }
    }
    __syncthreads();
    int d2;
    hd_find_digit<1>(s_h2, NBINS / 2, rank, d2, above);
    T = pre | (uint32_t)d2;
    quota = rank - above;
    for (int j = wave; j < n_seg; j += HD_WAVES) {
      const int s = seg_at(j);
      float v[4];
      const int i = s * LH_SEG + 4 * lane;
      lh_load(rs, i, s < n_wide, v);
      int sure = 0, tied = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk = order_key(v[e]);
        const bool ok = i + e < n_cand;
        sure += __popcll(__ballot(ok && kk > T));
        tied += __popcll(__ballot(ok && kk == T));
      }
      if (lane == 0) {
        s_kt[s] = (uint32_t)sure | ((uint32_t)tied << 16);
        s_above[s] = 0;
      }
    }
  }
  quota = max(quota, 0);  // keys equal to T that are kept, lowest positions first
  __syncthreads();

  // thread t: segments 2t and 2t + 1. Ties are kept lowest position first,
  // so the rows before a segment are its sure rows before plus
  // min(ties before it, quota): one scan of both counts.
  int sure[2], tied[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = 2 * tid + j;
    const uint32_t kt = s < n_seg ? s_kt[s] : 0u;
    sure[j] = (s < n_seg ? (int)s_above[s] : 0) + (int)(kt & 0xffffu);
    tied[j] = (int)(kt >> 16);
  }
  const int ss = sure[0] + sure[1], tt = tied[0] + tied[1];
  const int xs = wave_incl_scan(ss), xt = wave_incl_scan(tt);
  if (lane == WAVE - 1) {
    s_wsum[wave] = xs;
    s_wsum2[wave] = xt;
  }
  __syncthreads();
  int sb = xs - ss, tb = xt - tt;
#pragma unroll
  for (int w = 0; w < HD_WAVES; ++w) {
    sb += w < wave ? s_wsum[w] : 0;
    tb += w < wave ? s_wsum2[w] : 0;
  }
  uint32_t* s_start = s_h1;  // free once the set-aside keys are sorted out
  uint32_t* s_tb = s_kt;     // each thread overwrites only the entries it read
  if (2 * tid < n_seg) {
    s_start[2 * tid] = (uint32_t)(sb + min(tb, quota));
    s_tb[2 * tid] = (uint32_t)tb;
  }
  if (2 * tid + 1 < n_seg) {
    s_start[2 * tid + 1] = (uint32_t)(sb + sure[0] + min(tb + tied[0], quota));
    s_tb[2 * tid + 1] = (uint32_t)(tb + tied[0]);
  }
  if (2 * tid < n_seg && 2 * tid + 2 >= n_seg) s_start[n_seg] = (uint32_t)(sb + ss + min(tb + tt, quota));
  __syncthreads();

  // this workgroup's rows: kept candidates in ascending position, then the window
  const int per_head = (int)p.per_head;
  const int w_rows = (int)(p.n - p.n_cand);
  const int cand_rows = per_head - w_rows;
  const int total = (int)s_start[n_seg];
  const int o_lo = rep * p.rows_q + min(rep, p.rows_r);
  const int o_hi = o_lo + p.rows_q + (rep < p.rows_r ? 1 : 0);
  const int c_hi = min(o_hi, min(total, cand_rows));
  const bool walk = o_lo < c_hi;
  // the segments holding rows o_lo and c_hi - 1 (non-empty, so unique)
  if (walk) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int s = 2 * tid + j;
      if (s < n_seg) {
        const int st = (int)s_start[s], en = (int)s_start[s + 1];
        if (st <= o_lo && o_lo < en) s_first = s;
        if (st < c_hi && c_hi <= en) s_last = s;
      }
    }
  }
  __syncthreads();
  int32_t* out = p.kept_idx + (int64_t)h * per_head;
  uint32_t* s_pos = s_list;  // the list is no longer read
  if (walk) {
    const int sf = max(s_first, 0), sl = min(s_last, n_seg - 1);
    for (int s = sf + wave; s <= sl; s += HD_WAVES) {
      float v[4];
      const int i = s * LH_SEG + 4 * lane;
      lh_load(rs, i, s < n_wide, v);
      bool gt[4], eq[4], keep[4];
      int tc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk = order_key(v[e]);
        const bool ok = i + e < n_cand;
        gt[e] = ok && kk > T;
        eq[e] = ok && kk == T;
        tc += eq[e];
      }
      int tr = (int)s_tb[s] + wave_incl_scan(tc) - tc;  // tie rank of the lane's first tie
      int kc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        keep[e] = gt[e] || (eq[e] && tr < quota);
        tr += eq[e];
        kc += keep[e];
      }
      int o = (int)s_start[s] + wave_incl_scan(kc) - kc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (keep[e]) {
          if (o >= o_lo && o < c_hi) {
            out[o] = i + e;
            s_pos[o - o_lo] = (uint32_t)(i + e);
          }
          ++o;
        }
      }
    }
  }
  // window row j is row total + j
  const int win_lo = max(o_lo, total), win_hi = min(o_hi, min(total + w_rows, per_head));
  for (int o = win_lo + tid; o < win_hi; o += HD_THREADS) out[o] = n_cand + (o - total);
  if (tid == 0 && rep == 0) {
    p.head_offsets[h] = (int64_t)h * per_head;
    if (h == 0) p.head_offsets[p.Hkv] = (int64_t)p.Hkv * per_head;
  }
  __syncthreads();  // s_pos complete
  hd_copy_rows<D>(p, h, o_lo, o_hi, min(total, cand_rows), total, s_pos);
}

// The one-workgroup-per-head path serves per-head top-k budgets (and their
// keep-all / window-only ends) with at most HD_MAX candidates per head and
// Hkv * n < 2^31 (row counts fit 32 bits); thresholds, layer budgets and
// longer heads take the grid path.
bool use_head_path(const kvs_evict_desc& e) {
  const int64_t w = e.window < e.n_tok ? e.window : e.n_tok;
  return e.k >= 0 && e.scope == KVS_SCOPE_HEAD && e.n_tok - w <= HD_MAX &&
         (int64_t)e.n_kvheads * e.n_tok < ((int64_t)1 << 31);
}

// Per-head top-k with HD_MAX < candidates <= LH_MAX per head (and the same
// row-count limit) takes the long-head path.
bool use_long_path(const kvs_evict_desc& e) {
  const int64_t w = e.window < e.n_tok ? e.window : e.n_tok;
  const int64_t n_cand = e.n_tok - w;
  return e.k > 0 && e.k < n_cand && e.scope == KVS_SCOPE_HEAD && n_cand > HD_MAX && n_cand <= LH_MAX &&
         (int64_t)e.n_kvheads * e.n_tok < ((int64_t)1 << 31);
}

// Keys per thread of the grid kernels for this layer (see GRID_SMALL).
int grid_per(const kvs_evict_desc& e) {
  const int64_t nb2 = (e.n_tok + epb_of(8) - 1) / epb_of(8);
  return (int64_t)e.n_kvheads * nb2 <= GRID_SMALL ? 4 : 8;
}

struct WsLayout {
  size_t hist, blk, state, list, total;
  bool long_head;  // the long-head path's layout
};

// Grid path: histograms, block counts, per-head state. The head path uses no
// workspace (its state lives in LDS; it writes the kept indices directly).
// The long-head path's workspace (block histograms, segment counts, bin
// lists) is larger than the grid path's: it is taken when it fits `budget`
// bytes, else the grid path serves those heads too (the same selection).
WsLayout ws_layout(const kvs_evict_desc& e, size_t budget) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WsLayout L{};
  const int Hkv = e.n_kvheads;
  if (use_head_path(e)) {
    L.total = 256;
    return L;
  }
  if (use_long_path(e)) {  // block histograms, segment counts, head state, bin lists
    const int64_t w = e.window < e.n_tok ? e.window : e.n_tok;
    const int64_t nch = (e.n_tok - w + LH_CHUNK - 1) / LH_CHUNK;
    const int64_t n_seg = (e.n_tok - w + LH_SEG - 1) / LH_SEG;
    L.hist = 0;
    L.blk = al((size_t)Hkv * nch * NBINS * 4);                 // segment counts
    L.state = L.blk + al((size_t)Hkv * n_seg * 4);             // head state
    L.list = L.state + al((size_t)Hkv * 16);                   // bin lists
    L.total = L.list + al((size_t)Hkv * LH_CAP * 8);
    L.long_head = true;
    if (L.total <= budget) return L;
    L = WsLayout{};
  }
  const int64_t nb = (e.n_tok + epb_of(grid_per(e)) - 1) / epb_of(grid_per(e));
  L.hist = 0;
  L.blk = al((size_t)3 * Hkv * NBINS * 4);
  L.state = L.blk + al((size_t)Hkv * (nb > 0 ? nb : 1) * 16);
  L.total = L.state + al((size_t)Hkv * 16);
  return L;
}

}  // namespace

// Workspace of kv_evict_noalloc: a fixed device array of this library, one
// copy per GPU, held until the process ends. In host code `scratch` names a
// host-side stand-in, never device memory: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is passed to kernels.
static __device__ __align__(256) char scratch[EVICT_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_SCRATCH_DEVICES] = {};
}  // namespace

hipError_t evict_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= MAX_SCRATCH_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t evict_workspace_bytes(const kvs_evict_desc& e, size_t budget) { return ws_layout(e, budget).total; }

hipError_t launch_evict(const kvs_evict_desc& e, const float* scores, const uint16_t* K, const uint16_t* V,
                        int32_t* kept_idx, int64_t* head_offsets, uint16_t* K_out, uint16_t* V_out,
                        void* workspace, size_t workspace_bytes, hipStream_t s) {
  EvictParams p{};
  p.scores = scores;
  p.s_hs = e.score_head_stride;
  p.K = K;
  p.V = V;
  p.kv_hs = e.kv_head_stride;
  p.kv_ts = e.kv_tok_stride;
  p.kept_idx = kept_idx;
  p.head_offsets = head_offsets;
  p.K_out = K_out;
  p.V_out = V_out;
  p.Hkv = e.n_kvheads;
  p.D = e.head_dim;
  p.n = e.n_tok;
  const int64_t w = e.window < e.n_tok ? e.window : e.n_tok;
  p.n_cand = e.n_tok - w;
  const int per = grid_per(e);
  p.nb = (int)((e.n_tok + epb_of(per) - 1) / epb_of(per));
  p.tau = e.tau;
  p.layer = e.scope == KVS_SCOPE_LAYER && e.k >= 0;
  if (e.k < 0) {
    p.mode = MODE_TAU;
  } else {
    const int64_t cand = p.layer ? p.n_cand * p.Hkv : p.n_cand;
    p.kprime = e.k < cand ? e.k : cand;
    p.mode = p.kprime == 0 ? MODE_WINDOW : (p.kprime == cand ? MODE_ALL : MODE_TOPK);
  }
  const WsLayout L = ws_layout(e, workspace_bytes);
  char* ws = static_cast<char*>(workspace);

  if (use_head_path(e)) {
    const int64_t kc = p.mode == MODE_TOPK ? p.kprime : (p.mode == MODE_ALL ? p.n_cand : 0);
    p.per_head = kc + (p.n - p.n_cand);
    // workgroups per head: one per HD_ROWS_PER_WG kept rows, at most
    // HD_MAX_REPS, and no more than fill 512 workgroups over the heads
    int64_t reps = (p.per_head + HD_ROWS_PER_WG - 1) / HD_ROWS_PER_WG;
    const int64_t fill = (512 + p.Hkv - 1) / p.Hkv;
    reps = reps < fill ? reps : fill;
    reps = reps < HD_MAX_REPS ? reps : HD_MAX_REPS;
    reps = reps < 1 ? 1 : reps;
    const int64_t blocks = (int64_t)p.Hkv * reps;  // Hkv * n < 2^31 and reps <= 64
    p.rows_q = (int32_t)(p.per_head / reps);
    p.rows_r = (int32_t)(p.per_head % reps);
    if (p.D == 128)
      hipLaunchKernelGGL(evict_head<128>, dim3((unsigned)blocks), dim3(HD_THREADS), 0, s, p, (int)reps);
    else
      hipLaunchKernelGGL(evict_head<64>, dim3((unsigned)blocks), dim3(HD_THREADS), 0, s, p, (int)reps);
    return hipGetLastError();
  }

  if (L.long_head) {
    p.hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    p.seg_above = reinterpret_cast<uint32_t*>(ws + L.blk);
    p.lh_state = reinterpret_cast<int32_t*>(ws + L.state);
    p.lh_list = reinterpret_cast<uint2*>(ws + L.list);
    const int nch = (int)((p.n_cand + LH_CHUNK - 1) / LH_CHUNK);
    p.per_head = p.kprime + (p.n - p.n_cand);
    p.vec4 = (reinterpret_cast<uintptr_t>(scores) & 15u) == 0 && (p.s_hs & 3) == 0;
    // workgroups per head: one per LH_ROWS_PER_WG kept rows, at most
    // HD_MAX_REPS, no more than fill one workgroup per CU over the heads,
    // and enough that a workgroup's candidate rows fit its position list
    int64_t reps = (p.per_head + LH_ROWS_PER_WG - 1) / LH_ROWS_PER_WG;
    const int64_t fill = (256 + p.Hkv - 1) / p.Hkv;
    reps = reps < fill ? reps : fill;
    reps = reps < HD_MAX_REPS ? reps : HD_MAX_REPS;
    const int64_t need = (p.per_head + 2 * LH_CAP - 1) / (2 * LH_CAP);
    reps = reps > need ? reps : need;
    reps = reps < 1 ? 1 : reps;
    p.rows_q = (int32_t)(p.per_head / reps);
    p.rows_r = (int32_t)(p.per_head % reps);
    hipLaunchKernelGGL(evict_lh_hist, dim3((unsigned)(p.Hkv * nch)), dim3(HD_THREADS), 0, s, p, nch);
    hipLaunchKernelGGL(evict_lh_bin, dim3((unsigned)(p.Hkv * nch)), dim3(HD_THREADS), 0, s, p, nch);
    const unsigned blocks = (unsigned)(p.Hkv * reps);  // Hkv * n < 2^31, so Hkv * reps < 2^17
    if (p.D == 128)
      hipLaunchKernelGGL(evict_long_head<128>, dim3(blocks), dim3(HD_THREADS), 0, s, p, (int)reps);
    else
      hipLaunchKernelGGL(evict_long_head<64>, dim3(blocks), dim3(HD_THREADS), 0, s, p, (int)reps);
    return hipGetLastError();
  }

  p.hist = reinterpret_cast<uint32_t*>(ws + L.hist);
  p.blk = reinterpret_cast<int32_t*>(ws + L.blk);
  p.state = reinterpret_cast<int32_t*>(ws + L.state);

  const dim3 grid(p.nb > 0 ? p.nb : 1, p.Hkv);
  hipError_t err;
  if (p.mode == MODE_TOPK) {
    hipLaunchKernelGGL(evict_zero, dim3(64), dim3(256), 0, s, p.hist, (int64_t)3 * p.Hkv * NBINS);
    if (per == 4) {
      hipLaunchKernelGGL((evict_hist<0, 4>), grid, dim3(EV_THREADS), 0, s, p);
      hipLaunchKernelGGL((evict_hist<1, 4>), grid, dim3(EV_THREADS), 0, s, p);
      hipLaunchKernelGGL((evict_hist<2, 4>), grid, dim3(EV_THREADS), 0, s, p);
    } else {
      hipLaunchKernelGGL((evict_hist<0, 8>), grid, dim3(EV_THREADS), 0, s, p);
      hipLaunchKernelGGL((evict_hist<1, 8>), grid, dim3(EV_THREADS), 0, s, p);
      hipLaunchKernelGGL((evict_hist<2, 8>), grid, dim3(EV_THREADS), 0, s, p);
    }
  }
  if (p.nb > 0) {
    if (per == 4)
      hipLaunchKernelGGL(evict_count<4>, grid, dim3(EV_THREADS), 0, s, p);
    else
      hipLaunchKernelGGL(evict_count<8>, grid, dim3(EV_THREADS), 0, s, p);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const bool fused = p.Hkv <= FUSED_HEADS && (int64_t)p.Hkv * p.nb <= FUSED_ENTRIES;
  const dim3 wgrid = p.nb > 0 ? grid : dim3(1, 1);  // no keys: one block writes the (zero) offsets
  if (fused) {
    if (per == 4)
      hipLaunchKernelGGL(evict_write_fused<4>, wgrid, dim3(EV_THREADS), 0, s, p);
    else
      hipLaunchKernelGGL(evict_write_fused<8>, wgrid, dim3(EV_THREADS), 0, s, p);
  } else {
    hipLaunchKernelGGL(evict_scan, dim3(p.Hkv), dim3(EV_THREADS), 0, s, p);
    if (per == 4)
      hipLaunchKernelGGL(evict_write<4>, wgrid, dim3(EV_THREADS), 0, s, p);
    else
      hipLaunchKernelGGL(evict_write<8>, wgrid, dim3(EV_THREADS), 0, s, p);
  }
  const int64_t cap_rows = e.capacity;
  if (cap_rows > 0 && p.nb > 0) {
    const int64_t gblocks = (cap_rows + GROWS - 1) / GROWS;
    if (p.D == 128)
      hipLaunchKernelGGL(evict_gather<128>, dim3((unsigned)gblocks), dim3(GT), 0, s, p);
    else
      hipLaunchKernelGGL(evict_gather<64>, dim3((unsigned)gblocks), dim3(GT), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvs
