// LSE pass: lse_j = ln sum_{i visible to j} exp(scale * q_j . k_i) for every
// query row, the normaliser an attention kernel returns with its output
// ("[논문리뷰] KVpop ..." §1, transposed-attention pass), here without the PV
// product.
//
// Visibility:
//   REPEAT - the teacher-forced repeat of the context ("KVzap: Fast, Adaptive,
//            and Faithful KV Cache Pruning" §3.1; KVzip review, "Methods" and
//            "Methods: technical-details"): query j of chunk c sees all
//            context keys and the self keys of chunk c up to position j.
//   CAUSAL - key i is visible to query j iff i <= j.
//
// Layout of the work:
//   * a workgroup (4 waves) serves 8 query subtiles of one KV head; a subtile
//     is 32 consecutive positions of one query head, and subtiles are ordered
//     position-major then head, so the G heads of a GQA group at the same
//     positions sit in the same workgroup and share every key tile;
//   * each wave keeps its 2 subtiles in VGPRs as MFMA B operands (queries are
//     columns); key tiles of 32 rows stream through a double-buffered LDS
//     stage and are the A operands (keys are rows), so each lane's 16
//     accumulator registers are 16 keys of one query: the softmax reduction
//     is in-register, and the two half-waves merge once at the end;
//   * online softmax in the exp2 domain on raw dot products: a running sum l
//     of exp2(q.k * scale * log2 e - o) against an offset o that follows the
//     running max lazily (raised only when a tile's sum would grow large);
//   * tiles a subtile cannot see are skipped; only tiles cut by the causal
//     diagonal, a chunk edge or the end of the keys are masked per element.
#include "common.hpp"
#include "internal.hpp"

// No implicit a*b+c contraction in this file: the running-sum rescale relies
// on exp2(o_old - o_new) being exactly 1 when the max is unchanged, which
// needs o = fl(m * c2) rounded once and then used as is. (Explicit fmaf
// calls still produce FMAs.)
#pragma clang fp contract(off)

namespace kvs {
namespace {

struct LseParams {
  const uint16_t* Q;
  const uint16_t* K;      // context keys (REPEAT) or the sequence's keys (CAUSAL)
  const uint16_t* Kself;  // REPEAT self keys
  float* lse;
  int64_t q_hs, q_ts, k_hs, k_ts, ks_hs, ks_ts;
  int64_t n_ctx, n_q, chunk;
  int Hkv, G;
  int n_sub;  // subtiles per KV head = ceil(n_q / 32) * G
  float scale;
};

template <int D>
struct KTile {
  static constexpr int STEPS = D / 16;
  static constexpr int LDS_STRIDE = D * 2 + 16;
  static constexpr int CHUNKS = 32 * D / 8;
  static constexpr int BYTES = 32 * LDS_STRIDE;
};

constexpr int LSE_WAVES = 4;
constexpr float LAZY_LIMIT = 1048576.0f;  // 2^20: raise the offset when a tile's sum exceeds this
constexpr int LSE_NQ = 2;
constexpr int SUB_PER_BLOCK = LSE_WAVES * LSE_NQ;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(LSE_WAVES * WAVE, 3) void lse_kernel(LseParams p) {
  using T = KTile<D>;
  constexpr int NTHREADS = LSE_WAVES * WAVE;
  static_assert(T::CHUNKS % NTHREADS == 0, "tile chunks must split evenly over the threads");
  constexpr int CPT = T::CHUNKS / NTHREADS;
  constexpr int CHUNKS_PER_ROW = D / 8;

  __shared__ __attribute__((aligned(16))) char s_k[2][T::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int half = lane >> 5;
  const int col = lane & 31;

  const int b = blockIdx.x;
  const int h = b % p.Hkv;
  // Causal work grows with position: dispatch the last positions (longest
  // workgroups) first, so the short ones fill in at the end.
  const int nbx = (p.n_sub + SUB_PER_BLOCK - 1) / SUB_PER_BLOCK;
  const int bx = CAUSAL ? nbx - 1 - b / p.Hkv : b / p.Hkv;
  const int u_lo = bx * SUB_PER_BLOCK;
  const int u_hi = min(u_lo + SUB_PER_BLOCK, p.n_sub) - 1;

  // positions served by the block
  const int64_t pos_lo = (int64_t)(u_lo / p.G) * 32;
  const int64_t pos_end = min((int64_t)(u_hi / p.G) * 32 + 32, p.n_q);
  const int64_t chunk = CAUSAL ? 1 : p.chunk;

  // key segments: REPEAT -> context keys [0, n_ctx) then self keys
  // [chunk start of pos_lo, pos_end); CAUSAL -> keys [0, pos_end)
  const int64_t self_lo = CAUSAL ? 0 : (pos_lo / chunk) * chunk;
  const int64_t n_ctx_tiles = CAUSAL ? 0 : (p.n_ctx + 31) / 32;
  const int64_t n_self_tiles = (pos_end - self_lo + 31) / 32;
  const int64_t n_tiles = n_ctx_tiles + n_self_tiles;

  // ---- this wave's subtiles: resident queries (B operands)
  int sub_g[LSE_NQ];
  int64_t sub_pos[LSE_NQ];
  bool sub_ok[LSE_NQ];
  bf16x8 qreg[LSE_NQ][T::STEPS];
#pragma unroll
  for (int q = 0; q < LSE_NQ; ++q) {
    const int u = u_lo + wave * LSE_NQ + q;
    sub_ok[q] = u < p.n_sub;
    sub_g[q] = h * p.G + (sub_ok[q] ? u % p.G : 0);
    sub_pos[q] = sub_ok[q] ? (int64_t)(u / p.G) * 32 : 0;
    // queries past the end load the last row; their results are never written
    const int64_t j = min(sub_pos[q] + col, p.n_q - 1);
    const uint16_t* qp = p.Q + (int64_t)sub_g[q] * p.q_hs + j * p.q_ts + half * (D / 2);
#pragma unroll
    for (int s = 0; s < T::STEPS; ++s) {
      u32x4 v = ld16(qp + 8 * s);
      pin(v);
      qreg[q][s] = as_bf16x8(v);
    }
  }

  // Key tiles come in through buffer loads. A tile's resource starts at its
  // first row and covers only the rows its segment has, so rows past the end
  // read as zero; every such row is masked (ctx: key >= n_ctx; self/causal:
  // key > j), so its value never counts. A thread loads the pieces of rows
  // rr0, rr0 + RSTEP, ...; each load's whole byte offset is in its per-lane
  // offset, because the range check does not include the scalar offset.
  // Token strides are at most 2^22 elements, so 32 rows span at most 2^28
  // bytes.
  const int rr0 = tid / CHUNKS_PER_ROW, p16 = (tid % CHUNKS_PER_ROW) * 16;
  constexpr int RSTEP = NTHREADS / CHUNKS_PER_ROW;
  // two register sets: tile t is loaded into set t % 2 two iterations before
  // its use (see the loop below)
  u32x4 preA[CPT], preB[CPT];
  // (32-bit positions and scalar compares: every position is below 2^30)
  const int n_ctx_tiles_s = (int)n_ctx_tiles, n_ctx_s = (int)p.n_ctx, pos_end_s = (int)pos_end;
  const int self_lo_s = (int)self_lo, k_ts_s = (int)p.k_ts;
  const int ks_ts_s = CAUSAL ? k_ts_s : (int)p.ks_ts;
  const uint16_t* const ctx_base = p.K + (int64_t)h * p.k_hs;
  const uint16_t* const self_base = CAUSAL ? ctx_base : p.Kself + (int64_t)h * p.ks_hs;
  auto load_tile = [&](int tt, u32x4 (&pre)[CPT]) {
    const bool ctx = tt < n_ctx_tiles_s;
    const int k0 = ctx ? tt * 32 : self_lo_s + (tt - n_ctx_tiles_s) * 32;
    const int kend = ctx ? n_ctx_s : pos_end_s;
    const int ts = ctx ? k_ts_s : ks_ts_s;
    const int rows = min(kend - k0, 32);
    const __amdgpu_buffer_rsrc_t r = tile_rsrc((ctx ? ctx_base : self_base) + (int64_t)k0 * ts, rows * ts * 2);
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      pre[c] = buf_ld16(r, (rr0 + c * RSTEP) * ts * 2 + p16);
  };
  auto store_tile = [&](int buf, const u32x4 (&pre)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NTHREADS;
      const int rr = idx / CHUNKS_PER_ROW, part = idx % CHUNKS_PER_ROW;
      *reinterpret_cast<u32x4*>(&s_k[buf][rr * T::LDS_STRIDE + part * 16]) = pre[c];
    }
  };

  // Running state per subtile column: the exp2-domain offset o that every
  // term of l was computed against, and l. The offset follows the running max
  // lazily: a tile is first exponentiated against the current offset, and only
  // when its partial sum gets large (> 2^20, or +inf on the first visible
  // tile, whose offset starts at -FLT_MAX) is the offset raised to
  // fl(tile max * c2), with l rescaled by exp2(o_old - o_new). Offsets are
  // stored values used as is, so no rounding drift builds up; masked logits
  // are -inf and contribute exp2(-inf) = 0 (never inf - inf).
  const float c2 = p.scale * LOG2E;
  float o_run[LSE_NQ], l_run[LSE_NQ];
  // Per-lane visibility constants (positions fit in 32 bits): this lane's
  // query position j and the start of its repeat chunk; per subtile the chunk
  // starts of its first and last query.
  int lane_j[LSE_NQ], lane_cs[LSE_NQ], sub_pj[LSE_NQ], sub_cs_first[LSE_NQ], sub_cs_last[LSE_NQ];
#pragma unroll
  for (int q = 0; q < LSE_NQ; ++q) {
    o_run[q] = -3.402823466e38f;
    l_run[q] = 0.f;
    sub_pj[q] = (int)sub_pos[q];
    lane_j[q] = sub_pj[q] + col;
    lane_cs[q] = CAUSAL ? 0 : (int)((lane_j[q] / chunk) * chunk);
    sub_cs_first[q] = CAUSAL ? 0 : (int)((sub_pj[q] / chunk) * chunk);
    sub_cs_last[q] = CAUSAL ? 0 : (int)(((sub_pj[q] + 31) / chunk) * chunk);
  }
  const int n_ctx_i = (int)p.n_ctx, pos_end_i = (int)pos_end, self_lo_i = (int)self_lo;
  const int n_ctx_tiles_i = (int)n_ctx_tiles, n_tiles_i = (int)n_tiles;
  const int n_ctx_full_tiles = CAUSAL ? 0 : n_ctx_i / 32;  // context tiles with no key past the end
  bool all_sub_ok = true;
#pragma unroll
  for (int q = 0; q < LSE_NQ; ++q) all_sub_ok = all_sub_ok && sub_ok[q];

  // sum over a tile's 16 logits of exp2(x * c2 - o) (masked logits are -inf)
  auto exp_sum = [&](const f32x16& x, float o) {
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = fast_exp2(__builtin_fmaf(x[r], c2, -o));
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) e[r] += e[r + w];
    return e[0];
  };
  // (rare) raise subtile q's offset to fl(tile max * c2), rescale its sum,
  // and return the tile's sum against the new offset
  auto raise_offset = [&](int q, const f32x16& x) {
    float tm = max3(x[0], x[1], x[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) tm = max3(tm, x[r], x[r + 1]);
    tm = fmaxf(tm, x[15]);
    const float o_new = fmaxf(o_run[q], tm * c2);
    l_run[q] *= fast_exp2(o_run[q] - o_new);
    o_run[q] = o_new;
    return exp_sum(x, o_new);
  };
  // Lazy online-softmax update of subtile q with one tile's logits x. See the
  // running-state comment above.
  auto softmax_update = [&](int q, f32x16& x) {
    float sum = exp_sum(x, o_run[q]);
    if (sum > LAZY_LIMIT) sum = raise_offset(q, x);
    l_run[q] += sum;
  };

  // General tile: partial context tiles and self / causal tiles. Subtiles
  // that see none of the tile skip it; tiles cut by the end of the keys, the
  // causal diagonal or a chunk edge are masked per element.
  auto tile_general = [&](int tt, const bf16x8 (&a)[T::STEPS]) {
    const bool is_ctx = tt < n_ctx_tiles_i;
    const int k0 = is_ctx ? tt * 32 : self_lo_i + (tt - n_ctx_tiles_i) * 32;
    const int kend = is_ctx ? n_ctx_i : pos_end_i;
#pragma unroll
    for (int q = 0; q < LSE_NQ; ++q) {
      const int pj = sub_pj[q];
      bool run, full;
      if (is_ctx) {
        run = sub_ok[q];
        full = k0 + 31 < kend;
      } else {
        run = sub_ok[q] && !((k0 > pj + 31) || (k0 + 31 < sub_cs_first[q]));
        full = (k0 + 31 <= pj) && (k0 >= sub_cs_last[q]) && (k0 + 31 < kend);
      }
      if (!run) continue;
      f32x16 x = mfma32(a[0], qreg[q][0], f32x16{});
#pragma unroll
      for (int s = 1; s < T::STEPS; ++s) x = mfma32(a[s], qreg[q][s], x);
      if (!full) {
        const int kb = k0 + 4 * half;
        const int j = lane_j[q], cs = lane_cs[q];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 8 * (r >> 2) + (r & 3);
          const bool vis = is_ctx ? (key < kend) : (key <= j && key >= cs);
          x[r] = vis ? x[r] : -INFINITY;
        }
      }
      softmax_update(q, x);
    }
  };

  // Tile t goes through register set t % 2 and LDS buffer t % 2: its loads
  // are issued at the start of iteration t - 2 and stored at the end of
  // iteration t - 1, into the buffer that held tile t - 2, which every wave
  // finished before the barrier ending iteration t - 2. So two iterations of
  // matrix and exponential work cover a tile's load latency.
  if (n_tiles_i > 0) {
    load_tile(0, preA);
    store_tile(0, preA);
  }
  if (n_tiles_i > 1) load_tile(1, preB);
  __syncthreads();

  // one iteration: tile tt from LDS; the loads of tile tt + 2 into pl (the
  // set that held tile tt); tile tt + 1 from ps into the other buffer
  auto step = [&](int tt, u32x4 (&pl)[CPT], const u32x4 (&ps)[CPT]) {
    const int cur = tt & 1;
    if (tt + 2 < n_tiles_i) load_tile(tt + 2, pl);

    bf16x8 a[T::STEPS];
    const char* krow = &s_k[cur][col * T::LDS_STRIDE + half * (D / 2) * 2];
#pragma unroll
    for (int s = 0; s < T::STEPS; ++s) a[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 16 * s));

    if (tt < n_ctx_full_tiles && all_sub_ok) {
      // Fast path (all full context tiles): every key visible to every query
      // of both subtiles; straight-line code, no masks.
      // The exponentials run at raised wave priority: a wave whose logits
      // are ready finishes its VALU work ahead of the SIMD's other waves and
      // returns to the matrix core sooner, while their MFMAs keep it busy.
      f32x16 acc[LSE_NQ];
#pragma unroll
      for (int q = 0; q < LSE_NQ; ++q) {
        acc[q] = mfma32(a[0], qreg[q][0], f32x16{});
#pragma unroll
        for (int s = 1; s < T::STEPS; ++s) acc[q] = mfma32(a[s], qreg[q][s], acc[q]);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int q = 0; q < LSE_NQ; ++q) softmax_update(q, acc[q]);
      __builtin_amdgcn_s_setprio(0);
    } else {
      tile_general(tt, a);
    }

    if (tt + 1 < n_tiles_i) store_tile(cur ^ 1, ps);
    __syncthreads();
  };
  // (unrolled by two so that each register set stays a fixed set of registers)
  for (int tt = 0; tt < n_tiles_i; tt += 2) {
    step(tt, preA, preB);
    if (tt + 1 < n_tiles_i) step(tt + 1, preB, preA);
  }

  // ---- merge half-waves, write natural-log LSE. The lane index is taken
  // afresh here, so the half and column computed before the loop need not
  // stay in registers across it.
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int half_e = lane_e >> 5, col_e = lane_e & 31;
#pragma unroll
  for (int q = 0; q < LSE_NQ; ++q) {
    const float o_o = __shfl_xor(o_run[q], 32);
    const float l_o = __shfl_xor(l_run[q], 32);
    const float Mc = fmaxf(o_run[q], o_o);
    const float L = (l_run[q] > 0.f ? l_run[q] * fast_exp2(o_run[q] - Mc) : 0.f) +
                    (l_o > 0.f ? l_o * fast_exp2(o_o - Mc) : 0.f);
    const int64_t j = sub_pos[q] + col_e;
    if (half_e == 0 && sub_ok[q] && j < p.n_q) p.lse[(int64_t)sub_g[q] * p.n_q + j] = (Mc + __log2f(L)) * LN2;
  }
}

// Small layers (fewer workgroups of the kernel above than CUs): the pass is
// then as long as one wave's walk over the keys, so the keys are split
// instead. A workgroup serves LSE_NQ subtiles (one 32-position block of one
// query head each); all LSE_WAVES waves hold both as B operands and walk
// every LSE_WAVES-th key tile, reading each tile's A operands straight from
// memory (buffer loads in the operand layout, one tile ahead), with no LDS
// staging and no barrier in the loop. The waves' running (offset, sum)
// pairs are merged through LDS at the end. Same softmax arithmetic and
// visibility rules as lse_kernel.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(LSE_WAVES * WAVE, 2) void lse_split_kernel(LseParams p) {
  using T = KTile<D>;
  __shared__ float s_o[LSE_WAVES][LSE_NQ][WAVE], s_l[LSE_WAVES][LSE_NQ][WAVE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  const int b = blockIdx.x;
  const int h = b % p.Hkv;
  const int nbx = (p.n_sub + LSE_NQ - 1) / LSE_NQ;
  const int bx = CAUSAL ? nbx - 1 - b / p.Hkv : b / p.Hkv;
  const int u_lo = bx * LSE_NQ;
  const int u_hi = min(u_lo + LSE_NQ, p.n_sub) - 1;

  const int64_t pos_lo = (int64_t)(u_lo / p.G) * 32;
  const int64_t pos_end = min((int64_t)(u_hi / p.G) * 32 + 32, p.n_q);
  const int64_t chunk = CAUSAL ? 1 : p.chunk;
  const int64_t self_lo = CAUSAL ? 0 : (pos_lo / chunk) * chunk;
  const int64_t n_ctx_tiles = CAUSAL ? 0 : (p.n_ctx + 31) / 32;
  const int64_t n_tiles = n_ctx_tiles + (pos_end - self_lo + 31) / 32;

  int sub_g[LSE_NQ];
  int64_t sub_pos[LSE_NQ];
  bool sub_ok[LSE_NQ];
  bf16x8 qreg[LSE_NQ][T::STEPS];
#pragma unroll
  for (int q = 0; q < LSE_NQ; ++q) {
    const int u = u_lo + q;
    sub_ok[q] = u < p.n_sub;
    sub_g[q] = h * p.G + (sub_ok[q] ? u % p.G : 0);
    sub_pos[q] = sub_ok[q] ? (int64_t)(u / p.G) * 32 : 0;
    const int64_t j = min(sub_pos[q] + col, p.n_q - 1);
    const uint16_t* qp = p.Q + (int64_t)sub_g[q] * p.q_hs + j * p.q_ts + half * (D / 2);
#pragma unroll
    for (int s = 0; s < T::STEPS; ++s) {
      u32x4 v = ld16(qp + 8 * s);
      pin(v);
      qreg[q][s] = as_bf16x8(v);
    }
  }

  // A operands of tile tt (lane: key row col of the tile, elements
  // [half*D/2 + 8s, +8) of step s) through a buffer resource over the rows
  // the segment has; rows past the end read as zero and are masked.
  const int n_ctx_tiles_s = (int)n_ctx_tiles, n_ctx_s = (int)p.n_ctx, pos_end_s = (int)pos_end;
  const int self_lo_s = (int)self_lo, k_ts_s = (int)p.k_ts;
  const int ks_ts_s = CAUSAL ? k_ts_s : (int)p.ks_ts;
  const uint16_t* const ctx_base = p.K + (int64_t)h * p.k_hs;
  const uint16_t* const self_base = CAUSAL ? ctx_base : p.Kself + (int64_t)h * p.ks_hs;
  auto load_a = [&](int tt, bf16x8 (&a)[T::STEPS]) {
    const bool ctx = tt < n_ctx_tiles_s;
    const int k0 = ctx ? tt * 32 : self_lo_s + (tt - n_ctx_tiles_s) * 32;
    const int kend = ctx ? n_ctx_s : pos_end_s;
    const int ts = ctx ? k_ts_s : ks_ts_s;
    const int rows = min(kend - k0, 32);
    const __amdgpu_buffer_rsrc_t r = tile_rsrc((ctx ? ctx_base : self_base) + (int64_t)k0 * ts, rows * ts * 2);
    const int off = col * ts * 2 + half * D;
#pragma unroll
    for (int s = 0; s < T::STEPS; ++s) a[s] = as_bf16x8(buf_ld16(r, off + 16 * s));
  };

  const float c2 = p.scale * LOG2E;
  float o_run[LSE_NQ], l_run[LSE_NQ];
  int lane_j[LSE_NQ], lane_cs[LSE_NQ], sub_pj[LSE_NQ], sub_cs_first[LSE_NQ], sub_cs_last[LSE_NQ];
#pragma unroll
  for (int q = 0; q < LSE_NQ; ++q) {
    o_run[q] = -3.402823466e38f;
    l_run[q] = 0.f;
    sub_pj[q] = (int)sub_pos[q];
    lane_j[q] = sub_pj[q] + col;
    lane_cs[q] = CAUSAL ? 0 : (int)((lane_j[q] / chunk) * chunk);
    sub_cs_first[q] = CAUSAL ? 0 : (int)((sub_pj[q] / chunk) * chunk);
    sub_cs_last[q] = CAUSAL ? 0 : (int)(((sub_pj[q] + 31) / chunk) * chunk);
  }
  auto exp_sum = [&](const f32x16& x, float o) {
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = fast_exp2(__builtin_fmaf(x[r], c2, -o));
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) e[r] += e[r + w];
    return e[0];
  };
  auto softmax_update = [&](int q, const f32x16& x) {
    float sum = exp_sum(x, o_run[q]);
    if (sum > LAZY_LIMIT) {
      float tm = max3(x[0], x[1], x[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) tm = max3(tm, x[r], x[r + 1]);
      tm = fmaxf(tm, x[15]);
      const float o_new = fmaxf(o_run[q], tm * c2);
      l_run[q] *= fast_exp2(o_run[q] - o_new);
      o_run[q] = o_new;
      sum = exp_sum(x, o_new);
    }
    l_run[q] += sum;
  };

  // this wave's tiles: wave, wave + LSE_WAVES, ...; the next one's operands
  // are in flight while the current one is processed
  const int n_tiles_i = (int)n_tiles;
  bf16x8 a_cur[T::STEPS], a_nxt[T::STEPS];
  if (wave < n_tiles_i) load_a(wave, a_cur);
  for (int tt = wave; tt < n_tiles_i; tt += LSE_WAVES) {
    if (tt + LSE_WAVES < n_tiles_i) load_a(tt + LSE_WAVES, a_nxt);
    const bool is_ctx = tt < n_ctx_tiles_s;
    const int k0 = is_ctx ? tt * 32 : self_lo_s + (tt - n_ctx_tiles_s) * 32;
    const int kend = is_ctx ? n_ctx_s : pos_end_s;
#pragma unroll
    for (int q = 0; q < LSE_NQ; ++q) {
      const int pj = sub_pj[q];
      bool run, full;
      if (is_ctx) {
        run = sub_ok[q];
        full = k0 + 31 < kend;
      } else {
        run = sub_ok[q] && !((k0 > pj + 31) || (k0 + 31 < sub_cs_first[q]));
        full = (k0 + 31 <= pj) && (k0 >= sub_cs_last[q]) && (k0 + 31 < kend);
      }
      if (!run) continue;
      f32x16 x = mfma32(a_cur[0], qreg[q][0], f32x16{});
#pragma unroll
      for (int s = 1; s < T::STEPS; ++s) x = mfma32(a_cur[s], qreg[q][s], x);
      if (!full) {
        const int kb = k0 + 4 * half;
        const int j = lane_j[q], cs = lane_cs[q];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 8 * (r >> 2) + (r & 3);
          const bool vis = is_ctx ? (key < kend) : (key <= j && key >= cs);
          x[r] = vis ? x[r] : -INFINITY;
        }
      }
      softmax_update(q, x);
    }
#pragma unroll
    for (int s = 0; s < T::STEPS; ++s) a_cur[s] = a_nxt[s];
  }

  // ---- merge the waves' and half-waves' (offset, sum) pairs, write natural-log LSE
#pragma unroll
  for (int q = 0; q < LSE_NQ; ++q) {
    s_o[wave][q][lane] = o_run[q];
    s_l[wave][q][lane] = l_run[q];
  }
  __syncthreads();
  if (wave == 0 && half == 0) {
#pragma unroll
    for (int q = 0; q < LSE_NQ; ++q) {
      float Mc = -3.402823466e38f;
#pragma unroll
      for (int w = 0; w < LSE_WAVES; ++w)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) Mc = fmaxf(Mc, s_o[w][q][col + 32 * hf]);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < LSE_WAVES; ++w)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const float l = s_l[w][q][col + 32 * hf];
          L += l > 0.f ? l * fast_exp2(s_o[w][q][col + 32 * hf] - Mc) : 0.f;
        }
      const int64_t j = sub_pos[q] + col;
      if (sub_ok[q] && j < p.n_q) p.lse[(int64_t)sub_g[q] * p.n_q + j] = (Mc + __log2f(L)) * LN2;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t run(const LseParams& p, int nblocks, bool split, hipStream_t s) {
  if (split)
    hipLaunchKernelGGL((lse_split_kernel<D, CAUSAL>), dim3(nblocks), dim3(LSE_WAVES * WAVE), 0, s, p);
  else
    hipLaunchKernelGGL((lse_kernel<D, CAUSAL>), dim3(nblocks), dim3(LSE_WAVES * WAVE), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse(const kvs_attn_desc& d, const uint16_t* Q, const uint16_t* K, const uint16_t* Kself,
                      float* lse, int num_cus, hipStream_t s) {
  if (d.n_q == 0) return hipSuccess;
  LseParams p{};
  p.Q = Q; p.K = K; p.Kself = Kself; p.lse = lse;
  p.q_hs = d.q_head_stride; p.q_ts = d.q_tok_stride;
  p.k_hs = d.k_head_stride; p.k_ts = d.k_tok_stride;
  p.ks_hs = d.ks_head_stride; p.ks_ts = d.ks_tok_stride;
  p.n_ctx = d.n_ctx; p.n_q = d.n_q; p.chunk = d.chunk;
  p.Hkv = d.n_kvheads; p.G = d.n_qheads / d.n_kvheads; p.scale = d.scale;
  const int64_t n_sub = ((d.n_q + 31) / 32) * p.G;
  p.n_sub = (int)n_sub;
  // fewer workgroups than CUs: split the keys over the waves instead
  const bool split = ((n_sub + SUB_PER_BLOCK - 1) / SUB_PER_BLOCK) * p.Hkv < num_cus;
  const int64_t per_block = split ? LSE_NQ : SUB_PER_BLOCK;
  const int64_t nblocks = ((n_sub + per_block - 1) / per_block) * p.Hkv;
  const bool causal = d.mask == KVS_MASK_CAUSAL;
  if (d.head_dim == 128)
    return causal ? run<128, true>(p, (int)nblocks, split, s) : run<128, false>(p, (int)nblocks, split, s);
  return causal ? run<64, true>(p, (int)nblocks, split, s) : run<64, false>(p, (int)nblocks, split, s);
}

}  // namespace kvs
