// Attention forward that returns the output rows and the normalisers:
//   O_j = sum_{i visible to j} a_ji v_i,  LSE_j = ln sum_{i visible to j} exp(l_ji),
//   a_ji = exp(l_ji - LSE_j), l_ji = scale * q_j . k_i.
// O_j is the per-head sum that enters the residual update (Eq. 2 of
// "KVzap: Fast, Adaptive, and Faithful KV Cache Pruning", §3.2, before W_O);
// LSE_j is what the transposed scoring pass reuses ("[논문리뷰] KVpop ..." §1).
// Visibility is the LSE pass's: REPEAT (context keys, then the self keys of
// the query's chunk up to its position) or CAUSAL.
//
// Layout of the work:
//   * a workgroup has 12 waves (3 per SIMD, one workgroup per CU), each
//     owning one query subtile (32 positions of one query head); subtiles are
//     ordered position-major, so the heads of a GQA group at the same
//     positions share every key and value tile (384 queries per tile);
//   * key and value tiles of 32 rows go through a 2-stage LDS ring of 4
//     tiles per stage: one barrier per 128 keys, the next stage's tiles
//     loaded while this stage's are used. Each tile's loads are issued before
//     the S of the tile in use and stored after its PV product, so only one
//     tile's loads sit in registers and the whole tile's work covers their
//     latency; the matrix work of one wave overlaps the other waves'
//     exponentials (no second set of S accumulators, which would not fit 3
//     waves per SIMD);
//   * key tiles of 32 rows go through LDS as the A operand of S = K Q^T (keys
//     as rows, queries as columns), exactly as in the LSE pass; each lane's
//     16 accumulators are 16 keys of one query;
//   * the exponentials P (against a per-query offset) are packed to bf16 and
//     are, without any data movement, the B operand of O^T += V^T P^T: the
//     16 keys a lane holds are the 2 x 8 contraction elements it supplies;
//   * value tiles are stored transposed in LDS (rows = head dimension, 80-byte
//     rows), with the keys of each row in the order the P operand takes them
//     (key groups of 4 in the order 0 2 1 3 4 6 5 7), so the A operand V^T of
//     one MFMA is one 16-byte read;
//   * O^T accumulates in registers: a lane holds one query and D/2 of its
//     output elements; it never leaves the chip until the final scaling by
//     1 / sum P, which is per lane.
//   * The offset o (exp2 domain) is shared by the two half-waves of a query,
//     because their P values meet in one MFMA. It moves lazily: a tile is
//     exponentiated against the stored o, and only when some lane's partial
//     sum grows large (or overflows, on the first visible tile) does the
//     whole wave raise o to its new row maxima and rescale l and O.
#include "common.hpp"
#include "internal.hpp"

// Offsets are stored values used as is; no implicit contraction, so an
// unchanged offset rescales by exactly 1.
#pragma clang fp contract(off)

namespace kvs {
namespace {

struct AttnParams {
  const uint16_t* Q;
  const uint16_t* K;       // context keys (REPEAT) or the sequence's keys (CAUSAL)
  const uint16_t* Kself;   // REPEAT self keys
  const uint16_t* V;       // values of K (same strides as K)
  const uint16_t* Vself;   // values of Kself (same strides as Kself)
  uint16_t* O;             // [Hq, n_q, D], strides of Q
  float* lse;              // [Hq, n_q]
  int64_t q_hs, q_ts, k_hs, k_ts, ks_hs, ks_ts;
  int64_t n_ctx, n_q, chunk;
  int Hkv, G;
  int n_sub;  // subtiles per KV head = ceil(n_q / 32) * G
  float scale;
};

constexpr int AT_WAVES = 12;
constexpr int NSTAGE = 2;  // LDS ring stages: the one in use and the one being filled
constexpr int TPS = 4;     // 32-key tiles per stage
constexpr int AT_THREADS = AT_WAVES * WAVE;
constexpr float AT_LAZY = 1048576.0f;  // 2^20: raise the offset when a lane's tile sum exceeds this

template <int D>
struct ATile {
  static constexpr int STEPS = D / 16;         // k-steps of the QK^T chain
  static constexpr int K_STRIDE = D * 2 + 16;  // padded key rows, bytes
  static constexpr int K_BYTES = 32 * K_STRIDE;
  static constexpr int VT_STRIDE = 80;         // transposed value rows: 32 keys * 2 B + 16 B pad
  static constexpr int V_BYTES = D * VT_STRIDE;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int DB = D / 32;            // output row blocks of O^T
  static constexpr int CHUNKS = 32 * D / 8;    // 16-byte pieces per tile, per tensor
  static constexpr int CPR = D / 8;            // pieces per row
  static constexpr int KPT = (CHUNKS + AT_THREADS - 1) / AT_THREADS;  // K pieces per thread
  static constexpr int VUNITS = 16 * CPR;      // (key pair, piece) units of a V tile
  static constexpr int VPT = (VUNITS + AT_THREADS - 1) / AT_THREADS;  // V units per thread
  static constexpr int NPRE = KPT + 2 * VPT;
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 pack_bf16(const f32x16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (__bf16)x[base + t];
  return r;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(AT_THREADS, 1) void attn_kernel(AttnParams p) {
  using T = ATile<D>;
  __shared__ __attribute__((aligned(16))) char s_tile[NSTAGE][TPS][T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  const int b = blockIdx.x;
  const int h = b % p.Hkv;
  // Causal work grows with position: dispatch the last positions (longest
  // workgroups) first, so the short ones fill in at the end.
  const int nbx = (p.n_sub + AT_WAVES - 1) / AT_WAVES;
  const int bx = CAUSAL ? nbx - 1 - b / p.Hkv : b / p.Hkv;
  const int u_lo = bx * AT_WAVES;
  const int u_hi = min(u_lo + AT_WAVES, p.n_sub) - 1;

  const int64_t pos_lo = (int64_t)(u_lo / p.G) * 32;
  const int64_t pos_end = min((int64_t)(u_hi / p.G) * 32 + 32, p.n_q);
  const int64_t chunk = CAUSAL ? 1 : p.chunk;
  const int64_t self_lo = CAUSAL ? 0 : (pos_lo / chunk) * chunk;
  const int n_ctx_tiles = CAUSAL ? 0 : (int)((p.n_ctx + 31) / 32);
  const int n_tiles = n_ctx_tiles + (int)((pos_end - self_lo + 31) / 32);

  // ---- this wave's subtile: resident queries (B operands of S = K Q^T)
  const int u = u_lo + wave;
  const bool sub_ok = u < p.n_sub;
  const int g = h * p.G + (sub_ok ? u % p.G : 0);
  const int pj = sub_ok ? (u / p.G) * 32 : 0;  // first position of the subtile
  bf16x8 qreg[T::STEPS];
  {
    const int64_t j = min((int64_t)pj + col, p.n_q - 1);
    const uint16_t* qp = p.Q + (int64_t)g * p.q_hs + j * p.q_ts + half * (D / 2);
#pragma unroll
    for (int s = 0; s < T::STEPS; ++s) {
      u32x4 v = ld16(qp + 8 * s);
      pin(v);
      qreg[s] = as_bf16x8(v);
    }
  }

  // ---- tile loads: K and V rows through buffer resources that cover only
  // the rows a segment has (rows past the end read as zero and are masked)
  const int n_ctx_s = (int)p.n_ctx, pos_end_s = (int)pos_end, self_lo_s = (int)self_lo;
  const int k_ts_s = (int)p.k_ts, ks_ts_s = CAUSAL ? k_ts_s : (int)p.ks_ts;
  const int64_t kh = (int64_t)h * p.k_hs, ksh = CAUSAL ? kh : (int64_t)h * p.ks_hs;
  // Every thread loads up to KPT 16-byte pieces of the K tile and up to VPT
  // units of the V tile (one 16-byte piece of keys 2m and 2m+1), which it
  // stores transposed as 32-bit key pairs.
  u32x4 pre[T::NPRE];
  auto load_tile = [&](int tt) {
    const bool ctx = tt < n_ctx_tiles;
    const int k0 = ctx ? tt * 32 : self_lo_s + (tt - n_ctx_tiles) * 32;
    const int kend = ctx ? n_ctx_s : pos_end_s;
    const int ts = ctx ? k_ts_s : ks_ts_s;
    const int rows = min(kend - k0, 32);
    const int64_t off = (ctx ? kh : ksh) + (int64_t)k0 * ts;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc((ctx || CAUSAL ? p.K : p.Kself) + off, rows * ts * 2);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc((ctx || CAUSAL ? p.V : p.Vself) + off, rows * ts * 2);
#pragma unroll
    for (int c = 0; c < T::KPT; ++c) {
      const int idx = tid + c * AT_THREADS;
      if (idx < T::CHUNKS) pre[c] = buf_ld16(rk, (idx / T::CPR) * ts * 2 + (idx % T::CPR) * 16);
    }
#pragma unroll
    for (int u = 0; u < T::VPT; ++u) {
      const int unit = tid + u * AT_THREADS;
      if (unit < T::VUNITS) {
        const int m = unit & 15, part = unit >> 4;
        pre[T::KPT + 2 * u] = buf_ld16(rv, (2 * m) * ts * 2 + part * 16);
        pre[T::KPT + 2 * u + 1] = buf_ld16(rv, (2 * m + 1) * ts * 2 + part * 16);
      }
    }
  };
  // K rows as they are (padded). V transposed: elements (2m, d) and (2m+1, d)
  // form one 32-bit word of value row d at its pair slot (80-byte rows, so an
  // MFMA operand is one aligned 16-byte read); a half-wave's stores cover 16
  // pair slots in two row groups, walked so that they hit distinct banks.
  auto store_tile = [&](char* st) {
#pragma unroll
    for (int c = 0; c < T::KPT; ++c) {
      const int idx = tid + c * AT_THREADS;
      if (idx < T::CHUNKS) *reinterpret_cast<u32x4*>(st + (idx / T::CPR) * T::K_STRIDE + (idx % T::CPR) * 16) = pre[c];
    }
#pragma unroll
    for (int u = 0; u < T::VPT; ++u) {
      const int unit = tid + u * AT_THREADS;
      if (unit < T::VUNITS) {
        const int m = unit & 15, part = unit >> 4;
        // key pair m sits at pair slot 2 * grp(m / 2) + m % 2, grp swapping
        // key groups 1, 2 and 5, 6 (of 4 keys), so the 8 keys a lane feeds one
        // MFMA are 16 contiguous bytes
        const int g4 = m >> 1, sg = (g4 == 1 || g4 == 5) ? g4 + 1 : ((g4 == 2 || g4 == 6) ? g4 - 1 : g4);
        char* vt = st + T::K_BYTES + (8 * part) * T::VT_STRIDE + 4 * (2 * sg + (m & 1));
        // odd pieces walk their rows from row 4 on (data word e goes to rows 2e,
        // 2e+1 either way), so the two pieces of a half-wave store rows 4 or 12
        // apart: 16 banks apart on 32 banks, 16 or 48 on 64
        const bool odd = part & 1;
        u32x4 a0 = pre[T::KPT + 2 * u], a1 = pre[T::KPT + 2 * u + 1];
        if (odd) {
          a0 = u32x4{a0[2], a0[3], a0[0], a0[1]};
          a1 = u32x4{a1[2], a1[3], a1[0], a1[1]};
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          char* vr = vt + (((2 * w) + (odd ? 4 : 0)) & 7) * T::VT_STRIDE;
          *reinterpret_cast<uint32_t*>(vr) = __builtin_amdgcn_perm(a1[w], a0[w], 0x05040100u);
          *reinterpret_cast<uint32_t*>(vr + T::VT_STRIDE) = __builtin_amdgcn_perm(a1[w], a0[w], 0x07060302u);
        }
      }
    }
  };

  // ---- running state: shared offset o (exp2 domain), this lane's partial
  // sum l over the keys its half holds, and O^T
  const float c2 = p.scale * LOG2E;
  float o_run = -3.402823466e38f, l_run = 0.f;
  f32x16 oacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) oacc[db] = f32x16{};
  const int lane_j = pj + col;
  const int lane_cs = CAUSAL ? 0 : (int)((lane_j / chunk) * chunk);
  const int sub_cs_first = CAUSAL ? 0 : (int)((pj / chunk) * chunk);
  const int sub_cs_last = CAUSAL ? 0 : (int)(((pj + 31) / chunk) * chunk);
  const int n_ctx_full_tiles = CAUSAL ? 0 : n_ctx_s / 32;

  auto exp_tile = [&](const f32x16& x, float o, f32x16& e) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e[r] = fast_exp2(__builtin_fmaf(x[r], c2, -o));
      s += e[r];
    }
    return s;
  };

  // S = K Q^T of one tile (keys from LDS stage buf), raw dot products.
  auto qk = [&](const char* st) {
    const char* krow = st + col * T::K_STRIDE + half * D;
    bf16x8 a[T::STEPS];
#pragma unroll
    for (int s = 0; s < T::STEPS; ++s) a[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 16 * s));
    f32x16 x = mfma32(a[0], qreg[0], f32x16{});
#pragma unroll
    for (int s = 1; s < T::STEPS; ++s) x = mfma32(a[s], qreg[s], x);
    return x;
  };

  // Mask, exponentiate against the lazy offset, and O^T += V^T P^T for one
  // tile whose S is x (values from LDS stage buf).
  auto softmax_pv = [&](f32x16 x, const char* st, bool masked, int k0, int kend, bool is_ctx) {
    if (masked) {
      const int kb = k0 + 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + 8 * (r >> 2) + (r & 3);
        const bool vis = is_ctx ? (key < kend) : (key <= lane_j && key >= lane_cs);
        x[r] = vis ? x[r] : -INFINITY;
      }
    }
    f32x16 e;
    float sum = exp_tile(x, o_run, e);
    // wave-uniform: raise the shared offset when any lane's sum is large
    if (__builtin_amdgcn_ballot_w64(!(sum <= AT_LAZY))) {
      float tm = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tm = fmaxf(tm, x[r]);
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const float o_new = fmaxf(o_run, tm * c2);
      const float f = fast_exp2(o_run - o_new);
      l_run *= f;
#pragma unroll
      for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= f;
      o_run = o_new;
      sum = exp_tile(x, o_run, e);
    }
    l_run += sum;
    const bf16x8 pb0 = pack_bf16(e, 0), pb1 = pack_bf16(e, 8);
    const char* vrow = st + T::K_BYTES + col * T::VT_STRIDE + half * 16;
    // the PV MFMAs at raised wave priority: a wave whose exponentials are
    // done hands its matrix work to the core ahead of the SIMD's other waves,
    // which keep the VALU busy meanwhile
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
      const char* vr = vrow + 32 * db * T::VT_STRIDE;
      const bf16x8 v0 = as_bf16x8(*reinterpret_cast<const u32x4*>(vr));
      const bf16x8 v1 = as_bf16x8(*reinterpret_cast<const u32x4*>(vr + 32));
      oacc[db] = mfma32(v0, pb0, oacc[db]);
      oacc[db] = mfma32(v1, pb1, oacc[db]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // What this wave does with tile tt: skip it, or run it masked or not.
  struct TileInfo {
    int k0, kend;
    bool is_ctx, run, masked;
  };
  auto tile_info = [&](int tt) {
    TileInfo ti;
    ti.is_ctx = tt < n_ctx_tiles;
    ti.k0 = ti.is_ctx ? tt * 32 : self_lo_s + (tt - n_ctx_tiles) * 32;
    ti.kend = ti.is_ctx ? n_ctx_s : pos_end_s;
    if (tt < n_ctx_full_tiles) {
      ti.run = true;
      ti.masked = false;
    } else if (ti.is_ctx) {
      ti.run = true;
      ti.masked = !(ti.k0 + 31 < ti.kend);
    } else {
      ti.run = !((ti.k0 > pj + 31) || (ti.k0 + 31 < sub_cs_first));
      ti.masked = !((ti.k0 + 31 <= pj) && (ti.k0 >= sub_cs_last) && (ti.k0 + 31 < ti.kend));
    }
    ti.run = ti.run && sub_ok;
    return ti;
  };

  // Tiles TPS*i .. TPS*i + TPS-1 live in stage i % NSTAGE, stored NSTAGE-1
  // iterations ahead; one barrier per stage.
  constexpr int AHEAD = NSTAGE - 1;
  const int n_iters = (n_tiles + TPS - 1) / TPS;
  for (int t = 0; t < AHEAD * TPS && t < n_tiles; ++t) {
    load_tile(t);
    store_tile(s_tile[(t / TPS) % NSTAGE][t % TPS]);
  }
  __syncthreads();
  for (int it = 0; it < n_iters; ++it) {
#pragma unroll 1
    for (int sub = 0; sub < TPS; ++sub) {
      const int tt = TPS * it + sub;
      const int tl = TPS * (it + AHEAD) + sub;  // loaded now, into the stage of iteration it - 1
      if (tl < n_tiles) load_tile(tl);
      const TileInfo cur = tile_info(tt);
      const bool run = tt < n_tiles && cur.run;
      const char* st = s_tile[it % NSTAGE][sub];
      f32x16 x = f32x16{};
      if (run) x = qk(st);
      if (run) softmax_pv(x, st, cur.masked, cur.k0, cur.kend, cur.is_ctx);
      if (tl < n_tiles) store_tile(s_tile[(it + AHEAD) % NSTAGE][sub]);
    }
    __syncthreads();
  }

  // ---- finish: merge the halves' partial sums, write LSE and O = O^T / l
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const int64_t j = (int64_t)lane_j;
  if (sub_ok && j < p.n_q) {
    if (half == 0) p.lse[(int64_t)g * p.n_q + j] = (o_run + __log2f(l_tot)) * LN2;
    const float inv = 1.0f / l_tot;
    uint16_t* orow = p.O + (int64_t)g * p.q_hs + j * p.q_ts;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (__bf16)(oacc[db][4 * q4 + t] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * q4 + 4 * half) = v;
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t run(const AttnParams& p, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((attn_kernel<D, CAUSAL>), dim3(nblocks), dim3(AT_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const kvs_attn_desc& d, const uint16_t* Q, const uint16_t* K, const uint16_t* Kself,
                       const uint16_t* V, const uint16_t* Vself, uint16_t* O, float* lse, hipStream_t s) {
  if (d.n_q == 0) return hipSuccess;
  AttnParams p{};
  p.Q = Q; p.K = K; p.Kself = Kself; p.V = V; p.Vself = Vself; p.O = O; p.lse = lse;
  p.q_hs = d.q_head_stride; p.q_ts = d.q_tok_stride;
  p.k_hs = d.k_head_stride; p.k_ts = d.k_tok_stride;
  p.ks_hs = d.ks_head_stride; p.ks_ts = d.ks_tok_stride;
  p.n_ctx = d.n_ctx; p.n_q = d.n_q; p.chunk = d.chunk;
  p.Hkv = d.n_kvheads; p.G = d.n_qheads / d.n_kvheads; p.scale = d.scale;
  const int64_t n_sub = ((d.n_q + 31) / 32) * p.G;
  p.n_sub = (int)n_sub;
  const int64_t nblocks = ((n_sub + AT_WAVES - 1) / AT_WAVES) * p.Hkv;
  const bool causal = d.mask == KVS_MASK_CAUSAL;
  if (d.head_dim == 128) return causal ? run<128, true>(p, (int)nblocks, s) : run<128, false>(p, (int)nblocks, s);
  return causal ? run<64, true>(p, (int)nblocks, s) : run<64, false>(p, (int)nblocks, s);
}

}  // namespace kvs
