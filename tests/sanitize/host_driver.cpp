// Host-side checks of the C ABI and the input generator, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code only and
// run on a host without a GPU: every entry point is called with invalid
// descriptors (rejected before any HIP call), extreme sizes, NULL and
// misaligned pointers, and valid descriptors (which stop at KVS_ENODEV);
// the workspace-size queries at their limits; the status texts; and the
// generator's streams, normals and bf16 rounding. Exit status 0 = every
// expectation met (the sanitizers abort on their own findings).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "kvscore.h"

extern "C" {
uint64_t synth_stream_key(uint64_t seed, uint64_t stream);
void synth_u64(uint64_t key, uint64_t first, int64_t count, uint64_t* out);
void synth_normal_f32(uint64_t key, uint64_t first, int64_t count, double mean, double std, float* out);
void synth_normal_f64(uint64_t key, uint64_t first, int64_t count, double mean, double std, double* out);
void synth_f32_to_bf16(const float* in, int64_t count, uint16_t* out);
void synth_normal_bf16(uint64_t key, uint64_t first, int64_t count, double mean, double std, uint16_t* out);
}

static int g_fail = 0;
#define EXPECT(cond, ...)                                    \
  do {                                                       \
    if (!(cond)) {                                           \
      std::fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                     \
      std::fprintf(stderr, " [%s]\n", kvs_last_error());     \
      ++g_fail;                                              \
    }                                                        \
  } while (0)

// Distinct 16-byte-aligned stand-in addresses: never dereferenced (every call
// here is rejected or stops at the device check).
static void* fake(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t)0x100000 + 0x1000 * i); }

static kvs_attn_desc attn(int Hq = 8, int Hkv = 2, int D = 128, int64_t n_ctx = 300, int64_t n_q = 64) {
  kvs_attn_desc d;
  std::memset(&d, 0, sizeof d);
  d.n_qheads = Hq; d.n_kvheads = Hkv; d.head_dim = D; d.mask = KVS_MASK_REPEAT;
  d.n_ctx = n_ctx; d.n_q = n_q; d.chunk = 64;
  auto rows = [](int64_t n) { return n > ((int64_t)1 << 30) || n < 0 ? ((int64_t)1 << 30) : n; };
  d.q_head_stride = rows(n_q) * D; d.q_tok_stride = D;
  d.k_head_stride = rows(n_ctx) * D; d.k_tok_stride = D;
  d.ks_head_stride = rows(n_q) * D; d.ks_tok_stride = D;
  d.scale = 0.088f;
  return d;
}

static kvs_evict_desc evict(int Hkv = 2, int64_t n = 1000, int64_t k = 100, int64_t w = 32) {
  kvs_evict_desc e;
  std::memset(&e, 0, sizeof e);
  e.n_kvheads = Hkv; e.head_dim = 128; e.n_tok = n; e.k = k; e.tau = 0.f; e.scope = KVS_SCOPE_HEAD;
  e.window = w; e.capacity = Hkv * (w + k);
  e.kv_head_stride = n * 128; e.kv_tok_stride = 128; e.score_head_stride = n;
  return e;
}

static void attn_calls() {
  auto* Q = static_cast<const kvs_bf16*>(fake(1));
  auto* K = static_cast<const kvs_bf16*>(fake(2));
  auto* Ks = static_cast<const kvs_bf16*>(fake(3));
  auto* out = static_cast<float*>(fake(4));
  const kvs_attn_desc good = attn();
  EXPECT(kvscore_lse(&good, Q, K, Ks, out, nullptr) == KVS_ENODEV, "valid lse");
  EXPECT(kvscore_lse(nullptr, Q, K, Ks, out, nullptr) == KVS_EINVAL, "null desc");
  struct Bad { kvs_attn_desc d; int code; } bad[] = {
      {attn(8, 3), KVS_EINVAL}, {attn(8, 0), KVS_EINVAL}, {attn(8, 2, 96), KVS_EUNSUPPORTED},
      {attn(8, 2, 128, -1), KVS_EINVAL}, {attn(8, 2, 128, (int64_t)1 << 31), KVS_EUNSUPPORTED},
      {attn(8, 2, 128, 300, INT64_MAX), KVS_EUNSUPPORTED},
  };
  for (auto& b : bad) EXPECT(kvscore_lse(&b.d, Q, K, Ks, out, nullptr) == b.code, "bad lse desc");
  kvs_attn_desc d = good;
  d.q_tok_stride = 130; EXPECT(kvscore_lse(&d, Q, K, Ks, out, nullptr) == KVS_EUNSUPPORTED, "stride");
  d = good; d.k_tok_stride = INT64_MAX - 7; EXPECT(kvscore_lse(&d, Q, K, Ks, out, nullptr) == KVS_EUNSUPPORTED, "huge stride");
  d = good; d.scale = NAN; EXPECT(kvscore_lse(&d, Q, K, Ks, out, nullptr) == KVS_EINVAL, "nan scale");
  d = good; d.scale = INFINITY; EXPECT(kvscore_lse(&d, Q, K, Ks, out, nullptr) == KVS_EINVAL, "inf scale");
  d = good; d.chunk = 0; EXPECT(kvscore_lse(&d, Q, K, Ks, out, nullptr) == KVS_EINVAL, "chunk");
  d = good; d.reserved = 1; EXPECT(kvscore_lse(&d, Q, K, Ks, out, nullptr) == KVS_EINVAL, "reserved");
  d = good; d.mask = 9; EXPECT(kvscore_lse(&d, Q, K, Ks, out, nullptr) == KVS_EINVAL, "mask");
  EXPECT(kvscore_lse(&good, Q, K, nullptr, out, nullptr) == KVS_EINVAL, "null Kself");
  EXPECT(kvscore_lse(&good, reinterpret_cast<const kvs_bf16*>(0x100002), K, Ks, out, nullptr) == KVS_EUNSUPPORTED,
         "misaligned Q");
  // max / future mass / attention
  EXPECT(kvscore_max(&good, Q, K, out, nullptr, nullptr, out, 0, nullptr) == KVS_ENODEV, "valid max");
  EXPECT(kvscore_max(&good, Q, K, out, nullptr, nullptr, out, 2, nullptr) == KVS_EINVAL, "accumulate 2");
  kvs_attn_desc c = attn(8, 2, 128, 64, 64);
  c.mask = KVS_MASK_CAUSAL;
  for (int64_t w : {(int64_t)0, (int64_t)8, (int64_t)1 << 40, INT64_MAX})
    EXPECT(kvscore_futuremass(&c, Q, K, out, w, nullptr, nullptr, out, nullptr) == KVS_ENODEV, "valid futuremass");
  EXPECT(kvscore_futuremass(&c, Q, K, out, -1, nullptr, nullptr, out, nullptr) == KVS_EINVAL, "negative window");
  EXPECT(kvscore_futuremass(&good, Q, K, out, 8, nullptr, nullptr, out, nullptr) == KVS_EINVAL, "repeat futuremass");
  EXPECT(kvscore_attention(&good, Q, K, Ks, K, Ks, const_cast<kvs_bf16*>(Q), out, nullptr) == KVS_ENODEV,
         "valid attention");
  EXPECT(kvscore_attention(&good, Q, K, Ks, nullptr, Ks, const_cast<kvs_bf16*>(Q), out, nullptr) == KVS_EINVAL,
         "attention without V");
  // zero-length layers
  kvs_attn_desc z = attn(8, 2, 128, 0, 0);
  EXPECT(kvscore_lse(&z, nullptr, nullptr, nullptr, nullptr, nullptr) == KVS_ENODEV, "empty lse");
}

static void vnorm_calls() {
  kvs_vnorm_desc d;
  std::memset(&d, 0, sizeof d);
  d.n_kvheads = 2; d.head_dim = 128; d.n_tok = 100; d.d_model = 512;
  d.v_head_stride = 100 * 128; d.v_tok_stride = 128; d.wo_row_stride = 256;
  auto* V = static_cast<const kvs_bf16*>(fake(5));
  auto* W = static_cast<const kvs_bf16*>(fake(6));
  auto* out = static_cast<float*>(fake(7));
  EXPECT(kvscore_vnorm(&d, V, W, out, nullptr) == KVS_ENODEV, "valid vnorm");
  kvs_vnorm_desc b = d; b.wo_row_stride = 128; EXPECT(kvscore_vnorm(&b, V, W, out, nullptr) == KVS_EINVAL, "wo stride");
  b = d; b.n_kvheads = 70000; EXPECT(kvscore_vnorm(&b, V, W, out, nullptr) == KVS_EINVAL, "heads");
  b = d; b.n_tok = INT64_MAX; EXPECT(kvscore_vnorm(&b, V, W, out, nullptr) == KVS_EUNSUPPORTED, "tokens");
}

static void decode_calls() {
  kvs_decode_desc d;
  std::memset(&d, 0, sizeof d);
  d.n_qheads = 8; d.n_kvheads = 2; d.head_dim = 128; d.n_q = 1;
  d.q_head_stride = 128; d.q_tok_stride = 128; d.capacity = 5000; d.scale = 0.088f;
  const size_t ws = kvscore_decode_workspace_bytes(&d);
  EXPECT(ws > 0, "decode workspace");
  auto* Q = static_cast<const kvs_bf16*>(fake(8));
  auto* K = static_cast<const kvs_bf16*>(fake(9));
  auto* offs = static_cast<const int64_t*>(fake(10));
  auto* O = static_cast<kvs_bf16*>(fake(11));
  auto* lse = static_cast<float*>(fake(12));
  EXPECT(kvscore_decode(&d, Q, K, K, offs, O, lse, fake(13), ws, nullptr) == KVS_ENODEV, "valid decode");
  EXPECT(kvscore_decode(&d, Q, K, K, offs, O, lse, fake(13), ws - 1, nullptr) == KVS_EWORKSPACE, "small ws");
  kvs_decode_desc big = d;
  big.capacity = (int64_t)1 << 36;
  big.n_qheads = 65535; big.n_kvheads = 1;
  (void)kvscore_decode_workspace_bytes(&big);  // the size at the limits must not overflow silently
  big.n_q = 2; EXPECT(kvscore_decode_workspace_bytes(&big) == 0, "n_qheads * n_q above the limit");
  kvs_decode_desc b = d; b.head_stride_rows = 3000;
  EXPECT(kvscore_decode(&b, Q, K, K, offs, O, lse, fake(13), ws, nullptr) == KVS_EINVAL, "head regions");
}

static void evict_calls() {
  auto* s = static_cast<const float*>(fake(14));
  auto* K = static_cast<const kvs_bf16*>(fake(15));
  auto* kept = static_cast<int32_t*>(fake(16));
  auto* offs = static_cast<int64_t*>(fake(17));
  auto* Ko = static_cast<kvs_bf16*>(fake(18));
  const kvs_evict_desc good = evict();
  const size_t ws = kv_evict_workspace_bytes(&good);
  EXPECT(ws > 0 && ws % 256 == 0, "evict workspace");
  EXPECT(kv_evict(&good, s, K, K, kept, offs, Ko, Ko, fake(19), ws, nullptr) == KVS_ENODEV, "valid evict");
  EXPECT(kv_evict_noalloc(&good, s, K, K, kept, offs, Ko, Ko, nullptr) == KVS_ENODEV, "valid noalloc");
  kvs_evict_desc e = good; e.capacity -= 1;
  EXPECT(kv_evict(&e, s, K, K, kept, offs, Ko, Ko, fake(19), ws, nullptr) == KVS_ECAPACITY, "capacity");
  e = good; e.k = INT64_MAX; e.capacity = INT64_MAX;  // k clamps to the candidates, no overflow
  EXPECT(kv_evict(&e, s, K, K, kept, offs, Ko, Ko, fake(19), kv_evict_workspace_bytes(&e), nullptr) == KVS_ENODEV,
         "huge k");
  e = good; e.window = INT64_MAX; e.capacity = INT64_MAX;
  EXPECT(kv_evict(&e, s, K, K, kept, offs, Ko, Ko, fake(19), kv_evict_workspace_bytes(&e), nullptr) == KVS_ENODEV,
         "huge window");
  e = good; e.k = -1; e.capacity = 2 * 1000;
  EXPECT(kv_evict(&e, s, K, K, kept, offs, Ko, Ko, fake(19), kv_evict_workspace_bytes(&e), nullptr) == KVS_ENODEV,
         "threshold");
  e = good; e.scope = KVS_SCOPE_LAYER; e.k = 150; e.capacity = 2 * 32 + 150;
  EXPECT(kv_evict(&e, s, K, K, kept, offs, Ko, Ko, fake(19), kv_evict_workspace_bytes(&e), nullptr) == KVS_ENODEV,
         "layer budget");
  e = good; e.n_kvheads = 65535; e.n_tok = (int64_t)1 << 30; e.kv_head_stride = (int64_t)1 << 37;
  e.score_head_stride = (int64_t)1 << 30; e.k = -1; e.capacity = INT64_MAX;
  (void)kv_evict_workspace_bytes(&e);  // the largest layer's workspace size
  EXPECT(kv_evict_noalloc(&e, s, K, K, kept, offs, Ko, Ko, nullptr) == KVS_EWORKSPACE, "noalloc limit");
  e = good; e.n_tok = 0; e.capacity = 0;
  EXPECT(kv_evict(&e, nullptr, nullptr, nullptr, nullptr, offs, nullptr, nullptr, fake(19),
                  kv_evict_workspace_bytes(&e), nullptr) == KVS_ENODEV, "empty layer");
  EXPECT(kv_evict(&good, s, K, K, kept, offs, Ko, Ko, nullptr, ws, nullptr) == KVS_EWORKSPACE, "no workspace");
  EXPECT(kv_evict(&good, s, K, K, kept, offs, Ko, Ko, reinterpret_cast<void*>(0x100010), ws, nullptr) ==
             KVS_EWORKSPACE, "misaligned workspace");
  // streaming append
  kvs_stream_desc st;
  std::memset(&st, 0, sizeof st);
  st.n_kvheads = 2; st.head_dim = 128; st.n_seen = 10; st.n_new = 3; st.window = 4; st.tau = 0.1f;
  st.capacity = 64; st.new_head_stride = 3 * 128; st.new_tok_stride = 128; st.score_head_stride = 3;
  EXPECT(kv_stream_append(&st, s, K, K, Ko, Ko, kept, const_cast<float*>(s), offs, nullptr) == KVS_ENODEV,
         "valid append");
  kvs_stream_desc sb = st; sb.capacity = 12;
  EXPECT(kv_stream_append(&sb, s, K, K, Ko, Ko, kept, const_cast<float*>(s), offs, nullptr) == KVS_ECAPACITY,
         "append capacity");
  sb = st; sb.n_seen = INT64_MAX - 1;
  EXPECT(kv_stream_append(&sb, s, K, K, Ko, Ko, kept, const_cast<float*>(s), offs, nullptr) != KVS_OK,
         "append overflow");
}

static void status_texts() {
  for (int c = -3; c < 12; ++c) EXPECT(kvs_strerror(c) && std::strlen(kvs_strerror(c)) > 0, "strerror %d", c);
  EXPECT(kvs_last_error() != nullptr, "last error");
  EXPECT(kvs_version() > 0, "version");
}

static void generator() {
  const uint64_t key = synth_stream_key(3, 7);
  std::vector<uint64_t> a(1000), b(400);
  synth_u64(key, 0, 1000, a.data());
  synth_u64(key, 300, 400, b.data());
  EXPECT(std::memcmp(a.data() + 300, b.data(), 400 * 8) == 0, "stream elements depend on position only");
  std::vector<float> f(4097);
  std::vector<double> g(4097);
  std::vector<uint16_t> h(4097), h2(4097);
  synth_normal_f32(key, 5, 4097, 0.5, 2.0, f.data());
  synth_normal_f64(key, 5, 4097, 0.5, 2.0, g.data());
  for (size_t i = 0; i < f.size(); ++i) EXPECT(f[i] == (float)g[i], "f32 normal %zu", i);
  synth_normal_bf16(key, 5, 4097, 0.5, 2.0, h.data());
  synth_f32_to_bf16(f.data(), 4097, h2.data());
  EXPECT(std::memcmp(h.data(), h2.data(), h.size() * 2) == 0, "bf16 normals = rounded f32 normals");
  const float special[] = {0.f, -0.f, INFINITY, -INFINITY, NAN, 1e-45f, 3.4028235e38f, 1.00390625f, 1.01171875f};
  uint16_t sb[9];
  synth_f32_to_bf16(special, 9, sb);
  EXPECT(sb[0] == 0x0000 && sb[1] == 0x8000 && sb[2] == 0x7F80 && sb[3] == 0xFF80, "signed zeros and infinities");
  EXPECT((sb[4] & 0x7F80) == 0x7F80 && (sb[4] & 0x7F), "NaN stays NaN");
  EXPECT(sb[7] == 0x3F80 && sb[8] == 0x3F82, "round to nearest even at the halfway points");
  synth_u64(key, UINT64_MAX - 4, 3, a.data());  // counters near the top of the range
  synth_normal_f64(key, UINT64_MAX - 8, 3, 0.0, 1.0, g.data());
  for (int i = 0; i < 3; ++i) EXPECT(std::isfinite(g[i]), "normal near the counter limit");
}

int main() {
  attn_calls();
  vnorm_calls();
  decode_calls();
  evict_calls();
  status_texts();
  generator();
  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host driver: all expectations met\n");
  return 0;
}
