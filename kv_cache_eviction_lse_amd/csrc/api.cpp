// C ABI of libkvscore: argument checks, device check, launch.
//
// Every argument is checked on the host before any HIP call, so an invalid
// call returns its status without touching the device (and works on a host
// with no GPU). Valid calls then require a current gfx950 device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/kvscore.h"
#include "internal.hpp"

#define KVS_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return KVS_OK;
}

struct DevInfo {
  bool probed = false;
  bool usable = false;
  int num_cus = 0;
};
constexpr int MAX_DEVICES = 64;
DevInfo g_devs[MAX_DEVICES];
std::mutex g_dev_mu;

// The current device must be a gfx950 GPU. Fills *num_cus (and *dev_out, the
// current device's index, when given).
int check_device(int* num_cus, int* dev_out = nullptr) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(KVS_ENODEV, "no HIP device is available");
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    (void)hipGetLastError();
    return fail(KVS_ENODEV, "no current HIP device");
  }
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DevInfo& di = g_devs[dev];
  if (!di.probed) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(KVS_ENODEV, "cannot query device %d", dev);
    }
    di.usable = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    di.num_cus = prop.multiProcessorCount;
    di.probed = true;
    if (!di.usable) return fail(KVS_ENODEV, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (!di.usable) return fail(KVS_ENODEV, "device %d is not gfx950", dev);
  *num_cus = di.num_cus;
  if (dev_out) *dev_out = dev;
  return KVS_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t MAX_TOKENS = (int64_t)1 << 30;
// Tiles are read through buffer resources with 32-bit offsets: the score
// pass's 128-row tiles of rows 2^22 elements apart span 2^30 bytes.
constexpr int64_t MAX_TOK_STRIDE = (int64_t)1 << 22;

// Checks shared by the three scoring calls. `need_self` for REPEAT LSE.
int check_attn(const kvs_attn_desc* d, const kvs_bf16* Q, const kvs_bf16* K, const kvs_bf16* Kself,
               bool need_self) {
  if (!d) return fail(KVS_EINVAL, "descriptor is NULL");
  if (d->reserved != 0) return fail(KVS_EINVAL, "reserved field must be 0");
  if (d->n_qheads < 1 || d->n_kvheads < 1) return fail(KVS_EINVAL, "head counts must be >= 1");
  if (d->n_qheads % d->n_kvheads) return fail(KVS_EINVAL, "n_qheads (%d) is not a multiple of n_kvheads (%d)",
                                              d->n_qheads, d->n_kvheads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KVS_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
  if (d->mask != KVS_MASK_REPEAT && d->mask != KVS_MASK_CAUSAL) return fail(KVS_EINVAL, "unknown mask %d", d->mask);
  if (d->n_ctx < 0 || d->n_q < 0) return fail(KVS_EINVAL, "negative length");
  if (d->n_ctx > MAX_TOKENS || d->n_q > MAX_TOKENS) return fail(KVS_EUNSUPPORTED, "more than 2^30 tokens");
  if ((int64_t)d->n_qheads * (d->n_q + 31) > ((int64_t)1 << 31))
    return fail(KVS_EUNSUPPORTED, "n_qheads * n_q is too large");
  if (d->mask == KVS_MASK_REPEAT && d->chunk < 1) return fail(KVS_EINVAL, "chunk must be >= 1 for REPEAT");
  if (d->mask == KVS_MASK_CAUSAL && d->n_q != d->n_ctx)
    return fail(KVS_EINVAL, "CAUSAL needs n_q == n_ctx (%lld != %lld)", (long long)d->n_q, (long long)d->n_ctx);
  if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return fail(KVS_EINVAL, "scale must be finite and > 0");
  const int64_t st[6] = {d->q_head_stride, d->q_tok_stride, d->k_head_stride,
                         d->k_tok_stride, d->ks_head_stride, d->ks_tok_stride};
  for (int i = 0; i < 6; ++i) {
    if (st[i] < 0) return fail(KVS_EINVAL, "negative stride");
    if (st[i] % 8) return fail(KVS_EUNSUPPORTED, "strides must be multiples of 8 elements (16 bytes)");
  }
  if (d->q_tok_stride > MAX_TOK_STRIDE || d->k_tok_stride > MAX_TOK_STRIDE || d->ks_tok_stride > MAX_TOK_STRIDE)
    return fail(KVS_EUNSUPPORTED, "token strides above 2^22 elements");
  if (d->n_q > 0 && d->q_tok_stride < d->head_dim)
    return fail(KVS_EINVAL, "q_tok_stride is smaller than head_dim");
  if (d->n_ctx > 0 && d->k_tok_stride < d->head_dim)
    return fail(KVS_EINVAL, "k_tok_stride is smaller than head_dim");
  if (d->n_q > 0 && !Q) return fail(KVS_EINVAL, "Q is NULL");
  if (d->n_ctx > 0 && !K) return fail(KVS_EINVAL, "K is NULL");
  if (!aligned16(Q) || !aligned16(K)) return fail(KVS_EUNSUPPORTED, "Q and K must be 16-byte aligned");
  if (need_self && d->n_q > 0) {
    if (!Kself) return fail(KVS_EINVAL, "Kself is NULL (REPEAT)");
    if (!aligned16(Kself)) return fail(KVS_EUNSUPPORTED, "Kself must be 16-byte aligned");
    if (d->ks_tok_stride < d->head_dim) return fail(KVS_EINVAL, "ks_tok_stride is smaller than head_dim");
  }
  return KVS_OK;
}

}  // namespace

KVS_API const char* kvs_strerror(int status) {
  switch (status) {
    case KVS_OK: return "success";
    case KVS_EINVAL: return "invalid argument";
    case KVS_EUNSUPPORTED: return "unsupported shape, dtype or alignment";
    case KVS_ECAPACITY: return "output capacity too small";
    case KVS_EWORKSPACE: return "workspace missing or too small";
    case KVS_EHIP: return "HIP runtime error";
    case KVS_ENODEV: return "no usable gfx950 device";
    default: return "unknown status";
  }
}

KVS_API const char* kvs_last_error(void) { return g_last_error; }

KVS_API int kvs_version(void) { return 100; }

KVS_API int kvscore_lse(const kvs_attn_desc* d, const kvs_bf16* Q, const kvs_bf16* K, const kvs_bf16* Kself,
                        float* lse, void* stream) {
  int st = check_attn(d, Q, K, Kself, d && d->mask == KVS_MASK_REPEAT);
  if (st) return st;
  if (d->n_q > 0 && !lse) return fail(KVS_EINVAL, "lse is NULL");
  int cus;
  if ((st = check_device(&cus))) return st;
  return hip_status(kvs::launch_lse(*d, Q, K, Kself, lse, cus, static_cast<hipStream_t>(stream)), "kvscore_lse");
}

KVS_API int kvscore_attention(const kvs_attn_desc* d, const kvs_bf16* Q, const kvs_bf16* K, const kvs_bf16* Kself,
                              const kvs_bf16* V, const kvs_bf16* Vself, kvs_bf16* O, float* lse, void* stream) {
  const bool repeat = d && d->mask == KVS_MASK_REPEAT;
  int st = check_attn(d, Q, K, Kself, repeat);
  if (st) return st;
  if (d->n_q > 0 && (!lse || !O)) return fail(KVS_EINVAL, "O or lse is NULL");
  if (d->n_ctx > 0 && !V) return fail(KVS_EINVAL, "V is NULL");
  if (repeat && d->n_q > 0 && !Vself) return fail(KVS_EINVAL, "Vself is NULL (REPEAT)");
  if (!aligned16(V) || !aligned16(Vself) || !aligned16(O))
    return fail(KVS_EUNSUPPORTED, "V, Vself and O must be 16-byte aligned");
  int cus;
  if ((st = check_device(&cus))) return st;
  return hip_status(kvs::launch_attn(*d, Q, K, Kself, V, Vself, O, lse, static_cast<hipStream_t>(stream)),
                    "kvscore_attention");
}

KVS_API int kvscore_vnorm(const kvs_vnorm_desc* d, const kvs_bf16* V, const kvs_bf16* W_O, float* vnorm,
                          void* stream) {
  if (!d) return fail(KVS_EINVAL, "descriptor is NULL");
  if (d->reserved != 0) return fail(KVS_EINVAL, "reserved field must be 0");
  if (d->n_kvheads < 1 || d->n_kvheads > 65535) return fail(KVS_EINVAL, "n_kvheads must be in [1, 65535]");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KVS_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
  if (d->n_tok < 0 || d->d_model < 0) return fail(KVS_EINVAL, "negative size");
  if (d->n_tok > MAX_TOKENS) return fail(KVS_EUNSUPPORTED, "more than 2^30 tokens");
  if (((d->n_tok + 511) / 512) * d->n_kvheads >= ((int64_t)1 << 31))
    return fail(KVS_EUNSUPPORTED, "n_kvheads * n_tok is too large");
  const int64_t st[3] = {d->v_head_stride, d->v_tok_stride, d->wo_row_stride};
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return fail(KVS_EINVAL, "negative stride");
    if (st[i] % 8) return fail(KVS_EUNSUPPORTED, "strides must be multiples of 8 elements (16 bytes)");
  }
  if (d->n_tok > 0 && d->v_tok_stride < d->head_dim) return fail(KVS_EINVAL, "v_tok_stride is smaller than head_dim");
  if (d->v_tok_stride > MAX_TOK_STRIDE || d->wo_row_stride > MAX_TOK_STRIDE)
    return fail(KVS_EUNSUPPORTED, "row strides above 2^22 elements");
  if (d->d_model > 0 && d->wo_row_stride < (int64_t)d->n_kvheads * d->head_dim)
    return fail(KVS_EINVAL, "wo_row_stride is smaller than n_kvheads * head_dim");
  if (d->n_tok > 0 && (!V || !vnorm)) return fail(KVS_EINVAL, "V or vnorm is NULL");
  if (d->n_tok > 0 && d->d_model > 0 && !W_O) return fail(KVS_EINVAL, "W_O is NULL");
  if (!aligned16(V) || !aligned16(W_O)) return fail(KVS_EUNSUPPORTED, "V and W_O must be 16-byte aligned");
  int st_, cus;
  if ((st_ = check_device(&cus))) return st_;
  return hip_status(kvs::launch_vnorm(*d, V, W_O, vnorm, static_cast<hipStream_t>(stream)), "kvscore_vnorm");
}

namespace {
int check_decode(const kvs_decode_desc* d) {
  if (!d) return fail(KVS_EINVAL, "descriptor is NULL");
  if (d->reserved != 0) return fail(KVS_EINVAL, "reserved field must be 0");
  if (d->n_qheads < 1 || d->n_kvheads < 1 || d->n_kvheads > 65535)
    return fail(KVS_EINVAL, "head counts must be >= 1 (n_kvheads <= 65535)");
  if (d->n_qheads % d->n_kvheads) return fail(KVS_EINVAL, "n_qheads is not a multiple of n_kvheads");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KVS_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
  if (d->n_q < 1 || d->n_q > 4096) return fail(KVS_EINVAL, "n_q must be in [1, 4096]");
  if ((int64_t)d->n_qheads * d->n_q > 65535) return fail(KVS_EUNSUPPORTED, "n_qheads * n_q above 65535");
  if (d->capacity < 0 || d->capacity > MAX_TOKENS * 64) return fail(KVS_EINVAL, "capacity out of range");
  if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return fail(KVS_EINVAL, "scale must be finite and > 0");
  if (d->q_head_stride < 0 || d->q_tok_stride < 0) return fail(KVS_EINVAL, "negative stride");
  if (d->q_head_stride % 8 || d->q_tok_stride % 8)
    return fail(KVS_EUNSUPPORTED, "strides must be multiples of 8 elements (16 bytes)");
  if (d->n_q > 1 && d->q_tok_stride < d->head_dim) return fail(KVS_EINVAL, "q_tok_stride is smaller than head_dim");
  if (d->head_stride_rows < 0) return fail(KVS_EINVAL, "head_stride_rows must be >= 0");
  if (d->head_stride_rows > 0 && d->capacity / d->n_kvheads < d->head_stride_rows)
    return fail(KVS_EINVAL, "capacity is smaller than n_kvheads * head_stride_rows");
  return KVS_OK;
}
}  // namespace

KVS_API size_t kvscore_decode_workspace_bytes(const kvs_decode_desc* d) {
  if (check_decode(d)) return 0;
  return kvs::decode_workspace_bytes(*d);
}

KVS_API int kvscore_decode(const kvs_decode_desc* d, const kvs_bf16* Q, const kvs_bf16* K_cache,
                           const kvs_bf16* V_cache, const int64_t* head_offsets, kvs_bf16* O, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_decode(d);
  if (st) return st;
  if (!Q || !O || !lse || !head_offsets) return fail(KVS_EINVAL, "Q, O, lse or head_offsets is NULL");
  if (d->capacity > 0 && (!K_cache || !V_cache)) return fail(KVS_EINVAL, "K_cache or V_cache is NULL");
  if (!aligned16(Q) || !aligned16(O) || !aligned16(K_cache) || !aligned16(V_cache))
    return fail(KVS_EUNSUPPORTED, "Q, O, K_cache and V_cache must be 16-byte aligned");
  const size_t need = kvs::decode_workspace_bytes(*d);
  if (workspace_bytes < need) return fail(KVS_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if (need > 0 && (!workspace || !aligned16(workspace))) return fail(KVS_EWORKSPACE, "workspace is NULL or misaligned");
  int cus;
  if ((st = check_device(&cus))) return st;
  return hip_status(kvs::launch_decode(*d, Q, K_cache, V_cache, head_offsets, O, lse, workspace,
                                       static_cast<hipStream_t>(stream)),
                    "kvscore_decode");
}

namespace {
int check_stream(const kvs_stream_desc* d) {
  if (!d) return fail(KVS_EINVAL, "descriptor is NULL");
  if (d->reserved != 0) return fail(KVS_EINVAL, "reserved field must be 0");
  if (d->n_kvheads < 1 || d->n_kvheads > 65535) return fail(KVS_EINVAL, "n_kvheads must be in [1, 65535]");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KVS_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
  if (d->n_seen < 0 || d->n_new < 0 || d->window < 0) return fail(KVS_EINVAL, "negative size");
  // (each bounded before the sum, which then cannot overflow)
  if (d->n_seen > MAX_TOKENS || d->n_new > MAX_TOKENS || d->n_seen + d->n_new > MAX_TOKENS)
    return fail(KVS_EUNSUPPORTED, "more than 2^30 tokens");
  if (d->window > MAX_TOKENS) return fail(KVS_EUNSUPPORTED, "window above 2^30");
  const int64_t need = d->window > d->n_seen + d->n_new ? d->window : d->n_seen + d->n_new;
  if (d->capacity < need)
    return fail(KVS_ECAPACITY, "capacity %lld < %lld rows (window or every token)", (long long)d->capacity,
                (long long)need);
  if (d->capacity > MAX_TOKENS) return fail(KVS_EUNSUPPORTED, "capacity above 2^30 rows per head");
  if (d->new_head_stride < 0 || d->new_tok_stride < 0 || d->score_head_stride < 0)
    return fail(KVS_EINVAL, "negative stride");
  if (d->new_head_stride % 8 || d->new_tok_stride % 8)
    return fail(KVS_EUNSUPPORTED, "K_new/V_new strides must be multiples of 8 elements (16 bytes)");
  if (d->n_new > 1 && d->new_tok_stride < d->head_dim) return fail(KVS_EINVAL, "new_tok_stride is smaller than head_dim");
  if (d->n_kvheads > 1 && d->n_new > 0 && d->score_head_stride < d->n_new)
    return fail(KVS_EINVAL, "score_head_stride is smaller than n_new");
  return KVS_OK;
}
}  // namespace

KVS_API int kv_stream_append(const kvs_stream_desc* d, const float* new_scores, const kvs_bf16* K_new,
                             const kvs_bf16* V_new, kvs_bf16* K_cache, kvs_bf16* V_cache, int32_t* pos_cache,
                             float* win_scores, int64_t* head_len, void* stream) {
  int st = check_stream(d);
  if (st) return st;
  if (!K_cache || !V_cache || !pos_cache || !head_len) return fail(KVS_EINVAL, "a cache pointer is NULL");
  if (d->window > 0 && !win_scores) return fail(KVS_EINVAL, "win_scores is NULL");
  if (d->n_new > 0 && (!new_scores || !K_new || !V_new)) return fail(KVS_EINVAL, "an input pointer is NULL");
  if (!aligned16(K_new) || !aligned16(V_new) || !aligned16(K_cache) || !aligned16(V_cache))
    return fail(KVS_EUNSUPPORTED, "K_new, V_new, K_cache and V_cache must be 16-byte aligned");
  int cus;
  if ((st = check_device(&cus))) return st;
  return hip_status(kvs::launch_stream_append(*d, new_scores, K_new, V_new, K_cache, V_cache, pos_cache, win_scores,
                                              head_len, static_cast<hipStream_t>(stream)),
                    "kv_stream_append");
}

KVS_API int kvscore_max(const kvs_attn_desc* d, const kvs_bf16* Q, const kvs_bf16* K, const float* lse,
                        const float* vnorm, const float* hnorm, float* scores, int accumulate, void* stream) {
  int st = check_attn(d, Q, K, nullptr, false);
  if (st) return st;
  if (d->mask != KVS_MASK_REPEAT) return fail(KVS_EINVAL, "kvscore_max scores the context keys of a REPEAT layer");
  if (accumulate != 0 && accumulate != 1) return fail(KVS_EINVAL, "accumulate must be 0 or 1");
  if (d->n_q > 0 && !lse) return fail(KVS_EINVAL, "lse is NULL");
  if (d->n_ctx > 0 && !scores) return fail(KVS_EINVAL, "scores is NULL");
  int cus;
  if ((st = check_device(&cus))) return st;
  return hip_status(kvs::launch_score_max(*d, Q, K, lse, vnorm, hnorm, scores, accumulate, cus,
                                          static_cast<hipStream_t>(stream)),
                    "kvscore_max");
}

KVS_API int kvscore_futuremass(const kvs_attn_desc* d, const kvs_bf16* Q, const kvs_bf16* K, const float* lse,
                               int64_t window, const float* vnorm, const float* hnorm, float* target,
                               void* stream) {
  int st = check_attn(d, Q, K, nullptr, false);
  if (st) return st;
  if (d->mask != KVS_MASK_CAUSAL) return fail(KVS_EINVAL, "kvscore_futuremass needs a CAUSAL layer");
  if (window < 0) return fail(KVS_EINVAL, "window must be >= 0");
  if (d->n_ctx > 0 && (!lse || !target)) return fail(KVS_EINVAL, "lse or target is NULL");
  int cus;
  if ((st = check_device(&cus))) return st;
  return hip_status(kvs::launch_score_sum(*d, Q, K, lse, window, vnorm, hnorm, target, cus,
                                          static_cast<hipStream_t>(stream)),
                    "kvscore_futuremass");
}

namespace {
int check_evict(const kvs_evict_desc* e) {
  if (!e) return fail(KVS_EINVAL, "descriptor is NULL");
  if (e->scope != KVS_SCOPE_HEAD && e->scope != KVS_SCOPE_LAYER) return fail(KVS_EINVAL, "unknown scope %d", e->scope);
  if (e->n_kvheads < 1) return fail(KVS_EINVAL, "n_kvheads must be >= 1");
  if (e->n_kvheads > 65535) return fail(KVS_EUNSUPPORTED, "more than 65535 KV heads");
  if (e->head_dim != 64 && e->head_dim != 128)
    return fail(KVS_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", e->head_dim);
  if (e->n_tok < 0 || e->window < 0 || e->capacity < 0) return fail(KVS_EINVAL, "negative size");
  if (e->n_tok > MAX_TOKENS) return fail(KVS_EUNSUPPORTED, "more than 2^30 tokens");
  if (e->kv_head_stride < 0 || e->kv_tok_stride < 0 || e->score_head_stride < 0)
    return fail(KVS_EINVAL, "negative stride");
  if (e->kv_head_stride % 8 || e->kv_tok_stride % 8)
    return fail(KVS_EUNSUPPORTED, "K/V strides must be multiples of 8 elements (16 bytes)");
  if (e->n_tok > 0 && e->kv_tok_stride < e->head_dim) return fail(KVS_EINVAL, "kv_tok_stride is smaller than head_dim");
  if (e->n_kvheads > 1 && e->score_head_stride < e->n_tok)
    return fail(KVS_EINVAL, "score_head_stride is smaller than n_tok");
  if (e->scope == KVS_SCOPE_LAYER && (int64_t)e->n_kvheads * e->n_tok > (int64_t)INT32_MAX)
    return fail(KVS_EUNSUPPORTED, "a layer budget needs n_kvheads * n_tok < 2^31");
  return KVS_OK;
}
}  // namespace

KVS_API size_t kv_evict_workspace_bytes(const kvs_evict_desc* e) {
  if (check_evict(e)) return 0;
  return kvs::evict_workspace_bytes(*e);
}

namespace {
// Checks of kv_evict and kv_evict_noalloc other than the workspace.
int check_evict_call(const kvs_evict_desc* e, const float* scores, const kvs_bf16* K, const kvs_bf16* V,
                     const int32_t* kept_idx, const int64_t* head_offsets, const kvs_bf16* K_out,
                     const kvs_bf16* V_out) {
  int st = check_evict(e);
  if (st) return st;
  const int64_t w = e->window < e->n_tok ? e->window : e->n_tok;
  const int64_t cand = e->n_tok - w;
  int64_t need;
  if (e->k < 0) {
    need = e->n_tok * e->n_kvheads;
  } else if (e->scope == KVS_SCOPE_LAYER) {
    const int64_t all = cand * e->n_kvheads;
    need = w * e->n_kvheads + (e->k < all ? e->k : all);
  } else {
    need = (w + (e->k < cand ? e->k : cand)) * e->n_kvheads;
  }
  if (e->capacity < need)
    return fail(KVS_ECAPACITY, "capacity %lld < %lld rows needed", (long long)e->capacity, (long long)need);
  if (!head_offsets) return fail(KVS_EINVAL, "head_offsets is NULL");
  if (need > 0 && (!kept_idx || !K_out || !V_out)) return fail(KVS_EINVAL, "an output pointer is NULL");
  if (e->n_tok > 0 && (!scores || !K || !V)) return fail(KVS_EINVAL, "an input pointer is NULL");
  if (!aligned16(K) || !aligned16(V) || !aligned16(K_out) || !aligned16(V_out))
    return fail(KVS_EUNSUPPORTED, "K, V, K_out and V_out must be 16-byte aligned");
  return KVS_OK;
}
}  // namespace

KVS_API int kv_evict(const kvs_evict_desc* e, const float* scores, const kvs_bf16* K, const kvs_bf16* V,
                     int32_t* kept_idx, int64_t* head_offsets, kvs_bf16* K_out, kvs_bf16* V_out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_evict_call(e, scores, K, V, kept_idx, head_offsets, K_out, V_out);
  if (st) return st;
  const size_t ws = kvs::evict_workspace_bytes(*e);
  if (!workspace || workspace_bytes < ws)
    return fail(KVS_EWORKSPACE, "workspace of %zu bytes needed, %zu given", ws, workspace ? workspace_bytes : 0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(KVS_EWORKSPACE, "workspace must be 256-byte aligned");
  int cus;
  if ((st = check_device(&cus))) return st;
  return hip_status(kvs::launch_evict(*e, scores, K, V, kept_idx, head_offsets, K_out, V_out, workspace,
                                      workspace_bytes, static_cast<hipStream_t>(stream)),
                    "kv_evict");
}

KVS_API int kv_evict_noalloc(const kvs_evict_desc* e, const float* scores, const kvs_bf16* K, const kvs_bf16* V,
                             int32_t* kept_idx, int64_t* head_offsets, kvs_bf16* K_out, kvs_bf16* V_out,
                             void* stream) {
  int st = check_evict_call(e, scores, K, V, kept_idx, head_offsets, K_out, V_out);
  if (st) return st;
  const size_t ws = kvs::evict_workspace_bytes(*e, kvs::EVICT_SCRATCH_BYTES);
  static_assert(kvs::EVICT_SCRATCH_BYTES == KVS_EVICT_NOALLOC_MAX_WORKSPACE, "header and library disagree");
  if (ws > kvs::EVICT_SCRATCH_BYTES)
    return fail(KVS_EWORKSPACE, "this layer needs %zu bytes of workspace, above the %zu-byte built-in scratch of "
                "kv_evict_noalloc (use kv_evict with a workspace)", ws, kvs::EVICT_SCRATCH_BYTES);
  int cus, dev;
  if ((st = check_device(&cus, &dev))) return st;
  void* ws_dev = nullptr;  // this device's copy of the library's scratch array
  st = hip_status(kvs::evict_scratch(dev, &ws_dev), "kv_evict_noalloc: scratch lookup");
  if (st) return st;
  return hip_status(kvs::launch_evict(*e, scores, K, V, kept_idx, head_offsets, K_out, V_out, ws_dev,
                                      kvs::EVICT_SCRATCH_BYTES, static_cast<hipStream_t>(stream)),
                    "kv_evict_noalloc");
}
