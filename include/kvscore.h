/*
 * kvscore.h — C ABI of the KV-cache importance scoring and eviction library
 * (libkvscore.so, gfx950 / MI355X).
 *
 * What it computes, for one transformer layer, without ever storing an
 * attention map:
 *
 *   kvscore_lse        the log-sum-exp normaliser of every query row, the
 *                      quantity an attention kernel returns with its output
 *                      and that the KVpop review's transposed-attention pass
 *                      reuses ("[논문리뷰] KVpop ...", §1 Key Terms).
 *   kvscore_max        KVzip's score, the largest attention weight a context
 *                      key receives from any repeat query and any query head
 *                      of its GQA group ("KVzap: Fast, Adaptive, and Faithful
 *                      KV Cache Pruning", §3.1 Eq. 1), optionally weighted by
 *                      ||W_O v_i|| / ||h_j|| (same page, §3.2 Eq. 3, KVzip+).
 *   kvscore_futuremass KVpop's future-attention target: the attention mass a
 *                      key receives from queries at least `window` positions
 *                      later, i.e. after it has left the protected window
 *                      (KVpop review, §1 Key Terms), summed over the group.
 *   kv_evict           per KV head, keep the last `window` keys plus either
 *                      the k best-scoring other keys (KVpop review §3, per-head
 *                      top-k) or those scoring >= tau (KVzap page, threshold
 *                      rule and Algorithm 1), then copy the kept K and V rows
 *                      into one dense cache, head after head.
 *
 * Conventions shared by every call
 *   - Tensors are device pointers owned by the caller. The library allocates
 *     nothing and keeps no state between calls (kv_evict_noalloc's fixed
 *     scratch array, see there, only holds the last call's intermediates).
 *   - bf16 tensors are passed as their 16-bit patterns (kvs_bf16). The head
 *     dimension is contiguous; head and token strides are in elements.
 *   - Logit of query j (query head g) and key i: l = scale * q_j . k_i.
 *     Query head g reads KV head g / (n_qheads / n_kvheads).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream) and never synchronises. Arguments are checked on the
 *     host first; on any error nothing is launched and the status is
 *     returned. kvs_last_error() then holds a one-line reason (per thread).
 *   - Calls are thread-safe. Concurrent calls that write the same output race.
 */
#ifndef KVSCORE_H
#define KVSCORE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
enum {
  KVS_OK = 0,
  KVS_EINVAL = 1,        /* bad argument: null pointer, negative size, shape mismatch */
  KVS_EUNSUPPORTED = 2,  /* head_dim not 64/128, misaligned pointer or stride */
  KVS_ECAPACITY = 3,     /* output capacity smaller than the worst-case kept rows */
  KVS_EWORKSPACE = 4,    /* workspace missing or smaller than kv_evict_workspace_bytes */
  KVS_EHIP = 5,          /* HIP runtime or launch error (text in kvs_last_error) */
  KVS_ENODEV = 6         /* no usable gfx950 device is current */
};

/* ---- masks ----------------------------------------------------------- */
/* KVS_MASK_REPEAT: the teacher-forced repeat of the context (KVzap page §3.1
 * repeat prompt; KVzip review "Methods" and "Methods: technical-details").
 * Repeat query j belongs to chunk c = j / chunk and sees all n_ctx context
 * keys plus the self keys c*chunk .. j of its own chunk (diagonal included).
 * KVS_MASK_CAUSAL: plain causal self-attention over one sequence of n_ctx
 * tokens: query j sees keys 0 .. j. */
enum { KVS_MASK_REPEAT = 0, KVS_MASK_CAUSAL = 1 };

typedef uint16_t kvs_bf16; /* bfloat16 bit pattern */

/* Eviction budget scope (kvs_evict_desc.scope). */
enum { KVS_SCOPE_HEAD = 0, KVS_SCOPE_LAYER = 1 };

/* Shape of one layer's attention, shared by the three scoring calls.
 *   Q      [n_qheads, n_q, head_dim]    strides q_head_stride, q_tok_stride
 *   K      [n_kvheads, n_ctx, head_dim] strides k_head_stride, k_tok_stride
 *          (context keys; for CAUSAL the sequence's keys, n_q == n_ctx)
 *   Kself  [n_kvheads, n_q, head_dim]   strides ks_head_stride, ks_tok_stride
 *          (REPEAT only: the keys of the repeated copy; row j is query j's)
 * Requirements: n_qheads % n_kvheads == 0; head_dim is 64 or 128; every
 * pointer and every stride keeps rows 16-byte aligned (strides multiple of 8);
 * token strides are at least head_dim and at most 2^22 (KVS_EUNSUPPORTED).
 * chunk > 0 for REPEAT (the last chunk may be shorter); ignored for CAUSAL. */
typedef struct kvs_attn_desc {
  int32_t n_qheads;
  int32_t n_kvheads;
  int32_t head_dim;
  int32_t mask;
  int64_t n_ctx;
  int64_t n_q;
  int64_t chunk;
  int64_t q_head_stride, q_tok_stride;
  int64_t k_head_stride, k_tok_stride;
  int64_t ks_head_stride, ks_tok_stride;
  float scale;
  int32_t reserved; /* set to 0 */
} kvs_attn_desc;

/* LSE pass. lse [n_qheads, n_q] fp32, dense, natural log:
 *   lse[g][j] = ln sum_{i visible to j} exp(scale * q_j . k_i)
 * over the keys the mask makes visible (context + own-chunk self keys for
 * REPEAT, keys 0..j for CAUSAL). Kself is ignored (may be NULL) for CAUSAL.
 * Every query sees at least one key, so every value is finite. */
int kvscore_lse(const kvs_attn_desc* d, const kvs_bf16* Q, const kvs_bf16* K,
                const kvs_bf16* Kself, float* lse, void* stream);

/* Attention forward with its output (KVzap page §3.2 Eq. 2: the per-head
 * sum sum_i a_ji v_i that enters the residual update, before W_O; the LSE
 * it returns alongside is the normaliser the KVpop review §1 reuses):
 *   O[g][j]   = sum_{i visible to j} exp(scale * q_j . k_i - lse[g][j]) * v_i
 *   lse[g][j] = exactly what kvscore_lse computes (same visibility rules).
 * V      [n_kvheads, n_ctx, head_dim] bf16, the values of K (K's strides);
 * Vself  [n_kvheads, n_q, head_dim] bf16, the values of Kself (Kself's
 *        strides; REPEAT only, may be NULL for CAUSAL);
 * O      [n_qheads, n_q, head_dim] bf16 with Q's strides, overwritten
 *        (fp32 accumulation, rounded once to bf16);
 * lse    [n_qheads, n_q] fp32, dense, overwritten.
 * The probabilities enter the value product rounded to bf16 (as in a
 * bf16 flash-attention kernel); lse is computed in fp32 from the unrounded
 * exponentials. */
int kvscore_attention(const kvs_attn_desc* d, const kvs_bf16* Q,
                      const kvs_bf16* K, const kvs_bf16* Kself,
                      const kvs_bf16* V, const kvs_bf16* Vself,
                      kvs_bf16* O, float* lse, void* stream);

/* KVzip / KVzip+ max score (KVzap page §3.1 Eq. 1 and §3.2 Eq. 3), for the
 * context keys of a REPEAT layer; every repeat query sees every context key:
 *   s[h][i] = max_{g in group(h)} max_{j < n_q}
 *             exp(scale * q_j^g . k_i - lse[g][j]) * vnorm[h][i] / hnorm[j]
 * lse    [n_qheads, n_q] fp32 (normally kvscore_lse's output)
 * vnorm  [n_kvheads, n_ctx] fp32 >= 0, or NULL for 1 (||W_O v_i||)
 * hnorm  [n_q] fp32 > 0, or NULL for 1 (||h_j||, one per query position)
 * scores [n_kvheads, n_ctx] fp32, dense.
 * accumulate = 0 overwrites scores (0 when n_q == 0); accumulate = 1 keeps
 * the larger of the stored and the new value, so calling once per chunk of
 * queries (Q, lse, hnorm pointing at that chunk) equals one call over all.
 * The stored values must then be >= 0 (earlier scores). desc->mask must be
 * KVS_MASK_REPEAT; chunk and Kself play no part here. */
int kvscore_max(const kvs_attn_desc* d, const kvs_bf16* Q, const kvs_bf16* K,
                const float* lse, const float* vnorm, const float* hnorm,
                float* scores, int accumulate, void* stream);

/* KVpop future-attention target on CAUSAL self-attention (KVpop review §1):
 *   t[h][i] = sum_{g in group(h)} sum_{i + window <= j < n_ctx}
 *             exp(scale * q_j^g . k_i - lse[g][j]) * vnorm[h][i] / hnorm[j]
 * lse [n_qheads, n_ctx] (the CAUSAL kvscore_lse output); vnorm/hnorm as for
 * kvscore_max (NULL for 1); target [n_kvheads, n_ctx] fp32, overwritten.
 * Keys with i + window >= n_ctx get 0. window >= 0. The result is
 * deterministic: the same inputs give the same bits on every call. */
int kvscore_futuremass(const kvs_attn_desc* d, const kvs_bf16* Q,
                       const kvs_bf16* K, const float* lse, int64_t window,
                       const float* vnorm, const float* hnorm, float* target,
                       void* stream);

/* Value norms ||W_O v_i|| (KVzap page §3.2, Eq. 3 and its variable table),
 * the vnorm input of kvscore_max / kvscore_futuremass:
 *   vnorm[h][i] = || W_O[:, h*head_dim : (h+1)*head_dim] . v_i^h ||_2
 * V      [n_kvheads, n_tok, head_dim] bf16, strides v_head_stride,
 *        v_tok_stride (elements, multiples of 8, v_tok_stride >= head_dim);
 * W_O    [d_model, n_kvheads * head_dim] bf16, row stride wo_row_stride
 *        (elements, multiple of 8, >= n_kvheads * head_dim, <= 2^22);
 * vnorm  [n_kvheads, n_tok] fp32, dense, overwritten (0 when d_model == 0).
 * Products of bf16 values are exact; sums are fp32. */
typedef struct kvs_vnorm_desc {
  int32_t n_kvheads;
  int32_t head_dim;
  int64_t n_tok;
  int32_t d_model;
  int32_t reserved; /* set to 0 */
  int64_t v_head_stride, v_tok_stride;
  int64_t wo_row_stride;
} kvs_vnorm_desc;

int kvscore_vnorm(const kvs_vnorm_desc* d, const kvs_bf16* V,
                  const kvs_bf16* W_O, float* vnorm, void* stream);

/* Eviction of one layer's cache.
 *   scores [n_kvheads, n_tok] fp32, head stride score_head_stride (elements)
 *   K, V   [n_kvheads, n_tok, head_dim] bf16, strides kv_head_stride,
 *          kv_tok_stride (shared by K and V)
 * Per head h, with w = min(window, n_tok):
 *   window   positions n_tok - w .. n_tok - 1 are always kept;
 *   top-k    (k >= 0): plus the min(k, n_tok - w) other positions with the
 *            highest scores; equal scores are taken lowest position first,
 *            -0 equals +0 and NaN ranks below every number;
 *   threshold (k < 0): plus the other positions with score >= tau.
 * scope = KVS_SCOPE_LAYER with k >= 0 (the layer-wise top-k the KVzap page's
 *   §4.6 ablation compares thresholds against): one budget of min(k, all
 *   candidates) for the whole layer instead of k per head; the candidates of
 *   all heads are ranked together (equal scores: lower head first, then
 *   lower position), each head keeps its window and its share. Needs
 *   n_kvheads * n_tok < 2^31. Under a threshold the scope plays no part.
 * Outputs (device):
 *   head_offsets [n_kvheads + 1] int64: rows of head h are
 *                head_offsets[h] .. head_offsets[h+1]-1; [n_kvheads] = total
 *   kept_idx     [capacity] int32: position of each kept row, ascending
 *                within a head
 *   K_out, V_out [capacity, head_dim] bf16, dense: bit copies of the rows.
 * capacity must cover the worst case: n_kvheads * (min(k, n_tok - w) + w) in
 * top-k mode (n_kvheads * w + min(k, n_kvheads * (n_tok - w)) with a layer
 * budget), n_kvheads * n_tok in threshold mode (where the count is only
 * known on the device; read head_offsets after synchronising).
 * workspace: device memory of at least kv_evict_workspace_bytes(e) bytes,
 * 256-byte aligned, owned by the caller, contents need not be initialised. */
typedef struct kvs_evict_desc {
  int32_t n_kvheads;
  int32_t head_dim;
  int64_t n_tok;
  int64_t k;
  float tau;
  int32_t scope;    /* KVS_SCOPE_HEAD (0) or KVS_SCOPE_LAYER (1), see above */
  int64_t window;
  int64_t capacity;
  int64_t kv_head_stride, kv_tok_stride;
  int64_t score_head_stride;
} kvs_evict_desc;

size_t kv_evict_workspace_bytes(const kvs_evict_desc* e);

int kv_evict(const kvs_evict_desc* e, const float* scores, const kvs_bf16* K,
             const kvs_bf16* V, int32_t* kept_idx, int64_t* head_offsets,
             kvs_bf16* K_out, kvs_bf16* V_out, void* workspace,
             size_t workspace_bytes, void* stream);

/* Eviction that allocates nothing and takes no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same descriptor,
 * inputs, outputs, checks and results as kv_evict (it runs the same
 * kernels); the workspace kv_evict would take is instead a fixed device
 * array inside the library, KVS_EVICT_NOALLOC_MAX_WORKSPACE bytes, one copy
 * per GPU, held until the process ends. Per-head top-k over more than 16,384
 * candidates per head, whose fastest kernels need more workspace
 * (kv_evict_workspace_bytes(e)) than that array holds, takes the smaller
 * histogram-pass selection here instead (the same results). A layer whose
 * smallest workspace still exceeds the array returns KVS_EWORKSPACE (nothing
 * is launched). The first call on a device looks up that device's copy
 * (no allocation); no call allocates, frees or synchronises.
 * Every call on one GPU shares that GPU's array: calls ordered on one
 * stream are safe, but calls that can overlap in time on the same GPU
 * (different streams, or threads without ordering between them) race on it
 * and give wrong results. */
#define KVS_EVICT_NOALLOC_MAX_WORKSPACE ((size_t)4 << 20)

int kv_evict_noalloc(const kvs_evict_desc* e, const float* scores,
                     const kvs_bf16* K, const kvs_bf16* V, int32_t* kept_idx,
                     int64_t* head_offsets, kvs_bf16* K_out, kvs_bf16* V_out,
                     void* stream);

/* Decode attention over the compacted per-head cache (the cache kv_evict
 * writes: KVzap page Algorithm 1 keys[indices], values[indices], head after
 * head; the page's "Limitation 3" and FAQ "Q4" name this non-uniform,
 * per-head-length cache as what a variable-length kernel must serve):
 *   for query head g (KV head h = g / (n_qheads / n_kvheads)) and decode
 *   query t, over the rows r in [head_offsets[h], head_offsets[h+1]):
 *   O[g][t]   = sum_r exp(scale * q . k_r - lse[g][t]) * v_r
 *   lse[g][t] = ln sum_r exp(scale * q . k_r)   (-inf, with O = 0, for a
 *               head that kept no rows). Every decode query sees every row
 *               of its head.
 * Q        [n_qheads, n_q, head_dim] bf16, strides q_head_stride, q_tok_stride
 * K_cache, V_cache [capacity, head_dim] bf16, dense rows (kv_evict's K_out, V_out)
 * head_offsets [n_kvheads + 1] int64, device (kv_evict's); values are
 *        clamped to [0, capacity] and made non-decreasing before use.
 *        With head_stride_rows = S > 0 it is instead [n_kvheads] live row
 *        counts, head h's rows being [h*S, h*S + head_offsets[h]) (the
 *        per-head regions kv_stream_append keeps, its head_len; counts
 *        are clamped to [0, S]); then capacity must be >= n_kvheads * S.
 * O        [n_qheads, n_q, head_dim] bf16 with Q's strides, overwritten
 * lse      [n_qheads, n_q] fp32, dense, overwritten
 * workspace: device memory of at least kvscore_decode_workspace_bytes(d)
 *        bytes, 16-byte aligned, caller-owned, contents need not be set.
 * Scores, exponentials and sums are fp32; O is rounded once to bf16. */
typedef struct kvs_decode_desc {
  int32_t n_qheads;
  int32_t n_kvheads;
  int32_t head_dim;
  int32_t n_q;      /* decode queries per query head, >= 1 */
  int64_t q_head_stride, q_tok_stride;
  int64_t capacity; /* rows of K_cache / V_cache */
  float scale;
  int32_t reserved; /* set to 0 */
  int64_t head_stride_rows; /* 0: head_offsets is [n_kvheads + 1] offsets; S > 0: see above */
} kvs_decode_desc;

size_t kvscore_decode_workspace_bytes(const kvs_decode_desc* d);

int kvscore_decode(const kvs_decode_desc* d, const kvs_bf16* Q,
                   const kvs_bf16* K_cache, const kvs_bf16* V_cache,
                   const int64_t* head_offsets, kvs_bf16* O, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Threshold pruning as tokens arrive, for decoding. The KVzap page's keep
 * rule (keep token t iff score_t >= tau or t >= T - w, its thresholding
 * rule with the sliding window) re-applied at every sequence length T, as
 * its phase-agnostic criterion asks of a pruner that also runs while
 * decoding: when the token at position p arrives, the token at p - w leaves
 * the window and stays only if its score passes (NaN never does); a dropped
 * token never returns.
 * Cache of one layer, per KV head h a region of `capacity` rows of K_cache
 * and V_cache ([n_kvheads, capacity, head_dim] bf16, dense):
 *   rows [0, w)           the window ring: the window token at position p
 *                         is in row p mod w;
 *   rows [w, w + kept_h)  the tokens that left the window with a passing
 *                         score, in ascending position.
 * The live rows of head h are rows [0, head_len[h]) of its region, with
 * head_len[h] = min(n_seen, w) + kept_h: kvscore_decode reads the cache
 * directly with head_stride_rows = capacity and head_offsets = head_len.
 *   pos_cache  [n_kvheads, capacity] int32: position of each live row
 *   win_scores [n_kvheads, w] fp32: the score of each ring row's token
 *   head_len   [n_kvheads] int64: read and rewritten by each call; all
 *              zero for an empty cache (n_seen = 0). Values outside what
 *              the state allows are clamped, so no write leaves a region.
 * A call appends n_new tokens per head, positions n_seen .. n_seen+n_new-1:
 *   new_scores [n_kvheads, n_new] fp32, head stride score_head_stride;
 *   K_new, V_new [n_kvheads, n_new, head_dim] bf16, strides
 *              new_head_stride, new_tok_stride (shared).
 * capacity must be >= max(w, n_seen + n_new) (room for every token);
 * n_seen + n_new <= 2^30. The caller tracks n_seen (the same for every
 * head). One workgroup per head does the call: it is meant for the few
 * tokens of a decoding step, while kv_evict serves a whole prefill. */
typedef struct kvs_stream_desc {
  int32_t n_kvheads;
  int32_t head_dim;
  int64_t n_seen;   /* tokens appended before this call */
  int64_t n_new;    /* tokens appended by this call (0: nothing to do) */
  int64_t window;   /* w >= 0 */
  float tau;
  int32_t reserved; /* set to 0 */
  int64_t capacity; /* rows per head region */
  int64_t new_head_stride, new_tok_stride;
  int64_t score_head_stride;
} kvs_stream_desc;

int kv_stream_append(const kvs_stream_desc* d, const float* new_scores,
                     const kvs_bf16* K_new, const kvs_bf16* V_new,
                     kvs_bf16* K_cache, kvs_bf16* V_cache, int32_t* pos_cache,
                     float* win_scores, int64_t* head_len, void* stream);

/* ---- diagnostics ----------------------------------------------------- */
const char* kvs_strerror(int status);   /* static text for a status code */
const char* kvs_last_error(void);       /* this thread's last failure reason */
int kvs_version(void);                  /* major * 10000 + minor * 100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* KVSCORE_H */
