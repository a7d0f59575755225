// Host-side launch entry points of the kernels (called by api.cpp after the
// arguments have been validated). Each returns the hipError_t of its launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvscore.h"

namespace kvs {

hipError_t launch_lse(const kvs_attn_desc& d, const uint16_t* Q, const uint16_t* K, const uint16_t* Kself,
                      float* lse, int num_cus, hipStream_t s);

hipError_t launch_score_max(const kvs_attn_desc& d, const uint16_t* Q, const uint16_t* K, const float* lse,
                            const float* vnorm, const float* hnorm, float* scores, int accumulate,
                            int num_cus, hipStream_t s);

hipError_t launch_score_sum(const kvs_attn_desc& d, const uint16_t* Q, const uint16_t* K, const float* lse,
                            int64_t window, const float* vnorm, const float* hnorm, float* target,
                            int num_cus, hipStream_t s);

hipError_t launch_attn(const kvs_attn_desc& d, const uint16_t* Q, const uint16_t* K, const uint16_t* Kself,
                       const uint16_t* V, const uint16_t* Vself, uint16_t* O, float* lse, hipStream_t s);

hipError_t launch_vnorm(const kvs_vnorm_desc& d, const uint16_t* V, const uint16_t* W_O, float* vnorm,
                        hipStream_t s);

size_t decode_workspace_bytes(const kvs_decode_desc& d);

hipError_t launch_decode(const kvs_decode_desc& d, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                         const int64_t* offs, uint16_t* O, float* lse, void* workspace, hipStream_t s);

hipError_t launch_stream_append(const kvs_stream_desc& d, const float* new_scores, const uint16_t* K_new,
                                const uint16_t* V_new, uint16_t* K_cache, uint16_t* V_cache, int32_t* pos_cache,
                                float* win_scores, int64_t* head_len, hipStream_t s);

// Workspace of the eviction path the layer takes when `budget` bytes are
// available (long heads take the grid path when the long-head path's larger
// workspace does not fit); launch_evict chooses the same way from its
// workspace_bytes.
size_t evict_workspace_bytes(const kvs_evict_desc& e, size_t budget = ~(size_t)0);

// kv_evict_noalloc's workspace: a device array of EVICT_SCRATCH_BYTES per
// GPU. evict_scratch() returns its device address on device `dev`, which
// must be the current device (looked up on the first call per device).
constexpr size_t EVICT_SCRATCH_BYTES = (size_t)4 << 20;
constexpr int MAX_SCRATCH_DEVICES = 64;
hipError_t evict_scratch(int dev, void** ptr);

hipError_t launch_evict(const kvs_evict_desc& e, const float* scores, const uint16_t* K, const uint16_t* V,
                        int32_t* kept_idx, int64_t* head_offsets, uint16_t* K_out, uint16_t* V_out,
                        void* workspace, size_t workspace_bytes, hipStream_t s);

}  // namespace kvs
