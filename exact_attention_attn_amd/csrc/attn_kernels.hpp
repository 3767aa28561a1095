// attn_kernels.hpp -- host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// max_row / max_head (either may be NULL): largest pre-softmax logit per row
// [B,Hq,Lq] and per head [B,Hq]; max_head is filled with -inf on the stream
// first, then raised with atomics.
hipError_t launch_fwd(const void* q, const void* k, const void* v, const float* sinks, void* out,
                      float* lse, float* max_row, float* max_head, int B, int Hq, int Hkv, int Lq,
                      int Lk, int D, int window, float scale, bool in_f32, bool out_f32,
                      hipStream_t stream);

hipError_t launch_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seqlens_k, const int32_t* num_splits, float* o_part,
                         float* lse_part, int B, int Hq, int Hkv, int Lk_max, int D,
                         int max_splits, int window, float scale, hipStream_t stream);

// num_splits[b] from seqlens_k by policy (ATTN_SPLITS_*); one work-group.
hipError_t launch_plan(const int32_t* seqlens_k, int32_t* num_splits, int B, int Hq, int Hkv,
                       int Lk_max, int max_splits, int window, int policy, int param,
                       hipStream_t stream);

hipError_t launch_combine(const float* o_part, const float* lse_part, const int32_t* seqlens_k,
                          const int32_t* num_splits, const float* sinks, void* out, float* lse,
                          int B, int Hq, int D, int Lk_max, int max_splits, int window,
                          bool out_f32, hipStream_t stream);

}  // namespace attn
