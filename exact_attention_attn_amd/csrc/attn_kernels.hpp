// attn_kernels.hpp -- host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Host-side argument checks shared by the entry points (ATTN_* codes).
// check_decode: everything attn_decode_splitkv checks except its workspace
// pointers; check_combine_outputs: attn_combine's sinks, out and lse.
int check_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens_k,
                 const int32_t* num_splits, int B, int Hq, int Hkv, int Lk_max, int D,
                 int max_splits, float scale, int in_dtype);
int check_combine_outputs(const float* sinks, const void* out, const float* lse, int out_dtype);

// max_row / max_head (either may be NULL): largest pre-softmax logit per row
// [B,Hq,Lq] and per head [B,Hq]; max_head is filled with -inf on the stream
// first, then raised with atomics.
hipError_t launch_fwd(const void* q, const void* k, const void* v, const float* sinks, void* out,
                      float* lse, float* max_row, float* max_head, int B, int Hq, int Hkv, int Lq,
                      int Lk, int D, int window, float scale, bool in_f32, bool out_f32,
                      hipStream_t stream);

// Packed batch of sequences (bf16 inputs): q [Hq,total_q,D], k/v [Hkv,total_k,D],
// cu_q/cu_k [B+1] device offsets; max_seqlen_q bounds every sequence's rows.
hipError_t launch_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_q,
                             const int32_t* cu_k, const float* sinks, void* out, float* lse, int B,
                             int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q, int D,
                             int window, float scale, bool out_f32, hipStream_t stream);

hipError_t launch_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seqlens_k, const int32_t* num_splits, float* o_part,
                         float* lse_part, int B, int Hq, int Hkv, int Lk_max, int D,
                         int max_splits, int window, float scale, hipStream_t stream);

// Split-KV decode over a paged cache: pages [num_pages,Hkv,1<<page_shift,D],
// block_table [B,max_pages]; Lk_max = max_pages << page_shift.
hipError_t launch_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* seqlens_k,
                               const int32_t* num_splits, float* o_part, float* lse_part, int B,
                               int Hq, int Hkv, int Lk_max, int num_pages, int page_shift,
                               int max_pages, int D, int max_splits, int window, float scale,
                               hipStream_t stream);

// num_splits[b] from seqlens_k by policy (ATTN_SPLITS_*); one work-group.
hipError_t launch_plan(const int32_t* seqlens_k, int32_t* num_splits, int B, int Hq, int Hkv,
                       int Lk_max, int max_splits, int window, int policy, int param,
                       hipStream_t stream);

hipError_t launch_combine(const float* o_part, const float* lse_part, const int32_t* seqlens_k,
                          const int32_t* num_splits, const float* sinks, void* out, float* lse,
                          int B, int Hq, int D, int Lk_max, int max_splits, int window,
                          bool out_f32, hipStream_t stream);

// Backward: delta [B,Hq,Lq] workspace (D_i = <dO_i, O_i>), then dsink (when
// both dsink and sinks are given), dK/dV and dQ; every output fp32.
hipError_t launch_bwd(const void* q, const void* k, const void* v, const float* sinks,
                      const void* out, const void* dout, const float* lse, float* delta,
                      float* dq, float* dk, float* dv, float* dsink, int B, int Hq, int Hkv,
                      int Lq, int Lk, int D, int window, float scale, bool o_f32,
                      hipStream_t stream);

}  // namespace attn
