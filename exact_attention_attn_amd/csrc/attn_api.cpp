// attn_api.cpp -- the C ABI declared in include/attn.h: argument checks on the
// host, then one asynchronous launch on the caller's stream.  Nothing is
// allocated and no device query or synchronisation happens per call.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_kernels.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int D) { return D == 64 || D == 128; }

bool dtype_ok(int t) { return t == ATTN_BF16 || t == ATTN_F32; }

// Element counts must stay below 2^62 so that 64-bit offsets cannot overflow,
// and every row index the kernels form in 32-bit arithmetic below 2^31.
bool fits(long long a, long long b, long long c, long long d) {
  const long long lim = (long long)1 << 62;
  long long x = a;
  for (long long f : {b, c, d}) {
    if (f != 0 && x > lim / f) return false;
    x *= f;
  }
  return true;
}

int check_fwd(const void* q, const void* k, const void* v, const void* out, int B, int Hq, int Hkv,
              int Lq, int Lk, int D, float scale, int in_dtype, int out_dtype) {
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lk < 1) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || Lq > Lk) return ATTN_ERR_SHAPE;
  if (!fits(B, Hq, Lq, D) || !fits(B, Hkv, Lk, D)) return ATTN_ERR_SHAPE;
  // grid: one work-group per 128 (fp32) or 256 (bf16) query rows of each (batch, head)
  if ((long long)((Lq + 127) / 128) * Hq * B >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if ((long long)B * Hq >= (1LL << 31)) return ATTN_ERR_SHAPE;
  // K/V rows of one head are addressed with 32-bit byte offsets.
  if ((long long)Lk * D * 4 >= (1LL << 32)) return ATTN_ERR_SHAPE;
  if (!supported_dim(D) || !dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return ATTN_ERR_UNSUPPORTED;
  if (!(std::isfinite(scale) && scale > 0.0f)) return ATTN_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_VALUE;
  return ATTN_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

namespace attn {

int check_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens_k,
                 const int32_t* num_splits, int B, int Hq, int Hkv, int Lk_max, int D,
                 int max_splits, float scale, int in_dtype) {
  if (!q || !k_cache || !v_cache || !seqlens_k || !num_splits) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lk_max < 1) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || max_splits < 1 || max_splits > ATTN_MAX_SPLITS) return ATTN_ERR_SHAPE;
  if (!fits(B, Hkv, Lk_max, D) || !fits(B, Hq, max_splits, D)) return ATTN_ERR_SHAPE;
  if ((long long)B * Hq * max_splits >= (1LL << 31)) return ATTN_ERR_SHAPE;  // 32-bit item ids
  if ((long long)B * Hq >= (1LL << 31) || B > 65535 || Hq > 65535) return ATTN_ERR_SHAPE;
  if (!supported_dim(D) || in_dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!(std::isfinite(scale) && scale > 0.0f)) return ATTN_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(seqlens_k) & 3u) || (reinterpret_cast<uintptr_t>(num_splits) & 3u))
    return ATTN_ERR_VALUE;
  return ATTN_OK;
}

int check_combine_outputs(const float* sinks, const void* out, const float* lse, int out_dtype) {
  if (!out) return ATTN_ERR_NULL;
  if (!dtype_ok(out_dtype)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(out) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) ||
      (sinks && (reinterpret_cast<uintptr_t>(sinks) & 3u)))
    return ATTN_ERR_VALUE;
  return ATTN_OK;
}

}  // namespace attn

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, const float* sinks, void* out,
             float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int D, int window, float scale,
             int in_dtype, int out_dtype, void* stream) {
  int rc = check_fwd(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, out_dtype);
  if (rc != ATTN_OK) return rc;
  if ((lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) ||
      (sinks && (reinterpret_cast<uintptr_t>(sinks) & 3u)))
    return ATTN_ERR_VALUE;
  return from_hip(attn::launch_fwd(q, k, v, sinks, out, lse, nullptr, nullptr, B, Hq, Hkv, Lq, Lk,
                                   D, window, scale, in_dtype == ATTN_F32, out_dtype == ATTN_F32,
                                   static_cast<hipStream_t>(stream)));
}

int attn_fwd_max_logit(const void* q, const void* k, const void* v, const float* sinks, void* out,
                       float* lse, float* max_logit_row, float* max_logit_head, int B, int Hq,
                       int Hkv, int Lq, int Lk, int D, int window, float scale, int in_dtype,
                       int out_dtype, void* stream) {
  int rc = check_fwd(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, out_dtype);
  if (rc != ATTN_OK) return rc;
  for (const void* p : {(const void*)lse, (const void*)sinks, (const void*)max_logit_row,
                        (const void*)max_logit_head})
    if (p && (reinterpret_cast<uintptr_t>(p) & 3u)) return ATTN_ERR_VALUE;
  return from_hip(attn::launch_fwd(q, k, v, sinks, out, lse, max_logit_row, max_logit_head, B, Hq,
                                   Hkv, Lq, Lk, D, window, scale, in_dtype == ATTN_F32,
                                   out_dtype == ATTN_F32, static_cast<hipStream_t>(stream)));
}

int attn_bwd(const void* q, const void* k, const void* v, const float* sinks, const void* out,
             const void* dout, const float* lse, float* dq, float* dk, float* dv, float* dsink,
             float* delta, int B, int Hq, int Hkv, int Lq, int Lk, int D, int window, float scale,
             int in_dtype, int out_dtype, void* stream) {
  int rc = check_fwd(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, out_dtype);
  if (rc != ATTN_OK) return rc;
  if (!dout || !lse || !dq || !dk || !dv || !delta) return ATTN_ERR_NULL;
  if (in_dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (dsink && !sinks) return ATTN_ERR_VALUE;
  if ((long long)B * Hq * Lq >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return ATTN_ERR_VALUE;
  for (const void* p : {(const void*)lse, (const void*)delta, (const void*)sinks, (const void*)dsink})
    if (p && (reinterpret_cast<uintptr_t>(p) & 3u)) return ATTN_ERR_VALUE;
  return from_hip(attn::launch_bwd(q, k, v, sinks, out, dout, lse, delta, dq, dk, dv, dsink, B, Hq,
                                   Hkv, Lq, Lk, D, window, scale, out_dtype == ATTN_F32,
                                   static_cast<hipStream_t>(stream)));
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, const float* sinks, void* out, float* lse, int B,
                    int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q, int D, int window,
                    float scale, int in_dtype, int out_dtype, void* stream) {
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !out) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || total_q < 1 || total_k < 0 || max_seqlen_q < 1)
    return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || B > 65535 || max_seqlen_q > total_q) return ATTN_ERR_SHAPE;
  if (!fits(Hq, total_q, D, 1) || !fits(Hkv, total_k, D, 1) || !fits(B, Hq, 1, 1))
    return ATTN_ERR_SHAPE;
  if ((long long)((max_seqlen_q + 31) / 32) * Hq * B >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if ((long long)total_k * D * 4 >= (1LL << 32) || (long long)Hq * total_q >= (1LL << 31) ||
      (long long)Hkv * total_k >= (1LL << 31))
    return ATTN_ERR_SHAPE;
  if (!supported_dim(D) || in_dtype != ATTN_BF16 || !dtype_ok(out_dtype)) return ATTN_ERR_UNSUPPORTED;
  if (!(std::isfinite(scale) && scale > 0.0f)) return ATTN_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_VALUE;
  for (const void* p : {(const void*)cu_seqlens_q, (const void*)cu_seqlens_k, (const void*)lse,
                        (const void*)sinks})
    if (p && (reinterpret_cast<uintptr_t>(p) & 3u)) return ATTN_ERR_VALUE;
  return from_hip(attn::launch_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, sinks, out, lse, B,
                                          Hq, Hkv, total_q, total_k, max_seqlen_q, D, window,
                                          scale, out_dtype == ATTN_F32,
                                          static_cast<hipStream_t>(stream)));
}

int attn_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens_k, const int32_t* num_splits, float* o_part,
                        float* lse_part, int B, int Hq, int Hkv, int Lk_max, int D,
                        int max_splits, int window, float scale, int in_dtype, void* stream) {
  if (!o_part || !lse_part) return ATTN_ERR_NULL;
  const int rc = attn::check_decode(q, k_cache, v_cache, seqlens_k, num_splits, B, Hq, Hkv, Lk_max,
                                    D, max_splits, scale, in_dtype);
  if (rc != ATTN_OK) return rc;
  if (!aligned16(o_part) || (reinterpret_cast<uintptr_t>(lse_part) & 3u)) return ATTN_ERR_VALUE;
  return from_hip(attn::launch_decode(q, k_cache, v_cache, seqlens_k, num_splits, o_part, lse_part,
                                      B, Hq, Hkv, Lk_max, D, max_splits, window, scale,
                                      static_cast<hipStream_t>(stream)));
}

int attn_decode_splitkv_paged(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, const int32_t* seqlens_k,
                              const int32_t* num_splits, float* o_part, float* lse_part, int B,
                              int Hq, int Hkv, int num_pages, int page_size, int max_pages_per_seq,
                              int D, int max_splits, int window, float scale, int in_dtype,
                              void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seqlens_k || !num_splits || !o_part ||
      !lse_part)
    return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || num_pages < 1 || page_size < 1 || max_pages_per_seq < 1)
    return ATTN_ERR_SHAPE;
  if ((page_size & (page_size - 1)) != 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || max_splits < 1 || max_splits > ATTN_MAX_SPLITS) return ATTN_ERR_SHAPE;
  const long long Lk_max = (long long)max_pages_per_seq * page_size;
  if (Lk_max >= (1LL << 31) || !fits(num_pages, Hkv, page_size, D) || !fits(B, Hq, max_splits, D) ||
      !fits(B, max_pages_per_seq, 1, 1))
    return ATTN_ERR_SHAPE;
  if ((long long)B * Hq * max_splits >= (1LL << 31)) return ATTN_ERR_SHAPE;  // 32-bit item ids
  if ((long long)B * Hq >= (1LL << 31) || B > 65535 || Hq > 65535) return ATTN_ERR_SHAPE;
  if (!supported_dim(D) || in_dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!(std::isfinite(scale) && scale > 0.0f)) return ATTN_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o_part) ||
      (reinterpret_cast<uintptr_t>(lse_part) & 3u) || (reinterpret_cast<uintptr_t>(seqlens_k) & 3u) ||
      (reinterpret_cast<uintptr_t>(num_splits) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return ATTN_ERR_VALUE;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  return from_hip(attn::launch_decode_paged(q, k_pages, v_pages, block_table, seqlens_k,
                                            num_splits, o_part, lse_part, B, Hq, Hkv, (int)Lk_max,
                                            num_pages, shift, max_pages_per_seq, D, max_splits,
                                            window, scale, static_cast<hipStream_t>(stream)));
}

int attn_decode_plan(const int32_t* seqlens_k, int32_t* num_splits, int B, int Hq, int Hkv,
                     int Lk_max, int max_splits, int window, int policy, int param, void* stream) {
  if (!seqlens_k || !num_splits) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lk_max < 1) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || max_splits < 1 || max_splits > ATTN_MAX_SPLITS || B > 65535 || Hq > 65535)
    return ATTN_ERR_SHAPE;
  if ((long long)B * Hq * max_splits >= (1LL << 31)) return ATTN_ERR_SHAPE;  // 32-bit item counts
  if (policy != ATTN_SPLITS_AUTO && policy != ATTN_SPLITS_KEYS && policy != ATTN_SPLITS_COUNT)
    return ATTN_ERR_UNSUPPORTED;
  if (policy == ATTN_SPLITS_AUTO ? param < 0 : param < 1) return ATTN_ERR_VALUE;
  if ((reinterpret_cast<uintptr_t>(seqlens_k) & 3u) || (reinterpret_cast<uintptr_t>(num_splits) & 3u))
    return ATTN_ERR_VALUE;
  return from_hip(attn::launch_plan(seqlens_k, num_splits, B, Hq, Hkv, Lk_max, max_splits, window,
                                    policy, param, static_cast<hipStream_t>(stream)));
}

int attn_combine(const float* o_part, const float* lse_part, const int32_t* seqlens_k,
                 const int32_t* num_splits, const float* sinks, void* out, float* lse, int B,
                 int Hq, int D, int Lk_max, int max_splits, int window, int out_dtype,
                 void* stream) {
  if (!o_part || !lse_part || !seqlens_k || !num_splits || !out) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Lk_max < 1 || max_splits < 1 || max_splits > ATTN_MAX_SPLITS)
    return ATTN_ERR_SHAPE;
  if (!fits(B, Hq, max_splits, D) || (long long)B * Hq >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if (!supported_dim(D) || !dtype_ok(out_dtype)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(o_part) || !aligned16(out) || (reinterpret_cast<uintptr_t>(lse_part) & 3u) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) ||
      (sinks && (reinterpret_cast<uintptr_t>(sinks) & 3u)))
    return ATTN_ERR_VALUE;
  return from_hip(attn::launch_combine(o_part, lse_part, seqlens_k, num_splits, sinks, out, lse, B,
                                       Hq, D, Lk_max, max_splits, window, out_dtype == ATTN_F32,
                                       static_cast<hipStream_t>(stream)));
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "invalid shape (sizes, head ratio, Lq > Lk or max_splits)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dim, dtype or policy";
    case ATTN_ERR_VALUE: return "invalid value (scale, policy parameter or pointer alignment)";
    case ATTN_ERR_HIP: return "HIP launch failed";
    case ATTN_ERR_SCRATCH:
      return "split workspace larger than the library's fixed scratch (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

const char* attn_version(void) { return "attn-mi355x 0.1"; }

}  // extern "C"
