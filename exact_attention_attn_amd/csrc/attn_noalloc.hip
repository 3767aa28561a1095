// attn_noalloc.hip -- attn_decode_noalloc: the split-KV decode and its LSE
// combine in one call whose split workspace is a fixed device array of the
// library instead of a caller-owned buffer, so the call allocates nothing.
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, from the module's load until the
// process ends.  In host code its name is only a host-side stand-in, so the
// device address is looked up once per device with hipGetSymbolAddress (the
// first call on that device, with it current) and that address, never the
// name, is what the kernels get.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "attn_kernels.hpp"

namespace {

constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the scratch is a whole number of 256-byte blocks");

// o_part [B,Hq,max_splits,D] float32, then lse_part [B,Hq,max_splits] float32.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
char* g_ptr[kMaxDevices];            // device address of `scratch` on each device
hipError_t g_err[kMaxDevices];

// Device address of this device's scratch (nullptr, with *err set, on failure).
char* scratch_on(int dev, hipError_t* err) {
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? static_cast<char*>(p) : nullptr;
  });
  *err = g_err[dev];
  return g_ptr[dev];
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

extern "C" int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* seqlens_k, const int32_t* num_splits,
                                   const float* sinks, void* out, float* lse, int B, int Hq,
                                   int Hkv, int Lk_max, int D, int max_splits, int window,
                                   float scale, int in_dtype, int out_dtype, void* stream) {
  int rc = attn::check_decode(q, k_cache, v_cache, seqlens_k, num_splits, B, Hq, Hkv, Lk_max, D,
                              max_splits, scale, in_dtype);
  if (rc != ATTN_OK) return rc;
  rc = attn::check_combine_outputs(sinks, out, lse, out_dtype);
  if (rc != ATTN_OK) return rc;
  const size_t lanes = (size_t)B * Hq * max_splits;  // < 2^31 (checked above)
  const size_t o_bytes = round256(lanes * D * sizeof(float));
  if (o_bytes + lanes * sizeof(float) > kScratchBytes) return ATTN_ERR_SCRATCH;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  hipError_t e;
  char* base = scratch_on(dev, &e);
  if (!base) return ATTN_ERR_HIP;
  float* o_part = reinterpret_cast<float*>(base);
  float* lse_part = reinterpret_cast<float*>(base + o_bytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  e = attn::launch_decode(q, k_cache, v_cache, seqlens_k, num_splits, o_part, lse_part, B, Hq, Hkv,
                          Lk_max, D, max_splits, window, scale, s);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  e = attn::launch_combine(o_part, lse_part, seqlens_k, num_splits, sinks, out, lse, B, Hq, D,
                           Lk_max, max_splits, window, out_dtype == ATTN_F32, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
