// attn_common.hpp -- device helpers shared by the gfx950 attention kernels.
//
// Lane layouts of the CDNA4 matrix instructions used here (wave64):
//   v_mfma_f32_32x32x16_bf16  A[32x16]: lane l holds row l%32, k = (l/32)*8 + e (e < 8)
//                             B[16x32]: lane l holds col l%32, k = (l/32)*8 + e
//                             C[32x32]: lane l, reg r -> row (r/4)*8 + (l/32)*4 + r%4, col l%32
//   v_mfma_f32_32x32x2_f32    A: row l%32, k = l/32;  B: col l%32, k = l/32;  C as above.
//   ds_read_b64_tr_b16        within each 16-lane group, lane i receives element i%4 of
//                             the 8-byte blocks addressed by lanes i/4 + 4k, k = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __attribute__((address_space(3))) char lds_char;

// s_waitcnt immediate that waits for every outstanding vector-memory load
// (vmcnt = 0) and leaves the export and LDS counters unconstrained.
constexpr int kWaitVmcnt0 = (7 << 4) | (0xF << 8);

// Word 3 of a raw (unstructured) buffer resource on CDNA: 32-bit data format,
// no swizzle, no stride.
constexpr int kRawBufferWord3 = 0x00020000;

// Cache-policy operand of buffer loads and stores (gfx950): bit 0 sc0, bit 1
// nt, bit 4 sc1.
constexpr int kCpolSc1 = 16;

// s_waitcnt immediate for vmcnt <= n (0 <= n < 64), other counters unconstrained.
__host__ __device__ constexpr int wait_vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (0xF << 8);
}

// Wait until at most n vector-memory loads of this wave are outstanding; n is
// wave-uniform.  Counts the switch does not list fall back to waiting for all.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 1: __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(8)); break;
    default: __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(0)); break;
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x32_bf16  A[16x32]: lane l holds row l%16, k = (l/16)*8 + e (e < 8)
//                           B[32x16]: lane l holds col l%16, k = (l/16)*8 + e
//                           C[16x16]: lane l, reg r -> row (l/16)*4 + r, col l%16
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Reductions across lanes l and l^32 (the two k-halves that hold one column).
// permlane32_swap(x, x) yields x[l%32] and x[32 + l%32]; combining the two in a
// fixed order gives both lanes the same bits.
__device__ __forceinline__ float pair_max(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Whole-wave reductions in a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  bf16x2 p = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, p);
}

// Pack 8 floats to bf16 (round to nearest even, v_cvt_pk_bf16_f32), as four
// 32-bit words of two values each (first value in the low half).
__device__ __forceinline__ u32x4 pack_bf16_words(float a0, float a1, float a2, float a3, float a4,
                                                 float a5, float a6, float a7) {
  return (u32x4){pack2_bf16(a0, a1), pack2_bf16(a2, a3), pack2_bf16(a4, a5), pack2_bf16(a6, a7)};
}
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
  return __builtin_bit_cast(bf16x8, pack_bf16_words(a0, a1, a2, a3, a4, a5, a6, a7));
}

// Sums of bf16 values packed two to a 32-bit word (first value in the low
// half), added to acc in a fixed order by v_dot2c_f32_bf16 against (1, 1):
// each pair is added exactly, the running sum rounds as fp32 adds do.
// The instructions are written as inline asm because the builtin, given words
// held in a register tuple, lost their sub-register index (every dot product
// read the tuple's first register).  A VALU instruction that reads the result
// of a dot instruction needs 3 wait states on this chip; the compiler cannot
// see that inside asm, so each block ends with them (s_nop 2).  Consecutive
// dot2c instructions accumulating into the same register need none.
__device__ __forceinline__ float sum_bf16_words(u32x4 a, u32x4 b, float acc) {
  asm("v_dot2c_f32_bf16 %0, 0x3f803f80, %1\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %2\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %3\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %4\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %5\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %6\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %7\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %8\n\t"
      "s_nop 2"
      : "+v"(acc)
      : "v"(a.x), "v"(a.y), "v"(a.z), "v"(a.w), "v"(b.x), "v"(b.y), "v"(b.z), "v"(b.w));
  return acc;
}

// ---------------------------------------------------------------------------
// LDS tile layout for bf16 rows of D elements (D*2 bytes = D/8 chunks of 16 B).
// Chunk c of row r is stored at chunk position c ^ swz(r).  The XOR spreads
//  - the 16 rows read together by one 16-lane group of a K operand read, and
//  - the 4 rows x 64 B read together by a transposed V read
// over distinct LDS banks.
// ---------------------------------------------------------------------------
template <int D>
struct BfTile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (D == 128) {
      return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
      return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    }
  }
  // byte offset of (row r, byte b within the row)
  __device__ static __forceinline__ int off(int r, int byte) {
    return r * kRowBytes + ((((byte >> 4) ^ swz(r)) << 4) | (byte & 15));
  }
};

// 16-byte LDS read / write at a byte offset.
__device__ __forceinline__ u32x4 lds_read16(const lds_char* base, int off) {
  return *(const __attribute__((address_space(3))) u32x4*)(base + off);
}
__device__ __forceinline__ void lds_write16(lds_char* base, int off, u32x4 v) {
  *(__attribute__((address_space(3))) u32x4*)(base + off) = v;
}
__device__ __forceinline__ void lds_write8(lds_char* base, int off, u32x2 v) {
  *(__attribute__((address_space(3))) u32x2*)(base + off) = v;
}
__device__ __forceinline__ i16x4 lds_read_tr16(const lds_char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + off));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, r);
}

// Row permutation of the K operand of S^T = K Q^T.  Accumulator row
// r = J*8 + H*4 + I (J < 4, H < 2, I < 4) is given key pi(r) =
// (J/2)*16 + H*8 + (J%2)*4 + I, so accumulator register v of the lane half h
// holds key (v/8)*16 + h*8 + v%8: each half then owns 8 consecutive keys per
// 16-key k-step of P V, matching the transposed V read.
__device__ __forceinline__ int key_perm(int r) {
  int J = r >> 3, H = (r >> 2) & 1, I = r & 3;
  return ((J >> 1) << 4) | (H << 3) | ((J & 1) << 2) | I;
}
__device__ __forceinline__ int key_of_reg(int v, int half) {
  return ((v >> 3) << 4) | (half << 3) | (v & 7);
}

// Split rule of the split-KV decode (see attn_decode_splitkv in attn.h).
struct SplitRange {
  int lo, chunk, n_valid, Lk;
};
__device__ __forceinline__ SplitRange split_rule(int seqlen, int nsplit, int Lk_max, int max_splits,
                                                 int window) {
  SplitRange s;
  int Lk = min(max(seqlen, 0), Lk_max);
  int ns = min(max(nsplit, 1), max_splits);
  int lo = window > 0 ? max(0, Lk - window) : 0;
  int n = Lk - lo;
  s.lo = lo;
  s.Lk = Lk;
  if (n <= 0) {
    s.chunk = 64;
    s.n_valid = 0;
    return s;
  }
  int per = (n + ns - 1) / ns;
  s.chunk = (per + 63) / 64 * 64;
  s.n_valid = (n + s.chunk - 1) / s.chunk;
  return s;
}

// Work-group id -> logical work id so that each XCD (work-groups are dealt
// round-robin over 8 XCDs) runs one contiguous range of logical ids.
__device__ __forceinline__ int xcd_remap(int x, int total) {
  constexpr int kXcd = 8;
  int per = total / kXcd, rem = total % kXcd;
  int xcd = x % kXcd, idx = x / kXcd;
  return xcd * per + min(xcd, rem) + idx;
}

}  // namespace attn
