// attn_tiles.hpp -- tile machinery shared by the gfx950 prefill kernels
// (forward and backward): which key tiles a group of query rows sees, the
// swizzled LDS tile layout and its global->LDS copies, and the mapping of
// work-groups to (batch, KV head, head group, q-tile).
#pragma once

#include "attn_common.hpp"

namespace attn {
namespace {

constexpr int kRowsPerWave = 32;  // query rows per wave (one MFMA column block)

// Which key range a group of query rows needs, and how a tile relates to it.
struct RowSpan {
  int p_first, p_last;  // absolute positions of the first/last valid row
};

__device__ __forceinline__ int tile_kind(int t0, int bc, RowSpan s, int window, int Lk) {
  // 0: no key of the tile is visible to any row; 1: every pair visible; 2: mixed
  if (t0 > s.p_last) return 0;
  if (window > 0 && t0 + bc - 1 <= s.p_first - window) return 0;
  bool full = (t0 + bc - 1 <= s.p_first) && (t0 + bc <= Lk) &&
              (window <= 0 || t0 >= s.p_last - window + 1);
  return full ? 1 : 2;
}

// ------------------------------------------------------------------------
// bf16 inputs.  A work-group is 4 waves of 32 query rows each, drawn from the
// query heads of one KV head (4 heads x 32 rows when 4 divides the GQA group,
// 2 x 64, or 1 x 128), so every K/V tile brought into LDS serves 4 waves while
// the key span stays that of 32 (or 64, 128) rows.  Two work-groups per CU:
// each SIMD interleaves two waves, and one work-group computes while the
// other waits at its barrier.  K/V tiles of
// 64 keys are copied global -> LDS with buffer loads that write LDS directly
// (no staging registers) into a two-stage ring of separate LDS arrays, one
// tile ahead of its use; one barrier per tile.
//
// LDS tiles use the BfTile layout (16 B chunks XOR-swizzled by row, no
// padding), so one K or V tile is exactly 64 rows x 2D bytes and splits into
// whole 1 KB copy pieces of 1024/(2D) rows each.  A copy instruction writes
// its 64 x 16 B to consecutive LDS slots, so every lane fetches from global
// memory the chunk that the swizzle stores in its slot.  Each wave issues the
// same number of pieces per tile.  The swizzle depends only on the low four
// bits of a row, so a lane's operand read addresses are the same for every
// tile and for both 32-key halves of it, and are computed once.
// ------------------------------------------------------------------------
constexpr int kBfWaves = 4;
constexpr int kBfThreads = 64 * kBfWaves;
constexpr int kBc = 64;  // keys per tile

template <int D>
struct BfLayout {
  static constexpr int kRow = D * 2;                  // bytes of one K/V row
  static constexpr int kChunks = kRow / 16;           // 16 B chunks per row
  static constexpr int kRowsPerPiece = 1024 / kRow;   // rows per 1 KB copy piece
  static constexpr int kBytes = kBc * kRow;           // one K (or V) tile
  static constexpr int kPieces = kBytes / 1024;
  static constexpr int kPerWave = kPieces / kBfWaves;  // pieces per wave per tensor
  static_assert(kPieces % kBfWaves == 0, "pieces split evenly over the waves");
};

// Byte offset, within a tile of the global tensor, of the 16 B that lane
// `lane` copies for piece pc: the row of the lane's slot and the chunk that
// the swizzle stores there.
template <int D>
__device__ __forceinline__ uint32_t dma_src_off(int pc, int lane) {
  using L = BfLayout<D>;
  const int r = pc * L::kRowsPerPiece + lane / L::kChunks;
  const int c = (lane % L::kChunks) ^ BfTile<D>::swz(r);
  return (uint32_t)(r * L::kRow + c * 16);
}

template <int D>
struct TileCopy {
  using L = BfLayout<D>;
  uint32_t off[L::kPerWave];  // this lane's source offsets (K and V alike)
  int wave;
  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
#pragma unroll
    for (int j = 0; j < L::kPerWave; ++j) off[j] = dma_src_off<D>(w + j * kBfWaves, lane);
  }
  // Copy K and V rows [t*64, t*64+64) of one head into the two LDS arrays.
  // The buffer resources end at row Lk, so the rows of a last, partial tile
  // past Lk arrive as zeros (finite, and their scores are masked).
  __device__ __forceinline__ void issue(const uint16_t* kh, const uint16_t* vh, int t, int Lk,
                                        lds_char* kdst, lds_char* vdst) const {
    // The buffer-resource type exists only for the device; the host pass of
    // this file (which only needs the kernel launch stubs) skips the body.
#if defined(__HIP_DEVICE_COMPILE__)
    const size_t base = (size_t)t * kBc * L::kRow;
    const int bytes = min(kBc, Lk - t * kBc) * L::kRow;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)kh + base), 0, bytes, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)vh + base), 0, bytes, kRawBufferWord3);
#pragma unroll
    for (int j = 0; j < L::kPerWave; ++j) {
      const int pc = wave + j * kBfWaves;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, kdst + pc * 1024, 16, off[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vdst + pc * 1024, 16, off[j], 0, 0, 0);
    }
#endif
  }
};

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgValu = 0x002;
constexpr int kSgMfma = 0x008;
constexpr int kSgDsRead = 0x100;

template <int D>
struct BfSmem {
  using L = BfLayout<D>;
  template <int I>
  static __device__ __forceinline__ lds_char* k() {
    __shared__ __attribute__((aligned(1024))) char buf[L::kBytes];
    return (lds_char*)buf;
  }
  template <int I>
  static __device__ __forceinline__ lds_char* v() {
    __shared__ __attribute__((aligned(1024))) char buf[L::kBytes];
    return (lds_char*)buf;
  }
};

// Work of one bf16 work-group: the HG query heads hg*HG .. of KV head kvh
// (they share every K/V tile) over the same rows [r0, r0 + rows).  Longest
// q-tiles first within each (batch, KV head).
struct BfWork {
  int b, kvh, hg, qt;
};
// A packed batch mixes long and short sequences, and contiguous ranges per XCD
// would leave the XCDs that hold the long ones with most of the work: there
// the groups (b, kvh, hg) are dealt round-robin over the XCDs instead (each
// XCD still runs whole groups, so their K/V tiles stay in its L2).
template <bool VARLEN, typename Args>
__device__ __forceinline__ BfWork decode_bf_work(const Args& a, int n_hg) {
  constexpr int kXcd = 8;
  const int n_groups = n_hg * a.Hkv * a.B;
  const int total = a.n_qtiles * n_groups;
  int id;
  if (VARLEN && n_groups % kXcd == 0) {
    const int xcd = blockIdx.x % kXcd, k = blockIdx.x / kXcd;  // k-th work-group of this XCD
    id = ((k / a.n_qtiles) * kXcd + xcd) * a.n_qtiles + k % a.n_qtiles;
  } else {
    id = xcd_remap(blockIdx.x, total);
  }
  BfWork w;
  if (VARLEN) {
    w.qt = a.n_qtiles - 1 - id % a.n_qtiles;
    id /= a.n_qtiles;
    w.hg = id % n_hg;
    id /= n_hg;
  } else {
    // The head groups of one q-tile are consecutive ids, so they run side by
    // side on one XCD and each K/V tile comes from HBM once for all of them.
    w.hg = id % n_hg;
    id /= n_hg;
    w.qt = a.n_qtiles - 1 - id % a.n_qtiles;
    id /= a.n_qtiles;
  }
  w.kvh = id % a.Hkv;
  w.b = id / a.Hkv;
  return w;
}

// Query heads per work-group for a GQA group of G heads: the largest power
// of two <= kBfWaves that divides G.
__host__ __device__ __forceinline__ int bf_heads_per_group(int G) {
  return (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

// ---------------------------------------------------------------------------
// Row blocks of one wave: 32 consecutive rows of D elements, contiguous in
// HBM.  The MFMA layouts give a lane one row and runs of 4 or 8 consecutive d,
// so reading or writing such a block straight from the operand/accumulator
// registers touches 32 rows per instruction; these helpers go through an LDS
// block of the wave's own so that every global instruction covers whole rows.
// A wave reads back only what it wrote itself and LDS operations of one wave
// complete in order, so they need no barrier.
// ---------------------------------------------------------------------------

// Store o (MFMA 32x32 accumulators of O^T: lane col = row, d = db*32 + j*8 +
// half*4 + e in o[db][4j + e]) times mul as rows 0..nrows-1 of oblock (bf16 or
// fp32).  The LDS block holds rows of D*sizeof(OutT) bytes with 16 B chunks
// XOR-swizzled by row against bank conflicts; it is read back CH lanes per row.
template <int D, typename OutT>
__device__ __forceinline__ void store_rows_staged(const f32x16 (&o)[D / 32], float mul,
                                                  lds_char* stage, OutT* oblock, int nrows,
                                                  int col, int half, int lane) {
  constexpr int ROWB = D * (int)sizeof(OutT);  // bytes of one output row
  constexpr int CH = ROWB / 16;                // 16 B chunks per row (8 .. 32)
  constexpr int RPI = 64 / CH;                 // rows per store instruction
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int byte = (db * 32 + j * 8 + half * 4) * (int)sizeof(OutT);
      const int off = col * ROWB + ((((byte >> 4) ^ (col & (CH - 1))) << 4) | (byte & 15));
      const float x0 = o[db][j * 4 + 0] * mul, x1 = o[db][j * 4 + 1] * mul;
      const float x2 = o[db][j * 4 + 2] * mul, x3 = o[db][j * 4 + 3] * mul;
      if constexpr (sizeof(OutT) == 4)
        lds_write16(stage, off, __builtin_bit_cast(u32x4, ((f32x4){x0, x1, x2, x3})));
      else
        lds_write8(stage, off, (u32x2){pack2_bf16(x0, x1), pack2_bf16(x2, x3)});
    }
  }
  const int rr = lane / CH, cc = lane % CH;
#pragma unroll
  for (int i = 0; i < kRowsPerWave / RPI; ++i) {
    const int r = i * RPI + rr;
    const u32x4 v = lds_read16(stage, r * ROWB + ((cc ^ (r & (CH - 1))) << 4));
    // Streaming stores: each output row is written once and not read back
    // here; written through the caches they slow the K/V reads beside them.
    if (r < nrows)
      __builtin_nontemporal_store(v, (u32x4*)((char*)oblock + (size_t)r * ROWB + cc * 16));
  }
}

// Copy a block of 32 consecutive bf16 rows (nrows of them present; the rest
// arrive as zeros) into LDS in the BfTile layout, 1 KB per copy instruction.
template <int D>
__device__ __forceinline__ void copy_rows_to_lds(const uint16_t* src, int nrows, lds_char* dst,
                                                 int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = BfLayout<D>;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)src, 0, max(nrows, 0) * L::kRow, kRawBufferWord3);
#pragma unroll
  for (int pc = 0; pc < kRowsPerWave * L::kRow / 1024; ++pc)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + pc * 1024, 16, dma_src_off<D>(pc, lane), 0,
                                             0, 0);
#endif
}

// Load a block of 32 consecutive bf16 rows into registers, 1 KB of
// consecutive bytes per load instruction (rows past nrows read as zeros).
template <int D>
struct RowBlockRegs {
  static constexpr int kN = kRowsPerWave * D * 2 / 1024;  // loads per lane
  u32x4 v[kN];
  __device__ __forceinline__ void load(const uint16_t* src, int nrows, int lane) {
    constexpr int CHK = D / 8;  // 16 B chunks per row
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int q = i * 64 + lane;  // chunk index within the block
      v[i] = (u32x4){0, 0, 0, 0};
      if (q / CHK < nrows) v[i] = *(const u32x4*)(src + q * 8);
    }
  }
  // Write the block to region (BfTile layout) and read the MFMA operand of
  // row col back: f[ks] = d ks*16 + half*8 .. +8.
  __device__ __forceinline__ void to_operand(lds_char* region, int col, int half, int lane,
                                             bf16x8 (&f)[D / 16]) const {
    using T = BfTile<D>;
    constexpr int CHK = D / 8;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int q = i * 64 + lane;
      lds_write16(region, T::off(q / CHK, (q % CHK) * 16), v[i]);
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      f[ks] = as_bf16x8(lds_read16(region, T::off(col, (ks * 2 + half) * 16)));
  }
};

}  // namespace
}  // namespace attn
