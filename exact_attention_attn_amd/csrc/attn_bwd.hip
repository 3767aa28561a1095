// attn_bwd.hip -- backward of the sink/window/GQA attention for gfx950.
//
// Given dO and the forward's O and LSE (natural log, sink included), with
// P_ij = exp(s_ij - LSE_i), Psink_i = exp(sink - LSE_i) and D_i = <dO_i, O_i>:
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q,  dsink_h = -sum_{b,i} Psink_i D_i
// (the sink joins the normaliser and has no value vector, so it enters dS
// only through D).  Three kernels in stream order, all deterministic (no
// atomics):
//   bwd_dq_kernel     rows fixed, K/V tiles streamed (the forward's layout):
//                     D_i = <dO_i, O_i> from the forward's O in its prologue,
//                     then S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T;
//                     it also sums D_i = sum_j P_ij dP_ij with fp32 P, which
//                     is <dO_i, O_i> for the exact O, and leaves that in the
//                     workspace -- so dK/dV and dsink do not inherit the bf16
//                     rounding of P inside the forward's O (the dsink
//                     precision issue #2969 of the flash-attention profile);
//   bwd_dkdv_kernel   keys fixed (32 per wave, 32x32x16 MFMAs), the G query
//                     heads' Q/dO tiles streamed: S = Q K^T, dP = dO V^T,
//                     dV^T += dO^T P, dK^T += Q^T dS;
//   bwd_dsink_kernel  one work-group per query head, fixed summation order.
// The two-phase split (one pass with rows fixed, one with keys fixed) is the
// flash-attention profile's backward call flow; P and dS are rounded to bf16
// for the MFMAs and every sum is fp32.
#include "attn_common.hpp"
#include "attn_kernels.hpp"
#include "attn_tiles.hpp"


namespace attn {

namespace {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* o;       // forward output, bf16 or fp32
  const uint16_t* dout;
  const float* lse;    // forward LSE [B,Hq,Lq]
  const float* sinks;  // [Hq] or NULL
  float* delta;        // [B,Hq,Lq] workspace: D_i
  float* dq;           // [B,Hq,Lq,D]
  float* dk;           // [B,Hkv,Lk,D]
  float* dv;
  float* dsink;        // [Hq] or NULL
  int B, Hq, Hkv, Lq, Lk, window, n_qtiles;
  float c;      // scale * log2(e)
  float scale;
};

// dsink[h] = -sum over (b, i) of exp(sink_h - LSE) * D, one work-group of
// 1024 threads per head: each thread sums a fixed strided subset (kSinkUnroll
// loads in flight), then a fixed tree.
constexpr int kSinkThreads = 1024;
constexpr int kSinkUnroll = 4;

__global__ __launch_bounds__(kSinkThreads) void bwd_dsink_kernel(BwdArgs a) {
  __shared__ float part[kSinkThreads / 64];
  const int h = blockIdx.x;
  const float sink = a.sinks[h];
  float acc = 0.0f;
  const int n = a.B * a.Lq;
  for (int base = 0; base < n; base += kSinkThreads * kSinkUnroll) {
    float l[kSinkUnroll], d[kSinkUnroll];
#pragma unroll
    for (int u = 0; u < kSinkUnroll; ++u) {
      const int idx = base + u * kSinkThreads + (int)threadIdx.x;
      l[u] = 0.0f;  // unused: a missing row's term is skipped below
      d[u] = 0.0f;
      if (idx < n) {
        const int b = idx / a.Lq, i = idx % a.Lq;
        const size_t r = (size_t)(b * a.Hq + h) * a.Lq + i;
        l[u] = a.lse[r];  // >= sink: the LSE holds the sink term
        d[u] = a.delta[r];
      }
    }
#pragma unroll
    for (int u = 0; u < kSinkUnroll; ++u)
      if (base + u * kSinkThreads + (int)threadIdx.x < n)
        acc -= exp2_fast((sink - l[u]) * kLog2e) * d[u];
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kSinkThreads / 64; ++w) t += part[w];
    a.dsink[h] = t;
  }
}

// ---------------------------------------------------------------------------
// dQ: 4 waves x 32 rows per work-group (the forward's decomposition and K/V
// tile ring).  Per 64-key tile: S^T and dP^T (K and V rows read in key_perm
// order, Q^T and dO^T in VGPRs), dS^T in bf16, dQ^T += K^T dS^T with K^T
// from transposed LDS reads.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void dq_tile(const lds_char* ks_, const lds_char* vs_,
                                        const int (&ka)[D / 16], const int (&va)[2][D / 32],
                                        const bf16x8 (&qf)[D / 16], const bf16x8 (&df)[D / 16],
                                        f32x16 (&o)[D / 32], float& dsum, int kind, int t0,
                                        int vis_lo, int vis_hi, int half, float c, float lse2,
                                        float dl) {
  using L = BfLayout<D>;
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  f32x16 st0 = (f32x16){}, st1 = (f32x16){}, pt0 = (f32x16){}, pt1 = (f32x16){};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 k0 = as_bf16x8(lds_read16(ks_, ka[ks]));
    const bf16x8 k1 = as_bf16x8(lds_read16(ks_, ka[ks] + 32 * L::kRow));
    const bf16x8 v0 = as_bf16x8(lds_read16(vs_, ka[ks]));
    const bf16x8 v1 = as_bf16x8(lds_read16(vs_, ka[ks] + 32 * L::kRow));
    st0 = mfma_32x32x16(k0, qf[ks], st0);
    st1 = mfma_32x32x16(k1, qf[ks], st1);
    pt0 = mfma_32x32x16(v0, df[ks], pt0);
    pt1 = mfma_32x32x16(v1, df[ks], pt1);
  }
  __builtin_amdgcn_s_setprio(3);  // VALU phase: see the forward's softmax
  float sv[32];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    sv[v] = st0[v];
    sv[16 + v] = st1[v];
  }
  // Masked keys get score -inf (P = 0), in one block that only boundary
  // tiles run (a per-element select would run on every tile).
  if (kind == 2) {
    const unsigned lo = (unsigned)(vis_lo - t0);
    const unsigned span = (unsigned)(vis_hi - vis_lo);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const unsigned j = (unsigned)(kb * 32 + key_of_reg(v, half));
        sv[kb * 16 + v] = (j - lo <= span) ? sv[kb * 16 + v] : kNegInf;
      }
  }
  float ds[32];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float dp = kb ? pt1[v] : pt0[v];
      const float p = exp2_fast(__builtin_fmaf(sv[kb * 16 + v], c, -lse2));
      ds[kb * 16 + v] = p * (dp - dl);
      dsum = __builtin_fmaf(p, dp, dsum);
    }
  bf16x8 pf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const float* x = ds + kb * 16 + s2 * 8;
      pf[kb][s2] = pack_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int i = 0; i < 4 * NDB; ++i) {
    const int db = i % NDB, ks2 = i / NDB;
    const int rows = ks2 * 16 * L::kRow;
    const bf16x8 kt = join_tr(lds_read_tr16(ks_, va[0][db] + rows), lds_read_tr16(ks_, va[1][db] + rows));
    o[db] = mfma_32x32x16(kt, pf[ks2 >> 1][ks2 & 1], o[db]);
  }
}

template <int D, bool O_F32>
__global__ __launch_bounds__(kBfThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  lds_char* K0 = BfSmem<D>::template k<0>();
  lds_char* K1 = BfSmem<D>::template k<1>();
  lds_char* V0 = BfSmem<D>::template v<0>();
  lds_char* V1 = BfSmem<D>::template v<1>();

  const int G = a.Hq / a.Hkv;
  const int HG = bf_heads_per_group(G);
  const int rows = kBfWaves / HG * kRowsPerWave;
  const BfWork wk = decode_bf_work<false>(a, G / HG);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int h = wk.kvh * G + wk.hg * HG + wave % HG;
  const int off_q = a.Lk - a.Lq;
  const size_t q_row0 = (size_t)(wk.b * a.Hq + h) * a.Lq;
  const size_t k_row0 = (size_t)(wk.b * a.Hkv + wk.kvh) * a.Lk;
  const uint16_t* kh = a.k + k_row0 * D;
  const uint16_t* vh = a.v + k_row0 * D;

  const int r0 = wk.qt * rows;
  const int r_end = min(r0 + rows, a.Lq);
  const RowSpan wg_span = {r0 + off_q, r_end - 1 + off_q};
  const int w0 = r0 + (wave / HG) * kRowsPerWave;
  const bool wave_active = w0 < a.Lq;
  const RowSpan w_span = {w0 + off_q, min(w0 + kRowsPerWave, a.Lq) - 1 + off_q};
  const int key_lo = a.window > 0 ? max(0, wg_span.p_first - a.window + 1) : 0;
  const int key_hi = wg_span.p_last + 1;
  const int t_begin = key_lo / kBc, t_end = (key_hi + kBc - 1) / kBc;

  TileCopy<D> cp;
  cp.init(wave, lane);
  if (t_begin < t_end) cp.issue(kh, vh, t_begin, a.Lk, K0, V0);

  const int my_row = w0 + col;
  const bool row_valid = my_row < a.Lq;
  const int n_rows = wave_active ? min(kRowsPerWave, a.Lq - w0) : 0;
  // Q^T and dO^T operands (row w0+col, d = ks*16 + half*8 ..): both 32-row
  // blocks are loaded with whole-row instructions at once and turned into the
  // operand layout through the wave's half of K1 / V1, idle until the first
  // ring step refills it.
  bf16x8 qf[D / 16], df[D / 16];
  {
    RowBlockRegs<D> qb, gb;
    qb.load(a.q + (q_row0 + w0) * D, n_rows, lane);
    gb.load(a.dout + (q_row0 + w0) * D, n_rows, lane);
    lds_char* region = (wave < 2 ? K1 : V1) + (wave & 1) * (BfLayout<D>::kBytes / 2);
    qb.to_operand(region, col, half, lane, qf);
    gb.to_operand(region, col, half, lane, df);  // LDS in order: qf was read first
  }
  // An invalid row gets lse2 = +inf: its P is 0 and it adds nothing.
  const float lse2 = row_valid ? a.lse[q_row0 + my_row] * kLog2e : __builtin_huge_valf();
  // D_i = <dO_i, O_i> for dS in this kernel: the lane holds dO at d = 16 ks +
  // 8 half .. +8 of its row (df) and reads O at the same places; the halves'
  // sums meet in pair_sum.
  float dl = 0.0f;
  if (row_valid) {
    const size_t orow = (q_row0 + my_row) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int d0 = ks * 16 + half * 8;
      float ov[8];
      if constexpr (O_F32) {
        const f32x4 o0 = *(const f32x4*)((const float*)a.o + orow + d0);
        const f32x4 o1 = *(const f32x4*)((const float*)a.o + orow + d0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = o0[e];
          ov[e + 4] = o1[e];
        }
      } else {
        const u32x4 w = *(const u32x4*)((const uint16_t*)a.o + orow + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[2 * e] = __builtin_bit_cast(float, w[e] << 16);
          ov[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xffff0000u);
        }
      }
      const u32x4 g = __builtin_bit_cast(u32x4, df[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dl = __builtin_fmaf(__builtin_bit_cast(float, g[e] << 16), ov[2 * e], dl);
        dl = __builtin_fmaf(__builtin_bit_cast(float, g[e] & 0xffff0000u), ov[2 * e + 1], dl);
      }
    }
  }
  dl = pair_sum(dl);
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = (f32x16){};
  float dsum = 0.0f;  // sum_j P_ij dP_ij over this lane's keys
  const int p = my_row + off_q;
  int vis_hi = min(p, a.Lk - 1);
  int vis_lo = a.window > 0 ? p - a.window + 1 : 0;
  if (vis_hi < vis_lo) vis_lo = vis_hi = 1 << 30;  // no visible key: every key masked

  using T = BfTile<D>;
  int ka[D / 16], va[2][D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) ka[ks] = T::off(key_perm(col), (ks * 2 + half) * 16);
  const int vrow = half * 8 + ((lane & 15) >> 2);
  const int vbyte = (((lane >> 4) & 1) * 16 + (lane & 3) * 4) * 2;
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) va[e][db] = T::off(vrow + 4 * e, db * 64 + vbyte);

  auto step = [&](int t, const lds_char* ks_, const lds_char* vs_, lds_char* kn, lds_char* vn) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 1 < t_end) cp.issue(kh, vh, t + 1, a.Lk, kn, vn);
    const int kind = wave_active ? tile_kind(t * kBc, kBc, w_span, a.window, a.Lk) : 0;
    if (kind != 0)
      dq_tile<D>(ks_, vs_, ka, va, qf, df, o, dsum, kind, t * kBc, vis_lo, vis_hi, half, a.c, lse2,
                 dl);
  };
  for (int t = t_begin; t < t_end; t += 2) {
    step(t, K0, V0, K1, V1);
    if (t + 1 >= t_end) break;
    step(t + 1, K1, V1, K0, V0);
  }

  // D_i again, now as sum_j P_ij dP_ij with fp32 P: equal to <dO_i, O_i> for
  // the exact O, free of the bf16 rounding of P that the forward's O carries.
  // The dK/dV kernel, next on the stream, and dsink take it from the
  // workspace.
  const float d_exact = pair_sum(dsum);
  if (row_valid && half == 0) a.delta[q_row0 + my_row] = d_exact;
  // dQ (fp32, 16 KB per wave) through a whole K/V array per wave, once every
  // wave is done with the ring (the last step copies nothing).
  __syncthreads();
  lds_char* st = wave == 0 ? K0 : wave == 1 ? K1 : wave == 2 ? V0 : V1;
  store_rows_staged<D, float>(o, a.scale, st, a.dq + (q_row0 + w0) * D, n_rows, col, half, lane);
}

// ---------------------------------------------------------------------------
// dK, dV: a work-group owns 128 keys of one (batch, KV head), 32 per wave, and
// streams 32-row tiles of Q and dO (plus their LSE and D) of every query head
// of the group whose rows can see those keys, through a two-stage LDS ring.
// v_mfma_f32_32x32x16_bf16 throughout; per step, a wave computes for its 32
// keys x the tile's 32 rows:
//   S  = Q K^T    A: Q rows from LDS, read in key_perm order; B: K^T in VGPRs
//   dP = dO V^T   A: dO rows likewise; B: V^T from the work-group's V block
//   P = exp2(c S - LSE log2e), dS = P (dP - D)   (lane: one key, 16 rows)
//   dV^T += dO^T P, dK^T += Q^T dS   A: transposed LDS reads; B: P and dS
//                 straight from the accumulator registers (key_perm makes their
//                 row order the k order of these B operands)
// The S accumulator starts at -LSE/scale and the dP accumulator at -D, so the
// MFMAs deliver c S - LSE log2e (after one multiply by c) and dP - D directly.
// Every LDS operand read (16 B per lane) feeds a 32x32x16 MFMA: half the LDS
// bytes per flop of 16-key blocks on 16x16x32 MFMAs.  V sits in LDS (not in VGPRs) so
// that K^T, the dK^T/dV^T accumulators and two 32x32 tiles fit in the 256
// registers of two waves per SIMD; its rows are stored in key_perm order
// within each wave's 32 keys, so a V^T operand read has the address of the
// Q row read of the same k-step, and one set of address registers serves Q,
// dO and V.
// ---------------------------------------------------------------------------
constexpr int kKvWaveKeys = 32;
constexpr int kKvKeys = kKvWaveKeys * kBfWaves;  // keys per work-group
constexpr int kKvRows = 32;                      // query rows per streamed tile

template <int D>
struct KvSmem {
  static constexpr int kTile = kKvRows * D * 2;
  template <int I>
  static __device__ __forceinline__ lds_char* q() {
    __shared__ __attribute__((aligned(1024))) char buf[kTile];
    return (lds_char*)buf;
  }
  template <int I>
  static __device__ __forceinline__ lds_char* g() {
    __shared__ __attribute__((aligned(1024))) char buf[kTile];
    return (lds_char*)buf;
  }
  template <int I>
  static __device__ __forceinline__ lds_char* s() {  // 64 LSE slots, then 64 D slots
    __shared__ __attribute__((aligned(256))) char buf[512];
    return (lds_char*)buf;
  }
  static __device__ __forceinline__ lds_char* v() {  // the work-group's V rows
    __shared__ __attribute__((aligned(1024))) char buf[kKvKeys * D * 2];
    return (lds_char*)buf;
  }
};

// Copy of one 32-row tile of Q and dO (swizzled BfTile rows, 1 KB pieces split
// over the 4 waves) and its LSE and D (one dword per lane, waves 0 and 1);
// rows past Lq arrive as zeros.
template <int D>
struct RowTileCopy {
  static constexpr int kRow = D * 2;
  static constexpr int kPieces = kKvRows * kRow / 1024;  // per tensor
  static constexpr int kPerWave = 2 * kPieces / kBfWaves;
  uint32_t off[kPerWave];
  int wave, lane;
  __device__ __forceinline__ void init(int w, int l) {
    wave = w;
    lane = l;
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) off[j] = dma_src_off<D>((w + j * kBfWaves) % kPieces, l);
  }
  __device__ __forceinline__ void issue(const BwdArgs& a, size_t row0, int rows, lds_char* qd,
                                        lds_char* gd, lds_char* sd) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int bytes = rows * kRow;
    const __amdgpu_buffer_rsrc_t qr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + row0 * D), 0, bytes, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t gr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.dout + row0 * D), 0, bytes, kRawBufferWord3);
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int pc = wave + j * kBfWaves;
      if (pc < kPieces)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, qd + pc * 1024, 16, off[j], 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(gr, gd + (pc - kPieces) * 1024, 16, off[j], 0, 0, 0);
    }
    if (wave < 2) {
      const float* src = (wave == 0 ? a.lse : a.delta) + row0;
      const __amdgpu_buffer_rsrc_t sr =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, rows * 4, kRawBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, sd + wave * 256, 4, lane * 4, 0, 0, 0);
    }
#endif
  }
};

// The work-group's V rows [k0, k0 + 128) into the V block: LDS row R (BfTile
// swizzle) holds key k0 + (R & ~31) + key_perm(R & 31); keys past Lk arrive as
// zeros.  32 KB (D = 128) in 1 KB pieces, each wave a quarter.
template <int D>
__device__ __forceinline__ void copy_v_block(const uint16_t* vh, int k0, int Lk, lds_char* dst,
                                             int wave, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = BfLayout<D>;
  constexpr int kPieces = kKvKeys * L::kRow / 1024;
  const int bytes = min(kKvKeys, Lk - k0) * L::kRow;
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)vh + (size_t)k0 * L::kRow), 0, bytes, kRawBufferWord3);
#pragma unroll
  for (int j = 0; j < kPieces / kBfWaves; ++j) {
    const int pc = wave + j * kBfWaves;
    const int R = pc * L::kRowsPerPiece + lane / L::kChunks;
    const int g = (R & ~31) | key_perm(R & 31);
    const int c = (lane % L::kChunks) ^ BfTile<D>::swz(R);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, dst + pc * 1024, 16, (uint32_t)(g * L::kRow + c * 16),
                                             0, 0, 0);
  }
#endif
}

template <int D>
__device__ __forceinline__ void dkdv_tile(const lds_char* qs, const lds_char* gs, const lds_char* ss,
                                          const lds_char* vw, const int (&qa)[D / 16],
                                          const int (&ta)[2][D / 32], const bf16x8 (&kf)[D / 16],
                                          f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], int kind,
                                          int vis_lo, unsigned vis_span, int half, float c,
                                          float inv_scale) {
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int kRow = D * 2;
  // register v of the lane holds row key_of_reg(v, half): rows 8h .. 8h+7
  // (v < 8) and 16+8h .. 16+8h+7 (v >= 8), four per 16 B read
  f32x16 s, dp;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (j >> 1) * 16 + half * 8 + (j & 1) * 4;
    const f32x4 l = *(const __attribute__((address_space(3))) f32x4*)(ss + r * 4);
    const f32x4 d = *(const __attribute__((address_space(3))) f32x4*)(ss + 256 + r * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[4 * j + e] = -l[e] * inv_scale;
      dp[4 * j + e] = -d[e];
    }
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    s = mfma_32x32x16(as_bf16x8(lds_read16(qs, qa[ks])), kf[ks], s);
    dp = mfma_32x32x16(as_bf16x8(lds_read16(gs, qa[ks])), as_bf16x8(lds_read16(vw, qa[ks])), dp);
  }
  // register v sits at row offset key_of_reg(v, 0) from the lane's first row
  // (row_base + 8 half); it is visible iff that offset lies in [vis_lo,
  // vis_lo + vis_span].  Masked pairs get -inf (P = 0) in one block that only
  // boundary steps run.
  __builtin_amdgcn_s_setprio(3);  // VALU phase: see the forward's softmax
  if (kind == 2) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      s[v] = ((unsigned)(key_of_reg(v, 0) - vis_lo) <= vis_span) ? s[v] : kNegInf;
  }
  float pv[16], dsv[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float p = exp2_fast(s[v] * c);
    pv[v] = p;
    dsv[v] = p * dp[v];
  }
  bf16x8 pp[2], pd[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const float* x = pv + 8 * k2;
    const float* y = dsv + 8 * k2;
    pp[k2] = pack_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    pd[k2] = pack_bf16x8(y[0], y[1], y[2], y[3], y[4], y[5], y[6], y[7]);
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int rows = k2 * 16 * kRow;
      const bf16x8 gt = join_tr(lds_read_tr16(gs, ta[0][db] + rows), lds_read_tr16(gs, ta[1][db] + rows));
      dv[db] = mfma_32x32x16(gt, pp[k2], dv[db]);
      const bf16x8 qt = join_tr(lds_read_tr16(qs, ta[0][db] + rows), lds_read_tr16(qs, ta[1][db] + rows));
      dk[db] = mfma_32x32x16(qt, pd[k2], dk[db]);
    }
}

// Two waves per SIMD: D = 128 takes about 250 of their 256 registers each
// (D = 64 is held to the same occupancy).
template <int D>
__global__ __launch_bounds__(kBfThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdArgs a) {
  lds_char* Q0 = KvSmem<D>::template q<0>();
  lds_char* Q1 = KvSmem<D>::template q<1>();
  lds_char* G0 = KvSmem<D>::template g<0>();
  lds_char* G1 = KvSmem<D>::template g<1>();
  lds_char* S0 = KvSmem<D>::template s<0>();
  lds_char* S1 = KvSmem<D>::template s<1>();
  lds_char* VB = KvSmem<D>::v();

  // Key block kb of (batch, KV head) hh.  Each XCD (work-groups are dealt
  // round-robin over 8) runs whole (batch, KV head) groups, so the Q/dO tiles
  // they share stay in its L2, and takes its key blocks in ascending order:
  // under a causal mask the earliest keys see the most rows, so the longest
  // work-groups start first.
  const int nkb = (a.Lk + kKvKeys - 1) / kKvKeys;
  const int nh = a.Hkv * a.B;
  int kb, hh;
  if (nh % 8 == 0) {
    const int per = nh / 8, k = blockIdx.x / 8;
    kb = k / per;
    hh = (blockIdx.x % 8) * per + k % per;
  } else {
    const int id = xcd_remap(blockIdx.x, nkb * nh);
    kb = id % nkb;
    hh = id / nkb;
  }
  const int kvh = hh % a.Hkv;
  const int b = hh / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int k0 = kb * kKvKeys;
  const int kw0 = k0 + wave * kKvWaveKeys;
  const int key = kw0 + col;
  const int off_q = a.Lk - a.Lq;
  const size_t k_row0 = (size_t)(b * a.Hkv + kvh) * a.Lk;

  copy_v_block<D>(a.v + k_row0 * D, k0, a.Lk, VB, wave, lane);
  // K^T B operand of the wave's 32 keys: key col, d = 16 ks + 8 half ..
  bf16x8 kf[D / 16];
  {
    const int kr = min(key, a.Lk - 1);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      kf[ks] = as_bf16x8(*(const u32x4*)(a.k + (k_row0 + kr) * D + ks * 16 + half * 8));
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dk[db] = dv[db] = (f32x16){};

  // query rows that can see a key of [k0, k0 + 128): positions p in
  // [k0, k0 + 127 + window - 1] (or [k0, Lk) without a window)
  const int i_lo = max(0, k0 - off_q);
  const int i_hi = min(a.Lq, (a.window > 0 ? k0 + kKvKeys - 1 + a.window : a.Lk) - off_q);
  const int t_begin = i_lo / kKvRows;
  const int nt = i_hi > i_lo ? (i_hi + kKvRows - 1) / kKvRows - t_begin : 0;
  const int steps = G * nt;

  // per-lane LDS read addresses: Q/dO rows (and V rows) key_perm(col), chunk
  // 2 ks + half; transposed reads: rows 8 half + (l%16)/4 (+4), d = 32 db +
  // 16 ((l/16)%2) + 4 (l%4), as for V^T in the forward
  using T = BfTile<D>;
  int qa[D / 16], ta[2][D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qa[ks] = T::off(key_perm(col), (ks * 2 + half) * 16);
  {
    const int trow = half * 8 + ((lane & 15) >> 2);
    const int tbyte = (((lane >> 4) & 1) * 16 + (lane & 3) * 4) * 2;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) ta[e][db] = T::off(trow + 4 * e, db * 64 + tbyte);
  }
  const int vw_off = wave * kKvWaveKeys * D * 2;

  RowTileCopy<D> cp;
  cp.init(wave, lane);
  // step n: head g = n / nt of the group, row tile t_begin + n % nt
  auto tile_rows = [&](int n, size_t& row0, int& r0) {
    const int h = kvh * G + n / nt;
    r0 = (t_begin + n % nt) * kKvRows;
    row0 = (size_t)(b * a.Hq + h) * a.Lq + r0;
  };
  if (steps > 0) {
    size_t row0;
    int r0;
    tile_rows(0, row0, r0);
    cp.issue(a, row0, min(kKvRows, a.Lq - r0), Q0, G0, S0);
  }
  const float inv_scale = 1.0f / a.scale;
  auto step = [&](int n, const lds_char* qs, const lds_char* gs, const lds_char* ss, lds_char* qn,
                  lds_char* gn, lds_char* sn) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (n + 1 < steps) {
      size_t row0;
      int r0;
      tile_rows(n + 1, row0, r0);
      cp.issue(a, row0, min(kKvRows, a.Lq - r0), qn, gn, sn);
    }
    const int r0 = (t_begin + n % nt) * kKvRows;
    // rows [r0, r0+32) against the wave's keys [kw0, kw0+32)
    const int p_first = r0 + off_q, p_last = min(r0 + kKvRows, a.Lq) - 1 + off_q;
    int kind = 2;
    if (kw0 > p_last || kw0 >= a.Lk || (a.window > 0 && kw0 + kKvWaveKeys - 1 <= p_first - a.window))
      kind = 0;
    else if (r0 + kKvRows <= a.Lq && kw0 + kKvWaveKeys <= a.Lk && kw0 + kKvWaveKeys - 1 <= p_first &&
             (a.window <= 0 || kw0 > p_last - a.window))
      kind = 1;
    if (kind != 0) {
      // offsets o = row - (r0 + 8 half) of the lane's visible rows: o >= key -
      // off_q - r0 - 8 half (causal), o < that + window, o < Lq - r0 - 8 half;
      // none if key >= Lk
      const int o_lo = key - off_q - r0 - 8 * half;
      int o_hi = a.Lq - r0 - 8 * half - 1;
      if (a.window > 0) o_hi = min(o_hi, o_lo + a.window - 1);
      const unsigned span = (key < a.Lk && o_hi >= o_lo) ? (unsigned)(o_hi - o_lo) : 0u;
      const int lo = (key < a.Lk && o_hi >= o_lo) ? o_lo : (1 << 30);
      // the V block's per-wave base is re-derived every step so that the
      // compiler adds it per read instead of holding 8 summed addresses
      int vo = vw_off;
      asm volatile("" : "+s"(vo));
      dkdv_tile<D>(qs, gs, ss, VB + vo, qa, ta, kf, dk, dv, kind, lo, span, half, a.c, inv_scale);
    }
  };
  for (int n = 0; n < steps; n += 2) {
    step(n, Q0, G0, S0, Q1, G1, S1);
    if (n + 1 >= steps) break;
    step(n + 1, Q1, G1, S1, Q0, G0, S0);
  }
  // a work-group with no rows never waited for its V block
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  if (key >= a.Lk) return;
  // accumulator register 4j + e of block db: d = 32 db + 8 j + 4 half + e
  float* dkp = a.dk + (k_row0 + key) * D;
  float* dvp = a.dv + (k_row0 + key) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * db + 8 * j + 4 * half;
      const f32x4 xk = {dk[db][4 * j], dk[db][4 * j + 1], dk[db][4 * j + 2], dk[db][4 * j + 3]};
      const f32x4 xv = {dv[db][4 * j], dv[db][4 * j + 1], dv[db][4 * j + 2], dv[db][4 * j + 3]};
      *(f32x4*)(dkp + d) = xk * a.scale;
      *(f32x4*)(dvp + d) = xv;
    }
}

}  // namespace

hipError_t launch_bwd(const void* q, const void* k, const void* v, const float* sinks,
                      const void* out, const void* dout, const float* lse, float* delta,
                      float* dq, float* dk, float* dv, float* dsink, int B, int Hq, int Hkv,
                      int Lq, int Lk, int D, int window, float scale, bool o_f32,
                      hipStream_t stream) {
  BwdArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = out; a.dout = (const uint16_t*)dout; a.lse = lse; a.sinks = sinks; a.delta = delta;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dsink = dsink;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.window = window;
  a.c = scale * kLog2e;
  a.scale = scale;
  const int HG = bf_heads_per_group(Hq / Hkv);
  const int rows = kBfWaves / HG * kRowsPerWave;
  a.n_qtiles = (Lq + rows - 1) / rows;

  const int dq_grid = a.n_qtiles * (Hq / HG) * B;
  const int kv_grid = (Lk + kKvKeys - 1) / kKvKeys * Hkv * B;
  if (D == 128) {
    if (o_f32) hipLaunchKernelGGL((bwd_dq_kernel<128, true>), dim3(dq_grid), dim3(kBfThreads), 0, stream, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<128, false>), dim3(dq_grid), dim3(kBfThreads), 0, stream, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3(kv_grid), dim3(kBfThreads), 0, stream, a);
  } else {
    if (o_f32) hipLaunchKernelGGL((bwd_dq_kernel<64, true>), dim3(dq_grid), dim3(kBfThreads), 0, stream, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<64, false>), dim3(dq_grid), dim3(kBfThreads), 0, stream, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3(kv_grid), dim3(kBfThreads), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dsink from the D_i that the dQ kernel rewrote
  if (dsink && sinks)
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3(Hq), dim3(kSinkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
