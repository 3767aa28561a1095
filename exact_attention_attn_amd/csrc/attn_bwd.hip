// attn_bwd.hip -- backward of the sink/window/GQA attention for gfx950.
//
// Given dO and the forward's O and LSE (natural log, sink included), with
// P_ij = exp(s_ij - LSE_i), Psink_i = exp(sink - LSE_i) and D_i = <dO_i, O_i>:
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q,  dsink_h = -sum_{b,i} Psink_i D_i
// (the sink joins the normaliser and has no value vector, so it enters dS
// only through D).  Four kernels, all deterministic (no atomics):
//   bwd_delta_kernel  D_i = <dO_i, O_i> from the forward's O, for dS;
//   bwd_dq_kernel     rows fixed, K/V tiles streamed (the forward's layout):
//                     S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T; it
//                     also sums D_i = sum_j P_ij dP_ij with fp32 P, which is
//                     <dO_i, O_i> for the exact O -- so dsink does not inherit
//                     the bf16 rounding of P inside the forward's O (the dsink
//                     precision issue #2969 of the flash-attention profile);
//   bwd_dsink_kernel  one work-group per query head, fixed summation order;
//   bwd_dkdv_kernel   keys fixed (16 per wave, 16x16x32 MFMAs), the G query
//                     heads' Q/dO tiles streamed: S = Q K^T, dP = dO V^T,
//                     dV^T += dO^T P, dK^T += Q^T dS.
// The two-phase split (dK/dV, then dQ) is the flash-attention profile's
// backward call flow; P and dS are rounded to bf16 for the MFMAs and every
// sum is fp32.
#include "attn_common.hpp"
#include "attn_kernels.hpp"
#include "attn_tiles.hpp"

#include <type_traits>

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

// ---------------------------------------------------------------------------
// D_i = <dO_i, O_i>: 16 lanes per row, D/16 elements each, fixed reduction.
// A 16-lane group takes kDeltaRows rows per pass and issues all their loads
// (non-temporal: every byte is read once) before the first product.
// ---------------------------------------------------------------------------
constexpr int kDeltaRows = 4;

template <int D, bool O_F32>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  constexpr int E = D / 16;  // elements per lane: 8 (D = 128) or 4 (D = 64)
  constexpr int R = kDeltaRows;
  using OT = typename std::conditional<O_F32, float, uint16_t>::type;
  using GV = typename std::conditional<E == 8, u32x4, u32x2>::type;  // E bf16
  constexpr int ON = E * (int)sizeof(OT) / 16 > 0 ? E * (int)sizeof(OT) / 16 : 1;
  using OV = typename std::conditional<E * sizeof(OT) >= 16, u32x4, u32x2>::type;
  const long long rows = (long long)a.B * a.Hq * a.Lq;
  const int sub = threadIdx.x & 15;
  const long long groups = (long long)gridDim.x * 16;
  for (long long row0 = ((long long)blockIdx.x * 16 + (threadIdx.x >> 4)) * R; row0 < rows;
       row0 += groups * R) {
    GV g[R];
    OV o[R][ON];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const long long row = min(row0 + r, rows - 1);  // in bounds; the extra rows are not stored
      g[r] = __builtin_nontemporal_load((const GV*)(a.dout + row * D + sub * E));
#pragma unroll
      for (int j = 0; j < ON; ++j)
        o[r][j] = __builtin_nontemporal_load((const OV*)((const OT*)a.o + row * D + sub * E) + j);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint16_t* gs = (const uint16_t*)&g[r];
      const OT* os = (const OT*)&o[r][0];
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float go = __builtin_bit_cast(float, (uint32_t)gs[e] << 16);
        float ov;
        if constexpr (O_F32)
          ov = os[e];
        else
          ov = __builtin_bit_cast(float, (uint32_t)os[e] << 16);
        acc = __builtin_fmaf(go, ov, acc);
      }
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
      if (sub == 0 && row0 + r < rows) a.delta[row0 + r] = acc;
    }
  }
}

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
  float ds[32];
  const unsigned lo = (unsigned)(vis_lo - t0);
  const unsigned span = (unsigned)(vis_hi - vis_lo);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float s = kb ? st1[v] : st0[v];
      const float dp = kb ? pt1[v] : pt0[v];
      float p = exp2_fast(__builtin_fmaf(s, c, -lse2));
      if (kind == 2) {
        const unsigned j = (unsigned)(kb * 32 + key_of_reg(v, half));
        p = (j - lo <= span) ? p : 0.0f;
      }
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
#pragma unroll
  for (int i = 0; i < 4 * NDB; ++i) {
    const int db = i % NDB, ks2 = i / NDB;
    const int rows = ks2 * 16 * L::kRow;
    const bf16x8 kt = join_tr(lds_read_tr16(ks_, va[0][db] + rows), lds_read_tr16(ks_, va[1][db] + rows));
    o[db] = mfma_32x32x16(kt, pf[ks2 >> 1][ks2 & 1], o[db]);
  }
}

template <int D>
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
  const float dl = row_valid ? a.delta[q_row0 + my_row] : 0.0f;
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
  // It replaces the workspace value (the dK/dV kernel, earlier on the stream,
  // is done with it) for dsink.
  const float d_exact = pair_sum(dsum);
  if (row_valid && half == 0) a.delta[q_row0 + my_row] = d_exact;
  // dQ (fp32, 16 KB per wave) through a whole K/V array per wave, once every
  // wave is done with the ring (the last step copies nothing).
  __syncthreads();
  lds_char* st = wave == 0 ? K0 : wave == 1 ? K1 : wave == 2 ? V0 : V1;
  store_rows_staged<D, float>(o, a.scale, st, a.dq + (q_row0 + w0) * D, n_rows, col, half, lane);
}

// ---------------------------------------------------------------------------
// dK, dV: a work-group owns 64 keys of one (batch, KV head), 16 per wave, and
// streams 32-row tiles of Q and dO (plus their LSE and D) of every query head
// of the group whose rows can see those keys, through a two-stage LDS ring.
//
// v_mfma_f32_16x16x32_bf16 throughout.  S = Q K^T puts the keys in the lane
// (column) dimension: lane l of lane group g = l/16 holds key l%16 and, over
// its 2 row blocks x 4 registers, rows 8g .. 8g+7 of the tile -- because the
// A-operand rows of block b are read in the order m -> 8(m/4) + 4b + m%4.
// That is exactly the k-order the B operand (P or dS, rows x keys) of
// dV^T += dO^T P and dK^T += Q^T dS needs, so P and dS go to the MFMAs
// straight from their registers; dO^T and Q^T come from transposed LDS reads.
// ---------------------------------------------------------------------------
constexpr int kKvKeys = 64;  // keys per work-group
constexpr int kKvWaveKeys = 16;
constexpr int kKvRows = 32;  // query rows per streamed tile

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
  static __device__ __forceinline__ lds_char* s() {  // 64 LSE values, then 64 D values
    __shared__ __attribute__((aligned(256))) char buf[512];
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

template <int D>
__device__ __forceinline__ void dkdv_tile(const lds_char* qs, const lds_char* gs, const lds_char* ss,
                                          const int (&qa)[2][D / 32], const int (&ta)[2][D / 16],
                                          const bf16x8 (&kf)[D / 32], const bf16x8 (&vf)[D / 32],
                                          f32x4 (&dk)[D / 16], f32x4 (&dv)[D / 16], int kind,
                                          int row_base, int key, int p_off, int Lq, int Lk,
                                          int window, int g16, float c) {
  constexpr int KS = D / 32;
  constexpr int NDB = D / 16;
  f32x4 s[2] = {(f32x4){}, (f32x4){}}, dp[2] = {(f32x4){}, (f32x4){}};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = mfma_16x16x32(as_bf16x8(lds_read16(qs, qa[b][ks])), kf[ks], s[b]);
      dp[b] = mfma_16x16x32(as_bf16x8(lds_read16(gs, qa[b][ks])), vf[ks], dp[b]);
    }
  // LSE and D of the lane group's rows 8g16 .. 8g16+7
  const f32x4 l0 = *(const __attribute__((address_space(3))) f32x4*)(ss + g16 * 32);
  const f32x4 l1 = *(const __attribute__((address_space(3))) f32x4*)(ss + g16 * 32 + 16);
  const f32x4 d0 = *(const __attribute__((address_space(3))) f32x4*)(ss + 256 + g16 * 32);
  const f32x4 d1 = *(const __attribute__((address_space(3))) f32x4*)(ss + 256 + g16 * 32 + 16);
  float pv[8], dsv[8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lse = b ? l1[r] : l0[r];
      const float dlt = b ? d1[r] : d0[r];
      float p = exp2_fast(__builtin_fmaf(s[b][r], c, -lse * kLog2e));
      if (kind == 2) {
        const int i = row_base + 8 * g16 + 4 * b + r;  // query row
        const int pos = i + p_off;
        const bool vis = i < Lq && key < Lk && key <= pos && (window <= 0 || key > pos - window);
        p = vis ? p : 0.0f;
      }
      pv[4 * b + r] = p;
      dsv[4 * b + r] = p * (dp[b][r] - dlt);
    }
  const bf16x8 pp = pack_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
  const bf16x8 pd = pack_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const bf16x8 gt = join_tr(lds_read_tr16(gs, ta[0][db]), lds_read_tr16(gs, ta[1][db]));
    dv[db] = mfma_16x16x32(gt, pp, dv[db]);
    const bf16x8 qt = join_tr(lds_read_tr16(qs, ta[0][db]), lds_read_tr16(qs, ta[1][db]));
    dk[db] = mfma_16x16x32(qt, pd, dk[db]);
  }
}

// At most two waves per SIMD: the compiler then schedules with up to 256
// registers (176 used) instead of fitting three waves in 160, and the backward
// measured 3% faster on both the sliding-window and causal shapes.
template <int D>
__global__ __launch_bounds__(kBfThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdArgs a) {
  lds_char* Q0 = KvSmem<D>::template q<0>();
  lds_char* Q1 = KvSmem<D>::template q<1>();
  lds_char* G0 = KvSmem<D>::template g<0>();
  lds_char* G1 = KvSmem<D>::template g<1>();
  lds_char* S0 = KvSmem<D>::template s<0>();
  lds_char* S1 = KvSmem<D>::template s<1>();

  const int nkb = (a.Lk + kKvKeys - 1) / kKvKeys;
  const int id = xcd_remap(blockIdx.x, nkb * a.Hkv * a.B);
  const int kb = id % nkb;
  const int kvh = (id / nkb) % a.Hkv;
  const int b = id / (nkb * a.Hkv);
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g16 = lane >> 4;
  const int k0 = kb * kKvKeys;
  const int kw0 = k0 + wave * kKvWaveKeys;
  const int key = kw0 + (lane & 15);
  const int off_q = a.Lk - a.Lq;
  const size_t k_row0 = (size_t)(b * a.Hkv + kvh) * a.Lk;

  // K^T / V^T B operands of the wave's 16 keys: key l%16, d = 32ks + 8*(l/16) ..
  bf16x8 kf[D / 32], vf[D / 32];
  {
    const int kr = min(key, a.Lk - 1);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      kf[ks] = as_bf16x8(*(const u32x4*)(a.k + (k_row0 + kr) * D + ks * 32 + g16 * 8));
      vf[ks] = as_bf16x8(*(const u32x4*)(a.v + (k_row0 + kr) * D + ks * 32 + g16 * 8));
    }
  }
  f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) dk[db] = dv[db] = (f32x4){};

  // query rows that can see a key of [k0, k0 + 64): positions p in
  // [k0, k0 + 63 + window - 1] (or [k0, Lk) without a window)
  const int i_lo = max(0, k0 - off_q);
  const int i_hi = min(a.Lq, (a.window > 0 ? k0 + kKvKeys - 1 + a.window : a.Lk) - off_q);
  const int t_begin = i_lo / kKvRows;
  const int nt = i_hi > i_lo ? (i_hi + kKvRows - 1) / kKvRows - t_begin : 0;
  const int steps = G * nt;

  // per-lane LDS read addresses: Q/dO rows of block b in the order
  // m -> 8(m/4) + 4b + m%4, chunk 4ks + g16; transposed reads: rows 8g16 +
  // (l%16)/4 (+4), d = 16db + 4((l%16)%4)
  using T = BfTile<D>;
  int qa[2][D / 32], ta[2][D / 16];
  {
    const int m = lane & 15;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        qa[bb][ks] = T::off(8 * (m >> 2) + 4 * bb + (m & 3), (4 * ks + g16) * 16);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        ta[e][db] = T::off(8 * g16 + (m >> 2) + 4 * e, 2 * (16 * db + 4 * (m & 3)));
  }

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
    // rows [r0, r0+32) against the wave's keys [kw0, kw0+16)
    const int p_first = r0 + off_q, p_last = min(r0 + kKvRows, a.Lq) - 1 + off_q;
    int kind = 2;
    if (kw0 > p_last || kw0 >= a.Lk || (a.window > 0 && kw0 + kKvWaveKeys - 1 <= p_first - a.window))
      kind = 0;
    else if (r0 + kKvRows <= a.Lq && kw0 + kKvWaveKeys <= a.Lk && kw0 + kKvWaveKeys - 1 <= p_first &&
             (a.window <= 0 || kw0 > p_last - a.window))
      kind = 1;
    if (kind != 0)
      dkdv_tile<D>(qs, gs, ss, qa, ta, kf, vf, dk, dv, kind, r0, key, off_q, a.Lq, a.Lk, a.window,
                   g16, a.c);
  };
  for (int n = 0; n < steps; n += 2) {
    step(n, Q0, G0, S0, Q1, G1, S1);
    if (n + 1 >= steps) break;
    step(n + 1, Q1, G1, S1, Q0, G0, S0);
  }

  if (key >= a.Lk) return;
  float* dkp = a.dk + (k_row0 + key) * D;
  float* dvp = a.dv + (k_row0 + key) * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const int d = 16 * db + 4 * g16;
    *(f32x4*)(dkp + d) = dk[db] * a.scale;
    *(f32x4*)(dvp + d) = dv[db];
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

  const long long nrows = (long long)B * Hq * Lq;
  const int pre_grid = (int)min((nrows + 16 * kDeltaRows - 1) / (16 * kDeltaRows), 65536LL);
  if (D == 128) {
    if (o_f32) hipLaunchKernelGGL((bwd_delta_kernel<128, true>), dim3(pre_grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((bwd_delta_kernel<128, false>), dim3(pre_grid), dim3(256), 0, stream, a);
  } else {
    if (o_f32) hipLaunchKernelGGL((bwd_delta_kernel<64, true>), dim3(pre_grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((bwd_delta_kernel<64, false>), dim3(pre_grid), dim3(256), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int dq_grid = a.n_qtiles * (Hq / HG) * B;
  const int kv_grid = (Lk + kKvKeys - 1) / kKvKeys * Hkv * B;
  if (D == 128) {
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3(kv_grid), dim3(kBfThreads), 0, stream, a);
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(dq_grid), dim3(kBfThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3(kv_grid), dim3(kBfThreads), 0, stream, a);
    hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(dq_grid), dim3(kBfThreads), 0, stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dsink from the D_i that the dQ kernel rewrote
  if (dsink && sinks)
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3(Hq), dim3(kSinkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
