// attn_fwd.hip -- fused tiled exact-attention forward for gfx950 (MI355X).
//
// Each wave owns 32 query rows of one (batch, query head) and walks the K/V
// tiles of the head's KV head (GQA: h / (Hq/Hkv)) that its rows can see; the
// tiles are staged in LDS, double-buffered, one barrier per tile (layout and
// copies of the bf16 path below).  Per tile and wave:
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, K from LDS, Q^T held in VGPRs;
//                   each lane owns one query column and 32 keys of it
//   mask            only on tiles that cut the causal diagonal, the window
//                   edge or the end of the keys
//   online softmax  in the exp2 domain (running max m, partial sums); the
//                   accumulator is rebased only when the max grew by > 8
//                   (2^8 headroom keeps every term finite in fp32); a tile's
//                   fp32 probabilities join l beside the next tile's S^T MFMAs
//   O^T += V^T P^T  V read from LDS with ds_read_b64_tr_b16, P in bf16 (RNE);
//                   the rounded P are summed too (lb), since a lazily rebased
//                   dominant p lies in [1, 2^8) and its rounding (up to 2^-8
//                   relative) must cancel between O's numerator and normaliser
// Finalise: the sink logit joins with the rebased update of the Flint page
// ("fix two"): m' = max(m, sink*log2e), r = 2^(m - m'), e = 2^(sink*log2e - m'),
// O = acc*r/(lb*r + e), LSE = ln2*(m' + log2(l*r + e)).
// A wave's 32-row Q block comes in, and its O block goes out, through LDS as
// whole rows (copy_rows_to_lds, store_rows_staged).
//
// The float32-input variant is the same algorithm on v_mfma_f32_32x32x2_f32
// with 128-row work-groups of one head, 32-key tiles, register-staged copies
// and an fp32 LDS layout.
#include "attn_common.hpp"
#include "attn_kernels.hpp"
#include "attn_tiles.hpp"

#include <type_traits>

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = kRowsPerWave * kWaves;  // query rows per work-group
constexpr float kRebaseThreshold = 8.0f;    // log2 headroom before the accumulator is rebased

// Online-softmax state of the query column a lane owns.
struct Row {
  float m;   // reference max (log2 domain) of acc and l; -inf before any visible key
  float l;   // partial sum of this lane half (fp32 probabilities: the LSE's)
  float mx;  // largest raw score <q, k> seen (kept only when the max logit is asked for)
  float lb;  // partial sum of the probabilities as rounded to bf16 for P V (O's normaliser)
};

// Update the running state with a tile of raw scores s (already masked to -inf),
// turn s into probabilities in place and return the rescale factor for acc.
// With MAXL the exact running maximum of the raw scores is kept in row.mx
// (row.m lags it by up to the rebase threshold).
template <int N, bool MAXL, bool SUM = true>
__device__ __forceinline__ float softmax_tile(float (&s)[N], Row& row, float c) {
  float mx = s[0];
#pragma unroll
  for (int v = 1; v < N; ++v) mx = fmaxf(mx, s[v]);
  mx = pair_max(mx);
  if (MAXL) row.mx = fmaxf(row.mx, mx);
  float m_new = fmaxf(row.m, mx * c);
  float alpha = 1.0f;
  bool need = m_new > row.m + kRebaseThreshold;  // false while m_new = -inf
  if (__builtin_amdgcn_ballot_w64(need)) {
    alpha = need ? exp2_fast(row.m - m_new) : 1.0f;
    row.m = need ? m_new : row.m;
    row.l *= alpha;
    row.lb *= alpha;
  }
  float m_use = row.m == kNegInf ? 0.0f : row.m;
  float sum = 0.0f;
#pragma unroll
  for (int v = 0; v < N; ++v) {
    s[v] = exp2_fast(__builtin_fmaf(s[v], c, -m_use));
    if (SUM) sum += s[v];
  }
  if (SUM) row.l += sum;
  return alpha;
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float cc, float d);
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float cc, float d) {
  *(f32x4*)dst = (f32x4){a, b, cc, d};
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* dst, float a, float b, float cc, float d) {
  *(u32x2*)dst = (u32x2){pack2_bf16(a, b), pack2_bf16(cc, d)};
}

// Finalise with the sink and store O (4 consecutive d per register quad) and LSE.
template <int NDB, typename OutT>
__device__ __forceinline__ void finalize_store(const f32x16 (&o)[NDB], Row row, float sink_l2,
                                               OutT* orow, float* lse_dst, bool valid, int half) {
  float l_tot = pair_sum(row.l);
  float m_fin = fmaxf(row.m, sink_l2);
  float scale_o = 0.0f, lse = kNegInf;
  if (m_fin != kNegInf) {
    float r = exp2_fast(row.m - m_fin);  // row.m = -inf (no key) -> 0
    float den = l_tot * r + exp2_fast(sink_l2 - m_fin);
    scale_o = r / den;
    lse = (m_fin + log2_fast(den)) * kLn2;
  }
  if (!valid) return;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int d = db * 32 + j * 8 + half * 4;
      store4<OutT>(orow + d, o[db][j * 4 + 0] * scale_o, o[db][j * 4 + 1] * scale_o,
                   o[db][j * 4 + 2] * scale_o, o[db][j * 4 + 3] * scale_o);
    }
  }
  if (lse_dst && half == 0) *lse_dst = lse;
}

// Finalise with the sink and store the wave's block of 32 consecutive output
// rows (staged through LDS, see store_rows_staged) and the LSE.
// The accumulator holds sum_j bf16(p_j) v_j, so O is normalised by the sum of
// the same rounded p_j (a dominant key's rounding then cancels); the LSE takes
// the fp32 sum.  The sink has no value vector and joins both unrounded.
template <int D, typename OutT>
__device__ __forceinline__ void finalize_store_rows(const f32x16 (&o)[D / 32], Row row,
                                                    float sink_l2, lds_char* stage, OutT* oblock,
                                                    int nrows, float* lse_dst, int col, int half,
                                                    int lane) {
  float l_tot = pair_sum(row.l);
  float lb_tot = pair_sum(row.lb);
  float m_fin = fmaxf(row.m, sink_l2);
  float scale_o = 0.0f, lse = kNegInf;
  if (m_fin != kNegInf) {
    float r = exp2_fast(row.m - m_fin);  // row.m = -inf (no key) -> 0
    float e_sink = exp2_fast(sink_l2 - m_fin);
    float den = l_tot * r + e_sink;
    scale_o = r / (lb_tot * r + e_sink);
    lse = (m_fin + log2_fast(den)) * kLn2;
  }
  store_rows_staged<D, OutT>(o, scale_o, stage, oblock, nrows, col, half, lane);
  if (lse_dst && half == 0 && col < nrows) *lse_dst = lse;
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  void* out;
  float* lse;
  float* max_row;   // [B,Hq,Lq] largest pre-softmax logit per row, or NULL
  float* max_head;  // [B,Hq] largest per head (filled with -inf beforehand), or NULL
  const int32_t* cu_q;  // packed batch: [B+1] row offsets of the sequences
  const int32_t* cu_k;  // packed batch: [B+1] key offsets
  int total_q, total_k;
  int B, Hq, Hkv, Lq, Lk, window;  // packed batch: Lq = the longest sequence
  float c;      // scale * log2(e)
  float scale;  // softmax scale (the logit is scale * <q, k>)
  int n_qtiles;
};

// Atomic maximum of a float held in global memory (no NaNs): a non-negative
// float orders like its bits as a signed integer, a negative one inversely
// to its bits as an unsigned integer, and -inf (the initial value) is below
// every other value in both orders.
__device__ __forceinline__ void atomic_max_f32(float* addr, float v) {
  const int bits = __float_as_int(v);
  if (bits >= 0)
    atomicMax(reinterpret_cast<int*>(addr), bits);
  else
    atomicMin(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

// Store the max pre-softmax logit of the wave's rows: per row (one lane per
// row) and folded into the head's maximum (one atomic per wave).
__device__ __forceinline__ void store_max_logit(const FwdArgs& a, const Row& row, int b, int h,
                                                int my_row, bool valid, int half, int lane) {
  const float ml = valid ? a.scale * row.mx : kNegInf;  // scale > 0
  if (a.max_row && valid && half == 0) a.max_row[(size_t)(b * a.Hq + h) * a.Lq + my_row] = ml;
  if (a.max_head) {
    const float wm = wave_max(ml);
    if (lane == 0 && wm != kNegInf) atomic_max_f32(a.max_head + b * a.Hq + h, wm);
  }
}

__global__ void fill_kernel(float* p, int n, float value) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

// Decode the work-group id into (b, h, q-tile); longest q-tiles first within
// each (batch, KV head), and the G query heads of a KV head adjacent.
struct Work {
  int b, h, kvh, qt;
};
__device__ __forceinline__ Work decode_work(const FwdArgs& a) {
  int G = a.Hq / a.Hkv;
  int total = a.n_qtiles * a.Hq * a.B;
  int id = xcd_remap(blockIdx.x, total);
  Work w;
  int g = id % G;
  id /= G;
  w.qt = a.n_qtiles - 1 - id % a.n_qtiles;
  id /= a.n_qtiles;
  w.kvh = id % a.Hkv;
  w.b = id / a.Hkv;
  w.h = w.kvh * G + g;
  return w;
}


// One 64-key tile for the wave's 32 rows: S^T = K Q^T, mask, online softmax,
// O^T += V^T P^T.  Operand reads run ahead of the MFMAs that consume them
// (the two S^T accumulators and the D/32 O^T accumulators are independent
// chains, so consecutive MFMAs never wait on each other).
template <int D, bool MAXL>
__device__ __forceinline__ void bf16_tile(const lds_char* ks_, const lds_char* vs_,
                                          const int (&ka)[D / 16], const int (&va)[2][D / 32],
                                          const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32],
                                          Row& row, float (&pend)[32], int kind, int t0,
                                          int vis_lo, int vis_hi, int half, float c) {
  using L = BfLayout<D>;
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int KA = 4;  // K k-steps read ahead (both key blocks)

  // The previous tile's probabilities join the row sum here, beside this
  // tile's S^T MFMAs (the wave has no other VALU work there); the sum is
  // formed in the same order as it would be right after the exponentials.
  float prev = 0.0f;
#pragma unroll
  for (int v = 0; v < 32; ++v) prev += pend[v];

  // S^T for key blocks 0 and 1, k-steps interleaved.
  f32x16 st0 = (f32x16){}, st1 = (f32x16){};
  bf16x8 k0[KS], k1[KS];
#pragma unroll
  for (int ks = 0; ks < KA; ++ks) {
    k0[ks] = as_bf16x8(lds_read16(ks_, ka[ks]));
    k1[ks] = as_bf16x8(lds_read16(ks_, ka[ks] + 32 * L::kRow));
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + KA < KS) {
      k0[ks + KA] = as_bf16x8(lds_read16(ks_, ka[ks + KA]));
      k1[ks + KA] = as_bf16x8(lds_read16(ks_, ka[ks + KA] + 32 * L::kRow));
    }
    st0 = mfma_32x32x16(k0[ks], qf[ks], st0);
    st1 = mfma_32x32x16(k1[ks], qf[ks], st1);
  }
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2 * KA, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + KA < KS) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSgValu, 32 / KS, 0);
  }
  // Keep the sum in this block (it would otherwise sink past the mask branch).
  asm volatile("" : "+v"(prev));
  row.l += prev;

  // The first V operands of P V are read before the softmax, which hides
  // their LDS latency behind it.
  constexpr int NSTEP = 4 * NDB;  // (kb, s2, db) triples
  constexpr int VA = NDB;         // V operands read ahead
  bf16x8 vf[NSTEP];
  auto vread = [&](int i) {
    const int db = i % NDB, ks2 = i / NDB;  // ks2 = kb*2 + s2
    const int rows = ks2 * 16 * L::kRow;
    vf[i] = join_tr(lds_read_tr16(vs_, va[0][db] + rows), lds_read_tr16(vs_, va[1][db] + rows));
  };
#pragma unroll
  for (int i = 0; i < VA; ++i) vread(i);

  // The softmax below runs at raised wave priority: while this wave has VALU
  // work, the SIMD's other wave (in its MFMA phase) issues only between it.
  __builtin_amdgcn_s_setprio(3);
  float s[32];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    s[v] = st0[v];
    s[16 + v] = st1[v];
  }
  if (kind == 2) {
    // keep key offset j iff lo <= j <= hi, as one unsigned compare
    const unsigned lo = (unsigned)(vis_lo - t0);
    const unsigned span = (unsigned)(vis_hi - vis_lo);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const unsigned j = (unsigned)(kb * 32 + key_of_reg(v, half));
        s[kb * 16 + v] = (j - lo <= span) ? s[kb * 16 + v] : kNegInf;
      }
  }
  float alpha = softmax_tile<32, MAXL, false>(s, row, c);
#pragma unroll
  for (int v = 0; v < 32; ++v) pend[v] = s[v];
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
  }
  bf16x8 pf[2][2];
  u32x4 pw[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const float* x = s + kb * 16 + s2 * 8;
      pw[kb][s2] = pack_bf16_words(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
      pf[kb][s2] = __builtin_bit_cast(bf16x8, pw[kb][s2]);
    }
  row.lb = sum_bf16_words(pw[1][0], pw[1][1], sum_bf16_words(pw[0][0], pw[0][1], row.lb));

  __builtin_amdgcn_s_setprio(0);
  // O^T += V^T P^T: step (kb, s2) feeds the D/32 independent accumulators.
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    if (i + VA < NSTEP) vread(i + VA);
    const int db = i % NDB, ks2 = i / NDB;
    o[db] = mfma_32x32x16(vf[i], pf[ks2 >> 1][ks2 & 1], o[db]);
  }
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    if (i + VA < NSTEP) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 1);
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 1);
  }
}


// VARLEN: a packed batch (q [Hq,total_q,D], k/v [Hkv,total_k,D]); sequence b
// owns rows cu_q[b].. and keys cu_k[b].., and a work-group whose q-tile lies
// past its sequence's rows leaves at once.
template <int D, bool OUT_F32, bool MAXL, bool VARLEN>
__global__ __launch_bounds__(kBfThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  using L = BfLayout<D>;
  using OutT = typename std::conditional<OUT_F32, float, uint16_t>::type;
  lds_char* K0 = BfSmem<D>::template k<0>();
  lds_char* K1 = BfSmem<D>::template k<1>();
  lds_char* V0 = BfSmem<D>::template v<0>();
  lds_char* V1 = BfSmem<D>::template v<1>();

  const int G = a.Hq / a.Hkv;
  const int HG = bf_heads_per_group(G);
  const int rows = kBfWaves / HG * kRowsPerWave;  // query rows per work-group
  const BfWork wk = decode_bf_work<VARLEN>(a, G / HG);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int h = wk.kvh * G + wk.hg * HG + wave % HG;  // this wave's query head

  // Rows and keys of this (batch, head): dense [B,H,L,D], or one sequence of
  // a packed batch (offsets clamped into the packed tensors).
  int Lq = a.Lq, Lk = a.Lk;
  size_t q_row0, k_row0;  // first row of this (sequence, head) in q/out and in k/v
  if constexpr (VARLEN) {
    const int q0 = min(max(a.cu_q[wk.b], 0), a.total_q);
    const int k0 = min(max(a.cu_k[wk.b], 0), a.total_k);
    Lq = min(max(a.cu_q[wk.b + 1], q0), a.total_q) - q0;
    Lk = min(max(a.cu_k[wk.b + 1], k0), a.total_k) - k0;
    if (wk.qt * rows >= Lq) return;  // uniform: no barrier has been reached
    q_row0 = (size_t)h * a.total_q + q0;
    k_row0 = (size_t)wk.kvh * a.total_k + k0;
  } else {
    q_row0 = (size_t)(wk.b * a.Hq + h) * Lq;
    k_row0 = (size_t)(wk.b * a.Hkv + wk.kvh) * Lk;
  }
  const int off_q = Lk - Lq;
  const uint16_t* qh = (const uint16_t*)a.q + q_row0 * D;
  const uint16_t* kh = (const uint16_t*)a.k + k_row0 * D;
  const uint16_t* vh = (const uint16_t*)a.v + k_row0 * D;

  const int r0 = wk.qt * rows;
  const int r_end = min(r0 + rows, Lq);
  const RowSpan wg_span = {r0 + off_q, r_end - 1 + off_q};
  const int w0 = r0 + (wave / HG) * kRowsPerWave;
  const bool wave_active = w0 < Lq;
  const RowSpan w_span = {w0 + off_q, min(w0 + kRowsPerWave, Lq) - 1 + off_q};
  const int key_lo = a.window > 0 ? max(0, wg_span.p_first - a.window + 1) : 0;
  const int key_hi = wg_span.p_last + 1;
  const int t_begin = key_lo / kBc, t_end = (key_hi + kBc - 1) / kBc;

  // A wave's 32-row Q and O blocks (32 x D bf16, half of one K/V array) are
  // staged in LDS: waves 0 and 1 use a K array, waves 2 and 3 the V array.
  using T = BfTile<D>;
  const int blk = (wave & 1) * (L::kBytes / 2);
  const int n_rows = wave_active ? min(kRowsPerWave, Lq - w0) : 0;
  const int my_row = w0 + col;
  const bool row_valid = my_row < Lq;

  // Q^T operand: lane holds query row w0+col, d = ks*16 + half*8 .. +8.  The
  // block comes in through stage 1, idle until the first ring step refills it.
  bf16x8 qf[D / 16];
  lds_char* qst = (wave < 2 ? K1 : V1) + blk;
  copy_rows_to_lds<D>(qh + (size_t)w0 * D, n_rows, qst, lane);

  // Two-stage ring: tile t lives in stage (t - t_begin) % 2.
  TileCopy<D> cp;
  cp.init(wave, lane);
  if (t_begin < t_end) cp.issue(kh, vh, t_begin, Lk, K0, V0);  // no tile: no key visible

  // The Q copy was issued before the tile's, so it is done once only the
  // tile's copies are outstanding.
  if (t_begin < t_end)
    __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(2 * L::kPerWave));
  else
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = as_bf16x8(lds_read16(qst, T::off(col, (ks * 2 + half) * 16)));
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = (f32x16){};
  Row row = {kNegInf, 0.0f, kNegInf, 0.0f};
  float pend[32];  // probabilities of the last computed tile, not yet in row.l
#pragma unroll
  for (int v = 0; v < 32; ++v) pend[v] = 0.0f;
  const int p = my_row + off_q;
  int vis_hi = min(p, Lk - 1);
  int vis_lo = a.window > 0 ? p - a.window + 1 : 0;
  // A row before every key (p < 0: more queries than keys in a packed batch)
  // sees nothing; an empty range would wrap in the unsigned mask compare, so
  // it is moved far past every key instead.
  if (vis_hi < vis_lo) vis_lo = vis_hi = 1 << 30;

  // Per-lane operand read addresses within a stage.  K: row key_perm(col),
  // chunk ks*2 + half.  V (transposed reads): keys half*8 + (lane%16)/4 + 4e,
  // d = db*32 + ((lane/16)%2)*16 + (lane%4)*4.
  int ka[D / 16], va[2][D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) ka[ks] = T::off(key_perm(col), (ks * 2 + half) * 16);
  const int vrow = half * 8 + ((lane & 15) >> 2);
  const int vbyte = (((lane >> 4) & 1) * 16 + (lane & 3) * 4) * 2;
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) va[e][db] = T::off(vrow + 4 * e, db * 64 + vbyte);

  // One ring step: wait for tile t (the only copies in flight), release the
  // stage of tile t-1 and refill it with tile t+1, compute tile t.
  auto step = [&](int t, const lds_char* ks_, const lds_char* vs_, lds_char* kn, lds_char* vn) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 1 < t_end) cp.issue(kh, vh, t + 1, Lk, kn, vn);
    const int kind = wave_active ? tile_kind(t * kBc, kBc, w_span, a.window, Lk) : 0;
    if (kind != 0)
      bf16_tile<D, MAXL>(ks_, vs_, ka, va, qf, o, row, pend, kind, t * kBc, vis_lo, vis_hi,
                         half, a.c);
  };
  for (int t = t_begin; t < t_end; t += 2) {
    step(t, K0, V0, K1, V1);
    if (t + 1 >= t_end) break;
    step(t + 1, K1, V1, K0, V0);
  }
  {
    float prev = 0.0f;
#pragma unroll
    for (int v = 0; v < 32; ++v) prev += pend[v];
    row.l += prev;
  }

  // O staging: with bf16 output a wave's block fits the stage that held tile
  // t_end-2 (every wave passed the last step's barrier after computing it, and
  // no copy refills it); an f32 block needs a whole K/V array per wave, after
  // a barrier.
  lds_char* ost;
  if constexpr (OUT_F32) {
    __syncthreads();
    ost = wave == 0 ? K0 : wave == 1 ? K1 : wave == 2 ? V0 : V1;
  } else {
    const bool free0 = ((t_end - t_begin) & 1) == 0;
    ost = (wave < 2 ? (free0 ? K0 : K1) : (free0 ? V0 : V1)) + blk;
  }
  const float sink_l2 = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
  OutT* oblock = (OutT*)a.out + (q_row0 + w0) * D;
  float* lse_dst = a.lse ? a.lse + q_row0 + my_row : nullptr;
  finalize_store_rows<D, OutT>(o, row, sink_l2, ost, oblock, n_rows, lse_dst, col, half, lane);
  if (MAXL) store_max_logit(a, row, wk.b, h, my_row, row_valid, half, lane);
}

// ------------------------------------------------------------------------
// float32 inputs (v_mfma_f32_32x32x2_f32)
// ------------------------------------------------------------------------
template <int D, bool OUT_F32, bool MAXL>
__global__ __launch_bounds__(kThreads, 1) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BC = 32;
  constexpr int PITCH = D + 1;  // floats per LDS row (odd pitch spreads rows over banks)
  constexpr int TILE_FLOATS = BC * PITCH;
  constexpr int KS = D / 2;
  constexpr int NDB = D / 32;
  constexpr int LOADS = BC * D / 4 / kThreads;
  using OutT = typename std::conditional<OUT_F32, float, uint16_t>::type;

  __shared__ float smem[2][TILE_FLOATS];  // [K/V]; single buffer, registers prefetch

  const Work wk = decode_work(a);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int off_q = a.Lk - a.Lq;

  const float* qh = (const float*)a.q + ((size_t)(wk.b * a.Hq + wk.h) * a.Lq) * D;
  const float* kh = (const float*)a.k + ((size_t)(wk.b * a.Hkv + wk.kvh) * a.Lk) * D;
  const float* vh = (const float*)a.v + ((size_t)(wk.b * a.Hkv + wk.kvh) * a.Lk) * D;

  const int r0 = wk.qt * kBr;
  const int r_end = min(r0 + kBr, a.Lq);
  RowSpan wg_span = {r0 + off_q, r_end - 1 + off_q};
  const int w0 = r0 + wave * kRowsPerWave;
  const bool wave_active = w0 < a.Lq;
  RowSpan w_span = {w0 + off_q, min(w0 + kRowsPerWave, a.Lq) - 1 + off_q};
  int key_lo = a.window > 0 ? max(0, wg_span.p_first - a.window + 1) : 0;
  int key_hi = wg_span.p_last + 1;
  const int t_begin = key_lo / BC, t_end = (key_hi + BC - 1) / BC;

  const int my_row = w0 + col;
  const bool row_valid = my_row < a.Lq;
  float qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = row_valid ? qh[(size_t)my_row * D + ks * 2 + half] : 0.0f;

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = (f32x16){};
  Row row = {kNegInf, 0.0f, kNegInf, 0.0f};
  const int p = my_row + off_q;
  const int vis_hi = min(p, a.Lk - 1);
  const int vis_lo = a.window > 0 ? p - a.window + 1 : 0;

  f32x4 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int cid = threadIdx.x + i * kThreads;
      int r = cid / (D / 4), c4 = cid % (D / 4);
      int key = min(t * BC + r, a.Lk - 1);
      kreg[i] = *(const f32x4*)(kh + (size_t)key * D + c4 * 4);
      vreg[i] = *(const f32x4*)(vh + (size_t)key * D + c4 * 4);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int cid = threadIdx.x + i * kThreads;
      int r = cid / (D / 4), c4 = cid % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        smem[0][r * PITCH + c4 * 4 + e] = kreg[i][e];
        smem[1][r * PITCH + c4 * 4 + e] = vreg[i][e];
      }
    }
  };

  const int k_row = key_perm(col);
  if (t_begin < t_end) load_tile(t_begin);
  for (int t = t_begin; t < t_end; ++t) {
    __syncthreads();  // every wave is done with the previous tile
    store_tile();
    if (t + 1 < t_end) load_tile(t + 1);
    __syncthreads();
    const int t0 = t * BC;
    const int kind = wave_active ? tile_kind(t0, BC, w_span, a.window, a.Lk) : 0;
    if (kind != 0) {
      const float* ks_ = smem[0];
      const float* vs_ = smem[1];
      f32x16 st = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) st = mfma_32x32x2(ks_[k_row * PITCH + ks * 2 + half], qf[ks], st);
      float s[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = st[v];
      if (kind == 2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int j = t0 + key_of_reg(v, half);
          bool vis = (j >= vis_lo) & (j <= vis_hi);
          s[v] = vis ? s[v] : kNegInf;
        }
      }
      float alpha = softmax_tile<16, MAXL>(s, row, a.c);
      if (alpha != 1.0f) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      }
      // O^T += V^T P^T, 2 keys per step: step u takes register u of each half.
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          int key = key_of_reg(u, half);
          o[db] = mfma_32x32x2(vs_[key * PITCH + db * 32 + col], s[u], o[db]);
        }
    }
  }

  const float sink_l2 = a.sinks ? a.sinks[wk.h] * kLog2e : kNegInf;
  OutT* orow = (OutT*)a.out + ((size_t)(wk.b * a.Hq + wk.h) * a.Lq + my_row) * D;
  float* lse_dst = a.lse ? a.lse + (size_t)(wk.b * a.Hq + wk.h) * a.Lq + my_row : nullptr;
  finalize_store<NDB, OutT>(o, row, sink_l2, orow, lse_dst, row_valid, half);
  if (MAXL) store_max_logit(a, row, wk.b, wk.h, my_row, row_valid, half, lane);
}

template <typename K>
hipError_t launch(K kernel, int threads, const FwdArgs& a, hipStream_t stream, int heads_per_wg) {
  int total = a.n_qtiles * (a.Hq / heads_per_wg) * a.B;
  hipLaunchKernelGGL(kernel, dim3(total), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

template <bool OUT, bool MAXL>
hipError_t launch_typed(const FwdArgs& a, int D, bool in_f32, hipStream_t stream) {
  if (!in_f32) {
    const int HG = bf_heads_per_group(a.Hq / a.Hkv);
    return D == 128 ? launch(fwd_bf16_kernel<128, OUT, MAXL, false>, kBfThreads, a, stream, HG)
                    : launch(fwd_bf16_kernel<64, OUT, MAXL, false>, kBfThreads, a, stream, HG);
  }
  return D == 128 ? launch(fwd_f32_kernel<128, OUT, MAXL>, kThreads, a, stream, 1)
                  : launch(fwd_f32_kernel<64, OUT, MAXL>, kThreads, a, stream, 1);
}

}  // namespace

hipError_t launch_fwd(const void* q, const void* k, const void* v, const float* sinks, void* out,
                      float* lse, float* max_row, float* max_head, int B, int Hq, int Hkv, int Lq,
                      int Lk, int D, int window, float scale, bool in_f32, bool out_f32,
                      hipStream_t stream) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.sinks = sinks; a.out = out; a.lse = lse;
  a.max_row = max_row; a.max_head = max_head;
  a.cu_q = a.cu_k = nullptr;
  a.total_q = a.total_k = 0;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.window = window;
  a.c = scale * kLog2e;
  a.scale = scale;
  if (!in_f32) {
    const int rows = kBfWaves / bf_heads_per_group(Hq / Hkv) * kRowsPerWave;
    a.n_qtiles = (Lq + rows - 1) / rows;
  } else {
    a.n_qtiles = (Lq + kBr - 1) / kBr;
  }
  const bool maxl = max_row || max_head;
  if (max_head) {
    const int n = B * Hq;
    hipLaunchKernelGGL(fill_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, max_head, n,
                       kNegInf);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (out_f32) return maxl ? launch_typed<true, true>(a, D, in_f32, stream)
                           : launch_typed<true, false>(a, D, in_f32, stream);
  return maxl ? launch_typed<false, true>(a, D, in_f32, stream)
              : launch_typed<false, false>(a, D, in_f32, stream);
}

hipError_t launch_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_q,
                             const int32_t* cu_k, const float* sinks, void* out, float* lse, int B,
                             int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q, int D,
                             int window, float scale, bool out_f32, hipStream_t stream) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.sinks = sinks; a.out = out; a.lse = lse;
  a.max_row = a.max_head = nullptr;
  a.cu_q = cu_q; a.cu_k = cu_k; a.total_q = total_q; a.total_k = total_k;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = max_seqlen_q; a.Lk = 0; a.window = window;
  a.c = scale * kLog2e;
  a.scale = scale;
  const int HG = bf_heads_per_group(Hq / Hkv);
  const int rows = kBfWaves / HG * kRowsPerWave;
  a.n_qtiles = (max_seqlen_q + rows - 1) / rows;
  if (D == 128)
    return out_f32 ? launch(fwd_bf16_kernel<128, true, false, true>, kBfThreads, a, stream, HG)
                   : launch(fwd_bf16_kernel<128, false, false, true>, kBfThreads, a, stream, HG);
  return out_f32 ? launch(fwd_bf16_kernel<64, true, false, true>, kBfThreads, a, stream, HG)
                 : launch(fwd_bf16_kernel<64, false, false, true>, kBfThreads, a, stream, HG);
}

}  // namespace attn
