// attn_decode.hip -- split-KV decode and the valid-split LSE combine (gfx950).
//
// Decode: the work items are the splits of every (sequence, KV head,
// query-column group).  The G = Hq/Hkv query heads that share a KV head are
// the columns of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so each K/V byte of a
// split is read from HBM once for all of them.  Each work-group streams a
// contiguous range of items (about one with the launch's grid), 128-key
// tiles staged through LDS, with the next tile (and, at an item's end, the
// next item's first tile and Q) prefetched into registers while the current
// tile is computed.  Wave w scores keys [32w, 32w+32) of every tile with its own
// online-softmax state; at the end of an item the four states are merged
// through LDS into the split's normalised partial output and sink-free LSE.
//
// Combine: one wave per (sequence, query head).  Lane s holds the LSE of
// split s; only the n_valid splits that exist are loaded (FlashMLA patch
// stack page, section 3: no masked work for splits that do not exist, real
// splits accumulated in their order).  The sink joins as one more logit.
#include "attn.h"
#include "attn_common.hpp"
#include "attn_kernels.hpp"

#include <algorithm>
#include <atomic>

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeysPerWave = 32;
constexpr int kTileKeys = kKeysPerWave * kWaves;  // 128
constexpr float kRebaseThreshold = 8.0f;

struct DecArgs {
  const uint16_t* q;
  const uint16_t* k;  // [B,Hkv,Lk_max,D], or pages [num_pages,Hkv,page_size,D]
  const uint16_t* v;
  const int32_t* seqlens;
  const int32_t* nsplits;
  const int32_t* table;  // paged: block table [B, max_pages]
  float* o_part;
  float* lse_part;
  int B, Hq, Hkv, Lk_max, max_splits, window, n_qgroups;
  int max_pages, page_shift, num_pages;  // paged: page_size = 1 << page_shift
  float c;  // scale * log2(e)
};

// A work item: one split of one (sequence, KV head, query-column group).
struct Item {
  int b, kvh, qg, s, k_begin, k_end;
};

// Items of sequence b are ordered (kvh, qg, s) with s fastest, so that a run
// of consecutive items streams consecutive cache rows.
__device__ __forceinline__ int items_of(const DecArgs& a, int b, SplitRange& sr) {
  sr = split_rule(a.seqlens[b], a.nsplits[b], a.Lk_max, a.max_splits, a.window);
  return sr.n_valid * a.Hkv * a.n_qgroups;
}
__device__ __forceinline__ Item make_item(const DecArgs& a, int b, int r, const SplitRange& sr) {
  Item it;
  it.b = b;
  it.s = r % sr.n_valid;
  const int rest = r / sr.n_valid;
  it.qg = rest % a.n_qgroups;
  it.kvh = rest / a.n_qgroups;
  it.k_begin = sr.lo + it.s * sr.chunk;
  it.k_end = min(it.k_begin + sr.chunk, sr.Lk);
  return it;
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Split-KV decode: each work-group streams a contiguous range of the flat
// item list (its XCD's share, see below); the copy of the next tile (possibly
// the next item's first) is in flight while a tile is computed.
// PAGED: key j of sequence b is row j % page_size of page
// table[b][j / page_size]; each lane looks up the pages of its rows (page ids
// are clamped into the pool, so a bad table cannot address outside it).
template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecArgs a) {
  using Tile = BfTile<D>;
  constexpr int TILE_BYTES = kTileKeys * Tile::kRowBytes;
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int LOADS = TILE_BYTES / 16 / kThreads;

  // K and V tiles; at the end of an item, the per-wave O columns of the merge
  constexpr int MERGE_BYTES = kWaves * 32 * (D + 4) * 4;
  __shared__ __attribute__((aligned(16))) char
      tile_raw[2 * TILE_BYTES > MERGE_BYTES ? 2 * TILE_BYTES : MERGE_BYTES];
  lds_char* ks_ = (lds_char*)tile_raw;
  lds_char* vs_ = ks_ + TILE_BYTES;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int G = a.Hq / a.Hkv;

  // Total items and this work-group's range (every wave computes the same).
  // The lengths and split counts of sequences 0 .. 255 are loaded in
  // one round and kept in registers for both scans and the first item, so a
  // work-group waits for one round trip before it can stream; later
  // sequences are read again.
  constexpr int kPre = 4;
  int pre_sl[kPre], pre_ns[kPre], pre_n[kPre], pre_incl[kPre];
  long long pre_chunk[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int b = 64 * j + lane;
    pre_sl[j] = b < a.B ? a.seqlens[b] : 0;
    pre_ns[j] = b < a.B ? a.nsplits[b] : 1;
  }
  long long total = 0;
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const SplitRange sr = split_rule(pre_sl[j], pre_ns[j], a.Lk_max, a.max_splits, a.window);
    pre_n[j] = 64 * j + lane < a.B ? sr.n_valid * a.Hkv * a.n_qgroups : 0;
    pre_incl[j] = wave_incl_scan(pre_n[j], lane);
    pre_chunk[j] = __builtin_amdgcn_readfirstlane(__shfl(pre_incl[j], 63));
    total += pre_chunk[j];
  }
  for (int b0 = 64 * kPre; b0 < a.B; b0 += 64) {
    SplitRange sr;
    int n = (b0 + lane < a.B) ? items_of(a, b0 + lane, sr) : 0;
    total += __builtin_amdgcn_readfirstlane(__shfl(wave_incl_scan(n, lane), 63));
  }
  // Work-groups are dealt round-robin over the 8 XCDs.  Group x of the
  // X = min(8, grid) groups (work-groups x, x + X, ...; one XCD each) takes an
  // X-th of the items, its k-th work-group the k-th share of them: one item each, front-loaded in dispatch order, when there are no
  // more items than work-groups (the rest exit at once), else contiguous
  // ranges.
  // Item counts fit in 32 bits: the host bounds B*Hq*max_splits below 2^31.
  int lo, hi;
  {
    const int tot = (int)total;
    const int X = min(8, (int)gridDim.x);
    const int x = blockIdx.x % X, k = blockIdx.x / X;
    const int m = gridDim.x / X + (x < (int)(gridDim.x % X) ? 1 : 0);
    const int q8 = tot / X, r8 = tot % X;
    const int x_lo = x * q8 + min(x, r8), t = q8 + (x < r8 ? 1 : 0);
    if (t <= m) {
      lo = x_lo + k;
      hi = k < t ? lo + 1 : lo;
    } else {
      const int qq = t / m, rr = t % m;
      lo = x_lo + k * qq + min(k, rr);
      hi = lo + qq + (k < rr ? 1 : 0);
    }
  }
  if (lo >= hi) return;  // uniform over the work-group
  int items_left = (int)(hi - lo);

  // Locate the first item: sequence b and index r within it (the first lane
  // whose inclusive prefix passes lo).
  int cur_b = 0, cur_r = 0, cur_n = 0;
  SplitRange cur_sr;
  {
    long long base = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      if (!found && base + pre_chunk[j] > lo) {
        const unsigned long long m = __builtin_amdgcn_ballot_w64(base + pre_incl[j] > lo);
        const int l0 = __builtin_ctzll(m);
        const int excl = __builtin_amdgcn_readlane(pre_incl[j] - pre_n[j], l0);
        cur_b = 64 * j + l0;
        cur_r = (int)(lo - base - excl);
        cur_n = __builtin_amdgcn_readlane(pre_n[j], l0);
        cur_sr = split_rule(__builtin_amdgcn_readlane(pre_sl[j], l0),
                            __builtin_amdgcn_readlane(pre_ns[j], l0), a.Lk_max, a.max_splits,
                            a.window);
        found = true;
      }
      if (!found) base += pre_chunk[j];
    }
    for (int b0 = 64 * kPre; !found && b0 < a.B; b0 += 64) {
      SplitRange sr;
      int n = (b0 + lane < a.B) ? items_of(a, b0 + lane, sr) : 0;
      int incl = wave_incl_scan(n, lane);
      long long chunk = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
      if (base + chunk > lo) {
        unsigned long long m = __builtin_amdgcn_ballot_w64(base + incl > lo);
        int l0 = __builtin_ctzll(m);
        int excl = __builtin_amdgcn_readfirstlane(__shfl(incl - n, l0));
        cur_b = b0 + l0;
        cur_r = (int)(lo - base - excl);
        cur_n = items_of(a, cur_b, cur_sr);
        found = true;
      }
      base += chunk;
    }
  }
  Item it = make_item(a, cur_b, cur_r, cur_sr);

  // Advance to the next item (skipping sequences without keys).
  auto advance = [&]() {
    if (++cur_r >= cur_n) {
      cur_r = 0;
      do {  // a later sequence with items exists: items_left counts them
        ++cur_b;
        cur_n = cur_b < a.B ? items_of(a, cur_b, cur_sr) : 1;
      } while (cur_n == 0);
    }
    return make_item(a, cur_b, cur_r, cur_sr);
  };

  auto kv_base = [&](const Item& x, const uint16_t* p) {
    return p + ((size_t)(x.b * a.Hkv + x.kvh) * a.Lk_max) * D;
  };
  u32x4 kreg[LOADS], vreg[LOADS];
  // PAGED: page ids of the rows of the tile that load_tile fetches next.  They
  // are loaded one tile ahead, so the table's latency does not delay the K/V
  // loads that depend on it.
  int pid_next[PAGED ? LOADS : 1];
  auto lookup_pages = [&](const Item& x, int t0) {
    if constexpr (PAGED) {
      const int32_t* tb = a.table + (size_t)x.b * a.max_pages;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = (threadIdx.x + i * kThreads) / Tile::kChunks;
        pid_next[i] = tb[min(t0 + r, x.k_end - 1) >> a.page_shift];
      }
    }
  };
  // The item after the cursor, leaving the cursor where it is.
  auto peek = [&]() {
    const int b = cur_b, r = cur_r, n = cur_n;
    const SplitRange sr = cur_sr;
    const Item nxt = advance();
    cur_b = b; cur_r = r; cur_n = n; cur_sr = sr;
    return nxt;
  };
  auto load_tile = [&](const Item& x, int t0) {
    // Rows past the split are loaded from its last key: they are masked
    // (p = 0) and finite, so they add nothing.  Rows >= Lk are never read.
    // Each cache byte is read once: non-temporal loads keep it out of the caches.
    if constexpr (PAGED) {
      // page ids were looked up one tile earlier (lookup_pages)
      const int mask = (1 << a.page_shift) - 1;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        int cid = threadIdx.x + i * kThreads;
        int r = cid / Tile::kChunks, cch = cid % Tile::kChunks;
        int key = min(t0 + r, x.k_end - 1);
        const int pg = min(max(pid_next[i], 0), a.num_pages - 1);
        const size_t row = (((size_t)pg * a.Hkv + x.kvh) << a.page_shift) + (key & mask);
        kreg[i] = __builtin_nontemporal_load((const u32x4*)(a.k + row * D + cch * 8));
        vreg[i] = __builtin_nontemporal_load((const u32x4*)(a.v + row * D + cch * 8));
      }
    } else {
      const uint16_t* kh = kv_base(x, a.k);
      const uint16_t* vh = kv_base(x, a.v);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        int cid = threadIdx.x + i * kThreads;
        int r = cid / Tile::kChunks, cch = cid % Tile::kChunks;
        int key = min(t0 + r, x.k_end - 1);
        kreg[i] = __builtin_nontemporal_load((const u32x4*)(kh + (size_t)key * D + cch * 8));
        vreg[i] = __builtin_nontemporal_load((const u32x4*)(vh + (size_t)key * D + cch * 8));
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int cid = threadIdx.x + i * kThreads;
      int r = cid / Tile::kChunks, cch = cid % Tile::kChunks;
      int off = Tile::off(r, cch * 16);
      lds_write16(ks_, off, kreg[i]);
      lds_write16(vs_, off, vreg[i]);
    }
  };
  bf16x8 qf[KS];  // Q^T operand of the current item
  auto load_q = [&](const Item& x) {
    const int qcol = x.qg * 32 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (qcol < G) {
        const int h = x.kvh * G + qcol;
        v = *(const u32x4*)(a.q + ((size_t)(x.b * a.Hq + h)) * D + ks * 16 + half * 8);
      }
      qf[ks] = as_bf16x8(v);
    }
  };

  const int k_row = wave * kKeysPerWave + key_perm(col);
  const int tr_key = (lane & 15) >> 2;
  const int tr_d = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

  f32x16 o[NDB];
  // l_run sums the fp32 probabilities (for the LSE), lb_run the same values
  // as rounded to bf16 for P V (the partial output's normaliser, so that a
  // dominant key's rounding cancels).
  float m_run = kNegInf, l_run = 0.0f, lb_run = 0.0f;

  int t0 = it.k_begin;
  load_q(it);
  if constexpr (PAGED) {
    lookup_pages(it, t0);
    load_tile(it, t0);
    if (t0 + kTileKeys < it.k_end) lookup_pages(it, t0 + kTileKeys);
    else if (items_left > 1) { const Item nn = peek(); lookup_pages(nn, nn.k_begin); }
  } else {
    load_tile(it, t0);
  }
  while (true) {
    __syncthreads();  // every wave is done with the previous tile
    store_tile();
    if (t0 == it.k_begin) {  // a new item starts (its Q is in qf already)
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] = (f32x16){};
      m_run = kNegInf;
      l_run = 0.0f;
      lb_run = 0.0f;
    }
    // Prefetch the next tile: of this item, or the first of the next item.
    const bool last = t0 + kTileKeys >= it.k_end;
    Item nx = it;
    int nt0 = t0 + kTileKeys;
    const bool has_next = !last || items_left > 1;
    if (last && has_next) {
      nx = advance();
      nt0 = nx.k_begin;
    }
    if (has_next) load_tile(nx, nt0);
    if constexpr (PAGED) {
      // page ids of the tile after (nx, nt0): later in nx, or the first of
      // the item after it (items_left counts the current item)
      if (has_next) {
        if (nt0 + kTileKeys < nx.k_end) {
          lookup_pages(nx, nt0 + kTileKeys);
        } else if (items_left - (last ? 2 : 1) > 0) {
          const Item nn = peek();
          lookup_pages(nn, nn.k_begin);
        }
      }
    }
    __syncthreads();

    const int w0 = t0 + wave * kKeysPerWave;
    const bool active = w0 < it.k_end;
    f32x16 st = (f32x16){};
    if (active) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 kf = as_bf16x8(lds_read16(ks_, Tile::off(k_row, (ks * 2 + half) * 16)));
        st = mfma_32x32x16(kf, qf[ks], st);
      }
    }
    // Q of the next item: qf is free once the scores of the item's last tile
    // are issued, and the load overlaps the rest of this tile and the merge.
    if (last && has_next) load_q(nx);
    if (active) {
      float sv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[v] = st[v];
      if (w0 + kKeysPerWave > it.k_end) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          sv[v] = (w0 + key_of_reg(v, half) < it.k_end) ? sv[v] : kNegInf;
      }
      float mx = sv[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sv[v]);
      mx = pair_max(mx);
      float m_new = fmaxf(m_run, mx * a.c);
      bool need = m_new > m_run + kRebaseThreshold;
      if (__builtin_amdgcn_ballot_w64(need)) {
        float alpha = need ? exp2_fast(m_run - m_new) : 1.0f;
        m_run = need ? m_new : m_run;
        l_run *= alpha;
        lb_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      }
      float m_use = m_run == kNegInf ? 0.0f : m_run;
      float sum = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sv[v] = exp2_fast(__builtin_fmaf(sv[v], a.c, -m_use));
        sum += sv[v];
      }
      l_run += sum;
      bf16x8 pf[2];
      u32x4 pw[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const float* x = sv + s2 * 8;
        pw[s2] = pack_bf16_words(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
        pf[s2] = __builtin_bit_cast(bf16x8, pw[s2]);
      }
      lb_run = sum_bf16_words(pw[0], pw[1], lb_run);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          int key = wave * kKeysPerWave + s2 * 16 + half * 8 + tr_key;
          int dd = db * 32 + tr_d;
          i16x4 lo4 = lds_read_tr16(vs_, Tile::off(key, dd * 2));
          i16x4 hi4 = lds_read_tr16(vs_, Tile::off(key + 4, dd * 2));
          o[db] = mfma_32x32x16(join_tr(lo4, hi4), pf[s2], o[db]);
        }
    }

    if (last) {
      // Merge the four per-wave states of each query column into the split's
      // normalised partial output and its sink-free LSE, in one pass: once
      // every wave is done with this tile, its LDS holds the four waves'
      // unnormalised O columns ([wave][column] rows of D floats, padded by
      // 16 B that hold the column's max and sum), and the next tile is stored
      // only after the barrier at the top of the loop.
      const float l_tot = pair_sum(l_run);
      const float lb_tot = pair_sum(lb_run);
      const int n_cols = min(32, G - it.qg * 32);
      constexpr int NCH = D / 4;  // 16 B chunks per column
      constexpr int PITCH = (D + 4) * 4;
      lds_char* sm = ks_;
      __syncthreads();
      if (col < n_cols) {
        const int rbase = (wave * 32 + col) * PITCH;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            lds_write16(sm, rbase + (db * 8 + j * 2 + half) * 16,
                        __builtin_bit_cast(u32x4, (f32x4){o[db][j * 4], o[db][j * 4 + 1],
                                                          o[db][j * 4 + 2], o[db][j * 4 + 3]}));
          }
        // the column's running max and its two partial sums go into the row's padding
        if (half == 0)
          lds_write16(sm, rbase + D * 4,
                      (u32x4){__builtin_bit_cast(uint32_t, m_run), __builtin_bit_cast(uint32_t, l_tot),
                              __builtin_bit_cast(uint32_t, lb_tot), 0u});
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < n_cols * NCH; idx += kThreads) {
        const int cq = idx / NCH, ch = idx % NCH;
        float mw[kWaves], lw[kWaves], lbw[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const lds_char* pad = sm + (w * 32 + cq) * PITCH + D * 4;
          mw[w] = *(const __attribute__((address_space(3))) float*)pad;
          lw[w] = *(const __attribute__((address_space(3))) float*)(pad + 4);
          lbw[w] = *(const __attribute__((address_space(3))) float*)(pad + 8);
        }
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w]);
        float L = 0.0f, Lb = 0.0f;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float f = exp2_fast(mw[w] - M);  // -inf (wave saw no key) -> 0
          L += lw[w] * f;
          Lb += lbw[w] * f;
          const f32x4 x = __builtin_bit_cast(
              f32x4, lds_read16(sm, (w * 32 + cq) * PITCH + ch * 16));
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += x[e] * f;
        }
        const int hh = it.kvh * G + it.qg * 32 + cq;
        const size_t base = ((size_t)(it.b * a.Hq + hh) * a.max_splits + it.s);
        // Partial rows are stored with device scope (sc1): written through
        // the caches they slowed the key/value stream beside them by about
        // 8%, as non-temporal stores by 7%, this way by about 6%.  A buffer
        // resource must be uniform over the wave: it starts at the row of the
        // wave's first column, and the wave's other columns (64 / NCH in all)
        // are whole head strides of max_splits rows further on.
#if defined(__HIP_DEVICE_COMPILE__)
        {
          const int cq0 = __builtin_amdgcn_readfirstlane(cq);
          const size_t row0 =
              (size_t)(it.b * a.Hq + it.kvh * G + it.qg * 32 + cq0) * a.max_splits + it.s;
          const int hstride = a.max_splits * D * 4;  // bytes between heads
          const __amdgpu_buffer_rsrc_t prow = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(a.o_part + row0 * D), 0, (64 / NCH - 1) * hstride + D * 4, kRawBufferWord3);
          const f32x4 res = {acc[0] / Lb, acc[1] / Lb, acc[2] / Lb, acc[3] / Lb};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, res), prow,
                                                 (cq - cq0) * hstride + ch * 16, 0, kCpolSc1);
        }
#endif
        if (ch == 0) a.lse_part[base] = (M + log2_fast(L)) * kLn2;
      }
      --items_left;
    }
    if (!has_next) break;
    it = nx;
    t0 = nt0;
  }
}

struct CombArgs {
  const float* o_part;
  const float* lse_part;
  const int32_t* seqlens;
  const int32_t* nsplits;
  const float* sinks;
  void* out;
  float* lse;
  int B, Hq, Lk_max, max_splits, window;
};

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombArgs a) {
  constexpr int PER = D / 64;  // d values per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.x * kWaves + wave;
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const SplitRange sr = split_rule(a.seqlens[b], a.nsplits[b], a.Lk_max, a.max_splits, a.window);
  const int n = sr.n_valid;
  const size_t row = (size_t)bh * a.max_splits;

  float ls = lane < n ? a.lse_part[row + lane] : kNegInf;
  const float sig = a.sinks ? a.sinks[h] : kNegInf;
  const float M = fmaxf(wave_max(ls), sig);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  float lse_out = kNegInf, inv = 0.0f;
  if (M != kNegInf) {
    float w = lane < n ? exp2_fast((ls - M) * kLog2e) : 0.0f;
    float den = wave_sum(w) + (a.sinks ? exp2_fast((sig - M) * kLog2e) : 0.0f);
    const float* op = a.o_part + row * D + lane * PER;
    int s = 0;
    for (; s + 4 <= n; s += 4) {
      float x[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < PER; ++e) x[u][e] = op[(size_t)(s + u) * D + e];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), s + u));
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(ws, x[u][e], acc[e]);
      }
    }
    for (; s < n; ++s) {
      float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), s));
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(ws, op[(size_t)s * D + e], acc[e]);
    }
    inv = 1.0f / den;
    lse_out = M + log2_fast(den) * kLn2;
  }
  if constexpr (OUT_F32) {
    float* dst = (float*)a.out + (size_t)bh * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = acc[e] * inv;
  } else {
    uint16_t* dst = (uint16_t*)a.out + (size_t)bh * D + lane * PER;
    if constexpr (PER == 2) {
      *(uint32_t*)dst = pack2_bf16(acc[0] * inv, acc[1] * inv);
    } else {
      uint32_t pk = pack2_bf16(acc[0] * inv, 0.0f);
      dst[0] = (uint16_t)(pk & 0xFFFF);
    }
  }
  if (a.lse && lane == 0) a.lse[bh] = lse_out;
}

// ---------------------------------------------------------------------------
// Split-count planning (attn_decode_plan).  One work-group; for the auto
// policy every thread accumulates, over its sequences, the item count and the
// largest split of each candidate chunk target; threads 0..10 then price one
// candidate each, as the items of the most loaded compute unit times the
// largest split plus a per-item cost, and thread 0 takes the first of least
// estimated cost (rule stated in include/attn.h).  Item counts fit in 32 bits (the API bounds
// B*Hq*max_splits below 2^31); dividing by the candidate targets, which are
// compile-time constants, costs a multiply.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 256;
constexpr int kPlanCands = 11;
constexpr int kPlanChunks[kPlanCands] = {256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192};
constexpr long long kPlanItemCost = 400;  // per-item cost beyond its keys, in key rows

struct PlanArgs {
  const int32_t* seqlens;
  int32_t* nsplits;
  int B, Lk_max, max_splits, window, policy, param, slots, hq;
};

__device__ __forceinline__ int visible_n(int seqlen, int Lk_max, int window) {
  const int Lk = min(max(seqlen, 0), Lk_max);
  return Lk - (window > 0 ? max(0, Lk - window) : 0);
}
__device__ __forceinline__ int splits_for(int n, int target, int max_splits) {
  return min(max((n + target - 1) / target, 1), max_splits);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int s_items[kPlanCands][kPlanThreads / 64];
  __shared__ int s_z[kPlanCands][kPlanThreads / 64];
  __shared__ long long s_cost[kPlanCands];
  __shared__ int s_target;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.policy == ATTN_SPLITS_AUTO) {
    int items[kPlanCands], z[kPlanCands];
#pragma unroll
    for (int i = 0; i < kPlanCands; ++i) { items[i] = 0; z[i] = 0; }
    for (int b = tid; b < a.B; b += kPlanThreads) {
      const int n = visible_n(a.seqlens[b], a.Lk_max, a.window);
      if (n == 0) continue;
#pragma unroll
      for (int i = 0; i < kPlanCands; ++i) {
        const int ns = splits_for(n, kPlanChunks[i], a.max_splits);
        const int chunk = ((n + ns - 1) / ns + 63) / 64 * 64;
        items[i] += (n + chunk - 1) / chunk;
        z[i] = max(z[i], min(chunk, n));
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
      for (int i = 0; i < kPlanCands; ++i) {
        items[i] += __shfl_xor(items[i], o);
        z[i] = max(z[i], __shfl_xor(z[i], o));
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kPlanCands; ++i) { s_items[i][wave] = items[i]; s_z[i][wave] = z[i]; }
    }
    __syncthreads();
    if (tid < kPlanCands) {
      int it = 0, zz = 0;
#pragma unroll
      for (int w = 0; w < kPlanThreads / 64; ++w) {
        it += s_items[tid][w];
        zz = max(zz, s_z[tid][w]);
      }
      it *= a.hq;
      const unsigned S = (unsigned)a.slots;  // >= 1
      const long long per = ((unsigned)it + S - 1u) / S;  // < 2^32: it < 2^31, S <= 2^31
      s_cost[tid] = per * (zz + kPlanItemCost);
    }
    __syncthreads();
    if (tid == 0) {
      int best = 0;
      for (int i = 1; i < kPlanCands; ++i)
        if (s_cost[i] < s_cost[best]) best = i;
      s_target = kPlanChunks[best];
    }
    __syncthreads();
  }
  const int target = a.policy == ATTN_SPLITS_AUTO ? s_target : a.param;
  for (int b = tid; b < a.B; b += kPlanThreads) {
    const int ns = a.policy == ATTN_SPLITS_COUNT
                       ? min(max(a.param, 1), a.max_splits)
                       : splits_for(visible_n(a.seqlens[b], a.Lk_max, a.window), target, a.max_splits);
    a.nsplits[b] = ns;
  }
}

}  // namespace

// Compute units of the current device, read once per device.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seqlens_k, const int32_t* num_splits, float* o_part,
                         float* lse_part, int B, int Hq, int Hkv, int Lk_max, int D,
                         int max_splits, int window, float scale, hipStream_t stream) {
  return launch_decode_paged(q, k_cache, v_cache, nullptr, seqlens_k, num_splits, o_part, lse_part,
                             B, Hq, Hkv, Lk_max, 0, 0, 0, D, max_splits, window, scale, stream);
}

hipError_t launch_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* seqlens_k,
                               const int32_t* num_splits, float* o_part, float* lse_part, int B,
                               int Hq, int Hkv, int Lk_max, int num_pages, int page_shift,
                               int max_pages, int D, int max_splits, int window, float scale,
                               hipStream_t stream) {
  DecArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k_pages; a.v = (const uint16_t*)v_pages;
  a.seqlens = seqlens_k; a.nsplits = num_splits; a.o_part = o_part; a.lse_part = lse_part;
  a.table = block_table; a.num_pages = num_pages; a.page_shift = page_shift; a.max_pages = max_pages;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lk_max = Lk_max; a.max_splits = max_splits; a.window = window;
  int G = Hq / Hkv;
  a.n_qgroups = (G + 31) / 32;
  a.c = scale * kLog2e;
  // Far more work-groups than fit at once (two per compute unit), so that
  // the hardware hands the remaining items to whichever compute units are
  // free: work-groups with equal shares finished up to 2x apart when each
  // compute unit's two owned a fixed sixteenth of the items.  Capped at the
  // most items the launch can have (splits beyond a sequence's count exit at
  // once).
  const long long max_items = (long long)B * Hkv * a.n_qgroups * max_splits;
  dim3 grid((unsigned)std::min<long long>(32LL * cu_count(), max_items));
  const bool paged = block_table != nullptr;
  if (D == 128) {
    if (paged) hipLaunchKernelGGL((decode_kernel<128, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((decode_kernel<128, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (paged) hipLaunchKernelGGL((decode_kernel<64, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((decode_kernel<64, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* seqlens_k, int32_t* num_splits, int B, int Hq, int Hkv,
                       int Lk_max, int max_splits, int window, int policy, int param,
                       hipStream_t stream) {
  PlanArgs a;
  a.seqlens = seqlens_k; a.nsplits = num_splits;
  a.B = B; a.Lk_max = Lk_max; a.max_splits = max_splits; a.window = window;
  a.policy = policy; a.param = param;
  // the decode's own grid: launch_decode runs 2 work-groups per compute unit
  // The unit of throughput is the compute unit: one work-group per CU streams
  // about as fast as two, and the items are spread over CUs.
  a.slots = (policy == ATTN_SPLITS_AUTO && param > 0) ? param : cu_count();
  const int G = Hq / Hkv;
  a.hq = Hkv * ((G + 31) / 32);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const float* o_part, const float* lse_part, const int32_t* seqlens_k,
                          const int32_t* num_splits, const float* sinks, void* out, float* lse,
                          int B, int Hq, int D, int Lk_max, int max_splits, int window,
                          bool out_f32, hipStream_t stream) {
  CombArgs a;
  a.o_part = o_part; a.lse_part = lse_part; a.seqlens = seqlens_k; a.nsplits = num_splits;
  a.sinks = sinks; a.out = out; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Lk_max = Lk_max; a.max_splits = max_splits; a.window = window;
  dim3 grid((B * Hq + kWaves - 1) / kWaves);
  if (D == 128) {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<128, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((combine_kernel<128, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<64, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((combine_kernel<64, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn
