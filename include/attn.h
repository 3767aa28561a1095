/*
 * attn.h -- C ABI of the MI355X (gfx950) exact-attention library.
 *
 * Three calls form the path:
 *   attn_fwd             fused tiled attention forward (prefill): causal +
 *                        sliding window, GQA, learned per-head sink, LSE
 *                        (attn_fwd_max_logit: the same, plus the largest
 *                        pre-softmax logit per row and per head;
 *                        attn_fwd_varlen: a packed batch of sequences;
 *                        attn_bwd: dQ, dK, dV and dsink for a given dO);
 *   attn_decode_splitkv  split-KV decode: per-split partial outputs and LSEs
 *                        (attn_decode_plan: split counts chosen on the device;
 *                        attn_decode_splitkv_paged: over a paged cache);
 *   attn_combine         LSE-weighted merge of the valid splits, sink added once.
 *
 * Conventions shared by every call
 *  - Tensor pointers are HIP device pointers, owned by the caller, contiguous
 *    in the stated layout, and 16-byte aligned.  The library allocates no
 *    device or host memory and keeps no state between calls, except the one
 *    fixed device array of attn_decode_noalloc (see there).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work and return; ordering is the stream's.
 *  - Return value: ATTN_OK (0) or a positive ATTN_ERR_* code.  On an error
 *    nothing is launched.  Faults inside a kernel surface at the caller's
 *    next synchronisation, not here.
 *  - Element types: ATTN_BF16 (bfloat16) or ATTN_F32 for inputs (attn_fwd
 *    only; decode is bf16) and for outputs.  Accumulation is float32.
 *  - Masking (flash-attention repository profile, section 1 "capabilities":
 *    causal and sliding-window masks; Flint page: every token sees only the
 *    most recent 513 tokens): query row i of Lq sits at absolute position
 *    p = i + Lk - Lq (the queries are the last Lq positions) and sees key j
 *    iff j <= p and, when window > 0, j > p - window.  window <= 0: causal
 *    only.  The window counts the query's own key.
 *  - Sink (Flint page, "fix two"): sinks[h] is a logit of query head h in
 *    the same units as scale*<q,k>; it joins the softmax denominator and has
 *    no value vector:  O = sum_j e^{s_j - M} v_j / (sum_j e^{s_j - M} + e^{sink - M}).
 *    The kernels apply it with the rebased update (new max = max(content
 *    max, sink), every exponential <= 1), so it cannot overflow.
 *  - LSE is the natural-log sum of exponentials, the sink included.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ATTN_BF16 = 0, ATTN_F32 = 1 };

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL                     */
  ATTN_ERR_SHAPE = 2,       /* a size < 1 (Lq, Lk, B, heads), Hq % Hkv != 0,
                               Lq > Lk, max_splits outside [1, 64], a decode
                               with B*Hq*max_splits >= 2^31, or an index
                               space that overflows 64-bit offsets           */
  ATTN_ERR_UNSUPPORTED = 3, /* head dim not 64/128, unknown or unsupported dtype */
  ATTN_ERR_VALUE = 4,       /* scale not finite and > 0, or a misaligned pointer */
  ATTN_ERR_HIP = 5,         /* the HIP runtime rejected a launch, or the
                               fixed scratch of attn_decode_noalloc could not
                               be located on the current device              */
  ATTN_ERR_SCRATCH = 6      /* attn_decode_noalloc: the split workspace of the
                               call exceeds ATTN_NOALLOC_SCRATCH_BYTES        */
};

#define ATTN_SPLIT_ALIGN 64  /* split boundaries: multiples of 64 keys from the window start */
#define ATTN_MAX_SPLITS 64

/* Split-count policies of attn_decode_plan. */
enum { ATTN_SPLITS_AUTO = 0, ATTN_SPLITS_KEYS = 1, ATTN_SPLITS_COUNT = 2 };

/*
 * attn_fwd -- O = softmax(scale * Q K^T + mask, sink) V, and LSE.
 *
 * q    [B, Hq,  Lq, D]  in_dtype
 * k, v [B, Hkv, Lk, D]  in_dtype; query head h reads KV head h / (Hq/Hkv)
 * sinks [Hq] float32, or NULL for no sink
 * out  [B, Hq,  Lq, D]  out_dtype
 * lse  [B, Hq,  Lq]     float32, or NULL to skip
 * D in {64, 128}; window <= 0 means none; scale > 0 (e.g. 1/sqrt(D)).
 * A row that sees no key gets O = 0 and LSE = sink (or -inf without one).
 */
int attn_fwd(const void* q, const void* k, const void* v, const float* sinks, void* out,
             float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int D, int window, float scale,
             int in_dtype, int out_dtype, void* stream);

/*
 * attn_fwd_max_logit -- attn_fwd that also returns the largest pre-softmax
 * logit (flash-attention contribution-radar profile, task card for issue
 * #2986: expose the maximum pre-softmax logit of the forward pass, the max of
 * the scores rather than their log-sum-exp, for training monitoring).
 *
 * The logit is the score that enters the softmax, scale * <q_i, k_j>, over
 * the keys row i sees (same mask and GQA rules as attn_fwd); the sink is not
 * a score and is excluded.  Every argument of attn_fwd keeps its meaning, and
 * out/lse are bitwise those of attn_fwd.  Additionally:
 * max_logit_row  [B, Hq, Lq] float32, or NULL: the row's maximum;
 * max_logit_head [B, Hq]     float32, or NULL: the maximum over the head's
 *                rows.  The call first overwrites it with -inf on the stream,
 *                then raises it with atomic max operations (order-independent,
 *                so the result is deterministic).
 * Both NULL is allowed (then it is attn_fwd).  Extra pointers must be 4-byte
 * aligned (ATTN_ERR_VALUE otherwise).
 */
int attn_fwd_max_logit(const void* q, const void* k, const void* v, const float* sinks, void* out,
                       float* lse, float* max_logit_row, float* max_logit_head, int B, int Hq,
                       int Hkv, int Lq, int Lk, int D, int window, float scale, int in_dtype,
                       int out_dtype, void* stream);

/*
 * attn_fwd_varlen -- attn_fwd over a packed batch of sequences of different
 * lengths (flash-attention profile: varlen batches described by cu_seqlens,
 * section 1 capabilities and the call flow's cu_seqlens-to-blocks step).
 *
 * q    [Hq,  total_q, D] bf16 -- each head's rows of all sequences, packed
 * k, v [Hkv, total_k, D] bf16
 * cu_seqlens_q, cu_seqlens_k [B+1] int32 (device): sequence b owns query
 *      rows [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]); offsets are
 *      clamped into [0, total] in the kernel (a decreasing pair is empty).
 * out  [Hq, total_q, D] out_dtype;  lse [Hq, total_q] float32 or NULL
 * max_seqlen_q >= every sequence's query count (it sizes the grid; rows of a
 *      longer sequence past it are not written).
 * Within a sequence everything is as in attn_fwd (its queries are its last
 * Lq_b positions); a row that sees no key (Lk_b = 0, or Lq_b > Lk_b) gets
 * O = 0 and LSE = sink.  in_dtype must be ATTN_BF16.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, const float* sinks, void* out, float* lse, int B,
                    int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q, int D, int window,
                    float scale, int in_dtype, int out_dtype, void* stream);

/*
 * attn_bwd -- gradients of a loss through attn_fwd, given dO = dL/dO.
 *
 * With P_ij = exp(s_ij - LSE_i), Psink_i = exp(sink - LSE_i) (LSE of attn_fwd,
 * the sink included) and D_i = <dO_i, O_i>:  dV = P^T dO,  dS = P (dO V^T - D),
 * dQ = scale dS K,  dK = scale dS^T Q,  dsink_h = -sum_{b,i} Psink_i D_i.
 * The flash-attention profile's backward: a dQ phase (rows fixed), then a
 * dK/dV phase (keys fixed).  Its issue #2969 is that dsink loses precision
 * when D comes from a bf16-rounded O; here the dQ phase sums D_i = sum_j P_ij
 * (dO_i . v_j) in fp32, which does not depend on O at all, and dK, dV and
 * dsink use that.  O (bf16 or fp32) only feeds the D of the dQ phase's dS.
 *
 * q, dout [B,Hq,Lq,D] bf16; k, v [B,Hkv,Lk,D] bf16 (in_dtype must be ATTN_BF16)
 * out  [B,Hq,Lq,D] out_dtype: the O that attn_fwd returned for these inputs
 * lse  [B,Hq,Lq] float32: the LSE that attn_fwd returned
 * sinks [Hq] or NULL; mask, window, GQA and scale as in attn_fwd
 * dq [B,Hq,Lq,D], dk, dv [B,Hkv,Lk,D] float32 (fully written; GQA heads add
 *      into their KV head); dsink [Hq] float32 or NULL (requires sinks)
 * delta [B,Hq,Lq] float32: caller-owned workspace (D_i), overwritten; on
 *      return it holds sum_j P_ij dP_ij.
 * Deterministic: no atomics; every sum has a fixed order.
 */
int attn_bwd(const void* q, const void* k, const void* v, const float* sinks, const void* out,
             const void* dout, const float* lse, float* dq, float* dk, float* dv, float* dsink,
             float* delta, int B, int Hq, int Hkv, int Lq, int Lk, int D, int window, float scale,
             int in_dtype, int out_dtype, void* stream);

/*
 * attn_decode_splitkv -- one query per sequence over a KV cache, cut into splits.
 *
 * Split-KV decode (flash-attention profile: split-KV benchmarks; FlashMLA
 * patch stack page: split kernel + combine).  Sequence b's single query sits
 * at position seqlens_k[b] - 1 and sees keys [lo, Lk), lo = max(0, Lk - window)
 * (window <= 0: lo = 0).  With n = Lk - lo and ns = num_splits[b]:
 *   chunk   = round_up(ceil(n / ns), 64),  n_valid = ceil(n / chunk) (<= ns),
 *   split s covers [lo + s*chunk, min(lo + (s+1)*chunk, Lk)),  s < n_valid.
 * For each valid split the kernel writes, for every query head h,
 *   lse_part[b,h,s] = ln sum_{j in split} e^{s_j}          (no sink)
 *   o_part[b,h,s,:] = sum_{j in split} e^{s_j - lse} v_j   (normalised)
 * Lanes s >= n_valid are neither written nor ever read.
 *
 * q        [B, Hq, 1, D]        bf16
 * k_cache, v_cache [B, Hkv, Lk_max, D] bf16; rows >= seqlens_k[b] are never read
 * seqlens_k [B] int32 device, clamped in-kernel to [0, Lk_max]
 * num_splits [B] int32 device, clamped in-kernel to [1, max_splits]
 * o_part   [B, Hq, max_splits, D] float32 (caller-owned workspace)
 * lse_part [B, Hq, max_splits]    float32
 * max_splits in [1, 64]; in_dtype must be ATTN_BF16.
 */
int attn_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens_k, const int32_t* num_splits, float* o_part,
                        float* lse_part, int B, int Hq, int Hkv, int Lk_max, int D,
                        int max_splits, int window, float scale, int in_dtype, void* stream);

/*
 * attn_decode_splitkv_paged -- attn_decode_splitkv over a paged KV cache
 * (flash-attention profile: paged KV with a block_table for serving decode).
 *
 * k_pages, v_pages [num_pages, Hkv, page_size, D] bf16: a pool of pages.
 * block_table [B, max_pages_per_seq] int32 (device): key j of sequence b is
 *      row j % page_size of page block_table[b][j / page_size].  Only the
 *      slots of keys < seqlens_k[b] are read; a page id outside
 *      [0, num_pages) is clamped into it (wrong values, never a stray access).
 * page_size: a power of two.  Lk_max of the split rule and of attn_combine
 * is max_pages_per_seq * page_size.  Everything else is attn_decode_splitkv.
 */
int attn_decode_splitkv_paged(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, const int32_t* seqlens_k,
                              const int32_t* num_splits, float* o_part, float* lse_part, int B,
                              int Hq, int Hkv, int num_pages, int page_size, int max_pages_per_seq,
                              int D, int max_splits, int window, float scale, int in_dtype,
                              void* stream);

/*
 * attn_decode_plan -- choose num_splits[b] for attn_decode_splitkv on the
 * device, from seqlens_k and the shape, with no host synchronisation.
 *
 * Workload-aware partitioning (FlashMLA patch stack page, section 1: gather
 * the workload's shape, pick the partition by policy -- baseline, dynamic or
 * fixed -- and refuse what is illegal); the pages give no formula, the rules
 * below are this library's.  n_b is the number of keys sequence b's query
 * sees (Lk clamped to [0, Lk_max], window applied), and every result is
 * clamped to [1, max_splits]:
 *   ATTN_SPLITS_COUNT  num_splits[b] = param                      (param >= 1)
 *   ATTN_SPLITS_KEYS   num_splits[b] = ceil(n_b / param)          (param >= 1)
 *   ATTN_SPLITS_AUTO   num_splits[b] = ceil(n_b / c) for the chunk target c in
 *                      {256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096,
 *                      6144, 8192} that minimises
 *                        ceil(I / S) * (Z + 400),
 *                      with, for target c: I the decode's work items (valid
 *                      splits x Hkv x ceil((Hq/Hkv)/32)), Z the largest split
 *                      in keys and S the units the items are spread over
 *                      (param, or the compute units when param = 0).  The
 *                      first (smallest) such c wins.  The estimate is the
 *                      items of the most loaded unit, each priced as the
 *                      largest split plus a per-item cost of 400 key rows;
 *                      the form and the constant were fitted to decode +
 *                      combine times of every target on eight batch/length
 *                      mixes on MI355X (choice within 1% of the best).
 * seqlens_k [B] int32 (device); num_splits [B] int32 (device, written).
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE (sizes as in attn_decode_splitkv),
 * ATTN_ERR_UNSUPPORTED (unknown policy), ATTN_ERR_VALUE (param < 1 for
 * COUNT/KEYS, param < 0 for AUTO, misaligned pointer).
 */
int attn_decode_plan(const int32_t* seqlens_k, int32_t* num_splits, int B, int Hq, int Hkv,
                     int Lk_max, int max_splits, int window, int policy, int param, void* stream);

/*
 * attn_combine -- merge the valid split partials of each (b, h), sink once.
 *
 * Exact small-split combine (FlashMLA patch stack page, section 3): only the
 * n_valid lanes that exist are read (n_valid recomputed from seqlens_k,
 * num_splits and window by the rule above), in order s = 0, 1, ...:
 *   M = max(max_s lse_s, sink); w_s = e^{lse_s - M};
 *   den = sum_s w_s + e^{sink - M};  O = sum_s w_s O_s / den;  LSE = M + ln den.
 * The sink enters here and only here, as one more logit with a zero value.
 *
 * o_part, lse_part as written by attn_decode_splitkv; seqlens_k, num_splits,
 * Lk_max, max_splits and window must be the values given to that call.
 * sinks [Hq] float32 or NULL;  out [B, Hq, 1, D] out_dtype;  lse [B, Hq] or NULL
 * A sequence with no visible key gets O = 0 and LSE = sink (-inf without one).
 */
int attn_combine(const float* o_part, const float* lse_part, const int32_t* seqlens_k,
                 const int32_t* num_splits, const float* sinks, void* out, float* lse, int B,
                 int Hq, int D, int Lk_max, int max_splits, int window, int out_dtype,
                 void* stream);

/*
 * attn_decode_noalloc -- attn_decode_splitkv followed by attn_combine, in one
 * call that allocates nothing and takes no workspace argument.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The split
 * partials (o_part [B,Hq,max_splits,D] float32, then lse_part
 * [B,Hq,max_splits] float32 at the next 256-byte boundary) live in one fixed
 * device array of this library, ATTN_NOALLOC_SCRATCH_BYTES long (129 MiB:
 * 64 sequences x 64 query heads x 64 splits at D = 128), which each GPU the
 * call runs on holds from the first call on that device until the process
 * ends.  That first call locates the array on the current device (no
 * allocation); a failure there returns ATTN_ERR_HIP.  A call whose
 * workspace, B*Hq*max_splits*(D+1)*4 bytes plus alignment, exceeds the array
 * returns ATTN_ERR_SCRATCH and launches nothing.
 *
 * Arguments are those of attn_decode_splitkv and attn_combine, with the same
 * meaning, checks and results (out and lse are bitwise those of the two calls
 * on caller-owned workspace); sinks [Hq] or NULL, out [B,Hq,1,D] out_dtype,
 * lse [B,Hq] float32 or NULL.
 * Every call on a GPU uses that GPU's one array, which keeps the last call's
 * contents (each call writes every lane it reads first, so nothing needs
 * clearing): calls that overlap in time on one GPU -- on different streams,
 * or from several host threads -- race and give wrong results.  Order them
 * on one stream.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES 135266304u

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens_k, const int32_t* num_splits, const float* sinks,
                        void* out, float* lse, int B, int Hq, int Hkv, int Lk_max, int D,
                        int max_splits, int window, float scale, int in_dtype, int out_dtype,
                        void* stream);

/* Human-readable name of an ATTN_* return code (static string). */
const char* attn_strerror(int code);

/* Library version, "attn-mi355x <major>.<minor>". */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
