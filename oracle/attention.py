"""Float64 CPU oracle for exact attention with a learned per-head sink.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing).

What it computes (all arithmetic IEEE float64; inputs are the exact values the
GPU sees, i.e. bf16 or fp32 values upcast):

* ``attention_fwd`` -- causal (bottom-right aligned) attention over a sliding
  window, with GQA head sharing and an optional per-query-head sink logit that
  sits in the softmax denominator with no value vector.  The sink is the
  "virtual anchor" logit of the Flint model page (cf-1.com, section on why the
  kernel had to change) and the window is the "most recent 513 tokens" rule of
  the same section.  O and the natural-log LSE are the plain definition:

      s_j   = scale * <q_i, k_j>            for visible keys j
      M     = max(max_j s_j, sigma)
      l     = sum_j exp(s_j - M) + exp(sigma - M)
      O_i   = sum_j exp(s_j - M) v_j / l
      LSE_i = M + ln l

  The LSE includes the sink term, because after the "rebase" update the
  running denominator holds the sink's exponential (cf-1.com, fix two).  The
  sink is compared with the *scaled* scores without being scaled itself
  (cf-1.com, fix two: the sink is multiplied by log2(e) only, the running
  max by the softmax scale in log2 units).

* ``split_ranges`` / ``decode_partials`` / ``combine`` -- split-KV decode:
  each split yields a normalised partial output and its (sink-free) LSE; the
  combine reduces only the splits that exist, in their natural order, and adds
  the sink exactly once as one more logit (FlashMLA patch stack page, section
  3 "exact small-split combine").

* ``attention_bwd`` -- dQ, dK, dV and dsink of the forward for a given dO,
  the plain gradient formulas in float64 (the flash-attention profile's
  two-phase backward; its dsink precision issue #2969).

* ``max_logit_rows`` / ``max_logit`` -- the largest pre-softmax logit
  scale*<q_i,k_j> over the keys each row sees (sink excluded), per row and
  per head (flash-attention contribution-radar profile, task card for issue
  #2986).

* ``gather_paged`` / ``decode_paged`` / ``attention_fwd_varlen`` -- the
  serving layouts: a KV cache held in pages named by a block table, and a
  packed batch of sequences of different lengths delimited by cu_seqlens
  (flash-attention profile: paged KV and varlen among its capabilities).

* ``plan_splits`` -- the number of splits per sequence chosen by a policy
  (fixed count, fixed keys per split, or a workload-aware cost rule); the
  FlashMLA patch stack page (section 1) gives the idea but no formula, so the
  rule is the library's (include/attn.h) and only its arithmetic is checked.

* ``naive_sink_row_sum_f32`` / ``rebase_sink_f32`` -- the two sink updates of
  the cf-1.com page (fix two), evaluated in float32 so that tests can show the
  old additive form overflowing and the rebased form staying finite.

Readings of the pages where they are silent (each is listed in the design doc):
window W keeps keys with p - W < j <= p (W <= 0: no window); query row i of
Lq sits at absolute position p = i + Lk - Lq; the sink is per query head;
max_offset = 0 and v_descale = 1.

Parity pins: every public function here is pinned by tests/test_oracle.py
against brute force, torch's float64 CPU attention, closed forms and exact
integer counts.  Nothing is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

LOG2E = 1.4426950408889634  # log2(e)


# ---------------------------------------------------------------------------
# index helpers (kept as small functions so that tests can plant mistakes)
# ---------------------------------------------------------------------------

def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: G = Hq/Hkv consecutive query heads share one.

    GQA grouping as in the flash-attention repository profile (section 1,
    "capabilities": MQA/GQA) -- consecutive query heads form a group.
    """
    G = Hq // Hkv
    return h // G


def query_position(i: int, Lq: int, Lk: int) -> int:
    """Absolute position of query row i: the Lq queries are the last Lq positions."""
    return i + Lk - Lq


def visible_range(p: int, Lk: int, window: int) -> tuple[int, int]:
    """Half-open key range [lo, hi) that the query at absolute position p sees.

    Causal: keys j <= p.  Sliding window of W tokens including the query
    itself: j > p - W.  W <= 0 means no window.  Keys beyond Lk do not exist.
    """
    hi = min(p + 1, Lk)
    lo = 0 if window <= 0 else max(0, p - window + 1)
    return lo, max(lo, hi)


def effective_scale(scale: float) -> float:
    """The softmax scale as the library receives it: a float32, upcast."""
    return float(np.float32(scale))


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def _finish(scores: np.ndarray, vals: np.ndarray, sigma: float):
    """O and LSE of one block of query rows from their scores (-inf = masked).

    scores: [R, N] float64; vals: [N, D] float64; sigma: sink logit or -inf.
    """
    R = scores.shape[0]
    D = vals.shape[1]
    row_max = scores.max(axis=1) if scores.shape[1] else np.full(R, -np.inf)
    M = np.maximum(row_max, sigma)
    out = np.zeros((R, D))
    lse = np.full(R, -np.inf)
    ok = np.isfinite(M)  # rows that see at least one key or have a sink
    if ok.any():
        e = np.exp(scores[ok] - M[ok, None])           # masked entries -> 0
        den = e.sum(axis=1) + np.exp(sigma - M[ok])
        out[ok] = (e @ vals) / den[:, None]
        lse[ok] = M[ok] + np.log(den)
    return out, lse


def attention_rows(q, k, v, sinks, b: int, h: int, rows, window: int, scale: float):
    """O[b,h,rows,:] and LSE[b,h,rows] of the definition, for selected query rows.

    q: [B,Hq,Lq,D], k/v: [B,Hkv,Lk,D] (any real dtype; upcast to float64),
    sinks: [Hq] or None.  rows: iterable of query indices.
    """
    Hq, Lq = q.shape[1], q.shape[2]
    Hkv, Lk = k.shape[1], k.shape[2]
    kvh = kv_head_of(h, Hq, Hkv)
    sc = effective_scale(scale)
    sigma = -np.inf if sinks is None else float(np.float64(sinks[h]))
    rows = np.asarray(list(rows), dtype=np.int64)
    ranges = [visible_range(query_position(int(i), Lq, Lk), Lk, window) for i in rows]
    lo = min((r[0] for r in ranges), default=0)
    hi = max((r[1] for r in ranges), default=0)
    hi = max(hi, lo)
    Kb = np.asarray(k[b, kvh, lo:hi], dtype=np.float64)
    Vb = np.asarray(v[b, kvh, lo:hi], dtype=np.float64)
    Qb = np.asarray(q[b, h, rows], dtype=np.float64)
    scores = sc * (Qb @ Kb.T)
    cols = np.arange(lo, hi)
    for r, (a, z) in enumerate(ranges):
        scores[r, (cols < a) | (cols >= z)] = -np.inf
    return _finish(scores, Vb, sigma)


def attention_fwd(q, k, v, sinks, window: int, scale: float, block: int = 256):
    """Full O [B,Hq,Lq,D] and LSE [B,Hq,Lq] of the definition (float64).

    Query rows are evaluated ``block`` at a time purely to bound memory; each
    row's arithmetic is the definition above.
    """
    B, Hq, Lq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    out = np.zeros((B, Hq, Lq, D))
    lse = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, Lq, block):
                rows = range(r0, min(Lq, r0 + block))
                o, l = attention_rows(q, k, v, sinks, b, h, rows, window, scale)
                out[b, h, r0:r0 + len(rows)] = o
                lse[b, h, r0:r0 + len(rows)] = l
    return out, lse


# ---------------------------------------------------------------------------
# backward (gradients of a scalar loss L through O, given dO = dL/dO)
# ---------------------------------------------------------------------------

def _bwd_block(Q, K, V, dO, sigma, sc, ranges, lo):
    """Gradients of one block of rows of one (b, h) over keys [lo, lo+K.shape[0]).

    With P_ij = e^{s_ij - LSE_i} (the sink inside LSE), Psink_i = e^{sigma - LSE_i},
    O = P V and D_i = <dO_i, O_i>:
        dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
        dQ = scale dS K,  dK = scale dS^T Q,  dsink = -sum_i Psink_i D_i.
    The sink has no value vector, so it enters dS only through D.
    """
    R, N = Q.shape[0], K.shape[0]
    S = sc * (Q @ K.T)
    cols = np.arange(lo, lo + N)
    for r, (a, z) in enumerate(ranges):
        S[r, (cols < a) | (cols >= z)] = -np.inf
    row_max = S.max(axis=1) if N else np.full(R, -np.inf)
    M = np.maximum(row_max, sigma)
    ok = np.isfinite(M)
    P = np.zeros((R, N))
    psink = np.zeros(R)
    if ok.any():
        e = np.exp(S[ok] - M[ok, None])
        es = np.exp(sigma - M[ok]) if np.isfinite(sigma) else np.zeros(int(ok.sum()))
        den = e.sum(axis=1) + es
        P[ok] = e / den[:, None]
        psink[ok] = es / den
    O = P @ V
    Dv = (dO * O).sum(axis=1)
    dP = dO @ V.T
    dS = P * (dP - Dv[:, None])
    return sc * (dS @ K), sc * (dS.T @ Q), P.T @ dO, -float((psink * Dv).sum())


def attention_bwd(q, k, v, sinks, dout, window: int, scale: float, block: int = 256):
    """dQ [B,Hq,Lq,D], dK, dV [B,Hkv,Lk,D] and dsink [Hq] of the forward above.

    Plain float64 definition of the gradients (flash-attention profile: the
    backward takes dO and computes dK/dV and dQ in two phases; the dsink
    precision issue #2969 is why D_i = <dO_i, O_i> is taken from the float64
    O here).  Query heads of a GQA group add into their shared KV head; dsink
    sums over every batch and row.  Rows are taken ``block`` at a time only to
    bound memory.
    """
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    sc = effective_scale(scale)
    dq = np.zeros((B, Hq, Lq, D))
    dk = np.zeros((B, Hkv, Lk, D))
    dv = np.zeros((B, Hkv, Lk, D))
    dsink = np.zeros(Hq)
    for b in range(B):
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            sigma = -np.inf if sinks is None else float(np.float64(sinks[h]))
            for r0 in range(0, Lq, block):
                rows = range(r0, min(Lq, r0 + block))
                ranges = [visible_range(query_position(i, Lq, Lk), Lk, window) for i in rows]
                lo = min(r[0] for r in ranges)
                hi = max(max(r[1] for r in ranges), lo)
                Q = np.asarray(q[b, h, r0:r0 + len(rows)], dtype=np.float64)
                dO = np.asarray(dout[b, h, r0:r0 + len(rows)], dtype=np.float64)
                K = np.asarray(k[b, kvh, lo:hi], dtype=np.float64)
                V = np.asarray(v[b, kvh, lo:hi], dtype=np.float64)
                gq, gk, gv, gs = _bwd_block(Q, K, V, dO, sigma, sc, ranges, lo)
                dq[b, h, r0:r0 + len(rows)] = gq
                dk[b, kvh, lo:hi] += gk
                dv[b, kvh, lo:hi] += gv
                dsink[h] += gs
    return dq, dk, dv, dsink


# ---------------------------------------------------------------------------
# maximum pre-softmax logit
# ---------------------------------------------------------------------------

def max_logit_rows(q, k, b: int, h: int, rows, window: int, scale: float):
    """Largest pre-softmax logit of selected query rows of (b, h).

    The logit is the score that enters the softmax, s_ij = scale * <q_i, k_j>,
    taken over the keys row i sees (the same causal/window/GQA rules as the
    forward); the sink is a learned logit, not an entry of Q K^T, and is not
    included.  A row that sees no key gives -inf.  (flash-attention
    contribution-radar profile, task card for issue #2986: expose the maximum
    pre-softmax logit of the forward pass, i.e. max of Q K^T rather than the
    log-sum-exp, with causal masking and GQA.)
    """
    Hq, Lq = q.shape[1], q.shape[2]
    Hkv, Lk = k.shape[1], k.shape[2]
    kvh = kv_head_of(h, Hq, Hkv)
    sc = effective_scale(scale)
    out = []
    for i in rows:
        lo, hi = visible_range(query_position(int(i), Lq, Lk), Lk, window)
        if hi <= lo:
            out.append(-np.inf)
            continue
        qi = np.asarray(q[b, h, int(i)], dtype=np.float64)
        kk = np.asarray(k[b, kvh, lo:hi], dtype=np.float64)
        out.append(float((sc * (kk @ qi)).max()))
    return np.array(out, dtype=np.float64)


def max_logit(q, k, window: int, scale: float):
    """Per-row [B,Hq,Lq] and per-head [B,Hq] maxima of the pre-softmax logit.

    The per-head value is the maximum over the head's rows (the shape the
    issue #2986 task card proposes); -inf where nothing is visible.
    """
    B, Hq, Lq, _ = q.shape
    if Hq % k.shape[1]:
        raise ValueError("Hq must be a multiple of Hkv")
    row = np.full((B, Hq, Lq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            row[b, h] = max_logit_rows(q, k, b, h, range(Lq), window, scale)
    head = row.max(axis=2) if Lq else np.full((B, Hq), -np.inf)
    return row, head


# ---------------------------------------------------------------------------
# split-KV decode and combine
# ---------------------------------------------------------------------------

SPLIT_ALIGN = 64   # split boundaries fall on multiples of 64 keys from the window start
MAX_SPLITS = 64


def split_ranges(Lk: int, num_splits: int, window: int) -> list[tuple[int, int]]:
    """The non-empty key ranges of the splits of one decode sequence.

    The single query sits at position Lk - 1, so it sees [lo, Lk) with
    lo = max(0, Lk - W) (no window: lo = 0).  The visible length n is cut into
    chunks of ceil(n / num_splits) keys rounded up to a multiple of 64; only
    the ceil(n / chunk) chunks that hold keys exist ("valid" splits).  Splits
    whose range would be empty are not listed: they are never computed or
    read (FlashMLA patch stack page, section 3).
    """
    ns = min(max(int(num_splits), 1), MAX_SPLITS)
    Lk = max(int(Lk), 0)
    lo = 0 if window <= 0 else max(0, Lk - window)
    n = Lk - lo
    if n <= 0:
        return []
    per = -(-n // ns)
    chunk = -(-per // SPLIT_ALIGN) * SPLIT_ALIGN
    out = []
    s0 = lo
    while s0 < Lk:
        out.append((s0, min(s0 + chunk, Lk)))
        s0 += chunk
    return out


# Split-count planning.  The FlashMLA patch stack page (section 1) describes a
# workload-aware partition policy: gather the workload's shape, choose the
# partition by policy (baseline / dynamic / fixed), reject what is illegal.
# The pages give no formula; the rule below is this library's, stated in
# include/attn.h, and restated here step by step.
PLAN_COUNT, PLAN_KEYS, PLAN_AUTO = "count", "keys", "auto"
PLAN_CHUNKS = (256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192)
PLAN_ITEM_COST = 400  # per-item cost of the decode beyond its keys, in key rows


def visible_keys(seqlen: int, Lk_max: int, window: int) -> int:
    """Keys the decode query of a sequence sees after clamping Lk to [0, Lk_max]."""
    Lk = min(max(int(seqlen), 0), Lk_max)
    lo = max(0, Lk - window) if window > 0 else 0
    return Lk - lo


def plan_splits(seqlens, Hq: int, Hkv: int, Lk_max: int, window: int, max_splits: int,
                policy: str, param: int, slots: int) -> list[int]:
    """num_splits per sequence under a policy.

    count: every sequence gets param splits; keys: ceil(n/param) splits for n
    visible keys; auto: the chunk target c from PLAN_CHUNKS that minimises
        ceil(I / S) * (Z + PLAN_ITEM_COST),
    where for target c every sequence takes ceil(n/c) splits, I counts the
    decode's work items (valid splits x KV heads x query-column groups of
    32), Z is the largest split in keys and S the units the items are spread
    over (slots): the items of the most loaded unit, each priced as the
    largest split plus a fixed per-item cost.  The first such c wins.
    Splits are clamped to [1, max_splits] in every policy.
    """
    ns_of = lambda n, c: min(max(-(-n // c), 1), max_splits)
    ns_clamp = lambda x: min(max(int(x), 1), max_splits)
    lens = [visible_keys(x, Lk_max, window) for x in seqlens]
    if policy == PLAN_COUNT:
        return [ns_clamp(param) for _ in lens]
    if policy == PLAN_KEYS:
        return [ns_of(n, int(param)) for n in lens]
    if policy != PLAN_AUTO:
        raise ValueError(policy)
    G = Hq // Hkv
    hq = Hkv * (-(-G // 32))
    best = None
    for c in PLAN_CHUNKS:
        items, z = 0, 0
        for n in lens:
            if n == 0:
                continue
            parts = split_ranges(n, ns_of(n, c), 0)
            items += len(parts)
            z = max(z, max(e - a for a, e in parts))
        items *= hq
        per = -(-items // slots)
        cost = per * (z + PLAN_ITEM_COST)
        if best is None or cost < best[0]:
            best = (cost, c)
    return [ns_of(n, best[1]) for n in lens]


def decode_partials(q, k_cache, v_cache, seqlens, num_splits, window: int, scale: float,
                    max_splits: int = MAX_SPLITS):
    """Per-split normalised outputs and sink-free LSEs of a decode step.

    q: [B,Hq,1,D]; caches [B,Hkv,Lk_max,D]; seqlens, num_splits: [B] ints.
    Returns o_part [B,Hq,max_splits,D], lse_part [B,Hq,max_splits] (lanes of
    splits that do not exist hold NaN: nothing may read them), n_valid [B].

    For split s with key set J_s:  lse_s = ln sum_{J_s} e^{s_j},
    O_s = sum_{J_s} e^{s_j - lse_s} v_j  -- i.e. attention over J_s, no sink.
    """
    B, Hq, _, D = q.shape
    o_part = np.full((B, Hq, max_splits, D), np.nan)
    lse_part = np.full((B, Hq, max_splits), np.nan)
    n_valid = np.zeros(B, dtype=np.int64)
    for b in range(B):
        Lk = int(seqlens[b])
        sp = split_ranges(Lk, int(num_splits[b]), window)
        n_valid[b] = len(sp)
        for s, (a, z) in enumerate(sp):
            kk = k_cache[b:b + 1, :, a:z]
            vv = v_cache[b:b + 1, :, a:z]
            for h in range(Hq):
                # the query (position Lk-1) sees every key of [a, z): no window
                # or causal limit cuts inside a split.
                o, l = attention_rows(q[b:b + 1], kk, vv, None, 0, h, [0],
                                      window=0, scale=scale)
                o_part[b, h, s] = o[0]
                lse_part[b, h, s] = l[0]
    return o_part, lse_part, n_valid


def combine(o_part, lse_part, n_valid, sinks):
    """Merge the valid split partials of each (b, h) and add the sink once.

    M = max(max_s lse_s, sigma); w_s = e^{lse_s - M};
    den = sum_s w_s + e^{sigma - M}; O = sum_s w_s O_s / den; LSE = M + ln den.
    Only lanes s < n_valid[b] are read, in order s = 0, 1, ...
    """
    B, Hq, _, D = o_part.shape
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(n_valid[b])
        for h in range(Hq):
            sigma = -np.inf if sinks is None else float(np.float64(sinks[h]))
            ls = np.asarray(lse_part[b, h, :n], dtype=np.float64)
            M = max(ls.max() if n else -np.inf, sigma)
            if not np.isfinite(M):
                continue
            w = np.exp(ls - M)
            den = w.sum() + math.exp(sigma - M) if np.isfinite(sigma) else w.sum()
            acc = np.zeros(D)
            for s in range(n):
                acc += w[s] * np.asarray(o_part[b, h, s], dtype=np.float64)
            out[b, h] = acc / den
            lse[b, h] = M + math.log(den)
    return out, lse


def decode(q, k_cache, v_cache, seqlens, sinks, window: int, scale: float):
    """Unsplit decode: attention of each sequence's single query over its cache.

    Equal by definition to ``attention_fwd`` with Lq = 1 on K[:, :, :Lk_b].
    Returns O [B,Hq,D], LSE [B,Hq].
    """
    B, Hq, _, D = q.shape
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        Lk = int(seqlens[b])
        kk = k_cache[b:b + 1, :, :Lk]
        vv = v_cache[b:b + 1, :, :Lk]
        for h in range(Hq):
            o, l = attention_rows(q[b:b + 1], kk, vv, sinks, 0, h, [0], window, scale)
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse


# ---------------------------------------------------------------------------
# paged KV caches and variable-length batches (the serving layouts: the
# flash-attention profile lists paged KV -- block_table -- for decode and
# varlen batches described by cu_seqlens among its capabilities and call flow)
# ---------------------------------------------------------------------------

def page_slot(j: int, page_size: int) -> tuple[int, int]:
    """(block-table slot, row within the page) that holds key j."""
    return j // page_size, j % page_size


def gather_paged(pages, block_table, seqlens, page_size: int, Lk_max: int):
    """Dense cache [B,Hkv,Lk_max,D] of a paged one.

    pages [num_pages,Hkv,page_size,D]; block_table [B,max_pages] ints; key j
    of sequence b is row j % page_size of page block_table[b, j // page_size].
    Rows at or past seqlens[b] (clamped to [0, Lk_max]) stay NaN: no
    computation may read them.
    """
    pages = np.asarray(pages, dtype=np.float64)
    B = len(seqlens)
    _, Hkv, _, D = pages.shape
    dense = np.full((B, Hkv, Lk_max, D), np.nan)
    for b in range(B):
        Lk = min(max(int(seqlens[b]), 0), Lk_max)
        for j in range(Lk):
            slot, row = page_slot(j, page_size)
            dense[b, :, j] = pages[int(block_table[b][slot]), :, row]
    return dense


def decode_paged(q, k_pages, v_pages, block_table, seqlens, sinks, window: int, scale: float,
                 page_size: int, Lk_max: int):
    """Unsplit decode over a paged cache: the decode of the gathered cache."""
    kc = gather_paged(k_pages, block_table, seqlens, page_size, Lk_max)
    vc = gather_paged(v_pages, block_table, seqlens, page_size, Lk_max)
    sl = [min(max(int(x), 0), Lk_max) for x in seqlens]
    return decode(q, kc, vc, sl, sinks, window, scale)


def attention_fwd_varlen(q, k, v, cu_q, cu_k, sinks, window: int, scale: float):
    """Attention over a packed batch of sequences of different lengths.

    q [Hq,total_q,D], k/v [Hkv,total_k,D]; sequence b owns query rows
    cu_q[b]..cu_q[b+1] and keys cu_k[b]..cu_k[b+1].  Within a sequence the
    rules of ``attention_fwd`` hold (its queries are its last Lq_b positions;
    a row with no key gets O = 0 and LSE = sink).  Returns out [Hq,total_q,D]
    and lse [Hq,total_q].
    """
    Hq, total_q, D = q.shape
    out = np.zeros((Hq, total_q, D))
    lse = np.zeros((Hq, total_q))
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        if q1 <= q0:
            continue
        o, l = attention_fwd(np.asarray(q)[None, :, q0:q1], np.asarray(k)[None, :, k0:k1],
                             np.asarray(v)[None, :, k0:k1], sinks, window, scale)
        out[:, q0:q1] = o[0]
        lse[:, q0:q1] = l[0]
    return out, lse


# ---------------------------------------------------------------------------
# the two sink updates of the cf-1.com page (fix two), in float32
# ---------------------------------------------------------------------------

def naive_sink_row_sum_f32(row_max, row_sum, sink, scale_log2):
    """The old additive update: row_sum + 2^(sink*log2e - row_max*scale_log2).

    row_max is in raw-score units, scale_log2 = scale * log2(e); max_offset = 0.
    Evaluated in float32, as the kernel did.
    """
    f = np.float32
    with np.errstate(over="ignore"):
        t = f(f(sink) * f(LOG2E)) - f(f(row_max) * f(scale_log2))
        return f(row_sum) + np.exp2(f(t), dtype=np.float32)


def rebase_sink_f32(row_max, row_sum, sink, scale_log2):
    """The rebased update, float32: returns (new row_max, new row_sum, sink_rescale).

    old = row_max*scale_log2; new = max(old, sink*log2e);
    sink_rescale = 2^(old - new); row_sum = row_sum*sink_rescale + 2^(sink*log2e - new);
    row_max = new / scale_log2.  The output scale is sink_rescale / row_sum
    (v_descale = 1).  Every exponent is <= 0, so no term exceeds 1.
    """
    f = np.float32
    old = f(f(row_max) * f(scale_log2))
    sl = f(f(sink) * f(LOG2E))
    new = max(old, sl)
    rescale = np.exp2(f(old - new), dtype=np.float32)
    rs = f(f(row_sum) * rescale + np.exp2(f(sl - new), dtype=np.float32))
    return f(new / f(scale_log2)), rs, rescale
