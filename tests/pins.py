"""Independent checks that pin the float64 oracle (used by test_oracle.py).

Each function returns the largest discrepancy between the oracle and
something the pages or mathematics fix on their own: brute-force softmax with
plain Python loops, torch's float64 CPU attention (a library routine), closed
forms of the sink, exact visible-key counts, and split/merge identities.  They
are kept apart from the tests so that a test can plant a mistake in the oracle
and show that some pin catches it.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def brute_force(q, k, v, sinks, window, scale):
    """O, LSE by Python loops: softmax over the visible keys plus one extra
    key whose logit is the sink and whose value vector is zero."""
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    O = np.zeros((B, Hq, Lq, D))
    LSE = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Lq):
                pos = Lk - Lq + i
                logits, vals = [], []
                for j in range(Lk):
                    if j > pos:
                        continue
                    if window > 0 and pos - j >= window:
                        continue
                    logits.append(sc * math.fsum(q[b, h, i, d] * k[b, g, j, d] for d in range(D)))
                    vals.append([v[b, g, j, d] for d in range(D)])
                if sinks is not None:
                    logits.append(float(sinks[h]))
                    vals.append([0.0] * D)
                if not logits:
                    LSE[b, h, i] = -math.inf
                    continue
                top = max(logits)
                ws = [math.exp(x - top) for x in logits]
                tot = math.fsum(ws)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(w * val[d] for w, val in zip(ws, vals)) / tot
                LSE[b, h, i] = top + math.log(tot)
    return O, LSE


def torch_reference(q, k, v, sinks, window, scale):
    """O, LSE from torch's float64 CPU flash attention (returns the logsumexp).

    GQA by repeat_interleave of K/V along heads; causal + window as an additive
    -inf mask built from index comparisons; the sink as one extra key of zero
    vectors whose mask entry is the sink logit.
    """
    q_t = torch.from_numpy(np.asarray(q, dtype=np.float64))
    k_t = torch.from_numpy(np.asarray(k, dtype=np.float64))
    v_t = torch.from_numpy(np.asarray(v, dtype=np.float64))
    B, Hq, Lq, D = q_t.shape
    Hkv, Lk = k_t.shape[1], k_t.shape[2]
    G = Hq // Hkv
    k_t = k_t.repeat_interleave(G, dim=1)
    v_t = v_t.repeat_interleave(G, dim=1)
    pos = torch.arange(Lq).unsqueeze(1) + (Lk - Lq)
    key = torch.arange(Lk).unsqueeze(0)
    keep = key <= pos
    if window > 0:
        keep &= key > pos - window
    mask = torch.zeros(Lq, Lk, dtype=torch.float64).masked_fill(~keep, -math.inf)
    mask = mask.expand(B, Hq, Lq, Lk)
    if sinks is not None:
        k_t = torch.cat([k_t, torch.zeros(B, Hq, 1, D, dtype=torch.float64)], dim=2)
        v_t = torch.cat([v_t, torch.zeros(B, Hq, 1, D, dtype=torch.float64)], dim=2)
        col = torch.from_numpy(np.asarray(sinks, dtype=np.float64)).view(1, Hq, 1, 1)
        mask = torch.cat([mask, col.expand(B, Hq, Lq, 1)], dim=3)
    sc = float(np.float32(scale))
    o, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        q_t, k_t, v_t, 0.0, False, attn_mask=mask.contiguous(), scale=sc)
    return o.numpy(), lse.numpy()


def err_vs_brute(seed=0, B=2, Hq=4, Hkv=2, Lq=6, Lk=8, D=3, window=3, sink_scale=1.0,
                 with_sink=True):
    q, k, v = rand((B, Hq, Lq, D), seed), rand((B, Hkv, Lk, D), seed + 1), rand((B, Hkv, Lk, D), seed + 2)
    sinks = rand(Hq, seed + 3, sink_scale) if with_sink else None
    scale = 0.7
    o, l = oracle.attention_fwd(q, k, v, sinks, window, scale)
    ob, lb = brute_force(q, k, v, sinks, window, scale)
    return max(np.abs(o - ob).max(), np.abs(l - lb).max())


def err_vs_torch(seed=0, B=1, Hq=4, Hkv=2, Lq=100, Lk=130, D=16, window=7, with_sink=True):
    q, k, v = rand((B, Hq, Lq, D), seed), rand((B, Hkv, Lk, D), seed + 1), rand((B, Hkv, Lk, D), seed + 2)
    sinks = rand(Hq, seed + 3, 2.0) if with_sink else None
    scale = 1 / math.sqrt(D)
    o, l = oracle.attention_fwd(q, k, v, sinks, window, scale, block=37)
    ot, lt = torch_reference(q, k, v, sinks, window, scale)
    return max(np.abs(o - ot).max(), np.abs(l - lt).max())


def visible_count(i, Lq, Lk, window):
    """Number of keys the query row i sees, by counting integers."""
    p = i + Lk - Lq
    n = 0
    for j in range(Lk):
        if j <= p and (window <= 0 or p - j < window):
            n += 1
    return n


def err_counts(Lq=40, Lk=50, window=7, sink=None, D=2):
    """Q = 0 makes every score 0; V = 1 then gives O = n/(n + e^sigma) and
    LSE = ln(n + e^sigma) with n the exact visible-key count."""
    q = np.zeros((1, 1, Lq, D))
    k = rand((1, 1, Lk, D), 5)
    v = np.ones((1, 1, Lk, D))
    sinks = None if sink is None else np.array([sink])
    o, l = oracle.attention_fwd(q, k, v, sinks, window, 0.3)
    n = np.array([visible_count(i, Lq, Lk, window) for i in range(Lq)], dtype=np.float64)
    es = 0.0 if sink is None else math.exp(sink)
    want_o = n / (n + es)
    want_l = np.log(n + es)
    return max(np.abs(o[0, 0, :, 0] - want_o).max(), np.abs(l[0, 0] - want_l).max())


def err_sink_closed_form(seed=0, sigma=2.5, window=9, Lq=30, Lk=30, D=8):
    """Adding a sink sigma multiplies O by sigmoid(LSE0 - sigma) and turns
    LSE0 into logaddexp(LSE0, sigma), where 0 marks the sink-free result."""
    q, k, v = rand((1, 2, Lq, D), seed), rand((1, 1, Lk, D), seed + 1), rand((1, 1, Lk, D), seed + 2)
    o0, l0 = oracle.attention_fwd(q, k, v, None, window, 0.4)
    o1, l1 = oracle.attention_fwd(q, k, v, np.array([sigma, sigma]), window, 0.4)
    sig = 1.0 / (1.0 + np.exp(sigma - l0))
    return max(np.abs(o1 - o0 * sig[..., None]).max(), np.abs(l1 - np.logaddexp(l0, sigma)).max())


def err_gqa(seed=0, Hq=8, Hkv=2, L=40, D=8, window=11):
    """GQA equals MHA on K/V whose heads are repeated G times (consecutive)."""
    q, k, v = rand((2, Hq, L, D), seed), rand((2, Hkv, L, D), seed + 1), rand((2, Hkv, L, D), seed + 2)
    sinks = rand(Hq, seed + 3)
    o, l = oracle.attention_fwd(q, k, v, sinks, window, 0.5)
    G = Hq // Hkv
    o2, l2 = oracle.attention_fwd(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), sinks, window, 0.5)
    return max(np.abs(o - o2).max(), np.abs(l - l2).max())


def err_split_combine(Lks=(1, 2, 63, 64, 65, 127, 129, 700, 1025), windows=(0, 513, 64, 1),
                      splits=(1, 2, 3, 7, 31, 32, 33, 63, 64), Hq=4, Hkv=2, D=8, seed=0):
    """Split-KV partials merged by the combine equal the unsplit decode."""
    Lmax = max(Lks)
    B = len(Lks)
    q = rand((B, Hq, 1, D), seed)
    kc, vc = rand((B, Hkv, Lmax, D), seed + 1), rand((B, Hkv, Lmax, D), seed + 2)
    sinks = rand(Hq, seed + 3)
    seqlens = np.array(Lks)
    worst = 0.0
    for W in windows:
        ref_o, ref_l = oracle.decode(q, kc, vc, seqlens, sinks, W, 0.35)
        for ns in splits:
            nsv = np.full(B, ns)
            op, lp, nv = oracle.decode_partials(q, kc, vc, seqlens, nsv, W, 0.35)
            o, l = oracle.combine(op, lp, nv, sinks)
            worst = max(worst, np.abs(o - ref_o).max(), np.abs(l - ref_l).max())
    return worst


# --- maximum pre-softmax logit ------------------------------------------------

def brute_max_logit(q, k, window, scale):
    """Per-row max of scale*<q_i,k_j> over visible keys, by Python loops (-inf if none)."""
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.full((B, Hq, Lq), -math.inf)
    for b in range(B):
        for h in range(Hq):
            for i in range(Lq):
                pos = Lk - Lq + i
                for j in range(Lk):
                    if j > pos or (window > 0 and pos - j >= window):
                        continue
                    s = sc * math.fsum(q[b, h, i, d] * k[b, h // G, j, d] for d in range(D))
                    out[b, h, i] = max(out[b, h, i], s)
    return out


def err_max_logit_brute(seed=0, B=2, Hq=4, Hkv=2, Lq=6, Lk=9, D=3, window=3):
    q, k = rand((B, Hq, Lq, D), seed), rand((B, Hkv, Lk, D), seed + 1)
    row, head = oracle.max_logit(q, k, window, 0.7)
    want = brute_max_logit(q, k, window, 0.7)
    return max(np.abs(row - want).max(), np.abs(head - want.max(axis=2)).max())


def err_max_logit_ramp(Lq=37, Lk=50, window=7, scale=0.3, D=4):
    """Keys along one direction u with k_j = (j + 1) u, queries q = u (resp. -u):
    the row maximum is scale*(p + 1) at the last visible key p (resp.
    -scale*(lo + 1) at the first visible key lo), exact in float64."""
    u = np.zeros(D)
    u[1] = 1.0
    k = (np.arange(Lk, dtype=np.float64)[:, None] + 1.0) * u
    k = k[None, None]
    sc = float(np.float32(scale))
    worst = 0.0
    for sign in (1.0, -1.0):
        q = np.broadcast_to(sign * u, (1, 1, Lq, D)).copy()
        row, _ = oracle.max_logit(q, k, window, scale)
        for i in range(Lq):
            p = i + Lk - Lq
            lo = max(0, p - window + 1) if window > 0 else 0
            want = sc * (p + 1) if sign > 0 else -sc * (lo + 1)
            worst = max(worst, abs(row[0, 0, i] - want))
    return worst


def err_max_logit_lse_bounds(seed=0, Hq=4, Hkv=2, Lq=40, Lk=60, D=8, window=9):
    """Without a sink, max_j s_j <= LSE <= max_j s_j + ln(n) with n visible keys;
    returns how far the oracle's maximum falls outside these bounds."""
    q, k, v = rand((1, Hq, Lq, D), seed, 2.0), rand((1, Hkv, Lk, D), seed + 1), rand((1, Hkv, Lk, D), seed + 2)
    row, _ = oracle.max_logit(q, k, window, 0.5)
    _, lse = oracle.attention_fwd(q, k, v, None, window, 0.5)
    n = np.array([visible_count(i, Lq, Lk, window) for i in range(Lq)], dtype=np.float64)
    over = np.maximum(row - lse, 0.0)
    under = np.maximum(lse - (row + np.log(n)), 0.0)
    return max(over.max(), under.max())


def err_max_logit_torch(seed=0, B=2, Hq=6, Hkv=3, Lq=50, Lk=70, D=16, window=13):
    """torch: float64 matmul of repeated K heads, -inf where an index mask forbids, amax."""
    q, k = rand((B, Hq, Lq, D), seed), rand((B, Hkv, Lk, D), seed + 1)
    q_t = torch.from_numpy(q)
    k_t = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    sc = float(np.float32(0.25))
    s = sc * torch.matmul(q_t, k_t.transpose(-1, -2).contiguous())
    pos = torch.arange(Lq).unsqueeze(1) + (Lk - Lq)
    key = torch.arange(Lk).unsqueeze(0)
    keep = key <= pos
    if window > 0:
        keep &= key > pos - window
    want = s.masked_fill(~keep, -math.inf).amax(dim=-1).numpy()
    row, head = oracle.max_logit(q, k, window, 0.25)
    return max(np.abs(row - want).max(), np.abs(head - want.max(axis=2)).max())


def err_max_logit_gqa(seed=0, Hq=8, Hkv=2, L=30, D=8, window=5):
    q, k = rand((2, Hq, L, D), seed), rand((2, Hkv, L, D), seed + 1)
    row, head = oracle.max_logit(q, k, window, 0.5)
    row2, head2 = oracle.max_logit(q, np.repeat(k, Hq // Hkv, axis=1), window, 0.5)
    return max(np.abs(row - row2).max(), np.abs(head - head2).max())


# --- split-count planning -------------------------------------------------------

# The planning rule as include/attn.h states it, retyped here on purpose so
# that a changed constant in the oracle shows up.
RULE_CHUNKS = (256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192)
RULE_ITEM_COST = 400


def brute_plan_auto(seqlens, Hq, Hkv, Lk_max, window, max_splits, slots):
    """The auto policy by walking every split of every sequence key by key."""
    G = Hq // Hkv
    hq = Hkv * ((G + 31) // 32)
    lens = []
    for x in seqlens:
        Lk = min(max(int(x), 0), Lk_max)
        lo = max(0, Lk - window) if window > 0 else 0
        lens.append(Lk - lo)
    best_cost, best_c = None, None
    for c in RULE_CHUNKS:
        items, zmax = 0, 0
        for n in lens:
            if n == 0:
                continue
            ns = min(max(math.ceil(n / c), 1), max_splits)
            chunk = math.ceil(math.ceil(n / ns) / 64) * 64
            start = 0
            while start < n:                      # one split per step
                size = min(chunk, n - start)
                items += 1
                zmax = max(zmax, size)
                start += chunk
        items *= hq
        per = math.ceil(items / slots)
        cost = per * (zmax + RULE_ITEM_COST)
        if best_cost is None or cost < best_cost:
            best_cost, best_c = cost, c
    return [min(max(math.ceil(n / best_c), 1), max_splits) for n in lens]


def err_plan(seed=0, B=40, Lk_max=5000, window=0, Hq=64, Hkv=8, max_splits=64, slots=512):
    """Number of sequences whose planned split count differs from the
    closed forms (count, keys) and the brute-force auto rule."""
    rng = np.random.default_rng(seed)
    seqlens = list(rng.integers(-5, Lk_max + 300, B))
    bad = 0
    for p in (1, 7, 64, 100):
        got = oracle.plan_splits(seqlens, Hq, Hkv, Lk_max, window, max_splits, "count", p, slots)
        bad += sum(g != min(max(p, 1), max_splits) for g in got)
    for p in (64, 100, 1024):
        got = oracle.plan_splits(seqlens, Hq, Hkv, Lk_max, window, max_splits, "keys", p, slots)
        for g, x in zip(got, seqlens):
            Lk = min(max(int(x), 0), Lk_max)
            n = Lk - (max(0, Lk - window) if window > 0 else 0)
            bad += g != min(max(math.ceil(n / p), 1), max_splits)
    got = oracle.plan_splits(seqlens, Hq, Hkv, Lk_max, window, max_splits, "auto", 0, slots)
    want = brute_plan_auto(seqlens, Hq, Hkv, Lk_max, window, max_splits, slots)
    bad += sum(g != w for g, w in zip(got, want))
    return bad


# --- paged KV and varlen ---------------------------------------------------------

def make_paged(dense, seqlens, page_size, seed, extra_pages=3):
    """Scatter a dense cache [B,Hkv,Lk_max,D] into pages in a random order.

    Returns pages [num_pages,Hkv,page_size,D] (unused pages and rows NaN) and
    a block table [B,max_pages] whose unused slots name a NaN page."""
    rng = np.random.default_rng(seed)
    B, Hkv, Lk_max, D = dense.shape
    max_pages = -(-Lk_max // page_size)
    need = [-(-int(L) // page_size) for L in seqlens]
    num_pages = sum(need) + extra_pages
    order = rng.permutation(num_pages)
    pages = np.full((num_pages, Hkv, page_size, D), np.nan)
    table = np.full((B, max_pages), int(order[-1]), dtype=np.int64)  # a NaN page
    k = 0
    for b in range(B):
        for p in range(need[b]):
            pid = int(order[k]); k += 1
            table[b, p] = pid
            rows = dense[b, :, p * page_size:(p + 1) * page_size]
            pages[pid, :, :rows.shape[1]] = rows
    return pages, table


def err_paged(seed=0, B=5, Hq=4, Hkv=2, Lk_max=300, D=8, page_size=16, window=0):
    """Paged decode through a shuffled block table equals the dense decode."""
    rng = np.random.default_rng(seed)
    seqlens = rng.integers(1, Lk_max + 1, B)
    q = rand((B, Hq, 1, D), seed)
    kc, vc = rand((B, Hkv, Lk_max, D), seed + 1), rand((B, Hkv, Lk_max, D), seed + 2)
    sinks = rand(Hq, seed + 3)
    kp, table = make_paged(kc, seqlens, page_size, seed)
    vp, table2 = make_paged(vc, seqlens, page_size, seed)
    assert np.array_equal(table, table2)
    o, l = oracle.decode_paged(q, kp, vp, table, seqlens, sinks, window, 0.4, page_size, Lk_max)
    od, ld = oracle.decode(q, kc, vc, seqlens, sinks, window, 0.4)
    # key by key through the table, by hand
    worst = max(np.abs(o - od).max(), np.abs(l - ld).max())
    g = oracle.gather_paged(kp, table, seqlens, page_size, Lk_max)
    for b in range(B):
        for j in range(int(seqlens[b])):
            pid = table[b, j // page_size]
            worst = max(worst, np.abs(g[b, :, j] - kp[pid, :, j % page_size]).max())
        assert np.isnan(g[b, :, int(seqlens[b]):]).all()
    return worst


def err_varlen_equal_lengths(seed=0, B=3, Hq=4, Hkv=2, L=40, D=8, window=7):
    """Equal lengths: the packed batch equals the dense batched call."""
    q, k, v = rand((B, Hq, L, D), seed), rand((B, Hkv, L, D), seed + 1), rand((B, Hkv, L, D), seed + 2)
    sinks = rand(Hq, seed + 3)
    o, l = oracle.attention_fwd(q, k, v, sinks, window, 0.3)
    pack = lambda x: np.concatenate(list(x), axis=1)  # [B,H,L,D] -> [H,B*L,D]
    cu = np.arange(B + 1) * L
    ov, lv = oracle.attention_fwd_varlen(pack(q), pack(k), pack(v), cu, cu, sinks, window, 0.3)
    return max(np.abs(ov - pack(o)).max(), np.abs(lv - np.concatenate(list(l), axis=1)).max())


def err_varlen_brute(seed=0, Hq=2, Hkv=1, D=3, window=3):
    """Mixed lengths (Lq < Lk, Lq > Lk, empty) against brute force per sequence."""
    lq = [3, 1, 0, 4, 5]
    lk = [5, 1, 2, 4, 2]
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    q = rand((Hq, cu_q[-1], D), seed)
    k, v = rand((Hkv, cu_k[-1], D), seed + 1), rand((Hkv, cu_k[-1], D), seed + 2)
    sinks = rand(Hq, seed + 3)
    o, l = oracle.attention_fwd_varlen(q, k, v, cu_q, cu_k, sinks, window, 0.7)
    worst = 0.0
    for b in range(len(lq)):
        if lq[b] == 0:
            continue
        qs = q[None, :, cu_q[b]:cu_q[b + 1]]
        ks, vs = k[None, :, cu_k[b]:cu_k[b + 1]], v[None, :, cu_k[b]:cu_k[b + 1]]
        if lq[b] <= lk[b]:
            ob, lb = brute_force(qs, ks, vs, sinks, window, 0.7)
        else:
            # queries past the keys: the first lq-lk rows see nothing
            pad = lq[b] - lk[b]
            ob = np.zeros((1, Hq, lq[b], D))
            lb = np.broadcast_to(np.asarray(sinks, np.float64)[None, :, None], (1, Hq, lq[b])).copy()
            o2, l2 = brute_force(qs[:, :, pad:], ks, vs, sinks, window, 0.7)
            ob[:, :, pad:], lb[:, :, pad:] = o2, l2
        worst = max(worst, np.abs(o[:, cu_q[b]:cu_q[b + 1]] - ob[0]).max(),
                    np.abs(l[:, cu_q[b]:cu_q[b + 1]] - lb[0]).max())
    return worst


# --- backward ---------------------------------------------------------------------

def loss_fd(q, k, v, sinks, dout, window, scale):
    """L = <dout, O> from the forward oracle (for finite differences)."""
    o, _ = oracle.attention_fwd(q, k, v, sinks, window, scale)
    return float((np.asarray(dout) * o).sum())


def err_bwd_finite_diff(seed=0, B=1, Hq=2, Hkv=1, Lq=5, Lk=6, D=3, window=3, eps=1e-6):
    """Largest |analytic - central difference| over every element of q, k, v, sinks."""
    q, k, v = rand((B, Hq, Lq, D), seed), rand((B, Hkv, Lk, D), seed + 1), rand((B, Hkv, Lk, D), seed + 2)
    sinks = rand(Hq, seed + 3)
    dout = rand((B, Hq, Lq, D), seed + 4)
    dq, dk, dv, ds = oracle.attention_bwd(q, k, v, sinks, dout, window, 0.6)
    worst = 0.0
    for x, g in ((q, dq), (k, dk), (v, dv), (sinks, ds)):
        flat, gflat = x.reshape(-1), g.reshape(-1)
        for n in range(flat.size):
            old = flat[n]
            flat[n] = old + eps
            lp = loss_fd(q, k, v, sinks, dout, window, 0.6)
            flat[n] = old - eps
            lm = loss_fd(q, k, v, sinks, dout, window, 0.6)
            flat[n] = old
            worst = max(worst, abs((lp - lm) / (2 * eps) - gflat[n]))
    return worst


def torch_bwd(q, k, v, sinks, dout, window, scale):
    """Gradients by torch autograd in float64: logits with the sink as one more
    column (no value vector), index-built mask, GQA by repeat_interleave."""
    t = lambda x: torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    qt, kt, vt, st = t(q), t(k), t(v), t(sinks)
    B, Hq, Lq, D = qt.shape
    Hkv, Lk = kt.shape[1], kt.shape[2]
    G = Hq // Hkv
    kr, vr = kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1)
    sc = float(np.float32(scale))
    s = sc * torch.matmul(qt, kr.transpose(-1, -2))
    pos = torch.arange(Lq).unsqueeze(1) + (Lk - Lq)
    key = torch.arange(Lk).unsqueeze(0)
    keep = key <= pos
    if window > 0:
        keep &= key > pos - window
    s = s.masked_fill(~keep, -math.inf)
    logits = torch.cat([s, st.view(1, Hq, 1, 1).expand(B, Hq, Lq, 1)], dim=3)
    p = torch.softmax(logits, dim=3)[..., :Lk]
    o = torch.matmul(p, vr)
    (o * torch.tensor(np.asarray(dout, np.float64))).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), st.grad.numpy()


def err_bwd_torch(seed=0, B=2, Hq=4, Hkv=2, Lq=40, Lk=55, D=8, window=9):
    q, k, v = rand((B, Hq, Lq, D), seed), rand((B, Hkv, Lk, D), seed + 1), rand((B, Hkv, Lk, D), seed + 2)
    sinks = rand(Hq, seed + 3, 2.0)
    dout = rand((B, Hq, Lq, D), seed + 4)
    got = oracle.attention_bwd(q, k, v, sinks, dout, window, 0.35, block=17)
    want = torch_bwd(q, k, v, sinks, dout, window, 0.35)
    return max(np.abs(a - b).max() for a, b in zip(got, want))


def err_bwd_gqa(seed=0, Hq=6, Hkv=2, L=20, D=4, window=5):
    """GQA gradients: dK, dV of a KV head are the sums over its repeated MHA copies."""
    q, k, v = rand((1, Hq, L, D), seed), rand((1, Hkv, L, D), seed + 1), rand((1, Hkv, L, D), seed + 2)
    sinks, dout = rand(Hq, seed + 3), rand((1, Hq, L, D), seed + 4)
    G = Hq // Hkv
    dq, dk, dv, ds = oracle.attention_bwd(q, k, v, sinks, dout, window, 0.5)
    dq2, dk2, dv2, ds2 = oracle.attention_bwd(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                                              sinks, dout, window, 0.5)
    fold = lambda x: x.reshape(1, Hkv, G, L, D).sum(axis=2)
    return max(np.abs(dq - dq2).max(), np.abs(dk - fold(dk2)).max(), np.abs(dv - fold(dv2)).max(),
               np.abs(ds - ds2).max())


def err_bwd_shift_invariance(seed=0, Hq=2, L=30, D=4, window=7):
    """Shifting every logit and the sink by c leaves O unchanged, so with all keys
    equal to one vector u, dsink = -sum_i <dQ_i, u> / (scale |u|^2)."""
    u = np.array([0.3, -0.2, 0.5, 0.1])
    k = np.broadcast_to(u, (1, 1, L, D)).copy()
    q, v = rand((1, Hq, L, D), seed), rand((1, 1, L, D), seed + 2)
    sinks, dout = rand(Hq, seed + 3), rand((1, Hq, L, D), seed + 4)
    sc = float(np.float32(0.5))
    dq, _, _, ds = oracle.attention_bwd(q, k, v, sinks, dout, window, 0.5)
    want = -(dq[0] @ u).sum(axis=1) / (sc * float(u @ u))
    return np.abs(ds - want).max()
