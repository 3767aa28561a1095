"""GPU parity of the serving layouts: split-KV decode over a paged KV cache
(block table) and the forward over a packed varlen batch, against the oracle,
and against the dense entry points on the same data (to 1e-5: the same sums in
the same order, up to how each kernel contracts multiply-adds)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_attention_attn_amd as A
import oracle
from exact_attention_attn_amd import workloads as W

gpu_util = pytest.importorskip("gpu_util")
from gpu_util import compare, full_decode_inputs, host_values, run_decode, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

NAN_BF16 = np.uint16(0x7FC0)


def page_cache(dense_bits, seqlens, page_size, seed, junk_slots=False):
    """bf16 cache [B,Hkv,Lk_max,D] -> shuffled pages [num_pages,Hkv,page_size,D]
    (unused rows NaN) and a block table whose unused slots name a NaN page (or,
    with junk_slots, a page id far outside the pool: such slots are never read)."""
    rng = np.random.default_rng(seed)
    B, Hkv, Lk_max, D = dense_bits.shape
    max_pages = -(-Lk_max // page_size)
    need = [-(-int(L) // page_size) for L in seqlens]
    num_pages = sum(need) + 2
    order = rng.permutation(num_pages)
    pages = np.full((num_pages, Hkv, page_size, D), NAN_BF16, dtype=np.uint16)
    fill = 1 << 30 if junk_slots else int(order[-1])
    table = np.full((B, max_pages), fill, dtype=np.int32)
    i = 0
    for b in range(B):
        for p in range(need[b]):
            pid = int(order[i]); i += 1
            table[b, p] = pid
            lo, hi = p * page_size, min((p + 1) * page_size, int(seqlens[b]))
            pages[pid, :, :hi - lo] = dense_bits[b, :, lo:hi]
    return pages, table


def run_paged(q, kp, vp, table, seqlens, nsplits, sinks, window, scale, max_splits=64):
    B, Hq, _, D = q.shape
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    qd, kd, vd = to_dev(q, W.BF16), to_dev(kp, W.BF16), to_dev(vp, W.BF16)
    sl, ns, bt = dev(np.asarray(seqlens, np.int32)), dev(np.asarray(nsplits, np.int32)), dev(table)
    sd = torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    op = torch.full((B, Hq, max_splits, D), float("nan"), device="cuda")
    lp = torch.full((B, Hq, max_splits), float("nan"), device="cuda")
    out = torch.empty((B, Hq, 1, D), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    A.attn_decode_splitkv_paged(qd, kd, vd, bt, sl, ns, op, lp, window=window, scale=scale)
    A.attn_combine(op, lp, sl, ns, sd, out, lse, Lk_max=table.shape[1] * kp.shape[2], window=window)
    torch.cuda.synchronize()
    return op.cpu().numpy(), lp.cpu().numpy(), out[:, :, 0].cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("page_size", [1, 8, 16, 64, 256, 1024])
@pytest.mark.parametrize("window", [0, 513])
def test_paged_decode(gpu, page_size, window):
    w = W.SPLITKV_DECODE
    q, kc, vc, seqlens, ns, s = W.decode_inputs(w, B=12, Lk_max=4096, random_splits=True)
    seqlens[:4] = [1, 63, 64, 65]  # shorter than generated: rows past Lk stay NaN
    say(f"paged decode page_size={page_size} window={window}")
    kp, table = page_cache(kc, seqlens, page_size, seed=page_size, junk_slots=page_size == 64)
    vp, _ = page_cache(vc, seqlens, page_size, seed=page_size, junk_slots=page_size == 64)
    scale = w.D ** -0.5
    op, lp, o, l = run_paged(q, kp, vp, table, seqlens, ns, s, window, scale)
    # the dense decode on the same splits: the same sums in the same order (the
    # two kernels may contract multiply-adds differently, so not bit for bit)
    op_d, lp_d, o_d, l_d = run_decode(q, kc, vc, seqlens, ns, s, window, scale)
    d_o, d_l = np.abs(o - o_d).max(), np.abs(l - l_d).max()
    say(f"  paged vs dense: max|dO| {d_o:.3e} max|dLSE| {d_l:.3e}")
    assert d_o <= 1e-5 and d_l <= 1e-5, "paged and dense decode disagree"
    assert np.array_equal(np.isnan(op), np.isnan(op_d)), "different partial lanes written"
    Lk_max = table.shape[1] * page_size
    o_r, l_r = oracle.decode_paged(host_values(q, W.BF16), host_values(kp, W.BF16),
                                   host_values(vp, W.BF16), table, seqlens, s, window, scale,
                                   page_size, Lk_max)
    compare(o, l, o_r, l_r, f"paged decode ps={page_size} W={window}")


def test_paged_decode_auto_plan_full_split_range(gpu):
    """Long sequences on small pages: every split crosses many pages."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, D, Lk_max, ps = 3, 16, 2, 128, 20000, 16
    seqlens = np.array([20000, 7777, 129])
    bits = lambda shape: W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    q, kc, vc = bits((B, Hq, 1, D)), bits((B, Hkv, Lk_max, D)), bits((B, Hkv, Lk_max, D))
    sinks = rng.standard_normal(Hq).astype(np.float32)
    kp, table = page_cache(kc, seqlens, ps, seed=1)
    vp, _ = page_cache(vc, seqlens, ps, seed=1)
    for nsp in ([64, 64, 64], [1, 3, 2]):
        _, _, o, l = run_paged(q, kp, vp, table, seqlens, nsp, sinks, 0, D ** -0.5)
        o_r, l_r = oracle.decode_paged(host_values(q, W.BF16), host_values(kp, W.BF16),
                                       host_values(vp, W.BF16), table, seqlens, sinks, 0,
                                       D ** -0.5, ps, table.shape[1] * ps)
        compare(o, l, o_r, l_r, f"paged long ns={nsp}")


def pack(x_bits, lens):
    """[B,H,Lmax,D] -> [H,sum(lens),D] keeping each sequence's first lens[b] rows."""
    return np.ascontiguousarray(np.concatenate([x_bits[b, :, :L] for b, L in enumerate(lens)], axis=1))


def run_varlen(q, k, v, cu_q, cu_k, sinks, window, scale, max_q, out_f32=True):
    qd, kd, vd = to_dev(q, W.BF16), to_dev(k, W.BF16), to_dev(v, W.BF16)
    cq = torch.from_numpy(np.asarray(cu_q, np.int32)).cuda()
    ck = torch.from_numpy(np.asarray(cu_k, np.int32)).cuda()
    sd = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    out = torch.full(qd.shape, float("nan"), dtype=torch.float32 if out_f32 else torch.bfloat16,
                     device="cuda")
    lse = torch.full(qd.shape[:2], float("nan"), device="cuda")
    A.attn_fwd_varlen(qd, kd, vd, cq, ck, sd, out, lse, max_seqlen_q=max_q, window=window,
                      scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", ["self", "chunked", "edges"])
@pytest.mark.parametrize("D,Hq,Hkv,window", [(128, 64, 8, 513), (64, 8, 2, 0), (128, 4, 4, 100)])
def test_varlen_prefill(gpu, case, D, Hq, Hkv, window):
    rng = np.random.default_rng(D + Hq + len(case))
    if case == "self":
        lq = [1000, 1, 64, 700, 129, 333]
        lk = lq
    elif case == "chunked":   # new chunk of a longer context
        lq = [100, 257, 1, 64]
        lk = [600, 257, 900, 1064]
    else:                     # empty sequences, keys shorter than queries, no keys
        lq = [5, 0, 70, 33, 1]
        lk = [5, 3, 20, 0, 1]
    B = len(lq)
    Lmax_q, Lmax_k = max(lq), max(max(lk), 1)
    bits = lambda shape: W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    qb, kb, vb = bits((B, Hq, Lmax_q, D)), bits((B, Hkv, Lmax_k, D)), bits((B, Hkv, Lmax_k, D))
    q, k, v = pack(qb, lq), pack(kb, lk), pack(vb, lk)
    if k.shape[1] == 0:
        k = v = np.zeros((Hkv, 0, D), np.uint16)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    sinks = (rng.standard_normal(Hq) * 2).astype(np.float32)
    sinks[::8] = 20.0
    say(f"varlen {case} D={D} H={Hq}/{Hkv} W={window}")
    o, l = run_varlen(q, k, v, cu_q, cu_k, sinks, window, D ** -0.5, max(Lmax_q, 1))
    o_r, l_r = oracle.attention_fwd_varlen(host_values(q, W.BF16), host_values(k, W.BF16),
                                           host_values(v, W.BF16), cu_q, cu_k, sinks, window,
                                           D ** -0.5)
    compare(o, l, o_r, l_r, f"varlen {case}")
    # the dense forward of each sequence alone
    for b in range(B):
        if lq[b] == 0 or lq[b] > lk[b]:
            continue
        qd = to_dev(qb[b:b + 1, :, :lq[b]], W.BF16)
        kd, vd = to_dev(kb[b:b + 1, :, :lk[b]], W.BF16), to_dev(vb[b:b + 1, :, :lk[b]], W.BF16)
        out = torch.empty(qd.shape, device="cuda")
        lse = torch.empty(qd.shape[:3], device="cuda")
        A.attn_fwd(qd, kd, vd, torch.from_numpy(sinks).cuda(), out, lse, window=window,
                   scale=D ** -0.5)
        torch.cuda.synchronize()
        d_o = np.abs(out[0].cpu().numpy() - o[:, cu_q[b]:cu_q[b + 1]]).max()
        d_l = np.abs(lse[0].cpu().numpy() - l[:, cu_q[b]:cu_q[b + 1]]).max()
        assert d_o <= 1e-5 and d_l <= 1e-5, f"b={b}: varlen vs dense {d_o:.3e} {d_l:.3e}"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("page_size", [16, 256])
def test_paged_decode_full_size(gpu, page_size):
    """The benchmark's serving layout: the full split-KV decode cache (B64 Hq64
    Hkv8 D128, 1.0M cached keys) in shuffled pages of 16 or 256 keys, built on
    the device; paged decode + combine against the dense decode + combine on
    the same splits (the dense path is checked against the oracle at this
    size elsewhere), and two sequences against the oracle directly."""
    w = W.SPLITKV_DECODE
    q, kc, vc, seqlens, ns, s = full_decode_inputs()
    B, Hkv, Lk_max, D = kc.shape
    P = page_size
    mp = Lk_max // P
    need = [-(-int(L) // P) for L in seqlens]
    total = sum(need)
    perm = np.random.default_rng(P).permutation(total)
    table = np.full((B, mp), 1 << 30, dtype=np.int32)  # unused slots: never read
    src = np.empty(total, dtype=np.int64)
    i = 0
    for b in range(B):
        for p in range(need[b]):
            table[b, p] = perm[i]
            src[perm[i]] = b * mp + p
            i += 1
    say(f"paged decode full size, {P}-key pages: building {total} pages")
    qd = to_dev(q, W.BF16)
    sl = torch.from_numpy(np.asarray(seqlens, np.int32)).cuda()
    nsd = torch.from_numpy(np.asarray(ns, np.int32)).cuda()
    sd = torch.from_numpy(np.asarray(s, np.float32)).cuda()
    bt = torch.from_numpy(table).cuda()
    idx = torch.from_numpy(src).cuda()
    outs = {}
    for layout in ("dense", "paged"):
        kd, vd = to_dev(kc, W.BF16), to_dev(vc, W.BF16)
        if layout == "paged":
            page = lambda x: x.view(B, Hkv, mp, P, D).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, P, D)[idx].contiguous()
            kd, vd = page(kd), page(vd)
        op = torch.full((B, w.Hq, 64, D), float("nan"), device="cuda")
        lp = torch.full((B, w.Hq, 64), float("nan"), device="cuda")
        out = torch.empty((B, w.Hq, 1, D), device="cuda")
        lse = torch.empty((B, w.Hq), device="cuda")
        if layout == "paged":
            A.attn_decode_splitkv_paged(qd, kd, vd, bt, sl, nsd, op, lp, window=0, scale=w.scale)
        else:
            A.attn_decode_splitkv(qd, kd, vd, sl, nsd, op, lp, window=0, scale=w.scale)
        A.attn_combine(op, lp, sl, nsd, sd, out, lse, Lk_max=Lk_max, window=0)
        torch.cuda.synchronize()
        outs[layout] = (out[:, :, 0].cpu().numpy(), lse.cpu().numpy(), np.isnan(op.cpu().numpy()))
        del kd, vd, op, lp, out, lse
        torch.cuda.empty_cache()
    o, l, nan_p = outs["paged"]
    o_d, l_d, nan_d = outs["dense"]
    d_o, d_l = np.abs(o - o_d).max(), np.abs(l - l_d).max()
    say(f"  paged vs dense: max|dO| {d_o:.3e} max|dLSE| {d_l:.3e}")
    assert d_o <= 1e-5 and d_l <= 1e-5, "paged and dense decode disagree"
    assert np.array_equal(nan_p, nan_d), "different partial lanes written"
    picks = [int(np.argmax(seqlens)), 7]
    o_r, l_r = oracle.decode(host_values(q[picks], W.BF16), host_values(kc[picks], W.BF16),
                             host_values(vc[picks], W.BF16), seqlens[picks], s, 0, w.scale)
    compare(o[picks], l[picks], o_r, l_r, f"paged decode full size ps={P}")


@pytest.mark.timeout(900)
def test_varlen_prefill_bench_size(gpu):
    """The benchmark's packed batch: 8 sequences of U{1024..8192} rows (the same
    draw), Hq64 Hkv8 D128, window 513, no sinks, bf16 O.  Every sequence against
    the dense forward on it alone, and sampled 64-row blocks against the oracle
    on the slice of keys that decides them."""
    Hq, Hkv, D, window = 64, 8, 128, 513
    lens = np.random.default_rng(11).integers(1024, 8193, 8)
    rng = np.random.default_rng(12)
    tot = int(lens.sum())
    bits = lambda shape: W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    q, k, v = bits((Hq, tot, D)), bits((Hkv, tot, D)), bits((Hkv, tot, D))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    scale = D ** -0.5
    say(f"varlen bench size: {tot} rows")
    o, l = run_varlen(q, k, v, cu, cu, None, window, scale, int(lens.max()), out_f32=False)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    for b in range(len(lens)):
        a, e = int(cu[b]), int(cu[b + 1])
        qd = to_dev(q[None, :, a:e], W.BF16)
        kd, vd = to_dev(k[None, :, a:e], W.BF16), to_dev(v[None, :, a:e], W.BF16)
        out = torch.empty(qd.shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(qd.shape[:3], device="cuda")
        A.attn_fwd(qd, kd, vd, None, out, lse, window=window, scale=scale)
        torch.cuda.synchronize()
        d_o = np.abs(out[0].float().cpu().numpy() - o[:, a:e]).max()
        d_l = np.abs(lse[0].cpu().numpy() - l[:, a:e]).max()
        assert d_o <= 1e-5 and d_l <= 1e-5, f"b={b}: varlen vs dense {d_o:.3e} {d_l:.3e}"
    for b, h, r0 in ((0, 3, 0), (3, 17, 700), (7, 63, int(lens[7]) - 64)):
        a = int(cu[b])
        k0 = max(0, r0 - window + 1)
        sl = lambda x, hh, lo, hi: host_values(x[None, hh:hh + 1, a + lo:a + hi], W.BF16)
        o_r, l_r = oracle.attention_fwd(sl(q, h, r0, r0 + 64), sl(k, h // (Hq // Hkv), k0, r0 + 64),
                                        sl(v, h // (Hq // Hkv), k0, r0 + 64), None, window, scale)
        compare(o[h, a + r0:a + r0 + 64], l[h, a + r0:a + r0 + 64], o_r[0, 0], l_r[0, 0],
                f"varlen bench size b={b} h={h} rows {r0}..", bf16_out=True)
