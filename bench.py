"""Benchmark of the exact-attention hot path on one MI355X.

One step = the whole path on resident synthetic inputs:
  attn_fwd            long-context sliding-window prefill  B1 Hq64 Hkv8 L262144 D128 bf16,
                      window 513, sinks (heads h%4==0 at +30), O written in bf16
  attn_decode_splitkv split-KV decode  B64 Hq64 Hkv8 D128 bf16, Lk ~ U{1024..32768},
                      num_splits = clamp(ceil(Lk/1024), 1, 64)
  attn_combine        merge of the valid splits, sink added once

Prints one JSON line.  `value` is the step's prefill TFLOP/s (algorithmic
flops: 4*D per unmasked pair) from HIP events around each attn_fwd launch on
the stream it runs on; decode GB/s (algorithmic bytes: the K/V rows each
query sees plus q, O and LSE) is reported beside it.  The two smaller prefill
workloads (sliding-window B1 L8192, causal B4 L4096) are timed in loops of
their own after the step, each with its roofline fraction.  The float64 CPU
oracle is timed on a bounded sample of each prefill workload and of the
decode on the host cores.

Before the counted warm-up steps the step runs for a fixed amount of GPU time
(--prewarm-ms, default 250 ms): after an idle spell the first ~20 ms of load
run up to a quarter slower, and a handful of warm-up steps of a small
workload would not cover that.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def _code_only(text: str) -> str:
    """C++ source without comments and blank space (string literals are kept as they are)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


# The sources each profiled kernel is built from (its own file and the headers
# it includes); a change elsewhere leaves its stored counters valid.
KERNEL_SOURCES = {
    "fwd_bf16_kernel": ("attn_fwd.hip", "attn_common.hpp", "attn_tiles.hpp", "attn_kernels.hpp"),
    "decode_kernel": ("attn_decode.hip", "attn_common.hpp", "attn_kernels.hpp"),
    "combine_kernel": ("attn_decode.hip", "attn_common.hpp", "attn_kernels.hpp"),
}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code (comments ignored) of the sources that build `kernel`
    (a name of KERNEL_SOURCES, template arguments and workload allowed after
    it), plus their compile flags; stored counters are used only while it
    matches."""
    from exact_attention_attn_amd import build as B
    base = kernel.split("<")[0].split(":")[0]
    files = KERNEL_SOURCES[base]
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_attn_amd", "csrc")
    for name in files:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    flags = [B.SOURCE_FLAGS.get(n, []) for n in files]
    h.update(repr((B.DEVICE_FLAGS, flags)).encode())
    return h.hexdigest()[:16]


def stored_profile(kernel: str) -> dict:
    """What rocprofv3 counters measured for this kernel and workload with the current
    sources (HBM bytes per launch, sustained clock), or {} when they no longer apply."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
        return {}
    return ent


def stored_traffic(kernel: str):
    """HBM bytes per launch measured with rocprofv3 counters for the current sources, or None."""
    return stored_profile(kernel).get("bytes_per_launch")


def decode_bytes(seqlens, Hq, Hkv, D, window) -> int:
    lk = np.asarray(seqlens, np.int64)
    if window > 0:
        lk = np.minimum(lk, window)
    kv = int(lk.sum()) * Hkv * D * 2 * 2
    B = len(seqlens)
    return kv + B * Hq * D * 2 + B * Hq * D * 2 + B * Hq * 4 + Hq * 4


def prewarm(torch, stream, fn, warm_s):
    """Run fn on stream until at least warm_s seconds of GPU time have passed;
    return (GPU seconds spent, calls)."""
    spent, calls = 0.0, 0
    with torch.cuda.stream(stream):
        while spent < warm_s:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            spent += e0.elapsed_time(e1) * 1e-3
            calls += 5
    return spent, calls


def warm_then_time(torch, stream, fn, reps, warm_s=0.04):
    """Seconds per call of fn on stream, averaged over reps calls, after running
    it until at least warm_s seconds of GPU time have passed (after an idle
    spell the first ~20 ms of work run up to a quarter slower)."""
    with torch.cuda.stream(stream):
        spent = 0.0
        while spent < warm_s:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            spent += e0.elapsed_time(e1) * 1e-3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def time_calls(torch, stream, fn, reps):
    """Seconds per call of fn over reps back-to-back calls on stream (events)."""
    with torch.cuda.stream(stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def measure_split_policies(A, torch, dev, stream, qd, kd, vd, sl, ds, op, lp, dout, dlse, wd,
                           seqlens, reps=10, rounds=7):
    """GB/s of decode + combine under several split-count policies.

    Rows: the decode workload of the step, and two synthetic mixes drawn on
    the device (4 sequences of 32768 keys; 256 sequences of 128..2048 keys).
    Every rule times decode + combine with the counts planned beforehand (a
    caller plans once per step and can reuse the plan while its lengths
    stand); 'auto+plan' also times the planning launch (attn_decode_plan)
    inside every call.  auto_vs_best_fixed = auto / the fastest fixed rule.
    Each policy is timed in `rounds` interleaved rounds of `reps` calls.
    """
    def setup(q_, k_, v_, sl_, Lk_max, policy, param, with_plan=False):
        """The policy's planned counts and one decode + combine call (plus the
        planning launch when with_plan)."""
        B, Hq = q_.shape[0], q_.shape[1]
        ns = torch.empty(B, dtype=torch.int32, device=dev)
        plan = lambda: A.attn_decode_plan(sl_, ns, Hq=Hq, Hkv=k_.shape[1], Lk_max=Lk_max,
                                          policy=policy, param=param, stream=stream)
        if B == op.shape[0]:
            o_, l_, out_, lse_ = op, lp, dout, dlse
        else:
            o_ = torch.empty((B,) + tuple(op.shape[1:]), dtype=op.dtype, device=dev)
            l_ = torch.empty((B,) + tuple(lp.shape[1:]), dtype=lp.dtype, device=dev)
            out_ = torch.empty((B,) + tuple(dout.shape[1:]), dtype=dout.dtype, device=dev)
            lse_ = torch.empty((B,) + tuple(dlse.shape[1:]), dtype=dlse.dtype, device=dev)

        def once():
            if with_plan:
                plan()
            A.attn_decode_splitkv(q_, k_, v_, sl_, ns, o_, l_, window=0, scale=wd.scale,
                                  stream=stream)
            A.attn_combine(o_, l_, sl_, ns, ds, out_, lse_, Lk_max=Lk_max, window=0,
                           stream=stream)
        with torch.cuda.stream(stream):
            plan()
        label = f"{policy}({param})" if policy != "auto" else ("auto+plan" if with_plan else "auto")
        return label, ns, once

    rows = []
    Hq, Hkv, D = wd.Hq, wd.Hkv, wd.D
    mixes = [("splitkv_decode", qd, kd, vd, sl, wd.Lk_max, np.asarray(seqlens))]
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    for name, lens, Lk_max in (("B4 Lk32768", np.full(4, 32768), 32768),
                               ("B256 Lk128-2048", np.random.default_rng(7).integers(128, 2049, 256), 2048)):
        B = len(lens)
        q_ = torch.randn(B, Hq, 1, D, device=dev, generator=g).to(torch.bfloat16)
        k_ = torch.randn(B, Hkv, Lk_max, D, device=dev, generator=g).to(torch.bfloat16)
        v_ = torch.randn(B, Hkv, Lk_max, D, device=dev, generator=g).to(torch.bfloat16)
        mixes.append((name, q_, k_, v_, torch.from_numpy(lens.astype(np.int32)).to(dev), Lk_max, lens))
    for name, q_, k_, v_, sl_, Lk_max, lens in mixes:
        nbytes = decode_bytes(lens, Hq, Hkv, D, 0)
        cases = [setup(q_, k_, v_, sl_, Lk_max, pol, par)
                 for pol, par in (("auto", 0), ("keys", 1024), ("keys", 512), ("count", 1))]
        cases.append(setup(q_, k_, v_, sl_, Lk_max, "auto", 0, with_plan=True))
        # The policies alternate within each round (the starting one rotates), so a
        # slow drift of the clock touches all of them alike; the median per policy
        # over the rounds is reported.
        warm_then_time(torch, stream, lambda: [c[2]() for c in cases], 1)
        per = [[] for _ in cases]
        for r in range(rounds):
            for j in range(len(cases)):
                i = (j + r) % len(cases)
                per[i].append(time_calls(torch, stream, cases[i][2], reps))
        res = []
        for (label, ns, _), ts in zip(cases, per):
            ms = float(np.median(ts)) * 1e3
            res.append({"policy": label, "us": round(ms * 1e3, 1),
                        "GB/s": round(nbytes / ms / 1e6, 1), "total_splits": int(ns.sum().item())})
        best_fixed = min(r["us"] for r in res if not r["policy"].startswith("auto"))
        rows.append({"workload": name, "results": res,
                     "auto_vs_best_fixed": round(res[0]["us"] / best_fixed, 4),
                     "auto+plan_vs_best_fixed": round(res[-1]["us"] / best_fixed, 4)})
    return rows


def measure_backward(A, torch, dev, stream, q, k, v, s, wp, reps=10):
    """attn_bwd on a prefill workload's inputs: dQ, dK, dV and dsink for a
    seeded dO, given the bf16 O that the forward writes in the step.

    Algorithmic work is the five products of the backward (S, dP, dV, dK, dQ:
    10*D flops per unmasked pair, 2.5x the forward); the two phases both
    compute S and dP, so the kernels execute 14*D per pair.
    """
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dout = torch.randn(q.shape, device=dev, generator=g).to(torch.bfloat16)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(k.shape, dtype=torch.float32, device=dev)
    ds = torch.empty(s.shape, dtype=torch.float32, device=dev)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    with torch.cuda.stream(stream):
        A.attn_fwd(q, k, v, s, o, lse, window=wp.window, scale=wp.scale, stream=stream)
    run = lambda: A.attn_bwd(q, k, v, s, o, dout, lse, dq, dk, dv, ds, delta, window=wp.window,
                             scale=wp.scale, stream=stream)
    t = warm_then_time(torch, stream, run, reps)
    pairs = wp.flops() // (4 * wp.D)
    return {"entry": "attn_bwd (dQ, dK, dV, dsink), bf16 O", "workload": wp.name,
            "ms": round(t * 1e3, 4),
            "TFLOP/s": round(10 * wp.D * pairs / t / 1e12, 2),
            "frac": round(10 * wp.D * pairs / t / 1e12 / PEAK_BF16_TFLOPS, 4),
            "executed_TFLOP/s": round(14 * wp.D * pairs / t / 1e12, 2),
            "note": "TFLOP/s counts the 5 backward products (10*D per pair); both phases "
                    "compute S and dP (14*D per pair executed)"}


def combine_bytes(seqlens, nsplits, Hq, D, window, max_splits=64) -> int:
    """Bytes the combine must move: the valid splits' partial O rows (fp32) and
    LSEs, read, plus the bf16 O and fp32 LSE written.  The valid split count of
    a sequence follows the split rule of include/attn.h: per = ceil(n / ns),
    chunk = per rounded up to 64 keys, n_valid = ceil(n / chunk)."""
    total = 0
    for n, ns in zip(np.asarray(seqlens, np.int64), np.asarray(nsplits, np.int64)):
        n = min(int(n), window) if window > 0 else int(n)
        ns = min(max(int(ns), 1), max_splits)
        if n <= 0:
            continue
        per = -(-n // ns)
        chunk = -(-per // 64) * 64
        total += -(-n // chunk)
    B = len(seqlens)
    return total * Hq * (D + 1) * 4 + B * Hq * D * 2 + B * Hq * 4


def pairs_window(L: int, W: int) -> int:
    """Unmasked (query, key) pairs of one head: sum_i min(i + 1, W) (W <= 0: causal)."""
    if W <= 0 or W >= L:
        return L * (L + 1) // 2
    return W * (W + 1) // 2 + (L - W) * W


def measure_serving(A, torch, dev, stream, qd, kd, vd, sl, ns, op, lp, dout, dlse, ds, wd, seqlens,
                    dense_s, wp, reps=20):
    """Paged decode (pages shuffled) against the dense decode on the same cache,
    and the varlen forward on a packed batch, each timed with events on stream."""
    def timeit(fn):
        return warm_then_time(torch, stream, fn, reps)

    res = {"paged_decode": [], "varlen_prefill": None}
    nbytes = decode_bytes(seqlens, wd.Hq, wd.Hkv, wd.D, wd.window)
    res["paged_decode"].append({"layout": "dense", "us": round(dense_s * 1e6, 1),
                                "GB/s": round(nbytes / dense_s / 1e9, 1)})
    B, Hkv, Lk_max, D = kd.shape
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    for ps in (16, 256):
        npp = Lk_max // ps
        perm = torch.randperm(B * npp, device=dev, generator=g)
        inv = torch.empty_like(perm)
        inv[perm] = torch.arange(B * npp, device=dev)
        table = inv.view(B, npp).to(torch.int32).contiguous()   # page of (b, slot)

        def paged(x):
            ordered = x.view(B, Hkv, npp, ps, D).permute(0, 2, 1, 3, 4).reshape(B * npp, Hkv, ps, D)
            return ordered[perm].contiguous()
        kp, vp = paged(kd), paged(vd)

        def step():
            A.attn_decode_splitkv_paged(qd, kp, vp, table, sl, ns, op, lp, window=wd.window,
                                        scale=wd.scale, stream=stream)
            A.attn_combine(op, lp, sl, ns, ds, dout, dlse, Lk_max=npp * ps, window=wd.window,
                           stream=stream)
        t = timeit(step)
        res["paged_decode"].append({"layout": f"paged {ps}", "us": round(t * 1e6, 1),
                                    "GB/s": round(nbytes / t / 1e9, 1)})
        del kp, vp
        torch.cuda.empty_cache()

    # packed batch: 8 sequences of U{1024..8192} rows, the sliding-window prefill's heads
    lens = np.random.default_rng(11).integers(1024, 8193, 8)
    tot = int(lens.sum())
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    q = torch.randn(wp.Hq, tot, wp.D, device=dev, generator=g).to(torch.bfloat16)
    k = torch.randn(wp.Hkv, tot, wp.D, device=dev, generator=g).to(torch.bfloat16)
    v = torch.randn(wp.Hkv, tot, wp.D, device=dev, generator=g).to(torch.bfloat16)
    out = torch.empty_like(q)
    lse = torch.empty(wp.Hq, tot, device=dev)
    t = timeit(lambda: A.attn_fwd_varlen(q, k, v, cu, cu, None, out, lse,
                                         max_seqlen_q=int(lens.max()), window=wp.window,
                                         scale=wp.scale, stream=stream))
    flops = 4 * wp.D * wp.Hq * sum(pairs_window(int(L), wp.window) for L in lens)
    res["varlen_prefill"] = {"workload": f"8 sequences, lengths {sorted(int(x) for x in lens)}, "
                                         f"Hq{wp.Hq} Hkv{wp.Hkv} D{wp.D} window{wp.window}",
                             "ms": round(t * 1e3, 4), "TFLOP/s": round(flops / t / 1e12, 2)}
    return res


def run_sweep(A, W, torch, dev):
    """One JSON line per shape: attn_fwd TFLOP/s over sequence lengths, windows
    and head dims, and split-KV decode + combine GB/s over batch/length mixes.
    Inputs are seeded N(0, 1) values rounded to bf16, generated on the device."""
    g = torch.Generator(device=dev)
    stream = torch.cuda.Stream(device=dev)

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device=dev).to(torch.bfloat16)

    for D in (128, 64):
        for L, B in ((1024, 8), (4096, 2), (16384, 1)):
            Hq, Hkv = 64, 8
            g.manual_seed(L + D)
            q, k, v = rnd(B, Hq, L, D), rnd(B, Hkv, L, D), rnd(B, Hkv, L, D)
            sk = torch.randn(Hq, generator=g, device=dev)
            out = torch.empty_like(q)
            lse = torch.empty(B, Hq, L, dtype=torch.float32, device=dev)
            for Wn in (0, 129, 513, 2049):
                if Wn >= L:
                    continue
                t = warm_then_time(torch, stream, lambda: A.attn_fwd(
                    q, k, v, sk, out, lse, window=Wn, scale=D ** -0.5, stream=stream), 20)
                fl = 4.0 * D * B * Hq * pairs_window(L, Wn)
                print(json.dumps({"sweep": "attn_fwd", "B": B, "Hq": Hq, "Hkv": Hkv, "L": L,
                                  "D": D, "window": Wn, "ms": round(t * 1e3, 4),
                                  "TFLOP/s": round(fl / t / 1e12, 1),
                                  "frac": round(fl / t / 2.5e15, 4)}), flush=True)
            del q, k, v, out, lse
            torch.cuda.empty_cache()
    for D in (128, 64):
        for B, lo, hi in ((8, 65536, 131072), (32, 8192, 32768), (128, 1024, 16384),
                          (256, 512, 4096)):
            Hq, Hkv, MS = 64, 8, 64
            rng = np.random.default_rng([B, lo, D])
            seqlens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
            nsplits = W.splits_policy(seqlens, 1024, MS)
            g.manual_seed(B + D)
            q, kc, vc = rnd(B, Hq, 1, D), rnd(B, Hkv, hi, D), rnd(B, Hkv, hi, D)
            sk = torch.randn(Hq, generator=g, device=dev)
            sl, ns = torch.from_numpy(seqlens).to(dev), torch.from_numpy(nsplits).to(dev)
            op = torch.empty(B, Hq, MS, D, dtype=torch.float32, device=dev)
            lp = torch.empty(B, Hq, MS, dtype=torch.float32, device=dev)
            out = torch.empty(B, Hq, 1, D, dtype=torch.bfloat16, device=dev)
            lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)

            def both():
                A.attn_decode_splitkv(q, kc, vc, sl, ns, op, lp, scale=D ** -0.5, stream=stream)
                A.attn_combine(op, lp, sl, ns, sk, out, lse, Lk_max=hi, stream=stream)
            t = warm_then_time(torch, stream, both, 10)
            nb = decode_bytes(seqlens, Hq, Hkv, D, 0)
            print(json.dumps({"sweep": "decode+combine", "B": B, "Hq": Hq, "Hkv": Hkv,
                              "Lk": [lo, hi], "sum_Lk": int(seqlens.sum()), "D": D,
                              "splits": int(nsplits.sum()), "ms": round(t * 1e3, 4),
                              "GB/s": round(nb / t / 1e9, 1), "frac": round(nb / t / 8e12, 4)}),
                  flush=True)
            del q, kc, vc, op, lp
            torch.cuda.empty_cache()


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max((p.get("num_threads", 1) for p in threadpool_info()), default=1))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(w, q, k, v, sinks, budget_s=10.0):
    """Time the float64 oracle on whole (batch, head) slices of a prefill
    workload, in a fixed spread order, until ~budget_s of work; the rate is in
    the same algorithmic flops as the GPU's."""
    import oracle
    from exact_attention_attn_amd import workloads as W

    G = w.Hq // w.Hkv
    per_head = w.flops() // (w.B * w.Hq)
    order = [(b, h) for h in range(w.Hq) for b in range(w.B)]
    done, flops, t0 = 0, 0, time.perf_counter()
    for b, h in order:
        kvh = h // G
        oracle.attention_fwd(W.as_float(q[b:b + 1, h:h + 1], w.dtype),
                             W.as_float(k[b:b + 1, kvh:kvh + 1], w.dtype),
                             W.as_float(v[b:b + 1, kvh:kvh + 1], w.dtype), sinks[h:h + 1],
                             w.window, w.scale)
        done += 1
        flops += per_head
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"{done} of {w.B * w.Hq} (batch, head) slices of {w.name} (all rows), "
                      f"float64 numpy, {dt:.1f} s"}


def cpu_baseline_decode(wd, q, kv, seqlens, nsplits, sinks, budget_s=8.0):
    """Time the float64 oracle's split-KV decode + combine on whole sequences
    (the first ones of the decode workload; kv[b] = their K, V rows) until
    ~budget_s of work; rate in the GPU path's algorithmic bytes (bf16 K/V rows
    + q + O + LSE)."""
    import oracle
    from exact_attention_attn_amd import workloads as W

    threads = _blas_threads()
    done, nbytes, t0 = 0, 0, time.perf_counter()
    for b in range(len(kv)):
        qb = W.as_float(q[b:b + 1], wd.dtype)
        kb = W.as_float(kv[b][0], wd.dtype)
        vb = W.as_float(kv[b][1], wd.dtype)
        o_p, l_p, n_valid = oracle.decode_partials(qb, kb, vb, seqlens[b:b + 1], nsplits[b:b + 1],
                                                   wd.window, wd.scale)
        oracle.combine(o_p, l_p, n_valid, sinks)
        done += 1
        nbytes += decode_bytes(seqlens[b:b + 1], wd.Hq, wd.Hkv, wd.D, wd.window)
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {q.shape[0]} sequences of {wd.name} "
                      f"(sum Lk {int(np.asarray(seqlens[:done], np.int64).sum())}), "
                      f"float64 numpy, {dt:.1f} s"}


def time_launches(torch, stream, fn, n, prewarm_s=0.05):
    """Per-launch seconds of fn on stream (HIP events around each launch),
    after at least prewarm_s seconds of GPU time of fn."""
    warm_then_time(torch, stream, fn, 1, warm_s=prewarm_s)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    with torch.cuda.stream(stream):
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e-3


def prefill_roofline(wp, t, traffic, host_us=None):
    """Roofline object of one prefill workload from per-launch seconds t.

    frac is against the published bf16 peak (2.5 PF at 2.4 GHz).  When the
    counter profile of these sources is stored, the sustained clock it measured
    under this kernel (active cycles over dispatch time) is reported beside it,
    with the fraction of the peak at that clock (context, not the bar)."""
    tflops = wp.flops() / t.mean() / 1e12
    clock = stored_profile("fwd_bf16_kernel<128,false,false,false>:" + wp.name).get("clock_ghz")
    r = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
         "kernel": "fwd_bf16_kernel<128,false,false,false>",
         "flops_per_launch": wp.flops(),
         "ms_per_launch": round(t.mean() * 1e3, 4),
         "ms_median": round(float(np.median(t)) * 1e3, 4),
         "ms_min": round(float(t.min()) * 1e3, 4),
         "frac_median": round(wp.flops() / float(np.median(t)) / 1e12 / PEAK_BF16_TFLOPS, 4),
         "launches": int(len(t)),
         "sustained_clock_ghz": clock,
         "frac_at_sustained_clock": (round(tflops / (PEAK_BF16_TFLOPS * clock / 2.4), 4)
                                     if clock else None)}
    if host_us is not None:
        r["host_us_per_call"] = round(host_us, 1)
    return r


def describe(wp):
    return (f"{wp.name} B{wp.B} Hq{wp.Hq} Hkv{wp.Hkv} L{wp.L} D{wp.D} "
            f"window{wp.window if wp.window > 0 else 'none'}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-ms", type=float, default=250.0,
                    help="GPU time of untimed steps before the counted warm-up steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the step (no prefill legs, split-policy, serving, backward or "
                         "max-logit extras); the profiled runs of the step use this")
    ap.add_argument("--prefill", default="long_swa_prefill",
                    help="prefill workload of the step (long_swa_prefill is the headline)")
    ap.add_argument("--legs", default="swa_prefill,causal_prefill",
                    help="prefill workloads timed in loops of their own after the step")
    ap.add_argument("--leg-launches", type=int, default=100)
    ap.add_argument("--keys-per-split", type=int, default=0,
                    help="decode split policy: num_splits = clamp(ceil(Lk / this), 1, 64); "
                         "0 keeps the workload's 1024")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(a known-size reference for HBM byte counters)")
    ap.add_argument("--extras", default="split_policy,serving,backward,max_logit",
                    help="extras timed after the legs, a comma list of split_policy, serving, "
                         "backward, max_logit (all by default); the profiled runs of the "
                         "backward kernels use backward alone")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: attn_fwd and decode rates over a range of shapes, "
                         "one JSON line each")
    args = ap.parse_args()
    want = set(x for x in args.extras.split(",") if x)
    unknown = want - {"split_policy", "serving", "backward", "max_logit"}
    if unknown:
        ap.error(f"unknown extras: {sorted(unknown)}")
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import exact_attention_attn_amd as A
    from exact_attention_attn_amd import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    A.load_library()
    dev = torch.device("cuda", 0)
    if args.sweep:
        run_sweep(A, W, torch, dev)
        return

    def up(x, dtype):
        if dtype == W.BF16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    def say(msg):
        print(msg, file=sys.stderr, flush=True)

    # prefill inputs of the step (host copies kept for the oracle's sample)
    wp = W.WORKLOADS[args.prefill]
    say(f"bench: generating {wp.name}")
    host = {}
    qh, kh, vh, sh = W.prefill_inputs(wp)
    host[wp.name] = (qh, kh, vh, sh)
    q, k, v = up(qh, wp.dtype), up(kh, wp.dtype), up(vh, wp.dtype)
    s = torch.from_numpy(sh).to(dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    # decode inputs
    say("bench: generating splitkv_decode")
    wd = W.SPLITKV_DECODE
    dq, dk, dv, seqlens, nsplits, dsinks = W.decode_inputs(wd)
    if args.keys_per_split > 0:
        nsplits = W.splits_policy(seqlens, args.keys_per_split)
    qd, kd, vd = up(dq, W.BF16), up(dk, W.BF16), up(dv, W.BF16)
    # the first sequences' rows, kept for the oracle's decode timing
    kv_host = [(dk[b:b + 1, :, :int(seqlens[b])].copy(), dv[b:b + 1, :, :int(seqlens[b])].copy())
               for b in range(16)] if not args.no_cpu_baseline else []
    del dk, dv
    sl = torch.from_numpy(seqlens).to(dev)
    ns = torch.from_numpy(nsplits).to(dev)
    ds = torch.from_numpy(dsinks).to(dev)
    MS = 64
    op = torch.empty((wd.B, wd.Hq, MS, wd.D), dtype=torch.float32, device=dev)
    lp = torch.empty((wd.B, wd.Hq, MS), dtype=torch.float32, device=dev)
    dout = torch.empty((wd.B, wd.Hq, 1, wd.D), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((wd.B, wd.Hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream(device=dev)

    def launch_step():
        A.attn_fwd(q, k, v, s, out, lse, window=wp.window, scale=wp.scale, stream=stream)
        A.attn_decode_splitkv(qd, kd, vd, sl, ns, op, lp, window=wd.window, scale=wd.scale,
                              stream=stream)
        A.attn_combine(op, lp, sl, ns, ds, dout, dlse, Lk_max=wd.Lk_max, window=wd.window,
                       stream=stream)

    # pre-warm: untimed steps until prewarm_ms of GPU time have passed
    say("bench: pre-warm")
    prewarm_s, prewarm_steps = prewarm(torch, stream, launch_step, args.prewarm_ms * 1e-3)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
          for _ in range(args.warmup + args.steps)]

    def step(i):
        e = ev[i]
        e[0].record(stream)
        A.attn_fwd(q, k, v, s, out, lse, window=wp.window, scale=wp.scale, stream=stream)
        e[1].record(stream)
        A.attn_decode_splitkv(qd, kd, vd, sl, ns, op, lp, window=wd.window, scale=wd.scale,
                              stream=stream)
        e[2].record(stream)
        A.attn_combine(op, lp, sl, ns, ds, dout, dlse, Lk_max=wd.Lk_max, window=wd.window,
                       stream=stream)
        e[3].record(stream)

    say("bench: timed steps")
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, args.warmup + args.steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    timed = ev[args.warmup:]
    t_fwd = np.array([e[0].elapsed_time(e[1]) for e in timed]) * 1e-3
    t_dec = np.array([e[1].elapsed_time(e[2]) for e in timed]) * 1e-3
    t_cmb = np.array([e[2].elapsed_time(e[3]) for e in timed]) * 1e-3

    # Host time per ABI call (argument checks, marshalling and the launch), the
    # calls left to run asynchronously.
    def host_us(fn, n=50):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        for _ in range(n):
            fn()
        h1 = time.perf_counter()
        torch.cuda.synchronize()
        return (h1 - h0) / n * 1e6
    with torch.cuda.stream(stream):
        host_fwd = host_us(lambda: A.attn_fwd(q, k, v, s, out, lse, window=wp.window,
                                              scale=wp.scale, stream=stream), n=10)
        host_dec = host_us(lambda: A.attn_decode_splitkv(qd, kd, vd, sl, ns, op, lp,
                                                         window=wd.window, scale=wd.scale,
                                                         stream=stream), n=10)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Prefill legs: the other prefill workloads, each in a loop of its own.
    legs = {}
    leg_inputs = {}
    if not args.step_only:
        for name in [x for x in args.legs.split(",") if x and x != wp.name]:
            wl = W.WORKLOADS[name]
            say(f"bench: leg {name}")
            qh2, kh2, vh2, sh2 = W.prefill_inputs(wl)
            host[name] = (qh2, kh2, vh2, sh2)
            ql, kl, vl = up(qh2, wl.dtype), up(kh2, wl.dtype), up(vh2, wl.dtype)
            sk = torch.from_numpy(sh2).to(dev)
            ol = torch.empty(ql.shape, dtype=torch.bfloat16, device=dev)
            ll = torch.empty(ql.shape[:3], dtype=torch.float32, device=dev)
            fn = (lambda ql=ql, kl=kl, vl=vl, sk=sk, ol=ol, ll=ll, wl=wl:
                  A.attn_fwd(ql, kl, vl, sk, ol, ll, window=wl.window, scale=wl.scale,
                             stream=stream))
            t = time_launches(torch, stream, fn, args.leg_launches)
            traffic = stored_traffic("fwd_bf16_kernel<128,false,false,false>:" + wl.name)
            legs[name] = {"workload": describe(wl),
                          "roofline": prefill_roofline(wl, t, traffic)}
            leg_inputs[name] = (wl, ql, kl, vl, sk)

    # Extras on the sliding-window prefill's inputs (B1 L8192): backward,
    # split-count policies, serving layouts, the max-logit output.
    extras = {}
    if not args.step_only and "swa_prefill" in leg_inputs:
        wl, ql, kl, vl, sk = leg_inputs["swa_prefill"]
        say("bench: extras")
        if "split_policy" in want:
            extras["split_policy"] = measure_split_policies(
                A, torch, dev, stream, qd, kd, vd, sl, ds, op, lp, dout, dlse, wd, seqlens)
        if "serving" in want:
            extras["serving"] = measure_serving(
                A, torch, dev, stream, qd, kd, vd, sl, ns, op, lp, dout, dlse, ds, wd, seqlens,
                t_dec.mean() + t_cmb.mean(), wl)
        if "backward" in want:
            extras["backward"] = measure_backward(A, torch, dev, stream, ql, kl, vl, sk, wl)
            if "causal_prefill" in leg_inputs:
                wc, qc, kc, vc, sc = leg_inputs["causal_prefill"]
                extras["backward_causal"] = measure_backward(A, torch, dev, stream, qc, kc, vc,
                                                             sc, wc)
    if not args.step_only and "swa_prefill" in leg_inputs and "max_logit" in want:
        wl, ql, kl, vl, sk = leg_inputs["swa_prefill"]
        ol = torch.empty(ql.shape, dtype=torch.bfloat16, device=dev)
        ll = torch.empty(ql.shape[:3], dtype=torch.float32, device=dev)
        ml_row = torch.empty(ll.shape, dtype=torch.float32, device=dev)
        ml_head = torch.empty(ll.shape[:2], dtype=torch.float32, device=dev)
        t_ml = time_launches(torch, stream, lambda: A.attn_fwd_max_logit(
            ql, kl, vl, sk, ol, ll, ml_row, ml_head, window=wl.window, scale=wl.scale,
            stream=stream), 50)
        t_ref = legs["swa_prefill"]["roofline"]["ms_per_launch"] * 1e-3
        extras["max_logit"] = {
            "entry": "attn_fwd_max_logit (row [B,Hq,Lq] and head [B,Hq] maxima), swa_prefill",
            "ms_per_launch": round(t_ml.mean() * 1e3, 4),
            "TFLOP/s": round(wl.flops() / t_ml.mean() / 1e12, 2),
            "time_vs_attn_fwd": round(t_ml.mean() / t_ref, 4),
        }

    flops = wp.flops()
    tflops = flops / t_fwd.mean() / 1e12
    dbytes = decode_bytes(seqlens, wd.Hq, wd.Hkv, wd.D, wd.window)
    comb_bytes = combine_bytes(seqlens, nsplits, wd.Hq, wd.D, wd.window)
    dec_gbps = dbytes / (t_dec.mean() + t_cmb.mean()) / 1e9
    traffic = stored_traffic("fwd_bf16_kernel<128,false,false,false>:" + wp.name)
    dec_traffic = stored_traffic("decode_kernel<128,false>:" + wd.name)
    dec_only = dbytes / t_dec.mean() / 1e9

    res = {
        "metric": "attn fwd TFLOP/s (% bf16 MFMA peak); decode GB/s (% HBM peak)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm": {"gpu_ms": round(prewarm_s * 1e3, 1), "steps": prewarm_steps},
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{describe(wp)} + {wd.name} B{wd.B} Hq{wd.Hq} Hkv{wd.Hkv} D{wd.D} "
                        f"Lk<={wd.Lk_max}",
            "prefill_flops": flops,
            "decode_bytes": dbytes,
            "decode_sum_Lk": int(np.asarray(seqlens, np.int64).sum()),
            "decode_keys_per_split": args.keys_per_split or wd.keys_per_split,
        },
        "roofline": prefill_roofline(wp, t_fwd, traffic, host_fwd),
        "decode": {
            "GB/s": round(dec_gbps, 1),
            "frac_hbm": round(dec_gbps / PEAK_HBM_GBPS, 4),
            "decode_ms": round(t_dec.mean() * 1e3, 4),
            "combine_ms": round(t_cmb.mean() * 1e3, 4),
            "combine_GB/s": round(comb_bytes / t_cmb.mean() / 1e9, 1),
            "combine_bytes": comb_bytes,
            "note": "GB/s = algorithmic bytes (visible K/V rows + q + O + LSE) / (decode + combine time); "
                    "combine_GB/s = (valid partial O rows and LSEs read + O and LSE written) / combine time",
        },
        "roofline_decode": {
            "bound": "hbm",
            "achieved": round(dec_only, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(dec_only / PEAK_HBM_GBPS, 4),
            "traffic": dec_traffic,
            "kernel": "decode_kernel<128,false>",
            "ms_per_launch": round(t_dec.mean() * 1e3, 4),
            "ms_median": round(float(np.median(t_dec)) * 1e3, 4),
            "ms_min": round(float(t_dec.min()) * 1e3, 4),
            "host_us_per_call": round(host_dec, 1),
        },
    }
    if legs:
        res["prefill_legs"] = legs
    res.update(extras)
    if not args.no_cpu_baseline:
        say("bench: oracle baselines")
        res["cpu_baseline"] = cpu_baseline(wp, *host[wp.name])
        for name, leg in legs.items():
            leg["cpu_baseline"] = cpu_baseline(W.WORKLOADS[name], *host[name])
        res["cpu_baseline_decode"] = cpu_baseline_decode(wd, dq, kv_host, seqlens, nsplits, dsinks)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
