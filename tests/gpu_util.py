"""Helpers of the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI (via the Python binding), and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import exact_attention_attn_amd as A
from exact_attention_attn_amd import workloads as W

# Parity bar for bf16 inputs with fp32 accumulation, output read in fp32.
TOL_MAX = 1e-2
TOL_MEAN = 1e-3
TOL_LSE = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == W.BF16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def host_values(arr: np.ndarray, dtype: str) -> np.ndarray:
    """The float32 values the GPU sees (for the oracle)."""
    return W.as_float(arr, dtype)


def run_fwd(q, k, v, sinks, dtype, window, scale, out_f32=True, rows=None):
    """Run attn_fwd on host arrays; return O (float32) and LSE, optionally only rows.

    rows: None (everything) or a list of (b, h, row_index_array) to gather on device.
    """
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    sd = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    out = torch.empty(qd.shape, dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    A.attn_fwd(qd, kd, vd, sd, out, lse, window=window, scale=scale)
    torch.cuda.synchronize()
    if rows is None:
        return out.float().cpu().numpy(), lse.cpu().numpy()
    res = []
    for b, h, r in rows:
        idx = torch.from_numpy(np.asarray(r, np.int64)).cuda()
        res.append((out[b, h].index_select(0, idx).float().cpu().numpy(),
                    lse[b, h].index_select(0, idx).cpu().numpy()))
    del qd, kd, vd, out, lse
    return res


def run_fwd_max_logit(q, k, v, sinks, dtype, window, scale, out_f32=True, want_row=True,
                      want_head=True):
    """Run attn_fwd_max_logit; return O, LSE, row maxima and head maxima (None if not asked)."""
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    sd = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    out = torch.empty(qd.shape, dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    mrow = torch.full(qd.shape[:3], float("nan"), device="cuda") if want_row else None
    # stale contents must not leak: the call resets the head maxima itself
    mhead = torch.full(qd.shape[:2], 1e30, device="cuda") if want_head else None
    A.attn_fwd_max_logit(qd, kd, vd, sd, out, lse, mrow, mhead, window=window, scale=scale)
    torch.cuda.synchronize()
    res = (out.float().cpu().numpy(), lse.cpu().numpy(),
           None if mrow is None else mrow.cpu().numpy(),
           None if mhead is None else mhead.cpu().numpy())
    del qd, kd, vd, out, lse, mrow, mhead
    return res


def compare(o, l, o_ref, l_ref, what: str, tol_max=TOL_MAX, tol_mean=TOL_MEAN, tol_lse=TOL_LSE,
            bf16_out=False):
    o = np.asarray(o, np.float64)
    l = np.asarray(l, np.float64)
    assert np.isfinite(o).all(), f"{what}: non-finite O"
    d = np.abs(o - o_ref)
    if bf16_out:
        # The bar is for O as accumulated in fp32.  Storing it in bf16 adds its
        # own rounding, up to half an ulp of |O| per element, to each element
        # and so to the mean as well: for peaked scores |O| is about |v| and
        # that rounding alone averages about 1e-3.
        mag = np.maximum(np.maximum(np.abs(o_ref), np.abs(o)), 1e-30)
        half_ulp = 0.5 * np.exp2(np.floor(np.log2(mag)) - 7)
        assert (d <= tol_max + half_ulp).all(), f"{what}: max|dO| {d.max():.3e} beyond bf16 bound"
        assert d.mean() <= tol_mean + half_ulp.mean(), (
            f"{what}: mean|dO| = {d.mean():.3e} beyond {tol_mean} + bf16 rounding {half_ulp.mean():.3e}")
    else:
        assert d.max() <= tol_max, f"{what}: max|dO| = {d.max():.3e}"
        assert d.mean() <= tol_mean, f"{what}: mean|dO| = {d.mean():.3e}"
    both_inf = np.isneginf(l) & np.isneginf(l_ref)
    with np.errstate(invalid="ignore"):  # -inf - -inf where both rows see nothing
        dl = np.abs(np.where(both_inf, 0.0, l - l_ref))
    assert np.isfinite(dl).all() and dl.max() <= tol_lse, f"{what}: max|dLSE| = {dl.max():.3e}"
    return d.max(), d.mean(), dl.max()


def run_decode(q, kc, vc, seqlens, nsplits, sinks, window, scale, max_splits=64, out_f32=True,
               poison=True):
    """attn_decode_splitkv + attn_combine; returns partials (host) and O, LSE."""
    qd, kd, vd = to_dev(q, W.BF16), to_dev(kc, W.BF16), to_dev(vc, W.BF16)
    B, Hq, _, D = q.shape
    sl = torch.from_numpy(np.asarray(seqlens, np.int32)).cuda()
    ns = torch.from_numpy(np.asarray(nsplits, np.int32)).cuda()
    sd = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    fill = float("nan") if poison else 0.0
    op = torch.full((B, Hq, max_splits, D), fill, dtype=torch.float32, device="cuda")
    lp = torch.full((B, Hq, max_splits), fill, dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, 1, D), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    A.attn_decode_splitkv(qd, kd, vd, sl, ns, op, lp, window=window, scale=scale)
    A.attn_combine(op, lp, sl, ns, sd, out, lse, Lk_max=kc.shape[2], window=window)
    torch.cuda.synchronize()
    return (op.cpu().numpy(), lp.cpu().numpy(), out[:, :, 0].float().cpu().numpy(),
            lse.cpu().numpy())


def run_decode_repeated(q, kc, vc, seqlens, nsplits, sinks, window, scale, repeats=5,
                        max_splits=64):
    """attn_decode_splitkv + attn_combine `repeats` times on the same device
    inputs, buffers re-poisoned with NaN before each run; host copies of
    (partials O, partials LSE, O, LSE) per run."""
    qd, kd, vd = to_dev(q, W.BF16), to_dev(kc, W.BF16), to_dev(vc, W.BF16)
    B, Hq, _, D = q.shape
    sl = torch.from_numpy(np.asarray(seqlens, np.int32)).cuda()
    ns = torch.from_numpy(np.asarray(nsplits, np.int32)).cuda()
    sd = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    op = torch.empty((B, Hq, max_splits, D), dtype=torch.float32, device="cuda")
    lp = torch.empty((B, Hq, max_splits), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, 1, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    res = []
    for _ in range(repeats):
        op.fill_(float("nan"))
        lp.fill_(float("nan"))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        A.attn_decode_splitkv(qd, kd, vd, sl, ns, op, lp, window=window, scale=scale)
        A.attn_combine(op, lp, sl, ns, sd, out, lse, Lk_max=kc.shape[2], window=window)
        torch.cuda.synchronize()
        res.append((op.cpu().numpy(), lp.cpu().numpy(), out[:, :, 0].cpu().numpy(),
                    lse.cpu().numpy()))
    del qd, kd, vd, op, lp, out, lse
    return res


_FULL_DECODE = {}


def full_decode_inputs():
    """The split-KV decode workload at full size (host arrays, generated once per
    test session and shared by the test modules that use it)."""
    if not _FULL_DECODE:
        say("splitkv_decode full size: generating inputs")
        _FULL_DECODE["x"] = W.decode_inputs(W.SPLITKV_DECODE)
    return _FULL_DECODE["x"]
