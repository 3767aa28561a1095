"""GPU parity of attn_bwd (dQ, dK, dV, dsink) against the float64 oracle.

The kernels take O and LSE from attn_fwd (O in fp32), round P and dS to bf16
for the MFMAs and sum in fp32.  Bar, per gradient tensor X:
max|dX| <= TOL_MAX * max|X_ref| and mean|dX| <= TOL_MEAN * mean|X_ref|;
dsink: |d| <= TOL_SINK * max(1, |ref|).  The bound is derived from the bf16
rounding of P and dS in the tolerance section of the design notes.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_attention_attn_amd as A
import oracle
from exact_attention_attn_amd import workloads as W

gpu_util = pytest.importorskip("gpu_util")
from gpu_util import host_values, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN, TOL_SINK = 2e-2, 5e-3, 1e-4


def run_bwd(q, k, v, sinks, dout, window, scale, o_f32=True):
    qd, kd, vd, gd = (to_dev(x, W.BF16) for x in (q, k, v, dout))
    sd = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    out = torch.empty(qd.shape, dtype=torch.float32 if o_f32 else torch.bfloat16, device="cuda")
    lse = torch.empty(qd.shape[:3], device="cuda")
    A.attn_fwd(qd, kd, vd, sd, out, lse, window=window, scale=scale)
    dq = torch.full(qd.shape, float("nan"), device="cuda")
    dk = torch.full(kd.shape, float("nan"), device="cuda")
    dv = torch.full(kd.shape, float("nan"), device="cuda")
    ds = None if sd is None else torch.full(sd.shape, float("nan"), device="cuda")
    A.attn_bwd(qd, kd, vd, sd, out, gd, lse, dq, dk, dv, ds, window=window, scale=scale)
    torch.cuda.synchronize()
    res = [x.cpu().numpy() for x in (dq, dk, dv)] + [None if ds is None else ds.cpu().numpy()]
    del qd, kd, vd, gd, out, lse, dq, dk, dv, ds
    return res


def check_bwd(got, want, what):
    names = ("dq", "dk", "dv")
    for n, g, w in zip(names, got[:3], want[:3]):
        assert np.isfinite(g).all(), f"{what}: non-finite {n}"
        d = np.abs(g - w)
        rel_max = d.max() / max(np.abs(w).max(), 1e-30)
        rel_mean = d.mean() / max(np.abs(w).mean(), 1e-30)
        say(f"  {what} {n}: max {rel_max:.2e} mean {rel_mean:.2e} (relative)")
        assert rel_max <= TOL_MAX, f"{what}: {n} max rel {rel_max:.3e}"
        assert rel_mean <= TOL_MEAN, f"{what}: {n} mean rel {rel_mean:.3e}"
    if want[3] is not None and got[3] is not None:
        d = np.abs(got[3] - want[3]) / np.maximum(1.0, np.abs(want[3]))
        say(f"  {what} dsink: {d.max():.2e}")
        assert d.max() <= TOL_SINK, f"{what}: dsink {d.max():.3e}"


def inputs(rng, B, Hq, Hkv, Lq, Lk, D, sink_std=1.0):
    bits = lambda shape: W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    q, k, v, dout = bits((B, Hq, Lq, D)), bits((B, Hkv, Lk, D)), bits((B, Hkv, Lk, D)), bits((B, Hq, Lq, D))
    sinks = (rng.standard_normal(Hq) * sink_std).astype(np.float32)
    return q, k, v, dout, sinks


def oracle_bwd(q, k, v, sinks, dout, window, scale):
    return oracle.attention_bwd(host_values(q, W.BF16), host_values(k, W.BF16),
                                host_values(v, W.BF16), sinks, host_values(dout, W.BF16),
                                window, scale)


@pytest.mark.parametrize("o_f32", [True, False])
@pytest.mark.parametrize("name,L", [("swa_prefill", 700), ("causal_prefill", 400),
                                    ("long_swa_prefill", 900)])
def test_bwd_workload_reduced(gpu, name, L, o_f32):
    w = W.WORKLOADS[name]
    q, k, v, s = W.prefill_inputs(w, L=L)
    rng = np.random.default_rng(L)
    dout = W.f32_to_bf16_bits(rng.standard_normal(q.shape, dtype=np.float32))
    say(f"bwd {name} L={L} O {'fp32' if o_f32 else 'bf16'}")
    got = run_bwd(q, k, v, s, dout, w.window, w.scale, o_f32=o_f32)
    check_bwd(got, oracle_bwd(q, k, v, s, dout, w.window, w.scale), f"{name} L={L}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Lq,Lk,window,heads", [(1, 1, 0, (2, 1)), (65, 65, 0, (4, 2)),
                                                (129, 300, 0, (8, 1)), (200, 200, 1, (2, 2)),
                                                (333, 333, 100, (4, 4)), (257, 300, 513, (8, 2))])
def test_bwd_edges(gpu, D, Lq, Lk, window, heads):
    rng = np.random.default_rng(Lq * 7 + Lk + D)
    Hq, Hkv = heads
    q, k, v, dout, sinks = inputs(rng, 2, Hq, Hkv, Lq, Lk, D, sink_std=2.0)
    sinks[0] = 20.0
    say(f"bwd edge D={D} Lq={Lq} Lk={Lk} W={window} H={Hq}/{Hkv}")
    got = run_bwd(q, k, v, sinks, dout, window, D ** -0.5)
    check_bwd(got, oracle_bwd(q, k, v, sinks, dout, window, D ** -0.5), f"edge D={D} {Lq}/{Lk} W={window}")


def test_bwd_no_sink(gpu):
    rng = np.random.default_rng(1)
    q, k, v, dout, _ = inputs(rng, 1, 4, 2, 300, 300, 128)
    got = run_bwd(q, k, v, None, dout, 0, 128 ** -0.5)
    assert got[3] is None
    check_bwd(got, oracle_bwd(q, k, v, None, dout, 0, 128 ** -0.5), "no sink")


def test_bwd_deterministic(gpu):
    rng = np.random.default_rng(2)
    q, k, v, dout, s = inputs(rng, 2, 8, 2, 250, 250, 128)
    runs = [run_bwd(q, k, v, s, dout, 100, 128 ** -0.5) for _ in range(3)]
    for r in runs[1:]:
        for a, b in zip(r, runs[0]):
            assert np.array_equal(a, b)


def test_bwd_dsink_does_not_depend_on_o(gpu):
    """dsink takes D_i = sum_j P_ij dP_ij from the dQ phase, not <dO_i, O_i>:
    a bf16-rounded O (the dsink precision issue of the flash-attention
    profile) leaves it unchanged; dQ/dK/dV stay at the bar either way."""
    rng = np.random.default_rng(3)
    q, k, v, dout, s = inputs(rng, 4, 4, 1, 512, 512, 128, sink_std=0.5)
    s[0] = 20.0
    want = oracle_bwd(q, k, v, s, dout, 0, 128 ** -0.5)
    f32 = run_bwd(q, k, v, s, dout, 0, 128 ** -0.5, o_f32=True)
    b16 = run_bwd(q, k, v, s, dout, 0, 128 ** -0.5, o_f32=False)
    assert np.array_equal(f32[3], b16[3])
    check_bwd(f32, want, "fp32 O")
    check_bwd(b16, want, "bf16 O")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("o_f32", [False, True])
def test_bwd_full_size_swa_sampled(gpu, o_f32):
    """Full sliding-window workload: dK/dV of sampled 64-key blocks (every row
    that sees them, all heads of the KV head) and dQ of those rows, against the
    oracle on the slice of rows and keys that decides them exactly.  bf16 O is
    the launch the benchmark times."""
    w = W.SWA_PREFILL
    say("bwd full size: inputs")
    q, k, v, s = W.prefill_inputs(w)
    rng = np.random.default_rng(17)
    dout = W.f32_to_bf16_bits(rng.standard_normal(q.shape, dtype=np.float32))
    say("bwd full size: running")
    dq, dk, dv, ds = run_bwd(q, k, v, s, dout, w.window, w.scale, o_f32=o_f32)
    G = w.Hq // w.Hkv
    for kvh, k0 in ((0, 0), (3, 4032), (7, w.L - 64)):
        r_a, r_b = k0, min(w.L, k0 + 64 + w.window - 1)
        c_a = max(0, r_a - w.window + 1)
        heads = slice(kvh * G, (kvh + 1) * G)
        sub = lambda x, h, a, b: host_values(x[:, h, a:b], W.BF16)
        want = oracle.attention_bwd(sub(q, heads, r_a, r_b), sub(k, slice(kvh, kvh + 1), c_a, r_b),
                                    sub(v, slice(kvh, kvh + 1), c_a, r_b), s[heads],
                                    sub(dout, heads, r_a, r_b), w.window, w.scale)
        got = (dq[:, heads, r_a:r_b], dk[:, kvh:kvh + 1, k0:k0 + 64], dv[:, kvh:kvh + 1, k0:k0 + 64], None)
        ref = (want[0], want[1][:, :, k0 - c_a:k0 - c_a + 64], want[2][:, :, k0 - c_a:k0 - c_a + 64], None)
        check_bwd(got, ref, f"full swa kvh={kvh} keys {k0}..{k0 + 63}")


@pytest.mark.timeout(900)
def test_bwd_full_size_causal_sampled(gpu):
    """Full causal workload (B4 Hq32 Hkv8 L4096), bf16 O as the benchmark's
    causal backward launches it: dK/dV of two 64-key blocks of one (batch, KV
    head), every row that sees them being rows k0 .. L-1 of the group's heads,
    and dQ of those rows, against the oracle on rows [k0, L) and keys [0, L)
    (which decide them exactly under the causal mask); and dQ of rows 0..63,
    which see only keys 0..63."""
    w = W.CAUSAL_PREFILL
    say("bwd full size causal: inputs")
    q, k, v, s = W.prefill_inputs(w)
    rng = np.random.default_rng(23)
    dout = W.f32_to_bf16_bits(rng.standard_normal(q.shape, dtype=np.float32))
    say("bwd full size causal: running")
    dq, dk, dv, _ = run_bwd(q, k, v, s, dout, w.window, w.scale, o_f32=False)
    G = w.Hq // w.Hkv
    b, kvh = 1, 5
    heads = slice(kvh * G, (kvh + 1) * G)
    sub = lambda x, h, a, c: host_values(x[b:b + 1, h, a:c], W.BF16)
    for k0 in (w.L - 64, 1984):
        want = oracle.attention_bwd(sub(q, heads, k0, w.L), sub(k, slice(kvh, kvh + 1), 0, w.L),
                                    sub(v, slice(kvh, kvh + 1), 0, w.L), s[heads],
                                    sub(dout, heads, k0, w.L), w.window, w.scale)
        got = (dq[b:b + 1, heads, k0:], dk[b:b + 1, kvh:kvh + 1, k0:k0 + 64],
               dv[b:b + 1, kvh:kvh + 1, k0:k0 + 64], None)
        ref = (want[0], want[1][:, :, k0:k0 + 64], want[2][:, :, k0:k0 + 64], None)
        check_bwd(got, ref, f"full causal b={b} kvh={kvh} keys {k0}..{k0 + 63}")
    want = oracle.attention_bwd(sub(q, heads, 0, 64), sub(k, slice(kvh, kvh + 1), 0, 64),
                                sub(v, slice(kvh, kvh + 1), 0, 64), s[heads],
                                sub(dout, heads, 0, 64), w.window, w.scale)
    d = np.abs(dq[b:b + 1, heads, :64] - want[0])
    assert d.max() <= TOL_MAX * np.abs(want[0]).max(), f"full causal dq rows 0..63: {d.max():.3e}"
