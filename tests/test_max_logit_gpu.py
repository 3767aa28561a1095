"""GPU parity of attn_fwd_max_logit: the largest pre-softmax logit per row and
per head against the float64 oracle, and O/LSE bitwise equal to attn_fwd.

The kernel's scores are fp32 sums of exact bf16 products (fp32 products for
fp32 inputs), so the maximum differs from the float64 value only by
summation rounding: |d| <= 1e-4 + 1e-5 |max| is the bar here.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_attn_amd import workloads as W

gpu_util = pytest.importorskip("gpu_util")
from gpu_util import compare, host_values, run_fwd, run_fwd_max_logit, say  # noqa: E402

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-4, 1e-5


def check_max(got, want, what):
    assert got.shape == want.shape, what
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    assert np.all(got[~fin] == want[~fin]), f"{what}: non-finite values differ"
    d = np.abs(got[fin] - want[fin])
    bound = ATOL + RTOL * np.abs(want[fin])
    assert (d <= bound).all(), f"{what}: max|d max-logit| = {d.max():.3e}"


def oracle_max(q, k, dtype, window, scale):
    return oracle.max_logit(host_values(q, dtype), host_values(k, dtype), window, scale)


def same_as_fwd(q, k, v, s, dtype, window, scale, o, l, what):
    o2, l2 = run_fwd(q, k, v, s, dtype, window, scale)
    assert np.array_equal(o, o2) and np.array_equal(l, l2), f"{what}: O/LSE differ from attn_fwd"


def test_max_logit_tiny_f32(gpu):
    w = W.TINY_PREFILL
    q, k, v, s = W.prefill_inputs(w)
    say("max logit: tiny_prefill")
    o, l, mr, mh = run_fwd_max_logit(q, k, v, s, w.dtype, w.window, w.scale)
    want_r, want_h = oracle_max(q, k, w.dtype, w.window, w.scale)
    check_max(mr, want_r, "tiny rows")
    check_max(mh, want_h, "tiny heads")
    same_as_fwd(q, k, v, s, w.dtype, w.window, w.scale, o, l, "tiny")


@pytest.mark.parametrize("name,L", [("swa_prefill", 1000), ("causal_prefill", 700),
                                    ("long_swa_prefill", 1500)])
def test_max_logit_workload_reduced(gpu, name, L):
    w = W.WORKLOADS[name]
    q, k, v, s = W.prefill_inputs(w, L=L)
    say(f"max logit: {name} L={L}")
    o, l, mr, mh = run_fwd_max_logit(q, k, v, s, w.dtype, w.window, w.scale)
    want_r, want_h = oracle_max(q, k, w.dtype, w.window, w.scale)
    check_max(mr, want_r, f"{name} rows")
    check_max(mh, want_h, f"{name} heads")
    o_ref, l_ref = oracle.attention_fwd(host_values(q, w.dtype), host_values(k, w.dtype),
                                        host_values(v, w.dtype), s, w.window, w.scale)
    compare(o, l, o_ref, l_ref, f"{name} L={L} (max-logit entry point)")
    same_as_fwd(q, k, v, s, w.dtype, w.window, w.scale, o, l, name)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Lq,Lk", [(1, 1), (2, 2), (65, 65), (129, 129), (37, 300), (200, 1000)])
def test_max_logit_edges(gpu, D, Lq, Lk):
    rng = np.random.default_rng(Lq * 13 + Lk + D)
    for (Hq, Hkv) in ((2, 2), (8, 1), (4, 2)):
        q = W.f32_to_bf16_bits(rng.standard_normal((2, Hq, Lq, D), dtype=np.float32))
        k = W.f32_to_bf16_bits(rng.standard_normal((2, Hkv, Lk, D), dtype=np.float32) * 2)
        v = W.f32_to_bf16_bits(rng.standard_normal((2, Hkv, Lk, D), dtype=np.float32))
        for window in (0, 1, 64, 513):
            _, _, mr, mh = run_fwd_max_logit(q, k, v, None, W.BF16, window, D ** -0.5)
            want_r, want_h = oracle_max(q, k, W.BF16, window, D ** -0.5)
            what = f"D={D} Lq={Lq} Lk={Lk} H={Hq}/{Hkv} W={window}"
            check_max(mr, want_r, what + " rows")
            check_max(mh, want_h, what + " heads")


def test_max_logit_f32_inputs_and_only_one_output(gpu):
    rng = np.random.default_rng(5)
    L, D = 333, 128
    q = rng.standard_normal((2, 4, L, D), dtype=np.float32)
    k = rng.standard_normal((2, 2, L, D), dtype=np.float32)
    v = rng.standard_normal((2, 2, L, D), dtype=np.float32)
    want_r, want_h = oracle_max(q, k, W.F32, 200, D ** -0.5)
    _, _, mr, mh = run_fwd_max_logit(q, k, v, None, W.F32, 200, D ** -0.5, want_head=False)
    assert mh is None
    check_max(mr, want_r, "f32 rows only")
    _, _, mr, mh = run_fwd_max_logit(q, k, v, None, W.F32, 200, D ** -0.5, want_row=False)
    assert mr is None
    check_max(mh, want_h, "f32 heads only")


@pytest.mark.timeout(900)
def test_max_logit_full_size_swa(gpu):
    """Full swa_prefill: every head maximum against the kernel's own row maxima,
    sampled rows of four heads against the oracle."""
    w = W.SWA_PREFILL
    say("max logit: swa_prefill full size")
    q, k, v, s = W.prefill_inputs(w)
    o, l, mr, mh = run_fwd_max_logit(q, k, v, s, w.dtype, w.window, w.scale, out_f32=False)
    assert np.array_equal(mh, mr.max(axis=2))
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(11)
    for h in (0, 5, 33, 63):
        rows = np.unique(np.concatenate([[0, 1, 511, 512, 513, w.L - 1], rng.integers(0, w.L, 60)]))
        qs = host_values(q[:, h:h + 1], w.dtype)
        ks = host_values(k[:, h // G:h // G + 1], w.dtype)
        want = oracle.max_logit_rows(qs, ks, 0, 0, rows, w.window, w.scale)
        check_max(mr[0, h, rows], want, f"full swa h={h}")
