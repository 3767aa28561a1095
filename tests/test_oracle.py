"""Pins of the float64 oracle (CPU only).

Every function of oracle/attention.py is checked here against something other
than itself: brute force, a library routine, closed forms, exact counts or
split/merge identities.  The last tests plant mistakes in the oracle and show
that a pin catches each one.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.attention as oa
import pins

TOL = 1e-12


# --- forward ----------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 1, 2, 3, 5, 100])
@pytest.mark.parametrize("heads", [(1, 1), (2, 1), (4, 2), (3, 3)])
def test_brute_force_small(window, heads):
    Hq, Hkv = heads
    for seed, (Lq, Lk) in enumerate([(6, 8), (8, 8), (1, 5), (3, 3)]):
        assert pins.err_vs_brute(seed=seed, Hq=Hq, Hkv=Hkv, Lq=Lq, Lk=Lk, window=window) < TOL
        assert pins.err_vs_brute(seed=seed, Hq=Hq, Hkv=Hkv, Lq=Lq, Lk=Lk, window=window,
                                 with_sink=False) < TOL


def test_brute_force_extreme_sinks():
    for s in (30.0, 100.0):
        assert pins.err_vs_brute(seed=7, sink_scale=s) < TOL


@pytest.mark.parametrize("window", [0, 1, 7, 64, 129, 513])
@pytest.mark.parametrize("with_sink", [True, False])
def test_torch_flash_cpu(window, with_sink):
    assert pins.err_vs_torch(window=window, with_sink=with_sink) < 1e-12
    assert pins.err_vs_torch(seed=3, Hq=2, Hkv=2, Lq=77, Lk=77, window=window,
                             with_sink=with_sink) < 1e-12


@pytest.mark.parametrize("window", [1, 2, 7, 512, 513, 514, 50, 0])
@pytest.mark.parametrize("sink", [None, -3.0, 0.0, 2.0])
def test_exact_counts(window, sink):
    assert pins.err_counts(Lq=40, Lk=50, window=window, sink=sink) < TOL
    assert pins.err_counts(Lq=600, Lk=600, window=window, sink=sink) < TOL


def test_counts_no_sink_give_integers():
    q = np.zeros((1, 1, 700, 4))
    k = pins.rand((1, 1, 700, 4), 1)
    v = pins.rand((1, 1, 700, 4), 2)
    _, lse = oracle.attention_fwd(q, k, v, None, 513, 0.1)
    n = np.exp(lse[0, 0])
    assert np.allclose(n, np.minimum(np.arange(700) + 1, 513), rtol=0, atol=1e-9)


def test_window_at_least_length_is_full_causal():
    q, k, v = pins.rand((1, 2, 256, 8), 1), pins.rand((1, 1, 256, 8), 2), pins.rand((1, 1, 256, 8), 3)
    s = np.array([0.3, 100.0])
    a = oracle.attention_fwd(q, k, v, s, 513, 0.125)
    b = oracle.attention_fwd(q, k, v, s, 0, 0.125)
    c = oracle.attention_fwd(q, k, v, s, 256, 0.125)
    for x, y in ((a, b), (a, c)):
        assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])


def test_window_one_is_sigmoid_of_self_score():
    D = 8
    q, k, v = pins.rand((1, 1, 20, D), 1), pins.rand((1, 1, 20, D), 2), pins.rand((1, 1, 20, D), 3)
    sigma, scale = 0.4, 0.3
    o, l = oracle.attention_fwd(q, k, v, np.array([sigma]), 1, scale)
    sc = float(np.float32(scale))
    s_ii = sc * np.einsum("id,id->i", q[0, 0], k[0, 0])
    want = v[0, 0] / (1.0 + np.exp(sigma - s_ii))[:, None]
    assert np.abs(o[0, 0] - want).max() < TOL
    assert np.abs(l[0, 0] - np.logaddexp(s_ii, sigma)).max() < TOL


@pytest.mark.parametrize("sigma", [-30.0, -1.0, 0.0, 2.5, 20.0, 100.0])
def test_sink_closed_form(sigma):
    assert pins.err_sink_closed_form(sigma=sigma) < TOL


def test_sink_to_minus_infinity_is_plain_attention():
    q, k, v = pins.rand((1, 2, 30, 8), 1), pins.rand((1, 1, 30, 8), 2), pins.rand((1, 1, 30, 8), 3)
    a = oracle.attention_fwd(q, k, v, None, 9, 0.4)
    b = oracle.attention_fwd(q, k, v, np.array([-np.inf, -np.inf]), 9, 0.4)
    c = oracle.attention_fwd(q, k, v, np.array([-800.0, -800.0]), 9, 0.4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.abs(a[0] - c[0]).max() == 0.0


def test_sink_dominance():
    q, k, v = pins.rand((1, 1, 64, 16), 1), pins.rand((1, 1, 64, 16), 2), pins.rand((1, 1, 64, 16), 3)
    o, l = oracle.attention_fwd(q, k, v, np.array([100.0]), 0, 0.25)
    assert np.isfinite(o).all() and np.abs(o).max() < 1e-30
    assert np.abs(l - 100.0).max() < 1e-30
    for sigma in (20.0, 30.0):
        o, l = oracle.attention_fwd(q, k, v, np.array([sigma]), 0, 0.25)
        sc = 0.25 * np.einsum("id,jd->ij", q[0, 0], k[0, 0])
        smax = sc.max()
        n = np.arange(64) + 1
        bound = n * np.exp(smax - sigma) * np.abs(v).max()
        assert (np.abs(o[0, 0]).max(axis=1) <= bound).all()
        assert (l[0, 0] >= sigma).all() and (l[0, 0] - sigma < n * np.exp(smax - sigma)).all()


def test_gqa_is_repeated_mha():
    assert pins.err_gqa() < TOL
    assert pins.err_gqa(Hq=8, Hkv=8) < TOL
    assert pins.err_gqa(Hq=8, Hkv=1) < TOL


def test_empty_rows():
    # Lk = 0: no key is visible; O = 0 and LSE = sink (or -inf without one).
    q = pins.rand((1, 2, 1, 4), 1)
    k = np.zeros((1, 1, 0, 4))
    o, l = oracle.attention_rows(q, k, k, np.array([1.5, -2.0]), 0, 0, [0], 0, 0.5)
    assert np.array_equal(o, np.zeros((1, 4))) and l[0] == 1.5
    o, l = oracle.attention_rows(q, k, k, None, 0, 1, [0], 0, 0.5)
    assert np.array_equal(o, np.zeros((1, 4))) and l[0] == -np.inf


def test_convex_combination_bounds():
    q, k, v = pins.rand((1, 1, 90, 8), 1), pins.rand((1, 1, 90, 8), 2), pins.rand((1, 1, 90, 8), 3)
    o, _ = oracle.attention_fwd(q, k, v, None, 20, 0.5)
    for i in range(90):
        lo = max(0, i - 19)
        vis = v[0, 0, lo:i + 1]
        assert (o[0, 0, i] <= vis.max(axis=0) + 1e-12).all()
        assert (o[0, 0, i] >= vis.min(axis=0) - 1e-12).all()


# --- split-KV decode ----------------------------------------------------------

def test_split_ranges_partition():
    for W in (0, 1, 64, 513, 1000):
        for Lk in (0, 1, 2, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1025, 4097, 32768):
            lo = 0 if W <= 0 else max(0, Lk - W)
            for ns in range(1, 65):
                sp = oracle.split_ranges(Lk, ns, W)
                assert len(sp) <= ns
                covered = [j for a, z in sp for j in range(a, z)]
                assert covered == list(range(lo, Lk))
                assert all(z > a for a, z in sp)
                if sp:
                    chunk = sp[0][1] - sp[0][0] if len(sp) > 1 else None
                    if chunk is not None:
                        assert chunk % 64 == 0
                        assert all(z - a == chunk for a, z in sp[:-1])
                        # the smallest multiple of 64 that lets ns chunks cover the range
                        assert chunk == max(64, -(-(-(-(Lk - lo) // ns)) // 64) * 64)


def test_split_ranges_examples():
    # 1025 keys in 64 splits: chunks of 64, so 17 splits exist, the last holds one key.
    sp = oracle.split_ranges(1025, 64, 0)
    assert len(sp) == 17 and sp[-1] == (1024, 1025)
    assert oracle.split_ranges(0, 5, 0) == []
    assert oracle.split_ranges(32768, 64, 0) == [(512 * s, 512 * s + 512) for s in range(64)]
    assert oracle.split_ranges(5000, 3, 513) == [(4487, 4679), (4679, 4871), (4871, 5000)]


def test_split_combine_equals_unsplit():
    assert pins.err_split_combine() < TOL


def test_decode_equals_forward_with_one_query():
    q = pins.rand((3, 4, 1, 8), 1)
    kc, vc = pins.rand((3, 2, 300, 8), 2), pins.rand((3, 2, 300, 8), 3)
    sinks = pins.rand(4, 4)
    seqlens = np.array([300, 17, 129])
    for W in (0, 5, 513):
        o, l = oracle.decode(q, kc, vc, seqlens, sinks, W, 0.3)
        for b in range(3):
            L = seqlens[b]
            of, lf = oracle.attention_fwd(q[b:b + 1], kc[b:b + 1, :, :L], vc[b:b + 1, :, :L], sinks, W, 0.3)
            assert np.array_equal(o[b], of[0, :, 0]) and np.array_equal(l[b], lf[0, :, 0])


def test_combine_reads_only_valid_lanes():
    q = pins.rand((2, 2, 1, 8), 1)
    kc, vc = pins.rand((2, 1, 200, 8), 2), pins.rand((2, 1, 200, 8), 3)
    seqlens, ns = np.array([200, 70]), np.array([64, 64])
    op, lp, nv = oracle.decode_partials(q, kc, vc, seqlens, ns, 0, 0.3)
    assert list(nv) == [4, 2]
    assert np.isnan(op[0, :, 4:]).all() and np.isnan(lp[1, :, 2:]).all()
    o, l = oracle.combine(op, lp, nv, np.array([0.5, 9.0]))
    assert np.isfinite(o).all() and np.isfinite(l).all()


def test_combine_one_split_is_the_sink_rebase():
    # With one split the combine is the sink update of a single partial:
    # O = O_0 * sigmoid(lse_0 - sigma), LSE = logaddexp(lse_0, sigma).
    o_part = pins.rand((1, 1, 1, 8), 1)
    lse_part = np.array([[[3.0]]])
    for sigma in (-5.0, 3.0, 100.0):
        o, l = oracle.combine(o_part, lse_part, np.array([1]), np.array([sigma]))
        assert np.abs(o[0, 0] - o_part[0, 0, 0] / (1 + math.exp(sigma - 3.0))).max() < TOL
        assert abs(l[0, 0] - np.logaddexp(3.0, sigma)) < TOL


def test_combine_empty_sequence():
    o, l = oracle.combine(np.zeros((1, 2, 4, 3)), np.zeros((1, 2, 4)), np.array([0]), np.array([0.7, 2.0]))
    assert np.array_equal(o, np.zeros((1, 2, 3))) and list(l[0]) == [0.7, 2.0]
    o, l = oracle.combine(np.zeros((1, 1, 4, 3)), np.zeros((1, 1, 4)), np.array([0]), None)
    assert l[0, 0] == -np.inf and np.array_equal(o, np.zeros((1, 1, 3)))


# --- the two sink updates of the Flint patch (float32) ---------------------

def test_naive_sink_update_overflows_in_f32():
    # Running max 3.0 in raw units, scale 1/8: content exponent ~0.54, while
    # the sink +100 contributes 2^(144.27 - 0.54) -- beyond float32's range.
    scale_log2 = np.float32(0.125 * oracle.LOG2E)
    out = oracle.naive_sink_row_sum_f32(3.0, 5.0, 100.0, scale_log2)
    assert np.isinf(out)
    rm, rs, rescale = oracle.rebase_sink_f32(3.0, 5.0, 100.0, scale_log2)
    assert np.isfinite(rs) and np.isfinite(rescale) and rs >= 1.0 and rescale <= 1.0


@pytest.mark.parametrize("sink", [-40.0, -2.0, 0.0, 1.0, 20.0, 100.0])
def test_rebase_update_matches_definition(sink):
    # Online state of one row after all keys: row_max (raw units) and
    # row_sum = sum 2^((x_j - row_max) * scale_log2); the rebase then gives
    # LSE = ln2 * (new_max_log2 + log2 row_sum) and O = acc * rescale / row_sum.
    rng = np.random.default_rng(11)
    x = rng.standard_normal(40).astype(np.float32) * np.float32(8)     # raw q.k
    vals = rng.standard_normal((40, 4))
    scale = 0.125
    sl2 = np.float32(scale * oracle.LOG2E)
    row_max = np.float32(x.max())
    p = np.exp2((x - row_max) * sl2, dtype=np.float32)
    row_sum = np.float32(p.sum(dtype=np.float32))
    acc = (p[:, None].astype(np.float64) * vals).sum(axis=0)
    new_max, new_sum, rescale = oracle.rebase_sink_f32(row_max, row_sum, sink, sl2)
    lse = math.log(2) * (float(new_max) * float(sl2) + math.log2(float(new_sum)))
    o = acc * float(rescale) / float(new_sum)
    s = scale * x.astype(np.float64)
    want_l = np.logaddexp(np.logaddexp.reduce(s), sink)
    w = np.exp(s - want_l)
    want_o = (w[:, None] * vals).sum(axis=0)
    assert abs(lse - want_l) < 1e-5 * max(1.0, abs(want_l))
    assert np.abs(o - want_o).max() < 1e-5


# --- stored regression fixture ----------------------------------------------

def test_golden_fixture():
    here = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")
    with open(here) as f:
        g = json.load(f)
    q, k, v = (np.array(g[n]) for n in ("q", "k", "v"))
    o, l = oracle.attention_fwd(q, k, v, np.array(g["sinks"]), g["window"], g["scale"])
    assert np.abs(o - np.array(g["out"])).max() < 1e-14
    assert np.abs(l - np.array(g["lse"])).max() < 1e-14


# --- planted mistakes: each must be caught by some pin ------------------------

def _caught(monkeypatch, name, fake):
    with monkeypatch.context() as m:
        m.setattr(oa, name, fake)
        errs = [
            pins.err_vs_brute(window=3),
            pins.err_vs_brute(window=0, Hq=4, Hkv=2, Lq=5, Lk=8),
            pins.err_vs_torch(window=7),
            pins.err_counts(window=7, sink=1.0),
            pins.err_sink_closed_form(),
            pins.err_gqa(),
        ]
    return max(errs) > 1e-6


def test_pins_catch_window_off_by_one(monkeypatch):
    def fake(p, Lk, window):
        hi = min(p + 1, Lk)
        lo = 0 if window <= 0 else max(0, p - window)   # one key too many
        return lo, max(lo, hi)
    assert _caught(monkeypatch, "visible_range", fake)


def test_pins_catch_top_left_alignment(monkeypatch):
    assert _caught(monkeypatch, "query_position", lambda i, Lq, Lk: i)


def test_pins_catch_wrong_kv_head(monkeypatch):
    assert _caught(monkeypatch, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)


def test_pins_catch_sink_dropped_from_lse(monkeypatch):
    orig = oa._finish

    def fake(scores, vals, sigma):
        o, _ = orig(scores, vals, sigma)
        _, l = orig(scores, vals, -np.inf)
        return o, l
    assert _caught(monkeypatch, "_finish", fake)


def test_pins_catch_scaled_sink(monkeypatch):
    orig = oa.attention_rows

    def fake(q, k, v, sinks, b, h, rows, window, scale):
        s = None if sinks is None else np.asarray(sinks, dtype=np.float64) * scale
        return orig(q, k, v, s, b, h, rows, window, scale)
    with monkeypatch.context() as m:
        m.setattr(oa, "attention_rows", fake)
        assert pins.err_vs_torch(window=7) > 1e-6


def test_pins_catch_split_mistakes(monkeypatch):
    orig = oa.split_ranges

    def drop_last(Lk, ns, window):
        return orig(Lk, ns, window)[:-1] if ns > 1 else orig(Lk, ns, window)
    with monkeypatch.context() as m:
        m.setattr(oa, "split_ranges", drop_last)
        assert pins.err_split_combine(splits=(2, 7)) > 1e-6

    def overlap(Lk, ns, window):
        return [(max(0, a - 1), z) for a, z in orig(Lk, ns, window)]
    with monkeypatch.context() as m:
        m.setattr(oa, "split_ranges", overlap)
        assert pins.err_split_combine(splits=(2, 7)) > 1e-6


# --- maximum pre-softmax logit -------------------------------------------------

@pytest.mark.parametrize("window", [0, 1, 3, 20])
def test_max_logit_brute_force(window):
    assert pins.err_max_logit_brute(window=window) < 1e-12
    assert pins.err_max_logit_brute(window=window, Lq=4, Lk=9, Hq=3, Hkv=1) < 1e-12


@pytest.mark.parametrize("window", [0, 1, 7, 100])
def test_max_logit_ramp_closed_form(window):
    assert pins.err_max_logit_ramp(window=window) < 1e-12


def test_max_logit_within_lse_bounds():
    assert pins.err_max_logit_lse_bounds() < 1e-12
    assert pins.err_max_logit_lse_bounds(window=0, Lq=60, Lk=60) < 1e-12


def test_max_logit_torch_masked_max():
    assert pins.err_max_logit_torch() < 1e-12
    assert pins.err_max_logit_torch(window=0) < 1e-12


def test_max_logit_gqa_is_repeated_mha():
    assert pins.err_max_logit_gqa() == 0.0


def test_max_logit_ignores_sink_and_values():
    q, k = pins.rand((1, 2, 5, 4), 1), pins.rand((1, 1, 5, 4), 2)
    row, head = oracle.max_logit(q, k, 0, 0.5)
    # row 0 sees only key 0; the last row sees every key
    assert row[0, 0, 0] == pytest.approx(float(np.float32(0.5)) * float(q[0, 0, 0] @ k[0, 0, 0]), abs=1e-12)
    assert head.shape == (1, 2) and np.all(head == row.max(axis=2))


def _max_logit_caught(monkeypatch, name, fake):
    with monkeypatch.context() as m:
        m.setattr(oa, name, fake)
        errs = [pins.err_max_logit_brute(window=3), pins.err_max_logit_ramp(window=7),
                pins.err_max_logit_torch(), pins.err_max_logit_lse_bounds()]
    return max(errs) > 1e-6


def test_max_logit_pins_catch_index_mistakes(monkeypatch):
    def one_more_key(p, Lk, window):
        hi = min(p + 1, Lk)
        lo = 0 if window <= 0 else max(0, p - window)
        return lo, max(lo, hi)
    assert _max_logit_caught(monkeypatch, "visible_range", one_more_key)
    assert _max_logit_caught(monkeypatch, "query_position", lambda i, Lq, Lk: i)
    assert _max_logit_caught(monkeypatch, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)


def test_max_logit_pins_catch_missing_scale(monkeypatch):
    assert _max_logit_caught(monkeypatch, "effective_scale", lambda s: 1.0)


# --- split-count planning --------------------------------------------------------

@pytest.mark.parametrize("seed,B,Lk_max,window,Hq,Hkv,max_splits,slots", [
    (0, 40, 5000, 0, 64, 8, 64, 512), (1, 64, 32768, 0, 64, 8, 64, 512),
    (2, 3, 32768, 513, 64, 8, 64, 512), (3, 256, 2048, 0, 64, 8, 64, 512),
    (4, 16, 32768, 0, 64, 64, 64, 512), (5, 9, 100000, 0, 8, 1, 17, 77),
    (6, 1, 131072, 0, 64, 8, 64, 512), (7, 33, 9000, 1000, 40, 1, 64, 256),
])
def test_plan_matches_rule(seed, B, Lk_max, window, Hq, Hkv, max_splits, slots):
    assert pins.err_plan(seed, B, Lk_max, window, Hq, Hkv, max_splits, slots) == 0


def test_plan_properties():
    rng = np.random.default_rng(9)
    for _ in range(20):
        sl = list(rng.integers(0, 40000, int(rng.integers(1, 80))))
        ns = oracle.plan_splits(sl, 64, 8, 32768, 0, 64, "auto", 0, 512)
        assert all(1 <= x <= 64 for x in ns)
        # uniform lengths -> one chunk target for all: equal split counts
    assert len(set(oracle.plan_splits([20000] * 10, 64, 8, 32768, 0, 64, "auto", 0, 512))) == 1
    # empty sequences still get one (empty) split
    assert oracle.plan_splits([0, -3], 64, 8, 100, 0, 64, "auto", 0, 512) == [1, 1]


def test_plan_per_sequence_properties():
    """Properties any per-sequence plan must have, independent of the rule's
    constants: the counts follow their sequences under a permutation of the
    batch, empty sequences change nothing for the others (they add no work)
    and get one split (a fixed count under "count"), and no sequence gets more splits than it has 256-key
    chunks (the smallest target) or than max_splits."""
    rng = np.random.default_rng(31)
    for trial in range(12):
        B = int(rng.integers(1, 60))
        Lk_max = int(rng.choice([2048, 32768, 100000]))
        window = int(rng.choice([0, 513, 5000]))
        ms = int(rng.choice([8, 64]))
        sl = [int(x) for x in rng.integers(0, Lk_max + 10, B)]
        perm = rng.permutation(B)
        for policy, param in (("auto", 0), ("keys", 700), ("count", 5)):
            plan = lambda x: oracle.plan_splits(x, 64, 8, Lk_max, window, ms, policy, param, 256)
            ns = plan(sl)
            assert plan([sl[i] for i in perm]) == [ns[i] for i in perm]
            empty = 1 if policy != "count" else min(param, ms)
            assert plan(sl + [0, 0, 0]) == ns + [empty] * 3
            for n, x in zip(ns, sl):
                v = oa.visible_keys(x, Lk_max, window)
                assert 1 <= n <= ms
                if policy == "auto":
                    assert n <= max(1, -(-v // 256))


def test_plan_pins_catch_changed_rule(monkeypatch):
    with monkeypatch.context() as m:
        m.setattr(oa, "PLAN_ITEM_COST", 0)
        assert pins.err_plan(1, 64, 32768) > 0
    with monkeypatch.context() as m:
        m.setattr(oa, "PLAN_CHUNKS", (512, 1024, 2048))
        assert pins.err_plan(1, 64, 32768) > 0


# --- paged KV and varlen -------------------------------------------------------------

@pytest.mark.parametrize("page_size,window", [(16, 0), (1, 0), (64, 100), (7, 5)])
def test_paged_decode_equals_dense(page_size, window):
    assert pins.err_paged(page_size=page_size, window=window) < 1e-12


def test_varlen_equal_lengths_is_dense_batch():
    assert pins.err_varlen_equal_lengths() < 1e-12
    assert pins.err_varlen_equal_lengths(window=0, L=33) < 1e-12


@pytest.mark.parametrize("window", [0, 2, 3])
def test_varlen_brute_force(window):
    assert pins.err_varlen_brute(window=window) < 1e-12


def test_paged_varlen_pins_catch_mistakes(monkeypatch):
    with monkeypatch.context() as m:   # row within the page off by one
        m.setattr(oa, "page_slot", lambda j, ps: (j // ps, (j + 1) % ps))
        assert pins.err_paged(page_size=4, Lk_max=12) > 1e-6
    orig = oa.attention_fwd

    def global_positions(q, k, v, sinks, window, scale, block=256):
        # a mistake: every sequence aligned top-left instead of bottom-right
        Lq, Lk = q.shape[2], k.shape[2]
        if Lq < Lk:
            k, v = k[:, :, :Lq], v[:, :, :Lq]
        return orig(q, k, v, sinks, window, scale, block)
    with monkeypatch.context() as m:
        m.setattr(oa, "attention_fwd", global_positions)
        assert pins.err_varlen_brute(window=3) > 1e-6


# --- backward -----------------------------------------------------------------------

@pytest.mark.parametrize("window,Lq,Lk", [(3, 5, 6), (0, 4, 4), (1, 3, 5), (10, 6, 6)])
def test_bwd_finite_differences(window, Lq, Lk):
    assert pins.err_bwd_finite_diff(window=window, Lq=Lq, Lk=Lk) < 1e-7


def test_bwd_finite_differences_gqa_and_dominant_sink():
    assert pins.err_bwd_finite_diff(Hq=4, Hkv=2, seed=3) < 1e-7


@pytest.mark.parametrize("window", [0, 9])
def test_bwd_torch_autograd(window):
    assert pins.err_bwd_torch(window=window) < 1e-10


def test_bwd_gqa_is_summed_mha():
    assert pins.err_bwd_gqa() < 1e-12


def test_bwd_shift_invariance():
    assert pins.err_bwd_shift_invariance() < 1e-10


def test_bwd_no_sink_means_zero_dsink():
    q, k, v = pins.rand((1, 2, 6, 3), 0), pins.rand((1, 1, 6, 3), 1), pins.rand((1, 1, 6, 3), 2)
    dq, dk, dv, ds = oracle.attention_bwd(q, k, v, None, pins.rand((1, 2, 6, 3), 3), 0, 0.5)
    assert np.all(ds == 0.0)


def _bwd_caught(monkeypatch, name, fake):
    with monkeypatch.context() as m:
        m.setattr(oa, name, fake)
        errs = [pins.err_bwd_torch(window=9), pins.err_bwd_finite_diff(window=3)]
    return max(errs) > 1e-6


def test_bwd_pins_catch_mistakes(monkeypatch):
    orig = oa._bwd_block

    def no_D(Q, K, V, dO, sigma, sc, ranges, lo):       # dS = P * dP (the D term dropped)
        S = sc * (Q @ K.T)
        cols = np.arange(lo, lo + K.shape[0])
        for r, (a, z) in enumerate(ranges):
            S[r, (cols < a) | (cols >= z)] = -np.inf
        M = np.maximum(S.max(axis=1), sigma)
        e = np.exp(S - M[:, None])
        den = e.sum(axis=1) + np.exp(sigma - M)
        P = e / den[:, None]
        dS = P * (dO @ V.T)
        _, _, gv, gs = orig(Q, K, V, dO, sigma, sc, ranges, lo)
        return sc * (dS @ K), sc * (dS.T @ Q), gv, gs
    assert _bwd_caught(monkeypatch, "_bwd_block", no_D)

    def flipped_dsink(*a):
        gq, gk, gv, gs = orig(*a)
        return gq, gk, gv, -gs
    assert _bwd_caught(monkeypatch, "_bwd_block", flipped_dsink)

    def unscaled_dk(Q, K, V, dO, sigma, sc, ranges, lo):
        gq, gk, gv, gs = orig(Q, K, V, dO, sigma, sc, ranges, lo)
        return gq, gk / sc, gv, gs
    assert _bwd_caught(monkeypatch, "_bwd_block", unscaled_dk)
    assert _bwd_caught(monkeypatch, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
