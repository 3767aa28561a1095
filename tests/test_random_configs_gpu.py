"""GPU parity on seeded random configurations: every entry point against the
float64 oracle on shapes drawn together (batch, GQA group, head dim, lengths,
window, scale, sinks, score range, input and output dtype), so that
combinations no hand-picked case names are covered too.  Each case prints its
drawn configuration before it runs.  Same bars as the hand-picked tests.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_attn_amd import workloads as W

gpu_util = pytest.importorskip("gpu_util")
from gpu_util import compare, host_values, run_decode, run_fwd, say  # noqa: E402
from test_bwd_gpu import check_bwd, oracle_bwd, run_bwd  # noqa: E402
from test_serving_gpu import pack, run_varlen  # noqa: E402

pytestmark = pytest.mark.gpu

N_FWD, N_DEC, N_VARLEN, N_BWD = 32, 16, 8, 8


def _sinks(rng, Hq, allow_none=True):
    """None, or N(0, 2) logits with some heads forced to +30 (sink dominates) or
    -inf (no sink: plain attention)."""
    if allow_none and rng.random() < 0.2:
        return None
    s = (rng.standard_normal(Hq) * 2.0).astype(np.float32)
    for h in range(Hq):
        u = rng.random()
        if u < 0.1:
            s[h] = 30.0
        elif u < 0.2:
            s[h] = -np.inf
    return s


def _bits(rng, shape, amp):
    return W.f32_to_bf16_bits((rng.standard_normal(shape, dtype=np.float32) * amp).astype(np.float32))


def _window(rng, L):
    return int(rng.choice([0, 0, 1, 2, 513, int(rng.integers(1, L + 20))]))


@pytest.mark.parametrize("i", range(N_FWD))
def test_random_forward(gpu, i):
    rng = np.random.default_rng(1000 + i)
    D = int(rng.choice([64, 128]))
    dtype = W.F32 if rng.random() < 0.2 else W.BF16
    B, Hkv, G = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 4])), int(rng.choice([1, 2, 3, 4, 5, 8]))
    Hq = G * Hkv
    Lk = int(rng.integers(1, 700))
    Lq = Lk if rng.random() < 0.5 else int(rng.integers(1, Lk + 1))
    window = _window(rng, Lk)
    scale = D ** -0.5 * float(rng.choice([1.0, 0.5, 2.0]))
    amp = float(rng.choice([1.0, 1.0, 4.0]))  # x4: scores of std up to 16 (x2 scale: 32)
    out_f32 = bool(rng.random() < 0.5)
    sinks = _sinks(rng, Hq)
    what = (f"fwd #{i}: B={B} H={Hq}/{Hkv} Lq={Lq} Lk={Lk} D={D} {dtype} W={window} "
            f"scale={scale:.4f} amp={amp} out_f32={out_f32} sinks={'none' if sinks is None else 'yes'}")
    say(what)
    # q and k carry the score range; v stays N(0, 1), the workloads' values
    if dtype == W.F32:
        gen = lambda shape, a: (rng.standard_normal(shape, dtype=np.float32) * a).astype(np.float32)
    else:
        gen = lambda shape, a: _bits(rng, shape, a)
    q, k, v = gen((B, Hq, Lq, D), amp), gen((B, Hkv, Lk, D), amp), gen((B, Hkv, Lk, D), 1.0)
    o, l = run_fwd(q, k, v, sinks, dtype, window, scale, out_f32=out_f32)
    o_r, l_r = oracle.attention_fwd(host_values(q, dtype), host_values(k, dtype), host_values(v, dtype),
                                    sinks, window, scale)
    compare(o, l, o_r, l_r, what, bf16_out=not out_f32)


@pytest.mark.parametrize("i", range(N_DEC))
def test_random_decode(gpu, i):
    rng = np.random.default_rng(2000 + i)
    D = int(rng.choice([64, 128]))
    B, Hkv, G = int(rng.integers(1, 11)), int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8, 16]))
    Hq = G * Hkv
    Lmax = int(rng.integers(1, 3000))
    seqlens = rng.integers(0, Lmax, size=B, endpoint=True).astype(np.int32)
    seqlens[rng.random(B) < 0.15] = 0
    max_splits = int(rng.choice([8, 33, 64]))
    nsplits = rng.integers(1, max_splits, size=B, endpoint=True).astype(np.int32)
    window = _window(rng, Lmax)
    scale = D ** -0.5 * float(rng.choice([1.0, 0.5, 2.0]))
    amp = float(rng.choice([1.0, 1.0, 4.0]))
    out_f32 = bool(rng.random() < 0.5)
    sinks = _sinks(rng, Hq)
    what = (f"decode #{i}: B={B} H={Hq}/{Hkv} Lmax={Lmax} D={D} W={window} max_splits={max_splits} "
            f"scale={scale:.4f} amp={amp} out_f32={out_f32} sinks={'none' if sinks is None else 'yes'}")
    say(what)
    q = _bits(rng, (B, Hq, 1, D), amp)
    kc = _bits(rng, (B, Hkv, Lmax, D), amp)
    vc = _bits(rng, (B, Hkv, Lmax, D), 1.0)
    op, lp, o, l = run_decode(q, kc, vc, seqlens, nsplits, sinks, window, scale, max_splits=max_splits,
                              out_f32=out_f32)
    qf, kf, vf = (host_values(x, W.BF16) for x in (q, kc, vc))
    op_r, lp_r, nv = oracle.decode_partials(qf, kf, vf, seqlens, nsplits, window, scale)
    o_r, l_r = oracle.combine(op_r, lp_r, nv, sinks)
    for b in range(B):
        n = int(nv[b])
        if n:
            compare(op[b, :, :n], lp[b, :, :n], op_r[b, :, :n], lp_r[b, :, :n], f"{what} partials b={b}")
        assert np.isnan(op[b, :, n:]).all() and np.isnan(lp[b, :, n:]).all(), f"{what}: lane >= n_valid written"
    compare(o, l, o_r, l_r, what, bf16_out=not out_f32)
    ou, lu = oracle.decode(qf, kf, vf, seqlens, sinks, window, scale)
    compare(o, l, ou, lu, what + " vs unsplit", bf16_out=not out_f32)


@pytest.mark.parametrize("i", range(N_VARLEN))
def test_random_varlen(gpu, i):
    rng = np.random.default_rng(3000 + i)
    D = int(rng.choice([64, 128]))
    Hkv, G = int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8]))
    Hq = G * Hkv
    B = int(rng.integers(1, 7))
    lk = rng.integers(0, 500, size=B, endpoint=True)
    # mostly chunks of the key range (lq <= lk), sometimes longer than the keys
    lq = np.array([int(rng.integers(0, x + 1)) if rng.random() < 0.8 else int(rng.integers(0, 400))
                   for x in lk])
    window = _window(rng, int(lk.max()) if lk.max() > 0 else 1)
    scale = D ** -0.5 * float(rng.choice([1.0, 0.5]))
    out_f32 = bool(rng.random() < 0.5)
    sinks = _sinks(rng, Hq)
    what = (f"varlen #{i}: B={B} H={Hq}/{Hkv} D={D} W={window} lq={lq.tolist()} lk={lk.tolist()} "
            f"out_f32={out_f32}")
    say(what)
    Lq_max, Lk_max = max(int(lq.max()), 1), max(int(lk.max()), 1)
    qb, kb, vb = (_bits(rng, (B, H, L, D), 1.0) for H, L in ((Hq, Lq_max), (Hkv, Lk_max), (Hkv, Lk_max)))
    q, k, v = pack(qb, lq), pack(kb, lk), pack(vb, lk)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    if q.shape[1] == 0:
        pytest.skip("no query rows drawn")
    if k.shape[1] == 0:
        k = v = np.zeros((Hkv, 0, D), np.uint16)
    o, l = run_varlen(q, k, v, cu_q, cu_k, sinks, window, scale, Lq_max, out_f32=out_f32)
    o_r, l_r = oracle.attention_fwd_varlen(host_values(q, W.BF16), host_values(k, W.BF16),
                                           host_values(v, W.BF16), cu_q, cu_k, sinks, window, scale)
    compare(o, l, o_r, l_r, what, bf16_out=not out_f32)


@pytest.mark.parametrize("i", range(N_BWD))
def test_random_backward(gpu, i):
    rng = np.random.default_rng(4000 + i)
    D = int(rng.choice([64, 128]))
    B, Hkv, G = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8]))
    Hq = G * Hkv
    Lk = int(rng.integers(1, 400))
    Lq = Lk if rng.random() < 0.6 else int(rng.integers(1, Lk + 1))
    window = _window(rng, Lk)
    scale = D ** -0.5 * float(rng.choice([1.0, 0.5]))
    o_f32 = bool(rng.random() < 0.5)
    sinks = _sinks(rng, Hq)  # a -inf sink has dsink 0
    what = (f"bwd #{i}: B={B} H={Hq}/{Hkv} Lq={Lq} Lk={Lk} D={D} W={window} scale={scale:.4f} "
            f"o_f32={o_f32} sinks={'none' if sinks is None else 'yes'}")
    say(what)
    q, k, v, dout = (_bits(rng, s, 1.0) for s in ((B, Hq, Lq, D), (B, Hkv, Lk, D), (B, Hkv, Lk, D),
                                                  (B, Hq, Lq, D)))
    got = run_bwd(q, k, v, sinks, dout, window, scale, o_f32=o_f32)
    check_bwd(got, oracle_bwd(q, k, v, sinks, dout, window, scale), what)
