"""GPU parity beyond 2^32 elements: the largest launches (tensors of 5-17 GB, a paged pool of 2 x 13 GB) in
which element offsets pass 2^31 and 2^32, checked on sampled rows against the
float64 oracle.  Inputs are drawn on the device by a seeded torch generator;
the oracle reads the same values, copied back for the sampled rows' heads.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_attention_attn_amd as A
import oracle

gpu_util = pytest.importorskip("gpu_util")
from gpu_util import compare, say  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _release_device_memory():
    """Hand the tens of GB these launches reserve back to the device after each
    test, so that the tests after them start from an empty cache."""
    yield
    import gc

    gc.collect()
    torch.cuda.empty_cache()


def _randn(g, shape):
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)


def _host(t):
    return t.float().cpu().numpy()


@pytest.mark.timeout(900)
def test_forward_offsets_beyond_4g_elements(gpu):
    """Three long sliding-window sequences (B3 Hq64 Hkv8 L262144 D128, window
    513): q and O hold 6.4e9 elements each, so the last batch's rows sit past
    2^32 elements.  bf16 O, the launch the benchmark times."""
    B, Hq, Hkv, L, D, W = 3, 64, 8, 262144, 128, 513
    scale = D ** -0.5
    g = torch.Generator(device="cuda")
    g.manual_seed(5150)
    say("large forward: drawing inputs on the device")
    q, k, v = _randn(g, (B, Hq, L, D)), _randn(g, (B, Hkv, L, D)), _randn(g, (B, Hkv, L, D))
    rng = np.random.default_rng(5150)
    sinks = (rng.standard_normal(Hq) * 2.0).astype(np.float32)
    sinks[::4] = 30.0
    sd = torch.from_numpy(sinks).cuda()
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:3], device="cuda")
    say("large forward: running")
    A.attn_fwd(q, k, v, sd, out, lse, window=W, scale=scale)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for b, h in ((2, 63), (2, 0), (1, 37)):
        rows = sorted({0, 1, 511, 512, 513, 131071, 131072}
                      | set(range(L - 70, L))
                      | {int(x) for x in rng.integers(0, L, 40)})
        idx = torch.tensor(rows, device="cuda")
        say(f"large forward: b={b} h={h}, {len(rows)} rows")
        qs = _host(q[b:b + 1, h:h + 1])
        ks = _host(k[b:b + 1, h // G:h // G + 1])
        vs = _host(v[b:b + 1, h // G:h // G + 1])
        o_r, l_r = oracle.attention_rows(qs, ks, vs, sinks[h:h + 1], 0, 0, rows, W, scale)
        o = out[b, h].index_select(0, idx).float().cpu().numpy()
        l = lse[b, h].index_select(0, idx).cpu().numpy()
        compare(o, l, o_r, l_r, f"large forward b={b} h={h}", bf16_out=True)


@pytest.mark.timeout(900)
def test_decode_offsets_beyond_4g_elements(gpu):
    """Split-KV decode over a 128-sequence cache of 40000 keys (B128 Hq64 Hkv8
    D128): K and V hold 5.2e9 elements each; the last sequences' rows sit past
    2^32 elements.  1024 keys per split, as the benchmark's decode."""
    B, Hq, Hkv, Lmax, D = 128, 64, 8, 40000, 128
    scale = D ** -0.5
    g = torch.Generator(device="cuda")
    g.manual_seed(6160)
    say("large decode: drawing inputs on the device")
    q = _randn(g, (B, Hq, 1, D))
    kc, vc = _randn(g, (B, Hkv, Lmax, D)), _randn(g, (B, Hkv, Lmax, D))
    rng = np.random.default_rng(6160)
    seqlens = rng.integers(1024, Lmax, size=B, endpoint=True).astype(np.int32)
    seqlens[-1] = Lmax
    seqlens[64] = 1
    nsplits = np.minimum(-(-seqlens // 1024), 64).astype(np.int32)
    sinks = rng.standard_normal(Hq).astype(np.float32)
    sl = torch.from_numpy(seqlens).cuda()
    ns = torch.from_numpy(nsplits).cuda()
    sd = torch.from_numpy(sinks).cuda()
    op = torch.full((B, Hq, 64, D), float("nan"), device="cuda")
    lp = torch.full((B, Hq, 64), float("nan"), device="cuda")
    out = torch.empty((B, Hq, 1, D), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    say("large decode: running")
    A.attn_decode_splitkv(q, kc, vc, sl, ns, op, lp, window=0, scale=scale)
    A.attn_combine(op, lp, sl, ns, sd, out, lse, Lk_max=Lmax, window=0)
    torch.cuda.synchronize()
    for b in (127, 126, 64, 0):
        say(f"large decode: sequence {b} ({seqlens[b]} keys)")
        n = int(seqlens[b])
        o_r, l_r = oracle.decode(_host(q[b:b + 1]), _host(kc[b:b + 1, :, :n]), _host(vc[b:b + 1, :, :n]),
                                 seqlens[b:b + 1], sinks, 0, scale)
        compare(out[b:b + 1, :, 0].cpu().numpy(), lse[b:b + 1].cpu().numpy(), o_r, l_r,
                f"large decode b={b}")
        nv = oracle.decode_partials(_host(q[b:b + 1]), _host(kc[b:b + 1, :, :n]), _host(vc[b:b + 1, :, :n]),
                                    seqlens[b:b + 1], nsplits[b:b + 1], 0, scale)[2]
        assert torch.isnan(op[b, :, int(nv[0]):]).all(), f"large decode b={b}: lane >= n_valid written"


@pytest.mark.timeout(900)
def test_backward_offsets_beyond_4g_elements(gpu):
    """Backward of two long sliding-window sequences (B2 Hq64 Hkv8 L262144
    D128, window 513, bf16 O): q, dO and O hold 4.3e9 elements, dQ 17 GB of
    fp32.  dK/dV of 64-key blocks of the second sequence (every row that sees
    them, all heads of the KV head) and dQ of those rows, against the oracle on
    the slice of rows and keys that decides them exactly."""
    from test_bwd_gpu import check_bwd

    B, Hq, Hkv, L, D, W = 2, 64, 8, 262144, 128, 513
    scale = D ** -0.5
    g = torch.Generator(device="cuda")
    g.manual_seed(7170)
    say("large backward: drawing inputs on the device")
    q, k, v = _randn(g, (B, Hq, L, D)), _randn(g, (B, Hkv, L, D)), _randn(g, (B, Hkv, L, D))
    dout = _randn(g, (B, Hq, L, D))
    rng = np.random.default_rng(7170)
    sinks = (rng.standard_normal(Hq) * 2.0).astype(np.float32)
    sinks[::4] = 30.0
    sd = torch.from_numpy(sinks).cuda()
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:3], device="cuda")
    say("large backward: forward")
    A.attn_fwd(q, k, v, sd, out, lse, window=W, scale=scale)
    dq = torch.full(q.shape, float("nan"), device="cuda")
    dk = torch.full(k.shape, float("nan"), device="cuda")
    dv = torch.full(k.shape, float("nan"), device="cuda")
    ds = torch.full(sd.shape, float("nan"), device="cuda")
    say("large backward: running")
    A.attn_bwd(q, k, v, sd, out, dout, lse, dq, dk, dv, ds, window=W, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(ds).all(), "large backward: non-finite dsink"
    G = Hq // Hkv
    b = 1
    for kvh, k0 in ((7, L - 64), (4, 131072), (0, 0)):
        say(f"large backward: b={b} kvh={kvh} keys {k0}..{k0 + 63}")
        r_a, r_b = k0, min(L, k0 + 64 + W - 1)
        c_a = max(0, r_a - W + 1)
        heads = slice(kvh * G, (kvh + 1) * G)
        kv = slice(kvh, kvh + 1)
        want = oracle.attention_bwd(_host(q[b:b + 1, heads, r_a:r_b]), _host(k[b:b + 1, kv, c_a:r_b]),
                                    _host(v[b:b + 1, kv, c_a:r_b]), sinks[heads],
                                    _host(dout[b:b + 1, heads, r_a:r_b]), W, scale)
        got = (dq[b:b + 1, heads, r_a:r_b].cpu().numpy(), dk[b:b + 1, kv, k0:k0 + 64].cpu().numpy(),
               dv[b:b + 1, kv, k0:k0 + 64].cpu().numpy(), None)
        ref = (want[0], want[1][:, :, k0 - c_a:k0 - c_a + 64], want[2][:, :, k0 - c_a:k0 - c_a + 64], None)
        check_bwd(got, ref, f"large backward b={b} kvh={kvh} keys {k0}..{k0 + 63}")


@pytest.mark.timeout(900)
def test_paged_decode_offsets_beyond_4g_elements(gpu):
    """Paged split-KV decode over a pool of 16-key pages holding 6.4e9 elements
    per K and V (B128 Hq64 Hkv8 D128, 32768..65536 keys per sequence, pages
    shuffled over the pool): sampled sequences, their pages gathered from the
    pool by the block table, against the oracle."""
    B, Hq, Hkv, D, P = 128, 64, 8, 128, 16
    Lmax = 65536
    scale = D ** -0.5
    rng = np.random.default_rng(8180)
    seqlens = rng.integers(32768, Lmax, size=B, endpoint=True).astype(np.int32)
    need = -(-seqlens // P)
    total = int(need.sum())
    perm = rng.permutation(total).astype(np.int32)
    mp = Lmax // P
    table = np.full((B, mp), -1, dtype=np.int32)  # unused slots: never read
    cu = np.concatenate([[0], np.cumsum(need)])
    for b in range(B):
        table[b, :need[b]] = perm[cu[b]:cu[b + 1]]
    nsplits = np.minimum(-(-seqlens // 1024), 64).astype(np.int32)
    sinks = rng.standard_normal(Hq).astype(np.float32)
    g = torch.Generator(device="cuda")
    g.manual_seed(8180)
    say(f"large paged decode: drawing {total} pages on the device")
    q = _randn(g, (B, Hq, 1, D))
    kp, vp = _randn(g, (total, Hkv, P, D)), _randn(g, (total, Hkv, P, D))
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(seqlens).cuda()
    ns = torch.from_numpy(nsplits).cuda()
    sd = torch.from_numpy(sinks).cuda()
    op = torch.full((B, Hq, 64, D), float("nan"), device="cuda")
    lp = torch.full((B, Hq, 64), float("nan"), device="cuda")
    out = torch.empty((B, Hq, 1, D), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    say("large paged decode: running")
    A.attn_decode_splitkv_paged(q, kp, vp, bt, sl, ns, op, lp, window=0, scale=scale)
    A.attn_combine(op, lp, sl, ns, sd, out, lse, Lk_max=mp * P, window=0)
    torch.cuda.synchronize()
    high = int(np.argmax([table[b, :need[b]].max() for b in range(B)]))
    for b in sorted({0, 77, B - 1, high}):
        n = int(seqlens[b])
        say(f"large paged decode: sequence {b} ({n} keys, highest page {int(table[b, :need[b]].max())})")
        pages = bt[b, :need[b]].long()
        gather = lambda pool: pool[pages].permute(1, 0, 2, 3).reshape(Hkv, -1, D)[:, :n]
        o_r, l_r = oracle.decode(_host(q[b:b + 1]), _host(gather(kp))[None], _host(gather(vp))[None],
                                 seqlens[b:b + 1], sinks, 0, scale)
        compare(out[b:b + 1, :, 0].cpu().numpy(), lse[b:b + 1].cpu().numpy(), o_r, l_r,
                f"large paged decode b={b}")
