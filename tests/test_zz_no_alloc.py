"""attn_decode_noalloc (decode + combine with the library's fixed split
workspace) against attn_decode_splitkv + attn_combine on caller-owned
workspace: the same kernels, so the same bits; and against the oracle.

Two calls in a row, the second smaller (the scratch keeps the first call's
contents; the second must read only what it wrote), then a third on the first
shape again with other split counts.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_attention_attn_amd as A
import oracle
from exact_attention_attn_amd import workloads as W

gpu_util = pytest.importorskip("gpu_util")
from gpu_util import compare, host_values, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, D, Lk_max, seed, ns_max, window):
    rng = np.random.default_rng(seed)
    seqlens = rng.integers(1, Lk_max, size=B, endpoint=True).astype(np.int32)
    seqlens[0] = Lk_max
    nsplits = rng.integers(1, ns_max, size=B, endpoint=True).astype(np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, Hq, 1, D), dtype=np.float32))
    kc = W.normal_tensor((B, Hkv, Lk_max, D), W.BF16, seed, 1, lengths=seqlens)
    vc = W.normal_tensor((B, Hkv, Lk_max, D), W.BF16, seed, 2, lengths=seqlens)
    sinks = rng.standard_normal(Hq).astype(np.float32)
    sinks[0] = 20.0
    return q, kc, vc, seqlens, nsplits, sinks, window


def _run_both(q, kc, vc, seqlens, nsplits, sinks, window, max_splits, out_dtype):
    B, Hq, _, D = q.shape
    qd, kd, vd = to_dev(q, W.BF16), to_dev(kc, W.BF16), to_dev(vc, W.BF16)
    sl = torch.from_numpy(seqlens).cuda()
    ns = torch.from_numpy(nsplits).cuda()
    sd = torch.from_numpy(sinks).cuda()
    scale = D ** -0.5
    # existing entry points on caller-owned workspace
    op = torch.full((B, Hq, max_splits, D), float("nan"), dtype=torch.float32, device="cuda")
    lp = torch.full((B, Hq, max_splits), float("nan"), dtype=torch.float32, device="cuda")
    out_ref = torch.full((B, Hq, 1, D), float("nan"), dtype=out_dtype, device="cuda")
    lse_ref = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    A.attn_decode_splitkv(qd, kd, vd, sl, ns, op, lp, window=window, scale=scale)
    A.attn_combine(op, lp, sl, ns, sd, out_ref, lse_ref, Lk_max=kc.shape[2], window=window)
    # the allocation-free call
    out = torch.full((B, Hq, 1, D), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    A.attn_decode_noalloc(qd, kd, vd, sl, ns, sd, out, lse, max_splits=max_splits, window=window,
                          scale=scale)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy()[:, :, 0], lse.cpu().numpy(),
            out_ref.float().cpu().numpy()[:, :, 0], lse_ref.cpu().numpy())


def _check(case, max_splits, out_dtype, what):
    q, kc, vc, seqlens, nsplits, sinks, window = case
    say(f"no-alloc decode {what}: B={q.shape[0]} Hq={q.shape[1]} D={q.shape[3]} "
        f"Lk_max={kc.shape[2]} max_splits={max_splits}")
    o, l, o_ref, l_ref = _run_both(q, kc, vc, seqlens, nsplits, sinks, window, max_splits, out_dtype)
    assert np.array_equal(o, o_ref), f"{what}: O differs from decode + combine"
    assert np.array_equal(l, l_ref), f"{what}: LSE differs from decode + combine"
    D = q.shape[3]
    ou, lu = oracle.decode(*(host_values(x, W.BF16) for x in (q, kc, vc)), seqlens, sinks, window,
                           D ** -0.5)
    compare(o, l, ou, lu, f"no-alloc {what} vs oracle", bf16_out=out_dtype == torch.bfloat16)


def test_noalloc_matches_decode_and_combine(gpu):
    big = _case(B=24, Hq=32, Hkv=4, D=128, Lk_max=5000, seed=31, ns_max=64, window=0)
    small = _case(B=3, Hq=8, Hkv=1, D=64, Lk_max=700, seed=32, ns_max=8, window=513)
    _check(big, 64, torch.float32, "first call")
    _check(small, 8, torch.bfloat16, "second, smaller call")
    q, kc, vc, seqlens, nsplits, sinks, window = big
    again = (q, kc, vc, seqlens, np.maximum(nsplits // 2, 1).astype(np.int32), sinks, window)
    _check(again, 64, torch.float32, "third call, first shape, other splits")


def test_noalloc_rejects_oversize_workspace(gpu):
    # 65 x 64 x 64 lanes at D = 128 need more than the fixed scratch holds
    q = torch.zeros((65, 64, 1, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((65, 8, 64, 128), dtype=torch.bfloat16, device="cuda")
    sl = torch.full((65,), 64, dtype=torch.int32, device="cuda")
    out = torch.empty((65, 64, 1, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(A.AttnError) as e:
        A.attn_decode_noalloc(q, kc, kc, sl, sl, None, out, max_splits=64)
    assert e.value.code == 6
