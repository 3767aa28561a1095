"""GPU checks of attn_decode_plan: the split counts written on the device are
exactly the oracle's (integer work, bit-exact), and a decode run with the
planned counts matches the oracle attention."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_attention_attn_amd as A
import oracle
from exact_attention_attn_amd import workloads as W

gpu_util = pytest.importorskip("gpu_util")
from gpu_util import say  # noqa: E402
from test_parity_gpu import check_decode  # noqa: E402

pytestmark = pytest.mark.gpu


def device_plan(seqlens, Hq, Hkv, Lk_max, window, max_splits, policy, param):
    sl = torch.from_numpy(np.asarray(seqlens, np.int32)).cuda()
    ns = torch.full((len(seqlens),), -7, dtype=torch.int32, device="cuda")
    A.attn_decode_plan(sl, ns, Hq=Hq, Hkv=Hkv, Lk_max=Lk_max, max_splits=max_splits,
                       window=window, policy=policy, param=param)
    torch.cuda.synchronize()
    return ns.cpu().numpy().tolist()


def decode_slots():
    return torch.cuda.get_device_properties(0).multi_processor_count


SHAPES = [  # (B, Lk_max, window, Hq, Hkv, max_splits)
    (64, 32768, 0, 64, 8, 64), (4, 32768, 0, 64, 8, 64), (256, 2048, 0, 64, 8, 64),
    (64, 32768, 513, 64, 8, 64), (1, 131072, 0, 64, 8, 64), (1000, 5000, 0, 32, 8, 17),
    (7, 9000, 1000, 40, 1, 64), (3000, 300, 0, 128, 2, 1),
]


@pytest.mark.parametrize("B,Lk_max,window,Hq,Hkv,max_splits", SHAPES)
def test_plan_matches_oracle(gpu, B, Lk_max, window, Hq, Hkv, max_splits):
    rng = np.random.default_rng(B + Lk_max)
    seqlens = rng.integers(-10, Lk_max + 500, B).tolist()
    say(f"plan B={B} Lk_max={Lk_max} W={window} H={Hq}/{Hkv} ms={max_splits}")
    cases = [("auto", 0, decode_slots()), ("auto", 77, 77), ("auto", 512, 512),
             ("auto", 2**31 - 1, 2**31 - 1), ("keys", 1, 0),
             ("keys", 100, 0), ("keys", 1024, 0), ("count", 1, 0), ("count", 5, 0), ("count", 100, 0)]
    for policy, param, slots in cases:
        got = device_plan(seqlens, Hq, Hkv, Lk_max, window, max_splits, policy, param)
        want = oracle.plan_splits(seqlens, Hq, Hkv, Lk_max, window, max_splits, policy, param,
                                  max(slots, 1))
        assert got == want, f"{policy}({param}): {sum(g != w for g, w in zip(got, want))} differ"


def test_decode_with_auto_plan(gpu):
    w = W.SPLITKV_DECODE
    q, kc, vc, seqlens, _, s = W.decode_inputs(w, B=12, Lk_max=4096)
    seqlens[:4] = [1, 63, 64, 65]
    ns = device_plan(seqlens, w.Hq, w.Hkv, 4096, 0, 64, "auto", 0)
    assert ns == oracle.plan_splits(seqlens, w.Hq, w.Hkv, 4096, 0, 64, "auto", 0, decode_slots())
    say(f"decode with auto plan: {ns}")
    check_decode(q, kc, vc, seqlens, np.array(ns, np.int32), s, 0, "decode auto plan")
