"""CPU checks of the seeded input generators (no GPU)."""

import numpy as np
import torch

import oracle
from exact_attention_attn_amd import workloads as W


def test_bf16_encoding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, 65504.0], np.float32)])
    bits = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = W.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_streams_are_per_slice_and_reproducible():
    a = W.normal_tensor((2, 3, 16, 8), W.BF16, 9, W.T_Q)
    b = W.normal_tensor((2, 3, 16, 8), W.BF16, 9, W.T_Q)
    assert np.array_equal(a, b)
    c = W.normal_tensor((1, 1, 16, 8), W.BF16, 9, W.T_Q)
    assert np.array_equal(a[0, 0], c[0, 0])
    # shorter draws are prefixes of the same stream
    d = W.normal_tensor((2, 3, 10, 8), W.BF16, 9, W.T_Q)
    assert np.array_equal(a[:, :, :10], d)


def test_pairs_formula_counts_visible_keys():
    for w in (W.TINY_PREFILL, W.SWA_PREFILL, W.CAUSAL_PREFILL):
        L = 700
        Wd = w.window
        n = sum(oracle.visible_range(i, L, Wd)[1] - oracle.visible_range(i, L, Wd)[0] for i in range(L))
        small = W.Prefill(w.name, 1, 1, 1, L, w.D, w.dtype, Wd, 1, 0, 0, 1)
        assert small.pairs() == n
    assert W.SWA_PREFILL.flops() == 133_404_033_024
    assert W.CAUSAL_PREFILL.flops() == 4 * 128 * 4 * 32 * 4096 * 4097 // 2


def test_prefill_inputs_shapes_and_sinks():
    q, k, v, s = W.prefill_inputs(W.TINY_PREFILL)
    assert q.shape == (1, 2, 256, 64) and q.dtype == np.float32 and k.shape == (1, 1, 256, 64)
    assert s[1] == 100.0
    q, k, v, s = W.prefill_inputs(W.SWA_PREFILL, L=300)
    assert q.dtype == np.uint16 and q.shape == (1, 64, 300, 128)
    assert (s[::8] == 20.0).all() and (s[1::8] != 20.0).all()


def test_decode_inputs_poison_and_splits():
    q, k, v, seqlens, ns, s = W.decode_inputs(W.SPLITKV_DECODE, B=4, Lk_max=2048)
    assert ((seqlens >= 1024) & (seqlens <= 2048)).all()
    assert np.array_equal(ns, np.clip(-(-seqlens // W.SPLITKV_DECODE.keys_per_split), 1, 64))
    kf = W.bf16_bits_to_f32(k)
    for b in range(4):
        assert np.isnan(kf[b, :, seqlens[b]:]).all()
        assert np.isfinite(kf[b, :, :seqlens[b]]).all()
    _, _, _, _, ns2, _ = W.decode_inputs(W.SPLITKV_DECODE, B=8, Lk_max=2048, random_splits=True)
    assert ((ns2 >= 1) & (ns2 <= 64)).all()
