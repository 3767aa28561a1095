"""Seeded synthetic inputs for the attention workloads (no attention arithmetic here).

Both the HIP path's tests/bench and the float64 oracle read the arrays made
here; this module holds only random-number generation, bf16 encoding of the
draws, and the workload shapes.  Every slice (tensor, batch, head) has its own
counter-seeded stream ``default_rng([seed, tensor_id, b, h])``, so any slice
can be regenerated alone and large tensors are generated in parallel.

Workloads (shapes of the Flint model page: window 513, 262,144-token context,
and of the split-KV decode path):

====================  ==========================================================
tiny_prefill          B1 Hq2 Hkv1 L256 D64 fp32, window 513, head 1 sink = +100
swa_prefill           B1 Hq64 Hkv8 L8192 D128 bf16, window 513, sinks N(0, 2),
                      heads h % 8 == 0 forced to +20
causal_prefill        B4 Hq32 Hkv8 L4096 D128 bf16, causal, sinks N(0, 1)
splitkv_decode        B64 Hq64 Hkv8 Lq1 D128 bf16, Lk ~ U{1024..32768},
                      num_splits = clamp(ceil(Lk/1024), 1, 64), sinks N(0, 1),
                      cache rows >= Lk hold NaN
long_swa_prefill      B1 Hq64 Hkv8 L262144 D128 bf16, window 513, sinks N(0, 2),
                      heads h % 4 == 0 forced to +30
====================  ==========================================================
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BF16 = "bf16"
F32 = "f32"

T_Q, T_K, T_V, T_SINK, T_SEQ, T_SPLIT = range(6)

NAN_BF16 = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as bf16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns to the float32 values they represent (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    D: int
    dtype: str
    window: int           # <= 0: no window
    sink_std: float
    forced_every: int     # heads h % forced_every == 0 get forced_sink (0: none)
    forced_sink: float
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def pairs(self) -> int:
        """Unmasked (query, key) pairs: each row sees min(i+1, W) keys."""
        W = self.window if self.window > 0 else self.L
        L = self.L
        w = min(W, L)
        per_head = w * (w + 1) // 2 + (L - w) * w
        return per_head * self.B * self.Hq

    def flops(self) -> int:
        """Algorithmic flops: 2*D for q.k and 2*D for p.v per unmasked pair."""
        return 4 * self.D * self.pairs()


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lk_min: int
    Lk_max: int
    D: int
    dtype: str
    window: int
    sink_std: float
    keys_per_split: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


TINY_PREFILL = Prefill("tiny_prefill", 1, 2, 1, 256, 64, F32, 513, 1.0, 0, 0.0, 1)
SWA_PREFILL = Prefill("swa_prefill", 1, 64, 8, 8192, 128, BF16, 513, 2.0, 8, 20.0, 2)
CAUSAL_PREFILL = Prefill("causal_prefill", 4, 32, 8, 4096, 128, BF16, 0, 1.0, 0, 0.0, 3)
SPLITKV_DECODE = Decode("splitkv_decode", 64, 64, 8, 1024, 32768, 128, BF16, 0, 1.0, 1024, 4)
LONG_SWA_PREFILL = Prefill("long_swa_prefill", 1, 64, 8, 262144, 128, BF16, 513, 2.0, 4, 30.0, 5)

WORKLOADS = {w.name: w for w in (TINY_PREFILL, SWA_PREFILL, CAUSAL_PREFILL, SPLITKV_DECODE,
                                  LONG_SWA_PREFILL)}


def _rng(seed: int, tensor: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tensor, b, h])


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_tensor(shape, dtype: str, seed: int, tensor: int, std: float = 1.0,
                  lengths=None) -> np.ndarray:
    """[B, H, L, D] draws from N(0, std^2), one stream per (b, h) slice.

    Returns uint16 bf16 bit patterns for ``bf16`` and float32 for ``f32``.
    With ``lengths`` ([B] ints), slice (b, h) draws only its first lengths[b]
    rows; the rows after them hold NaN.
    """
    B, H, L, D = shape
    out = np.empty(shape, dtype=np.uint16 if dtype == BF16 else np.float32)

    def fill(bh):
        b, h = divmod(bh, H)
        n = L if lengths is None else max(0, min(L, int(lengths[b])))
        x = _rng(seed, tensor, b, h).standard_normal((n, D), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[b, h, :n] = f32_to_bf16_bits(x) if dtype == BF16 else x
        if n < L:
            out[b, h, n:] = NAN_BF16 if dtype == BF16 else np.float32(np.nan)

    n = B * H
    if n * L * D >= (1 << 22) and n > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n)))
    else:
        for bh in range(n):
            fill(bh)
    return out


def sinks_for(Hq: int, std: float, seed: int, forced_every: int = 0, forced: float = 0.0,
              forced_heads=()) -> np.ndarray:
    """Per-query-head sink logits ~ N(0, std^2) (float32), some heads forced."""
    s = _rng(seed, T_SINK).standard_normal(Hq, dtype=np.float32) * np.float32(std)
    if forced_every:
        s[::forced_every] = np.float32(forced)
    for h, val in forced_heads:
        s[h] = np.float32(val)
    return s.astype(np.float32)


def prefill_inputs(w: Prefill, L: int | None = None):
    """q [B,Hq,L,D], k, v [B,Hkv,L,D], sinks [Hq] for a prefill workload.

    ``L`` overrides the sequence length (same streams, shorter draw) for
    reduced-size parity runs.
    """
    L = w.L if L is None else L
    q = normal_tensor((w.B, w.Hq, L, w.D), w.dtype, w.seed, T_Q)
    k = normal_tensor((w.B, w.Hkv, L, w.D), w.dtype, w.seed, T_K)
    v = normal_tensor((w.B, w.Hkv, L, w.D), w.dtype, w.seed, T_V)
    if w.name == "tiny_prefill":
        sinks = sinks_for(w.Hq, w.sink_std, w.seed, forced_heads=[(1, 100.0)])
    else:
        sinks = sinks_for(w.Hq, w.sink_std, w.seed, w.forced_every, w.forced_sink)
    return q, k, v, sinks


def splits_policy(seqlens: np.ndarray, keys_per_split: int, max_splits: int = 64) -> np.ndarray:
    """num_splits per sequence: clamp(ceil(Lk / keys_per_split), 1, max_splits)."""
    ns = -(-np.asarray(seqlens, dtype=np.int64) // keys_per_split)
    return np.clip(ns, 1, max_splits).astype(np.int32)


def decode_inputs(w: Decode, B: int | None = None, Lk_max: int | None = None,
                  random_splits: bool = False, poison: bool = True):
    """q [B,Hq,1,D], k/v cache [B,Hkv,Lk_max,D], seqlens [B], num_splits [B], sinks [Hq].

    Cache rows at or beyond each sequence's length hold NaN (when ``poison``)
    so that a read of them shows in the output.
    """
    B = w.B if B is None else B
    Lk_max = w.Lk_max if Lk_max is None else Lk_max
    lo = min(w.Lk_min, Lk_max)
    seqlens = _rng(w.seed, T_SEQ).integers(lo, Lk_max, size=B, endpoint=True).astype(np.int32)
    if random_splits:
        num_splits = _rng(w.seed, T_SPLIT).integers(1, 64, size=B, endpoint=True).astype(np.int32)
    else:
        num_splits = splits_policy(seqlens, w.keys_per_split)
    q = normal_tensor((B, w.Hq, 1, w.D), w.dtype, w.seed, T_Q)
    k = normal_tensor((B, w.Hkv, Lk_max, w.D), w.dtype, w.seed, T_K, lengths=seqlens)
    v = normal_tensor((B, w.Hkv, Lk_max, w.D), w.dtype, w.seed, T_V, lengths=seqlens)
    if not poison:
        for b in range(B):
            k[b, :, seqlens[b]:] = 0
            v[b, :, seqlens[b]:] = 0
    sinks = sinks_for(w.Hq, w.sink_std, w.seed)
    return q, k, v, seqlens, num_splits, sinks


def as_float(x: np.ndarray, dtype: str) -> np.ndarray:
    """The float32 values an input array represents (bf16 bits decoded)."""
    return bf16_bits_to_f32(x) if dtype == BF16 else np.asarray(x, dtype=np.float32)
