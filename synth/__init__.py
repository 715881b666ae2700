"""Seeded synthetic K/V tensors shaped like the workloads the CacheGen pages evaluate.

The pages measure on real KV caches of Llama-7B / Mistral-7B / Llama-34B / Llama-70B
contexts drawn from LongChat, TriviaQA and NarrativeQA (CacheGen blog, section 3.1,
experiment setup and metrics; gptget summary, experiment design).  None of those weights or datasets
exist here, so every tensor is synthetic: per (kv, layer) an AR(1) process over
tokens (token-wise locality, the property the method exploits — sciencestack TL;DR
and CacheGen blog section 1) times a lognormal per-channel scale, with a few
outlier channels.

This module holds no arithmetic of the codec.  It is the only code shared by the
oracle side and the GPU side: both receive the same fp16 arrays from it.

Recipe, per (kv, l) with ``rng = Generator(PCG64(SeedSequence([seed, kv, l])))``:

1. ``scale[c] = exp(0.5 * N(0,1))``                       (lognormal(0, 0.5))
2. ``perm = rng.permutation(C)[:round(f*C)]; scale[perm] *= 8``   (outliers)
3. ``x_0 = N(0,1) / sqrt(1 - rho^2)``                      (stationary start)
4. ``x_t = rho * x_{t-1} + N(0,1)``, noise drawn token-major [t, C] in float64
5. store ``float16(scale[c] * x_t[c])`` (numpy's round-to-nearest-even cast)
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "gen_row", "gen_kv", "layer_rhos",
           "quality_schedule"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    tokens: int
    channels: int
    seed: int
    rho: float                  # AR(1) coefficient (ignored when rho_range is set)
    outlier_frac: float
    chunk_tokens: int
    group_tokens: int
    layer_group_end: tuple      # exclusive ends of the shallow/medium/deep groups
    layer_step: tuple           # delta step per layer group, in channel-std units
    quality_mult: tuple = (1.0, 1.5, 2.5)   # H, M, L step multipliers
    qualities: tuple = (0,)     # qualities encoded (0=H, 1=M, 2=L)
    rho_range: Optional[tuple] = None       # per-layer rho ~ U(lo, hi) (long-context shape)
    decode_selection: Optional[tuple] = None  # per-chunk quality of the decoded selection
    streamed: bool = False

    @property
    def n_chunks(self) -> int:
        return -(-self.tokens // self.chunk_tokens)

    @property
    def elements(self) -> int:
        return 2 * self.layers * self.tokens * self.channels

    @property
    def quality_mask(self) -> int:
        m = 0
        for q in self.qualities:
            m |= 1 << q
        return m

    def selection(self):
        """Quality of every chunk in the decoded selection."""
        if self.decode_selection is not None:
            return tuple(self.decode_selection)
        if self.streamed:
            return tuple(int(v) for v in quality_schedule(self))
        return tuple([self.qualities[0]] * self.n_chunks)


def _proportional_groups(L: int):
    # shallow / medium / deep thirds scaled from the 32-layer split 10 / 20 / 32
    return (L * 10 // 32, L * 20 // 32, L)


WORKLOADS = {
    # Tiny: one layer group, step 0.5 std, one quality, one chunk.
    "tiny": Workload("tiny", 2, 64, 128, seed=0, rho=0.8, outlier_frac=0.0,
                     chunk_tokens=64, group_tokens=10, layer_group_end=(2,),
                     layer_step=(0.5,)),
    # Llama-7B shape, one 1536-token chunk, quality H.
    "llama7b": Workload("llama7b", 32, 1536, 4096, seed=1, rho=0.85, outlier_frac=0.02,
                        chunk_tokens=1536, group_tokens=10, layer_group_end=(10, 20, 32),
                        layer_step=(0.5, 1.0, 1.5)),
    # Mistral-7B GQA shape, 9K context, 6 chunks x {H,M,L}, decode H,M,L,H,M,L.
    "mistral7b_9k": Workload("mistral7b_9k", 32, 9216, 1024, seed=2, rho=0.85,
                             outlier_frac=0.02, chunk_tokens=1536, group_tokens=10,
                             layer_group_end=(10, 20, 32), layer_step=(0.5, 1.0, 1.5),
                             qualities=(0, 1, 2), decode_selection=(0, 1, 2, 0, 1, 2)),
    # Llama-34B GQA shape, 80K context, quality M, per-layer rho.
    "llama34b_80k": Workload("llama34b_80k", 48, 81920, 1024, seed=3, rho=0.85,
                             outlier_frac=0.02, chunk_tokens=1536, group_tokens=10,
                             layer_group_end=_proportional_groups(48),
                             layer_step=(0.5, 1.0, 1.5), qualities=(1,),
                             rho_range=(0.75, 0.92)),
    # Llama-70B GQA shape, 16K context streamed from pinned host memory, seeded schedule.
    "llama70b_16k": Workload("llama70b_16k", 80, 16384, 1024, seed=4, rho=0.85,
                             outlier_frac=0.03, chunk_tokens=1536, group_tokens=10,
                             layer_group_end=_proportional_groups(80),
                             layer_step=(0.5, 1.0, 1.5), qualities=(0, 1, 2),
                             streamed=True),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (smaller test shapes)."""
    w = WORKLOADS[name]
    return dataclasses.replace(w, **overrides) if overrides else w


def layer_rhos(w: Workload) -> np.ndarray:
    """AR(1) coefficient of every layer (shared by K and V)."""
    if w.rho_range is None:
        return np.full(w.layers, w.rho, dtype=np.float64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 1000])))
    lo, hi = w.rho_range
    return rng.uniform(lo, hi, w.layers)


def quality_schedule(w: Workload) -> np.ndarray:
    """Seeded per-chunk quality (0=H, 1=M, 2=L) of the streamed workload."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 2000])))
    return rng.integers(0, 3, w.n_chunks)


def gen_row(seed: int, kv: int, layer: int, tokens: int, channels: int, rho: float,
            outlier_frac: float, out: Optional[np.ndarray] = None,
            context: Optional[int] = None) -> np.ndarray:
    """One [tokens, channels] fp16 slice (kv, layer) of the synthetic cache.

    ``context`` draws the token sequence from its own stream,
    ``PCG64(SeedSequence([seed, kv, layer, context]))``, keeping the channel
    scales and outliers of ``seed``: another context of the same model."""
    from scipy.signal import lfilter
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, kv, layer])))
    scale = np.exp(0.5 * rng.standard_normal(channels))
    n_out = int(round(outlier_frac * channels))
    if n_out > 0:
        perm = rng.permutation(channels)[:n_out]
        scale[perm] *= 8.0
    if context is not None:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, kv, layer, context])))
    drive = np.empty((tokens, channels), dtype=np.float64)
    drive[0] = rng.standard_normal(channels) / math.sqrt(1.0 - rho * rho)
    if tokens > 1:
        drive[1:] = rng.standard_normal((tokens - 1, channels))
    # x_t = rho * x_{t-1} + e_t with x_0 = drive[0]
    x = lfilter([1.0], [1.0, -rho], drive, axis=0)
    x *= scale[None, :]
    if out is None:
        out = np.empty((tokens, channels), dtype=np.float16)
    out[...] = x.astype(np.float16)
    return out


def gen_kv(w: Workload, out_k: Optional[np.ndarray] = None,
           out_v: Optional[np.ndarray] = None, layers: Optional[Sequence[int]] = None,
           threads: Optional[int] = None, context: Optional[int] = None):
    """K and V, each [layers, tokens, channels] fp16, written into out_k / out_v if given.

    ``layers`` restricts generation to some layers (others are left untouched);
    ``context`` gives another context of the same model (see gen_row).
    Rows are generated in parallel; each row has its own seeded stream, so the
    result does not depend on the thread count.
    """
    L, T, C = w.layers, w.tokens, w.channels
    if out_k is None:
        out_k = np.empty((L, T, C), dtype=np.float16)
    if out_v is None:
        out_v = np.empty((L, T, C), dtype=np.float16)
    rhos = layer_rhos(w)
    todo = [(kv, l) for kv in (0, 1) for l in (range(L) if layers is None else layers)]
    outs = (out_k, out_v)

    def one(item):
        kv, l = item
        gen_row(w.seed, kv, l, T, C, float(rhos[l]), w.outlier_frac, out=outs[kv][l],
                context=context)

    n = threads or min(16, os.cpu_count() or 1)
    if n <= 1 or len(todo) <= 1:
        for it in todo:
            one(it)
    else:
        with _cf.ThreadPoolExecutor(n) as ex:
            list(ex.map(one, todo))
    return out_k, out_v
