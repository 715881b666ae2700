"""Seeded synthetic bandwidth traces and a link that follows them.

The pages test the adaptive streaming under a fluctuating link of about 3 Gbps
(CacheGen blog, section 2.2) without giving the traces.  Here a trace is a
piecewise-constant bandwidth, one value per step: log-bandwidth is an AR(1)
process around log(mean) so that the link has slow swings and quick dips,
clipped to a floor.  This module is input generation and simulation only: it
holds none of the codec's or the controller's arithmetic, and serves both the
oracle side and the library side.

Recipe, with ``rng = Generator(PCG64(SeedSequence([seed, 5000])))``:

1. ``z_0 = N(0,1) * sigma``, ``z_i = phi * z_{i-1} + sqrt(1 - phi^2) * sigma * N(0,1)``
2. ``gbps_i = max(floor_gbps, mean_gbps * exp(z_i - sigma^2 / 2))``
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["bandwidth_trace", "Link"]


def bandwidth_trace(seed: int, n_steps: int, mean_gbps: float = 3.0, sigma: float = 0.45,
                    phi: float = 0.9, floor_gbps: float = 0.2) -> np.ndarray:
    """Gbit/s per step (float64, n_steps values)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 5000])))
    eps = rng.standard_normal(n_steps)
    z = np.empty(n_steps)
    z[0] = eps[0] * sigma
    a = math.sqrt(1.0 - phi * phi) * sigma
    for i in range(1, n_steps):
        z[i] = phi * z[i - 1] + a * eps[i]
    return np.maximum(floor_gbps, mean_gbps * np.exp(z - 0.5 * sigma * sigma))


class Link:
    """A link whose bandwidth follows a trace (one value per step_ms), with a
    clock: send(nbytes) returns the milliseconds the transfer takes from the
    current time and advances the clock by that much."""

    def __init__(self, gbps: np.ndarray, step_ms: float, start_ms: float = 0.0):
        self.bpms = np.asarray(gbps, dtype=np.float64) * 1e9 / 8.0 / 1e3  # bytes per ms
        self.step_ms = float(step_ms)
        self.now = float(start_ms)

    def send(self, nbytes: int) -> float:
        left = float(nbytes)
        t = self.now
        while left > 0.0:
            i = int(t // self.step_ms)
            if i >= len(self.bpms):
                raise ValueError("transfer runs past the end of the trace")
            seg_end = (i + 1) * self.step_ms
            can = (seg_end - t) * self.bpms[i]
            if can >= left:
                t += left / self.bpms[i]
                left = 0.0
            else:
                left -= can
                t = seg_end
        dt = t - self.now
        self.now = t
        return dt
