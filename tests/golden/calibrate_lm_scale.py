"""LM-head scale of the 30-layer random-init workload (test infrastructure).

The workload fixes the LM-head scale s so that about 20 tokens are accepted
per denoising step on average over its fixed 12-step run.  With a random
untied head W (entries of standard deviation 0.02, independent of the hidden
state) and the RMS-normalised hidden state n (|n|^2 = d_model), the logits of
a position are z_v = s n.W_v: independent over v and normal with standard
deviation sigma = s * 0.02 * sqrt(d_model), whatever the canvas holds.  So the
acceptance count of a step depends only on sigma and the step's temperature,
and this script estimates it by drawing such logits and running the oracle's
own entropy and acceptance rule, then bisects s.

    python tests/golden/calibrate_lm_scale.py     # prints the scale
"""
from __future__ import annotations

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

from oracle import sampler as smp  # noqa: E402


def mean_accepted(scale: float, d_model: int = 2816, vocab: int = 262144, canvas: int = 256,
                  n_steps: int = 12, seed: int = 0, chunk: int = 32) -> float:
    """Mean accepted count per step over the n_steps temperatures."""
    rng = np.random.default_rng(seed)
    sigma = scale * 0.02 * np.sqrt(d_model)
    counts = []
    for t in range(n_steps):
        tau = smp.temperature(t, n_steps)
        H = np.empty(canvas)
        for r0 in range(0, canvas, chunk):
            z = rng.standard_normal((min(chunk, canvas - r0), vocab)) * sigma
            H[r0:r0 + z.shape[0]] = smp.row_statistics(z, tau)[1]
        counts.append(smp.accept_set(H)[1])
    return float(np.mean(counts))


def calibrate(target: float = 20.0, lo: float = 4.0, hi: float = 64.0, iters: int = 10) -> float:
    for _ in range(iters):
        mid = np.sqrt(lo * hi)
        if mean_accepted(mid) < target:
            lo = mid
        else:
            hi = mid
    return float(np.sqrt(lo * hi))


if __name__ == "__main__":
    s = calibrate()
    print(f"lm_scale {s:.3f}: mean accepted per step {mean_accepted(s):.2f}")
