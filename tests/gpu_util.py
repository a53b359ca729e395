"""Helpers shared by the GPU parity tests: build the same seeded problem for
the HIP path (through the C ABI) and for the oracle, and compare decisions
with near-tie reporting."""
from __future__ import annotations

import sys

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_cuda():
    import torch
    return torch


def to_np(t):
    torch = torch_cuda()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def compare_decisions(name, gpu, ora, margin, eps, max_ties=0):
    """Equal everywhere except where the oracle's margin for that decision is
    below eps (a near-tie, where either answer is valid).  Returns the number
    of near-tie mismatches; fails on any other mismatch."""
    gpu = np.asarray(gpu)
    ora = np.asarray(ora)
    bad = np.nonzero(gpu != ora)[0]
    if bad.size == 0:
        return 0
    m = np.asarray(margin)
    m = m[bad] if m.ndim else np.full(bad.size, float(m))
    hard = bad[m >= eps]
    assert hard.size == 0, (f"{name}: {hard.size} mismatches with margin >= {eps}: idx {hard[:8]} "
                            f"gpu {gpu[hard[:8]]} oracle {ora[hard[:8]]} margins {m[m >= eps][:8]}")
    assert bad.size <= max_ties, f"{name}: {bad.size} near-tie mismatches (allowed {max_ties})"
    say(f"{name}: {bad.size} near-tie mismatches (margins {m[:4]})")
    return int(bad.size)


def allclose_report(name, got, want, atol, rtol):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    lim = np.asarray(atol) + rtol * np.abs(want)
    worst = float(np.max(err - lim)) if err.size else 0.0
    say(f"{name}: max abs err {err.max():.3e}, max rel {np.max(err / (np.abs(want) + 1e-30)):.3e}, "
        f"worst margin to bound {worst:.3e}")
    assert np.all(err <= lim), f"{name}: {int(np.sum(err > lim))} elements outside atol={atol} rtol={rtol}"


def bar_or_twin(name, got, want, twin, atol, rtol, factor=2.0):
    """Parity against the oracle at full size.

    Within the elementwise bar |got - want| <= atol + rtol |want| everywhere,
    or, where the bar is tighter than what two correct fp32-accumulating
    evaluations of the same definition differ by on this problem (`twin` is
    the oracle evaluated with fp32 products and sums; bf16 rounding of the
    activations turns last-bit differences into whole-ulp ones and the layers
    amplify them), the GPU's error distribution must stay within `factor`
    times the twin's at the median, p99, p99.99 and max."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    twin = np.asarray(twin, dtype=np.float64)
    err = np.abs(got - want).reshape(-1)
    terr = np.abs(twin - want).reshape(-1)
    lim = (atol + rtol * np.abs(want)).reshape(-1)
    qs = (0.5, 0.99, 0.9999, 1.0)
    ge = np.quantile(err, qs) if err.size else np.zeros(4)
    te = np.quantile(terr, qs) if terr.size else np.zeros(4)
    out = int(np.sum(err > lim))
    say(f"{name}: gpu |err| median/p99/p99.99/max {ge[0]:.2e}/{ge[1]:.2e}/{ge[2]:.2e}/{ge[3]:.2e}; "
        f"fp32 twin {te[0]:.2e}/{te[1]:.2e}/{te[2]:.2e}/{te[3]:.2e}; outside the bar: gpu {out}, "
        f"twin {int(np.sum(terr > lim))}")
    if out == 0:
        return
    bad = [f"q{q}" for q, g, t in zip(qs, ge, te) if g > factor * max(t, 1e-12)]
    assert not bad, f"{name}: {out} elements outside the bar and beyond {factor}x the fp32 twin at {bad}"
