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
    bad, out = _twin_check(name, got, want, twin, atol, rtol, factor)
    assert not bad, f"{name}: {out} elements outside the bar and beyond {factor}x the fp32 twin at {bad}"
    return out


def _twin_check(name, got, want, twins, atol, rtol, factor):
    """(quantiles where the GPU exceeds factor x the twins' envelope, number
    of elements outside the bar).  twins: one fp32 evaluation or a list of
    them; the envelope is their largest error at each quantile."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if not isinstance(twins, (list, tuple)):
        twins = [twins]
    err = np.abs(got - want).reshape(-1)
    lim = (atol + rtol * np.abs(want)).reshape(-1)
    qs = (0.5, 0.99, 0.9999, 1.0)
    ge = np.quantile(err, qs) if err.size else np.zeros(4)
    te = np.zeros(4)
    t_out = 0
    for tw in twins:
        terr = np.abs(np.asarray(tw, dtype=np.float64) - want).reshape(-1)
        te = np.maximum(te, np.quantile(terr, qs) if terr.size else np.zeros(4))
        t_out = max(t_out, int(np.sum(terr > lim)))
    out = int(np.sum(err > lim))
    say(f"{name}: gpu |err| median/p99/p99.99/max {ge[0]:.2e}/{ge[1]:.2e}/{ge[2]:.2e}/{ge[3]:.2e}; "
        f"fp32 twin{'s' if len(twins) > 1 else ''} {te[0]:.2e}/{te[1]:.2e}/{te[2]:.2e}/{te[3]:.2e}; "
        f"outside the bar: gpu {out}, twin {t_out}")
    if out == 0:
        return [], 0
    return [f"q{q}" for q, g, t in zip(qs, ge, te) if g > factor * max(t, 1e-12)], out


def bar_then_twin(name, got, want, twin_fn, atol, rtol, factor=2.0):
    """bar_or_twin with the fp32 twin evaluated only when some element is
    outside the elementwise bar (twin_fn() returns it).  Returns the number
    of elements outside the bar."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    out = int(np.sum(err > atol + rtol * np.abs(want)))
    if out == 0:
        q = np.quantile(err.reshape(-1), (0.5, 0.99, 1.0)) if err.size else np.zeros(3)
        say(f"{name}: gpu |err| median/p99/max {q[0]:.2e}/{q[1]:.2e}/{q[2]:.2e}; all within the bar")
        return 0
    say(f"{name}: {out} of {err.size} elements outside the bar; evaluating the fp32 twin")
    first = twin_fn()
    bad, out = _twin_check(name, got, want, first, atol, rtol, factor)
    if bad:
        # one fp32 evaluation is one sample of how such evaluations drift: on a
        # small problem its error can be far below the typical one (when no
        # bf16 rounding boundary happens to be crossed in a canvas, bidirectional
        # attention keeps all its rows exact); a second evaluation, K summed
        # in reverse order, widens the sample
        from oracle import model as om
        say(f"{name}: beyond {factor}x the first twin at {bad}; evaluating the reverse-order twin")
        with om.twin_order("rev"):
            second = twin_fn()
        bad, out = _twin_check(name, got, want, [first, second], atol, rtol, factor)
    assert not bad, f"{name}: {out} elements outside the bar and beyond {factor}x the fp32 twins at {bad}"
    return out


def compare_step_decisions(name, z, H, am, acc, samp, nxt, stop, o, max_ties=4):
    """One canvas's step decisions from the GPU's own logits z [C, V] and
    entropies H [C] against the oracle's sampler output o on the same inputs.

    Each decision must be equal wherever the oracle's margin for it exceeds
    what the measured errors can move: argmax by twice the largest logit
    error; the accepted set by (K + 2) times the largest entropy error (K
    boundary sums of entropies, plus the gap across the boundary); the sample
    of a position accepted on both sides by the total variation between the
    two tempered distributions (the GPU's recomputed from its logits), which
    bounds the difference of the two CDFs.  Re-noised positions are equal
    (Philox stream 1), and so is the stop flag.  Returns the number of
    near-tie mismatches."""
    from oracle import sampler as smp
    z = np.asarray(z, dtype=np.float64)
    dz = float(np.abs(z - np.asarray(o["z"], dtype=np.float64)).max())  # o["z"]: the oracle's logits
    dH = float(np.abs(np.asarray(H, dtype=np.float64) - o["H"]).max())
    ties = compare_decisions(f"{name} argmax", am, o["argmax"], o["margin_argmax"], 2 * dz + 1e-6, max_ties)
    K = int(o["n_accepted"])
    ties += compare_decisions(f"{name} accepted", acc, o["accepted"], o["margin_accept"], (K + 2) * dH + 1e-6,
                              max_ties)
    pg, _, _ = smp.row_statistics(z, o["tau"])
    tv = float(np.abs(pg - o["p"]).sum(axis=1).max())
    both = acc & o["accepted"]
    ties += compare_decisions(f"{name} sample (accepted)", samp[both], o["sample"][both], o["margin_sample"][both],
                              tv + 1e-6, max_ties)
    same = acc == o["accepted"]
    assert np.array_equal(nxt[same & ~acc], o["next_tokens"][same & ~acc]), f"{name}: re-noised tokens differ"
    assert int(stop) == int(o["stop"]) or o["margin_stop"] < dH, f"{name}: stop flag differs"
    say(f"{name}: accepted {int(acc.sum())} (oracle {K}), max |dz| {dz:.2e}, max |dH| {dH:.2e}, "
        f"sample TV bound {tv:.2e}, near-tie decisions {ties}")
    return ties


def entropy_check(name, H, z_gpu, z_oracle, H_oracle, tau, frac_literal=0.99):
    """Device entropies against the oracle's: every position within 1e-3
    nats or, where its logits differ (within the logit bar), within the
    first-order change those measured differences cause,
    |dH| <= sum_v p_v |a_v - E_p a| |da_v| (a = z / tau), with 50% slack
    plus the second-order term max|da|^2 and 1e-5 for the fp32 statistics;
    and at least frac_literal of the positions within the literal 1e-3.
    Returns the number of positions beyond 1e-3."""
    from oracle import sampler as smp
    zo = np.asarray(z_oracle, dtype=np.float64)
    da = (np.asarray(z_gpu, dtype=np.float64) - zo) / tau
    p, _, _ = smp.row_statistics(zo, tau)
    a = zo / tau
    abar = (p * a).sum(-1, keepdims=True)
    first = (p * np.abs(a - abar) * np.abs(da)).sum(-1)
    bound = np.maximum(1e-3, 1.5 * first + np.max(da * da, axis=-1) + 1e-5)
    err = np.abs(np.asarray(H, dtype=np.float64) - np.asarray(H_oracle, dtype=np.float64))
    beyond = int(np.sum(err > 1e-3))
    i = int(np.argmax(err))
    say(f"{name}: max |dH| {err.max():.3e} (its logit-propagated bound {bound[i]:.3e}); {beyond} of {err.size} "
        f"positions beyond 1e-3 nats")
    assert np.all(err <= bound), f"{name}: {int(np.sum(err > bound))} positions beyond the propagated bound"
    assert beyond <= (1.0 - frac_literal) * err.size, f"{name}: {beyond} positions beyond 1e-3 nats"
    return beyond
