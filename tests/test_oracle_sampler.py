"""Pins for the oracle's sampler: closed forms, brute force, statistics,
published constants.  CPU only."""
import itertools
import math
import os

import numpy as np
import pytest

from oracle import philox, sampler as smp
from oracle.numerics import entropy_direct

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        assert r[0] == "10"
        c0, c1, c2, c3, k0, k1 = (int(x, 16) for x in r[1:7])
        want = tuple(int(x, 16) for x in r[7:11])
        got = philox.philox4x32_10(c0, c1, c2, c3, k0, k1)
        assert tuple(int(g) for g in got) == want


def test_temperature_endpoints_and_monotone_in_budget():
    # docs table: linear 0.8 -> 0.4 over the budget; report Fig. 9: larger N, milder annealing
    for n in (2, 12, 48, 192):
        assert smp.temperature(0, n) == float(np.float32(0.8))
        assert smp.temperature(n - 1, n) == float(np.float32(0.4))
        taus = [smp.temperature(t, n) for t in range(n)]
        assert all(a > b for a, b in zip(taus, taus[1:]))
    assert smp.temperature(0, 1) == float(np.float32(0.8))
    dec = [smp.temperature(0, n) - smp.temperature(1, n) for n in (12, 48, 192)]
    assert dec[0] > dec[1] > dec[2]
    # linear: equal decrements up to fp32 rounding
    taus = np.array([smp.temperature(t, 48) for t in range(48)])
    assert np.allclose(np.diff(taus), -0.4 / 47, atol=1e-7)


def test_entropy_identity_and_special_cases():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 3, size=(16, 4096))
    for tau in (0.8, 0.4):
        p, H, g = smp.row_statistics(z, tau)
        a = z / tau
        m = a.max(1, keepdims=True)
        S = np.exp(a - m).sum(1)
        T = (np.exp(a - m) * (a - m)).sum(1)
        assert np.allclose(H, np.log(S) - T / S, rtol=0, atol=1e-10)
        assert np.allclose(p.sum(1), 1.0, atol=1e-12)
        assert (g == np.argmax(z, 1)).all()
    # tile-merge identity T' = e^{m-m'} (T + (m - m') S) for a split row
    a = z[0] / 0.8
    h1, h2 = a[:2048], a[2048:]
    def st(x, m):
        e = np.exp(x - m)
        return e.sum(), (e * (x - m)).sum()
    m1, m2 = h1.max(), h2.max()
    M = max(m1, m2)
    S1, T1 = st(h1, m1)
    S2, T2 = st(h2, m2)
    S = np.exp(m1 - M) * S1 + np.exp(m2 - M) * S2
    T = np.exp(m1 - M) * (T1 + (m1 - M) * S1) + np.exp(m2 - M) * (T2 + (m2 - M) * S2)
    Sd, Td = st(a, M)
    assert np.isclose(S, Sd, rtol=1e-12) and np.isclose(T, Td, rtol=1e-12)
    # equal logits -> ln V
    for V, want in ((4096, 8.3177662), (262144, 12.4766493)):
        _, H, _ = smp.row_statistics(np.zeros((1, V)), 0.8)
        assert abs(H[0] - want) < 1e-7
    # one logit dominant by 1000 -> ~0; two-way tie -> ln 2
    z = np.zeros((2, 4096))
    z[0, 17] = 1000.0
    z[1, 5] = z[1, 9] = 1000.0
    _, H, g = smp.row_statistics(z, 1.0)
    assert H[0] < 1e-12 and abs(H[1] - math.log(2)) < 1e-12
    assert g[1] == 5  # ties -> lowest id


def test_entropy_direct_matches_definition_small():
    p = np.array([[0.5, 0.25, 0.25, 0.0]])
    assert abs(entropy_direct(p)[0] - (0.5 * math.log(2) + 0.5 * math.log(4))) < 1e-15


def _brute_force_max_subset(H, bound):
    n = len(H)
    best = 0
    for r in range(n, 0, -1):
        for sub in itertools.combinations(range(n), r):
            if sum(H[i] for i in sub) <= bound:
                return r
    return best


@pytest.mark.parametrize("seed", range(12))
def test_accept_invariants_and_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = 12
    H = np.abs(rng.exponential(0.03 if seed % 2 else 0.2, size=n))
    if seed % 3 == 0:
        H[3] = H[7]  # entropy tie
    mask, K, order, _ = smp.accept_set(H, 0.1)
    assert mask.sum() == K >= 1
    assert mask[np.argmin(H)]  # argmin (lowest index on ties) always accepted
    if K > 1:
        assert H[mask].sum() <= 0.1
    best = _brute_force_max_subset(list(H), 0.1)
    assert K == max(best, 1)
    # accepted set = the K smallest (ties by index)
    assert set(np.nonzero(mask)[0]) == set(order[:K])


def test_accept_inclusive_bound_and_forced_single():
    H = np.array([0.05, 0.05, 0.5])
    mask, K, _, _ = smp.accept_set(H, 0.1)
    assert K == 2  # 0.05 + 0.05 == 0.1 is kept (inclusive)
    H = np.array([0.7, 0.3, 0.9])
    mask, K, _, _ = smp.accept_set(H, 0.1)
    assert K == 1 and mask[1]


def test_renoise_is_philox_stream1_and_uniform():
    seed, t, b, V = 1234567, 5, 2, 4096
    tok = smp.renoise_tokens(seed, t, b, 256, V)
    w0, _, _, _ = philox.philox4x32_10(np.arange(256), t, b, 1, seed & 0xFFFFFFFF, seed >> 32)
    assert (tok == (w0.astype(np.uint64) >> np.uint64(20)).astype(np.int64)).all()
    # chi-square uniformity over 10^6 draws (many seeds, positions)
    n = 1 << 20
    pos = np.arange(n) % 256
    steps = np.arange(n) // 256
    w0, _, _, _ = philox.philox4x32_10(pos, steps, 0, 1, 99, 0)
    toks = philox.word_to_token(w0, V)
    cnt = np.bincount(toks, minlength=V)
    exp = n / V
    chi2 = ((cnt - exp) ** 2 / exp).sum()
    from scipy.stats import chi2 as c2
    assert c2.sf(chi2, V - 1) > 1e-3


def test_renoise_independent_of_logits():
    rng = np.random.default_rng(0)
    z1 = rng.normal(0, 1, (64, 4096))
    z2 = rng.normal(0, 5, (64, 4096))
    o1 = smp.sample_from_logits(z1, 3, 48, 7, 0)
    o2 = smp.sample_from_logits(z2, 3, 48, 7, 0)
    fresh = smp.renoise_tokens(7, 3, 0, 64, 4096)
    for o in (o1, o2):
        rej = ~o["accepted"]
        assert (o["next_tokens"][rej] == fresh[rej]).all()
        assert (o["next_tokens"][o["accepted"]] == o["sample"][o["accepted"]]).all()


def test_tile_sampling_exact_distribution_on_grid():
    # The two-level draw with 24-bit uniforms induces P(v) that differs from p_v
    # only by the grid quantisation: count the u1 and u2 grid points exactly.
    rng = np.random.default_rng(3)
    z = rng.normal(0, 1, (1, 8))
    p, _, _ = smp.row_statistics(z, 1.0)
    p = p[0]
    tile = 4
    Z = p.reshape(2, 4).sum(1)
    cz = np.cumsum(Z)
    grid = 2 ** 24
    u = np.arange(grid, dtype=np.float64) / grid
    k_of_u = np.searchsorted(cz, u, side="right")  # first k with cz > u
    k_of_u = np.minimum(k_of_u, 1)
    pk = np.bincount(k_of_u, minlength=2) / grid
    probs = np.zeros(8)
    for k in range(2):
        cin = np.cumsum(p[k * tile:(k + 1) * tile])
        v_of_u = np.minimum(np.searchsorted(cin, u * Z[k], side="right"), tile - 1)
        pv = np.bincount(v_of_u, minlength=tile) / grid
        probs[k * tile:(k + 1) * tile] = pk[k] * pv
    assert np.max(np.abs(probs - p)) < 4.0 / grid
    # and the oracle function agrees with the grid map on sampled u's
    u1 = u[::65537][:200]
    u2 = u[::40009][:200]
    s, _ = smp.categorical_tiles(np.tile(p, (200, 1)), u1, u2, tile=tile)
    for i in range(200):
        k = min(int(np.searchsorted(cz, u1[i], side="right")), 1)
        cin = np.cumsum(p[k * tile:(k + 1) * tile])
        v = min(int(np.searchsorted(cin, u2[i] * Z[k], side="right")), tile - 1)
        assert s[i] == k * tile + v


def test_tile_sampling_chi_square_and_one_hot():
    rng = np.random.default_rng(5)
    z = rng.normal(0, 1, 8)
    p = np.exp(z) / np.exp(z).sum()
    n = 1 << 20
    w0, w1, _, _ = philox.philox4x32_10(np.arange(n) % 4096, np.arange(n) // 4096, 0, 2, 11, 0)
    u1, u2 = philox.word_to_unit(w0), philox.word_to_unit(w1)
    # vectorised two-level draw for the toy (V = 8, tile 4)
    Z = p.reshape(2, 4).sum(1)
    k = np.minimum(np.searchsorted(np.cumsum(Z), u1, side="right"), 1)
    cin = np.stack([np.cumsum(p[:4]), np.cumsum(p[4:])])
    v = np.array([min(int(np.searchsorted(cin[kk], uu * Z[kk], side="right")), 3)
                  for kk, uu in zip(k[:20000], u2[:20000])])
    s = k[:20000] * 4 + v
    cnt = np.bincount(s, minlength=8)
    exp = p * len(s)
    chi2 = ((cnt - exp) ** 2 / exp).sum()
    from scipy.stats import chi2 as c2
    assert c2.sf(chi2, 7) > 1e-3
    one = np.zeros((3, 512))
    one[:, 300] = 1.0
    s, _ = smp.categorical_tiles(one, np.array([0.0, 0.5, 0.999]), np.array([0.999, 0.0, 0.5]))
    assert (s == 300).all()


def test_stop_truth_table():
    H_lo = np.full(8, 0.001)
    H_hi = np.full(8, 0.01)
    g = np.arange(8)
    g2 = g.copy()
    g2[3] = 99
    assert smp.stop_test(H_lo, g, g, 3, True)[0]
    assert not smp.stop_test(H_lo, g, g2, 3, True)[0]    # low H, argmax changed
    assert not smp.stop_test(H_hi, g, g, 3, True)[0]     # same argmax, H >= threshold
    assert not smp.stop_test(H_lo, g, None, 0, True)[0]  # t = 0
    assert not smp.stop_test(H_lo, g, g, 3, False)[0]    # fixed-step run
    Hb = np.full(8, 0.005)
    assert not smp.stop_test(Hb, g, g, 3, True)[0]       # strict


def test_initial_canvas_stream0():
    tok = smp.initial_canvas(42, 3, 256, 262144)
    w0, _, _, _ = philox.philox4x32_10(np.arange(256), 0, 3, 0, 42, 0)
    assert (tok == (w0.astype(np.uint64) >> np.uint64(14)).astype(np.int64)).all()


def test_full30_lm_scale_gives_about_20_accepted_per_step():
    """The 30-layer workload's LM-head scale: with iid normal logits of
    standard deviation s * 0.02 * sqrt(d_model) (an untied random head and a
    unit-RMS hidden state), the oracle's acceptance rule takes about 20 tokens
    per step on average over the 12 temperatures of the run.  (Positions of
    one canvas have correlated hidden states, so the model itself accepts a
    few fewer than independent positions would: 19-20 at this scale.)"""
    import os
    import sys
    from synth.configs import WORKLOADS
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    from calibrate_lm_scale import mean_accepted
    wl = WORKLOADS["full30"]
    m = mean_accepted(wl.lm_scale, d_model=wl.model.d_model, vocab=wl.model.vocab, canvas=wl.canvas,
                      n_steps=wl.n_steps, seed=1)
    assert 15.0 <= m <= 30.0, m
