"""Entropy-bounded sampler, re-noise and adaptive stop (ORACLE — test infrastructure only).

Follows the sampler the DiffusionGemma pages describe:

* DiffusionGemma docs (ai.google.dev, Korean), table "recommended serving
  configuration": step budget 48; temperature linear from 0.8 to 0.4;
  adaptive early stop when the canvas-mean entropy is under 0.005 and two
  consecutive denoiser predictions agree; token selection keeps the
  lowest-entropy tokens while the summed ("mutual-information") bound stays
  under the entropy bound 0.1, and fully re-noises the tokens not selected.
* euno.news (from VentureBeat), "what DiffusionGemma does": the canvas starts
  as 256 random placeholder tokens; every step scores all positions, keeps
  the confident ones and re-randomises the rest, so earlier choices can be
  revised.
* DiffusionGemma Technical Report digest (METAL MEDIA), Figure 3: the noise
  end of the discrete diffusion path is the uniform distribution over tokens;
  Figure 9: a larger step budget gives milder annealing.

Where the pages leave a step open, the reading taken is stated at the
function that implements it.  All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np

from . import philox
from .numerics import entropy_direct

TAU_START = 0.8
TAU_END = 0.4
ENTROPY_BOUND = 0.1
STOP_THRESHOLD = 0.005
TILE_V = 256  # vocabulary tile of the two-level categorical sample


def temperature(t: int, n_steps: int) -> float:
    """Linear schedule over the step budget (not over the steps actually taken).

    tau_t = 0.8 + (0.4 - 0.8) * t / (N - 1), evaluated in fp64 and rounded once
    to fp32 (so both ends are exact: 0.8f and 0.4f); tau = 0.8 when N = 1."""
    if n_steps <= 1:
        tau = TAU_START
    else:
        tau = TAU_START + (TAU_END - TAU_START) * (t / (n_steps - 1))
    return float(np.float32(tau))


def initial_canvas(seed: int, block: int, canvas: int, vocab: int) -> np.ndarray:
    """Uniform random tokens from stream 0 with step field 0."""
    w0, _, _, _ = philox.words(seed, np.arange(canvas), 0, block, philox.STREAM_INIT)
    return philox.word_to_token(w0, vocab)


def renoise_tokens(seed: int, step: int, block: int, canvas: int, vocab: int) -> np.ndarray:
    """Fresh uniform tokens from stream 1 (all V ids, current token included)."""
    w0, _, _, _ = philox.words(seed, np.arange(canvas), step, block, philox.STREAM_RENOISE)
    return philox.word_to_token(w0, vocab)


def sample_uniforms(seed: int, step: int, block: int, canvas: int):
    """(u1, u2) per position from stream 2, words 0 and 1."""
    w0, w1, _, _ = philox.words(seed, np.arange(canvas), step, block, philox.STREAM_SAMPLE)
    return philox.word_to_unit(w0), philox.word_to_unit(w1)


def row_statistics(z: np.ndarray, tau: float):
    """Per-position tempered distribution, its entropy and the argmax.

    a = z / tau;  p = softmax(a);  H = -sum p ln p (direct);  g = argmax z with
    ties to the lowest id.  The entropy of the tempered distribution (the one
    the sampler draws from) drives both acceptance and the stop test."""
    z = np.asarray(z, dtype=np.float64)
    a = z / np.float64(tau)
    m = a.max(axis=-1, keepdims=True)
    e = np.exp(a - m)
    p = e / e.sum(axis=-1, keepdims=True)
    H = entropy_direct(p)
    g = np.argmax(z, axis=-1)  # first occurrence of the maximum
    return p, H, g


def categorical_tiles(p: np.ndarray, u1: np.ndarray, u2: np.ndarray, tile: int = TILE_V):
    """Exact categorical draw by tile composition, one row per position.

    The vocabulary is split into consecutive tiles of ``tile`` ids with masses
    Z_k.  The tile is the first k whose cumulative mass exceeds u1; inside it
    the token is the first v whose in-tile cumulative mass exceeds u2 * Z_k.
    Since u1 and u2 are independent, P(token = v) = p_v.  If rounding leaves
    no index passing a test, the last index with positive mass is taken.

    Returns (tokens, margins) where margins holds, per row, the distance of
    u1 and of u2*Z_k from the nearest cumulative boundary (for near-tie
    reporting)."""
    rows, V = p.shape
    n_t = V // tile
    pt = p.reshape(rows, n_t, tile)
    Z = pt.sum(axis=-1)                           # [rows, n_t]
    cz = np.cumsum(Z, axis=-1)
    out = np.empty(rows, dtype=np.int64)
    margin = np.empty(rows, dtype=np.float64)
    for r in range(rows):
        ks = np.nonzero(cz[r] > u1[r])[0]
        if ks.size:
            k = int(ks[0])
        else:
            k = int(np.nonzero(Z[r] > 0)[0][-1])
        cin = np.cumsum(pt[r, k])
        thr = u2[r] * Z[r, k]
        vs = np.nonzero(cin > thr)[0]
        if vs.size:
            v = int(vs[0])
        else:
            v = int(np.nonzero(pt[r, k] > 0)[0][-1])
        out[r] = k * tile + v
        m1 = np.min(np.abs(cz[r] - u1[r]))
        m2 = np.min(np.abs(cin - thr)) / max(Z[r, k], 1e-300)
        margin[r] = min(m1, m2)
    return out, margin


def accept_set(H: np.ndarray, bound: float = ENTROPY_BOUND):
    """Lowest-entropy positions whose summed entropy stays within the bound.

    Positions are ordered by (H ascending, index ascending); c_k is the sum of
    the first k entropies; the accepted count is the largest k with c_k <= bound
    (inclusive), and at least 1, so the single lowest-entropy position is always
    accepted.  The summed entropy of the accepted set is an upper bound on the
    mutual information among them, which is the bound the pages name.

    Returns (mask, K, order, margin) where margin is the distance of the
    boundary sums c_K and c_{K+1} from the bound, and the smallest entropy gap
    across the boundary (both matter to which set is chosen)."""
    H = np.asarray(H, dtype=np.float64)
    n = H.shape[0]
    order = np.lexsort((np.arange(n), H))
    c = np.concatenate([[0.0], np.cumsum(H[order])])  # c[k] = sum of first k
    ok = np.nonzero(c <= bound)[0]
    K = int(ok[-1]) if ok.size else 0
    K = max(K, 1)
    mask = np.zeros(n, dtype=bool)
    mask[order[:K]] = True
    margins = [abs(c[K] - bound)]
    if K < n:
        margins.append(abs(c[K + 1] - bound))
        margins.append(abs(H[order[K]] - H[order[K - 1]]))
    return mask, K, order, float(min(margins))


def stop_test(H: np.ndarray, g: np.ndarray, g_prev, t: int, adaptive: bool,
              threshold: float = STOP_THRESHOLD):
    """Stop when adaptive, t >= 1, the canvas-mean entropy is strictly under the
    threshold, and the argmax prediction equals the previous step's at every
    position.  Returns (stop, mean_H)."""
    mean_h = float(np.mean(H))
    same = g_prev is not None and bool(np.all(np.asarray(g) == np.asarray(g_prev)))
    return bool(adaptive and t >= 1 and mean_h < threshold and same), mean_h


def sample_from_logits(z, t, n_steps, seed, block, g_prev=None, adaptive=True,
                       bound=ENTROPY_BOUND, threshold=STOP_THRESHOLD):
    """The whole per-step sampler for one canvas from its logits z [C, V].

    Returns a dict with the tempered probabilities, entropies, argmax, sample,
    accepted mask and count, next canvas tokens, mean entropy, stop flag and
    the decision margins."""
    z = np.asarray(z, dtype=np.float64)
    C, V = z.shape
    tau = temperature(t, n_steps)
    p, H, g = row_statistics(z, tau)
    u1, u2 = sample_uniforms(seed, t, block, C)
    s, smargin = categorical_tiles(p, u1, u2)
    mask, K, order, amargin = accept_set(H, bound)
    fresh = renoise_tokens(seed, t, block, C, V)
    nxt = np.where(mask, s, fresh)
    stop, mean_h = stop_test(H, g, g_prev, t, adaptive, threshold)
    top2 = np.sort(z, axis=-1)[:, -2:]
    return {
        "tau": tau, "p": p, "H": H, "argmax": g, "sample": s, "accepted": mask,
        "n_accepted": K, "order": order, "next_tokens": nxt, "mean_H": mean_h, "stop": stop,
        "margin_sample": smargin, "margin_accept": amargin,
        "margin_argmax": top2[:, 1] - top2[:, 0], "margin_stop": abs(mean_h - threshold),
    }
