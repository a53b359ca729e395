"""The three pipeline calls, composed from the model and the sampler
(ORACLE — test infrastructure only).

DiffusionGemma Technical Report digest (METAL MEDIA), Figure 4: (1) context
encoding by the causal encoder into the KV cache, (2) the denoising loop over
a noisy canvas, (3) encode & append of the finished canvas.  The LLM-Wiki
digest's key points add the block-autoregressive commit (the finished canvas
joins the history and the next block starts) and the self-conditioning
signal.

Readings: the encoder and the denoiser are the same weights with a different
canvas mask and no LM head; the committed tokens are the last step's argmax
(the stop rule certifies that prediction as stable); the canvas K, V of a
denoising step are transient and never written to the cache.
"""
from __future__ import annotations

import numpy as np

from synth.configs import ModelShape

from . import sampler as smp
from .model import KVCache, Weights, embed, final_logits, layer_forward


def encode_append(shape: ModelShape, W: Weights, cache: KVCache, tokens: np.ndarray,
                  trace: dict | None = None) -> None:
    """Causally encode tokens [B, n] at positions L..L+n-1 and append their K, V."""
    tokens = np.atleast_2d(np.asarray(tokens))
    n = tokens.shape[1]
    if cache.length + n > cache.capacity:
        raise ValueError("KV capacity exceeded")
    x = embed(shape, W, tokens)
    for layer in range(shape.n_layers):
        x = layer_forward(shape, W, layer, x, cache, causal=True, append=True, trace=trace)
    cache.length += n


def ar_step(shape: ModelShape, W: Weights, cache: KVCache, tokens, lm_scale: float,
            trace: dict | None = None):
    """One autoregressive decode step on the same weights, the baseline the
    pages set the diffusion step against (DiffusionGemma Technical Report
    digest, Figure 11, the per-step cost of AR decoding): each sequence's
    latest token, tokens [B], is encoded causally at position L and appended
    to the cache (the encoder's path for a one-token block), and the next
    token is the argmax of its logits (greedy, ties to the lower id).
    Returns (next [B], z [B, V]); trace as in ``denoise_logits``."""
    tokens = np.asarray(tokens).reshape(-1, 1)
    if cache.length + 1 > cache.capacity:
        raise ValueError("KV capacity exceeded")
    x = embed(shape, W, tokens)
    for layer in range(shape.n_layers):
        x = layer_forward(shape, W, layer, x, cache, causal=True, append=True, trace=trace)
    cache.length += 1
    z = final_logits(shape, W, x[:, -1], lm_scale)
    return np.argmax(z, axis=-1), z


def denoise_logits(shape: ModelShape, W: Weights, cache: KVCache, tokens: np.ndarray,
                   sc_probs, lm_scale: float, trace: dict | None = None) -> np.ndarray:
    """Denoiser forward: logits [B, C, V] for the canvas tokens [B, C]."""
    x = embed(shape, W, tokens, sc_probs)
    for layer in range(shape.n_layers):
        x = layer_forward(shape, W, layer, x, cache, causal=False, append=False, trace=trace)
    if trace is not None:
        trace["x_final"] = x.copy()
    return final_logits(shape, W, x, lm_scale)


def denoise_step(shape: ModelShape, W: Weights, cache: KVCache, tokens, sc_probs, t: int,
                 n_steps: int, seeds, block: int, lm_scale: float, prev_argmax=None,
                 adaptive: bool = True, trace: dict | None = None):
    """One denoising step for B canvases.  Returns the logits and, per canvas,
    the sampler's outputs (see ``sampler.sample_from_logits``)."""
    tokens = np.atleast_2d(np.asarray(tokens))
    z = denoise_logits(shape, W, cache, tokens, sc_probs, lm_scale, trace)
    outs = []
    for b in range(tokens.shape[0]):
        gp = None if prev_argmax is None else prev_argmax[b]
        outs.append(smp.sample_from_logits(z[b], t, n_steps, seeds[b], block, gp, adaptive))
    return z, outs


def commit_tokens(argmax: np.ndarray) -> np.ndarray:
    """Tokens committed at the end of a canvas: the final step's argmax."""
    return np.asarray(argmax)


def run_canvas(shape: ModelShape, W: Weights, cache: KVCache, n_steps: int, seeds, block: int,
               lm_scale: float, adaptive: bool, canvas: int, first_tokens=None, sc_probs=None,
               commit: bool = True, log: list | None = None):
    """Denoise one block of B canvases for up to n_steps, then optionally
    commit (encode & append).  Returns (committed tokens [B, C], steps taken)."""
    B = len(seeds)
    if first_tokens is None:
        tokens = np.stack([smp.initial_canvas(s, block, canvas, shape.vocab) for s in seeds])
    else:
        tokens = np.asarray(first_tokens)
    prev = None
    steps = 0
    for t in range(n_steps):
        z, outs = denoise_step(shape, W, cache, tokens, sc_probs, t, n_steps, seeds, block,
                               lm_scale, prev, adaptive)
        steps = t + 1
        if log is not None:
            log.append({"t": t, "z": z, "outs": outs, "tokens": tokens.copy()})
        prev = np.stack([o["argmax"] for o in outs])
        tokens = np.stack([o["next_tokens"] for o in outs])
        sc_probs = np.stack([o["p"] for o in outs])
        if all(o["stop"] for o in outs):
            break
    committed = commit_tokens(prev)
    if commit:
        encode_append(shape, W, cache, committed)
    return committed, steps
