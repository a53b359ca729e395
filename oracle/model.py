"""Decoder forward in plain fp64 (ORACLE — test infrastructure only).

What the pages fix about the network:

* DiffusionGemma Technical Report digest (METAL MEDIA), Figure 4: the prompt
  goes through a causal encoder that fills the KV cache; the denoiser refines
  the canvas with bidirectional attention inside the canvas and attention to
  the cache; a finished canvas is re-encoded causally and appended.
* same digest, Table 1: a mixture-of-experts transformer, 8 of 128 experts
  active plus 1 shared expert, a 262k vocabulary, and an extra MLP for
  self-conditioning (7.8M parameters).
* LLM-Wiki digest of the PyTorchKR review ("DiffusionGemma 기술 문서 리뷰"),
  key points: causal attention over the clean context, bidirectional inside
  the noisy canvas; the previous prediction's probabilities re-enter the next
  step as a continuous signal.
* euno.news (from VentureBeat), "how it was built": the serving stack switches
  between causal and bidirectional attention by phase.

Readings where the pages are silent (shapes come from the workload
definitions): pre-norm RMSNorm with gain 1 and eps 1e-6; RoPE (RoFormer
pairing, base 10000) on q and k at absolute positions; attention scale
1/sqrt(d_head), no softcap, no window, no QK-norm; grouped-query attention
(query head h reads KV head h // (n_q/n_kv)); router = linear map, top-k by
logit (ties to the lower expert id), softmax over the k selected; every
expert and the shared expert are GeGLU (tanh GELU) blocks; the shared expert
has weight 1; self-conditioning = expected embedding under the previous
step's tempered distribution, through a bias-free 2-matrix tanh-GELU MLP,
added to the token embedding; untied LM head multiplied by the workload's
LM-head scale.

Storage/rounding contract (bf16 models): weights as stored (fp8 weights:
E4M3 code times its output row's fp32 scale; MXFP4 weights: E2M1 code times
the E8M0 scale of its block of 32 inputs; both exact in float64); residual stream
fp32 on the GPU (fp64 here); GEMM inputs (norm outputs, attention output,
GeGLU hidden, expected embedding, self-cond hidden, self-cond probabilities)
rounded to bf16; q/k/v rounded to bf16 after RoPE (k, v are the cache
entries).  fp32 models round nothing.
"""
from __future__ import annotations

import contextlib

import numpy as np

import synth
from synth.configs import ModelShape

from .numerics import e4m3_decode, gelu_tanh, mxfp4_dequantize, rmsnorm, rope, round_bf16


class Weights:
    """Logical weights of a synthetic model as float64 arrays ([out][in])."""

    def __init__(self, shape: ModelShape, cache: bool = True):
        self.shape = shape
        self._cache = {} if cache else None

    def _dtype_of(self, name: str) -> str:
        # expert weights: the routed experts and the shared expert alike
        s = self.shape
        if name in ("ex_g", "ex_u", "ex_d", "sh_g", "sh_u", "sh_d"):
            return s.expert_dtype
        if name == "lm_head":
            return s.lm_dtype
        return s.dtype

    def _shape_of(self, name: str):
        s = self.shape
        d = s.d_model
        return {
            "embed": (s.vocab, d), "lm_head": (s.vocab, d),
            "sc_up": (s.d_selfcond, d), "sc_down": (d, s.d_selfcond),
            "wqkv": (s.qkv_rows, d), "wo": (d, s.q_dim), "wr": (s.n_experts, d),
            "sh_g": (s.d_shared, d), "sh_u": (s.d_shared, d), "sh_d": (d, s.d_shared),
            "ex_g": (s.n_experts, s.d_expert, d), "ex_u": (s.n_experts, s.d_expert, d),
            "ex_d": (s.n_experts, d, s.d_expert),
        }[name]

    def get(self, name: str, layer: int | None = None) -> np.ndarray:
        key = (name, layer)
        if self._cache is not None and key in self._cache:
            return self._cache[key]
        tid = synth.TID[name] if layer is None else synth.layer_tid(layer, name)
        if name == "lm_head" and self.shape.tied_head:
            tid = synth.TID["embed"]  # input recipe: the head is drawn from the embedding's stream
        dt = self._dtype_of(name)
        shp = self._shape_of(name)
        if dt == "fp8":
            # stored codes and per-output-row fp32 scales, dequantised exactly
            rows = int(np.prod(shp[:-1]))
            codes, sc = synth.e4m3_rows(self.shape.weight_seed, tid, rows, shp[-1], self.shape.weight_std)
            w = (e4m3_decode(codes) * sc.astype(np.float64)[:, None]).reshape(shp)
            if self._cache is not None:
                self._cache[key] = w
            return w
        if dt == "mxfp4":
            # stored E2M1 codes and an E8M0 scale per 32 inputs, dequantised exactly
            rows = int(np.prod(shp[:-1]))
            codes, sc = synth.mxfp4_rows(self.shape.weight_seed, tid, rows, shp[-1], self.shape.weight_std)
            w = mxfp4_dequantize(codes, sc).reshape(shp)
            if self._cache is not None:
                self._cache[key] = w
            return w
        w = synth.normal(self.shape.weight_seed, tid, shp, self.shape.weight_std,
                         "bf16_f64" if dt == "bf16" else "f32").astype(np.float64, copy=False)
        if self._cache is not None:
            self._cache[key] = w
        return w

    def drop_layer(self, layer: int):
        if self._cache is not None:
            for k in [k for k in self._cache if k[1] == layer]:
                del self._cache[k]


# Every product below is evaluated by mm(), every RMSNorm by norm(), every
# attention softmax by attention(), every residual sum by resid().  By default
# all of them work in float64.  accumulation("f32") evaluates the same
# definition in float32 arithmetic (the operands of each product are exact
# float32 copies of the bf16 values that feed it; products, sums, the norm's
# mean of squares, the softmax and the residual stream in float32; storage
# roundings unchanged): a second correct evaluation order, used only to
# measure how far two such evaluations drift apart on a given problem (bf16
# rounding of activations turns last-bit differences into whole-ulp ones).
# Expected values always come from the float64 default.
_ACC = ["f64"]


@contextlib.contextmanager
def accumulation(kind: str):
    if kind not in ("f64", "f32"):
        raise ValueError(kind)
    old = _ACC[0]
    _ACC[0] = kind
    try:
        yield
    finally:
        _ACC[0] = old


# The float32 evaluation sums each product's K terms in the BLAS order of the
# operands as given ("fwd") or with the K axis reversed ("rev"): two correct
# float32 evaluations of the same definition, so that the spread between
# such evaluations is measured with more than one sample.
_ORDER = ["fwd"]


@contextlib.contextmanager
def twin_order(kind: str):
    if kind not in ("fwd", "rev"):
        raise ValueError(kind)
    old = _ORDER[0]
    _ORDER[0] = kind
    try:
        yield
    finally:
        _ORDER[0] = old


def mm(a, b) -> np.ndarray:
    if _ACC[0] == "f64":
        return np.asarray(a) @ np.asarray(b)
    a32, b32 = np.asarray(a, dtype=np.float32), np.asarray(b, dtype=np.float32)
    if _ORDER[0] == "rev":
        a32 = np.ascontiguousarray(a32[..., ::-1])
        b32 = np.ascontiguousarray(np.flip(b32, axis=-2))
    return (a32 @ b32).astype(np.float64)


def norm(shape: ModelShape, x: np.ndarray) -> np.ndarray:
    """RMSNorm (gain 1) in the current accumulation precision."""
    if _ACC[0] == "f64":
        return rmsnorm(x, shape.norm_eps)
    x32 = np.asarray(x, dtype=np.float32)
    ms = np.mean(x32 * x32, axis=-1, keepdims=True, dtype=np.float32)
    return (x32 / np.sqrt(ms + np.float32(shape.norm_eps))).astype(np.float64)


def resid(x: np.ndarray) -> np.ndarray:
    """A residual-stream value: kept in float64 by default, float32 in the
    float32 evaluation (the GPU's residual is float32)."""
    return x if _ACC[0] == "f64" else np.asarray(x, dtype=np.float32).astype(np.float64)


def round_act(shape: ModelShape, x: np.ndarray) -> np.ndarray:
    """Activation storage rounding at GEMM inputs: bf16 for bf16 models."""
    return round_bf16(x) if shape.dtype == "bf16" else x


class KVCache:
    """Per-layer K and V, [B, n_kv, capacity, d_head] float64 (bf16 values for
    bf16 models), with a common length for the batch."""

    def __init__(self, shape: ModelShape, batch: int, capacity: int):
        self.shape = shape
        self.k = [np.zeros((batch, shape.n_kv_heads, capacity, shape.d_head)) for _ in range(shape.n_layers)]
        self.v = [np.zeros((batch, shape.n_kv_heads, capacity, shape.d_head)) for _ in range(shape.n_layers)]
        self.length = 0
        self.capacity = capacity


def embed(shape: ModelShape, W: Weights, tokens: np.ndarray, sc_probs=None) -> np.ndarray:
    """x = E[tok] (+ MLP_sc(sum_v P[v] E[v]) when self-conditioning is given).

    tokens: [B, n]; sc_probs: [B, n, V] or None.  Returns the residual [B, n, d]."""
    E = W.get("embed")
    x = E[np.asarray(tokens)]
    if sc_probs is not None:
        P = round_act(shape, np.asarray(sc_probs, dtype=np.float64))
        ebar = round_act(shape, mm(P, E))                       # expected embedding
        h = round_act(shape, gelu_tanh(mm(ebar, W.get("sc_up").T)))
        x = resid(x + mm(h, W.get("sc_down").T))
    return x


def attention(shape: ModelShape, q, k_all, v_all, n_prefix: int, causal: bool) -> np.ndarray:
    """softmax(q K^T / sqrt(d)) V over the joint key list [prefix ; canvas].

    q: [n, Hq, d] for one sequence; k_all/v_all: [Hkv, n_prefix + n, d].
    Every prefix key is visible; canvas key j is visible to canvas query i
    always (denoise) or when j <= i (causal encode).  Returns [n, Hq, d]."""
    n = q.shape[0]
    group = shape.n_q_heads // shape.n_kv_heads
    n_keys = k_all.shape[1]
    mask = np.ones((n, n_keys), dtype=bool)
    if causal:
        i = np.arange(n)[:, None]
        j = np.arange(n_keys)[None, :] - n_prefix
        mask = (j < 0) | (j <= i)
    out = np.empty_like(q)
    scale = 1.0 / np.sqrt(shape.d_head)
    for h in range(shape.n_q_heads):
        hk = h // group
        s = mm(q[:, h, :], k_all[hk].T) * scale
        s = np.where(mask, s, -np.inf)
        if _ACC[0] == "f32":
            s = s.astype(np.float32)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        pr = (e / e.sum(axis=1, keepdims=True)).astype(np.float64)
        out[:, h, :] = mm(pr, v_all[hk])
    return out


def route(shape: ModelShape, r: np.ndarray):
    """Top-k experts per token by router logit (ties to the lower id) and the
    softmax over the k selected logits.  r: [T, E] -> ids [T, k], w [T, k]."""
    T, E = r.shape
    ids = np.empty((T, shape.top_k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -r[t]))
        ids[t] = order[: shape.top_k]
    sel = np.take_along_axis(r, ids, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    return ids, w


def geglu(shape: ModelShape, u, wg, wu, wd):
    """Wd (gelu_tanh(Wg u) * (Wu u)), hidden rounded as a GEMM input."""
    h = round_act(shape, gelu_tanh(mm(u, wg.T)) * mm(u, wu.T))
    return mm(h, wd.T)


def moe(shape: ModelShape, W: Weights, layer: int, n2: np.ndarray, ret_routing=False):
    """Shared expert + weighted sum of the top-k routed experts, in rank order.

    n2: [T, d] (already rounded).  Returns y [T, d]."""
    r = mm(n2, W.get("wr", layer).T)
    ids, w = route(shape, r)
    y = geglu(shape, n2, W.get("sh_g", layer), W.get("sh_u", layer), W.get("sh_d", layer))
    exg, exu, exd = W.get("ex_g", layer), W.get("ex_u", layer), W.get("ex_d", layer)
    T = n2.shape[0]
    outs = np.zeros((T, shape.top_k, shape.d_model))
    for e in np.unique(ids):
        tok, slot = np.nonzero(ids == e)
        outs[tok, slot] = geglu(shape, n2[tok], exg[e], exu[e], exd[e])
    for j in range(shape.top_k):
        y = y + w[:, j:j + 1] * outs[:, j]
    if ret_routing:
        return y, r, ids, w
    return y


def layer_forward(shape: ModelShape, W: Weights, layer: int, x: np.ndarray, cache: KVCache,
                  causal: bool, append: bool, trace: dict | None = None) -> np.ndarray:
    """One pre-norm block over the canvas x [B, n, d] at positions L..L+n-1.

    causal/append = True is the encoder (causal canvas mask; k, v written to
    cache rows [L, L+n)); False is the denoiser (bidirectional canvas; the
    cache is read, never written)."""
    B, n, d = x.shape
    L = cache.length
    s = shape
    nrm = round_act(s, norm(s, x))
    qkv = mm(nrm, W.get("wqkv", layer).T)                           # [B, n, rows]
    q = qkv[..., : s.q_dim].reshape(B, n, s.n_q_heads, s.d_head)
    k = qkv[..., s.q_dim: s.q_dim + s.kv_dim].reshape(B, n, s.n_kv_heads, s.d_head)
    v = qkv[..., s.q_dim + s.kv_dim:].reshape(B, n, s.n_kv_heads, s.d_head)
    pos = L + np.arange(n)
    q = round_act(s, rope(q, pos, s.rope_base))
    k = round_act(s, rope(k, pos, s.rope_base))
    v = round_act(s, v)
    o = np.empty((B, n, s.n_q_heads, s.d_head))
    for b in range(B):
        kk = np.concatenate([cache.k[layer][b, :, :L], k[b].transpose(1, 0, 2)], axis=1)
        vv = np.concatenate([cache.v[layer][b, :, :L], v[b].transpose(1, 0, 2)], axis=1)
        o[b] = attention(s, q[b], kk, vv, L, causal)
    if append:
        cache.k[layer][:, :, L:L + n] = k.transpose(0, 2, 1, 3)
        cache.v[layer][:, :, L:L + n] = v.transpose(0, 2, 1, 3)
    o = round_act(s, o.reshape(B, n, s.q_dim))
    x = resid(x + mm(o, W.get("wo", layer).T))
    n2 = round_act(s, norm(s, x)).reshape(B * n, d)
    y, r, ids, w = moe(s, W, layer, n2, ret_routing=True)
    if trace is not None:
        trace.setdefault("router_logits", []).append(r)
        trace.setdefault("expert_ids", []).append(ids)
        trace.setdefault("x_attn", []).append(x.copy())
    return resid(x + y.reshape(B, n, d))


def final_logits(shape: ModelShape, W: Weights, x: np.ndarray, lm_scale: float) -> np.ndarray:
    """z = s_lm * (RMSNorm(x) W_lm^T)."""
    nrm = round_act(shape, norm(shape, x))
    return lm_scale * mm(nrm, W.get("lm_head").T)
