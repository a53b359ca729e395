"""GPU checks at the pages' full sizes.

* One full-width layer + LM head (d_model 2816, 16/8 heads of 256, 128
  experts top-8 + shared, vocab 262144), bf16, single step at t = 1 with a
  random N(0,1) 2048-row cache and Dirichlet(0.05) self-conditioning: logits
  and entropies against the oracle with the oracle's routes forced, route
  flips only at near-ties, sampler decisions bit-exact from the oracle's
  logits, the product step's invariants.
* The 30-layer model in the launch configuration of bench.py (4096-token
  prefix, 256-token canvas): the first 64 prefix positions of every layer's
  cache (causal, so the oracle computes them alone), determinism, the cache
  left untouched by denoising, per-step sampler invariants, commit."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import model as om
from oracle import sampler as smp
from oracle import step as ost
from synth.configs import WORKLOADS

from .gpu_util import allclose_report, compare_decisions, say
from .test_gpu_model import ATOL, RTOL, ROUTE_EPS, _err_summary, _route_margins, entropy_tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import discrete_text_diffusion_amd as dg
    from discrete_text_diffusion_amd import runtime as rt
    assert torch.cuda.is_available()
    return torch, dg, rt


def _invariants(cv, seeds, t, C, V, prev=None, adaptive=False):
    B = cv.batch
    H = cv.entropy.cpu().numpy().reshape(B, C).astype(np.float64)
    acc = cv.accepted.cpu().numpy().reshape(B, C).astype(bool)
    samp = cv.sample.cpu().numpy().reshape(B, C)
    nxt = cv.tokens.cpu().numpy().reshape(B, C)
    nacc = cv.n_accepted.cpu().numpy()
    for b in range(B):
        K = int(acc[b].sum())
        assert K == nacc[b] >= 1
        order = np.lexsort((np.arange(C), H[b]))
        assert set(np.nonzero(acc[b])[0]) == set(order[:K])
        if K > 1:
            assert H[b][acc[b]].sum() <= 0.1 + 1e-5
        fresh = smp.renoise_tokens(seeds[b], t, 0, C, V)
        assert np.array_equal(nxt[b], np.where(acc[b], samp[b], fresh))
        assert (0 <= samp[b]).all() and (samp[b] < V).all()
    return H


def test_full_layer_step_matches_oracle(env):
    torch, dg, rt = env
    wl = WORKLOADS["layer1"]
    shape, C, L = wl.model, wl.canvas, wl.prefix
    t, N = wl.first_step, wl.n_steps
    say(f"layer1: building model and inputs (V={shape.vocab}, cache {L})")
    model = rt.DeviceModel(shape, wl.lm_scale)
    cfg = model.cfg
    cache = rt.DeviceCache(shape, 1, L + C)
    cache.fill_random(L, seed=0, std=1.0)
    cv = rt.DeviceCanvas(shape, 1, C, [0])
    ws = rt.Workspace(cfg, 1, C)
    st = rt.stream_handle()
    dg.dg_init_canvas(cfg, cv.struct, 0, st)
    P = synth.dirichlet_rows(0, synth.TID["dirichlet"], C, shape.vocab, wl.dirichlet_alpha)
    d_P = torch.from_numpy(P.reshape(-1)).cuda()
    cv.set_sc_probs(d_P)
    torch.cuda.synchronize()
    tok = cv.tokens.cpu().numpy().reshape(1, C)
    assert np.array_equal(tok[0], smp.initial_canvas(0, 0, C, shape.vocab))
    # oracle: same random cache (logical [layer][batch][kv_head][row][d_head])
    say("layer1: oracle forward")
    W = om.Weights(shape)
    oc = om.KVCache(shape, 1, L + C)
    for name, tid in (("k", synth.TID["kv_k"]), ("v", synth.TID["kv_v"])):
        vals = synth.bf16_bits_to_f32(synth.normal(0, tid, (1, 1, shape.n_kv_heads, L, shape.d_head), 1.0))
        getattr(oc, name)[0][:, :, :L] = vals[0].astype(np.float64)
    oc.length = L
    tr = {}
    zo = ost.denoise_logits(shape, W, oc, tok, P.astype(np.float64)[None], wl.lm_scale, trace=tr)[0]
    margins = _route_margins(shape, tr)
    say(f"layer1: oracle routing margins min {margins.min():.2e}")
    # GPU with the oracle's routes
    T = C
    out = torch.empty(T * shape.vocab, dtype=torch.float32, device="cuda")
    rout = torch.empty(T * shape.n_experts, dtype=torch.float32, device="cuda")
    force = torch.from_numpy(np.ascontiguousarray(np.stack(tr["expert_ids"]), dtype=np.int32).reshape(-1)).cuda()
    k_before = cache.k.clone()
    dg.dg_test_forward_logits(cfg, model.weights, cache.struct, cv.struct, rt.step_params(t, N, 0, False),
                              force.data_ptr(), rout.data_ptr(), out.data_ptr(), ws.ptr, ws.size, st)
    torch.cuda.synchronize()
    assert torch.equal(k_before, cache.k)
    z = out.cpu().numpy().reshape(C, shape.vocab)
    rg = rout.cpu().numpy().reshape(1, T, shape.n_experts)
    _err_summary("layer1 router logits (oracle routes)", rg, np.stack(tr["router_logits"]))
    _err_summary("layer1 logits (oracle routes)", z, zo)
    tau = smp.temperature(t, N)
    _, Hg, _ = smp.row_statistics(z, tau)
    _, Ho, _ = smp.row_statistics(zo, tau)
    _err_summary("layer1 entropy (oracle routes)", Hg, Ho)
    allclose_report("layer1 logits (oracle routes)", z, zo, ATOL, RTOL)
    allclose_report("layer1 entropy (oracle routes)", Hg, Ho, 1e-3, 0.0)
    # unforced: layer-0 route flips only at oracle near-ties
    dg.dg_test_forward_logits(cfg, model.weights, cache.struct, cv.struct, rt.step_params(t, N, 0, False),
                              None, rout.data_ptr(), out.data_ptr(), ws.ptr, ws.size, st)
    torch.cuda.synchronize()
    ru = rout.cpu().numpy().reshape(T, shape.n_experts)
    gtop = np.sort(np.argsort(-ru, axis=1, kind="stable")[:, :shape.top_k], axis=1)
    otop = np.sort(tr["expert_ids"][0], axis=1)
    flips = np.nonzero(np.any(gtop != otop, axis=1))[0]
    say(f"layer1 unforced: route flips {flips.size} at oracle margins {margins[0][flips]}")
    assert np.all(margins[0][flips] < ROUTE_EPS["bf16"])
    # sampler decisions from the oracle's own logits: bit-exact up to reported near-ties
    say("layer1: sampler from oracle logits")
    cv2 = rt.DeviceCanvas(shape, 1, C, [0])
    prev = np.argmax(zo, axis=-1).astype(np.int32)
    cv2.prev_argmax.copy_(torch.from_numpy(prev))
    d_z = torch.from_numpy(zo.astype(np.float32)).cuda()
    dg.dg_test_sample_from_logits(cfg, d_z.data_ptr(), cv2.struct, rt.step_params(t, N, 0, True), ws.ptr, ws.size, st)
    torch.cuda.synchronize()
    o = smp.sample_from_logits(zo.astype(np.float32).astype(np.float64), t, N, 0, 0, prev, True)
    allclose_report("layer1 sampler entropy", cv2.entropy.cpu().numpy(), o["H"], 1e-3, 0.0)
    assert np.array_equal(cv2.argmax.cpu().numpy(), o["argmax"])
    compare_decisions("layer1 sample", cv2.sample.cpu().numpy(), o["sample"], o["margin_sample"], 1e-5)
    compare_decisions("layer1 accepted", cv2.accepted.cpu().numpy().astype(bool), o["accepted"],
                      o["margin_accept"], 1e-5)
    assert int(cv2.stop.item()) == int(o["stop"])
    # the product step: invariants and agreement of its entropies with the oracle
    say("layer1: product step")
    dg.dg_denoise_step(cfg, model.weights, cache.struct, cv.struct, rt.step_params(t, N, 0, False), ws.ptr, ws.size,
                       st)
    torch.cuda.synchronize()
    H = _invariants(cv, [0], t, C, shape.vocab)
    if flips.size == 0:
        allclose_report("layer1 product-step entropy", H[0], Ho, 1e-3, 0.0)
    assert torch.equal(k_before, cache.k)


@pytest.fixture(scope="module")
def full30(env):
    torch, dg, rt = env
    wl = WORKLOADS["full30"]
    shape = wl.model
    say("full30: building the 30-layer model")
    model = rt.DeviceModel(shape, wl.lm_scale)
    cache = rt.DeviceCache(shape, 1, wl.prefix + wl.canvas)
    cv = rt.DeviceCanvas(shape, 1, wl.canvas, [0])
    ws = rt.Workspace(model.cfg, 1, wl.canvas)
    prompt = synth.tokens(0, synth.TID["prompt"], wl.prefix, shape.vocab)
    d_prompt = torch.from_numpy(prompt).cuda()
    say("full30: encoding the 4096-token prefix")
    dg.dg_encode_append(model.cfg, model.weights, cache.struct, d_prompt.data_ptr(), 1, wl.prefix, ws.ptr, ws.size,
                        rt.stream_handle())
    torch.cuda.synchronize()
    return dict(wl=wl, shape=shape, model=model, cache=cache, cv=cv, ws=ws, prompt=prompt)


def test_full30_prefix_cache_sampled_against_oracle(env, full30):
    """Causal: the first n prefix positions depend on themselves only, so the
    oracle encodes them alone (layer by layer, weights regenerated per layer)
    and every layer's K and V rows [0, n) are compared."""
    torch, dg, rt = env
    shape, cache, prompt = full30["shape"], full30["cache"], full30["prompt"]
    n = 48
    say(f"full30: oracle encode of the first {n} prefix tokens, 30 layers")
    W = om.Weights(shape)
    oc = om.KVCache(dataclasses.replace(shape), 1, n)
    x = om.embed(shape, W, prompt[None, :n])
    gk = cache.view("k")
    gv = cache.view("v")
    for layer in range(shape.n_layers):
        x = om.layer_forward(shape, W, layer, x, oc, causal=True, append=True)
        W.drop_layer(layer)
        allclose_report(f"full30 cache k L{layer}", gk[layer, :, :, :n].float().cpu().numpy(), oc.k[layer][:, :, :n],
                        ATOL, RTOL)
        allclose_report(f"full30 cache v L{layer}", gv[layer, :, :, :n].float().cpu().numpy(), oc.v[layer][:, :, :n],
                        ATOL, RTOL)


def test_full30_step_properties(env, full30):
    """Determinism, untouched cache, per-step invariants and the commit at the
    benchmark's configuration."""
    torch, dg, rt = env
    wl, shape, model, cache, cv, ws = (full30[k] for k in ("wl", "shape", "model", "cache", "cv", "ws"))
    cfg, st, C, V = model.cfg, rt.stream_handle(), wl.canvas, shape.vocab
    L = cache.length
    k_before = cache.k[: cache.k.numel() // 30].clone()  # layer 0 is enough to see any write
    gk = cache.view("k")
    prefix_before = gk[0, :, :, :L].clone()
    runs = []
    for rep in range(2):
        say(f"full30: 3 denoising steps, repetition {rep}")
        dg.dg_init_canvas(cfg, cv.struct, 0, st)
        for t in range(3):
            dg.dg_denoise_step(cfg, model.weights, cache.struct, cv.struct, rt.step_params(t, 12, 0, False), ws.ptr,
                               ws.size, st)
            torch.cuda.synchronize()
            if rep == 0:
                _invariants(cv, [0], t, C, V)
        runs.append([x.clone() for x in (cv.tokens, cv.entropy, cv.argmax, cv.p_side, cv.p_scale)])
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    assert torch.equal(k_before, cache.k[: cache.k.numel() // 30])
    say("full30: commit")
    dg.dg_commit_block(cfg, model.weights, cache.struct, cv.struct, rt.step_params(2, 12, 0), ws.ptr, ws.size, st)
    torch.cuda.synchronize()
    assert cache.length == L + C
    assert torch.equal(cv.committed, runs[0][2])
    assert torch.equal(prefix_before, gk[0, :, :, :L])          # rows below L untouched
    assert gk[0, 0, 0, L:L + C].abs().sum().item() > 0           # rows [L, L + C) appended
    nxt = cv.tokens.cpu().numpy()
    assert np.array_equal(nxt, smp.initial_canvas(0, 1, C, V))
    cache.struct.length = L
