"""GPU checks of the fp8 workload: the one-layer full-width model with E4M3
expert (routed and shared) and LM-head weights, per-output-feature fp32
scales, bf16 activations; a batch of 4 independent canvases of 256 over
8192-row random N(0,1) caches; 12 steps with sampler seeds 0..3.

* First step (t = 0) with the oracle's routes forced: logits of 64 sampled
  positions per canvas (every vocabulary tile) within |g - o| <= 3e-2 +
  1e-2|o| (or the fp32-twin criterion), their entropies within 1e-3 nats,
  router logits close; unforced route flips only at oracle near-ties.
* A canvas of the batch, run alone over its own cache rows, gives the same
  logits (within the bar: the K splits depend on the batch's row count) and
  entropies: canvases share no data.
* The 12-step product run: per-step sampler invariants, determinism."""
import numpy as np
import pytest

import synth
from oracle import model as om
from oracle import sampler as smp
from synth.configs import WORKLOADS

from .gpu_util import allclose_report, bar_or_twin, say
from .test_gpu_full import _invariants
from .test_gpu_model import RTOL, ROUTE_EPS, _err_summary, _route_margins, flip_margin_bound

pytestmark = pytest.mark.gpu

ATOL_FP8 = 3e-2
ROWS = np.arange(0, 256, 4)  # sampled canvas positions (0 .. 255): 64 per canvas


@pytest.fixture(scope="module")
def env():
    import torch
    import discrete_text_diffusion_amd as dg
    from discrete_text_diffusion_amd import runtime as rt
    assert torch.cuda.is_available()
    return torch, dg, rt


def _oracle_cache(shape, B, L, cap):
    oc = om.KVCache(shape, B, cap)
    for name, tid in (("k", synth.TID["kv_k"]), ("v", synth.TID["kv_v"])):
        vals = synth.bf16_bits_to_f32(synth.normal(0, tid, (1, B, shape.n_kv_heads, L, shape.d_head), 1.0))
        getattr(oc, name)[0][:, :, :L] = vals[0].astype(np.float64)
    oc.length = L
    return oc


@pytest.fixture(scope="module")
def fp8b4(env):
    torch, dg, rt = env
    wl = WORKLOADS["fp8batch4"]
    shape, B, C, L = wl.model, wl.batch, wl.canvas, wl.prefix
    say(f"fp8batch4: building the fp8 model, B={B}, cache {L}")
    model = rt.DeviceModel(shape, wl.lm_scale)
    cache = rt.DeviceCache(shape, B, L + C)
    cache.fill_random(L, seed=0, std=1.0)
    seeds = list(wl.sampler_seeds)
    cv = rt.DeviceCanvas(shape, B, C, seeds)
    ws = rt.Workspace(model.cfg, B, C)
    dg.dg_init_canvas(model.cfg, cv.struct, 0, rt.stream_handle())
    torch.cuda.synchronize()
    tok = cv.tokens.cpu().numpy().reshape(B, C)
    for b in range(B):
        assert np.array_equal(tok[b], smp.initial_canvas(seeds[b], 0, C, shape.vocab))
    return dict(wl=wl, shape=shape, model=model, cache=cache, cv=cv, ws=ws, tok=tok, seeds=seeds,
                W=om.Weights(shape), oc=_oracle_cache(shape, B, L, L + C))


def _gpu_logits(env, f, force=None, rows=None):
    torch, dg, rt = env
    shape, wl = f["shape"], f["wl"]
    B, C = wl.batch, wl.canvas
    out = torch.empty(B * C * shape.vocab, dtype=torch.float32, device="cuda")
    rout = torch.empty(B * C * shape.n_experts, dtype=torch.float32, device="cuda")
    d_force = None
    if force is not None:
        d_force = torch.from_numpy(np.ascontiguousarray(force, dtype=np.int32).reshape(-1)).cuda()
    dg.dg_test_forward_logits(f["model"].cfg, f["model"].weights, f["cache"].struct, f["cv"].struct,
                              rt.step_params(0, wl.n_steps, 0, False), d_force.data_ptr() if d_force is not None else None,
                              rout.data_ptr(), out.data_ptr(), f["ws"].ptr, f["ws"].size, rt.stream_handle())
    torch.cuda.synchronize()
    z = out.view(B, C, shape.vocab)
    if rows is not None:
        z = z[:, torch.from_numpy(rows).cuda()]
    return z.cpu().numpy(), rout.cpu().numpy().reshape(1, B * C, shape.n_experts)


def _oracle_hidden(f, trace, fixed_ids=None):
    """Final residual [B, C, d] of the denoiser at t = 0 (no self-conditioning)."""
    shape = f["shape"]
    orig = om.route
    if fixed_ids is not None:
        ids = list(fixed_ids)

        def fixed(shape_, r):
            sel = ids.pop(0)
            s_ = np.take_along_axis(r, sel, axis=1)
            e = np.exp(s_ - s_.max(axis=1, keepdims=True))
            return sel, e / e.sum(axis=1, keepdims=True)

        om.route = fixed
    try:
        x = om.embed(shape, f["W"], f["tok"])
        return om.layer_forward(shape, f["W"], 0, x, f["oc"], causal=False, append=False, trace=trace)
    finally:
        om.route = orig


def test_fp8_first_step_logits_match_oracle(env, fp8b4):
    f = fp8b4
    shape, wl = f["shape"], f["wl"]
    kv_before = f["cache"].valid_rows()
    say("fp8batch4: oracle layer forward (1024 canvas tokens)")
    tr = {}
    x = _oracle_hidden(f, tr)
    margins = _route_margins(shape, tr)
    say(f"fp8batch4: oracle routing margins min {margins.min():.2e}")
    zo = om.final_logits(shape, f["W"], x[:, ROWS], wl.lm_scale)
    say("fp8batch4: fp32 twin on the oracle's routes")
    trt = {}
    with om.accumulation("f32"):
        xt = _oracle_hidden(f, trt, tr["expert_ids"])
        zt = om.final_logits(shape, f["W"], xt[:, ROWS], wl.lm_scale)
    z, rg = _gpu_logits(env, f, force=np.stack(tr["expert_ids"]), rows=ROWS)
    torch = env[0]
    assert all(torch.equal(a, b) for a, b in zip(kv_before, f["cache"].valid_rows()))
    _err_summary("fp8batch4 router logits (oracle routes)", rg, np.stack(tr["router_logits"]))
    bar_or_twin("fp8batch4 router logits (oracle routes)", rg, np.stack(tr["router_logits"]),
                np.stack(trt["router_logits"]), ROUTE_EPS["bf16"], 0.0)
    bar_or_twin("fp8batch4 logits (oracle routes)", z, zo, zt, ATOL_FP8, RTOL)
    tau = smp.temperature(0, wl.n_steps)
    _, Hg, _ = smp.row_statistics(z.reshape(-1, shape.vocab), tau)
    _, Ho, _ = smp.row_statistics(zo.reshape(-1, shape.vocab), tau)
    allclose_report("fp8batch4 entropy (oracle routes)", Hg, Ho, 1e-3, 0.0)
    _, ru = _gpu_logits(env, f, rows=ROWS)
    gtop = np.sort(np.argsort(-ru[0], axis=1, kind="stable")[:, :shape.top_k], axis=1)
    otop = np.sort(tr["expert_ids"][0], axis=1)
    flips = np.nonzero(np.any(gtop != otop, axis=1))[0]
    bound = flip_margin_bound(rg, np.stack(tr["router_logits"]))
    say(f"fp8batch4 unforced: route flips {flips.size} at oracle margins {margins[0][flips]} (bound {bound:.2e})")
    assert np.all(margins[0][flips] < bound)
    f["zo"], f["zt"], f["flips"] = zo, zt, flips.size


def test_fp8_batch_matches_single_canvas(env, fp8b4):
    """Canvas b of the batch, run alone over its own cache rows with its own
    seed: logits within the bar, step entropies within 1e-3 nats (the row
    count changes only the K-split summation order)."""
    torch, dg, rt = env
    f = fp8b4
    shape, wl = f["shape"], f["wl"]
    B, C, L = wl.batch, wl.canvas, wl.prefix
    st = rt.stream_handle()
    cfg = f["model"].cfg
    # both runs on the batch's own routes, so only the summation order differs
    zb, rb = _gpu_logits(env, f, rows=np.arange(C))
    ids = np.argsort(-rb[0], axis=1, kind="stable")[:, :shape.top_k].reshape(B, C, shape.top_k)
    zb, _ = _gpu_logits(env, f, force=ids.reshape(1, B * C, shape.top_k), rows=np.arange(C))
    b = 2
    d_force1 = torch.from_numpy(np.ascontiguousarray(ids[b:b + 1], dtype=np.int32).reshape(-1)).cuda()
    one = rt.DeviceCache(shape, 1, L + C)
    for name in ("k", "v"):
        one.view(name)[:, 0].copy_(f["cache"].view(name)[:, b])
    one.struct.length = L
    cv1 = rt.DeviceCanvas(shape, 1, C, [f["seeds"][b]])
    cv1.tokens.copy_(f["cv"].tokens.view(B, C)[b])
    ws1 = rt.Workspace(cfg, 1, C)
    out = torch.empty(C * shape.vocab, dtype=torch.float32, device="cuda")
    dg.dg_test_forward_logits(cfg, f["model"].weights, one.struct, cv1.struct, rt.step_params(0, wl.n_steps, 0, False),
                              d_force1.data_ptr(), None, out.data_ptr(), ws1.ptr, ws1.size, st)
    torch.cuda.synchronize()
    z1 = out.view(C, shape.vocab).cpu().numpy()
    d = np.abs(z1 - zb[b])
    say(f"fp8batch4: canvas {b} alone vs in the batch (same routes): {int(np.sum(d > 0))} differing logits, "
        f"max {d.max():.2e}")
    allclose_report(f"fp8batch4 canvas {b} alone vs batched logits", z1, zb[b], ATOL_FP8, RTOL)
    # full steps: batch and single
    cvb = f["cv"]
    tok0 = cvb.tokens.clone()
    dg.dg_denoise_step(cfg, f["model"].weights, f["cache"].struct, cvb.struct, rt.step_params(0, wl.n_steps, 0, False),
                       f["ws"].ptr, f["ws"].size, st)
    dg.dg_denoise_step(cfg, f["model"].weights, one.struct, cv1.struct, rt.step_params(0, wl.n_steps, 0, False),
                       ws1.ptr, ws1.size, st)
    torch.cuda.synchronize()
    # entropy bar: the first-order entropy change the two runs' measured logit
    # difference allows (twice, for the second-order terms), at least 1e-3
    tau = smp.temperature(0, wl.n_steps)
    pz, _, _ = smp.row_statistics(zb[b], tau)
    a = zb[b] / tau
    abar = (pz * a).sum(-1, keepdims=True)
    hbar = np.maximum(1e-3, 2.0 * (pz * np.abs(a - abar) * d / tau).sum(-1))
    say(f"fp8batch4: entropy bar from the logit difference: max {hbar.max():.2e}")
    allclose_report(f"fp8batch4 canvas {b} alone vs batched entropy", cv1.entropy.cpu().numpy(),
                    cvb.entropy.view(B, C)[b].cpu().numpy(), hbar, 0.0)
    same = float((cv1.argmax == cvb.argmax.view(B, C)[b]).float().mean().item())
    say(f"fp8batch4 canvas {b}: argmax agreement {same:.4f}")
    cvb.tokens.copy_(tok0)


def test_fp8_twelve_steps(env, fp8b4):
    """The workload's run: 12 steps for the 4 canvases; per-step invariants,
    and two runs from the same start agree bit for bit."""
    torch, dg, rt = env
    f = fp8b4
    shape, wl = f["shape"], f["wl"]
    B, C, V = wl.batch, wl.canvas, shape.vocab
    cfg, st = f["model"].cfg, rt.stream_handle()
    cv = f["cv"]
    runs = []
    for rep in range(2):
        dg.dg_init_canvas(cfg, cv.struct, 0, st)
        accepted = []
        for t in range(wl.n_steps):
            dg.dg_denoise_step(cfg, f["model"].weights, f["cache"].struct, cv.struct,
                               rt.step_params(t, wl.n_steps, 0, wl.adaptive), f["ws"].ptr, f["ws"].size, st)
            torch.cuda.synchronize()
            if rep == 0:
                _invariants(cv, f["seeds"], t, C, V)
                accepted.append(cv.n_accepted.cpu().numpy().tolist())
        if rep == 0:
            say(f"fp8batch4: accepted per step {accepted}")
        runs.append([x.clone() for x in (cv.tokens, cv.entropy, cv.argmax, cv.p_side, cv.p_scale)])
    for a, b in zip(*runs):
        assert torch.equal(a, b)
