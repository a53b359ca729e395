"""GPU checks of the long-context workload: the one-layer full-width bf16
model over a 32768-token causal prefix, 8 consecutive 256-token canvases of
up to 48 adaptive steps, each committed by encode & append (final cache
34816 positions).

* A one-layer model's cache row j holds k, v of token j at position j alone
  (the layer's only attention comes after its K/V projection), so the oracle
  computes any row by itself: sampled rows of the 32768-token encode, and of
  canvases appended at positions 32768 and beyond, against the oracle.
* The denoising step at the last canvas's context (34560 cached keys plus the
  256 canvas keys) over a seeded N(0,1) cache: logits of every canvas position,
  their entropies and the router logits against the oracle (routes forced).
* The 8-canvas generation on the GPU: per-step sampler invariants, the cache
  growing by 256 rows per commit with rows below untouched, and encode &
  append of a canvas equal (within the bar) to one encode of prefix + canvas."""
import numpy as np
import pytest

import synth
from oracle import model as om
from oracle import sampler as smp
from oracle import step as ost
from synth.configs import WORKLOADS

from .gpu_util import allclose_report, bar_or_twin, say
from .test_gpu_full import _invariants
from .test_gpu_model import ATOL, RTOL, ROUTE_EPS, _route_margins

pytestmark = pytest.mark.gpu

SAMPLE_POS = np.array([0, 1, 255, 256, 4095, 16383, 30001, 32766, 32767])
ROWS = np.arange(256)  # every canvas position


@pytest.fixture(scope="module")
def env():
    import torch
    import discrete_text_diffusion_amd as dg
    from discrete_text_diffusion_amd import runtime as rt
    assert torch.cuda.is_available()
    return torch, dg, rt


@pytest.fixture(scope="module")
def longctx(env):
    torch, dg, rt = env
    wl = WORKLOADS["longctx"]
    shape, C = wl.model, wl.canvas
    cap = wl.prefix + wl.n_blocks * C
    say(f"longctx: building the one-layer model, cache capacity {cap}")
    model = rt.DeviceModel(shape, wl.lm_scale)
    ws = rt.Workspace(model.cfg, 1, C)
    return dict(wl=wl, shape=shape, model=model, ws=ws, cap=cap, W=om.Weights(shape))


def _oracle_row_kv(shape, W, token: int, pos: int):
    """k, v [n_kv, d_head] of one token at absolute position pos (layer 0)."""
    oc = om.KVCache(shape, 1, pos + 1)
    oc.length = pos
    om.layer_forward(shape, W, 0, om.embed(shape, W, np.array([[token]])), oc, causal=True, append=True)
    return oc.k[0][0, :, pos], oc.v[0][0, :, pos]


def _check_rows(f, cache, tokens_at, positions, what):
    k, v = cache.view("k"), cache.view("v")
    for p in positions:
        ko, vo = _oracle_row_kv(f["shape"], f["W"], int(tokens_at(p)), int(p))
        allclose_report(f"{what} k row {p}", k[0, 0, :, p].float().cpu().numpy(), ko, ATOL, RTOL)
        allclose_report(f"{what} v row {p}", v[0, 0, :, p].float().cpu().numpy(), vo, ATOL, RTOL)


def test_longctx_denoise_step_at_full_context(env, longctx):
    """One step of the last canvas: 34560 cached keys + 256 canvas keys."""
    torch, dg, rt = env
    f = longctx
    shape, wl, C = f["shape"], f["wl"], f["wl"].canvas
    L = f["cap"] - C
    cache = rt.DeviceCache(shape, 1, f["cap"])
    cache.fill_random(L, seed=0, std=1.0)
    cv = rt.DeviceCanvas(shape, 1, C, [3])
    st = rt.stream_handle()
    dg.dg_init_canvas(model_cfg := f["model"].cfg, cv.struct, 7, st)
    torch.cuda.synchronize()
    tok = cv.tokens.cpu().numpy().reshape(1, C)
    oc = om.KVCache(shape, 1, f["cap"])
    for name, tid in (("k", synth.TID["kv_k"]), ("v", synth.TID["kv_v"])):
        vals = synth.bf16_bits_to_f32(synth.normal(0, tid, (1, 1, shape.n_kv_heads, L, shape.d_head), 1.0))
        getattr(oc, name)[0][:, :, :L] = vals[0].astype(np.float64)
    oc.length = L
    say(f"longctx: oracle denoise forward over {L} + {C} keys")
    tr = {}
    x = om.embed(shape, f["W"], tok)
    x = om.layer_forward(shape, f["W"], 0, x, oc, causal=False, append=False, trace=tr)
    zo = om.final_logits(shape, f["W"], x[:, ROWS], wl.lm_scale)[0]
    say("longctx: fp32 twin on the oracle's routes")
    ids = list(tr["expert_ids"])
    orig = om.route

    def fixed(shape_, r):
        sel = ids.pop(0)
        s_ = np.take_along_axis(r, sel, axis=1)
        e = np.exp(s_ - s_.max(axis=1, keepdims=True))
        return sel, e / e.sum(axis=1, keepdims=True)

    om.route = fixed
    trt = {}
    try:
        with om.accumulation("f32"):
            xt = om.layer_forward(shape, f["W"], 0, om.embed(shape, f["W"], tok), oc, causal=False, append=False,
                                  trace=trt)
            zt = om.final_logits(shape, f["W"], xt[:, ROWS], wl.lm_scale)[0]
    finally:
        om.route = orig
    out = torch.empty(C * shape.vocab, dtype=torch.float32, device="cuda")
    rout = torch.empty(C * shape.n_experts, dtype=torch.float32, device="cuda")
    d_force = torch.from_numpy(np.ascontiguousarray(np.stack(tr["expert_ids"]), dtype=np.int32).reshape(-1)).cuda()
    dg.dg_test_forward_logits(model_cfg, f["model"].weights, cache.struct, cv.struct, rt.step_params(0, wl.n_steps, 7),
                              d_force.data_ptr(), rout.data_ptr(), out.data_ptr(), f["ws"].ptr, f["ws"].size, st)
    torch.cuda.synchronize()
    z = out.view(C, shape.vocab)[torch.from_numpy(ROWS).cuda()].cpu().numpy()
    rg = rout.cpu().numpy().reshape(1, C, shape.n_experts)
    bar_or_twin("longctx router logits (oracle routes)", rg, np.stack(tr["router_logits"]),
                np.stack(trt["router_logits"]), ROUTE_EPS["bf16"], 0.0)
    bar_or_twin("longctx logits (oracle routes)", z, zo, zt, ATOL, RTOL)
    tau = smp.temperature(0, wl.n_steps)
    allclose_report("longctx entropy (oracle routes)", smp.row_statistics(z, tau)[1], smp.row_statistics(zo, tau)[1],
                    1e-3, 0.0)
    say(f"longctx: oracle route margin min {_route_margins(shape, tr).min():.2e}")


def test_longctx_generation(env, longctx):
    torch, dg, rt = env
    f = longctx
    shape, wl, C, V = f["shape"], f["wl"], f["wl"].canvas, f["shape"].vocab
    cfg, st, ws = f["model"].cfg, rt.stream_handle(), f["ws"]
    cache = rt.DeviceCache(shape, 1, f["cap"])
    prompt = synth.tokens(0, synth.TID["prompt"], wl.prefix, V)
    say(f"longctx: encoding the {wl.prefix}-token prefix")
    d_prompt = torch.from_numpy(prompt).cuda()
    dg.dg_encode_append(cfg, f["model"].weights, cache.struct, d_prompt.data_ptr(), 1, wl.prefix, ws.ptr, ws.size, st)
    torch.cuda.synchronize()
    assert cache.length == wl.prefix
    _check_rows(f, cache, lambda p: prompt[p], SAMPLE_POS, "longctx prefix")
    seed = 5
    cv = rt.DeviceCanvas(shape, 1, C, [seed])
    dg.dg_init_canvas(cfg, cv.struct, 0, st)
    steps = []
    for block in range(wl.n_blocks):
        L = cache.length
        head = cache.view("k")[0, 0, :, :L:997].clone()
        cv.prev_argmax.fill_(-1)
        t_used = 0
        for t in range(wl.n_steps):
            dg.dg_denoise_step(cfg, f["model"].weights, cache.struct, cv.struct,
                               rt.step_params(t, wl.n_steps, block, wl.adaptive), ws.ptr, ws.size, st)
            torch.cuda.synchronize()
            nxt = cv.tokens.cpu().numpy()
            acc = cv.accepted.cpu().numpy().astype(bool)
            samp = cv.sample.cpu().numpy()
            fresh = smp.renoise_tokens(seed, t, block, C, V)
            assert np.array_equal(nxt, np.where(acc, samp, fresh))
            assert int(cv.n_accepted.item()) == int(acc.sum()) >= 1
            t_used = t + 1
            if int(cv.stop.item()):
                break
        steps.append(t_used)
        dg.dg_commit_block(cfg, f["model"].weights, cache.struct, cv.struct, rt.step_params(t_used - 1, wl.n_steps, block),
                           ws.ptr, ws.size, st)
        torch.cuda.synchronize()
        assert cache.length == L + C
        assert torch.equal(head, cache.view("k")[0, 0, :, :L:997])
        assert np.array_equal(cv.tokens.cpu().numpy(), smp.initial_canvas(seed, block + 1, C, V))
        say(f"longctx: block {block} committed after {t_used} steps, cache {cache.length}")
    assert cache.length == f["cap"] == 34816
    # encode & append of a canvas of known tokens at the full context, then the
    # same canvas at the same positions in one encode with its prefix
    say("longctx: appended rows of oracle-chosen tokens at positions 34560..")
    L = cache.length - C
    cache.struct.length = L
    canvas_tok = synth.tokens(9, synth.TID["prompt"], C, V)
    cv.argmax.copy_(torch.from_numpy(canvas_tok))
    dg.dg_commit_block(cfg, f["model"].weights, cache.struct, cv.struct, rt.step_params(0, wl.n_steps, 8), ws.ptr,
                       ws.size, st)
    torch.cuda.synchronize()
    _check_rows(f, cache, lambda p: canvas_tok[p - L], L + np.array([0, 1, 100, 254, 255]), "longctx appended")
    # P8 at 32768 positions: encode(prefix) then append(canvas) gives the
    # rows of one encode(prefix + canvas) (the same 1024-token chunks and a
    # final 256-token chunk on both sides, so the same arithmetic)
    say("longctx: append vs one encode of prefix + canvas")
    one = rt.DeviceCache(shape, 1, wl.prefix + C)
    dg.dg_encode_append(cfg, f["model"].weights, one.struct, d_prompt.data_ptr(), 1, wl.prefix, ws.ptr, ws.size, st)
    dg.dg_commit_block(cfg, f["model"].weights, one.struct, cv.struct, rt.step_params(0, wl.n_steps, 8), ws.ptr,
                       ws.size, st)
    two = rt.DeviceCache(shape, 1, wl.prefix + C)
    d_all = torch.from_numpy(np.concatenate([prompt, canvas_tok]).astype(np.int32)).cuda()
    dg.dg_encode_append(cfg, f["model"].weights, two.struct, d_all.data_ptr(), 1, wl.prefix + C, ws.ptr, ws.size, st)
    torch.cuda.synchronize()
    for name in ("k", "v"):
        x, y = one.view(name), two.view(name)
        nd = int((x != y).sum().item())
        say(f"longctx append vs one encode ({name}): {nd} differing elements")
        assert nd == 0
    say(f"longctx: steps per block {steps}")
