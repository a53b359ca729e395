"""GPU parity of the full path (encode, forward logits, denoising loop,
commit) against the oracle on the same seeded inputs."""
import numpy as np
import pytest

import synth
from oracle import model as om
from oracle import sampler as smp
from oracle import step as ost
from synth.configs import MINI_BF16, TINY, WORKLOADS

from .gpu_util import allclose_report, compare_decisions, say

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2  # logits bar (bf16); fp32 models are held to the same bar and print their error


@pytest.fixture(scope="module")
def env():
    import torch
    import discrete_text_diffusion_amd as dg
    from discrete_text_diffusion_amd import runtime as rt
    assert torch.cuda.is_available()
    return torch, dg, rt


class Problem:
    """Same model, prompt and canvas on both sides."""

    def __init__(self, env, shape, lm_scale, prefix, C, B=1, cap_extra=0, seeds=None):
        torch, dg, rt = env
        self.env = env
        self.shape, self.C, self.B, self.prefix = shape, C, B, prefix
        self.lm_scale = lm_scale
        self.seeds = seeds or [17 + b for b in range(B)]
        self.cap = prefix + C + cap_extra
        self.cfg = rt.model_config(shape)
        self.model = rt.DeviceModel(shape, lm_scale)
        self.cache = rt.DeviceCache(shape, B, self.cap)
        self.canvas = rt.DeviceCanvas(shape, B, C, self.seeds)
        self.ws = rt.Workspace(self.cfg, B, C)
        self.st = rt.stream_handle()
        self.W = om.Weights(shape)
        self.ocache = om.KVCache(shape, B, self.cap)
        self.prompt = np.stack([synth.tokens(b, synth.TID["prompt"], prefix, shape.vocab) for b in range(B)])

    def encode_prefix(self):
        torch, dg, rt = self.env
        say(f"encode prefix {self.prefix} (B={self.B})")
        d_tok = torch.from_numpy(self.prompt.astype(np.int32).reshape(-1)).cuda()
        dg.dg_encode_append(self.cfg, self.model.weights, self.cache.struct, d_tok.data_ptr(), self.B, self.prefix,
                            self.ws.ptr, self.ws.size, self.st)
        torch.cuda.synchronize()
        ost.encode_append(self.shape, self.W, self.ocache, self.prompt)

    def compare_cache(self, rows):
        torch = self.env[0]
        for name, ocache in (("k", self.ocache.k), ("v", self.ocache.v)):
            got = self.cache.view(name).float().cpu().numpy()
            for l in range(self.shape.n_layers):
                allclose_report(f"cache {name} L{l}", got[l][:, :, :rows], ocache[l][:, :, :rows], ATOL, RTOL)


@pytest.fixture(scope="module")
def tiny(env):
    wl = WORKLOADS["tiny"]
    pb = Problem(env, wl.model, wl.lm_scale, wl.prefix, wl.canvas, cap_extra=wl.canvas)
    pb.encode_prefix()
    return pb


@pytest.fixture(scope="module")
def mini(env):
    pb = Problem(env, MINI_BF16, 6.0, 40, 48, B=2, cap_extra=48)
    pb.encode_prefix()
    return pb


def _forward_logits(pb, t, n_steps, sc_probs=None, force_ids=None):
    torch, dg, rt = pb.env
    T = pb.B * pb.C
    out = torch.empty(T * pb.shape.vocab, dtype=torch.float32, device="cuda")
    if sc_probs is not None:
        pb.canvas.set_sc_probs(torch.from_numpy(sc_probs.astype(np.float32).reshape(-1)).cuda())
    d_force = None
    if force_ids is not None:
        d_force = torch.from_numpy(np.ascontiguousarray(force_ids, dtype=np.int32).reshape(-1)).cuda()
    dg.dg_test_forward_logits(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct,
                              rt.step_params(t, n_steps), d_force.data_ptr() if d_force is not None else None,
                              out.data_ptr(), pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    pb.canvas.set_sc_probs(None)
    return out.cpu().numpy().reshape(pb.B, pb.C, pb.shape.vocab)


def _route_margins(shape, trace):
    """Per layer and token: gap between the k-th and (k+1)-th router logit."""
    out = []
    for r in trace["router_logits"]:
        srt = -np.sort(-r, axis=1)
        out.append(srt[:, shape.top_k - 1] - srt[:, shape.top_k] if shape.top_k < shape.n_experts
                   else np.full(r.shape[0], np.inf))
    return np.stack(out)


def _forced_ids(trace):
    return np.stack(trace["expert_ids"])  # [layers][T][k]


@pytest.mark.parametrize("which", ["tiny", "mini"])
def test_encode_cache_matches_oracle(which, request):
    pb = request.getfixturevalue(which)
    pb.compare_cache(pb.prefix)


@pytest.mark.parametrize("which", ["tiny", "mini"])
def test_forward_logits_match_oracle(which, request):
    pb = request.getfixturevalue(which)
    torch, dg, rt = pb.env
    say(f"forward logits {which}")
    dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 0, pb.st)
    torch.cuda.synchronize()
    tok = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
    for b in range(pb.B):
        assert np.array_equal(tok[b], smp.initial_canvas(pb.seeds[b], 0, pb.C, pb.shape.vocab))
    k_before = pb.cache.k.clone()
    tr = {}
    zo = ost.denoise_logits(pb.shape, pb.W, pb.ocache, tok, None, pb.lm_scale, trace=tr)
    margins = _route_margins(pb.shape, tr)
    say(f"oracle routing margins: min {margins.min():.3e}, #<1e-3: {int((margins < 1e-3).sum())}")
    # routes forced to the oracle's choice: continuous outputs must match
    z = _forward_logits(pb, 0, 48, force_ids=_forced_ids(tr))
    assert torch.equal(k_before, pb.cache.k), "denoiser wrote the cache"
    allclose_report(f"logits {which} (oracle routes)", z, zo, ATOL, RTOL)
    _, Hg, _ = smp.row_statistics(z.reshape(-1, pb.shape.vocab), smp.temperature(0, 48))
    _, Ho, _ = smp.row_statistics(zo.reshape(-1, pb.shape.vocab), smp.temperature(0, 48))
    allclose_report(f"entropy of logits {which} (oracle routes)", Hg, Ho, 1e-3, 0.0)
    # unforced: report how far routing near-ties move the result
    zu = _forward_logits(pb, 0, 48)
    du = np.abs(zu - zo).max(axis=-1).reshape(-1)
    say(f"unforced: rows with max|dz| > {ATOL}: {int((du > ATOL).sum())} of {du.size}; max {du.max():.3e}")
    # self-conditioning from an external distribution
    rng = np.random.default_rng(1)
    P = rng.dirichlet(np.full(pb.shape.vocab, 0.05), size=pb.B * pb.C).reshape(pb.B, pb.C, -1)
    P = P.astype(np.float32)
    tr2 = {}
    zo2 = ost.denoise_logits(pb.shape, pb.W, pb.ocache, tok, P.astype(np.float64), pb.lm_scale, trace=tr2)
    z2 = _forward_logits(pb, 1, 48, P, force_ids=_forced_ids(tr2))
    allclose_report(f"logits+selfcond {which} (oracle routes)", z2, zo2, ATOL, RTOL)
    assert np.abs(zo2 - zo).max() > 1e-3  # the self-conditioning term is not negligible


@pytest.mark.parametrize("which", ["tiny", "mini"])
def test_denoise_loop_and_commit_match_oracle(which, request):
    """Up to 48 adaptive steps compared step by step (canvas, entropies,
    argmax, accepted set, next tokens, stop), then the commit.  The comparison
    stops early only at a reported near-tie (a routing margin or a decision
    margin below the fp32/bf16 error), where both trajectories are valid."""
    pb = request.getfixturevalue(which)
    torch, dg, rt = pb.env
    say(f"denoise loop {which}")
    n_steps = 48
    L0 = pb.cache.length
    dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 0, pb.st)
    pb.canvas.prev_argmax.fill_(-1)
    torch.cuda.synchronize()
    otok = np.stack([smp.initial_canvas(s, 0, pb.C, pb.shape.vocab) for s in pb.seeds])
    oprev = None
    osc = None
    steps = 0
    for t in range(n_steps):
        tr = {}
        z, outs = ost.denoise_step(pb.shape, pb.W, pb.ocache, otok, osc, t, n_steps, pb.seeds, 0, pb.lm_scale,
                                   oprev, True, trace=tr)
        rmin = float(_route_margins(pb.shape, tr).min())
        if rmin < 2e-3:
            say(f"step {t}: oracle routing margin {rmin:.2e} is a near-tie; stopping the step-by-step comparison")
            break
        gtok_in = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
        assert np.array_equal(gtok_in, otok), f"canvas diverged before step {t}"
        dg.dg_denoise_step(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct,
                           rt.step_params(t, n_steps, block=0, adaptive=True), pb.ws.ptr, pb.ws.size, pb.st)
        torch.cuda.synchronize()
        H = pb.canvas.entropy.cpu().numpy().reshape(pb.B, pb.C)
        am = pb.canvas.argmax.cpu().numpy().reshape(pb.B, pb.C)
        acc = pb.canvas.accepted.cpu().numpy().reshape(pb.B, pb.C).astype(bool)
        stop = pb.canvas.stop.cpu().numpy()
        gnext = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
        ties = 0
        for b, o in enumerate(outs):
            herr = np.abs(H[b] - o["H"]).max()
            assert herr < 1e-3, f"step {t}: entropy error {herr}"
            ties += compare_decisions(f"t{t} argmax", am[b], o["argmax"], o["margin_argmax"], 2 * ATOL, max_ties=2)
            ties += compare_decisions(f"t{t} accepted", acc[b], o["accepted"], o["margin_accept"], 2e-3, max_ties=2)
            ties += compare_decisions(f"t{t} next tokens", gnext[b], o["next_tokens"],
                                      np.where(o["accepted"], o["margin_sample"], 1.0), 1e-5, max_ties=1)
            assert int(stop[b]) == int(o["stop"]) or o["margin_stop"] < 1e-3
        steps = t + 1
        oprev = np.stack([o["argmax"] for o in outs])
        otok = np.stack([o["next_tokens"] for o in outs])
        osc = np.stack([o["p"] for o in outs])
        if ties:
            say(f"near-tie decision at step {t}; stopping the step-by-step comparison")
            if not np.array_equal(am, oprev):
                return
            break
        if all(o["stop"] for o in outs):
            say(f"{which}: adaptive stop at step {t}")
            break
    say(f"{which}: {steps} steps compared")
    assert steps >= 1
    # commit: argmax of the last step appended by the causal encoder
    dg.dg_commit_block(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct,
                       rt.step_params(steps - 1, n_steps, block=0), pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    com = pb.canvas.committed.cpu().numpy().reshape(pb.B, pb.C)
    assert np.array_equal(com, oprev)
    assert pb.cache.length == L0 + pb.C
    ost.encode_append(pb.shape, pb.W, pb.ocache, com)
    pb.compare_cache(pb.cache.length)
    nxt = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
    for b in range(pb.B):
        assert np.array_equal(nxt[b], smp.initial_canvas(pb.seeds[b], 1, pb.C, pb.shape.vocab))


def test_denoise_step_is_deterministic(mini):
    pb = mini
    torch, dg, rt = pb.env
    say("determinism")
    outs = []
    for rep in range(2):
        dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 5, pb.st)
        dg.dg_denoise_step(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct, rt.step_params(0, 12, 5),
                           pb.ws.ptr, pb.ws.size, pb.st)
        dg.dg_denoise_step(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct, rt.step_params(1, 12, 5),
                           pb.ws.ptr, pb.ws.size, pb.st)
        torch.cuda.synchronize()
        outs.append([x.clone() for x in (pb.canvas.tokens, pb.canvas.entropy, pb.canvas.p_side, pb.canvas.p_scale)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
