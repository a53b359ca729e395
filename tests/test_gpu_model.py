"""GPU parity of the full path (encode, forward logits, denoising loop,
commit) against the oracle on the same seeded inputs."""
import numpy as np
import pytest

import synth
from oracle import model as om
from oracle import sampler as smp
from oracle import step as ost
from dataclasses import replace

from synth.configs import MINI_BF16, TINY, WORKLOADS

# the small bf16 shape with fp8 expert and LM-head weights, and with MXFP4 experts
MINI_FP8 = replace(MINI_BF16, expert_dtype="fp8", lm_dtype="fp8")
MINI_MX4 = replace(MINI_BF16, expert_dtype="mxfp4")

from .gpu_util import allclose_report, bar_or_twin, bar_then_twin, compare_decisions, compare_step_decisions, say

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2  # logits bar (bf16); fp32 models are held to the same bar and print their error
ATOL_FP8 = 3e-2          # logits bar with fp8 expert / LM-head weights


def atol_for(shape):
    return ATOL_FP8 if "fp8" in (shape.expert_dtype, shape.lm_dtype) else ATOL


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
        self.atol = atol_for(shape)
        self.lm_scale = lm_scale
        self.seeds = seeds or [17 + b for b in range(B)]
        self.cap = prefix + C + cap_extra
        self.cfg = rt.model_config(shape)
        self.model = rt.DeviceModel(shape, lm_scale)
        self.cache = rt.DeviceCache(shape, B, self.cap)
        self.canvas = rt.DeviceCanvas(shape, B, C, self.seeds)
        self.ws = rt.Workspace(self.cfg, B, C)
        self.guard_workspace(self.ws)
        self.st = rt.stream_handle()
        self.W = om.Weights(shape)
        self.ocache = om.KVCache(shape, B, self.cap)
        self.prompt = np.stack([synth.tokens(b, synth.TID["prompt"], prefix, shape.vocab) for b in range(B)])

    GUARD = 4 << 20

    def guard_workspace(self, ws):
        """Re-seat ws on a buffer followed by GUARD bytes of 0xA5 (checked by
        check_guards: no launch may write past dg_workspace_bytes)."""
        torch = self.env[0]
        buf = torch.full((ws.size + 256 + self.GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
        off = (-buf.data_ptr()) % 256
        ws.buf, ws.ptr = buf, buf.data_ptr() + off
        self.guards = getattr(self, "guards", []) + [buf[off + ws.size:off + ws.size + self.GUARD]]
        return ws

    def check_guards(self):
        self.env[0].cuda.synchronize()
        for g in self.guards:
            assert bool((g == 0xA5).all()), "a launch wrote past the workspace"

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
                allclose_report(f"cache {name} L{l}", got[l][:, :, :rows], ocache[l][:, :, :rows], self.atol, RTOL)


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


@pytest.fixture(scope="module")
def tiny_tied(env):
    # LM head tied to the embedding: the model predicts its own input tokens
    # with confidence, the canvas reaches a fixed point and the adaptive stop
    # fires (at the second step)
    wl = WORKLOADS["tiny"]
    pb = Problem(env, replace(wl.model, tied_head=True), 20.0, wl.prefix, wl.canvas, cap_extra=wl.canvas)
    pb.encode_prefix()
    return pb


@pytest.fixture(scope="module")
def mini_tied(env):
    # the same for the bf16 mini model: partial acceptance for a dozen steps,
    # then both canvases stop in the same step (the 13th)
    pb = Problem(env, replace(MINI_BF16, tied_head=True), 60.0, 40, 48, B=2, cap_extra=48)
    pb.encode_prefix()
    return pb


@pytest.fixture(scope="module")
def mini8(env):
    pb = Problem(env, MINI_FP8, 6.0, 40, 48, B=2, cap_extra=48)
    pb.encode_prefix()
    return pb


@pytest.fixture(scope="module")
def mini4(env):
    pb = Problem(env, MINI_MX4, 6.0, 40, 48, B=2, cap_extra=48)
    pb.encode_prefix()
    return pb


def _forward_logits(pb, t, n_steps, sc_probs=None, force_ids=None, want_router=False):
    torch, dg, rt = pb.env
    T = pb.B * pb.C
    out = torch.empty(T * pb.shape.vocab, dtype=torch.float32, device="cuda")
    rout = torch.empty(pb.shape.n_layers * T * pb.shape.n_experts, dtype=torch.float32, device="cuda")
    if sc_probs is not None:
        pb.canvas.set_sc_probs(torch.from_numpy(sc_probs.astype(np.float32).reshape(-1)).cuda())
    d_force = None
    if force_ids is not None:
        d_force = torch.from_numpy(np.ascontiguousarray(force_ids, dtype=np.int32).reshape(-1)).cuda()
    dg.dg_test_forward_logits(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct,
                              rt.step_params(t, n_steps), d_force.data_ptr() if d_force is not None else None,
                              rout.data_ptr(), out.data_ptr(), pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    pb.canvas.set_sc_probs(None)
    z = out.cpu().numpy().reshape(pb.B, pb.C, pb.shape.vocab)
    if want_router:
        return z, rout.cpu().numpy().reshape(pb.shape.n_layers, T, pb.shape.n_experts)
    return z


def _err_summary(name, got, want):
    e = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64)).reshape(-1)
    q = np.quantile(e, [0.5, 0.99, 0.9999]) if e.size else [0, 0, 0]
    say(f"{name}: |err| median {q[0]:.2e}  p99 {q[1]:.2e}  p99.99 {q[2]:.2e}  max {e.max():.2e}")
    return float(e.max())


# Router-logit margin below which a route decision counts as a near-tie: a few
# times the largest GPU-vs-oracle router-logit error measured with the
# oracle's routes forced (fp32: ~5e-7; bf16: ~2e-3, the tail where a bf16
# rounding of an activation fell on the other side of a boundary and
# propagated).
ROUTE_EPS = {"f32": 1e-5, "bf16": 5e-3}


def flip_margin_bound(got, want, dtype="bf16"):
    """Largest oracle margin (k-th minus (k+1)-th router logit) at which a
    GPU route may differ from the oracle's: a flip needs the two logits'
    errors to sum past the margin, so twice the largest router-logit error
    measured with the oracle's routes forced (that error is itself held to
    the fp32 twin), and at least the fixed near-tie threshold."""
    e = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    return max(ROUTE_EPS[dtype], 2.0 * float(e.max()) if e.size else 0.0)


# Typical (median) router-logit error bound with forced routes.
ROUTE_MEDIAN = {"f32": 1e-6, "bf16": 1e-4}


def check_sampler_invariants(pb, t, n_steps, prev_before, adaptive=True, block=0):
    """Properties every step must satisfy, checked on the GPU's own outputs
    against the sampler's definition (entropy-bounded acceptance, Philox
    re-noise, stop rule)."""
    B, C, V = pb.B, pb.C, pb.shape.vocab
    H = pb.canvas.entropy.cpu().numpy().reshape(B, C).astype(np.float64)
    acc = pb.canvas.accepted.cpu().numpy().reshape(B, C).astype(bool)
    samp = pb.canvas.sample.cpu().numpy().reshape(B, C)
    am = pb.canvas.argmax.cpu().numpy().reshape(B, C)
    nxt = pb.canvas.tokens.cpu().numpy().reshape(B, C)
    nacc = pb.canvas.n_accepted.cpu().numpy()
    stop = pb.canvas.stop.cpu().numpy()
    mean = pb.canvas.mean_entropy.cpu().numpy()
    for b in range(B):
        K = int(acc[b].sum())
        assert K == nacc[b] >= 1
        order = np.lexsort((np.arange(C), H[b]))
        assert set(np.nonzero(acc[b])[0]) == set(order[:K])      # the K lowest entropies
        if K > 1:
            assert H[b][acc[b]].sum() <= 0.1 + 1e-5
        if K < C:
            assert np.sort(H[b])[:K + 1].sum() > 0.1 - 1e-5      # one more would break the bound
        fresh = smp.renoise_tokens(pb.seeds[b], t, block, C, V)
        assert np.array_equal(nxt[b], np.where(acc[b], samp[b], fresh))
        assert abs(mean[b] - H[b].mean()) < 1e-5
        want_stop = adaptive and t >= 1 and mean[b] < 0.005 and prev_before is not None and \
            np.array_equal(am[b], prev_before[b])
        assert int(stop[b]) == int(want_stop)
    return am.copy()


def _route_margins(shape, trace):
    """Per layer and token: gap between the k-th and (k+1)-th router logit."""
    out = []
    for r in trace["router_logits"]:
        srt = -np.sort(-r, axis=1)
        out.append(srt[:, shape.top_k - 1] - srt[:, shape.top_k] if shape.top_k < shape.n_experts
                   else np.full(r.shape[0], np.inf))
    return np.stack(out)


def entropy_tolerance(z_oracle, tau, atol=ATOL):
    """Per-row entropy bar: the pages' 1e-3 nats, or the first-order entropy
    change the logit bar allows, whichever is larger.  With a = z/tau,
    dH = -sum_v p_v (a_v - E_p[a]) da_v, so |dH| <= E_p[|a - E_p a| (2e-2 + 1e-2|z|)] / tau.
    For the pages' workloads (near-uniform rows) this is below 1e-3; sharp
    test shapes need the propagated bound."""
    p, _, _ = smp.row_statistics(z_oracle, tau)
    a = z_oracle / tau
    abar = (p * a).sum(-1, keepdims=True)
    prop = (p * np.abs(a - abar) * (atol + RTOL * np.abs(z_oracle))).sum(-1) / tau
    return np.maximum(1e-3, prop)


def _forced_ids(trace):
    return np.stack(trace["expert_ids"])  # [layers][T][k]


@pytest.mark.parametrize("which", ["tiny", "mini", "mini8", "mini4"])
def test_encode_cache_matches_oracle(which, request):
    pb = request.getfixturevalue(which)
    pb.compare_cache(pb.prefix)
    pb.check_guards()


@pytest.mark.parametrize("which", ["tiny", "mini", "mini8", "mini4"])
def test_forward_logits_match_oracle(which, request):
    pb = request.getfixturevalue(which)
    torch, dg, rt = pb.env
    say(f"forward logits {which}")
    dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 0, pb.st)
    torch.cuda.synchronize()
    tok = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
    for b in range(pb.B):
        assert np.array_equal(tok[b], smp.initial_canvas(pb.seeds[b], 0, pb.C, pb.shape.vocab))
    kv_before = pb.cache.valid_rows()
    tr = {}
    zo = ost.denoise_logits(pb.shape, pb.W, pb.ocache, tok, None, pb.lm_scale, trace=tr)
    margins = _route_margins(pb.shape, tr)
    say(f"oracle routing margins: min {margins.min():.3e}, #<1e-3: {int((margins < 1e-3).sum())}")
    # routes forced to the oracle's choice: continuous outputs must match
    z, rg = _forward_logits(pb, 0, 48, force_ids=_forced_ids(tr), want_router=True)
    assert all(torch.equal(x, y) for x, y in zip(kv_before, pb.cache.valid_rows())), "denoiser wrote cache rows < length"
    ro = np.stack(tr["router_logits"])
    rerr = _err_summary(f"router logits {which} (oracle routes)", rg, ro)
    assert float(np.median(np.abs(rg - ro))) < ROUTE_MEDIAN[pb.shape.dtype]
    assert rerr < ROUTE_EPS[pb.shape.dtype]
    _err_summary(f"logits {which} (oracle routes)", z, zo)
    _, Hg, _ = smp.row_statistics(z.reshape(-1, pb.shape.vocab), smp.temperature(0, 48))
    _, Ho, _ = smp.row_statistics(zo.reshape(-1, pb.shape.vocab), smp.temperature(0, 48))
    _err_summary(f"entropy {which} (oracle routes)", Hg, Ho)
    allclose_report(f"logits {which} (oracle routes)", z, zo, pb.atol, RTOL)
    allclose_report(f"entropy of logits {which} (oracle routes)", Hg, Ho,
                    entropy_tolerance(zo.reshape(-1, pb.shape.vocab), smp.temperature(0, 48), pb.atol), 0.0)
    # unforced: the first layer sees the same inputs; any route that differs
    # there must be an oracle near-tie
    zu, ru = _forward_logits(pb, 0, 48, want_router=True)
    k = pb.shape.top_k
    gtop = np.sort(np.argsort(-ru[0], axis=1, kind="stable")[:, :k], axis=1)
    otop = np.sort(tr["expert_ids"][0], axis=1)
    flips = np.nonzero(np.any(gtop != otop, axis=1))[0]
    say(f"unforced: layer-0 route flips {flips.size} (oracle margins {margins[0][flips]})")
    assert np.all(margins[0][flips] < ROUTE_EPS[pb.shape.dtype])
    du = np.abs(zu - zo).max(axis=-1).reshape(-1)
    say(f"unforced: rows with max|dz| > {pb.atol}: {int((du > pb.atol).sum())} of {du.size}; max {du.max():.3e}")
    # self-conditioning from an external distribution
    rng = np.random.default_rng(1)
    P = rng.dirichlet(np.full(pb.shape.vocab, 0.05), size=pb.B * pb.C).reshape(pb.B, pb.C, -1)
    P = P.astype(np.float32)
    tr2 = {}
    zo2 = ost.denoise_logits(pb.shape, pb.W, pb.ocache, tok, P.astype(np.float64), pb.lm_scale, trace=tr2)
    z2 = _forward_logits(pb, 1, 48, P, force_ids=_forced_ids(tr2))
    allclose_report(f"logits+selfcond {which} (oracle routes)", z2, zo2, pb.atol, RTOL)
    assert np.abs(zo2 - zo).max() > 1e-3  # the self-conditioning term is not negligible
    pb.check_guards()


@pytest.mark.parametrize("which", ["tiny", "mini", "mini8", "mini4"])
def test_denoise_loop_and_commit_match_oracle(which, request):
    """48 adaptive steps on the GPU.  Every step is checked against the
    sampler's definition (check_sampler_invariants).  The oracle runs the same
    trajectory and is compared step by step (canvas, entropies, argmax,
    accepted set, next tokens, stop) until the first near-tie (a routing or
    decision margin below the measured GPU-vs-oracle error), after which both
    trajectories are valid and only the invariants are checked.  Then the
    commit is compared with the oracle's encode & append of the same tokens."""
    pb = request.getfixturevalue(which)
    torch, dg, rt = pb.env
    say(f"denoise loop {which}")
    n_steps = 48
    L0 = pb.cache.length
    dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 0, pb.st)
    pb.canvas.prev_argmax.fill_(-1)
    torch.cuda.synchronize()
    otok = np.stack([smp.initial_canvas(s, 0, pb.C, pb.shape.vocab) for s in pb.seeds])
    oprev, osc = None, None
    tracking = True
    compared = 0
    gprev = None
    t_last = 0
    for t in range(n_steps):
        if tracking:
            tr = {}
            z, outs = ost.denoise_step(pb.shape, pb.W, pb.ocache, otok, osc, t, n_steps, pb.seeds, 0, pb.lm_scale,
                                       oprev, True, trace=tr)
            rmin = float(_route_margins(pb.shape, tr).min())
            if rmin < ROUTE_EPS[pb.shape.dtype]:
                say(f"step {t}: oracle routing margin {rmin:.2e} is a near-tie; oracle comparison ends here")
                tracking = False
        gtok_in = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
        if tracking:
            assert np.array_equal(gtok_in, otok), f"canvas diverged before step {t}"
        dg.dg_denoise_step(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct,
                           rt.step_params(t, n_steps, block=0, adaptive=True), pb.ws.ptr, pb.ws.size, pb.st)
        torch.cuda.synchronize()
        am = check_sampler_invariants(pb, t, n_steps, gprev)
        gprev = am
        t_last = t
        if tracking:
            H = pb.canvas.entropy.cpu().numpy().reshape(pb.B, pb.C)
            acc = pb.canvas.accepted.cpu().numpy().reshape(pb.B, pb.C).astype(bool)
            gnext = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
            stop = pb.canvas.stop.cpu().numpy()
            ties = 0
            for b, o in enumerate(outs):
                herr = np.abs(H[b] - o["H"])
                tol = entropy_tolerance(z[b], o["tau"], pb.atol)
                assert np.all(herr <= tol), f"step {t}: entropy error {herr.max()} (bar {tol.min()})"
                ties += compare_decisions(f"t{t} argmax", am[b], o["argmax"], o["margin_argmax"], 2 * pb.atol, max_ties=2)
                ties += compare_decisions(f"t{t} accepted", acc[b], o["accepted"], o["margin_accept"], 2e-3,
                                          max_ties=2)
                ties += compare_decisions(f"t{t} next tokens", gnext[b], o["next_tokens"],
                                          np.where(o["accepted"], o["margin_sample"], 1.0), 1e-5, max_ties=1)
                assert int(stop[b]) == int(o["stop"]) or o["margin_stop"] < 1e-3
            compared = t + 1
            oprev = np.stack([o["argmax"] for o in outs])
            otok = np.stack([o["next_tokens"] for o in outs])
            osc = np.stack([o["p"] for o in outs])
            if ties:
                say(f"near-tie decision at step {t}; oracle comparison ends here")
                tracking = False
        if int(pb.canvas.stop.cpu().numpy().min()) == 1:
            say(f"{which}: adaptive stop at step {t}")
            break
    say(f"{which}: {t_last + 1} GPU steps checked against the definition, {compared} compared with the oracle")
    # commit: the last step's argmax is appended by the causal encoder.  The
    # tokens come from the oracle's trajectory (its last compared argmax, or
    # its initial canvas), written into the GPU's argmax slot, so the cache
    # comparison uses no GPU-derived input on the oracle side.
    ocom = oprev if oprev is not None else otok
    pb.canvas.argmax.copy_(torch.from_numpy(np.ascontiguousarray(ocom, dtype=np.int32).reshape(-1)))
    dg.dg_commit_block(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct,
                       rt.step_params(t_last, n_steps, block=0), pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    com = pb.canvas.committed.cpu().numpy().reshape(pb.B, pb.C)
    assert np.array_equal(com, ocom)
    assert pb.cache.length == L0 + pb.C
    ost.encode_append(pb.shape, pb.W, pb.ocache, ocom)
    pb.compare_cache(pb.cache.length)
    nxt = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
    for b in range(pb.B):
        assert np.array_equal(nxt[b], smp.initial_canvas(pb.seeds[b], 1, pb.C, pb.shape.vocab))
    pb.check_guards()


@pytest.mark.parametrize("which", ["tiny", "mini", "mini8", "mini4", "tiny_tied", "mini_tied"])
def test_forced_route_loop_matches_oracle(which, request):
    """Every step of a 12-step schedule (48 steps with adaptive stopping for
    the tied-head models, until the oracle stops) compared with the oracle on the
    oracle's routes (dg_test_denoise_step: the product's whole step with
    every layer's experts forced).  The GPU carries its own self-conditioning
    input from step to step (the previous step's tempered distribution,
    normalised in place by its sampler: bf16 for the bf16 models), while the
    oracle uses its own fp64 distribution; each step's canvas tokens and
    previous argmax are the oracle's, so a near-tie decision in one step does
    not end the comparison.  Per step: logits within the bar (or the fp32-twin
    criterion), the device's own entropies within the entropy bar, decisions
    equal up to margin-certified near-ties."""
    pb = request.getfixturevalue(which)
    torch, dg, rt = pb.env
    shape, B, C, V = pb.shape, pb.B, pb.C, pb.shape.vocab
    tied = shape.tied_head
    N = 48 if tied else 12
    stopped_at = None
    tsc = None  # the fp32 twin's own self-conditioning input
    say(f"forced-route loop {which}")
    dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 0, pb.st)
    pb.canvas.prev_argmax.fill_(-1)
    torch.cuda.synchronize()
    otok = np.stack([smp.initial_canvas(s, 0, C, V) for s in pb.seeds])
    assert np.array_equal(pb.canvas.tokens.cpu().numpy().reshape(B, C), otok)
    oprev, osc = None, None
    worst_dz, worst_dh, ties = 0.0, 0.0, 0
    out = torch.empty(B * C * V, dtype=torch.float32, device="cuda")
    for t in range(N):
        tr = {}
        zo, outs = ost.denoise_step(shape, pb.W, pb.ocache, otok, osc, t, N, pb.seeds, 0, pb.lm_scale, oprev, True,
                                    trace=tr)
        pb.canvas.tokens.copy_(torch.from_numpy(np.ascontiguousarray(otok, dtype=np.int32).reshape(-1)))
        if oprev is not None:
            pb.canvas.prev_argmax.copy_(torch.from_numpy(np.ascontiguousarray(oprev, dtype=np.int32).reshape(-1)))
        d_force = torch.from_numpy(np.ascontiguousarray(_forced_ids(tr), dtype=np.int32).reshape(-1)).cuda()
        dg.dg_test_denoise_step(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct,
                                rt.step_params(t, N, block=0, adaptive=True), d_force.data_ptr(), None,
                                out.data_ptr(), pb.ws.ptr, pb.ws.size, pb.st)
        torch.cuda.synchronize()
        z = out.cpu().numpy().reshape(B, C, V)
        H = pb.canvas.entropy.cpu().numpy().reshape(B, C).astype(np.float64)
        am = pb.canvas.argmax.cpu().numpy().reshape(B, C)
        acc = pb.canvas.accepted.cpu().numpy().reshape(B, C).astype(bool)
        samp = pb.canvas.sample.cpu().numpy().reshape(B, C)
        nxt = pb.canvas.tokens.cpu().numpy().reshape(B, C)
        stop = pb.canvas.stop.cpu().numpy()

        # The fp32 twin runs a trajectory of its own, like the GPU: the same
        # canvas and routes, and its own previous step's distribution as the
        # self-conditioning input, so its error against the oracle carries the
        # same step-to-step drift as the GPU's (the GPU's input comes from its
        # own logits, not the oracle's).
        def twin():
            with om.accumulation("f32"):
                return _f32_twin_on_inputs(pb, otok, tsc, tr["expert_ids"])

        zt = twin()
        calls = [0]

        def twin_fn():
            calls[0] += 1
            return zt if calls[0] == 1 else twin()

        bar_then_twin(f"loop {which} t{t} logits", z, zo, twin_fn, pb.atol, RTOL)
        for b, o in enumerate(outs):
            tol = entropy_tolerance(zo[b], o["tau"], pb.atol)
            allclose_report(f"loop {which} t{t} b{b} device entropy", H[b], o["H"], tol, 0.0)
            ties += compare_step_decisions(f"loop {which} t{t} b{b}", z[b], H[b], am[b], acc[b], samp[b], nxt[b],
                                           stop[b], dict(o, z=zo[b]))
        worst_dz = max(worst_dz, float(np.abs(z - zo).max()))
        worst_dh = max(worst_dh, float(np.abs(H - np.stack([o["H"] for o in outs])).max()))
        tsc = np.stack([smp.sample_from_logits(zt[b], t, N, pb.seeds[b], 0, None, True)["p"] for b in range(B)])
        oprev = np.stack([o["argmax"] for o in outs])
        otok = np.stack([o["next_tokens"] for o in outs])
        osc = np.stack([o["p"] for o in outs])
        if all(o["stop"] for o in outs):
            # the oracle's adaptive stop: every canvas's flag set on the device too
            assert stop.tolist() == [1] * B, (t, stop)
            stopped_at = t
            break
    say(f"forced-route loop {which}: {t + 1} steps compared; max |dz| {worst_dz:.2e}, max |dH| {worst_dh:.2e}, "
        f"near-tie decisions {ties}; adaptive stop at step {stopped_at}")
    if tied:
        assert stopped_at is not None and stopped_at < N - 1
    pb.check_guards()


def _f32_twin_on_inputs(pb, tok, sc, expert_ids):
    """The oracle's logits on the given canvas and self-conditioning input,
    every layer's experts fixed to expert_ids (used inside an accumulation
    context)."""
    ids = list(expert_ids)
    orig = om.route

    def fixed(shape_, r):
        sel = ids.pop(0)
        s_ = np.take_along_axis(r, sel, axis=1)
        e = np.exp(s_ - s_.max(axis=1, keepdims=True))
        return sel, e / e.sum(axis=1, keepdims=True)

    om.route = fixed
    try:
        return ost.denoise_logits(pb.shape, pb.W, pb.ocache, tok, sc, pb.lm_scale)
    finally:
        om.route = orig


@pytest.mark.parametrize("which", ["mini", "mini8", "mini4"])
def test_skewed_routing_matches_oracle(which, request):
    """Every token of every layer routed to the same k experts (in one order):
    those experts' segments span several row tiles, the others receive no
    token, and the grouped GEMMs' tile list is far below its worst case.
    Logits and entropies against the oracle run on the same routes (weights
    from each token's own router logits on both sides)."""
    pb = request.getfixturevalue(which)
    torch, dg, rt = pb.env
    shape = pb.shape
    T, k = pb.B * pb.C, shape.top_k
    dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 0, pb.st)
    torch.cuda.synchronize()
    tok = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
    sel = np.tile(np.arange(shape.n_experts - 1, shape.n_experts - 1 - k, -1), (T, 1))  # ids E-1 .. E-k
    force = np.stack([sel] * shape.n_layers)
    say(f"skewed routing {which}: {T} tokens x top-{k} onto experts {sel[0].tolist()}")
    orig = om.route

    def fixed(shape_, r):
        s_ = np.take_along_axis(r, sel, axis=1)
        e = np.exp(s_ - s_.max(axis=1, keepdims=True))
        return sel.copy(), e / e.sum(axis=1, keepdims=True)

    om.route = fixed
    try:
        zo = ost.denoise_logits(shape, pb.W, pb.ocache, tok, None, pb.lm_scale)
    finally:
        om.route = orig
    z = _forward_logits(pb, 0, 48, force_ids=force)
    _err_summary(f"logits {which} (skewed routes)", z, zo)
    allclose_report(f"logits {which} (skewed routes)", z, zo, pb.atol, RTOL)
    tau = smp.temperature(0, 48)
    _, Hg, _ = smp.row_statistics(z.reshape(-1, shape.vocab), tau)
    _, Ho, _ = smp.row_statistics(zo.reshape(-1, shape.vocab), tau)
    allclose_report(f"entropy {which} (skewed routes)", Hg, Ho,
                    entropy_tolerance(zo.reshape(-1, shape.vocab), tau, pb.atol), 0.0)
    pb.check_guards()


@pytest.mark.parametrize("shape,C", [(MINI_BF16, 33), (TINY, 17)])
def test_empty_prefix_ragged_canvas(env, shape, C):
    """Degenerate context: no prefix (cache length 0, the canvas attends only
    to itself) and a canvas size that is a multiple of no tile.  Logits and
    entropies on the oracle's routes, then one full step's decisions."""
    torch, dg, rt = env
    pb = Problem(env, shape, 6.0, 0, C, B=1, cap_extra=-C % 8)  # bf16 caches hold a multiple of 8 rows
    assert pb.cache.struct.length == 0 and pb.ocache.length == 0
    say(f"empty prefix, canvas {C}, {shape.dtype}")
    dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 0, pb.st)
    torch.cuda.synchronize()
    tok = pb.canvas.tokens.cpu().numpy().reshape(pb.B, pb.C)
    tr = {}
    zo = ost.denoise_logits(pb.shape, pb.W, pb.ocache, tok, None, pb.lm_scale, trace=tr)
    z = _forward_logits(pb, 0, 48, force_ids=_forced_ids(tr))
    _err_summary(f"logits empty prefix C={C}", z, zo)
    allclose_report(f"logits empty prefix C={C}", z, zo, pb.atol, RTOL)
    tau = smp.temperature(0, 48)
    _, Hg, _ = smp.row_statistics(z.reshape(-1, shape.vocab), tau)
    _, Ho, _ = smp.row_statistics(zo.reshape(-1, shape.vocab), tau)
    allclose_report(f"entropy empty prefix C={C}", Hg, Ho,
                    entropy_tolerance(zo.reshape(-1, shape.vocab), tau, pb.atol), 0.0)
    dg.dg_denoise_step(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct, rt.step_params(0, 48),
                       pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    check_sampler_invariants(pb, 0, 48, None)
    assert pb.cache.struct.length == 0
    pb.check_guards()


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
    pb.check_guards()


# Router-logit margin under which an autoregressive row's route may differ
# from the oracle's with no forcing available: twice the largest bf16
# router-logit error measured with forced routes (~5e-3), and the fp32 bar.
AR_FLIP = {"f32": 1e-5, "bf16": 1e-2}


@pytest.mark.parametrize("which", ["tiny", "mini", "mini8", "mini4", "mini_long"])
def test_ar_decode_matches_oracle(env, which):
    """Greedy single-token decode on the same weights: every step's logits,
    next token and appended K/V rows against the oracle's, teacher-forced with
    the oracle's greedy tokens so both sides see the same inputs.  Steps
    alternate the logits-capturing entry with the product entry (next token
    only).  The cache is sized to the last step, so one more step is refused
    without writing anything.  mini_long decodes after a 4096-row seeded
    N(0,1) cache (no encoder), where the attention splits the keys 32 ways."""
    torch, dg, rt = env
    shape, lm_scale, prefix, B = {
        "tiny": (WORKLOADS["tiny"].model, WORKLOADS["tiny"].lm_scale, 24, 1),
        "mini": (MINI_BF16, 6.0, 40, 2),
        "mini8": (MINI_FP8, 6.0, 40, 2),
        "mini4": (MINI_MX4, 6.0, 40, 2),
        "mini_long": (MINI_BF16, 6.0, 4096, 1),
    }[which]
    n_dec = 8
    pb = Problem(env, shape, lm_scale, prefix, 1, B=B, cap_extra=n_dec - 1)
    assert pb.cap == prefix + n_dec and pb.cap % 8 == 0
    ws = pb.guard_workspace(rt.Workspace(pb.cfg, B, 1))
    if which == "mini_long":
        pb.cache.fill_random(prefix, seed=0, std=1.0)
        pb.cache.struct.length = prefix
        for name, tid in (("k", synth.TID["kv_k"]), ("v", synth.TID["kv_v"])):
            vals = synth.bf16_bits_to_f32(synth.normal(0, tid, (shape.n_layers, B, shape.n_kv_heads, prefix,
                                                                shape.d_head), 1.0))
            for l in range(shape.n_layers):
                getattr(pb.ocache, name)[l][:, :, :prefix] = vals[l].astype(np.float64)
        pb.ocache.length = prefix
        torch.cuda.synchronize()
    else:
        pb.encode_prefix()
    V = shape.vocab
    d_tok = torch.empty(B, dtype=torch.int32, device="cuda")
    d_next = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    d_logits = torch.empty(B * V, dtype=torch.float32, device="cuda")
    cur = np.array([synth.tokens(b, synth.TID["prompt"], 1, V, start=prefix)[0] for b in range(B)])
    compared = []
    for i in range(n_dec):
        tr = {}
        nxt_o, zo = ost.ar_step(shape, pb.W, pb.ocache, cur, pb.lm_scale, trace=tr)
        d_tok.copy_(torch.from_numpy(cur.astype(np.int32)))
        L0 = pb.cache.length
        say(f"AR {which} step {i} at position {L0} (B={B})")
        if i % 2 == 0:
            dg.dg_test_ar_step(pb.cfg, pb.model.weights, pb.cache.struct, d_tok.data_ptr(), B, d_next.data_ptr(),
                               d_logits.data_ptr(), ws.ptr, ws.size, pb.st)
        else:
            dg.dg_ar_step(pb.cfg, pb.model.weights, pb.cache.struct, d_tok.data_ptr(), B, d_next.data_ptr(),
                          ws.ptr, ws.size, pb.st)
        torch.cuda.synchronize()
        assert pb.cache.length == L0 + 1 == pb.ocache.length
        ok = np.all(_route_margins(shape, tr) >= AR_FLIP[shape.dtype], axis=0)  # [B]: no near-tie route
        compared.append(ok)
        if i % 2 == 0 and ok.any():
            z = d_logits.cpu().numpy().reshape(B, V)
            _err_summary(f"AR logits {which} step {i}", z[ok], zo[ok])
            allclose_report(f"AR logits {which} step {i}", z[ok], zo[ok], pb.atol, RTOL)
        nxt = d_next.cpu().numpy()
        top = -np.sort(-zo, axis=1)
        bar = 2.0 * (pb.atol + RTOL * np.abs(top[:, 0]))  # two logits each off by the logit bar
        clear = ok & (top[:, 0] - top[:, 1] > bar)
        assert np.array_equal(nxt[clear], nxt_o[clear]), (nxt, nxt_o)
        # elsewhere the GPU's pick must be one of the oracle's near-maximal ids
        assert np.all((nxt >= 0) & (nxt < V))
        assert np.all(zo[np.arange(B), nxt][ok] >= top[ok, 0] - bar[ok])
        # the appended K/V rows, for sequences with no near-tie route
        for name, oc in (("k", pb.ocache.k), ("v", pb.ocache.v)):
            got = pb.cache.view(name).float().cpu().numpy()
            for b in np.nonzero(ok)[0]:
                for l in range(shape.n_layers):
                    allclose_report(f"AR cache {name} L{l} b{b} row {L0}", got[l][b][:, L0], oc[l][b][:, L0],
                                    pb.atol, RTOL)
        cur = nxt_o
    compared = np.stack(compared)
    say(f"AR {which}: {int(compared.sum())} of {compared.size} rows compared")
    assert compared.mean() >= 0.5
    pb.compare_cache(prefix)  # the prompt rows are untouched
    # a full cache: refused before anything is written
    k0, v0 = pb.cache.k.clone(), pb.cache.v.clone()
    with pytest.raises(dg.DGError) as e:
        dg.dg_ar_step(pb.cfg, pb.model.weights, pb.cache.struct, d_tok.data_ptr(), B, d_next.data_ptr(),
                      ws.ptr, ws.size, pb.st)
    assert e.value.status == dg.DG_ERR_KV_CAPACITY
    with pytest.raises(dg.DGError) as e:
        dg.dg_test_ar_step(pb.cfg, pb.model.weights, pb.cache.struct, d_tok.data_ptr(), B, d_next.data_ptr(),
                           None, ws.ptr, ws.size, pb.st)
    assert e.value.status == dg.DG_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert pb.cache.length == pb.cap
    assert torch.equal(k0, pb.cache.k) and torch.equal(v0, pb.cache.v)
    pb.check_guards()


def _f32_twin_on_routes(pb, tok, expert_ids):
    """The oracle's definition evaluated with fp32 products and sums on the
    oracle's own routes (the fp32 twin of the full-size parity criterion)."""
    ids = list(expert_ids)
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
            zt = ost.denoise_logits(pb.shape, pb.W, pb.ocache, tok, None, pb.lm_scale, trace=trt)
    finally:
        om.route = orig
    return zt, trt


def test_long_prefill_matches_oracle(env):
    """Prompt encoding at length: a 4096-token prompt through a 3-layer bf16
    model in one causal pass (the attention splits the keys and merges the
    splits; every later layer's K/V rows depend on the earlier layers' causal
    attention over up to 4096 keys).  With the oracle's routes forced, every
    K/V row of every layer is compared with the oracle's causal encode (the
    bar, or the fp32-twin criterion); the product encode (its own routing) is
    compared below the first oracle route near-tie of the layers before."""
    torch, dg, rt = env
    shape = replace(MINI_BF16, n_layers=3)
    n = 4096
    pb = Problem(env, shape, 6.0, n, 8, B=1, cap_extra=-8)
    assert pb.cap == n
    say(f"long prefill: oracle encode of {n} tokens, {shape.n_layers} layers")
    tr = {}
    ost.encode_append(shape, pb.W, pb.ocache, pb.prompt, trace=tr)
    ids = np.stack(tr["expert_ids"])  # [layers][n][k]
    margins = _route_margins(shape, tr)
    d_tok = torch.from_numpy(pb.prompt.astype(np.int32).reshape(-1)).cuda()
    d_force = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)).cuda()
    say("long prefill: GPU encode on the oracle's routes")
    dg.dg_test_encode_append(pb.cfg, pb.model.weights, pb.cache.struct, d_tok.data_ptr(), 1, n, d_force.data_ptr(),
                             None, pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    assert pb.cache.length == n
    twin = {}

    def twin_cache():
        if not twin:
            say("long prefill: fp32 twin encode on the oracle's routes")
            tc = om.KVCache(shape, 1, n)
            left = list(ids)
            orig = om.route

            def fixed(shape_, r):
                sel = left.pop(0)
                s_ = np.take_along_axis(r, sel, axis=1)
                e = np.exp(s_ - s_.max(axis=1, keepdims=True))
                return sel, e / e.sum(axis=1, keepdims=True)

            om.route = fixed
            try:
                with om.accumulation("f32"):
                    ost.encode_append(shape, pb.W, tc, pb.prompt)
            finally:
                om.route = orig
            twin["c"] = tc
        return twin["c"]

    gk, gv = pb.cache.view("k").float().cpu().numpy(), pb.cache.view("v").float().cpu().numpy()
    for l in range(shape.n_layers):
        bar_then_twin(f"long prefill forced k L{l}", gk[l], pb.ocache.k[l], lambda: twin_cache().k[l], pb.atol, RTOL)
        bar_then_twin(f"long prefill forced v L{l}", gv[l], pb.ocache.v[l], lambda: twin_cache().v[l], pb.atol, RTOL)
    # the product encode, own routing: rows below the first near-tie of any earlier layer
    pc = rt.DeviceCache(shape, 1, n)
    dg.dg_encode_append(pb.cfg, pb.model.weights, pc.struct, d_tok.data_ptr(), 1, n, pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    pk, pv = pc.view("k").float().cpu().numpy(), pc.view("v").float().cpu().numpy()
    rows = n
    for l in range(shape.n_layers):
        if rows == 0:
            break
        bar_then_twin(f"long prefill product k L{l} rows<{rows}", pk[l][:, :, :rows], pb.ocache.k[l][:, :, :rows],
                      lambda: twin_cache().k[l][:, :, :rows], pb.atol, RTOL)
        bar_then_twin(f"long prefill product v L{l} rows<{rows}", pv[l][:, :, :rows], pb.ocache.v[l][:, :, :rows],
                      lambda: twin_cache().v[l][:, :, :rows], pb.atol, RTOL)
        ties = np.nonzero(margins[l] < ROUTE_EPS["bf16"])[0]
        rows = min(rows, int(ties[0]) if ties.size else n)
    say(f"long prefill: product encode compared below row {rows} after the last layer")
    pb.check_guards()


@pytest.mark.parametrize("B", [24, 48])
def test_many_canvases_match_oracle(env, B):
    """24 or 48 canvases of 48 tokens: 1152 or 2304 tokens in one step, so the
    routing sort runs in 1024-token chunks and the grouped expert GEMMs take
    64- and 128-row tiles (288 and 576 rows per expert on average).
    Logits, router logits and entropies on the oracle's routes (4.7M logits:
    the elementwise bar, or the fp32-twin criterion where the bf16 tail
    reaches it), then one full step's sampler invariants on every canvas."""
    torch, dg, rt = env
    C, prefix = 48, 16
    pb = Problem(env, MINI_BF16, 6.0, prefix, C, B=B)
    pb.encode_prefix()
    pb.compare_cache(prefix)
    say(f"{B} canvases of {C}")
    dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 0, pb.st)
    torch.cuda.synchronize()
    tok = pb.canvas.tokens.cpu().numpy().reshape(B, C)
    tr = {}
    zo = ost.denoise_logits(pb.shape, pb.W, pb.ocache, tok, None, pb.lm_scale, trace=tr)
    zt, trt = _f32_twin_on_routes(pb, tok, tr["expert_ids"])
    z, rg = _forward_logits(pb, 0, 48, force_ids=_forced_ids(tr), want_router=True)
    bar_or_twin(f"router logits {B}x{C} (oracle routes)", rg, np.stack(tr["router_logits"]),
                np.stack(trt["router_logits"]), ROUTE_EPS["bf16"], 0.0)
    bar_or_twin(f"logits {B}x{C} (oracle routes)", z, zo, zt, pb.atol, RTOL)
    tau = smp.temperature(0, 48)
    V = pb.shape.vocab
    _, Hg, _ = smp.row_statistics(z.reshape(-1, V), tau)
    _, Ho, _ = smp.row_statistics(zo.reshape(-1, V), tau)
    _, Ht, _ = smp.row_statistics(zt.reshape(-1, V), tau)
    bar_or_twin(f"entropy {B}x{C}", Hg, Ho, Ht, entropy_tolerance(zo.reshape(-1, V), tau, pb.atol), 0.0)
    dg.dg_denoise_step(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct, rt.step_params(0, 48),
                       pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    check_sampler_invariants(pb, 0, 48, None)
    assert pb.cache.struct.length == prefix
    pb.check_guards()


@pytest.mark.parametrize("which", ["tiny", "mini", "mini8", "mini4"])
def test_commit_and_step_matches_oracle(env, which):
    """dg_commit_and_step (commit of one block and the next block's first
    step in one pass) against the oracle's commit and step: the appended K/V
    rows (causal encode of the last step's argmax), the next canvas's noise,
    the step's entropies (rows without a near-tie route) and its sampler
    invariants."""
    torch, dg, rt = env
    shape, lm_scale, prefix, C, B = {
        "tiny": (WORKLOADS["tiny"].model, WORKLOADS["tiny"].lm_scale, 24, 32, 1),
        "mini": (MINI_BF16, 6.0, 40, 48, 2),
        "mini8": (MINI_FP8, 6.0, 40, 48, 2),
        "mini4": (MINI_MX4, 6.0, 40, 48, 2),
    }[which]
    pb = Problem(env, shape, lm_scale, prefix, C, B=B, cap_extra=C + (-(prefix + 2 * C)) % 8)
    pb.encode_prefix()
    say(f"commit+step {which}")
    dg.dg_init_canvas(pb.cfg, pb.canvas.struct, 0, pb.st)
    for t in range(2):
        dg.dg_denoise_step(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct, rt.step_params(t, 2),
                           pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    am = pb.canvas.argmax.cpu().numpy().reshape(B, C)
    dg.dg_commit_and_step(pb.cfg, pb.model.weights, pb.cache.struct, pb.canvas.struct, rt.step_params(1, 2, 0),
                          rt.step_params(0, 2, 1), pb.ws.ptr, pb.ws.size, pb.st)
    torch.cuda.synchronize()
    assert pb.cache.struct.length == prefix + C
    assert np.array_equal(pb.canvas.committed.cpu().numpy().reshape(B, C), am)
    ost.encode_append(shape, pb.W, pb.ocache, am)
    pb.compare_cache(prefix + C)
    tok = np.stack([smp.initial_canvas(pb.seeds[b], 1, C, shape.vocab) for b in range(B)])
    tr = {}
    zo = ost.denoise_logits(shape, pb.W, pb.ocache, tok, None, pb.lm_scale, trace=tr)
    ok = np.all(_route_margins(shape, tr) >= AR_FLIP[shape.dtype], axis=0).reshape(B, C)  # [T] rows
    say(f"commit+step {which}: {int(ok.sum())} of {ok.size} rows without a near-tie route")
    assert ok.mean() >= 0.5
    tau = smp.temperature(0, 2)
    _, Ho, _ = smp.row_statistics(zo.reshape(-1, shape.vocab), tau)
    Hg = pb.canvas.entropy.cpu().numpy().astype(np.float64)
    tol = entropy_tolerance(zo.reshape(-1, shape.vocab), tau, pb.atol)
    allclose_report(f"commit+step entropy {which}", Hg[ok.reshape(-1)], Ho[ok.reshape(-1)], tol[ok.reshape(-1)], 0.0)
    check_sampler_invariants(pb, 0, 2, None, block=1)
    pb.check_guards()
