"""The step as a function of its documented state, and its non-finite flag:

* resume: the canvas state after step t (tokens, the carried
  self-conditioning input p_side / p_scale, the previous argmax) and the KV
  cache, copied to the host, loaded into fresh device buffers with a fresh
  workspace, and continued, give bitwise the outputs of the uninterrupted
  run (the library keeps no state between calls);
* non-finite logits: a row with a NaN or +inf logit gets entropy +inf, its
  canvas's DG_FLAG_NONFINITE bit is set, every token stays a valid id, and the
  other canvas of the batch is untouched (its decisions equal the oracle's)."""
import numpy as np
import pytest

from oracle import sampler as smp
from synth.configs import MINI_BF16

from .gpu_util import allclose_report, compare_decisions, say

pytestmark = pytest.mark.gpu

STATE = ("tokens", "p_side", "p_scale", "prev_argmax")
OUTS = ("tokens", "entropy", "sample", "argmax", "prev_argmax", "accepted", "n_accepted", "mean_entropy", "stop",
        "flags", "p_side", "p_scale")


@pytest.fixture(scope="module")
def env():
    import torch
    import discrete_text_diffusion_amd as dg
    from discrete_text_diffusion_amd import runtime as rt
    assert torch.cuda.is_available()
    return torch, dg, rt


def test_resume_from_saved_state_is_bitwise(env):
    torch, dg, rt = env
    shape, B, C, L, N = MINI_BF16, 2, 48, 40, 12
    model = rt.DeviceModel(shape, 6.0)
    cfg, st = model.cfg, rt.stream_handle()

    def fresh():
        cache = rt.DeviceCache(shape, B, L + C)
        cv = rt.DeviceCanvas(shape, B, C, [3, 4])
        return cache, cv, rt.Workspace(cfg, B, C)

    cache, cv, ws = fresh()
    cache.fill_random(L, seed=0, std=1.0)
    dg.dg_init_canvas(cfg, cv.struct, 0, st)
    say("resume: uninterrupted 4 steps")
    saved = None
    for t in range(4):
        dg.dg_denoise_step(cfg, model.weights, cache.struct, cv.struct, rt.step_params(t, N), ws.ptr, ws.size, st)
        torch.cuda.synchronize()
        if t == 1:
            saved = {n: getattr(cv, n).cpu().clone() for n in STATE}
            saved_kv = [x.cpu().clone() for x in (cache.k, cache.v)]
    want = {n: getattr(cv, n).cpu().clone() for n in OUTS}
    want_kv = [x.cpu().clone() for x in (cache.k, cache.v)]  # incl. the canvas rows step 3 wrote
    del ws
    say("resume: reload after step 1 into fresh buffers, continue with steps 2, 3")
    cache2, cv2, ws2 = fresh()
    cache2.k.copy_(saved_kv[0])
    cache2.v.copy_(saved_kv[1])
    cache2.struct.length = L
    for n in STATE:
        getattr(cv2, n).copy_(saved[n])
    for t in (2, 3):
        dg.dg_denoise_step(cfg, model.weights, cache2.struct, cv2.struct, rt.step_params(t, N), ws2.ptr, ws2.size, st)
    torch.cuda.synchronize()
    for n in OUTS:
        if n == "flags":
            continue  # sticky per canvas, not part of the carried state
        assert torch.equal(getattr(cv2, n).cpu(), want[n]), f"resumed run differs in {n}"
    assert torch.equal(cache2.k.cpu(), want_kv[0]) and torch.equal(cache2.v.cpu(), want_kv[1])
    say("resume: every output bitwise equal to the uninterrupted run")


def test_nonfinite_logits_are_flagged(env):
    torch, dg, rt = env
    shape, B, C, t, N = MINI_BF16, 2, 64, 3, 48
    V = shape.vocab
    rng = np.random.default_rng(11)
    z = (rng.standard_normal((B * C, V)) * 3.0).astype(np.float32)
    bad_nan, bad_inf = 5, 40              # rows of canvas 0
    z[bad_nan, 1234] = np.nan
    z[bad_inf, 77] = np.inf
    seeds = [21, 22]
    cv = rt.DeviceCanvas(shape, B, C, seeds)
    prev = rng.integers(0, V, size=B * C).astype(np.int32)
    cv.prev_argmax.copy_(torch.from_numpy(prev))
    cfg = rt.model_config(shape)
    ws = rt.Workspace(cfg, B, C)
    d_z = torch.from_numpy(z).cuda()
    dg.dg_test_sample_from_logits(cfg, d_z.data_ptr(), cv.struct, rt.step_params(t, N, 0, True), ws.ptr, ws.size,
                                  rt.stream_handle())
    torch.cuda.synchronize()
    H = cv.entropy.cpu().numpy().reshape(B, C)
    flags = cv.flags.cpu().numpy()
    for name in ("tokens", "sample", "argmax"):
        ids = getattr(cv, name).cpu().numpy()
        assert ids.min() >= 0 and ids.max() < V, f"{name} holds an invalid id"
    assert np.isposinf(H[0, bad_nan]) and np.isposinf(H[0, bad_inf])
    ok = np.ones(C, dtype=bool)
    ok[[bad_nan, bad_inf]] = False
    assert np.all(np.isfinite(H[0, ok])) and np.all(np.isfinite(H[1]))
    assert flags[0] & 1 and not flags[1] & 1
    acc = cv.accepted.cpu().numpy().reshape(B, C).astype(bool)
    assert not acc[0, bad_nan] and not acc[0, bad_inf]
    # canvas 0's finite rows: entropies as the definition gives them
    tau = smp.temperature(t, N)
    Ho = smp.row_statistics(z[:C][ok].astype(np.float64), tau)[1]
    allclose_report("finite rows of the flagged canvas: entropy", H[0, ok], Ho, 1e-3, 0.0)
    # canvas 1: the oracle's decisions
    o = smp.sample_from_logits(z[C:].astype(np.float64), t, N, seeds[1], 0, prev[C:], True)
    allclose_report("unflagged canvas: entropy", H[1], o["H"], 1e-3, 0.0)
    compare_decisions("unflagged canvas: sample", cv.sample.cpu().numpy()[C:], o["sample"], o["margin_sample"], 1e-5)
    compare_decisions("unflagged canvas: accepted", acc[1], o["accepted"], o["margin_accept"], 1e-5, max_ties=2)
    say(f"non-finite rows: H = +inf, flags {flags.tolist()}, every id valid")
