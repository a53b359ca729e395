"""dg_denoise_step_noalloc (static scratch, no workspace argument) against
dg_denoise_step with a caller workspace on the same inputs: two calls in a
row, the second with a smaller canvas, each a two-step sequence (t = 0, then
t = 1 reading the carried self-conditioning input).  The two entry points
run the same launches, so every output must be bitwise equal; a step too
large for the scratch is refused before anything is written."""
import numpy as np
import pytest

from synth.configs import FULL_LAYER, MINI_BF16

pytestmark = pytest.mark.gpu

CASES = {
    # name: shape, LM-head scale, cache rows, (batch, canvas) of the two calls
    "mini": (MINI_BF16, 6.0, 40, [(2, 48), (1, 16)]),
    "full_width": (FULL_LAYER, 1.0, 2048, [(1, 256), (1, 64)]),
}


@pytest.fixture(scope="module")
def env():
    import torch
    import discrete_text_diffusion_amd as dg
    from discrete_text_diffusion_amd import runtime as rt
    assert torch.cuda.is_available()
    return torch, dg, rt


def _outputs(cv):
    return {n: getattr(cv, n).clone() for n in ("tokens", "entropy", "sample", "argmax", "prev_argmax", "accepted",
                                                "n_accepted", "mean_entropy", "stop", "flags", "p_side", "p_scale")}


@pytest.mark.parametrize("which", list(CASES))
def test_noalloc_step_matches_workspace_step(env, which):
    torch, dg, rt = env
    shape, lm_scale, L, sizes = CASES[which]
    print(f"noalloc {which}: building model", flush=True)
    model = rt.DeviceModel(shape, lm_scale)
    cfg, st = model.cfg, rt.stream_handle()
    for B, C in sizes:
        print(f"noalloc {which}: batch {B} x canvas {C}", flush=True)
        cache = rt.DeviceCache(shape, B, L + C)
        cache.fill_random(L, seed=0, std=1.0)
        seeds = [11 + b for b in range(B)]
        ref = rt.DeviceCanvas(shape, B, C, seeds)
        got = rt.DeviceCanvas(shape, B, C, seeds)
        ws = rt.Workspace(cfg, B, C)
        for cv in (ref, got):
            dg.dg_init_canvas(cfg, cv.struct, 0, st)
        for t in (0, 1):
            p = rt.step_params(t, 12, 0, True)
            dg.dg_denoise_step(cfg, model.weights, cache.struct, ref.struct, p, ws.ptr, ws.size, st)
            dg.dg_denoise_step_noalloc(cfg, model.weights, cache.struct, got.struct, p, st)
            torch.cuda.synchronize()
            a, b = _outputs(ref), _outputs(got)
            for name in a:
                assert torch.equal(a[name], b[name]), f"{which} B={B} C={C} t={t}: {name} differs"
            print(f"noalloc {which} B={B} C={C} t={t}: all outputs equal (accepted "
                  f"{ref.n_accepted.cpu().numpy().tolist()})", flush=True)
        assert cache.struct.length == L
        del ws, cache
    if which == "full_width":
        # two 256-token canvases need more than the scratch holds: refused, nothing written
        cv = rt.DeviceCanvas(shape, 2, 256, [1, 2])
        big = rt.DeviceCache(shape, 2, L + 256)
        big.struct.length = L
        dg.dg_init_canvas(cfg, cv.struct, 0, st)
        torch.cuda.synchronize()
        before = _outputs(cv)
        with pytest.raises(dg.DGError) as e:
            dg.dg_denoise_step_noalloc(cfg, model.weights, big.struct, cv.struct, rt.step_params(0, 12), st)
        assert e.value.status == dg.DG_ERR_SCRATCH_LIMIT
        torch.cuda.synchronize()
        after = _outputs(cv)
        assert all(torch.equal(before[n], after[n]) for n in before)
