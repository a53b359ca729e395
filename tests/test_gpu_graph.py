"""One denoising step captured in a HIP graph (torch.cuda.CUDAGraph on the
capture stream; the library records no memset or allocation) and replayed:
every replay, each from the same saved canvas state and with eager work of
the program in between, must reproduce the eager step's outputs bitwise."""
import numpy as np
import pytest

from synth.configs import MINI_BF16

pytestmark = pytest.mark.gpu

STATE = ("tokens", "p_side", "p_scale", "prev_argmax")
OUTS = ("tokens", "entropy", "sample", "argmax", "prev_argmax", "accepted", "n_accepted", "mean_entropy", "stop",
        "flags", "p_side", "p_scale")


def test_graph_replay_matches_eager_step():
    import torch
    import discrete_text_diffusion_amd as dg
    from discrete_text_diffusion_amd import runtime as rt
    assert torch.cuda.is_available()
    shape, B, C, L = MINI_BF16, 2, 48, 40
    model = rt.DeviceModel(shape, 6.0)
    cfg = model.cfg
    cache = rt.DeviceCache(shape, B, L + C)
    cache.fill_random(L, seed=0, std=1.0)
    cv = rt.DeviceCanvas(shape, B, C, [3, 4])
    other = rt.DeviceCanvas(shape, B, C, [5, 6])
    ws = rt.Workspace(cfg, B, C)
    ws2 = rt.Workspace(cfg, B, C)
    st = rt.stream_handle()
    dg.dg_init_canvas(cfg, cv.struct, 0, st)
    dg.dg_init_canvas(cfg, other.struct, 0, st)
    # step 0 eagerly, so that step 1 reads a carried self-conditioning input
    dg.dg_denoise_step(cfg, model.weights, cache.struct, cv.struct, rt.step_params(0, 12), ws.ptr, ws.size, st)
    torch.cuda.synchronize()
    saved = {n: getattr(cv, n).clone() for n in STATE}
    p1 = rt.step_params(1, 12)
    dg.dg_denoise_step(cfg, model.weights, cache.struct, cv.struct, p1, ws.ptr, ws.size, st)
    torch.cuda.synchronize()
    eager = {n: getattr(cv, n).clone() for n in OUTS}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dg.dg_denoise_step(cfg, model.weights, cache.struct, cv.struct, p1, ws.ptr, ws.size, rt.stream_handle())
    for rep in range(4):
        for n in STATE:
            getattr(cv, n).copy_(saved[n])
        g.replay()
        # the program's own eager work between replays (another canvas, its own workspace)
        dg.dg_denoise_step(cfg, model.weights, cache.struct, other.struct, rt.step_params(rep % 12, 12), ws2.ptr,
                           ws2.size, rt.stream_handle())
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(getattr(cv, n), eager[n]), f"replay {rep}: {n} differs from the eager step"
        print(f"graph replay {rep}: equal to the eager step", flush=True)
    assert cache.struct.length == L
    del g
