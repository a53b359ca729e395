"""GPU checks of the MXFP4 expert weights (OCP Microscaling Formats v1.0:
E2M1 elements, an E8M0 scale per 32 inputs):

* the input recipe's device quantiser gives the host quantiser's codes and
  scales bit for bit;
* dg_pack_weight_mxfp4 writes the layout its header states;
* the batch-4 one-layer workload with MXFP4 experts (fp8 LM head): first-step
  logits of sampled positions against the oracle on the oracle's routes,
  within |g - o| <= 3e-2 + 1e-2|o| (or the fp32-twin criterion), entropies
  within 1e-3 nats, route flips only at near-ties.
The small MXFP4 model is run through the whole path in test_gpu_model
("mini4")."""
import numpy as np
import pytest

import synth
from oracle import model as om
from oracle import sampler as smp
from synth.configs import WORKLOADS

from .gpu_util import allclose_report, bar_or_twin, say
from .test_gpu_fp8 import ROWS, _gpu_logits, _oracle_cache, _oracle_hidden
from .test_gpu_model import RTOL, ROUTE_EPS, _err_summary, _route_margins, flip_margin_bound

pytestmark = pytest.mark.gpu

ATOL_Q = 3e-2  # logits bar of the quantised-weight workloads


@pytest.fixture(scope="module")
def env():
    import torch
    import discrete_text_diffusion_amd as dg
    from discrete_text_diffusion_amd import runtime as rt
    assert torch.cuda.is_available()
    return torch, dg, rt


@pytest.mark.parametrize("rows,cols,tensor", [(48, 256, 901), (704, 2816, synth.layer_tid(0, "ex_g"))])
def test_device_quantiser_matches_host(env, rows, cols, tensor):
    torch, dg, rt = env
    codes = torch.empty(rows * cols, dtype=torch.uint8, device="cuda")
    sc = torch.empty(rows * cols // 32, dtype=torch.uint8, device="cuda")
    synth.dev_mxfp4_rows(codes.data_ptr(), sc.data_ptr(), rows, cols, 0, tensor, 0.02, rt.stream_handle())
    torch.cuda.synchronize()
    hc, hs = synth.mxfp4_rows(0, tensor, rows, cols, 0.02)
    assert np.array_equal(codes.cpu().numpy().reshape(rows, cols), hc)
    assert np.array_equal(sc.cpu().numpy().reshape(rows, cols // 32), hs)
    say(f"mxfp4 device quantiser {rows}x{cols}: codes and scales equal to the host's")


def _layout(codes, scales):
    """The MXFP4 weight layout of dg_pack_weight_mxfp4, written out."""
    rows, cols = codes.shape
    out = np.zeros(rows * cols // 32 * 17, dtype=np.uint8)
    for nt in range(rows // 16):
        for kb in range(cols // 64):
            base = (nt * (cols // 64) + kb) * 544
            for l in range(64):
                r = nt * 16 + l % 16
                for h in range(2):
                    for q in range(4):
                        c = kb * 64 + 32 * h + 8 * (l // 16) + 2 * q
                        out[base + 8 * l + 4 * h + q] = (codes[r, c] & 15) | ((codes[r, c + 1] & 15) << 4)
            for r in range(16):
                for h in range(2):
                    out[base + 512 + 2 * r + h] = scales[nt * 16 + r, kb * 2 + h]
    return out


def test_pack_layout(env):
    torch, dg, rt = env
    rng = np.random.default_rng(3)
    rows, cols = 32, 128
    codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    scales = rng.integers(100, 140, (rows, cols // 32)).astype(np.uint8)
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    out = torch.zeros(rows * cols // 32 * 17, dtype=torch.uint8, device="cuda")
    dg.dg_pack_weight_mxfp4(out.data_ptr(), dc.data_ptr(), ds.data_ptr(), rows, cols, rt.stream_handle())
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), _layout(codes, scales))
    for bad in ((rows - 8, cols), (rows, cols - 32)):
        with pytest.raises(RuntimeError):
            dg.dg_pack_weight_mxfp4(out.data_ptr(), dc.data_ptr(), ds.data_ptr(), *bad, rt.stream_handle())


@pytest.fixture(scope="module")
def mx4b4(env):
    torch, dg, rt = env
    wl = WORKLOADS["mx4batch4"]
    shape, B, C, L = wl.model, wl.batch, wl.canvas, wl.prefix
    say(f"mx4batch4: building the MXFP4-expert model, B={B}, cache {L}")
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


def test_mx4_first_step_logits_match_oracle(env, mx4b4):
    f = mx4b4
    shape, wl = f["shape"], f["wl"]
    kv_before = f["cache"].valid_rows()
    say("mx4batch4: oracle layer forward (1024 canvas tokens)")
    tr = {}
    x = _oracle_hidden(f, tr)
    margins = _route_margins(shape, tr)
    zo = om.final_logits(shape, f["W"], x[:, ROWS], wl.lm_scale)
    say("mx4batch4: fp32 twin on the oracle's routes")
    trt = {}
    with om.accumulation("f32"):
        xt = _oracle_hidden(f, trt, tr["expert_ids"])
        zt = om.final_logits(shape, f["W"], xt[:, ROWS], wl.lm_scale)
    z, rg = _gpu_logits(env, f, force=np.stack(tr["expert_ids"]), rows=ROWS)
    torch = env[0]
    assert all(torch.equal(a, b) for a, b in zip(kv_before, f["cache"].valid_rows()))
    _err_summary("mx4batch4 router logits (oracle routes)", rg, np.stack(tr["router_logits"]))
    bar_or_twin("mx4batch4 router logits (oracle routes)", rg, np.stack(tr["router_logits"]),
                np.stack(trt["router_logits"]), ROUTE_EPS["bf16"], 0.0)
    bar_or_twin("mx4batch4 logits (oracle routes)", z, zo, zt, ATOL_Q, RTOL)
    tau = smp.temperature(0, wl.n_steps)
    _, Hg, _ = smp.row_statistics(z.reshape(-1, shape.vocab), tau)
    _, Ho, _ = smp.row_statistics(zo.reshape(-1, shape.vocab), tau)
    allclose_report("mx4batch4 entropy (oracle routes)", Hg, Ho, 1e-3, 0.0)
    _, ru = _gpu_logits(env, f, rows=ROWS)
    gtop = np.sort(np.argsort(-ru[0], axis=1, kind="stable")[:, :shape.top_k], axis=1)
    otop = np.sort(tr["expert_ids"][0], axis=1)
    flips = np.nonzero(np.any(gtop != otop, axis=1))[0]
    bound = flip_margin_bound(rg, np.stack(tr["router_logits"]))
    say(f"mx4batch4 unforced: route flips {flips.size} at oracle margins {margins[0][flips]} (bound {bound:.2e})")
    assert np.all(margins[0][flips] < bound)
