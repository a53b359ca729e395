"""GPU parity of the sampler, stop test, routing, device Philox, weight
packing and the device input generator against the oracle / definitions.
Decisions are fed the oracle's own inputs and must match bit for bit (up to
reported near-ties)."""
import numpy as np
import pytest

import synth
from oracle import philox, sampler as smp
from oracle import model as om
from synth.configs import FULL_LAYER, MINI_BF16, TINY

from .gpu_util import allclose_report, compare_decisions, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import discrete_text_diffusion_amd as dg
    from discrete_text_diffusion_amd import runtime as rt
    assert torch.cuda.is_available()
    return torch, dg, rt


def test_device_generator_matches_host(env):
    torch, dg, rt = env
    say("device synth vs host")
    st = rt.stream_handle()
    n = 300001
    t = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    synth.dev_normal(t.data_ptr(), n, 3, 123, 0.02, "bf16", st, start=17)
    assert np.array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), synth.normal(3, 123, (n,), 0.02, "bf16", start=17))
    f = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.dev_normal(f.data_ptr(), n, 5, 7, 1.0, "f32", st)
    assert np.array_equal(f.cpu().numpy(), synth.normal(5, 7, (n,), 1.0, "f32"))
    k = torch.empty(n, dtype=torch.int32, device="cuda")
    synth.dev_tokens(k.data_ptr(), n, 9, 10, 262144, st)
    assert np.array_equal(k.cpu().numpy(), synth.tokens(9, 10, n, 262144))
    r, c = 96, 40
    tt = torch.empty(r * c, dtype=torch.float32, device="cuda")
    synth.dev_normal_f32_transposed(tt.data_ptr(), r, c, 0, 1, 0.02, st)
    assert np.array_equal(tt.cpu().numpy().reshape(c, r), synth.normal(0, 1, (r, c), 0.02, "f32").T)
    # fp8 weight recipe: per-row scales and E4M3 codes
    r, c = 4096, 704
    codes = torch.empty(r * c, dtype=torch.uint8, device="cuda")
    sc = torch.empty(r, dtype=torch.float32, device="cuda")
    synth.dev_e4m3_rows(codes.data_ptr(), sc.data_ptr(), r, c, 0, synth.layer_tid(0, "ex_d"), 0.02, st)
    hc, hs = synth.e4m3_rows(0, synth.layer_tid(0, "ex_d"), r, c, 0.02)
    assert np.array_equal(sc.cpu().numpy(), hs)
    assert np.array_equal(codes.cpu().numpy().reshape(r, c), hc)


def test_pack_layout_matches_header_definition(env):
    torch, dg, rt = env
    say("pack layout")
    rng = np.random.default_rng(0)
    rows, cols = 48, 96
    src = rng.integers(0, 0x7F00, size=(rows, cols), dtype=np.uint16)
    want = np.empty(rows * cols, dtype=np.uint16)
    for r in range(rows):
        for c in range(cols):
            off = ((r // 16) * (cols // 32) + c // 32) * 512 + (((c % 32) // 8) * 16 + r % 16) * 8 + c % 8
            want[off] = src[r, c]
    d_src = torch.from_numpy(src.view(np.int16).reshape(-1)).cuda()
    d_dst = torch.empty_like(d_src)
    dg.dg_pack_weight_bf16(d_dst.data_ptr(), d_src.data_ptr(), rows, cols, rt.stream_handle())
    assert np.array_equal(d_dst.cpu().numpy().view(np.uint16), want)
    d_srct = torch.from_numpy(np.ascontiguousarray(src.T).view(np.int16).reshape(-1)).cuda()
    dg.dg_pack_weight_bf16_transposed(d_dst.data_ptr(), d_srct.data_ptr(), rows, cols, rt.stream_handle())
    assert np.array_equal(d_dst.cpu().numpy().view(np.uint16), want)
    # fp8 layout: 16 x 32 tiles of 512 bytes
    src8 = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    want8 = np.empty(rows * cols, dtype=np.uint8)
    for r in range(rows):
        for c in range(cols):
            want8[((r // 16) * (cols // 32) + c // 32) * 512 + (((c % 32) // 8) * 16 + r % 16) * 8 + c % 8] = src8[r, c]
    d8 = torch.from_numpy(src8.reshape(-1)).cuda()
    o8 = torch.empty_like(d8)
    dg.dg_pack_weight_fp8(o8.data_ptr(), d8.data_ptr(), rows, cols, rt.stream_handle())
    assert np.array_equal(o8.cpu().numpy(), want8)


def _canvas(env, shape, B, C, seeds, selfcond=False):
    torch, dg, rt = env
    return rt.DeviceCanvas(shape, B, C, seeds, selfcond=selfcond)


def test_init_canvas_is_philox_stream0(env):
    torch, dg, rt = env
    say("init canvas")
    cv = _canvas(env, FULL_LAYER, 2, 256, [11, (1 << 40) + 5])
    cfg = rt.model_config(FULL_LAYER)
    dg.dg_init_canvas(cfg, cv.struct, 3, rt.stream_handle())
    got = cv.tokens.cpu().numpy().reshape(2, 256)
    for b, s in enumerate([11, (1 << 40) + 5]):
        assert np.array_equal(got[b], smp.initial_canvas(s, 3, 256, FULL_LAYER.vocab))


def _logits(rng, rows, V, scale_lo, scale_hi):
    sc = np.exp(rng.uniform(np.log(scale_lo), np.log(scale_hi), size=(rows, 1)))
    return (rng.standard_normal((rows, V)) * sc).astype(np.float32)


@pytest.mark.parametrize("shape,C,B,t,adaptive", [(TINY, 32, 1, 3, True), (MINI_BF16, 256, 2, 5, True),
                                                  (MINI_BF16, 200, 1, 0, False), (FULL_LAYER, 64, 1, 1, False)])
def test_sampler_from_oracle_logits(env, shape, C, B, t, adaptive):
    torch, dg, rt = env
    say(f"sampler parity V={shape.vocab} C={C} B={B} t={t}")
    rng = np.random.default_rng(C + B + t)
    V = shape.vocab
    n_steps = 48
    seeds = [1000 + b for b in range(B)]
    z = _logits(rng, B * C, V, 0.3, 120.0)
    prev = rng.integers(0, V, size=B * C).astype(np.int32)
    cv = _canvas(env, shape, B, C, seeds, selfcond=True)
    cv.prev_argmax.copy_(torch.from_numpy(prev))
    cfg = rt.model_config(shape)
    ws = rt.Workspace(cfg, B, C)
    d_z = torch.from_numpy(z).cuda()
    p = rt.step_params(t, n_steps, block=2, adaptive=adaptive)
    dg.dg_test_sample_from_logits(cfg, d_z.data_ptr(), cv.struct, p, ws.ptr, ws.size, rt.stream_handle())
    torch.cuda.synchronize()
    H = cv.entropy.cpu().numpy().reshape(B, C)
    samp = cv.sample.cpu().numpy().reshape(B, C)
    amax = cv.argmax.cpu().numpy().reshape(B, C)
    acc = cv.accepted.cpu().numpy().reshape(B, C).astype(bool)
    nxt = cv.tokens.cpu().numpy().reshape(B, C)
    nacc = cv.n_accepted.cpu().numpy()
    stop = cv.stop.cpu().numpy()
    mean = cv.mean_entropy.cpu().numpy()
    prev_after = cv.prev_argmax.cpu().numpy().reshape(B, C)
    for b in range(B):
        o = smp.sample_from_logits(z[b * C:(b + 1) * C].astype(np.float64), t, n_steps, seeds[b], 2,
                                   prev[b * C:(b + 1) * C], adaptive)
        allclose_report("entropy", H[b], o["H"], 1e-3, 0.0)
        assert np.array_equal(amax[b], o["argmax"])
        assert np.array_equal(prev_after[b], o["argmax"])
        compare_decisions("sample", samp[b], o["sample"], o["margin_sample"], 1e-5)
        ties = compare_decisions("accepted", acc[b], o["accepted"], o["margin_accept"], 1e-5, max_ties=2)
        if ties == 0:
            assert nacc[b] == o["n_accepted"]
            assert np.array_equal(nxt[b], np.where(o["accepted"], samp[b], smp.renoise_tokens(seeds[b], t, 2, C, V)))
        assert abs(mean[b] - o["mean_H"]) < 1e-4
        assert stop[b] == o["stop"]
    if B == 2:
        assert nacc.min() >= 1


def test_stop_fires_on_confident_repeated_prediction(env):
    torch, dg, rt = env
    say("stop test")
    shape, B, C, V = MINI_BF16, 1, 64, MINI_BF16.vocab
    rng = np.random.default_rng(7)
    z = rng.standard_normal((C, V)).astype(np.float32)
    top = rng.integers(0, V, size=C)
    z[np.arange(C), top] += 60.0
    cfg = rt.model_config(shape)
    ws = rt.Workspace(cfg, B, C)
    d_z = torch.from_numpy(z).cuda()
    for prev, want in ((top.astype(np.int32), 1), (np.roll(top, 1).astype(np.int32), 0)):
        for t, adaptive, w2 in ((5, True, want), (0, True, 0), (5, False, 0)):
            cv = _canvas(env, shape, B, C, [3])
            cv.prev_argmax.copy_(torch.from_numpy(prev))
            dg.dg_test_sample_from_logits(cfg, d_z.data_ptr(), cv.struct, rt.step_params(t, 48, 0, adaptive),
                                          ws.ptr, ws.size, rt.stream_handle())
            torch.cuda.synchronize()
            o = smp.sample_from_logits(z.astype(np.float64), t, 48, 3, 0, prev, adaptive)
            assert int(cv.stop.item()) == int(o["stop"]) == w2


@pytest.mark.parametrize("shape,T,skew", [(MINI_BF16, 48, False), (FULL_LAYER, 256, False), (TINY, 96, False),
                                          (FULL_LAYER, 1024, False), (MINI_BF16, 1025, False),
                                          (FULL_LAYER, 3000, False), (FULL_LAYER, 16384, False),
                                          (FULL_LAYER, 5000, True)])
def test_routing_from_oracle_logits(env, shape, T, skew):
    """Above 1024 tokens the sort runs over 1024-token chunks (a one-token last
    chunk at 1025, a ragged one at 3000, sixteen at 16384); skew sends every
    token to the same top_k experts, 5000 rows each."""
    torch, dg, rt = env
    say(f"routing parity E={shape.n_experts} k={shape.top_k} T={T} skew={skew}")
    rng = np.random.default_rng(T)
    r = rng.standard_normal((T, shape.n_experts)).astype(np.float32)
    if skew:
        r[:, -shape.top_k:] += 20.0
    r[0, 3] = r[0, 5] = 9.0 + (30.0 if skew else 0.0)  # exact tie: lower id first
    cfg = rt.model_config(shape)
    ws = rt.Workspace(cfg, 1, T)
    k = shape.top_k
    n_sh = shape.d_shared // shape.d_expert
    i32 = dict(dtype=torch.int32, device="cuda")
    ids = torch.empty(T * k, **i32)
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    row_token = torch.empty(T * k + n_sh * T, **i32)
    inv = torch.empty(T * k, **i32)
    offs = torch.empty(shape.n_experts + 1, **i32)
    d_r = torch.from_numpy(r).cuda()
    dg.dg_test_route_from_logits(cfg, d_r.data_ptr(), T, ids.data_ptr(), w.data_ptr(), row_token.data_ptr(),
                                 inv.data_ptr(), offs.data_ptr(), ws.ptr, ws.size, rt.stream_handle())
    torch.cuda.synchronize()
    o_ids, o_w = om.route(shape, r.astype(np.float64))
    assert np.array_equal(ids.cpu().numpy().reshape(T, k), o_ids)
    allclose_report("router weights", w.cpu().numpy().reshape(T, k), o_w, 1e-6, 1e-5)
    # stable counting sort by (expert, token)
    pairs = sorted(((int(o_ids[t, j]), t, j) for t in range(T) for j in range(k)))
    want_tok = np.array([p[1] for p in pairs] + [t for _ in range(n_sh) for t in range(T)])
    assert np.array_equal(row_token.cpu().numpy(), want_tok)
    want_inv = np.empty(T * k, dtype=np.int64)
    for pos, (_, t, j) in enumerate(pairs):
        want_inv[t * k + j] = pos
    assert np.array_equal(inv.cpu().numpy(), want_inv)
    counts = np.bincount(o_ids.reshape(-1), minlength=shape.n_experts)
    assert np.array_equal(offs.cpu().numpy(), np.concatenate([[0], np.cumsum(counts)]))
