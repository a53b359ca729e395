"""Pins for the oracle's network pieces: library routines, brute force,
invariants, the parameter counts the report prints.  CPU only."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from synth.configs import FULL_30, FULL_LAYER, TINY, WORKLOADS
from oracle import model as om
from oracle import step as ost
from oracle.numerics import e4m3_decode, e4m3_round, gelu_tanh, rmsnorm, rope, round_bf16


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 100000), rng.normal(0, 1e-3, 1000),
                        np.ldexp(rng.uniform(1, 2, 1000), -130)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_e4m3_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 100, 20000), rng.normal(0, 0.01, 2000)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4m3_round(x.astype(np.float64)), want)


def test_e4m3_decode_matches_torch_and_spec():
    """Every E4M3 code against torch's float8_e4m3fn (a library decode) and
    the values the OCP FP8 specification fixes: max normal 448 (S.1111.110),
    min normal 2^-6, min subnormal 2^-9, one = 0.0111.000, and the NaN codes."""
    codes = np.arange(256, dtype=np.uint8)
    got = e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], want[~nan])
    spec = {0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x38: 1.0, 0x00: 0.0, 0x07: 7 * 2.0 ** -9,
            0x77: 240.0}
    for c, v in spec.items():
        assert got[c] == v, hex(c)


def test_synth_fp8_rows_quantiser():
    """The fp8 weight recipe (per-row scale = max|w|/448, RNE to E4M3 of w/s)
    against torch's float->float8_e4m3fn cast of the same fp32 ratios, and the
    rounding bound of the decoded values: |q s - w| <= half a step (2^-4 |w|
    for normals, 2^-10 s below 2^-6 s), the row maximum exact at +-448 s."""
    rows, cols = 48, 704
    tid = synth.layer_tid(0, "ex_g")
    codes, sc = synth.e4m3_rows(0, tid, rows, cols, 0.02)
    w = synth.normal(0, tid, (rows, cols), 0.02, "bf16_f64")
    w32 = w.astype(np.float32)
    s_want = (np.abs(w32).max(axis=1) / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(sc, s_want)
    ratio = (w32 / sc[:, None]).astype(np.float32)
    want = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, want)
    deq = e4m3_decode(codes) * sc.astype(np.float64)[:, None]
    a = np.abs(w)
    small = a < 2.0 ** -6 * sc[:, None]
    bound = np.where(small, 2.0 ** -10 * sc[:, None], 2.0 ** -4 * a)
    assert np.all(np.abs(deq - w) <= bound * (1 + 1e-12))
    imax = np.argmax(a, axis=1)
    assert np.array_equal(np.abs(e4m3_decode(codes[np.arange(rows), imax])), np.full(rows, 448.0))
    # oracle weights of an fp8 model are exactly these decoded values
    fp8_shape = replace(TINY, dtype="bf16", expert_dtype="fp8", lm_dtype="fp8", d_expert=cols // 4,
                        n_experts=1)
    W = om.Weights(fp8_shape)
    c2, s2 = synth.e4m3_rows(0, synth.layer_tid(0, "ex_d"), fp8_shape.d_model, fp8_shape.d_expert, 0.02)
    assert np.array_equal(W.get("ex_d", 0)[0], e4m3_decode(c2) * s2.astype(np.float64)[:, None])
    # the shared expert is an expert too: stored in fp8 as well
    c3, s3 = synth.e4m3_rows(0, synth.layer_tid(0, "sh_d"), fp8_shape.d_model, fp8_shape.d_shared, 0.02)
    assert np.array_equal(W.get("sh_d", 0), e4m3_decode(c3) * s3.astype(np.float64)[:, None])


def test_gelu_and_rmsnorm():
    x = np.linspace(-6, 6, 1001)
    want = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.allclose(gelu_tanh(x), want, atol=1e-14)
    rng = np.random.default_rng(2)
    y = rmsnorm(rng.normal(0, 3, (7, 2816)), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-12)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(1, 1, 64))
    k = rng.normal(size=(1, 1, 64))
    for p in (0, 5, 4096, 34815):
        qr = rope(q, np.array([p]), 10000.0)
        assert np.isclose(np.linalg.norm(qr), np.linalg.norm(q), rtol=1e-12)
    # q(m) . k(n) depends only on m - n
    dots = []
    for m, n in ((10, 3), (107, 100), (5007, 5000)):
        dots.append(float((rope(q, np.array([m]), 1e4) * rope(k, np.array([n]), 1e4)).sum()))
    assert np.allclose(dots, dots[0], rtol=1e-9)
    # pairing: position 1, frequency 0 rotates (x0, x1) by 1 radian
    e = np.zeros((1, 1, 4))
    e[..., 0] = 1.0
    r = rope(e, np.array([1]), 10000.0)
    assert np.isclose(r[0, 0, 0], np.cos(1.0)) and np.isclose(r[0, 0, 1], np.sin(1.0))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_matches_sdpa_with_explicit_mask(causal):
    s = TINY
    rng = np.random.default_rng(4)
    n, L = 16, 24
    q = rng.normal(size=(n, s.n_q_heads, s.d_head))
    kk = rng.normal(size=(s.n_kv_heads, L + n, s.d_head))
    vv = rng.normal(size=(s.n_kv_heads, L + n, s.d_head))
    got = om.attention(s, q, kk, vv, L, causal)
    mask = np.ones((n, L + n), dtype=bool)
    if causal:
        for i in range(n):
            mask[i, L + i + 1:] = False
    g = s.n_q_heads // s.n_kv_heads
    qt = torch.from_numpy(q.transpose(1, 0, 2))
    kt = torch.from_numpy(np.repeat(kk, g, axis=0))
    vt = torch.from_numpy(np.repeat(vv, g, axis=0))
    want = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask)).numpy().transpose(1, 0, 2)
    assert np.allclose(got, want, atol=1e-12)
    # brute force per query, explicit loops over visible keys
    for i in (0, n - 1):
        for h in (0, s.n_q_heads - 1):
            vis = np.nonzero(mask[i])[0]
            sc = np.array([q[i, h] @ kk[h // g, j] / np.sqrt(s.d_head) for j in vis])
            w = np.exp(sc - sc.max())
            w /= w.sum()
            o = sum(w[a] * vv[h // g, j] for a, j in enumerate(vis))
            assert np.allclose(got[i, h], o, atol=1e-12)


def _tiny_model(layers=1):
    s = replace(TINY, n_layers=layers)
    return s, om.Weights(s)


def test_encode_mask_perturbation_invariants():
    s, W = _tiny_model(2)
    tok = synth.tokens(0, 10, 20, s.vocab)[None]
    c1 = om.KVCache(s, 1, 64)
    ost.encode_append(s, W, c1, tok[:, :8])
    tok2 = tok.copy()
    tok2[0, 15] = (tok2[0, 15] + 1) % s.vocab
    a = om.KVCache(s, 1, 64)
    b = om.KVCache(s, 1, 64)
    for c in (a, b):
        c.k = [x.copy() for x in c1.k]
        c.v = [x.copy() for x in c1.v]
        c.length = c1.length
    ost.encode_append(s, W, a, tok[:, 8:])
    ost.encode_append(s, W, b, tok2[:, 8:])
    for layer in range(2):
        # causal: positions before the change are unchanged (up to fp64 summation
        # order inside the library matmul, which groups tokens by expert), the
        # changed position moves by O(1)
        assert np.allclose(a.k[layer][:, :, :15], b.k[layer][:, :, :15], rtol=0, atol=1e-12)
        assert np.abs(a.k[layer][:, :, 15] - b.k[layer][:, :, 15]).max() > 1e-3
    # denoise: a change anywhere in the canvas changes every canvas position,
    # and the cache is never written
    before = [x.copy() for x in a.k]
    z1 = ost.denoise_logits(s, W, a, tok[:, :12], None, 8.0)
    tok3 = tok[:, :12].copy()
    tok3[0, 11] = (tok3[0, 11] + 7) % s.vocab
    z2 = ost.denoise_logits(s, W, a, tok3, None, 8.0)
    assert all(np.abs(z1[0, i] - z2[0, i]).max() > 1e-6 for i in range(12))
    assert all(np.array_equal(x, y) for x, y in zip(before, a.k))


def test_append_equals_reencode():
    s, W = _tiny_model(2)
    tok = synth.tokens(1, 10, 40, s.vocab)[None]
    a = om.KVCache(s, 1, 64)
    ost.encode_append(s, W, a, tok[:, :24])
    ost.encode_append(s, W, a, tok[:, 24:])
    b = om.KVCache(s, 1, 64)
    ost.encode_append(s, W, b, tok)
    assert a.length == b.length == 40
    for layer in range(2):
        assert np.allclose(a.k[layer], b.k[layer], rtol=0, atol=1e-12)
        assert np.allclose(a.v[layer], b.v[layer], rtol=0, atol=1e-12)


def test_ar_step_equals_one_shot_causal_forward():
    """The incremental AR step (prefix in the cache, one token appended per
    step) against a one-shot causal forward of the whole sequence with no
    cache: the logits of the last position and the argmax agree, and the
    cache holds the whole sequence's K, V afterwards."""
    s, W = _tiny_model(2)
    tok = synth.tokens(2, 11, 30, s.vocab).reshape(2, 15)
    lm = 8.0
    a = om.KVCache(s, 2, 32)
    ost.encode_append(s, W, a, tok[:, :12])
    for i in range(12, 15):
        nxt, z = ost.ar_step(s, W, a, tok[:, i], lm)
        fresh = om.KVCache(s, 2, 32)
        x = om.embed(s, W, tok[:, :i + 1])
        for layer in range(s.n_layers):
            x = om.layer_forward(s, W, layer, x, fresh, causal=True, append=True)
        z1 = om.final_logits(s, W, x[:, -1], lm)
        assert np.allclose(z, z1, rtol=0, atol=1e-10)
        assert np.array_equal(nxt, np.argmax(z1, axis=-1))
        assert a.length == i + 1
        for layer in range(s.n_layers):
            assert np.allclose(a.k[layer][:, :, :i + 1], fresh.k[layer][:, :, :i + 1], rtol=0, atol=1e-12)
    # greedy ties go to the lower id
    zt = np.zeros((1, s.vocab))
    zt[0, [7, 3]] = 1.0
    assert int(np.argmax(zt, axis=-1)[0]) == 3


def test_route_topk_and_weights():
    s = TINY
    rng = np.random.default_rng(5)
    r = rng.normal(size=(64, s.n_experts))
    r[3, 2] = r[3, 5] = 10.0  # tie at the top: lower id first
    ids, w = om.route(s, r)
    for t in range(64):
        full = sorted(range(s.n_experts), key=lambda e: (-r[t, e], e))
        assert list(ids[t]) == full[: s.top_k]
    assert list(ids[3]) == [2, 5]
    assert np.allclose(w.sum(1), 1.0, atol=1e-14)


def test_moe_equals_dense_sum_with_zero_weights():
    s, W = _tiny_model(1)
    rng = np.random.default_rng(6)
    n2 = rng.normal(size=(32, s.d_model))
    y, r, ids, w = om.moe(s, W, 0, n2, ret_routing=True)
    dense = om.geglu(s, n2, W.get("sh_g", 0), W.get("sh_u", 0), W.get("sh_d", 0))
    gate = np.zeros((32, s.n_experts))
    for t in range(32):
        gate[t, ids[t]] = w[t]
    for e in range(s.n_experts):
        dense = dense + gate[:, e:e + 1] * om.geglu(s, n2, W.get("ex_g", 0)[e], W.get("ex_u", 0)[e],
                                                    W.get("ex_d", 0)[e])
    assert np.allclose(y, dense, atol=1e-12)


def test_parameter_counts_match_report_table1():
    c = FULL_30.param_counts()
    # Technical Report digest, Table 1: total 25.2B, embedder 740M, self-cond 7.8M
    assert abs(c["total_tied_head"] / 1e9 - 25.2) < 0.1
    assert abs(c["embed"] / 1e6 - 740) < 5
    assert abs(c["selfcond"] / 1e6 - 7.8) < 0.2
    # 8 of 128 experts active; active count near the report's 3.85B (3.8 / "4B" elsewhere)
    assert 3.6e9 < c["active_tied_head"] < 3.9e9
    assert TINY.param_counts()["total_untied_head"] == 4329472


def test_synth_c_matches_numpy_definition():
    for dt in ("bf16", "f32"):
        a = synth.normal(7, 1234, (5000,), 0.02, dt, start=999)
        b = synth.normal_np(7, 1234, 5000, 0.02, dt, start=999)
        assert np.array_equal(a, b)
    assert np.array_equal(synth.tokens(3, 10, 4000, 262144), synth.tokens_np(3, 10, 4000, 262144))
    x = synth.bf16_bits_to_f32(synth.normal(0, 1, (1 << 20,), 0.02)).astype(np.float64)
    assert abs(x.std() - 0.02) < 2e-4 and abs(x.mean()) < 1e-4
    d = synth.dirichlet_rows(0, 7, 2, 4096, 0.05)
    assert np.allclose(d.sum(1), 1.0, atol=1e-5) and (d >= 0).all()


def test_resume_from_saved_state_is_identical():
    """Resume invariant of the oracle's step: the state after step t (canvas
    tokens, the tempered distribution carried as self-conditioning input, the
    previous argmax, the cache) copied and continued from gives exactly the
    uninterrupted run's outputs."""
    import copy
    from oracle import sampler as smp
    from oracle import step as ost
    from synth.configs import TINY
    shape, C, L, N = TINY, 16, 24, 6
    W = om.Weights(shape)
    cache = om.KVCache(shape, 1, L + C)
    prompt = synth.tokens(0, synth.TID["prompt"], L, shape.vocab)[None]
    ost.encode_append(shape, W, cache, prompt)
    tok = smp.initial_canvas(5, 0, C, shape.vocab)[None]

    def run(tok, sc, prev, cache, ts):
        outs = []
        for t in ts:
            _, o = ost.denoise_step(shape, W, cache, tok, sc, t, N, [5], 0, 8.0, prev, True)
            o = o[0]
            outs.append(o)
            tok, sc, prev = o["next_tokens"][None], o["p"][None], o["argmax"][None]
        return outs, (tok, sc, prev)

    full, _ = run(tok, None, None, cache, range(4))
    first, state = run(tok, None, None, cache, range(2))
    saved = copy.deepcopy((state, cache))
    rest, _ = run(*saved[0], saved[1], range(2, 4))
    for a, b in zip(full[2:], rest):
        for key in ("H", "sample", "argmax", "accepted", "next_tokens", "p"):
            assert np.array_equal(a[key], b[key]), key


def test_tied_head_reads_the_embedding_and_reaches_the_stop():
    """A tied head is the embedding matrix itself (same values); the model then
    scores its own input token highest by far (the self dot product of a row
    against the cross terms), so with a sharp head every position is accepted,
    the next step's canvas is the same and the adaptive stop fires at t = 1:
    argmax unchanged and the canvas-mean entropy below the threshold."""
    wl = WORKLOADS["tiny"]
    shape = replace(wl.model, tied_head=True)
    W = om.Weights(shape)
    assert np.array_equal(W.get("lm_head"), W.get("embed"))
    assert not np.array_equal(om.Weights(wl.model).get("lm_head"), W.get("embed"))
    cache = om.KVCache(shape, 1, wl.prefix + wl.canvas)
    ost.encode_append(shape, W, cache, np.stack([synth.tokens(0, synth.TID["prompt"], wl.prefix, shape.vocab)]))
    log = []
    _, steps = ost.run_canvas(shape, W, cache, 48, [17], 0, 20.0, True, wl.canvas, commit=False, log=log)
    assert steps == 2
    o0, o1 = log[0]["outs"][0], log[1]["outs"][0]
    assert o0["n_accepted"] == wl.canvas and not o0["stop"]  # t = 0 never stops
    assert np.array_equal(o0["argmax"], log[0]["tokens"][0])   # the input tokens predicted back
    assert np.array_equal(o1["argmax"], o0["argmax"]) and o1["mean_H"] < 0.005 and o1["stop"]
