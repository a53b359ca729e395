"""Pins of the MXFP4 weight format: the oracle's E2M1 / E8M0 decode and the
input recipe's block quantiser (OCP Microscaling Formats v1.0: 32-element
blocks, FP4 E2M1 elements, E8M0 shared scale)."""
import os
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle.numerics import e2m1_decode, e2m1_value, e8m0_decode, mxfp4_dequantize
from synth.configs import MINI_BF16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_mx_fp4_e2m1.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        rows.append((int(code, 2), float(val)))
    return rows


def test_e2m1_decode_matches_the_spec_table():
    rows = _golden()
    assert [c for c, _ in rows] == list(range(16))
    for c, v in rows:
        got = e2m1_value(c)
        assert got == v and np.signbit(got) == np.signbit(v), (c, got, v)
    assert np.array_equal(e2m1_decode(np.arange(16)), np.array([v for _, v in rows]))
    with pytest.raises(ValueError):
        e2m1_decode([16])


def test_e8m0_decode():
    assert e8m0_decode(127) == 1.0
    assert e8m0_decode(0) == 2.0 ** -127
    assert e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(e8m0_decode(255))
    c = np.arange(255)
    assert np.array_equal(e8m0_decode(c[1:]) / e8m0_decode(c[:-1]), np.full(254, 2.0))


def test_dequantize_applies_each_block_scale():
    codes = np.full((2, 96), 2, dtype=np.uint8)  # 1.0 everywhere
    codes[1, 40] = 15                             # -6.0
    sc = np.array([[127, 128, 120], [130, 127, 127]], dtype=np.uint8)
    w = mxfp4_dequantize(codes, sc)
    assert np.array_equal(w[0], np.concatenate([np.full(32, 1.0), np.full(32, 2.0), np.full(32, 2.0 ** -7)]))
    assert w[1, 0] == 8.0 and w[1, 40] == -6.0 and w[1, 95] == 1.0


def _quant_values(w):
    c, s = synth.mxfp4_quantize(np.asarray(w, dtype=np.float32)[None, :])
    return c[0], s[0], mxfp4_dequantize(c, s)[0]


def test_quantiser_round_trips_representable_blocks():
    rng = np.random.default_rng(0)
    for E in (-20, -7, 0, 5):
        codes = rng.integers(0, 16, 64).astype(np.uint8)
        codes[3] = 7       # 6.0: the block maximum sets the exponent
        codes[40] = 14     # -4.0
        w = e2m1_decode(codes) * 2.0 ** E
        c, s, back = _quant_values(w)
        assert np.array_equal(s, [E + 127, E + 127])
        assert np.array_equal(back, w)
        assert np.array_equal(c & 7, codes & 7)  # signs of zero may differ


def test_quantiser_rounds_to_nearest_even_and_saturates():
    X = 2.0 ** -3
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 4.0])
    w = np.zeros(32)
    w[:8] = ties * X
    w[8:16] = -ties * X
    w[16] = 7.5 * X   # largest block value: exponent floor(log2 7.5) - 2 = 0 -> X, saturates to 6
    c, s, back = _quant_values(w)
    assert s[0] == 127 - 3
    assert np.array_equal(back[:8], want * X)
    assert np.array_equal(back[8:16], -want * X)
    assert back[16] == 6.0 * X
    # just off the midpoints: to the nearer neighbour
    eps = 1e-3
    w2 = np.zeros(32)
    w2[:7] = (ties[:7] + eps) * X
    w2[7] = 4.0 * X
    _, _, back2 = _quant_values(w2)
    assert np.array_equal(back2[:7], np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]) * X)


def test_quantiser_scale_choice_and_error_bound():
    w = synth.normal(0, 77, (64, 256), 0.02, "bf16_f64").astype(np.float32)
    c, s = synth.mxfp4_quantize(w)
    X = e8m0_decode(s)                               # [64][8]
    amax = np.abs(w.astype(np.float64)).reshape(64, 8, 32).max(axis=2)
    r = amax / X
    assert np.all((r >= 4.0) & (r < 8.0))            # the block maximum's binade is [4, 8)
    d = mxfp4_dequantize(c, s)
    x = np.abs(w.astype(np.float64)) / np.repeat(X, 32, axis=1)
    half_step = np.where(x < 2.0, 0.25, np.where(x < 4.0, 0.5, 1.0))
    bound = np.where(x > 6.0, x - 6.0, half_step) * np.repeat(X, 32, axis=1)
    assert np.all(np.abs(d - w) <= bound + 0.0)
    assert np.all(np.sign(d) * np.sign(w) >= 0)


def test_quantiser_zero_block():
    c, s, back = _quant_values(np.zeros(32))
    assert s[0] == 0 and np.all(c == 0) and np.all(back == 0.0)


def test_rows_generator_is_the_quantiser_on_the_bf16_tensor():
    rows, cols = 48, 128
    c, s = synth.mxfp4_rows(0, 123, rows, cols, 0.02)
    w = synth.normal(0, 123, (rows, cols), 0.02, "bf16_f64").astype(np.float32)
    c2, s2 = synth.mxfp4_quantize(w)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def test_oracle_weights_of_an_mxfp4_model():
    from oracle import model as om
    shape = replace(MINI_BF16, expert_dtype="mxfp4")
    W = om.Weights(shape)
    g = W.get("ex_g", 0)
    c, s = synth.mxfp4_rows(shape.weight_seed, synth.layer_tid(0, "ex_g"), shape.n_experts * shape.d_expert,
                            shape.d_model, shape.weight_std)
    assert np.array_equal(g.reshape(-1, shape.d_model), mxfp4_dequantize(c, s))
    # the dense weights stay bf16
    assert np.array_equal(W.get("wqkv", 0), om.Weights(MINI_BF16).get("wqkv", 0))
