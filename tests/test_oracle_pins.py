"""Closed-form pins of the oracle's self-conditioning input, GeGLU block and
LM head on hand-set weights (CPU only).

The synthetic weights are random, so nothing printed on the pages fixes a
value of these functions.  Here the weights are chosen by hand so that the
answer follows from the definitions without evaluating them the way the
oracle does: one-hot and two-hot probability rows make the expected
embedding an embedding row or the mean of two; pre-activations of 0 and of
+-10 make the tanh-GELU exactly 0, the identity, or zero to 1e-20; unit
rows in the LM head read single coordinates of the normalised state.  Each
case fails under the mistakes a reader could make in that code: swapped
gate/up roles, a transposed or swapped self-conditioning matrix, a missing
term, a wrong normalisation.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from synth.configs import TINY
from oracle import model as om
from oracle import step as ost


class HandWeights:
    """Weights given as explicit arrays, read through the oracle's interface."""

    def __init__(self, shape, mats):
        self.shape = shape
        self.mats = {k: np.asarray(v, dtype=np.float64) for k, v in mats.items()}

    def get(self, name, layer=None):
        return self.mats[name]


# d_model 4, self-conditioning width 3, vocabulary 5; fp32 model: no storage rounding
SHAPE = replace(TINY, d_model=4, d_selfcond=3, vocab=5, n_layers=1)

E = np.array([
    [0.5, -1.0, 2.0, 0.25],
    [1.5, 0.0, -0.5, 1.0],
    [1.0, 0.0, 0.0, 0.0],
    [0.0, 1.0, 0.0, 0.0],
    [0.0, 0.0, 3.0, -2.0],
])


def _sc_weights(sc_up, sc_down):
    return HandWeights(SHAPE, {"embed": E, "sc_up": sc_up, "sc_down": sc_down})


def _gelu_tanh_torch(v):
    return float(torch.nn.functional.gelu(torch.tensor(float(v), dtype=torch.float64), approximate="tanh"))


def test_selfcond_one_hot_reads_the_embedding_row():
    """P one-hot at id 2 makes the expected embedding E[2] = e_0.  sc_up's
    rows dotted with e_0 give pre-activations (0, 10, -10): hidden (0, 10,
    ~0), so the input becomes E[tok] + 10 * sc_down[:, 1]."""
    sc_up = np.array([[0.0, 7.0, -1.0, 2.0],
                      [10.0, 3.0, 0.0, 0.0],
                      [-10.0, 0.0, 5.0, 1.0]])
    sc_down = np.array([[1.0, 0.5, 4.0],
                        [2.0, -1.0, 4.0],
                        [3.0, 0.25, 4.0],
                        [4.0, 2.0, 4.0]])
    W = _sc_weights(sc_up, sc_down)
    tokens = np.array([[0, 4]])
    P = np.zeros((1, 2, 5))
    P[0, :, 2] = 1.0
    x = om.embed(SHAPE, W, tokens, P)
    want = E[[0, 4]] + 10.0 * sc_down[:, 1][None, :]
    assert np.allclose(x[0], want, rtol=0, atol=1e-12)
    # the gelu(-10) term is below 1e-20 and gelu(10) = 10 to 1e-14 (tanh form)
    assert abs(_gelu_tanh_torch(-10.0)) < 1e-20 and abs(_gelu_tanh_torch(10.0) - 10.0) < 1e-13
    # without self-conditioning the input is the embedding row alone
    assert np.array_equal(om.embed(SHAPE, W, tokens, None)[0], E[[0, 4]])
    # swapping the two matrices' roles, or using sc_down transposed, changes the answer
    swapped = _sc_weights(sc_down.T, sc_up.T)
    assert not np.allclose(om.embed(SHAPE, swapped, tokens, P)[0], want, atol=1e-3)


def test_selfcond_two_hot_gives_the_mean_embedding():
    """P = 1/2 on ids 2 and 3: the expected embedding is (E[2] + E[3]) / 2 =
    (1/2, 1/2, 0, 0).  sc_up row 0 = (20, 0, 0, 0) gives pre-activation 10,
    row 1 = (0, 2, 0, 0) gives 1, row 2 = (0, 0, 9, 9) gives 0: hidden
    (10, gelu(1), 0).  gelu(1) comes from the library's tanh-GELU."""
    sc_up = np.array([[20.0, 0.0, 0.0, 0.0],
                      [0.0, 2.0, 0.0, 0.0],
                      [0.0, 0.0, 9.0, 9.0]])
    sc_down = np.array([[1.0, 0.0, 5.0],
                        [0.0, 1.0, 5.0],
                        [1.0, 1.0, 5.0],
                        [-1.0, 2.0, 5.0]])
    W = _sc_weights(sc_up, sc_down)
    P = np.zeros((1, 1, 5))
    P[0, 0, 2] = P[0, 0, 3] = 0.5
    x = om.embed(SHAPE, W, np.array([[1]]), P)
    g1 = _gelu_tanh_torch(1.0)
    assert abs(g1 - 0.8411919906082768) < 1e-15  # 0.5 (1 + tanh(sqrt(2/pi) 1.044715))
    h = np.array([10.0, g1, 0.0])
    want = E[1] + sc_down @ h
    assert np.allclose(x[0, 0], want, rtol=0, atol=1e-12)
    # weighting by P, not a plain average of the row: moving the mass changes ebar
    P2 = np.zeros((1, 1, 5))
    P2[0, 0, 2], P2[0, 0, 3] = 0.75, 0.25
    x2 = om.embed(SHAPE, W, np.array([[1]]), P2)
    h2 = np.array([_gelu_tanh_torch(15.0), _gelu_tanh_torch(0.5), 0.0])
    assert np.allclose(x2[0, 0], E[1] + sc_down @ h2, rtol=0, atol=1e-12)


def test_selfcond_rounds_the_expected_embedding_in_bf16_models():
    """bf16 models round the expected embedding before the MLP: P = (1/3,
    2/3) over ids 2, 3 gives ebar = (1/3, 2/3, 0, 0), stored as the bf16
    values 0.333984375 and 0.66796875; with sc_up row 0 = e_0 scaled by 30
    the pre-activation is 30 * 0.333984375 = 10.01953125 (not 10)."""
    shape = replace(SHAPE, dtype="bf16", expert_dtype="bf16", lm_dtype="bf16")
    sc_up = np.array([[30.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    sc_down = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 0.0], [0.0, 0.0, 0.0], [0.0, 0.0, 0.0]])
    W = HandWeights(shape, {"embed": E, "sc_up": sc_up, "sc_down": sc_down})
    P = np.zeros((1, 1, 5))
    P[0, 0, 2], P[0, 0, 3] = 1.0 / 3.0, 2.0 / 3.0
    x = om.embed(shape, W, np.array([[3]]), P)
    # P itself is rounded to bf16 first: 1/3 -> 0.333984375, 2/3 -> 0.66796875
    pre = 30.0 * 0.333984375
    h = float(torch.tensor(_gelu_tanh_torch(pre)).to(torch.bfloat16).double())
    assert x[0, 0, 0] == E[3, 0] + h
    assert x[0, 0, 1] == E[3, 1]


GE_SHAPE = replace(TINY, d_model=4, n_layers=1)


def test_geglu_gate_and_up_roles():
    """u = e_0.  Gate rows give (2, 0), up rows give (-3, 5): hidden
    (gelu(2) * -3, gelu(0) * 5) = (-3 gelu(2), 0); W_d = [[1, 0], [0, 1],
    [1, 1]] reads it back.  Swapping gate and up gives gelu(-3) * 2 instead,
    about 0.0073 against -5.86."""
    u = np.array([[1.0, 0.0, 0.0, 0.0]])
    wg = np.array([[2.0, 1.0, 1.0, 1.0], [0.0, 4.0, 4.0, 4.0]])
    wu = np.array([[-3.0, 9.0, 9.0, 9.0], [5.0, 9.0, 9.0, 9.0]])
    wd = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    got = om.geglu(GE_SHAPE, u, wg, wu, wd)
    g2 = _gelu_tanh_torch(2.0)
    assert abs(g2 - 1.954597694087775) < 1e-14  # 1 + tanh(sqrt(2/pi) 2.35772)
    want = np.array([[-3.0 * g2, 0.0, -3.0 * g2]])
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    swapped = om.geglu(GE_SHAPE, u, wu, wg, wd)
    assert abs(swapped[0, 0] - want[0, 0]) > 5.0
    # the shared expert enters with weight 1 and the routed ones with their gate weights:
    # a layer's MoE output is shared + sum_j w_j expert_j (checked in test_oracle_model)


def test_final_logits_read_the_normalised_state():
    """x = (3, 4, 0, 0): mean square 25/4, so RMSNorm(x) = (1.2, 1.6, 0, 0)
    (eps 1e-6 moves it by 8e-8 relative).  Unit and sum rows of W_lm read
    those coordinates; the LM-head scale multiplies every logit."""
    shape = replace(TINY, d_model=4, vocab=4, n_layers=1)
    wlm = np.array([[1.0, 0.0, 0.0, 0.0],
                    [0.0, 1.0, 0.0, 0.0],
                    [1.0, 1.0, 0.0, 0.0],
                    [0.0, -1.0, 5.0, 5.0]])
    W = HandWeights(shape, {"lm_head": wlm})
    x = np.array([[[3.0, 4.0, 0.0, 0.0]]])
    z = om.final_logits(shape, W, x, 2.0)
    r = np.sqrt(25.0 / 4.0 + 1e-6)
    want = 2.0 * np.array([3.0, 4.0, 7.0, -4.0]) / r
    assert np.allclose(z[0, 0], want, rtol=1e-14, atol=0)
    assert abs(r - 2.5) < 1e-6
    # rows, not columns, of W_lm are the vocabulary entries
    zt = om.final_logits(shape, HandWeights(shape, {"lm_head": wlm.T}), x, 2.0)
    assert not np.allclose(zt, z)


def test_denoise_logits_without_layers_is_embedding_then_head():
    """With zero layers the denoiser's logits are the LM head of the
    embedding plus the self-conditioning term: a composition check of the
    pieces above in the order the step runs them."""
    shape = replace(SHAPE, n_layers=0)
    sc_up = np.array([[20.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    sc_down = np.array([[0.0, 0.0, 0.0], [0.0, 0.0, 0.0], [1.0, 0.0, 0.0], [0.0, 0.0, 0.0]])
    wlm = np.eye(5, 4)
    W = HandWeights(shape, {"embed": E, "sc_up": sc_up, "sc_down": sc_down, "lm_head": wlm})
    P = np.zeros((1, 1, 5))
    P[0, 0, 2] = 1.0  # ebar = e_0, pre-activation 20: hidden (20, 0, 0)
    z = ost.denoise_logits(shape, W, om.KVCache(shape, 1, 1), np.array([[3]]), P, 1.0)
    xin = E[3] + np.array([0.0, 0.0, 20.0, 0.0])  # (0, 1, 20, 0)
    n = xin / np.sqrt(np.mean(xin ** 2) + 1e-6)
    assert np.allclose(z[0, 0], np.concatenate([n, [0.0]]), rtol=1e-12, atol=1e-15)


def test_float32_twin_orders():
    """The float32 evaluations used to measure drift: both orders are float32
    sums of the exact products (within K * 2^-24 relative of the float64
    result), they differ from each other in the last bits, and neither
    changes the float64 default."""
    rng = np.random.default_rng(5)
    a = rng.standard_normal((8, 4096))
    b = rng.standard_normal((4096, 16))
    exact = a @ b
    with om.twin_order("rev"):
        assert np.array_equal(om.mm(a, b), exact)          # f64 default unaffected
    a32 = a.astype(np.float32).astype(np.float64)
    b32 = b.astype(np.float32).astype(np.float64)
    ref = a32 @ b32
    bound = 4096 * 2.0 ** -24 * (np.abs(a32) @ np.abs(b32))
    with om.accumulation("f32"):
        fwd = om.mm(a, b)
        with om.twin_order("rev"):
            rev = om.mm(a, b)
    assert np.all(np.abs(fwd - ref) <= bound) and np.all(np.abs(rev - ref) <= bound)
    assert not np.array_equal(fwd, rev)
    with pytest.raises(ValueError):
        with om.twin_order("sideways"):
            pass
