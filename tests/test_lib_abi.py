"""CPU checks of the C-ABI library: it loads, exports every symbol that
include/dg.h declares, and its host-only entry points behave (no GPU needed:
argument errors are found before anything is launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def dg():
    import discrete_text_diffusion_amd as m
    return m


def test_library_exports_every_declared_symbol(dg):
    lib = ctypes.CDLL(dg.LIB_PATH)
    names = _declared()
    assert "dg_denoise_step" in names and "dg_encode_append" in names and "dg_commit_block" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dg.EXPORTED)


def test_temperature_matches_oracle_schedule(dg):
    from oracle.sampler import temperature
    for n in (1, 2, 12, 48, 192):
        for t in range(n):
            assert np.float32(dg.dg_temperature(t, n)) == np.float32(temperature(t, n))


def test_workspace_and_config_checks(dg):
    from synth.configs import FULL_30, MINI_BF16, TINY
    from discrete_text_diffusion_amd.runtime import model_config
    for shp in (TINY, MINI_BF16, FULL_30):
        assert dg.dg_workspace_bytes(model_config(shp), 1, 256) > 0
    bad = model_config(MINI_BF16)
    bad.d_head = 128  # bf16 path needs d_head 256
    assert dg.dg_workspace_bytes(bad, 1, 256) == 0
    # fp8 expert / LM-head weights: bf16 models only; fp8 experts need d_model % 128
    from dataclasses import replace
    from synth.configs import FULL_LAYER_FP8
    assert dg.dg_workspace_bytes(model_config(FULL_LAYER_FP8), 4, 256) > 0
    assert dg.dg_workspace_bytes(model_config(replace(TINY, expert_dtype="fp8")), 1, 32) == 0
    odd = model_config(replace(MINI_BF16, expert_dtype="fp8"))
    odd.d_model = 320
    assert dg.dg_workspace_bytes(odd, 1, 32) == 0
    assert dg.dg_workspace_bytes(model_config(replace(MINI_BF16, lm_dtype="fp8")), 1, 32) > 0


def test_argument_errors_are_reported_before_launch(dg):
    from synth.configs import TINY
    from discrete_text_diffusion_amd.runtime import model_config
    cfg = model_config(TINY)
    w = dg.Weights()
    cache = dg.KVCache(None, None, 1, 16, 0)
    cv = dg.Canvas()
    p = dg.StepParams(0, 48, 0, 1, 0.1, 0.005)
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step(cfg, w, cache, cv, p, None, 0, None)
    assert e.value.status == dg.DG_ERR_INVALID_ARG
    with pytest.raises(dg.DGError) as e:
        dg.dg_encode_append(cfg, w, cache, None, 1, 8, None, 0, None)
    assert e.value.status == dg.DG_ERR_INVALID_ARG
    with pytest.raises(dg.DGError):
        dg.dg_pack_weight_bf16(None, None, 17, 32, None)
    assert dg.dg_status_string(dg.DG_ERR_KV_CAPACITY) == "KV cache capacity exceeded"


def _fake_structs(dg, shape, B, C, cap, length):
    """Weights, cache and canvas whose device pointers are fake (aligned,
    never dereferenced): every call below is rejected by the host-side checks
    before anything is enqueued."""
    fake = 1 << 40
    layers = (dg.LayerWeights * shape.n_layers)(
        *[dg.LayerWeights(*([fake] * 9 + [None] * 6)) for _ in range(shape.n_layers)])
    w = dg.Weights(fake, fake, fake, fake, fake, layers, 1.0, None)
    cache = dg.KVCache(fake, fake, B, cap, length)
    cv = dg.Canvas(B, C, fake, fake, None, None, None, *([fake] * 9), fake)
    return w, cache, cv, fake


def test_new_entry_points_check_arguments_on_the_host(dg):
    from synth.configs import TINY
    from discrete_text_diffusion_amd.runtime import model_config
    cfg = model_config(TINY)
    step = lambda t, n, b: dg.StepParams(t, n, b, 1, 0.1, 0.005)  # noqa: E731

    def status(fn, *args):
        with pytest.raises(dg.DGError) as e:
            fn(*args)
        return e.value.status

    w, cache, cv, fake = _fake_structs(dg, TINY, 1, 32, 64, 16)
    big = 1 << 50
    # commit + next step: the next step must be step 0 of the following block
    assert status(dg.dg_commit_and_step, cfg, w, cache, cv, step(5, 12, 0), step(1, 12, 1), fake, big,
                  None) == dg.DG_ERR_INVALID_ARG
    assert status(dg.dg_commit_and_step, cfg, w, cache, cv, step(5, 12, 0), step(0, 12, 2), fake, big,
                  None) == dg.DG_ERR_INVALID_ARG
    # committed rows and the next canvas's scratch rows: 16 + 2 x 32 > 64
    assert status(dg.dg_commit_and_step, cfg, w, cache, cv, step(5, 12, 0), step(0, 12, 1), fake, big,
                  None) == dg.DG_ERR_KV_CAPACITY
    # single-token decode: batch, full cache, workspace
    assert status(dg.dg_ar_step, cfg, w, cache, fake, 0, fake, fake, big, None) == dg.DG_ERR_INVALID_ARG
    full = dg.KVCache(fake, fake, 1, 64, 64)
    assert status(dg.dg_ar_step, cfg, w, full, fake, 1, fake, fake, big, None) == dg.DG_ERR_KV_CAPACITY
    assert status(dg.dg_ar_step, cfg, w, cache, fake, 1, fake, None, 0, None) == dg.DG_ERR_WORKSPACE
    assert status(dg.dg_test_ar_step, cfg, w, cache, fake, 1, fake, None, fake, big, None) == dg.DG_ERR_INVALID_ARG
    assert cache.length == 16 and full.length == 64
    # more than 16384 canvas tokens in one denoising step
    w2, cache2, cv2, _ = _fake_structs(dg, TINY, 17, 1024, 1024, 0)
    assert status(dg.dg_denoise_step, cfg, w2, cache2, cv2, step(0, 12, 0), fake, big,
                  None) == dg.DG_ERR_UNSUPPORTED


def test_noalloc_step_limit_is_checked_on_the_host(dg):
    """dg_denoise_step_noalloc refuses a step whose scratch exceeds its static
    array before touching the GPU: two 256-token canvases at the pages' full
    width need about 560 MiB of the 320 MiB it holds; a malformed call is an
    argument error first."""
    from synth.configs import FULL_LAYER
    from discrete_text_diffusion_amd.runtime import model_config
    cfg = model_config(FULL_LAYER)
    step = dg.StepParams(0, 12, 0, 1, 0.1, 0.005)
    w, cache, cv, fake = _fake_structs(dg, FULL_LAYER, 2, 256, 2048 + 256, 2048)
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step_noalloc(cfg, w, cache, cv, step, None)
    assert e.value.status == dg.DG_ERR_SCRATCH_LIMIT
    assert "no-allocation scratch" in dg.dg_status_string(dg.DG_ERR_SCRATCH_LIMIT)
    bad = dg.Canvas(0, 256, fake, fake, None, None, None, *([fake] * 9), fake)
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step_noalloc(cfg, w, cache, bad, step, None)
    assert e.value.status == dg.DG_ERR_INVALID_ARG
    assert dg.DG_NOALLOC_SCRATCH_BYTES == 320 << 20
