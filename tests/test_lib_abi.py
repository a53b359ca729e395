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
