"""ORACLE — plain, slow, fp64 CPU implementation of one denoising step of the
block-diffusion MoE decoder, and of the encode-and-append around it.

This package is TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code
with the HIP path (``discrete_text_diffusion_amd``); the only module both use is
``synth`` (seeded inputs, no method arithmetic).

Modules:
  philox   — Philox4x32-10 from Salmon et al. (SC'11); pinned to the published
             known-answer vectors.
  numerics — bf16 / e4m3 rounding, RMSNorm, tanh-GELU, RoPE, softmax, entropy.
  model    — embedding + self-conditioning, attention with explicit masks,
             MoE routing and experts, LM head.
  sampler  — temperature schedule, entropy, tile-composition sampling,
             entropy-bounded acceptance, re-noise, stop test.
  step     — encode_append / denoise_step / run_canvas.

Pins (tests/test_oracle_*.py) check each part against closed forms, brute
force, library routines and the pages' fixed constants.
"""
