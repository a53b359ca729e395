"""Workload definitions: model shapes and the seeded synthetic run recipes.

These are inputs (sizes, dtypes, seeds, the LM-head scale of the random-init
models), shared by the oracle and the GPU path.  The sampler's own constants
(temperature endpoints, entropy bound, stop threshold) are not here: each side
states them itself.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    n_experts: int
    top_k: int
    d_expert: int
    d_shared: int
    vocab: int
    d_selfcond: int
    dtype: str = "bf16"          # dense weights and activation storage: "f32" | "bf16"
    expert_dtype: str = "bf16"   # routed and shared experts: "f32" | "bf16" | "fp8" | "mxfp4"
    lm_dtype: str = "bf16"       # "f32" | "bf16" | "fp8"
    rope_base: float = 10000.0
    norm_eps: float = 1e-6
    weight_std: float = 0.02
    weight_seed: int = 0
    # LM head tied to the embedding (generated from the embedding's tensor id,
    # so both are the same matrix); the page workloads keep separate heads
    tied_head: bool = False

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.d_head

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.d_head

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.d_head

    def param_counts(self) -> dict:
        d = self.d_model
        per_layer_dense = self.qkv_rows * d + d * self.q_dim + self.n_experts * d + 3 * self.d_shared * d
        per_layer_experts = self.n_experts * 3 * self.d_expert * d
        embed = self.vocab * d
        sc = 2 * d * self.d_selfcond
        total_tied = self.n_layers * (per_layer_dense + per_layer_experts) + embed + sc
        active = (self.n_layers * (per_layer_dense + self.top_k * 3 * self.d_expert * d)
                  + embed + sc)
        return {
            "per_layer": per_layer_dense + per_layer_experts,
            "embed": embed,
            "selfcond": sc,
            "total_tied_head": total_tied,
            "total_untied_head": total_tied + embed,
            "active_tied_head": active,
        }


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: int
    canvas: int
    prefix: int                  # prompt tokens causally encoded before the first canvas
    prefix_mode: str = "encode"  # "encode" (run the causal encoder) | "random_kv" (N(0,1) cache)
    n_steps: int = 48
    adaptive: bool = True
    lm_scale: float = 1.0
    n_blocks: int = 1
    sampler_seeds: tuple = (0,)
    prompt_seed: int = 0
    selfcond_init: str = "none"  # "none" | "dirichlet" (external P for the first step)
    dirichlet_alpha: float = 0.05
    first_step: int = 0


TINY = ModelShape(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, d_head=64, n_experts=8,
                  top_k=2, d_expert=128, d_shared=128, vocab=4096, d_selfcond=128,
                  dtype="f32", expert_dtype="f32", lm_dtype="f32")

FULL_LAYER = ModelShape(n_layers=1, d_model=2816, n_q_heads=16, n_kv_heads=8, d_head=256,
                        n_experts=128, top_k=8, d_expert=704, d_shared=2112, vocab=262144,
                        d_selfcond=1408)

FULL_30 = replace(FULL_LAYER, n_layers=30)

FULL_LAYER_FP8 = replace(FULL_LAYER, expert_dtype="fp8", lm_dtype="fp8")

# 4-bit experts (OCP MXFP4: E2M1 elements, an E8M0 scale per 32 inputs), the
# rest bf16: the 30-layer model and the one-layer model of the fp8 workload
# with its experts in MXFP4 instead of fp8 (LM head fp8).
FULL_30_MX4 = replace(FULL_30, expert_dtype="mxfp4")
FULL_LAYER_MX4 = replace(FULL_LAYER, expert_dtype="mxfp4", lm_dtype="fp8")

# Small bf16 shape for parity tests of the MFMA path: several K chunks, 16
# vocabulary tiles, ragged expert segments, a shared expert split in two
# d_expert-wide slices.  Not one of the pages' workloads.
MINI_BF16 = ModelShape(n_layers=2, d_model=256, n_q_heads=2, n_kv_heads=1, d_head=256, n_experts=16,
                       top_k=4, d_expert=128, d_shared=256, vocab=4096, d_selfcond=128)

WORKLOADS = {
    # 2-layer fp32 denoiser; prefix 64 encoded causally; canvas 32; <=48 adaptive steps.
    "tiny": Workload("tiny", TINY, batch=1, canvas=32, prefix=64, n_steps=48, adaptive=True,
                     lm_scale=8.0),
    # one full-width layer + LM head; random N(0,1) cache of 2048; Dirichlet(0.05) self-cond;
    # single step at t = 1 of a 48-step budget.
    "layer1": Workload("layer1", FULL_LAYER, batch=1, canvas=256, prefix=2048,
                       prefix_mode="random_kv", n_steps=48, adaptive=False, lm_scale=1.0,
                       selfcond_init="dirichlet", first_step=1),
    # full 30-layer model; 4096-token causal prefix; one canvas; fixed 12 / 48 and adaptive.
    # LM-head scale 7.6: about 20 accepted tokens per step over the 12-step run, measured on
    # the model itself (mean over sampler seeds 0..3: 7.0 -> 16.0, 7.5 -> 19.3, 8.0 -> 22.5);
    # tests/golden/calibrate_lm_scale.py gives the independent-positions estimate.
    "full30": Workload("full30", FULL_30, batch=1, canvas=256, prefix=4096, n_steps=12,
                       adaptive=False, lm_scale=7.6),
    # long context on the one-layer model: 32768 prefix, 8 committed canvases.
    "longctx": Workload("longctx", FULL_LAYER, batch=1, canvas=256, prefix=32768, n_steps=48,
                        adaptive=True, n_blocks=8, lm_scale=1.0),
    # fp8 experts + LM head, 4 independent canvases over 8192-row prefixes (random N(0,1)
    # cache as in the one-layer workload), 12 steps, sampler seeds 0..3.
    "fp8batch4": Workload("fp8batch4", FULL_LAYER_FP8, batch=4, canvas=256, prefix=8192,
                          prefix_mode="random_kv", n_steps=12, adaptive=False, lm_scale=1.0,
                          sampler_seeds=(0, 1, 2, 3)),
    # the 30-layer workload with MXFP4 experts (same LM-head scale)
    "full30_mx4": Workload("full30_mx4", FULL_30_MX4, batch=1, canvas=256, prefix=4096, n_steps=12,
                           adaptive=False, lm_scale=7.6),
    # the fp8 batch-4 workload with MXFP4 experts
    "mx4batch4": Workload("mx4batch4", FULL_LAYER_MX4, batch=4, canvas=256, prefix=8192,
                          prefix_mode="random_kv", n_steps=12, adaptive=False, lm_scale=1.0,
                          sampler_seeds=(0, 1, 2, 3)),
}
