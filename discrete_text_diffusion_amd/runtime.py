"""Device-memory holders for the C ABI: model weights, KV cache, canvas state
and workspace, allocated as torch tensors on the GPU (PyTorch is used for
memory and streams only).  Synthetic weights are filled in place by the
seeded device generator (``synth``) and packed into the weight layout by the
library's own pack kernel.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

import synth
from synth.configs import ModelShape

from . import (Canvas, KVCache, LayerWeights, ModelConfig, StepParams, Weights, DG_DTYPE_BF16, DG_DTYPE_F32,
               DG_DTYPE_FP8_E4M3, DG_DTYPE_MXFP4, dg_pack_weight_bf16, dg_pack_weight_bf16_transposed,
               dg_pack_weight_fp8, dg_pack_weight_mxfp4, dg_workspace_bytes)


def stream_handle(stream: torch.cuda.Stream | None = None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


_DTYPE = {"f32": DG_DTYPE_F32, "bf16": DG_DTYPE_BF16, "fp8": DG_DTYPE_FP8_E4M3, "mxfp4": DG_DTYPE_MXFP4}


def model_config(shape: ModelShape) -> ModelConfig:
    return ModelConfig(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.d_head,
                       shape.n_experts, shape.top_k, shape.d_expert, shape.d_shared, shape.vocab,
                       shape.d_selfcond, _DTYPE[shape.dtype], shape.rope_base, shape.norm_eps,
                       _DTYPE[shape.expert_dtype], _DTYPE[shape.lm_dtype])


def _tdtype(shape: ModelShape):
    return torch.bfloat16 if shape.dtype == "bf16" else torch.float32


class DeviceModel:
    """Synthetic model weights on the GPU in the library's layout."""

    def __init__(self, shape: ModelShape, lm_scale: float, device="cuda", selfcond: bool = True):
        self.shape = shape
        self.cfg = model_config(shape)
        self.device = torch.device(device)
        self.bf = shape.dtype == "bf16"
        self.tensors = {}
        st = stream_handle()
        d = shape.d_model
        tmp = None
        if self.bf:
            # largest logical matrix, reused as the staging buffer for packing
            biggest = max(shape.vocab * d, shape.n_experts * shape.d_expert * d, shape.qkv_rows * d)
            tmp = torch.empty(biggest, dtype=torch.bfloat16, device=self.device)

        def fill8(name, tid, rows, cols, groups=1):
            # fp8: per-output-row scales and E4M3 codes, packed to the fp8 layout
            n = groups * rows * cols
            codes = tmp.view(torch.uint8)[:n]
            sc = torch.empty(groups * rows, dtype=torch.float32, device=self.device)
            synth.dev_e4m3_rows(codes.data_ptr(), sc.data_ptr(), groups * rows, cols, shape.weight_seed, tid,
                                shape.weight_std, st)
            t = torch.empty(n, dtype=torch.uint8, device=self.device)
            dg_pack_weight_fp8(t.data_ptr(), codes.data_ptr(), groups * rows, cols, st)
            self.tensors[name] = t
            self.tensors[name + "_scale"] = sc
            return t

        def fill4(name, tid, rows, cols, groups=1):
            # MXFP4: E2M1 codes (one per byte) and E8M0 block scales, packed to
            # the MXFP4 layout (17 bytes per 32 weights)
            n = groups * rows * cols
            codes = tmp.view(torch.uint8)[:n]
            sc = torch.empty(n // 32, dtype=torch.uint8, device=self.device)
            synth.dev_mxfp4_rows(codes.data_ptr(), sc.data_ptr(), groups * rows, cols, shape.weight_seed, tid,
                                 shape.weight_std, st)
            t = torch.empty(n // 32 * 17, dtype=torch.uint8, device=self.device)
            dg_pack_weight_mxfp4(t.data_ptr(), codes.data_ptr(), sc.data_ptr(), groups * rows, cols, st)
            torch.cuda.synchronize()  # sc is freed on return
            self.tensors[name] = t
            return t

        def fill(name, tid, rows, cols, groups=1, pack=True, keep_plain=False, fp8=False, mx4=False):
            if fp8:
                return fill8(name, tid, rows, cols, groups)
            if mx4:
                return fill4(name, tid, rows, cols, groups)
            n = groups * rows * cols
            if not self.bf:
                t = torch.empty(n, dtype=torch.float32, device=self.device)
                synth.dev_normal(t.data_ptr(), n, shape.weight_seed, tid, shape.weight_std, "f32", st)
                self.tensors[name] = t
                return t
            synth.dev_normal(tmp.data_ptr(), n, shape.weight_seed, tid, shape.weight_std, "bf16", st)
            if keep_plain:
                self.tensors[name + "_plain"] = tmp[:n].clone()
            if pack:
                # a bank of `groups` matrices packed one after the other is the
                # packed form of the stacked [groups*rows][cols] matrix (rows % 16 == 0)
                t = torch.empty(n, dtype=torch.bfloat16, device=self.device)
                dg_pack_weight_bf16(t.data_ptr(), tmp.data_ptr(), groups * rows, cols, st)
                self.tensors[name] = t
                return t
            return None

        E = shape.n_experts
        # embedding: row-major for the gather, E^T in weight layout for self-conditioning
        if self.bf:
            n = shape.vocab * d
            synth.dev_normal(tmp.data_ptr(), n, shape.weight_seed, synth.TID["embed"], shape.weight_std, "bf16", st)
            emb = tmp[:n].clone()
            self.tensors["embed"] = emb
            if selfcond:
                et = torch.empty(n, dtype=torch.bfloat16, device=self.device)
                dg_pack_weight_bf16_transposed(et.data_ptr(), emb.data_ptr(), d, shape.vocab, st)
                self.tensors["embed_t"] = et
        else:
            fill("embed", synth.TID["embed"], shape.vocab, d)
            et = None
            if selfcond:
                et = torch.empty(shape.vocab * d, dtype=torch.float32, device=self.device)
                synth.dev_normal_f32_transposed(et.data_ptr(), shape.vocab, d, shape.weight_seed,
                                                synth.TID["embed"], shape.weight_std, st)
            self.tensors["embed_t"] = et
        # a tied head is drawn from the embedding's stream: the same matrix
        fill("lm_head", synth.TID["embed" if shape.tied_head else "lm_head"], shape.vocab, d,
             fp8=shape.lm_dtype == "fp8")
        fill("sc_up", synth.TID["sc_up"], shape.d_selfcond, d)
        fill("sc_down", synth.TID["sc_down"], d, shape.d_selfcond)
        self.layer_structs = (LayerWeights * shape.n_layers)()
        for l in range(shape.n_layers):
            lt = {}
            lt["wqkv"] = fill(f"L{l}.wqkv", synth.layer_tid(l, "wqkv"), shape.qkv_rows, d)
            lt["wo"] = fill(f"L{l}.wo", synth.layer_tid(l, "wo"), d, shape.q_dim)
            lt["wr"] = fill(f"L{l}.wr", synth.layer_tid(l, "wr"), E, d)
            x8, x4 = shape.expert_dtype == "fp8", shape.expert_dtype == "mxfp4"
            lt["sh_g"] = fill(f"L{l}.sh_g", synth.layer_tid(l, "sh_g"), shape.d_shared, d, fp8=x8, mx4=x4)
            lt["sh_u"] = fill(f"L{l}.sh_u", synth.layer_tid(l, "sh_u"), shape.d_shared, d, fp8=x8, mx4=x4)
            lt["sh_d"] = fill(f"L{l}.sh_d", synth.layer_tid(l, "sh_d"), d, shape.d_shared, fp8=x8, mx4=x4)
            lt["ex_g"] = fill(f"L{l}.ex_g", synth.layer_tid(l, "ex_g"), shape.d_expert, d, groups=E, fp8=x8, mx4=x4)
            lt["ex_u"] = fill(f"L{l}.ex_u", synth.layer_tid(l, "ex_u"), shape.d_expert, d, groups=E, fp8=x8, mx4=x4)
            lt["ex_d"] = fill(f"L{l}.ex_d", synth.layer_tid(l, "ex_d"), d, shape.d_expert, groups=E, fp8=x8, mx4=x4)
            ls = self.layer_structs[l]
            for k, v in lt.items():
                setattr(ls, k, v.data_ptr())
                if x8 and k in ("sh_g", "sh_u", "sh_d", "ex_g", "ex_u", "ex_d"):
                    setattr(ls, k + "_scale", self.tensors[f"L{l}.{k}_scale"].data_ptr())
        del tmp
        tn = self.tensors
        self.weights = Weights(tn["embed"].data_ptr(),
                               tn["embed_t"].data_ptr() if tn.get("embed_t") is not None else None,
                               tn["lm_head"].data_ptr(), tn["sc_up"].data_ptr(), tn["sc_down"].data_ptr(),
                               ctypes.cast(self.layer_structs, ctypes.POINTER(LayerWeights)), float(lm_scale),
                               tn["lm_head_scale"].data_ptr() if shape.lm_dtype == "fp8" else None)
        torch.cuda.synchronize()

    def set_lm_scale(self, s: float):
        self.weights.lm_scale = float(s)

    def bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors.values() if t is not None)


class DeviceCache:
    def __init__(self, shape: ModelShape, batch: int, capacity: int, device="cuda"):
        n = shape.n_layers * batch * shape.n_kv_heads * capacity * shape.d_head
        dt = _tdtype(shape)
        self.k = torch.zeros(n, dtype=dt, device=device)
        self.v = torch.zeros(n, dtype=dt, device=device)  # V^T, [d_head][row] per head
        self.shape = shape
        self.struct = KVCache(self.k.data_ptr(), self.v.data_ptr(), batch, capacity, 0)

    @property
    def length(self) -> int:
        return self.struct.length

    def view(self, which: str):
        """Logical [layer][batch][kv_head][row][d_head] view (V is stored
        transposed, [d_head][row] per head)."""
        s = self.shape
        if which == "k":
            return self.k.view(s.n_layers, self.struct.batch, s.n_kv_heads, self.struct.capacity, s.d_head)
        return self.v.view(s.n_layers, self.struct.batch, s.n_kv_heads, s.d_head,
                           self.struct.capacity).transpose(-1, -2)

    def valid_rows(self):
        """Copies of K and V rows [0, length) (what the denoiser must leave as is)."""
        L = self.struct.length
        return self.view("k")[:, :, :, :L].clone(), self.view("v")[:, :, :, :L].clone()

    def fill_random(self, length: int, seed: int = 0, std: float = 1.0):
        """N(0, std) fill of rows [0, length) (synthetic prefix, no encoder)."""
        s = self.shape
        st = stream_handle()
        for name, tid in (("k", synth.TID["kv_k"]), ("v", synth.TID["kv_v"])):
            view = self.view(name)
            tmp = torch.empty(s.n_layers * self.struct.batch * s.n_kv_heads * length * s.d_head,
                              dtype=self.k.dtype, device=view.device)
            synth.dev_normal(tmp.data_ptr(), tmp.numel(), seed, tid, std, s.dtype, st)
            view[:, :, :, :length].copy_(tmp.view(s.n_layers, self.struct.batch, s.n_kv_heads, length, s.d_head))
        self.struct.length = length


class DeviceCanvas:
    """Canvas tokens, sampler outputs and the self-conditioning state."""

    def __init__(self, shape: ModelShape, batch: int, canvas: int, seeds, device="cuda", selfcond=True):
        T = batch * canvas
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.batch, self.canvas = batch, canvas
        self.tokens = torch.zeros(T, **i32)
        self.seeds = torch.tensor(np.asarray(seeds, dtype=np.uint64).view(np.int64), dtype=torch.int64, device=dev)
        self.p_side = torch.zeros(T * shape.vocab, dtype=_tdtype(shape), device=dev) if selfcond else None
        self.p_scale = torch.zeros(T * (shape.vocab // 256), dtype=torch.float32, device=dev) if selfcond else None
        self.entropy = torch.zeros(T, dtype=torch.float32, device=dev)
        self.sample = torch.zeros(T, **i32)
        self.argmax = torch.zeros(T, **i32)
        self.prev_argmax = torch.full((T,), -1, **i32)
        self.accepted = torch.zeros(T, dtype=torch.uint8, device=dev)
        self.n_accepted = torch.zeros(batch, **i32)
        self.mean_entropy = torch.zeros(batch, dtype=torch.float32, device=dev)
        self.stop = torch.zeros(batch, **i32)
        self.flags = torch.zeros(batch, **i32)
        self.committed = torch.zeros(T, **i32)
        self.sc_probs = None
        self.struct = Canvas(batch, canvas, self.tokens.data_ptr(), self.seeds.data_ptr(), None,
                             self.p_side.data_ptr() if selfcond else None,
                             self.p_scale.data_ptr() if selfcond else None,
                             self.entropy.data_ptr(), self.sample.data_ptr(), self.argmax.data_ptr(),
                             self.prev_argmax.data_ptr(), self.accepted.data_ptr(), self.n_accepted.data_ptr(),
                             self.mean_entropy.data_ptr(), self.stop.data_ptr(), self.flags.data_ptr(),
                             self.committed.data_ptr())

    def set_sc_probs(self, probs: torch.Tensor | None):
        self.sc_probs = probs
        self.struct.sc_probs = probs.data_ptr() if probs is not None else None


class Workspace:
    def __init__(self, cfg: ModelConfig, batch: int, max_canvas: int, device="cuda"):
        self.nbytes = dg_workspace_bytes(cfg, batch, max_canvas)
        if self.nbytes == 0:
            raise ValueError("unsupported configuration")
        self.buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        base = self.buf.data_ptr()
        self.ptr = (base + 255) & ~255

    @property
    def size(self) -> int:
        return self.nbytes


def step_params(t: int, n_steps: int, block: int = 0, adaptive: bool = True) -> StepParams:
    return StepParams(t, n_steps, block, 1 if adaptive else 0, 0.1, 0.005)
