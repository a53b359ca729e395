"""Python binding of libdg.so — the gfx950 block-diffusion denoising step.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/dg.h``.  Functions keep the C names and
raise ``DGError`` on a non-zero status.  Importing this package fails loudly
if the HIP library has not been built (``python -m
discrete_text_diffusion_amd.build`` or ``__graft_entry__.build()``): there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -m discrete_text_diffusion_amd.build); there is no CPU fallback")

_lib = ctypes.CDLL(LIB_PATH)

DG_OK = 0
DG_ERR_INVALID_ARG = -1
DG_ERR_UNSUPPORTED = -2
DG_ERR_KV_CAPACITY = -3
DG_ERR_WORKSPACE = -4
DG_ERR_HIP = -5
DG_ERR_SCRATCH_LIMIT = -6
DG_NOALLOC_SCRATCH_BYTES = 320 << 20
DG_DTYPE_F32 = 0
DG_DTYPE_BF16 = 1
DG_DTYPE_FP8_E4M3 = 2
DG_DTYPE_MXFP4 = 3
DG_FLAG_NONFINITE = 1
DG_ENTROPY_BOUND = 0.1
DG_STOP_THRESHOLD = 0.005


class DGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dg_status_string(status)} ({status})")


class ModelConfig(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("d_head", c_int32), ("n_experts", c_int32), ("top_k", c_int32), ("d_expert", c_int32),
                ("d_shared", c_int32), ("vocab", c_int32), ("d_selfcond", c_int32), ("dtype", c_int32),
                ("rope_base", c_float), ("norm_eps", c_float), ("expert_dtype", c_int32), ("lm_dtype", c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("wqkv", "wo", "wr", "sh_g", "sh_u", "sh_d", "ex_g", "ex_u", "ex_d",
                                        "ex_g_scale", "ex_u_scale", "ex_d_scale", "sh_g_scale", "sh_u_scale",
                                        "sh_d_scale")]


class Weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("embed_t", c_void_p), ("lm_head", c_void_p), ("sc_up", c_void_p),
                ("sc_down", c_void_p), ("layers", POINTER(LayerWeights)), ("lm_scale", c_float),
                ("lm_head_scale", c_void_p)]


class KVCache(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("batch", c_int32), ("capacity", c_int32), ("length", c_int32)]


class Canvas(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("canvas", c_int32), ("tokens", c_void_p), ("seeds", c_void_p),
                ("sc_probs", c_void_p), ("p_side", c_void_p), ("p_scale", c_void_p), ("entropy", c_void_p),
                ("sample", c_void_p), ("argmax", c_void_p), ("prev_argmax", c_void_p), ("accepted", c_void_p),
                ("n_accepted", c_void_p), ("mean_entropy", c_void_p), ("stop", c_void_p), ("flags", c_void_p),
                ("committed", c_void_p)]


class Trace(ctypes.Structure):
    _fields_ = [("events", POINTER(c_void_p)), ("phase", POINTER(c_int32)), ("capacity", c_int32),
                ("count", c_int32), ("mask", c_uint32)]


PHASES = ("selfcond", "embed", "qkv", "attn", "oproj", "route", "moe_up", "moe_down", "combine", "lmhead",
          "sampler")


class StepParams(ctypes.Structure):
    _fields_ = [("t", c_int32), ("n_steps", c_int32), ("block", c_int32), ("adaptive", c_int32),
                ("entropy_bound", c_float), ("stop_threshold", c_float)]


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_P = POINTER
_temperature = _sig("dg_temperature", c_float, c_int32, c_int32)
_ws_bytes = _sig("dg_workspace_bytes", c_size_t, _P(ModelConfig), c_int32, c_int32)
_pack = _sig("dg_pack_weight_bf16", c_int32, c_void_p, c_void_p, c_int64, c_int64, c_void_p)
_pack_t = _sig("dg_pack_weight_bf16_transposed", c_int32, c_void_p, c_void_p, c_int64, c_int64, c_void_p)
_pack8 = _sig("dg_pack_weight_fp8", c_int32, c_void_p, c_void_p, c_int64, c_int64, c_void_p)
_pack4 = _sig("dg_pack_weight_mxfp4", c_int32, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p)
_init_canvas = _sig("dg_init_canvas", c_int32, _P(ModelConfig), _P(Canvas), c_int32, c_void_p)
_encode = _sig("dg_encode_append", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), c_void_p, c_int32, c_int32,
               c_void_p, c_size_t, c_void_p)
_denoise = _sig("dg_denoise_step", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), _P(Canvas), _P(StepParams),
                c_void_p, c_size_t, c_void_p)
_commit = _sig("dg_commit_block", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), _P(Canvas), _P(StepParams),
               c_void_p, c_size_t, c_void_p)
_commit_step = _sig("dg_commit_and_step", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), _P(Canvas),
                    _P(StepParams), _P(StepParams), c_void_p, c_size_t, c_void_p)
_ar = _sig("dg_ar_step", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), c_void_p, c_int32, c_void_p, c_void_p,
           c_size_t, c_void_p)
_denoise_tr = _sig("dg_denoise_step_traced", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), _P(Canvas),
                   _P(StepParams), c_void_p, c_size_t, c_void_p, _P(Trace))
_encode_tr = _sig("dg_encode_append_traced", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), c_void_p, c_int32,
                  c_int32, c_void_p, c_size_t, c_void_p, _P(Trace))
_status = _sig("dg_status_string", ctypes.c_char_p, c_int32)
_t_sample = _sig("dg_test_sample_from_logits", c_int32, _P(ModelConfig), c_void_p, _P(Canvas), _P(StepParams),
                 c_void_p, c_size_t, c_void_p)
_t_route = _sig("dg_test_route_from_logits", c_int32, _P(ModelConfig), c_void_p, c_int32, c_void_p, c_void_p,
                c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p)
_t_logits = _sig("dg_test_forward_logits", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), _P(Canvas),
                 _P(StepParams), c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p)

_noalloc = _sig("dg_denoise_step_noalloc", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), _P(Canvas),
                _P(StepParams), c_void_p)
_t_step = _sig("dg_test_denoise_step", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), _P(Canvas),
               _P(StepParams), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p)
_t_encode = _sig("dg_test_encode_append", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), c_void_p, c_int32,
                 c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p)
_t_ar = _sig("dg_test_ar_step", c_int32, _P(ModelConfig), _P(Weights), _P(KVCache), c_void_p, c_int32, c_void_p,
             c_void_p, c_void_p, c_size_t, c_void_p)

EXPORTED = ("dg_temperature", "dg_workspace_bytes", "dg_pack_weight_bf16", "dg_pack_weight_bf16_transposed",
            "dg_pack_weight_fp8", "dg_pack_weight_mxfp4",
            "dg_init_canvas", "dg_encode_append", "dg_denoise_step", "dg_commit_block", "dg_status_string",
            "dg_test_sample_from_logits", "dg_test_route_from_logits", "dg_test_forward_logits",
            "dg_denoise_step_traced", "dg_encode_append_traced", "dg_test_encode_append", "dg_ar_step", "dg_commit_and_step",
            "dg_test_ar_step", "dg_test_denoise_step", "dg_denoise_step_noalloc")


def _check(rc: int, where: str):
    if rc != DG_OK:
        raise DGError(rc, where)


def dg_status_string(status: int) -> str:
    return _status(status).decode()


def dg_temperature(t: int, n_steps: int) -> float:
    return float(_temperature(t, n_steps))


def dg_workspace_bytes(cfg: ModelConfig, batch: int, max_canvas: int) -> int:
    return int(_ws_bytes(ctypes.byref(cfg), batch, max_canvas))


def dg_pack_weight_bf16(dst, src, rows: int, cols: int, stream) -> None:
    _check(_pack(dst, src, rows, cols, stream), "dg_pack_weight_bf16")


def dg_pack_weight_bf16_transposed(dst, src, rows: int, cols: int, stream) -> None:
    _check(_pack_t(dst, src, rows, cols, stream), "dg_pack_weight_bf16_transposed")


def dg_pack_weight_fp8(dst, src, rows: int, cols: int, stream) -> None:
    _check(_pack8(dst, src, rows, cols, stream), "dg_pack_weight_fp8")


def dg_pack_weight_mxfp4(dst, codes, scales, rows: int, cols: int, stream) -> None:
    _check(_pack4(dst, codes, scales, rows, cols, stream), "dg_pack_weight_mxfp4")


def dg_init_canvas(cfg, canvas, block: int, stream) -> None:
    _check(_init_canvas(ctypes.byref(cfg), ctypes.byref(canvas), block, stream), "dg_init_canvas")


def dg_encode_append(cfg, weights, cache, d_tokens, batch: int, n_tokens: int, ws, ws_bytes: int, stream) -> None:
    _check(_encode(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), d_tokens, batch, n_tokens, ws,
                   ws_bytes, stream), "dg_encode_append")


def dg_denoise_step(cfg, weights, cache, canvas, params, ws, ws_bytes: int, stream) -> None:
    _check(_denoise(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(canvas),
                    ctypes.byref(params), ws, ws_bytes, stream), "dg_denoise_step")


def dg_denoise_step_noalloc(cfg, weights, cache, canvas, params, stream) -> None:
    _check(_noalloc(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(canvas),
                    ctypes.byref(params), stream), "dg_denoise_step_noalloc")


def dg_commit_block(cfg, weights, cache, canvas, params, ws, ws_bytes: int, stream) -> None:
    _check(_commit(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(canvas),
                   ctypes.byref(params), ws, ws_bytes, stream), "dg_commit_block")


def dg_commit_and_step(cfg, weights, cache, canvas, p_commit, p_next, ws, ws_bytes: int, stream) -> None:
    _check(_commit_step(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(canvas),
                        ctypes.byref(p_commit), ctypes.byref(p_next), ws, ws_bytes, stream), "dg_commit_and_step")


def dg_ar_step(cfg, weights, cache, d_tokens, batch: int, d_next, ws, ws_bytes: int, stream) -> None:
    _check(_ar(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), d_tokens, batch, d_next, ws, ws_bytes,
               stream), "dg_ar_step")


def dg_test_ar_step(cfg, weights, cache, d_tokens, batch: int, d_next, d_logits, ws, ws_bytes: int, stream) -> None:
    _check(_t_ar(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), d_tokens, batch, d_next, d_logits, ws,
                 ws_bytes, stream), "dg_test_ar_step")


def dg_test_sample_from_logits(cfg, d_logits, canvas, params, ws, ws_bytes: int, stream) -> None:
    _check(_t_sample(ctypes.byref(cfg), d_logits, ctypes.byref(canvas), ctypes.byref(params), ws, ws_bytes, stream),
           "dg_test_sample_from_logits")


def dg_test_route_from_logits(cfg, d_logits, T: int, ids, w, row_token, inv, offsets, ws, ws_bytes: int,
                              stream) -> None:
    _check(_t_route(ctypes.byref(cfg), d_logits, T, ids, w, row_token, inv, offsets, ws, ws_bytes, stream),
           "dg_test_route_from_logits")


def dg_test_forward_logits(cfg, weights, cache, canvas, params, d_force_ids, d_router_logits, d_logits, ws,
                           ws_bytes: int, stream) -> None:
    _check(_t_logits(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(canvas),
                     ctypes.byref(params), d_force_ids, d_router_logits, d_logits, ws, ws_bytes, stream),
           "dg_test_forward_logits")


def dg_test_denoise_step(cfg, weights, cache, canvas, params, d_force_ids, d_router_logits, d_logits, ws,
                         ws_bytes: int, stream, d_teacher_x=None, d_layer_out=None) -> None:
    _check(_t_step(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(canvas),
                   ctypes.byref(params), d_force_ids, d_router_logits, d_logits, d_teacher_x, d_layer_out, ws,
                   ws_bytes, stream), "dg_test_denoise_step")


def dg_denoise_step_traced(cfg, weights, cache, canvas, params, ws, ws_bytes: int, stream, trace) -> None:
    _check(_denoise_tr(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(canvas),
                       ctypes.byref(params), ws, ws_bytes, stream, ctypes.byref(trace) if trace is not None else None),
           "dg_denoise_step_traced")


def dg_encode_append_traced(cfg, weights, cache, d_tokens, batch: int, n_tokens: int, ws, ws_bytes: int, stream,
                            trace) -> None:
    _check(_encode_tr(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), d_tokens, batch, n_tokens, ws,
                      ws_bytes, stream, ctypes.byref(trace) if trace is not None else None),
           "dg_encode_append_traced")


def dg_test_encode_append(cfg, weights, cache, d_tokens, batch: int, n_tokens: int, d_force_ids, d_router_logits, ws,
                          ws_bytes: int, stream) -> None:
    _check(_t_encode(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), d_tokens, batch, n_tokens,
                     d_force_ids, d_router_logits, ws, ws_bytes, stream), "dg_test_encode_append")
