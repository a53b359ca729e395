"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module manufactures inputs only (weights, prompt tokens, KV-cache fills,
Dirichlet self-conditioning rows) and holds none of the decoding method's
arithmetic.  The definition of every generator is in ``gen.c``; ``gen_dev.hip``
is its device twin for model sizes the host cannot fill quickly.  A pure-numpy
restatement (``*_np``) exists for the small cases the tests use to pin the C
code.

Tensor ids (``TID``) name each logical weight of the model; logical layouts
are row-major ``[out][in]`` (``[E][out][in]`` for expert banks).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdgsynth.so")
_lib = None

# Tensor ids for the synthetic generator.
TID = {
    "embed": 1,
    "lm_head": 2,
    "sc_up": 3,
    "sc_down": 4,
    "kv_k": 5,
    "kv_v": 6,
    "dirichlet": 7,
    "prompt": 10,
}
LAYER_TID_BASE = 100
LAYER_TID_STRIDE = 16
LAYER_TENSORS = ("wqkv", "wo", "wr", "sh_g", "sh_u", "sh_d", "ex_g", "ex_u", "ex_d")


def layer_tid(layer: int, name: str) -> int:
    return LAYER_TID_BASE + LAYER_TID_STRIDE * layer + LAYER_TENSORS.index(name)


def build(force: bool = False) -> str:
    """Compile gen.c into libdgsynth.so (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", src, "-o", _LIB_PATH + ".tmp", "-lm"]
        )
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _get_lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, f32, i64 = ctypes.c_uint64, ctypes.c_float, ctypes.c_int64
        vp = ctypes.c_void_p
        lib.synth_scale_for_std.argtypes = [ctypes.c_double]
        lib.synth_scale_for_std.restype = f32
        lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, f32, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, f32, vp]
        lib.synth_normal_bf16_as_f64.argtypes = [u64, u64, u64, u64, f32, vp]
        lib.synth_tokens.argtypes = [u64, u64, u64, u64, ctypes.c_uint32, vp]
        lib.synth_dirichlet_rows.argtypes = [u64, u64, i64, i64, ctypes.c_double, vp]
        lib.synth_e4m3_rows.argtypes = [u64, u64, i64, i64, f32, vp, vp]
        lib.synth_mxfp4_quantize.argtypes = [vp, i64, i64, vp, vp]
        lib.synth_mxfp4_rows.argtypes = [u64, u64, i64, i64, f32, vp, vp]
        _lib = lib
    return _lib


def scale_for_std(std: float) -> np.float32:
    return np.float32(_get_lib().synth_scale_for_std(float(std)))


def normal(seed: int, tensor: int, shape, std: float, dtype: str = "bf16", start: int = 0):
    """N(0, std^2)-shaped values (Irwin-Hall of 4 uniforms).

    dtype "bf16" returns uint16 bit patterns, "f32" returns float32,
    "bf16_f64" the bf16 values widened to float64."""
    n = int(np.prod(shape))
    lib = _get_lib()
    sc = ctypes.c_float(scale_for_std(std))
    if dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.synth_normal_bf16(seed, tensor, start, n, sc, out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib.synth_normal_f32(seed, tensor, start, n, sc, out.ctypes.data)
    elif dtype == "bf16_f64":
        out = np.empty(n, dtype=np.float64)
        lib.synth_normal_bf16_as_f64(seed, tensor, start, n, sc, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def tokens(seed: int, tensor: int, n: int, vocab: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _get_lib().synth_tokens(seed, tensor, start, n, vocab, out.ctypes.data)
    return out


def dirichlet_rows(seed: int, tensor: int, rows: int, vocab: int, alpha: float) -> np.ndarray:
    out = np.empty((rows, vocab), dtype=np.float32)
    _get_lib().synth_dirichlet_rows(seed, tensor, rows, vocab, alpha, out.ctypes.data)
    return out


def e4m3_rows(seed: int, tensor: int, rows: int, cols: int, std: float):
    """fp8 form of the bf16 normal tensor [rows][cols]: per-row scale
    s_r = fp32(max|w_r| / 448) and OCP E4M3 codes of fp32(w / s_r) (round to
    nearest even).  Returns (codes uint8 [rows][cols], scales float32 [rows])."""
    codes = np.empty((rows, cols), dtype=np.uint8)
    sc = np.empty(rows, dtype=np.float32)
    _get_lib().synth_e4m3_rows(seed, tensor, rows, cols, ctypes.c_float(scale_for_std(std)), codes.ctypes.data,
                               sc.ctypes.data)
    return codes, sc


def mxfp4_quantize(w: np.ndarray):
    """MXFP4 form of the float32 values w [rows][cols] (cols % 32 == 0), by
    blocks of 32 consecutive values of a row: (element codes uint8
    [rows][cols], one E2M1 code per byte; E8M0 scale codes uint8
    [rows][cols / 32]).  The recipe is stated in gen.c."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    codes = np.empty((rows, cols), dtype=np.uint8)
    sc = np.empty((rows, cols // 32), dtype=np.uint8)
    _get_lib().synth_mxfp4_quantize(w.ctypes.data, rows, cols, codes.ctypes.data, sc.ctypes.data)
    return codes, sc


def mxfp4_rows(seed: int, tensor: int, rows: int, cols: int, std: float):
    """MXFP4 form of the bf16 normal tensor [rows][cols]: (codes uint8
    [rows][cols], scale codes uint8 [rows][cols / 32])."""
    codes = np.empty((rows, cols), dtype=np.uint8)
    sc = np.empty((rows, cols // 32), dtype=np.uint8)
    _get_lib().synth_mxfp4_rows(seed, tensor, rows, cols, ctypes.c_float(scale_for_std(std)), codes.ctypes.data,
                                sc.ctypes.data)
    return codes, sc


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (u16.astype(np.uint32) << 16).view(np.float32)


# ---- pure-numpy restatement of the same definitions (small sizes only) ----
_M64 = (1 << 64) - 1


def hash_np(seed: int, tensor: int, idx: np.ndarray) -> np.ndarray:
    idx = idx.astype(np.uint64)
    with np.errstate(over="ignore"):
        z = (np.uint64(seed & _M64) + np.uint64(0x9E3779B97F4A7C15) * (idx + np.uint64(1))
             + np.uint64((0xD1B54A32D192ED03 * (tensor + 1)) & _M64))
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def normal_np(seed: int, tensor: int, n: int, std: float, dtype: str = "bf16", start: int = 0):
    z = hash_np(seed, tensor, np.arange(start, start + n, dtype=np.uint64))
    m = np.uint64(0xFFFF)
    s = ((z & m).astype(np.int64) + ((z >> np.uint64(16)) & m).astype(np.int64)
         + ((z >> np.uint64(32)) & m).astype(np.int64) + (z >> np.uint64(48)).astype(np.int64) - 131070)
    scale = np.float32(std / np.sqrt((65536.0 * 65536.0 - 1.0) / 3.0))
    f = s.astype(np.float32) * scale
    if dtype == "f32":
        return f
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def tokens_np(seed: int, tensor: int, n: int, vocab: int, start: int = 0) -> np.ndarray:
    z = hash_np(seed, tensor, np.arange(start, start + n, dtype=np.uint64))
    hi = z >> np.uint64(32)
    with np.errstate(over="ignore"):
        return ((hi * np.uint64(vocab)) >> np.uint64(32)).astype(np.int32)


# ---- device twin (gen_dev.hip): fills device buffers in place ----
_DEV_LIB_PATH = os.path.join(_HERE, "libdgsynth_dev.so")
_dev_lib = None


def build_dev(arch: str = "gfx950") -> str:
    src = os.path.join(_HERE, "gen_dev.hip")
    subprocess.check_call(["/opt/rocm/bin/hipcc", f"--offload-arch={arch}", "-O3", "-fPIC", "-shared",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           src, "-o", _DEV_LIB_PATH + ".tmp"])
    os.replace(_DEV_LIB_PATH + ".tmp", _DEV_LIB_PATH)
    return _DEV_LIB_PATH


def _get_dev_lib():
    global _dev_lib
    if _dev_lib is None:
        if not os.path.exists(_DEV_LIB_PATH):
            raise ImportError(f"{_DEV_LIB_PATH} missing: run synth.build_dev()")
        lib = ctypes.CDLL(_DEV_LIB_PATH)
        u64, vp = ctypes.c_uint64, ctypes.c_void_p
        lib.synth_dev_normal_bf16.argtypes = [vp, u64, u64, u64, u64, ctypes.c_float, vp]
        lib.synth_dev_normal_f32.argtypes = [vp, u64, u64, u64, u64, ctypes.c_float, vp]
        lib.synth_dev_tokens.argtypes = [vp, u64, u64, u64, u64, ctypes.c_uint32, vp]
        lib.synth_dev_normal_f32_transposed.argtypes = [vp, u64, u64, u64, u64, ctypes.c_float, vp]
        lib.synth_dev_e4m3_rows.argtypes = [vp, vp, u64, u64, u64, u64, ctypes.c_float, vp]
        lib.synth_dev_mxfp4_rows.argtypes = [vp, vp, u64, u64, u64, u64, ctypes.c_float, vp]
        for f in (lib.synth_dev_normal_bf16, lib.synth_dev_normal_f32, lib.synth_dev_tokens,
                  lib.synth_dev_normal_f32_transposed, lib.synth_dev_e4m3_rows, lib.synth_dev_mxfp4_rows):
            f.restype = ctypes.c_int
        _dev_lib = lib
    return _dev_lib


def dev_normal(ptr: int, count: int, seed: int, tensor: int, std: float, dtype: str, stream: int,
               start: int = 0) -> None:
    """Fill `count` elements at device address `ptr` (bf16 bits or fp32)."""
    lib = _get_dev_lib()
    sc = ctypes.c_float(scale_for_std(std))
    f = lib.synth_dev_normal_bf16 if dtype == "bf16" else lib.synth_dev_normal_f32
    if f(ptr, seed, tensor, start, count, sc, stream) != 0:
        raise RuntimeError("synth device fill failed")


def dev_tokens(ptr: int, count: int, seed: int, tensor: int, vocab: int, stream: int, start: int = 0) -> None:
    if _get_dev_lib().synth_dev_tokens(ptr, seed, tensor, start, count, vocab, stream) != 0:
        raise RuntimeError("synth device tokens failed")


def dev_normal_f32_transposed(ptr: int, rows: int, cols: int, seed: int, tensor: int, std: float,
                              stream: int) -> None:
    """fp32 fill of the transpose of the logical [rows][cols] tensor `tensor`."""
    sc = ctypes.c_float(scale_for_std(std))
    if _get_dev_lib().synth_dev_normal_f32_transposed(ptr, seed, tensor, rows, cols, sc, stream) != 0:
        raise RuntimeError("synth device fill failed")


def dev_e4m3_rows(codes_ptr: int, scale_ptr: int, rows: int, cols: int, seed: int, tensor: int, std: float,
                  stream: int) -> None:
    """Device twin of e4m3_rows: codes [rows][cols] (uint8) and scales [rows] (fp32)."""
    sc = ctypes.c_float(scale_for_std(std))
    if _get_dev_lib().synth_dev_e4m3_rows(codes_ptr, scale_ptr, seed, tensor, rows, cols, sc, stream) != 0:
        raise RuntimeError("synth device fp8 fill failed")


def dev_mxfp4_rows(codes_ptr: int, scale_ptr: int, rows: int, cols: int, seed: int, tensor: int, std: float,
                   stream: int) -> None:
    """Device twin of mxfp4_rows: codes [rows][cols] (uint8, one E2M1 code
    each) and scale codes [rows][cols / 32] (uint8, E8M0)."""
    sc = ctypes.c_float(scale_for_std(std))
    if _get_dev_lib().synth_dev_mxfp4_rows(codes_ptr, scale_ptr, seed, tensor, rows, cols, sc, stream) != 0:
        raise RuntimeError("synth device mxfp4 fill failed")
