// Shared device helpers for the gfx950 kernels of the denoising step:
// storage types, bf16 rounding, the sampler's Philox4x32-10, wave reductions
// and the MFMA operand types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define DG_WAVE 64

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Eight OCP E4M3 codes (bytes of w, lowest first) -> eight bf16, exactly
// (every E4M3 value is a bf16 value; the conversion's scale is 1).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint2 w) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight MXFP4 elements (the E2M1 codes in the nibbles of q, lowest first)
// times their block scale 2^(code - 127), as eight bf16: exact for scale
// codes 1..254 (every such product is a bf16 value); code 0 gives zeros.
__device__ __forceinline__ bf16x8_t mx4x8_to_bf16(uint32_t q, uint32_t scale_code) {
  const float sc = __uint_as_float(scale_code << 23);
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 0);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 1);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 2);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 3);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ float bf2f(bf16_t u) { return __uint_as_float((uint32_t)u << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Activation storage: bf16 models keep GEMM inputs in bf16, fp32 models in fp32.
template <typename T> __device__ __forceinline__ float ld_act(const T* p);
template <> __device__ __forceinline__ float ld_act<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_act<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <typename T> __device__ __forceinline__ T to_act(float f);
template <> __device__ __forceinline__ float to_act<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t to_act<bf16_t>(float f) { return f2bf(f); }

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// two-multiply S-box with a Weyl key schedule.  Sampler counter layout:
// (position, step, block, stream); key = the canvas seed's two 32-bit halves.
struct dg_u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ dg_u32x4 dg_philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                             uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo_a = 0xD2511F53u * c0, hi_a = __umulhi(0xD2511F53u, c0);
    const uint32_t lo_b = 0xCD9E8D57u * c2, hi_b = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi_b ^ c1 ^ k0, n2 = hi_a ^ c3 ^ k1;
    c0 = n0; c1 = lo_b; c2 = n2; c3 = lo_a;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

enum { DG_STREAM_INIT = 0, DG_STREAM_RENOISE = 1, DG_STREAM_SAMPLE = 2 };

// word -> token in [0, V): multiply-shift (exact w >> (32-b) for V = 2^b).
__device__ __forceinline__ int32_t dg_word_token(uint32_t w, uint32_t vocab) {
  return (int32_t)(((uint64_t)w * (uint64_t)vocab) >> 32);
}
// word -> 24-bit uniform in [0, 1)
__device__ __forceinline__ float dg_word_unit(uint32_t w) { return (float)(w >> 8) * 5.9604644775390625e-8f; }

// ---------------------------------------------------------------------------
// Wave-level reductions (64 lanes) via DPP-free shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wave (Hillis-Steele).
__device__ __forceinline__ float wave_incl_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    float t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ float gelu_tanh(float x) {
  const float k0 = 0.7978845608028654f, k1 = 0.044715f;
  return 0.5f * x * (1.0f + tanhf(k0 * (x + k1 * x * x * x)));
}

// Bounds of a launch checked on the host; kernels also guard their indexes.
#define DG_CEIL_DIV(a, b) (((a) + (b) - 1) / (b))
