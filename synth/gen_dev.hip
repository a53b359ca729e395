// Device twin of gen.c: the same seeded definitions, evaluated on the GPU so
// large synthetic models (tens of GB) can be filled in place.  Integer
// arithmetic plus one fp32 multiply, so values equal gen.c bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t synth_hash(uint64_t seed, uint64_t tensor, uint64_t i) {
  uint64_t z = seed + 0x9E3779B97F4A7C15ull * (i + 1) + 0xD1B54A32D192ED03ull * (tensor + 1);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float synth_normal_value(uint64_t z, float scale) {
  const int32_t s = (int32_t)(z & 0xFFFF) + (int32_t)((z >> 16) & 0xFFFF) + (int32_t)((z >> 32) & 0xFFFF) +
                    (int32_t)(z >> 48) - 131070;
  return __fmul_rn((float)s, scale);
}

__global__ void k_normal_bf16(uint16_t* out, uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, float scale) {
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += (uint64_t)gridDim.x * blockDim.x) {
    uint32_t u = __float_as_uint(synth_normal_value(synth_hash(seed, tensor, start + j), scale));
    u += 0x7FFFu + ((u >> 16) & 1u);
    out[j] = (uint16_t)(u >> 16);
  }
}

__global__ void k_normal_f32(float* out, uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, float scale) {
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += (uint64_t)gridDim.x * blockDim.x)
    out[j] = synth_normal_value(synth_hash(seed, tensor, start + j), scale);
}

__global__ void k_tokens(int32_t* out, uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, uint32_t vocab) {
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t hi = synth_hash(seed, tensor, start + j) >> 32;
    out[j] = (int32_t)((hi * (uint64_t)vocab) >> 32);
  }
}

// Transposed fill of a logical [rows][cols] matrix: out[c*rows + r] = value(r*cols + c).
__global__ void k_normal_f32_t(float* out, uint64_t seed, uint64_t tensor, uint64_t rows, uint64_t cols, float scale) {
  const uint64_t count = rows * cols;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t c = j / rows, r = j - c * rows;
    out[j] = synth_normal_value(synth_hash(seed, tensor, r * cols + c), scale);
  }
}

__device__ __forceinline__ float synth_bf16_value(uint64_t seed, uint64_t tensor, uint64_t i, float scale) {
  uint32_t u = __float_as_uint(synth_normal_value(synth_hash(seed, tensor, i), scale));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xFFFF0000u);
}

// OCP E4M3 code of x, round to nearest even (|x| >= 464 saturates to 448).
__device__ __forceinline__ uint8_t synth_e4m3_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E80000u) return sign | 0x7Eu;
  if (a < 0x3C800000u) return sign | (uint8_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  return sign | (uint8_t)((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

// One workgroup per row: row maximum of |w|, then the codes.
__global__ __launch_bounds__(256) void k_e4m3_rows(uint8_t* codes, float* row_scale, uint64_t seed, uint64_t tensor,
                                                   uint64_t cols, float scale) {
  __shared__ float red[4];
  const uint64_t r = blockIdx.x;
  float mx = 0.0f;
  for (uint64_t c = threadIdx.x; c < cols; c += 256)
    mx = fmaxf(mx, fabsf(synth_bf16_value(seed, tensor, r * cols + c, scale)));
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = mx > 0.0f ? __fdiv_rn(mx, 448.0f) : 1.0f;
  if (threadIdx.x == 0) row_scale[r] = s;
  for (uint64_t c = threadIdx.x; c < cols; c += 256)
    codes[r * cols + c] = synth_e4m3_rne(__fdiv_rn(synth_bf16_value(seed, tensor, r * cols + c, scale), s));
}

// E2M1 code of x (finite), round to nearest even on {0, 0.5, 1, 1.5, 2, 3, 4, 6}
// (the host file's definition).
__device__ __forceinline__ uint8_t synth_e2m1_rne(float x) {
  const uint8_t sign = (__float_as_uint(x) >> 31) ? 8u : 0u;
  const float a = fabsf(x);
  uint8_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return sign | c;
}

// One thread per block of 32 values of a row: shared exponent, then the codes.
__global__ __launch_bounds__(256) void k_mxfp4_rows(uint8_t* codes, uint8_t* scales, uint64_t seed, uint64_t tensor,
                                                    uint64_t rows, uint64_t cols, float scale) {
  const uint64_t nb = cols / 32;
  for (uint64_t q = (uint64_t)blockIdx.x * 256 + threadIdx.x; q < rows * nb; q += (uint64_t)gridDim.x * 256) {
    const uint64_t r = q / nb, b = q - r * nb;
    const uint64_t i0 = r * cols + b * 32;
    float mx = 0.0f;
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(synth_bf16_value(seed, tensor, i0 + i, scale)));
    if (mx == 0.0f) {
      scales[q] = 0;
      for (int i = 0; i < 32; ++i) codes[i0 + i] = 0;
      continue;
    }
    int e2;
    frexpf(mx, &e2);
    const int E = min(127, max(-127, e2 - 1 - 2));
    scales[q] = (uint8_t)(E + 127);
    for (int i = 0; i < 32; ++i) codes[i0 + i] = synth_e2m1_rne(ldexpf(synth_bf16_value(seed, tensor, i0 + i, scale), -E));
  }
}

dim3 grid_for(uint64_t count) {
  uint64_t b = (count + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return dim3((unsigned)b);
}

}  // namespace

extern "C" {

int synth_dev_normal_bf16(void* out, uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, float scale,
                          void* stream) {
  hipLaunchKernelGGL(k_normal_bf16, grid_for(count), dim3(256), 0, (hipStream_t)stream, (uint16_t*)out, seed, tensor,
                     start, count, scale);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int synth_dev_normal_f32(void* out, uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, float scale,
                         void* stream) {
  hipLaunchKernelGGL(k_normal_f32, grid_for(count), dim3(256), 0, (hipStream_t)stream, (float*)out, seed, tensor, start,
                     count, scale);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int synth_dev_normal_f32_transposed(void* out, uint64_t seed, uint64_t tensor, uint64_t rows, uint64_t cols,
                                    float scale, void* stream) {
  hipLaunchKernelGGL(k_normal_f32_t, grid_for(rows * cols), dim3(256), 0, (hipStream_t)stream, (float*)out, seed,
                     tensor, rows, cols, scale);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int synth_dev_tokens(void* out, uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, uint32_t vocab,
                     void* stream) {
  hipLaunchKernelGGL(k_tokens, grid_for(count), dim3(256), 0, (hipStream_t)stream, (int32_t*)out, seed, tensor, start,
                     count, vocab);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int synth_dev_e4m3_rows(void* codes, void* row_scale, uint64_t seed, uint64_t tensor, uint64_t rows, uint64_t cols,
                        float scale, void* stream) {
  if (rows == 0 || rows > 0x7FFFFFFFull) return -1;
  hipLaunchKernelGGL(k_e4m3_rows, dim3((unsigned)rows), dim3(256), 0, (hipStream_t)stream, (uint8_t*)codes,
                     (float*)row_scale, seed, tensor, cols, scale);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int synth_dev_mxfp4_rows(void* codes, void* scales, uint64_t seed, uint64_t tensor, uint64_t rows, uint64_t cols,
                         float scale, void* stream) {
  if (rows == 0 || cols % 32) return -1;
  hipLaunchKernelGGL(k_mxfp4_rows, grid_for(rows * (cols / 32)), dim3(256), 0, (hipStream_t)stream, (uint8_t*)codes,
                     (uint8_t*)scales, seed, tensor, rows, cols, scale);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
