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

}  // extern "C"
