// Row-wise kernels of the denoising step: token embedding (+ self-conditioning
// term), RMSNorm (gain 1) fused with residual updates, the fixed-order MoE
// combine, split-K reductions and the initial canvas noise.
#include "dg_internal.h"

namespace {

// Deterministic block sum (256 threads): butterfly inside waves, then the 4
// wave sums in wave order.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

template <typename TA>
__device__ __forceinline__ void write_norm(const float* x, TA* n, int d, float eps, float* red) {
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) ss = fmaf(x[i], x[i], ss);
  const float tot = block_sum256(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += 256) n[i] = to_act<TA>(x[i] * inv);
}

// x[t] = E[tok[t]] (+ sum_s add[s][t], split order); n[t] = RMSNorm(x[t]).
template <typename TA>
__global__ __launch_bounds__(256) void k_embed_norm(const int32_t* tok, const TA* emb, const float* add, int n_add,
                                                   int64_t add_stride, float* x, TA* n, int d, float eps) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const TA* e = emb + (int64_t)tok[t] * d;
  float* xr = x + t * d;
  constexpr int kMaxS = 16;
  for (int i = threadIdx.x; i < d; i += 256) {
    float v = ld_act<TA>(e + i);
    if (n_add > 0) {
      float p[kMaxS];
#pragma unroll
      for (int s = 0; s < kMaxS; ++s) p[s] = s < n_add ? add[(int64_t)s * add_stride + t * d + i] : 0.f;
      float acc = p[0];
#pragma unroll
      for (int s = 1; s < kMaxS; ++s) acc += p[s];
      v += acc;
    }
    xr[i] = v;
  }
  __syncthreads();
  write_norm<TA>(xr, n + t * d, d, eps, red);
}

// x[t] = src[t]; n[t] = RMSNorm(x[t])  (a residual given from outside: the
// teacher-forced test path).
template <typename TA>
__global__ __launch_bounds__(256) void k_set_norm(const float* src, float* x, TA* n, int d, float eps) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  float* xr = x + t * d;
  for (int i = threadIdx.x; i < d; i += 256) xr[i] = src[t * d + i];
  __syncthreads();
  write_norm<TA>(xr, n + t * d, d, eps, red);
}

// x[t] += sum_s part[s][t] (split order); n[t] = RMSNorm(x[t]).
template <typename TA>
__global__ __launch_bounds__(256) void k_resid_norm(float* x, const float* part, int n_split, int64_t split_stride,
                                                   TA* n, int d, float eps) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  float* xr = x + t * d;
  constexpr int kMaxS = 16;
  for (int i = threadIdx.x; i < d; i += 256) {
    float v[kMaxS];
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) v[s] = s < n_split ? part[(int64_t)s * split_stride + t * d + i] : 0.f;
    float acc = v[0];
#pragma unroll
    for (int s = 1; s < kMaxS; ++s) acc += v[s];
    xr[i] += acc;
  }
  __syncthreads();
  write_norm<TA>(xr, n + t * d, d, eps, red);
}

// y_t = sum_c Y[T*k + c*T + t] (shared-expert slices) + sum_j w[t][j] Y[inv[t*k+j]]
// in rank order; x[t] += y_t; n[t] = RMSNorm(x[t]).
template <typename TA>
__global__ __launch_bounds__(256) void k_combine_norm(float* x, const float* Y, const int32_t* inv, const float* w,
                                                     int T, int k, int n_sh, TA* n, int d, float eps) {
  __shared__ float red[4];
  __shared__ int32_t rows[16];
  __shared__ float wts[16];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = inv[t * k + threadIdx.x];
    wts[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  float* xr = x + t * d;
  const int64_t sh0 = (int64_t)T * k;
  if ((d & 3) == 0) {
    for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
      float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int c = 0; c < n_sh; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(Y + (sh0 + (int64_t)c * T + t) * d + i);
        y.x += v.x; y.y += v.y; y.z += v.z; y.w += v.w;
      }
      for (int j = 0; j < k; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(Y + (int64_t)rows[j] * d + i);
        const float wj = wts[j];
        y.x = fmaf(wj, v.x, y.x); y.y = fmaf(wj, v.y, y.y); y.z = fmaf(wj, v.z, y.z); y.w = fmaf(wj, v.w, y.w);
      }
      float4 xv = *reinterpret_cast<float4*>(xr + i);
      xv.x += y.x; xv.y += y.y; xv.z += y.z; xv.w += y.w;
      *reinterpret_cast<float4*>(xr + i) = xv;
    }
  } else {
    for (int i = threadIdx.x; i < d; i += 256) {
      float y = 0.f;
      for (int c = 0; c < n_sh; ++c) y += Y[(sh0 + (int64_t)c * T + t) * d + i];
      for (int j = 0; j < k; ++j) y = fmaf(wts[j], Y[(int64_t)rows[j] * d + i], y);
      xr[i] += y;
    }
  }
  __syncthreads();
  write_norm<TA>(xr, n + t * d, d, eps, red);
}

// Wide forms for d % 4 == 0 and d <= 4096: 1024 threads per row, one float4
// of the row per thread held in registers from the residual update to the
// norm, every load of a thread issued before the first add.
__device__ __forceinline__ float block_sum1024(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) t += red[w];
  return t;
}

template <typename TA>
__device__ __forceinline__ void write_norm4(float* xr, TA* nr, int i, bool on, float4 v, float eps, int d,
                                            float* red) {
  const float ss = on ? ((v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w)) : 0.f;
  const float tot = block_sum1024(ss, red);
  if (!on) return;
  *reinterpret_cast<float4*>(xr + i) = v;
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  if constexpr (sizeof(TA) == 2) {
    const uint32_t lo = (uint32_t)f2bf(v.x * inv) | ((uint32_t)f2bf(v.y * inv) << 16);
    const uint32_t hi = (uint32_t)f2bf(v.z * inv) | ((uint32_t)f2bf(v.w * inv) << 16);
    *reinterpret_cast<uint2*>(nr + i) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(nr + i) = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
  }
}

template <typename TA>
__global__ __launch_bounds__(1024) void k_resid_norm4(float* x, const float* part, int n_split, int64_t split_stride,
                                                     TA* n, int d, float eps) {
  __shared__ float red[16];
  const int64_t t = blockIdx.x;
  const int i = threadIdx.x * 4;
  const bool on = i < d;
  float* xr = x + t * d;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (on) {
    constexpr int kMaxS = 16;
    float4 p[kMaxS];
#pragma unroll
    for (int s = 0; s < kMaxS; ++s)
      p[s] = s < n_split ? *reinterpret_cast<const float4*>(part + (int64_t)s * split_stride + t * d + i)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 acc = p[0];
#pragma unroll
    for (int s = 1; s < kMaxS; ++s) {
      acc.x += p[s].x; acc.y += p[s].y; acc.z += p[s].z; acc.w += p[s].w;
    }
    v = *reinterpret_cast<const float4*>(xr + i);
    v.x += acc.x; v.y += acc.y; v.z += acc.z; v.w += acc.w;
  }
  write_norm4<TA>(xr, n + t * d, i, on, v, eps, d, red);
}

template <typename TA>
__global__ __launch_bounds__(1024) void k_combine_norm4(float* x, const float* Y, const int32_t* inv, const float* w,
                                                       int T, int k, int n_sh, TA* n, int d, float eps) {
  __shared__ float red[16];
  const int64_t t = blockIdx.x;
  const int i = threadIdx.x * 4;
  const bool on = i < d;
  float* xr = x + t * d;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (on) {
    constexpr int kMaxK = 16, kMaxSh = 8;
    const int64_t sh0 = (int64_t)T * k;
    float4 ys[kMaxSh], yr[kMaxK];
    float wj[kMaxK];
#pragma unroll
    for (int c = 0; c < kMaxSh; ++c)
      ys[c] = c < n_sh ? *reinterpret_cast<const float4*>(Y + (sh0 + (int64_t)c * T + t) * d + i)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      wj[j] = j < k ? w[t * k + j] : 0.f;
      yr[j] = j < k ? *reinterpret_cast<const float4*>(Y + (int64_t)inv[t * k + j] * d + i)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // shared-expert slices in slice order, then the routed outputs in rank order
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int c = 0; c < kMaxSh; ++c)
      if (c < n_sh) { y.x += ys[c].x; y.y += ys[c].y; y.z += ys[c].z; y.w += ys[c].w; }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) {
        y.x = fmaf(wj[j], yr[j].x, y.x); y.y = fmaf(wj[j], yr[j].y, y.y);
        y.z = fmaf(wj[j], yr[j].z, y.z); y.w = fmaf(wj[j], yr[j].w, y.w);
      }
    v = *reinterpret_cast<const float4*>(xr + i);
    v.x += y.x; v.y += y.y; v.z += y.z; v.w += y.w;
  }
  write_norm4<TA>(xr, n + t * d, i, on, v, eps, d, red);
}

// out[t][i] = act(sum_s part[s][t][i]) (split order).
template <typename TA>
__global__ __launch_bounds__(256) void k_reduce_splits(const float* part, int n_split, int64_t split_stride,
                                                      int64_t n_elems, TA* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_elems) return;
  constexpr int kMaxS = 32;
  float v[kMaxS];
#pragma unroll
  for (int s = 0; s < kMaxS; ++s) v[s] = s < n_split ? part[(int64_t)s * split_stride + i] : 0.f;
  float acc = v[0];
#pragma unroll
  for (int s = 1; s < kMaxS; ++s) acc += v[s];
  out[i] = to_act<TA>(acc);
}

// tokens[b][i] = uniform token from Philox stream 0 (step field 0) of canvas b.
__global__ __launch_bounds__(256) void k_init_canvas(int32_t* tokens, const uint64_t* seeds, int B, int C, int block,
                                                    uint32_t vocab) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= B * C) return;
  const int b = i / C, pos = i - b * C;
  const uint64_t sd = seeds[b];
  const dg_u32x4 w = dg_philox((uint32_t)pos, 0u, (uint32_t)block, DG_STREAM_INIT, (uint32_t)sd, (uint32_t)(sd >> 32));
  tokens[i] = dg_word_token(w.x, vocab);
}

// Small device-side copy (kept as a kernel so captured graphs hold no memcpy nodes).
__global__ __launch_bounds__(256) void k_copy_i32(int32_t* dst, const int32_t* src, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

#define DG_OK_OR_HIP() (hipGetLastError() == hipSuccess ? 0 : -5)

int launch_embed_norm(int dtype, const int32_t* tok, const void* emb, const float* add, int n_add, int64_t add_stride,
                      float* x, void* n, int T, int d, float eps, hipStream_t s) {
  if (n_add < 0 || n_add > 16 || (n_add > 0 && !add)) return -1;
  if (dtype == 1)
    hipLaunchKernelGGL(k_embed_norm<bf16_t>, dim3(T), dim3(256), 0, s, tok, (const bf16_t*)emb, add, n_add, add_stride,
                       x, (bf16_t*)n, d, eps);
  else
    hipLaunchKernelGGL(k_embed_norm<float>, dim3(T), dim3(256), 0, s, tok, (const float*)emb, add, n_add, add_stride,
                       x, (float*)n, d, eps);
  return DG_OK_OR_HIP();
}

int launch_set_norm(int dtype, const float* src, float* x, void* n, int T, int d, float eps, hipStream_t s) {
  if (T < 1 || d < 1) return -1;
  if (dtype == 1)
    hipLaunchKernelGGL(k_set_norm<bf16_t>, dim3(T), dim3(256), 0, s, src, x, (bf16_t*)n, d, eps);
  else
    hipLaunchKernelGGL(k_set_norm<float>, dim3(T), dim3(256), 0, s, src, x, (float*)n, d, eps);
  return DG_OK_OR_HIP();
}

int launch_resid_norm(int dtype, float* x, const float* part, int n_split, int64_t split_stride, void* n, int T, int d,
                      float eps, hipStream_t s) {
  if (n_split < 1 || n_split > 16) return -1;
  if (d % 4 == 0 && d <= 4096 && split_stride % 4 == 0) {
    if (dtype == 1)
      hipLaunchKernelGGL(k_resid_norm4<bf16_t>, dim3(T), dim3(1024), 0, s, x, part, n_split, split_stride, (bf16_t*)n, d,
                         eps);
    else
      hipLaunchKernelGGL(k_resid_norm4<float>, dim3(T), dim3(1024), 0, s, x, part, n_split, split_stride, (float*)n, d,
                         eps);
    return DG_OK_OR_HIP();
  }
  if (dtype == 1)
    hipLaunchKernelGGL(k_resid_norm<bf16_t>, dim3(T), dim3(256), 0, s, x, part, n_split, split_stride, (bf16_t*)n, d, eps);
  else
    hipLaunchKernelGGL(k_resid_norm<float>, dim3(T), dim3(256), 0, s, x, part, n_split, split_stride, (float*)n, d, eps);
  return DG_OK_OR_HIP();
}

int launch_combine_norm(int dtype, float* x, const float* Y, const int32_t* inv, const float* w, int T, int k, int n_sh,
                        void* n, int d, float eps, hipStream_t s) {
  if (k > 16) return -1;
  if (d % 4 == 0 && d <= 4096 && n_sh <= 8) {
    if (dtype == 1)
      hipLaunchKernelGGL(k_combine_norm4<bf16_t>, dim3(T), dim3(1024), 0, s, x, Y, inv, w, T, k, n_sh, (bf16_t*)n, d, eps);
    else
      hipLaunchKernelGGL(k_combine_norm4<float>, dim3(T), dim3(1024), 0, s, x, Y, inv, w, T, k, n_sh, (float*)n, d, eps);
    return DG_OK_OR_HIP();
  }
  if (dtype == 1)
    hipLaunchKernelGGL(k_combine_norm<bf16_t>, dim3(T), dim3(256), 0, s, x, Y, inv, w, T, k, n_sh, (bf16_t*)n, d, eps);
  else
    hipLaunchKernelGGL(k_combine_norm<float>, dim3(T), dim3(256), 0, s, x, Y, inv, w, T, k, n_sh, (float*)n, d, eps);
  return DG_OK_OR_HIP();
}

int launch_reduce_splits(int dtype, const float* part, int n_split, int64_t split_stride, int64_t n_elems, void* out,
                         hipStream_t s) {
  if (n_split < 1 || n_split > 32) return -1;
  const dim3 g((unsigned)DG_CEIL_DIV(n_elems, 256));
  if (dtype == 1) hipLaunchKernelGGL(k_reduce_splits<bf16_t>, g, dim3(256), 0, s, part, n_split, split_stride, n_elems, (bf16_t*)out);
  else hipLaunchKernelGGL(k_reduce_splits<float>, g, dim3(256), 0, s, part, n_split, split_stride, n_elems, (float*)out);
  return DG_OK_OR_HIP();
}

int launch_init_canvas(int32_t* tokens, const uint64_t* seeds, int B, int C, int block, int vocab, hipStream_t s) {
  hipLaunchKernelGGL(k_init_canvas, dim3(DG_CEIL_DIV(B * C, 256)), dim3(256), 0, s, tokens, seeds, B, C, block,
                     (uint32_t)vocab);
  return DG_OK_OR_HIP();
}

int launch_copy_i32(int32_t* dst, const int32_t* src, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_i32, dim3(DG_CEIL_DIV(n, 256)), dim3(256), 0, s, dst, src, n);
  return DG_OK_OR_HIP();
}
