// MoE routing for the denoising step: top-k experts per token from the router
// logits (ties to the lower expert id), softmax over the k selected logits,
// and a stable counting of the (token, slot) pairs into per-expert segments
// with the GEMM row tiles that cover them.
//
// Pair rows: [0, T*k) are the routed pairs ordered by (expert, token); the
// shared expert is split into `n_sh` virtual groups of width d_expert, each
// seeing every token, at rows T*k + c*T + t.
#include "dg_internal.h"

namespace {

// One wave per token.  Router logits arrive as `n_split` fp32 partial sums
// [split][T][E] added in split order.
__global__ __launch_bounds__(256) void k_topk(const float* part, int n_split, int64_t split_stride, int T, int E,
                                              int k, const int32_t* forced, int32_t* ids, float* w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  constexpr int kMaxPerLane = 4;  // E <= 256
  float r[kMaxPerLane];
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) {
    const int e = lane + q * 64;
    float v = -INFINITY;
    if (e < E) {
      v = 0.f;
      for (int s = 0; s < n_split; ++s) v += part[(int64_t)s * split_stride + (int64_t)t * E + e];
    }
    r[q] = v;
  }
  float sel_v[16];
  int sel_e[16];
  if (forced) {
    // test path: the caller fixes the k experts (in rank order); weights still
    // come from this token's router logits
    for (int j = 0; j < k; ++j) {
      int e = forced[t * k + j];
      if (e < 0 || e >= E) e = 0;  // keep the grouped GEMMs in bounds on bad test input
      const int q = e >> 6;
      float mine = r[0];
#pragma unroll
      for (int qq = 1; qq < kMaxPerLane; ++qq)
        if (qq == q) mine = r[qq];
      sel_v[j] = __shfl(mine, e & 63, 64);
      sel_e[j] = e;
    }
  }
  for (int j = 0; j < (forced ? 0 : k); ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q) {
      const int e = lane + q * 64;
      if (e < E && (r[q] > bv || (r[q] == bv && e < be))) { bv = r[q]; be = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    sel_v[j] = bv;
    sel_e[j] = be;
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q)
      if (lane + q * 64 == be) r[q] = -INFINITY;  // taken
  }
  if (lane == 0) {
    float m = sel_v[0];
    for (int j = 1; j < k; ++j) m = fmaxf(m, sel_v[j]);
    float den = 0.f;
    for (int j = 0; j < k; ++j) den += expf(sel_v[j] - m);
    for (int j = 0; j < k; ++j) {
      ids[t * k + j] = sel_e[j];
      w[t * k + j] = expf(sel_v[j] - m) / den;
    }
  }
}

// Single workgroup: bitonic sort of (expert << 20 | pair) keys in LDS, then
// segment offsets, the row -> token map, the inverse permutation and the
// GEMM row tiles (routed segments first, then the shared-expert slices).
__global__ __launch_bounds__(1024) void k_route_sort(const int32_t* ids, int T, int k, int E, int n_sh, int bm,
                                                     int32_t* row_token, int32_t* inv, int32_t* offsets,
                                                     GemmTile* tiles, int32_t* n_tiles) {
  extern __shared__ uint32_t sm[];
  const int npairs = T * k;
  int np2 = 1;
  while (np2 < npairs) np2 <<= 1;
  uint32_t* key = sm;
  int32_t* cnt = reinterpret_cast<int32_t*>(sm + np2);  // [E]
  int32_t* toff = cnt + 256;                           // [E+1] tile offsets
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int i = tid; i < np2; i += nt) key[i] = i < npairs ? ((uint32_t)ids[i] << 20) | (uint32_t)i : 0xFFFFFFFFu;
  for (int i = tid; i < E; i += nt) cnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < npairs; i += nt) atomicAdd(&cnt[ids[i]], 1);
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = tid; i < (np2 >> 1); i += nt) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint32_t a = key[lo], b = key[hi];
        if ((a > b) == up) { key[lo] = b; key[hi] = a; }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0, tof = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = off;
      toff[e] = tof;
      off += cnt[e];
      tof += (cnt[e] + bm - 1) / bm;
    }
    offsets[E] = off;
    toff[E] = tof;
    const int per_sh = (T + bm - 1) / bm;
    n_tiles[0] = tof + n_sh * per_sh;
  }
  __syncthreads();
  for (int p = tid; p < npairs; p += nt) {
    const uint32_t q = key[p] & 0xFFFFFu;
    row_token[p] = (int32_t)(q / (uint32_t)k);
    inv[q] = p;
  }
  for (int e = tid; e < E; e += nt) {
    const int base = offsets[e], n = cnt[e];
    for (int i = 0, j = toff[e]; i * bm < n; ++i, ++j) tiles[j] = GemmTile{e, base + i * bm, min(bm, n - i * bm), 0};
  }
  const int per_sh = (T + bm - 1) / bm;
  for (int i = tid; i < n_sh * per_sh; i += nt) {
    const int c = i / per_sh, q = i - c * per_sh;
    tiles[toff[E] + i] = GemmTile{E + c, npairs + c * T + q * bm, min(bm, T - q * bm), 0};
  }
  for (int i = tid; i < n_sh * T; i += nt) row_token[npairs + i] = i % T;
}

}  // namespace

int launch_topk(const float* part, int n_split, int64_t split_stride, int T, int E, int k, const int32_t* forced,
                int32_t* ids, float* w, hipStream_t s) {
  if (E > 256 || k > 16 || k > E) return -1;
  hipLaunchKernelGGL(k_topk, dim3(DG_CEIL_DIV(T, 4)), dim3(256), 0, s, part, n_split, split_stride, T, E, k, forced, ids,
                     w);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

size_t route_sort_lds_bytes(int npairs) {
  int np2 = 1;
  while (np2 < npairs) np2 <<= 1;
  return (size_t)np2 * 4 + 2 * 256 * 4 + 64;
}

int launch_route_sort(const int32_t* ids, int T, int k, int E, int n_sh, int bm, int32_t* row_token, int32_t* inv,
                      int32_t* offsets, GemmTile* tiles, int32_t* n_tiles, hipStream_t s) {
  if (E > 255) return -1;
  const size_t lds = route_sort_lds_bytes(T * k);
  if (lds > 65536) return -1;
  hipLaunchKernelGGL(k_route_sort, dim3(1), dim3(1024), lds, s, ids, T, k, E, n_sh, bm, row_token, inv, offsets,
                     tiles, n_tiles);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
