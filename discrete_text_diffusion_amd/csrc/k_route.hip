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
                                              int k, const int32_t* forced, int32_t* ids, float* w,
                                              float* r_out) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  constexpr int kMaxPerLane = 4;  // E <= 256
  constexpr int kMaxSplit = 8;    // partial sums are added in split order
  float r[kMaxPerLane];
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) {
    const int e = lane + q * 64;
    float v = -INFINITY;
    if (e < E) {
      float ps[kMaxSplit];
#pragma unroll
      for (int s = 0; s < kMaxSplit; ++s)
        ps[s] = s < n_split ? part[(int64_t)s * split_stride + (int64_t)t * E + e] : 0.f;
      v = ps[0];
#pragma unroll
      for (int s = 1; s < kMaxSplit; ++s) v += ps[s];
    }
    r[q] = v;
    if (r_out && e < E) r_out[(int64_t)t * E + e] = v;
  }
  float sel_v[16];
  int sel_e[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    sel_v[j] = -INFINITY;
    sel_e[j] = 0;
  }
  if (forced) {
    // test path: the caller fixes the k experts (in rank order); weights still
    // come from this token's router logits
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= k) break;
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
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (forced || j >= k) break;
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
#pragma unroll
    for (int j = 1; j < 16; ++j)
      if (j < k) m = fmaxf(m, sel_v[j]);
    float ex[16];
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      ex[j] = j < k ? expf(sel_v[j] - m) : 0.f;
      den += ex[j];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) {
        ids[t * k + j] = sel_e[j];
        w[t * k + j] = ex[j] / den;
      }
  }
}

// Single workgroup: stable counting of the (token, slot) pairs by expert.
// A bitmap marks which tokens chose each expert; a pair's position inside
// its expert segment is the number of earlier tokens in that expert's row
// (per-word prefix counts + one popcount), so the order within a segment is
// by token id.  Then segment offsets, the row -> token map, the inverse
// permutation and the GEMM row tiles (routed segments, then the
// shared-expert slices).  Requires T <= 64 * kMaxWords.
constexpr int kMaxWords = 16;  // 1024 tokens

__global__ __launch_bounds__(1024) void k_route_sort(const int32_t* ids, int T, int k, int E, int n_sh, int bm,
                                                     int32_t* row_token, int32_t* inv, int32_t* offsets,
                                                     GemmTile* tiles, int32_t* n_tiles) {
  __shared__ unsigned long long bits[256 * kMaxWords];
  __shared__ int32_t wpre[256 * kMaxWords];
  __shared__ int32_t cnt[256];
  __shared__ int32_t off[257];
  __shared__ int32_t toff[257];
  const int npairs = T * k;
  const int W = (T + 63) >> 6;
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int i = tid; i < E * W; i += nt) bits[i] = 0ull;
  __syncthreads();
  for (int q = tid; q < npairs; q += nt) {
    const int e = ids[q], t = q / k;
    atomicOr(&bits[e * W + (t >> 6)], 1ull << (t & 63));
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      wpre[e * W + w] = run;
      run += __popcll(bits[e * W + w]);
    }
    cnt[e] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, tf = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = o;
      toff[e] = tf;
      o += cnt[e];
      tf += (cnt[e] + bm - 1) / bm;
    }
    off[E] = o;
    toff[E] = tf;
    n_tiles[0] = tf + n_sh * ((T + bm - 1) / bm);
  }
  __syncthreads();
  for (int e = tid; e <= E; e += nt) offsets[e] = off[e];
  for (int q = tid; q < npairs; q += nt) {
    const int e = ids[q], t = q / k;
    const unsigned long long below = bits[e * W + (t >> 6)] & ((1ull << (t & 63)) - 1ull);
    const int p = off[e] + wpre[e * W + (t >> 6)] + __popcll(below);
    row_token[p] = t;
    inv[q] = p;
  }
  for (int e = tid; e < E; e += nt) {
    const int base = off[e], n = cnt[e];
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
                int32_t* ids, float* w, float* r_out, hipStream_t s) {
  if (E > 256 || k > 16 || k > E || n_split < 1 || n_split > 8) return -1;
  hipLaunchKernelGGL(k_topk, dim3(DG_CEIL_DIV(T, 4)), dim3(256), 0, s, part, n_split, split_stride, T, E, k, forced, ids,
                     w, r_out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int route_max_tokens() { return 64 * kMaxWords; }

int launch_route_sort(const int32_t* ids, int T, int k, int E, int n_sh, int bm, int32_t* row_token, int32_t* inv,
                      int32_t* offsets, GemmTile* tiles, int32_t* n_tiles, hipStream_t s) {
  if (E > 256 || T > 64 * kMaxWords || T < 1) return -1;
  hipLaunchKernelGGL(k_route_sort, dim3(1), dim3(1024), 0, s, ids, T, k, E, n_sh, bm, row_token, inv, offsets,
                     tiles, n_tiles);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
