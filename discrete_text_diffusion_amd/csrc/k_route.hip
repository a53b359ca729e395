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
// [split][T][E] added in split order.  Selection in k rounds: each logit
// becomes a 64-bit key (order-preserving image of the value, then the
// complement of the expert id, so equal values rank the lower id first; -0
// is read as +0), and each round takes the wave's largest live key (within
// 16-lane rows by DPP, then the four row maxima as scalars) and retires it.
// The weights are the softmax over the k selected logits, summed in rank
// order.
// One wave per workgroup (one token): the waves never wait for each other.
// Every partial load is issued up front and unconditionally (clamped
// indices; the values past n_split or E are discarded), so all of them are in
// flight together.
constexpr int kTopkWaves = 1;

__device__ __forceinline__ uint32_t float_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, true);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int NQ>  // logits per lane: E <= 64 NQ
__global__ __launch_bounds__(64 * kTopkWaves) void k_topk(const float* part, int n_split, int64_t split_stride,
                                                          int T, int E, int k, const int32_t* forced, int32_t* ids,
                                                          float* w, float* r_out) {
  __shared__ __attribute__((aligned(16))) float lg[kTopkWaves][256];
  __shared__ float sv[kTopkWaves][16];
  __shared__ int se[kTopkWaves][16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + wave;
  const bool live = t < T;
  constexpr int kMaxSplit = 16;  // partial sums are added in split order
  const int tc = live ? t : 0;
  float ps[NQ][kMaxSplit];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int ec = min(lane + q * 64, E - 1);
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s)
      ps[q][s] = part[(int64_t)min(s, n_split - 1) * split_stride + (int64_t)tc * E + ec];
  }
  float r[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + q * 64;
    float v = ps[q][0];
#pragma unroll
    for (int s = 1; s < kMaxSplit; ++s) v += s < n_split ? ps[q][s] : 0.f;
    v = (live && e < E) ? v : -INFINITY;
    if (live && e < E && r_out) r_out[(int64_t)t * E + e] = v;
    r[q] = v;
  }
  if (!live) return;
  if (forced) {
    // test path: the caller fixes the k experts (in rank order); weights still
    // come from this token's router logits
#pragma unroll
    for (int q = 0; q < NQ; ++q) lg[wave][lane + q * 64] = r[q];
    __syncthreads();
    if (lane < k) {
      int e = forced[t * k + lane];
      if (e < 0 || e >= E) e = 0;  // keep the grouped GEMMs in bounds on bad test input
      sv[wave][lane] = lg[wave][e];
      se[wave][lane] = e;
    }
  } else {
    // keys of the live logits; 0 (below every live key) past E and once taken
    uint64_t key[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + q * 64;
      key[q] = e < E ? ((uint64_t)float_order(r[q] + 0.f) << 32) | (uint32_t)~e : 0ull;
    }
    for (int j = 0; j < k; ++j) {
      uint64_t b = key[0];
#pragma unroll
      for (int q = 1; q < NQ; ++q) b = max_u64(b, key[q]);
      b = max_u64(b, dpp_u64<0xB1>(b));   // quad_perm xor 1
      b = max_u64(b, dpp_u64<0x4E>(b));   // quad_perm xor 2
      b = max_u64(b, dpp_u64<0x141>(b));  // row half mirror
      b = max_u64(b, dpp_u64<0x140>(b));  // row mirror: the row's maximum in every lane
      b = max_u64(max_u64(readlane_u64(b, 0), readlane_u64(b, 16)),
                  max_u64(readlane_u64(b, 32), readlane_u64(b, 48)));
      const int e = (int)~(uint32_t)b;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (lane + q * 64 == e) key[q] = 0ull;
      if (lane == 0) {
        sv[wave][j] = order_float((uint32_t)(b >> 32));
        se[wave][j] = e;
      }
    }
  }
  __syncthreads();
  if (lane < k) {
    const float m = sv[wave][0];
    float den = 0.f;
    for (int j = 0; j < k; ++j) den += expf(sv[wave][j] - m);
    ids[t * k + lane] = se[wave][lane];
    w[t * k + lane] = expf(sv[wave][lane] - m) / den;
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
  // exclusive prefix sums of the segment sizes and tile counts over the
  // experts: first wave, four experts per lane
  if (tid < 64) {
    int c4[4], t4[4], cs = 0, ts = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      c4[q] = e < E ? cnt[e] : 0;
      t4[q] = (c4[q] + bm - 1) / bm;
      cs += c4[q];
      ts += t4[q];
    }
    int ci = cs, ti = ts;  // inclusive scans over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int cu = __shfl_up(ci, o, 64), tu = __shfl_up(ti, o, 64);
      if (tid >= o) { ci += cu; ti += tu; }
    }
    int co = ci - cs, to = ti - ts;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e <= E) { off[e] = co; toff[e] = to; }
      co += c4[q];
      to += t4[q];
    }
    if (tid == 63) {
      off[E] = co;  // the totals (E = 256 has no lane for them above)
      toff[E] = to;
      n_tiles[0] = ti + n_sh * ((T + bm - 1) / bm);
    }
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
    const int span = (toff[e] << 16) | (toff[e + 1] - toff[e]);
    for (int i = 0, j = toff[e]; i * bm < n; ++i, ++j) tiles[j] = GemmTile{e, base + i * bm, min(bm, n - i * bm), span};
  }
  const int per_sh = (T + bm - 1) / bm;
  for (int i = tid; i < n_sh * per_sh; i += nt) {
    const int c = i / per_sh, q = i - c * per_sh;
    tiles[toff[E] + i] = GemmTile{E + c, npairs + c * T + q * bm, min(bm, T - q * bm), ((toff[E] + c * per_sh) << 16) | per_sh};
  }
  for (int i = tid; i < n_sh * T; i += nt) row_token[npairs + i] = i % T;
}

// More tokens than one workgroup's bitmaps hold: the same stable counting
// over chunks of kChunk tokens in three launches.  (1) per chunk, the pairs
// of every expert; (2) one workgroup: per expert, the pairs in earlier chunks
// (summed in chunk order), the segment offsets and the GEMM row tiles as
// above; (3) per chunk, the bitmaps again and each pair's row = segment start
// + the expert's pairs in earlier chunks + the earlier tokens of its chunk.
// The rows come out exactly as the one-workgroup sort would place them.
constexpr int kChunk = 64 * kMaxWords;
constexpr int kMaxChunks = 64;

__global__ __launch_bounds__(1024) void k_route_count(const int32_t* ids, int T, int k, int E, int32_t* ccnt) {
  __shared__ int32_t cnt[256];
  const int c = blockIdx.x, t0 = c * kChunk, tn = min(kChunk, T - t0);
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int e = tid; e < E; e += nt) cnt[e] = 0;
  __syncthreads();
  const int32_t* cid = ids + (int64_t)t0 * k;
  for (int q = tid; q < tn * k; q += nt) atomicAdd(&cnt[cid[q]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += nt) ccnt[c * E + e] = cnt[e];
}

__global__ __launch_bounds__(1024) void k_route_scan(int32_t* ccnt, int nchunks, int T, int k, int E, int n_sh,
                                                    int bm, int32_t* offsets, GemmTile* tiles, int32_t* n_tiles) {
  __shared__ int32_t cnt[256];
  __shared__ int32_t off[257];
  __shared__ int32_t toff[257];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int npairs = T * k;
  for (int e = tid; e < E; e += nt) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int v = ccnt[c * E + e];
      ccnt[c * E + e] = run;
      run += v;
    }
    cnt[e] = run;
  }
  __syncthreads();
  if (tid < 64) {
    int c4[4], t4[4], cs = 0, ts = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      c4[q] = e < E ? cnt[e] : 0;
      t4[q] = (c4[q] + bm - 1) / bm;
      cs += c4[q];
      ts += t4[q];
    }
    int ci = cs, ti = ts;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int cu = __shfl_up(ci, o, 64), tu = __shfl_up(ti, o, 64);
      if (tid >= o) { ci += cu; ti += tu; }
    }
    int co = ci - cs, to = ti - ts;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e <= E) { off[e] = co; toff[e] = to; }
      co += c4[q];
      to += t4[q];
    }
    if (tid == 63) {
      off[E] = co;
      toff[E] = to;
      n_tiles[0] = ti + n_sh * ((T + bm - 1) / bm);
    }
  }
  __syncthreads();
  for (int e = tid; e <= E; e += nt) offsets[e] = off[e];
  for (int i = tid; i < nchunks * E; i += nt) ccnt[i] += off[i % E];  // absolute first row of (chunk, expert)
  for (int e = tid; e < E; e += nt) {
    const int base = off[e], n = cnt[e];
    const int span = (toff[e] << 16) | (toff[e + 1] - toff[e]);
    for (int i = 0, j = toff[e]; i * bm < n; ++i, ++j) tiles[j] = GemmTile{e, base + i * bm, min(bm, n - i * bm), span};
  }
  const int per_sh = (T + bm - 1) / bm;
  for (int i = tid; i < n_sh * per_sh; i += nt) {
    const int c = i / per_sh, q = i - c * per_sh;
    tiles[toff[E] + i] = GemmTile{E + c, npairs + c * T + q * bm, min(bm, T - q * bm), ((toff[E] + c * per_sh) << 16) | per_sh};
  }
}

__global__ __launch_bounds__(1024) void k_route_place(const int32_t* ids, const int32_t* cbase, int T, int k, int E,
                                                     int n_sh, int32_t* row_token, int32_t* inv) {
  __shared__ unsigned long long bits[256 * kMaxWords];
  __shared__ int32_t wpre[256 * kMaxWords];
  const int c = blockIdx.x, t0 = c * kChunk, tn = min(kChunk, T - t0);
  const int W = (tn + 63) >> 6;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int32_t* cid = ids + (int64_t)t0 * k;
  for (int i = tid; i < E * W; i += nt) bits[i] = 0ull;
  __syncthreads();
  for (int q = tid; q < tn * k; q += nt) {
    const int e = cid[q], t = q / k;
    atomicOr(&bits[e * W + (t >> 6)], 1ull << (t & 63));
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      wpre[e * W + w] = run;
      run += __popcll(bits[e * W + w]);
    }
  }
  __syncthreads();
  for (int q = tid; q < tn * k; q += nt) {
    const int e = cid[q], t = q / k;
    const unsigned long long below = bits[e * W + (t >> 6)] & ((1ull << (t & 63)) - 1ull);
    const int p = cbase[c * E + e] + wpre[e * W + (t >> 6)] + __popcll(below);
    row_token[p] = t0 + t;
    inv[(int64_t)t0 * k + q] = p;
  }
  const int npairs = T * k;
  for (int i = tid; i < n_sh * tn; i += nt) {
    const int sh = i / tn, t = i - sh * tn;
    row_token[npairs + sh * T + t0 + t] = t0 + t;
  }
}

}  // namespace

int launch_topk(const float* part, int n_split, int64_t split_stride, int T, int E, int k, const int32_t* forced,
                int32_t* ids, float* w, float* r_out, hipStream_t s) {
  if (E > 256 || k > 16 || k > E || n_split < 1 || n_split > 16) return -1;
  const dim3 g(DG_CEIL_DIV(T, kTopkWaves)), b(64 * kTopkWaves);
  if (E <= 64) hipLaunchKernelGGL(k_topk<1>, g, b, 0, s, part, n_split, split_stride, T, E, k, forced, ids, w, r_out);
  else if (E <= 128) hipLaunchKernelGGL(k_topk<2>, g, b, 0, s, part, n_split, split_stride, T, E, k, forced, ids, w, r_out);
  else hipLaunchKernelGGL(k_topk<4>, g, b, 0, s, part, n_split, split_stride, T, E, k, forced, ids, w, r_out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int route_max_tokens() { return kChunk * kMaxChunks; }

int route_chunk_words(int T) { return T > kChunk ? DG_CEIL_DIV(T, kChunk) * 256 : 0; }

int launch_route_sort(const int32_t* ids, int T, int k, int E, int n_sh, int bm, int32_t* row_token, int32_t* inv,
                      int32_t* offsets, GemmTile* tiles, int32_t* n_tiles, int32_t* chunk_counts, hipStream_t s) {
  if (E > 256 || T > kChunk * kMaxChunks || T < 1 || (int64_t)T * (k + n_sh) > INT32_MAX) return -1;
  if (T <= kChunk) {
    hipLaunchKernelGGL(k_route_sort, dim3(1), dim3(1024), 0, s, ids, T, k, E, n_sh, bm, row_token, inv, offsets,
                       tiles, n_tiles);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  if (!chunk_counts) return -1;
  const int nchunks = DG_CEIL_DIV(T, kChunk);
  hipLaunchKernelGGL(k_route_count, dim3(nchunks), dim3(1024), 0, s, ids, T, k, E, chunk_counts);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, s, chunk_counts, nchunks, T, k, E, n_sh, bm, offsets, tiles,
                     n_tiles);
  hipLaunchKernelGGL(k_route_place, dim3(nchunks), dim3(1024), 0, s, ids, chunk_counts, T, k, E, n_sh, row_token, inv);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
