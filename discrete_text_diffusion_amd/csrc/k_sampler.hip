// Entropy-bounded sampler and adaptive stop test, from the per-(row, tile)
// statistics of the LM head.
//
// Row merge (one workgroup per canvas position): with M = max_k m_k and
// w_k = exp(m_k - M) S_k,
//   S = sum_k w_k,  T = sum_k exp(m_k - M) (T_k + (m_k - M) S_k),
//   H = ln S - T / S   (entropy of softmax(z / tau)),
// the sampled tile is the first k whose cumulative w exceeds u1 * S, the
// sampled token is that tile's candidate (drawn in the LM head at u2), and
// the argmax is the tile maximum with the lowest id.
//
// Select (one workgroup per canvas): positions sorted by (H, position); the
// accepted count is the largest prefix whose summed entropy is <= the bound
// (at least 1); accepted positions take their sample, the others a fresh
// uniform token (Philox stream 1).  Stop when adaptive, t >= 1, the mean
// entropy is strictly under the threshold and the argmax equals the previous
// step's at every position.
#include "dg_internal.h"

namespace {

struct SelArgs {
  const float* H;
  const int32_t* sample;
  const int32_t* argmax;
  int32_t* prev_argmax;
  int32_t* tokens;      // out: next canvas
  uint8_t* accepted;
  int32_t* n_accepted;  // [B]
  float* mean_entropy;  // [B]
  int32_t* stop;        // [B]
  uint32_t* flags;      // [B]
  const uint64_t* seeds;
  int32_t C, step, block, vocab, adaptive;
  float bound, threshold;
};

__device__ __forceinline__ float block_scan256(float v, float* tmp, float& total) {
  // inclusive scan over 256 threads in thread order
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  float base = 0.f;
  for (int w = 0; w < wave; ++w) base += tmp[w];
  total = ((tmp[0] + tmp[1]) + tmp[2]) + tmp[3];
  return base + incl;
}

__global__ __launch_bounds__(256) void k_row_merge(const float4* part_f, const int2* part_i, int n_vt, int rows,
                                                  int C, const uint64_t* seeds, int step, int block, float* H,
                                                  int32_t* sample, int32_t* argmax, float* p_scale) {
  __shared__ float tmp[4];
  __shared__ float red[4];
  __shared__ int ired[4];
  __shared__ float fred2[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = DG_CEIL_DIV(n_vt, 256);
  const int k0 = tid * per, k1 = min(n_vt, k0 + per);
  const float4* pf = part_f + row * n_vt;
  const int2* pi = part_i + row * n_vt;
  // global max of m_k
  float mloc = -INFINITY;
  for (int k = k0; k < k1; ++k) mloc = fmaxf(mloc, pf[k].x);
  mloc = wave_max(mloc);
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // tile masses, T contribution, argmax candidate
  float s = 0.f, t = 0.f;
  float bz = -INFINITY;
  int bk = 0x7FFFFFFF;
  for (int k = k0; k < k1; ++k) {
    const float4 v = pf[k];
    const float sc = expf(v.x - M);
    s += sc * v.y;
    t += sc * (v.z + (v.x - M) * v.y);
    if (v.w > bz) { bz = v.w; bk = k; }
  }
  float S;
  const float incl = block_scan256(s, tmp, S);
  __syncthreads();
  // T total in thread order
  const float tw = wave_sum(t);
  if (lane == 0) fred2[wave] = tw;
  // argmax: largest zmax, lowest tile on ties
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float oz = __shfl_xor(bz, o, 64);
    const int ok = __shfl_xor(bk, o, 64);
    if (oz > bz || (oz == bz && ok < bk)) { bz = oz; bk = ok; }
  }
  __shared__ float bzs[4];
  __shared__ int bks[4];
  if (lane == 0) { bzs[wave] = bz; bks[wave] = bk; }
  // sampled tile
  const int canvas_id = (int)(row / C), pos = (int)(row - (int64_t)canvas_id * C);
  const uint64_t seed = seeds[canvas_id];
  const dg_u32x4 w = dg_philox((uint32_t)pos, (uint32_t)step, (uint32_t)block, DG_STREAM_SAMPLE, (uint32_t)seed,
                               (uint32_t)(seed >> 32));
  const float thr = dg_word_unit(w.x) * S;
  int hit = 0x7FFFFFFF, lastpos = -1;
  float run = incl - s;
  for (int k = k0; k < k1; ++k) {
    const float4 v = pf[k];
    const float wk = expf(v.x - M) * v.y;
    run += wk;
    if (hit == 0x7FFFFFFF && run > thr) hit = k;
    if (wk > 0.f) lastpos = k;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    hit = min(hit, __shfl_xor(hit, o, 64));
    lastpos = max(lastpos, __shfl_xor(lastpos, o, 64));
  }
  __shared__ int hits[4], lasts[4];
  if (lane == 0) { hits[wave] = hit; lasts[wave] = lastpos; }
  __syncthreads();
  if (tid == 0) {
    const float T = ((fred2[0] + fred2[1]) + fred2[2]) + fred2[3];
    float h = logf(S) - T / S;
    if (!(h >= 0.f)) h = (h != h) ? INFINITY : 0.f;  // rounding below 0 -> 0; NaN -> +inf
    H[row] = h;
    int kk = min(min(hits[0], hits[1]), min(hits[2], hits[3]));
    if (kk == 0x7FFFFFFF) kk = max(max(lasts[0], lasts[1]), max(lasts[2], lasts[3]));
    if (kk < 0) kk = 0;
    sample[row] = pi[kk].x;
    float z = bzs[0];
    int zk = bks[0];
    for (int q = 1; q < 4; ++q)
      if (bzs[q] > z || (bzs[q] == z && bks[q] < zk)) { z = bzs[q]; zk = bks[q]; }
    argmax[row] = pi[zk < n_vt ? zk : 0].y;
  }
  if (p_scale) {
    const float invS = 1.0f / S;
    for (int k = k0; k < k1; ++k) p_scale[(int64_t)k * rows + row] = expf(pf[k].x - M) * invS;  // tile-major
  }
  (void)ired;
}

// One workgroup of 1024 threads per canvas (C <= 1024).
__global__ __launch_bounds__(1024) void k_select(SelArgs a) {
  __shared__ unsigned long long keys[1024];
  __shared__ float wsum[16];
  __shared__ int wcnt[16];
  __shared__ int wsame[16];
  __shared__ int wbad[16];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int C = a.C;
  int np2 = 1;
  while (np2 < C) np2 <<= 1;
  const int64_t base = (int64_t)b * C;
  float h = 0.f;
  bool bad = false;
  if (tid < C) {
    h = a.H[base + tid];
    bad = !(h < INFINITY);
  }
  if (tid < np2)
    keys[tid] = tid < C ? (((unsigned long long)__float_as_uint(h)) << 32) | (unsigned)tid : ~0ull;
  // mean entropy in position order and the argmax comparison
  const float hs = wave_sum(tid < C ? h : 0.f);
  const bool same = tid >= C || a.argmax[base + tid] == a.prev_argmax[base + tid];
  const uint64_t sb = __ballot(!same);
  const uint64_t bb = __ballot(bad);
  if (lane == 0) { wsum[wave] = hs; wsame[wave] = sb == 0; wbad[wave] = bb != 0; }
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      if (tid < (np2 >> 1)) {
        const int lo = 2 * tid - (tid & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned long long x = keys[lo], y = keys[hi];
        if ((x > y) == up) { keys[lo] = y; keys[hi] = x; }
      }
    }
  }
  __syncthreads();
  // inclusive prefix of sorted entropies, count of prefixes within the bound
  const float hv = tid < C ? __uint_as_float((uint32_t)(keys[tid] >> 32)) : 0.f;
  float incl = wave_incl_scan(hv);
  __shared__ float wtot[16];
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  for (int w2 = 0; w2 < wave; ++w2) incl += wtot[w2];
  const bool within = tid < C && incl <= a.bound;
  const uint64_t cb = __ballot(within);
  if (lane == 0) wcnt[wave] = __popcll(cb);
  __syncthreads();
  int K = 0;
  for (int w2 = 0; w2 < nw; ++w2) K += wcnt[w2];
  if (K < 1) K = 1;
  if (tid < C) {
    const int pos = (int)(keys[tid] & 0xFFFFFFFFu);
    a.accepted[base + pos] = tid < K ? 1 : 0;
    int nxt;
    if (tid < K) {
      nxt = a.sample[base + pos];
    } else {
      const uint64_t sd = a.seeds[b];
      const dg_u32x4 w = dg_philox((uint32_t)pos, (uint32_t)a.step, (uint32_t)a.block, DG_STREAM_RENOISE,
                                   (uint32_t)sd, (uint32_t)(sd >> 32));
      nxt = dg_word_token(w.x, (uint32_t)a.vocab);
    }
    a.tokens[base + pos] = nxt;
  }
  __syncthreads();
  if (tid < C) a.prev_argmax[base + tid] = a.argmax[base + tid];
  if (tid == 0) {
    float tot = 0.f;
    int all_same = 1, any_bad = 0;
    for (int w2 = 0; w2 < nw; ++w2) {
      tot += wsum[w2];
      all_same &= wsame[w2];
      any_bad |= wbad[w2];
    }
    const float mean = tot / (float)C;
    a.mean_entropy[b] = mean;
    a.n_accepted[b] = K;
    a.stop[b] = (a.adaptive && a.step >= 1 && mean < a.threshold && all_same) ? 1 : 0;
    if (any_bad) a.flags[b] |= 1u;
  }
}

}  // namespace

// The carried self-conditioning input, in place: p[row][v] = exp(a - m_k)
// (as the LM head wrote it) times the row's tile factor exp(m_k - m) / S
// (tile-major [vocab/256][rows]) = the tempered probability, rounded once
// more to the model dtype.  Eight ids per thread (one 256-id tile each).
template <typename TA>
__global__ __launch_bounds__(256) void k_normalize_side(TA* p, const float* scale, int rows, int vocab) {
  const int64_t per_row = vocab >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * per_row) return;
  const int row = (int)(i / per_row);
  const int v0 = (int)(i - (int64_t)row * per_row) * 8;
  const float f = scale[(int64_t)(v0 >> 8) * rows + row];
  TA* q = p + (int64_t)row * vocab + v0;
  if constexpr (sizeof(TA) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(q);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf2f((bf16_t)(w[j] & 0xFFFFu)) * f, hi = bf2f((bf16_t)(w[j] >> 16)) * f;
      w[j] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
    }
    *reinterpret_cast<uint4*>(q) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* q4 = reinterpret_cast<float4*>(q);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float4 v = q4[j];
      v.x *= f; v.y *= f; v.z *= f; v.w *= f;
      q4[j] = v;
    }
  }
}

int launch_row_merge(const float4* part_f, const int2* part_i, int n_vt, int rows, int C, const uint64_t* seeds,
                     int step, int block, float* H, int32_t* sample, int32_t* argmax, float* p_scale, hipStream_t s) {
  hipLaunchKernelGGL(k_row_merge, dim3(rows), dim3(256), 0, s, part_f, part_i, n_vt, rows, C, seeds, step, block, H,
                     sample, argmax, p_scale);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_select(const float* H, const int32_t* sample, const int32_t* argmax, int32_t* prev_argmax, int32_t* tokens,
                  uint8_t* accepted, int32_t* n_accepted, float* mean_entropy, int32_t* stop, uint32_t* flags,
                  const uint64_t* seeds, int B, int C, int step, int block, int vocab, int adaptive, float bound,
                  float threshold, hipStream_t s) {
  if (C > 1024) return -1;
  SelArgs a{H, sample, argmax, prev_argmax, tokens, accepted, n_accepted, mean_entropy, stop, flags, seeds,
            C, step, block, vocab, adaptive, bound, threshold};
  int threads = 64;
  while (threads < C) threads <<= 1;
  hipLaunchKernelGGL(k_select, dim3(B), dim3(threads), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_normalize_side(int bf16, void* p, const float* scale, int rows, int vocab, hipStream_t s) {
  if (!p || !scale || rows < 1 || vocab % 256) return -1;
  const dim3 g((unsigned)DG_CEIL_DIV((int64_t)rows * (vocab >> 3), 256));
  if (bf16) hipLaunchKernelGGL(k_normalize_side<bf16_t>, g, dim3(256), 0, s, (bf16_t*)p, scale, rows, vocab);
  else hipLaunchKernelGGL(k_normalize_side<float>, g, dim3(256), 0, s, (float*)p, scale, rows, vocab);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
