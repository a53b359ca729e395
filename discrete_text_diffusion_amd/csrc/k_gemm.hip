// Weight-streaming GEMMs of the denoising step on gfx950.
//
//   out[row][n] = sum_k act[row][k] * W[n][k]
//
// W is a pre-packed bf16 matrix ("weight layout"): 16-row x 32-column tiles of
// 1 KiB, tile (nt, kt) at element offset (nt*KT + kt)*512, and inside a tile
// lane l of a wave holds the 8 consecutive k of row nt*16 + l%16 starting at
// kt*32 + 8*(l/16).  One wave therefore loads one MFMA A operand as one
// contiguous 1 KiB read, and a wave walking K for a fixed 16-row tile streams
// a contiguous run of KT KiB.
//
// A workgroup of 4 waves owns 4*NWT feature tiles (16 features each) and one
// row tile of BM activation rows.  Activations are staged through LDS in
// K-chunks of KC (double buffered) and shared by the 4 waves; weights go
// straight from HBM into registers, one K-chunk ahead of the MFMAs.  The MFMA
// is v_mfma_f32_16x16x32_bf16 with the weights as A (16 features x 32 k) and
// the activations as B (32 k x 16 rows): lane l ends with 4 consecutive
// features 4*(l/16)+e of row l%16.
//
// Block ids are remapped so that blocks sharing data (the feature blocks of
// one row tile, or the row tiles of one feature block) sit on the same XCD:
// hardware dispatches block b to XCD b % 8.
#include <type_traits>

#include "dg_internal.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int xcd_logical_block(int nblocks) {
  const int hw = blockIdx.x;
  const int per = nblocks >> 3;
  return (hw & 7) * per + (hw >> 3);
}

__device__ __forceinline__ void decode_block(const GemmArgs& a, int lb, int& tile, int& fb, int& ks) {
  // order: split outermost, then (tile, fb) with the chosen one fastest
  const int per_split = a.max_tiles * a.n_fb;
  ks = lb / per_split;
  const int r = lb - ks * per_split;
  if (a.tile_fastest) {
    tile = r % a.max_tiles;
    fb = r / a.max_tiles;
  } else {
    fb = r % a.n_fb;
    tile = r / a.n_fb;
  }
}

template <typename TA>
__device__ __forceinline__ void store_act2(void* base, int64_t idx, float v0, float v1);
template <>
__device__ __forceinline__ void store_act2<bf16_t>(void* base, int64_t idx, float v0, float v1) {
  const uint32_t pk = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
  *reinterpret_cast<uint32_t*>(reinterpret_cast<bf16_t*>(base) + idx) = pk;
}
template <>
__device__ __forceinline__ void store_act2<float>(void* base, int64_t idx, float v0, float v1) {
  *reinterpret_cast<float2*>(reinterpret_cast<float*>(base) + idx) = make_float2(v0, v1);
}

// Epilogue for two adjacent output features n, n+1 of one output row.
// g0/g1 are the (gate) accumulators; u0/u1 the up accumulators for GeGLU.
template <typename TA>
__device__ __forceinline__ void epi_pair(const GemmArgs& a, int ks, int orow, int n, float g0, float g1,
                                         float u0, float u1) {
  switch (a.epi) {
    case EPI_STORE_F32: {
      float* o = a.out_f32 + (int64_t)ks * a.split_stride + (int64_t)orow * a.ldo + n;
      *reinterpret_cast<float2*>(o) = make_float2(a.alpha * g0, a.alpha * g1);
      break;
    }
    case EPI_RESID: {
      float2* o = reinterpret_cast<float2*>(a.out_f32 + (int64_t)orow * a.ldo + n);
      float2 x = *o;
      x.x += g0;
      x.y += g1;
      *o = x;
      break;
    }
    case EPI_GEGLU:
      store_act2<TA>(a.out_act, (int64_t)orow * a.ldo + n, gelu_tanh(g0) * u0, gelu_tanh(g1) * u1);
      break;
    case EPI_GELU:
      store_act2<TA>(a.out_act, (int64_t)orow * a.ldo + n, gelu_tanh(g0), gelu_tanh(g1));
      break;
    case EPI_STORE_ACT:
      store_act2<TA>(a.out_act, (int64_t)orow * a.ldo + n, a.alpha * g0, a.alpha * g1);
      break;
    case EPI_QKV: {
      const QkvEpi& q = a.qkv;
      const int seq = orow / q.seq_len;
      const int i = orow - seq * q.seq_len;
      float v0 = g0, v1 = g1;
      if (n < q.q_dim + q.kv_dim) {
        // RoPE on (2j, 2j+1) of the head at absolute position pos0 + i; the
        // angle is formed in fp64 so long positions keep full accuracy.
        const int dd = n % q.d_head;
        const int j = dd >> 1;
        const double inv_freq = exp2(-(2.0 * j / q.d_head) * log2((double)q.rope_base));
        const double ang = (double)(q.pos0 + i) * inv_freq;
        double sd, cd;
        sincos(ang, &sd, &cd);
        const float c = (float)cd, s = (float)sd;
        v0 = g0 * c - g1 * s;
        v1 = g0 * s + g1 * c;
      }
      if (n < q.q_dim) {
        store_act2<TA>(q.q, (int64_t)orow * q.q_dim + n, v0, v1);
      } else {
        const bool is_k = n < q.q_dim + q.kv_dim;
        const int nn = n - q.q_dim - (is_k ? 0 : q.kv_dim);
        const int h = nn / q.d_head, dd = nn - h * q.d_head;
        const int64_t head = (int64_t)seq * q.kv_b_stride + (int64_t)h * q.kv_h_stride;
        if (is_k) {
          store_act2<TA>(q.k, head + (int64_t)(q.kv_row0 + i) * q.d_head + dd, v0, v1);
        } else {  // V is stored transposed: [d_head][rows]
          TA* vb = reinterpret_cast<TA*>(q.v) + head + (int64_t)dd * q.v_pitch + q.kv_row0 + i;
          vb[0] = to_act<TA>(v0);
          vb[q.v_pitch] = to_act<TA>(v1);
        }
      }
      break;
    }
    default:
      break;
  }
}

__device__ __forceinline__ uint4 pack8_bf16(const float* f) {
  uint4 r;
  r.x = (uint32_t)f2bf(f[0]) | ((uint32_t)f2bf(f[1]) << 16);
  r.y = (uint32_t)f2bf(f[2]) | ((uint32_t)f2bf(f[3]) << 16);
  r.z = (uint32_t)f2bf(f[4]) | ((uint32_t)f2bf(f[5]) << 16);
  r.w = (uint32_t)f2bf(f[6]) | ((uint32_t)f2bf(f[7]) << 16);
  return r;
}

// Load 8 consecutive activation values of one row as 8 bf16 (16 bytes).
template <int ACT>
__device__ __forceinline__ uint4 load_act8(const GemmArgs& a, int arow, int k) {
  if constexpr (ACT == ACT_BF16) {
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.act) + (int64_t)arow * a.act_ld + k);
  } else if constexpr (ACT == ACT_F32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.act) + (int64_t)arow * a.act_ld + k);
    const float4 x = p[0], y = p[1];
    const float f[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    return pack8_bf16(f);
  } else {
    // ACT_BF16_SCALED: raw bf16; the per-(row, 256-wide K tile) scale is
    // applied to the partial sums (see wsgemm_mainloop)
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.act) + (int64_t)arow * a.act_ld + k);
  }
}

struct GroupW {
  const bf16_t* w0;
  const bf16_t* w1;
  int kt, kt_off;
};

__device__ __forceinline__ GroupW group_weights(const GemmArgs& a, int g) {
  GroupW r;
  if (g < a.n_main) {
    r.w0 = reinterpret_cast<const bf16_t*>(a.w0) + (int64_t)g * a.w_group_stride;
    r.w1 = a.w1 ? reinterpret_cast<const bf16_t*>(a.w1) + (int64_t)g * a.w_group_stride : nullptr;
    r.kt = a.kt_main;
    r.kt_off = 0;
  } else {
    const int c = g - a.n_main;
    r.w0 = reinterpret_cast<const bf16_t*>(a.w0_alt) + (int64_t)c * a.w_alt_stride;
    r.w1 = a.w1_alt ? reinterpret_cast<const bf16_t*>(a.w1_alt) + (int64_t)c * a.w_alt_stride : nullptr;
    r.kt = a.kt_alt;
    r.kt_off = c * a.kt_off_alt;
  }
  return r;
}

// Main loop shared by the generic and the LM-head kernels.
template <int BM, int NWT, int KC, bool GEGLU, int ACT>
__device__ __forceinline__ void wsgemm_mainloop(const GemmArgs& a, const GemmTile& td, int fb, int ks,
                                                bf16_t* xs, f32x4_t (&acc)[NWT][BM / 16],
                                                f32x4_t (&accu)[NWT][BM / 16]) {
  constexpr int MW = BM / 16;
  constexpr int KS = KC / 32;          // MFMA k-steps per chunk
  constexpr int LD = KC + 8;           // LDS row pitch (bf16), padded by 16 bytes
  constexpr int VPR = KC / 8;          // 16-byte vectors per row per chunk
  constexpr int NV = BM * VPR;         // vectors per chunk
  constexpr int VPT = (NV + kThreads - 1) / kThreads;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const GroupW gw = group_weights(a, td.group);

#pragma unroll
  for (int i = 0; i < NWT; ++i)
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (GEGLU || ACT == ACT_BF16_SCALED) accu[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  const int kb = ks * a.k_split;
  const int ke = min(a.K, kb + a.k_split);
  const int nchunks = (ke - kb) / KC;
  if (nchunks <= 0) return;

  // activation rows of this tile
  int arow[VPT];
  bool aval[VPT];
#pragma unroll
  for (int q = 0; q < VPT; ++q) {
    const int v = tid + q * kThreads;
    const int r = v / VPR;
    aval[q] = (v < NV) && (r < td.nrows);
    const int orow = td.row0 + (r < td.nrows ? r : 0);
    arow[q] = a.row_map ? a.row_map[orow] : orow;
  }

  // weight tile pointers of this wave
  const bf16_t* wp0[NWT];
  const bf16_t* wp1[NWT];
  bool wval[NWT];
#pragma unroll
  for (int i = 0; i < NWT; ++i) {
    const int ft = (fb * 4 + wave) * NWT + i;
    wval[i] = ft * 16 < a.N;
    const int64_t off = ((int64_t)(wval[i] ? ft : 0) * gw.kt + gw.kt_off) * 512 + lane * 8;
    wp0[i] = gw.w0 + off;
    wp1[i] = GEGLU ? gw.w1 + off : nullptr;
  }

  bf16x8_t wa[2][KS][NWT];
  bf16x8_t wb[2][KS][NWT];
  uint4 xv[VPT];

  auto load_w = [&](auto BUF, int k0) {
    constexpr int buf = decltype(BUF)::value;
    const int kt0 = k0 >> 5;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < NWT; ++i) {
        if (wval[i]) {
          wa[buf][s][i] = *reinterpret_cast<const bf16x8_t*>(wp0[i] + (int64_t)(kt0 + s) * 512);
          if constexpr (GEGLU) wb[buf][s][i] = *reinterpret_cast<const bf16x8_t*>(wp1[i] + (int64_t)(kt0 + s) * 512);
        }
      }
  };
  auto load_x = [&](int k0) {
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int v = tid + q * kThreads;
      if (aval[q]) xv[q] = load_act8<ACT>(a, arow[q], k0 + (v % VPR) * 8);
      else xv[q] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int v = tid + q * kThreads;
      if (v < NV) *reinterpret_cast<uint4*>(xs + buf * BM * LD + (v / VPR) * LD + (v % VPR) * 8) = xv[q];
    }
  };
  // one K-chunk: prefetch the next chunk (weights to registers, activations
  // to registers then LDS), MFMAs on the current one
  auto chunk = [&](auto CUR, int c) {
    constexpr int cur = decltype(CUR)::value;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_x(kb + (c + 1) * KC);
      load_w(std::integral_constant<int, cur ^ 1>{}, kb + (c + 1) * KC);
    }
    const bf16_t* xb = xs + cur * BM * LD;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8_t bx[MW];
#pragma unroll
      for (int j = 0; j < MW; ++j)
        bx[j] = *reinterpret_cast<const bf16x8_t*>(xb + (j * 16 + (lane & 15)) * LD + s * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int i = 0; i < NWT; ++i) {
        if (!wval[i]) continue;
#pragma unroll
        for (int j = 0; j < MW; ++j) {
          if constexpr (ACT == ACT_BF16_SCALED) {
            accu[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[cur][s][i], bx[j], accu[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[cur][s][i], bx[j], acc[i][j], 0, 0, 0);
            if constexpr (GEGLU)
              accu[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[cur][s][i], bx[j], accu[i][j], 0, 0, 0);
          }
        }
      }
    }
    if constexpr (ACT == ACT_BF16_SCALED) {
      // end of a 256-wide K tile: acc += scale[row][tile] * partial
      const int kend = kb + (c + 1) * KC;
      if ((kend & 255) == 0) {
        const int tile = (kend >> 8) - 1;
#pragma unroll
        for (int j = 0; j < MW; ++j) {
          const int r = j * 16 + (lane & 15);
          float sc = 0.f;
          if (r < td.nrows) {
            const int orow = td.row0 + r;
            const int ar = a.row_map ? a.row_map[orow] : orow;
            sc = a.act_scale[(int64_t)ar * a.scale_ld + tile];
          }
#pragma unroll
          for (int i = 0; i < NWT; ++i) {
            acc[i][j] += sc * accu[i][j];
            accu[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
    if (more) store_x(cur ^ 1);
    __syncthreads();
  };

  load_x(kb);
  load_w(std::integral_constant<int, 0>{}, kb);
  store_x(0);
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    chunk(std::integral_constant<int, 0>{}, c);
    if (c + 1 < nchunks) chunk(std::integral_constant<int, 1>{}, c + 1);
  }
}

template <int BM, int NWT, int KC, bool GEGLU, int ACT>
__global__ __launch_bounds__(kThreads) void k_wsgemm(GemmArgs a) {
  constexpr int MW = BM / 16;
  constexpr int LD = KC + 8;
  __shared__ __attribute__((aligned(16))) bf16_t xs[2 * BM * LD];

  int tile, fb, ks;
  decode_block(a, xcd_logical_block(a.nblocks), tile, fb, ks);
  if (ks >= a.n_split || fb >= a.n_fb) return;
  const int ntiles = a.tiles ? *a.n_tiles_dev : a.max_tiles;
  if (tile >= ntiles) return;
  GemmTile td;
  if (a.tiles) td = a.tiles[tile];
  else td = GemmTile{0, tile * BM, min(BM, a.M - tile * BM), 0};
  if (td.nrows <= 0) return;

  f32x4_t acc[NWT][MW], accu[NWT][MW];
  wsgemm_mainloop<BM, NWT, KC, GEGLU, ACT>(a, td, fb, ks, xs, acc, accu);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NWT; ++i) {
    const int ft = (fb * 4 + wave) * NWT + i;
    const int n = ft * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      const int r = j * 16 + (lane & 15);
      if (ft * 16 < a.N && r < td.nrows) {
        const int orow = td.row0 + r;
        const f32x4_t g = acc[i][j];
        f32x4_t u = g;
        if constexpr (GEGLU) u = accu[i][j];
        epi_pair<bf16_t>(a, ks, orow, n, g[0], g[1], u[0], u[1]);
        epi_pair<bf16_t>(a, ks, orow, n + 2, g[2], g[3], u[2], u[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// LM head: z = alpha * (h W^T) for a 256-id vocabulary tile per workgroup and
// BM rows, followed by the per-(row, tile) sampler statistics of
// a = z / tau:  m_k = max a,  S_k = sum exp(a - m_k),  T_k = sum exp(a - m_k)(a - m_k),
// zmax_k / argmax (first index), and the in-tile inverse-CDF candidate at the
// row's u2 (first id whose in-tile cumulative mass exceeds u2 * S_k).  The
// logits themselves are never written (except on the test path).
__device__ __forceinline__ void row_tile_stats(const float* zrow, int row, int vt, const LmArgs& lm) {
  const int lane = threadIdx.x & 63;
  const float4 z4 = *reinterpret_cast<const float4*>(zrow + lane * 4);
  const float z[4] = {z4.x, z4.y, z4.z, z4.w};
  // argmax of z, lowest id on ties
  float bz = z[0];
  int bi = 0;
#pragma unroll
  for (int e = 1; e < 4; ++e)
    if (z[e] > bz) { bz = z[e]; bi = e; }
  bi += lane * 4;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float oz = __shfl_xor(bz, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (oz > bz || (oz == bz && oi < bi)) { bz = oz; bi = oi; }
  }
  float av[4], ex[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    av[e] = z[e] * lm.inv_tau;
    mloc = fmaxf(mloc, av[e]);
  }
  const float m = wave_max(mloc);
  float s = 0.f, t = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ex[e] = expf(av[e] - m);
    s += ex[e];
    t += ex[e] * (av[e] - m);
  }
  const float incl = wave_incl_scan(s);
  const float S = __shfl(incl, 63, 64);
  const float T = wave_sum(t);
  // u2 of this row: Philox stream 2, word 1
  const int canvas_id = row / lm.canvas, pos = row - canvas_id * lm.canvas;
  const uint64_t seed = lm.seeds[canvas_id];
  const dg_u32x4 w = dg_philox((uint32_t)pos, (uint32_t)lm.step, (uint32_t)lm.block, DG_STREAM_SAMPLE,
                               (uint32_t)seed, (uint32_t)(seed >> 32));
  const float thr = dg_word_unit(w.y) * S;
  float run = incl - s;
  int hit = -1, lastpos = -1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    run += ex[e];
    if (hit < 0 && run > thr) hit = e;
    if (ex[e] > 0.f) lastpos = e;
  }
  const uint64_t hb = __ballot(hit >= 0);
  int cand;
  if (hb) {
    const int src = __builtin_ctzll(hb);
    cand = __shfl(lane * 4 + hit, src, 64);
  } else {
    const uint64_t pb = __ballot(lastpos >= 0);
    const int src = 63 - __builtin_clzll(pb);
    cand = __shfl(lane * 4 + lastpos, src, 64);
  }
  const int64_t col = (int64_t)vt * 256;
  if (lm.p_side) {
    const int64_t pidx = (int64_t)row * lm.vocab + col + lane * 4;
    if (lm.p_side_f32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(lm.p_side) + pidx) = make_float4(ex[0], ex[1], ex[2], ex[3]);
    } else {
      const uint32_t lo = (uint32_t)f2bf(ex[0]) | ((uint32_t)f2bf(ex[1]) << 16);
      const uint32_t hi = (uint32_t)f2bf(ex[2]) | ((uint32_t)f2bf(ex[3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(lm.p_side) + pidx) = make_uint2(lo, hi);
    }
  }
  if (lm.logits)
    *reinterpret_cast<float4*>(lm.logits + (int64_t)row * lm.vocab + col + lane * 4) = z4;
  if (lane == 0) {
    const int nvt = lm.vocab >> 8;
    lm.part_f[(int64_t)row * nvt + vt] = make_float4(m, S, T, bz);
    lm.part_i[(int64_t)row * nvt + vt] = make_int2((int)col + cand, (int)col + bi);
  }
}

constexpr int LM_KC = 64;
constexpr int LM_ZLD = 256 + 4;  // fp32 pitch of the logit tile in LDS
constexpr int LM_Z_BYTES = 64 * LM_ZLD * 4;

template <int BM>
__global__ __launch_bounds__(kThreads) void k_lmhead(GemmArgs a, LmArgs lm) {
  constexpr int MW = BM / 16;
  constexpr int XS_BYTES = 2 * BM * (LM_KC + 8) * 2;
  constexpr int LDS = XS_BYTES > LM_Z_BYTES ? XS_BYTES : LM_Z_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS];
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem);
  float* zt = reinterpret_cast<float*>(smem);

  int tile, fb, ks;
  decode_block(a, xcd_logical_block(a.nblocks), tile, fb, ks);
  if (fb >= a.n_fb || tile >= a.max_tiles) return;
  const GemmTile td{0, tile * BM, min(BM, a.M - tile * BM), 0};

  f32x4_t acc[4][MW], accu[4][MW];
  wsgemm_mainloop<BM, 4, LM_KC, false, ACT_BF16>(a, td, fb, 0, xs, acc, accu);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // halves of 64 rows through a 64 x 256 fp32 tile in LDS
#pragma unroll
  for (int half = 0; half < BM / 64; ++half) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = wave * 64 + i * 16 + (lane >> 4) * 4;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = half * 4 + jj;
        const int r = jj * 16 + (lane & 15);
        const f32x4_t v = acc[i][j];
        *reinterpret_cast<float4*>(zt + r * LM_ZLD + c) =
            make_float4(a.alpha * v[0], a.alpha * v[1], a.alpha * v[2], a.alpha * v[3]);
      }
    }
    __syncthreads();
    for (int rr = wave; rr < 64; rr += 4) {
      const int r = half * 64 + rr;
      if (r < td.nrows) row_tile_stats(zt + rr * LM_ZLD, td.row0 + r, fb, lm);
    }
    __syncthreads();
  }
}

// Per-(row, tile) statistics straight from fp32 logits (fp32 models and the
// sampler test entry point): one wave per (row, tile).
__global__ __launch_bounds__(kThreads) void k_partials_from_logits(const float* logits, int rows, LmArgs lm) {
  const int nvt = lm.vocab >> 8;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= rows * nvt) return;
  const int row = w / nvt, vt = w - row * nvt;
  row_tile_stats(logits + (int64_t)row * lm.vocab + (int64_t)vt * 256, row, vt, lm);
}

// ---------------------------------------------------------------------------
// fp32 models: plain FMA GEMM, weights row-major [N][K] fp32, two adjacent
// features per thread so RoPE pairs and GeGLU stay in one thread.
constexpr int SIMPLE_BM = 16;

__global__ __launch_bounds__(kThreads) void k_gemm_simple(GemmArgs a) {
  const int np = blockIdx.x * 64 + (threadIdx.x & 63);  // feature pair
  const int n = np * 2;
  const int tile = blockIdx.y, ks = blockIdx.z;
  const int ntiles = a.tiles ? *a.n_tiles_dev : a.max_tiles;
  if (tile >= ntiles || n >= a.N) return;
  GemmTile td;
  if (a.tiles) td = a.tiles[tile];
  else td = GemmTile{0, tile * SIMPLE_BM, min(SIMPLE_BM, a.M - tile * SIMPLE_BM), 0};
  const int g = td.group;
  const float *w0, *w1;
  int64_t ldw;
  int koff;
  if (g < a.n_main) {
    w0 = reinterpret_cast<const float*>(a.w0) + (int64_t)g * a.w_group_stride;
    w1 = a.w1 ? reinterpret_cast<const float*>(a.w1) + (int64_t)g * a.w_group_stride : nullptr;
    ldw = (int64_t)a.kt_main * 32;
    koff = 0;
  } else {
    const int c = g - a.n_main;
    w0 = reinterpret_cast<const float*>(a.w0_alt) + (int64_t)c * a.w_alt_stride;
    w1 = a.w1_alt ? reinterpret_cast<const float*>(a.w1_alt) + (int64_t)c * a.w_alt_stride : nullptr;
    ldw = (int64_t)a.kt_alt * 32;
    koff = c * a.kt_off_alt * 32;
  }
  const int kb = ks * a.k_split, ke = min(a.K, kb + a.k_split);
  for (int r = threadIdx.x >> 6; r < td.nrows; r += 4) {
    const int orow = td.row0 + r;
    const int arow = a.row_map ? a.row_map[orow] : orow;
    const float* x = reinterpret_cast<const float*>(a.act) + (int64_t)arow * a.act_ld;
    const float* xs = a.act_scale ? a.act_scale + (int64_t)arow * a.scale_ld : nullptr;
    float g0 = 0.f, g1 = 0.f, u0 = 0.f, u1 = 0.f;
    for (int k = kb; k < ke; ++k) {
      const float xv = xs ? x[k] * xs[k >> 8] : x[k];
      g0 = fmaf(xv, w0[(int64_t)n * ldw + koff + k], g0);
      g1 = fmaf(xv, w0[(int64_t)(n + 1) * ldw + koff + k], g1);
      if (w1) {
        u0 = fmaf(xv, w1[(int64_t)n * ldw + koff + k], u0);
        u1 = fmaf(xv, w1[(int64_t)(n + 1) * ldw + koff + k], u1);
      }
    }
    epi_pair<float>(a, ks, orow, n, g0, g1, u0, u1);
  }
}

// Logical bf16 [rows][cols] -> weight layout (see the top of this file).  The
// source is row-major [rows][cols], or [cols][rows] when `transposed`.
__global__ __launch_bounds__(kThreads) void k_pack_bf16(bf16_t* dst, const bf16_t* src, int64_t rows, int64_t cols,
                                                       int transposed) {
  const int64_t kt_n = cols / 32;
  const int64_t tiles = (rows / 16) * kt_n;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tiles) return;
  const int lane = threadIdx.x & 63;
  const int64_t nt = t / kt_n, kt = t - nt * kt_n;
  const int64_t r = nt * 16 + (lane & 15);
  const int64_t c = kt * 32 + (lane >> 4) * 8;
  uint4 v;
  if (!transposed) {
    v = *reinterpret_cast<const uint4*>(src + r * cols + c);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)src[(c + 2 * e) * rows + r] | ((uint32_t)src[(c + 2 * e + 1) * rows + r] << 16);
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  *reinterpret_cast<uint4*>(dst + t * 512 + lane * 8) = v;
}

}  // namespace

// ---------------------------------------------------------------------------
static int round8(int n) { return (n + 7) & ~7; }

template <int BM, int NWT, int KC, bool GEGLU>
static void launch_t(const GemmArgs& a0, int act, hipStream_t s) {
  GemmArgs a = a0;
  a.nblocks = round8(a.n_split * a.max_tiles * a.n_fb);
  dim3 grid(a.nblocks);
  if (act == ACT_BF16) hipLaunchKernelGGL((k_wsgemm<BM, NWT, KC, GEGLU, ACT_BF16>), grid, dim3(kThreads), 0, s, a);
  else if (act == ACT_F32) hipLaunchKernelGGL((k_wsgemm<BM, NWT, KC, GEGLU, ACT_F32>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((k_wsgemm<BM, NWT, KC, GEGLU, ACT_BF16_SCALED>), grid, dim3(kThreads), 0, s, a);
}

int launch_wsgemm(const GemmArgs& a, int bm, int nwt, int kc, bool geglu, hipStream_t s) {
  if (a.K % kc != 0 || a.k_split % kc != 0 || a.N % 16 != 0) return -1;
  if (a.act_kind == ACT_BF16_SCALED && (a.k_split % 256 != 0 || a.K % 256 != 0 || geglu)) return -1;
#define DG_CASE(BM_, NWT_, KC_, GG_)                                   \
  if (bm == BM_ && nwt == NWT_ && kc == KC_ && geglu == GG_) {         \
    launch_t<BM_, NWT_, KC_, GG_>(a, a.act_kind, s);                   \
    return hipGetLastError() == hipSuccess ? 0 : -5;                   \
  }
  DG_CASE(128, 1, 64, false)
  DG_CASE(64, 1, 64, false)
  DG_CASE(32, 1, 64, true)
  DG_CASE(32, 1, 128, true)
  DG_CASE(32, 2, 64, false)
  DG_CASE(32, 1, 64, false)
  DG_CASE(64, 2, 64, false)
  DG_CASE(128, 2, 64, false)
  DG_CASE(256, 2, 64, false)
#undef DG_CASE
  return -2;
}

int launch_lmhead(const GemmArgs& a0, const LmArgs& lm, int bm, hipStream_t s) {
  GemmArgs a = a0;
  a.n_split = 1;
  a.nblocks = round8(a.max_tiles * a.n_fb);
  if (bm == 64) hipLaunchKernelGGL(k_lmhead<64>, dim3(a.nblocks), dim3(kThreads), 0, s, a, lm);
  else if (bm == 128) hipLaunchKernelGGL(k_lmhead<128>, dim3(a.nblocks), dim3(kThreads), 0, s, a, lm);
  else return -2;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_gemm_simple(const GemmArgs& a, hipStream_t s) {
  dim3 grid(DG_CEIL_DIV(a.N / 2, 64), a.max_tiles, a.n_split);
  hipLaunchKernelGGL(k_gemm_simple, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_pack_bf16(bf16_t* dst, const bf16_t* src, int64_t rows, int64_t cols, int transposed, hipStream_t s) {
  if (rows % 16 || cols % 32) return -1;
  const int64_t tiles = (rows / 16) * (cols / 32);
  hipLaunchKernelGGL(k_pack_bf16, dim3((unsigned)DG_CEIL_DIV(tiles, 4)), dim3(kThreads), 0, s, dst, src, rows, cols,
                     transposed);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_lm_partials_from_logits(const float* logits, int rows, const LmArgs& lm, hipStream_t s) {
  const int64_t waves = (int64_t)rows * (lm.vocab >> 8);
  hipLaunchKernelGGL(k_partials_from_logits, dim3((unsigned)DG_CEIL_DIV(waves, 4)), dim3(kThreads), 0, s,
                     logits, rows, lm);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
