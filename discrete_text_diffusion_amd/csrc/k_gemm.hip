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
#include <string.h>

#include <type_traits>

#include "dg_internal.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int xcd_logical_block(int nblocks) {
  const int hw = blockIdx.x;
  const int per = nblocks >> 3;
  return (hw & 7) * per + (hw >> 3);
}

// The workgroup's (row tile, feature block, split), or false if it has
// none.  The grid covers max_tiles row tiles; a grouped GEMM's tile list
// holds only *n_tiles_dev of them, known on the device.  The valid workgroups
// are dealt to the 8 XCDs in equal contiguous shares (hardware block b runs on
// XCD b % 8), so every XCD gets the same amount of work and neighbouring
// logical blocks (data they share) stay on one XCD.  Inside a share the split
// is outermost, then
//  * group_major (grouped GEMMs): group by group (a group's tiles are
//    contiguous in the list), feature block by feature block inside a group,
//    the group's row tiles fastest.  Group g owns blocks
//    [n_fb first_g, n_fb (first_g + count_g)), so tile r / n_fb of block r is
//    one of g's and carries g's span;
//  * otherwise (tile, feature block) with the one tile_fastest names fastest.
template <int BM>
__device__ __forceinline__ bool block_work(const GemmArgs& a, GemmTile& td, int& fb, int& ks) {
  const int ntiles = a.tiles ? *a.n_tiles_dev : a.max_tiles;
  const int valid = a.n_split * ntiles * a.n_fb;
  const int share = (valid + 7) >> 3;
  const int i = blockIdx.x >> 3;
  const int lb = (blockIdx.x & 7) * share + i;
  if (i >= share || lb >= valid) return false;
  const int per_split = ntiles * a.n_fb;
  ks = lb / per_split;
  const int r = lb - ks * per_split;
  if (a.group_major) {
    td = a.tiles[r / a.n_fb];
    const int first = (int)((uint32_t)td.span >> 16), count = td.span & 0xffff;
    const int local = r - a.n_fb * first;
    fb = local / count;
    if (count > 1) td = a.tiles[first + (local - fb * count)];
    return true;
  }
  // (selects of values: a select between the two references made the
  // compiler round-trip them through scratch memory)
  const int fast = a.tile_fastest ? ntiles : a.n_fb;
  const int lo = r % fast, hi = r / fast;
  const int tile = a.tile_fastest ? lo : hi;
  fb = a.tile_fastest ? hi : lo;
  if (a.tiles) td = a.tiles[tile];
  else td = GemmTile{0, tile * BM, min(BM, a.M - tile * BM), 0};
  return true;
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
    case EPI_GEGLU_PARTS: {
      float* o = a.out_f32 + (int64_t)ks * a.split_stride + (int64_t)orow * a.ldo + n;
      *reinterpret_cast<float2*>(o) = make_float2(g0, g1);
      *reinterpret_cast<float2*>(o + (int64_t)a.n_split * a.split_stride) = make_float2(u0, u1);
      break;
    }
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
        // RoPE on (2j, 2j+1) of the head at absolute position pos0 + i, the
        // rotation read from the call's table (rope_cs)
        const int j = (n % q.d_head) >> 1;
        const float2 cs = q.rope[(int64_t)i * (q.d_head >> 1) + j];
        v0 = g0 * cs.x - g1 * cs.y;
        v1 = g0 * cs.y + g1 * cs.x;
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
        } else {  // V is stored transposed, [d_head][rows], in the activation type
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

// RoPE rotation of pair j of a d_head-wide head at position pos: angle
// pos * base^(-2j / d_head), formed in fp64 so long positions keep full
// accuracy, (cos, sin) rounded to fp32.
__device__ __forceinline__ float2 rope_cs(int pos, int j, int d_head, float base) {
  const double inv_freq = exp2(-(2.0 * j / d_head) * log2((double)base));
  const double ang = (double)pos * inv_freq;
  double sd, cd;
  sincos(ang, &sd, &cd);
  return make_float2((float)cd, (float)sd);
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
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.act) + (int64_t)arow * a.act_ld + k);
    const float4 x = p[0], y = p[1];
    const float f[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    return pack8_bf16(f);
  }
}

struct GroupW {
  const char* w0;  // first byte of the group's (packed) matrix
  const char* w1;
  const float* s0;  // fp8: per-feature scales of the group (null otherwise)
  const float* s1;
  int kt, kt_off;
};

// Weight formats of the streaming kernel.
constexpr int WF_BF16 = 0, WF_FP8 = 1, WF_MX4 = 2;

// Bytes of `elems` weights in format wf (MXFP4: 17 bytes per 32 weights, 16
// of E2M1 codes and one scale; elems is a multiple of 16 x 64).
__device__ __forceinline__ int64_t weight_bytes(int64_t elems, int wf) {
  return wf == WF_MX4 ? elems / 32 * 17 : elems * (wf == WF_FP8 ? 1 : 2);
}

// Weight and scale bases of group g (an expert, or a shared-expert slice).
__device__ __forceinline__ GroupW group_weights(const GemmArgs& a, int g, int wf) {
  GroupW r;
  if (g < a.n_main) {
    r.w0 = reinterpret_cast<const char*>(a.w0) + weight_bytes((int64_t)g * a.w_group_stride, wf);
    r.w1 = a.w1 ? reinterpret_cast<const char*>(a.w1) + weight_bytes((int64_t)g * a.w_group_stride, wf) : nullptr;
    r.s0 = a.ws0 ? a.ws0 + (int64_t)g * a.ws_group_stride : nullptr;
    r.s1 = a.ws1 ? a.ws1 + (int64_t)g * a.ws_group_stride : nullptr;
    r.kt = a.kt_main;
    r.kt_off = 0;
  } else {
    const int c = g - a.n_main;
    r.w0 = reinterpret_cast<const char*>(a.w0_alt) + weight_bytes((int64_t)c * a.w_alt_stride, wf);
    r.w1 = a.w1_alt ? reinterpret_cast<const char*>(a.w1_alt) + weight_bytes((int64_t)c * a.w_alt_stride, wf)
                    : nullptr;
    r.s0 = a.ws0_alt ? a.ws0_alt + (int64_t)c * a.ws_alt_stride : nullptr;
    r.s1 = a.ws1_alt ? a.ws1_alt + (int64_t)c * a.ws_alt_stride : nullptr;
    r.kt = a.kt_alt;
    r.kt_off = c * a.kt_off_alt;
  }
  return r;
}

// Weight operand registers per 32-wide K step: one 16-byte bf16 fragment, or
// 8 fp8 codes converted to bf16 when the MFMA consumes them.  MXFP4 holds one
// 64-wide superblock per two K steps (entry s / 2): the lane's 8 bytes of E2M1
// codes (K step 2j in .q.x, 2j + 1 in .q.y) and its row's two scale codes
// (low byte for step 2j).
struct Mx4Frag {
  uint2 q;
  uint32_t s;
};
template <int WF> struct WFrag { typedef bf16x8_t type; };
template <> struct WFrag<WF_FP8> { typedef uint2 type; };
template <> struct WFrag<WF_MX4> { typedef Mx4Frag type; };
__device__ __forceinline__ bf16x8_t wfrag_bf16(bf16x8_t w) { return w; }
__device__ __forceinline__ bf16x8_t wfrag_bf16(uint2 w) { return fp8x8_to_bf16(w); }

// Main loop of the weight-streaming kernel.  WS: stages of
// the weight register ring (weights are loaded WS - 1 chunks ahead of their
// MFMAs); activations are always one chunk ahead, double buffered in LDS.
template <int BM, int NWT, int KC, bool GEGLU, int ACT, int WF = WF_BF16, int WS = 2>
__device__ __forceinline__ void wsgemm_mainloop(const GemmArgs& a, const GemmTile& td, const GroupW& gw, int fb,
                                                int ks, bf16_t* xs, f32x4_t (&acc)[NWT][BM / 16],
                                                f32x4_t (&accu)[NWT][BM / 16]) {
  constexpr int MW = BM / 16;
  constexpr int KS = KC / 32;          // MFMA k-steps per chunk
  constexpr int LD = KC + 8;           // LDS row pitch (bf16), padded by 16 bytes
  constexpr int VPR = KC / 8;          // 16-byte vectors per row per chunk
  constexpr int NV = BM * VPR;         // vectors per chunk
  constexpr int VPT = (NV + kThreads - 1) / kThreads;

  constexpr bool FP8 = WF == WF_FP8, MX4 = WF == WF_MX4;
  static_assert(!MX4 || KC % 64 == 0, "MXFP4 chunks are whole 64-wide superblocks");
  constexpr int TILE_B = FP8 ? 512 : 1024;  // bytes of one 16 x 32 weight tile
  constexpr int LANE_B = FP8 ? 8 : 16;      // bytes of one lane's fragment
  constexpr int SB_B = 544;                 // MXFP4: one 16 x 64 superblock
  using W_t = typename WFrag<WF>::type;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

#pragma unroll
  for (int i = 0; i < NWT; ++i)
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (GEGLU) accu[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
  const char* wp0[NWT];
  const char* wp1[NWT];
  bool wval[NWT];
#pragma unroll
  for (int i = 0; i < NWT; ++i) {
    const int ft = (fb * 4 + wave) * NWT + i;
    wval[i] = ft * 16 < a.N;
    const int64_t off = MX4 ? ((int64_t)(wval[i] ? ft : 0) * (gw.kt >> 1) + (gw.kt_off >> 1)) * SB_B + lane * 8
                            : ((int64_t)(wval[i] ? ft : 0) * gw.kt + gw.kt_off) * TILE_B + lane * LANE_B;
    wp0[i] = gw.w0 + off;
    wp1[i] = GEGLU ? gw.w1 + off : nullptr;
  }

  W_t wa[WS][KS][NWT];
  W_t wb[WS][KS][NWT];
  uint4 xv[VPT];

  // Every global load is unconditional: invalid feature tiles read tile 0,
  // rows past the tile read its first row (zeroed when staged), and the
  // prefetches past the last chunk re-read the last chunk.  Loads issued on
  // every path keep the compiler's wait counts exact; a load under a branch
  // makes it wait, conservatively, for the next chunk's loads before the
  // current chunk's MFMAs.
  // MXFP4: the lane's scale codes sit 512 + 2 (row) bytes into the superblock
  const int sofs = 512 - lane * 8 + 2 * (lane & 15);
  auto load_w = [&](auto BUF, int k0) {
    constexpr int buf = decltype(BUF)::value;
    if constexpr (MX4) {
      const int sb0 = k0 >> 6;
#pragma unroll
      for (int s = 0; s < KS / 2; ++s)
#pragma unroll
        for (int i = 0; i < NWT; ++i) {
          const char* p = wp0[i] + (int64_t)(sb0 + s) * SB_B;
          wa[buf][s][i].q = *reinterpret_cast<const uint2*>(p);
          wa[buf][s][i].s = *reinterpret_cast<const uint16_t*>(p + sofs);
          if constexpr (GEGLU) {
            const char* p1 = wp1[i] + (int64_t)(sb0 + s) * SB_B;
            wb[buf][s][i].q = *reinterpret_cast<const uint2*>(p1);
            wb[buf][s][i].s = *reinterpret_cast<const uint16_t*>(p1 + sofs);
          }
        }
    } else {
      const int kt0 = k0 >> 5;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int i = 0; i < NWT; ++i) {
          wa[buf][s][i] = *reinterpret_cast<const W_t*>(wp0[i] + (int64_t)(kt0 + s) * TILE_B);
          if constexpr (GEGLU) wb[buf][s][i] = *reinterpret_cast<const W_t*>(wp1[i] + (int64_t)(kt0 + s) * TILE_B);
        }
    }
  };
  auto load_x = [&](int k0) {
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int v = tid + q * kThreads;
      xv[q] = load_act8<ACT>(a, arow[q], k0 + (v % VPR) * 8);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int v = tid + q * kThreads;
      const uint4 x = aval[q] ? xv[q] : make_uint4(0, 0, 0, 0);
      if (v < NV) *reinterpret_cast<uint4*>(xs + buf * BM * LD + (v / VPR) * LD + (v % VPR) * 8) = x;
    }
  };
  // one K-chunk: prefetch (activations of chunk c + 1 to registers then LDS,
  // weights of chunk c + WS - 1 to registers), MFMAs on chunk c
  auto chunk = [&](auto CUR, int c) {
    constexpr int cur = decltype(CUR)::value;  // weight stage of chunk c
    load_x(kb + min(c + 1, nchunks - 1) * KC);
    load_w(std::integral_constant<int, (cur + WS - 1) % WS>{}, kb + min(c + WS - 1, nchunks - 1) * KC);
    const bf16_t* xb = xs + (c & 1) * BM * LD;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8_t bx[MW];
#pragma unroll
      for (int j = 0; j < MW; ++j)
        bx[j] = *reinterpret_cast<const bf16x8_t*>(xb + (j * 16 + (lane & 15)) * LD + s * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int i = 0; i < NWT; ++i) {
        if (!wval[i]) continue;
        bf16x8_t wai, wbi;
        if constexpr (MX4) {
          const Mx4Frag fa = wa[cur][s >> 1][i];
          wai = mx4x8_to_bf16((s & 1) ? fa.q.y : fa.q.x, ((s & 1) ? fa.s >> 8 : fa.s) & 0xffu);
          wbi = wai;
          if constexpr (GEGLU) {
            const Mx4Frag fb_ = wb[cur][s >> 1][i];
            wbi = mx4x8_to_bf16((s & 1) ? fb_.q.y : fb_.q.x, ((s & 1) ? fb_.s >> 8 : fb_.s) & 0xffu);
          }
        } else {
          wai = wfrag_bf16(wa[cur][s][i]);
          wbi = wai;
          if constexpr (GEGLU) wbi = wfrag_bf16(wb[cur][s][i]);
        }
#pragma unroll
        for (int j = 0; j < MW; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wai, bx[j], acc[i][j], 0, 0, 0);
          if constexpr (GEGLU) accu[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wbi, bx[j], accu[i][j], 0, 0, 0);
        }
      }
    }
    store_x((c + 1) & 1);
    __syncthreads();
  };

  load_x(kb);
  load_w(std::integral_constant<int, 0>{}, kb);
  if constexpr (WS > 2) load_w(std::integral_constant<int, 1>{}, kb + min(1, nchunks - 1) * KC);
  if constexpr (WS > 3) load_w(std::integral_constant<int, 2>{}, kb + min(2, nchunks - 1) * KC);
  static_assert(WS >= 2 && WS <= 4, "weight ring of 2 to 4 stages");
  store_x(0);
  __syncthreads();
  for (int c = 0; c < nchunks; c += WS) {
    chunk(std::integral_constant<int, 0>{}, c);
    if (c + 1 < nchunks) chunk(std::integral_constant<int, 1>{}, c + 1);
    if constexpr (WS > 2) {
      if (c + 2 < nchunks) chunk(std::integral_constant<int, 2>{}, c + 2);
    }
    if constexpr (WS > 3) {
      if (c + 3 < nchunks) chunk(std::integral_constant<int, 3>{}, c + 3);
    }
  }
}

// Epilogue of a 4-wave streaming workgroup: wave w holds features
// ((fb * 4 + w) * NWT + i) * 16 + 4 (lane / 16) + e of rows j * 16 + lane % 16.
template <int BM, int NWT, bool GEGLU, int WF>
__device__ __forceinline__ void ws_epilogue(const GemmArgs& a, const GemmTile& td, const GroupW& gw, int fb, int ks,
                                            const f32x4_t (&acc)[NWT][BM / 16], const f32x4_t (&accu)[NWT][BM / 16]) {
  constexpr int MW = BM / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NWT; ++i) {
    const int ft = (fb * 4 + wave) * NWT + i;
    const int n = ft * 16 + (lane >> 4) * 4;
    // fp8: per-feature scales of the four features this lane holds
    f32x4_t sg = f32x4_t{1.f, 1.f, 1.f, 1.f}, su = sg;
    constexpr bool FP8 = WF == WF_FP8;
    if constexpr (FP8) {
      if (ft * 16 < a.N) {
        const float4 v0 = *reinterpret_cast<const float4*>(gw.s0 + n);
        sg = f32x4_t{v0.x, v0.y, v0.z, v0.w};
        if constexpr (GEGLU) {
          const float4 v1 = *reinterpret_cast<const float4*>(gw.s1 + n);
          su = f32x4_t{v1.x, v1.y, v1.z, v1.w};
        }
      }
    }
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      const int r = j * 16 + (lane & 15);
      if (ft * 16 < a.N && r < td.nrows) {
        const int orow = td.row0 + r;
        f32x4_t g = acc[i][j];
        f32x4_t u = g;
        if constexpr (GEGLU) u = accu[i][j];
        if constexpr (FP8) {
          g *= sg;
          u *= su;
        }
        epi_pair<bf16_t>(a, ks, orow, n, g[0], g[1], u[0], u[1]);
        epi_pair<bf16_t>(a, ks, orow, n + 2, g[2], g[3], u[2], u[3]);
      }
    }
  }
}

// 32-row tiles are held to 128 registers (four workgroups per CU): they fit
// without spilling, and the extra waves keep more weight loads in flight
// (MXFP4 down projection 52 -> 44 us); taller tiles keep their registers.
template <int BM, int NWT, int KC, bool GEGLU, int ACT, int WF, int WS = 2>
__global__ __launch_bounds__(kThreads, BM <= 32 ? 4 : 1) void k_wsgemm(GemmArgs a) {
  constexpr int MW = BM / 16;
  constexpr int LD = KC + 8;
  __shared__ __attribute__((aligned(16))) bf16_t xs[2 * BM * LD];

  GemmTile td;
  int fb, ks;
  if (!block_work<BM>(a, td, fb, ks)) return;
  if (td.nrows <= 0) return;

  f32x4_t acc[NWT][MW], accu[NWT][MW];
  const GroupW gw = group_weights(a, td.group, WF);
  wsgemm_mainloop<BM, NWT, KC, GEGLU, ACT, WF, WS>(a, td, gw, fb, ks, xs, acc, accu);

  ws_epilogue<BM, NWT, GEGLU, WF>(a, td, gw, fb, ks, acc, accu);
}

// ---------------------------------------------------------------------------
// LM head: z = alpha * (h W^T) for a 256-id vocabulary tile per workgroup and
// BM rows, followed by the per-(row, tile) sampler statistics of
// a = z / tau:  m_k = max a,  S_k = sum exp(a - m_k),  T_k = sum exp(a - m_k)(a - m_k),
// zmax_k / argmax (first index), and the in-tile inverse-CDF candidate at the
// row's u2 (first id whose in-tile cumulative mass exceeds u2 * S_k).  The
// logits themselves are never written (except on the test path).
// u2 of a row: Philox stream 2 (sampling), word 1, at (position, step, block).
__device__ __forceinline__ float row_u2_seeded(int row, uint64_t seed, const LmArgs& lm) {
  const int pos = row % lm.canvas;
  const dg_u32x4 w = dg_philox((uint32_t)pos, (uint32_t)lm.step, (uint32_t)lm.block, DG_STREAM_SAMPLE,
                               (uint32_t)seed, (uint32_t)(seed >> 32));
  return dg_word_unit(w.y);
}
__device__ __forceinline__ float row_u2(int row, const LmArgs& lm) {
  return row_u2_seeded(row, lm.seeds[row / lm.canvas], lm);
}

// Cross-lane steps inside one 16-lane DPP row.  The butterfly pairs (xor 1,
// xor 2, then the half-row and row mirrors) combine groups that already hold
// identical partials, so every lane of the row ends with the bitwise-same
// result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
constexpr int DPP_SHR1 = 0x111, DPP_SHR2 = 0x112, DPP_SHR4 = 0x114, DPP_SHR8 = 0x118;

__device__ __forceinline__ float row16_sum(float x) {
  x = x + dpp_f<DPP_XOR1>(x);
  x = x + dpp_f<DPP_XOR2>(x);
  x = x + dpp_f<DPP_HALF_MIRROR>(x);
  return x + dpp_f<DPP_MIRROR>(x);
}
__device__ __forceinline__ int row16_max(int x) {
  x = max(x, dpp_i<DPP_XOR1>(x));
  x = max(x, dpp_i<DPP_XOR2>(x));
  x = max(x, dpp_i<DPP_HALF_MIRROR>(x));
  return max(x, dpp_i<DPP_MIRROR>(x));
}
// inclusive prefix sum over the lanes of a row (lanes before the row's first read 0)
__device__ __forceinline__ float row16_incl_scan(float x) {
  x = x + dpp_f<DPP_SHR1>(x);
  x = x + dpp_f<DPP_SHR2>(x);
  x = x + dpp_f<DPP_SHR4>(x);
  return x + dpp_f<DPP_SHR8>(x);
}

// Statistics of four rows x one 256-id tile per wave: lane l works on row
// l / 16 and the 16 ids 64 q + 4 (l % 16) + e (q, e < 4), read as four
// float4 whose 16 lanes cover 256 contiguous bytes each.  z0: row 0 of the
// group, rows `pitch` floats apart; rows >= nrows are not written.  u2: the
// sampling uniform of this lane's row.
__device__ __forceinline__ void tile_stats4(const float* z0, int64_t pitch, int nrows, int row0, int vt,
                                            const LmArgs& lm, float u2) {
  const int lane = threadIdx.x & 63, r = lane >> 4, sl = lane & 15;
  const float* zr = z0 + (int64_t)min(r, nrows - 1) * pitch + 4 * sl;
  float z[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(zr + 64 * q);
    z[4 * q] = v.x; z[4 * q + 1] = v.y; z[4 * q + 2] = v.z; z[4 * q + 3] = v.w;
  }
  // zmax and its first id (k runs over this lane's ids in increasing order)
  float bz = z[0];
  int bc = 4 * sl;
#pragma unroll
  for (int k = 1; k < 16; ++k)
    if (z[k] > bz) { bz = z[k]; bc = 64 * (k >> 2) + 4 * sl + (k & 3); }
  auto argmax_step = [&](float oz, int oc) {
    if (oz > bz || (oz == bz && oc < bc)) { bz = oz; bc = oc; }
  };
  argmax_step(dpp_f<DPP_XOR1>(bz), dpp_i<DPP_XOR1>(bc));
  argmax_step(dpp_f<DPP_XOR2>(bz), dpp_i<DPP_XOR2>(bc));
  argmax_step(dpp_f<DPP_HALF_MIRROR>(bz), dpp_i<DPP_HALF_MIRROR>(bc));
  argmax_step(dpp_f<DPP_MIRROR>(bz), dpp_i<DPP_MIRROR>(bc));
  // a = z / tau (tau > 0, so max a = round(zmax / tau)); exp(a - m) and moments
  // exp(d) = 2^(d log2 e) on the hardware exp2 (about 1 ulp): the epilogue is
  // VALU-bound, and the statistics it feeds carry looser tolerances
  const float m = bz * lm.inv_tau;
  float ex[16], w[4];
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float d = z[k] * lm.inv_tau - m;
    ex[k] = __builtin_amdgcn_exp2f(d * 1.4426950408889634f);
    t = fmaf(ex[k], d, t);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = (ex[4 * q] + ex[4 * q + 1]) + (ex[4 * q + 2] + ex[4 * q + 3]);
  const float S = row16_sum((w[0] + w[1]) + (w[2] + w[3]));
  const float T = row16_sum(t);
  // inverse CDF inside the tile: first id whose cumulative mass exceeds u2 S,
  // walking 64-id blocks, then lanes, then the lane's four ids
  const float thr = u2 * S;
  float base = 0.f;
  int qs = -1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float bq = row16_sum(w[q]);
    if (qs < 0) {
      if (base + bq > thr) qs = q;
      else base += bq;
    }
  }
  int cand = -1;
  if (qs >= 0) {
    const float wq = qs == 0 ? w[0] : qs == 1 ? w[1] : qs == 2 ? w[2] : w[3];
    const float incl = row16_incl_scan(wq);
    const uint64_t hits = __ballot(base + incl > thr);
    const uint32_t rowhits = (uint32_t)(hits >> (16 * r)) & 0xFFFFu;
    if (rowhits && sl == __builtin_ctz(rowhits)) {
      float run = base + (incl - wq);
      int e_hit = -1, e_last = -1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = qs == 0 ? ex[e] : qs == 1 ? ex[4 + e] : qs == 2 ? ex[8 + e] : ex[12 + e];
        run += x;
        if (e_hit < 0 && run > thr) e_hit = e;
        if (x > 0.f) e_last = e;
      }
      const int e = e_hit >= 0 ? e_hit : e_last;
      if (e >= 0) cand = 64 * qs + 4 * sl + e;
    }
    cand = row16_max(cand);
  }
  if (cand < 0) {  // mass never exceeded u2 S (rounding): last id with mass
    int lastc = -1;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (ex[k] > 0.f) lastc = max(lastc, 64 * (k >> 2) + 4 * sl + (k & 3));
    cand = row16_max(lastc);
  }
  if (cand < 0) cand = bc;  // no id with mass at all (non-finite logits): the argmax, still a valid id
  if (r >= nrows) return;
  const int row = row0 + r;
  const int64_t col = (int64_t)vt * 256;
  if (lm.p_side) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t pidx = (int64_t)row * lm.vocab + col + 64 * q + 4 * sl;
      if (lm.p_side_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(lm.p_side) + pidx) =
            make_float4(ex[4 * q], ex[4 * q + 1], ex[4 * q + 2], ex[4 * q + 3]);
      } else {
        // hardware round-to-nearest-even conversion (v_cvt_pk_bf16_f32)
        const bf16x2_t lo = {(__bf16)ex[4 * q], (__bf16)ex[4 * q + 1]};
        const bf16x2_t hi = {(__bf16)ex[4 * q + 2], (__bf16)ex[4 * q + 3]};
        *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(lm.p_side) + pidx) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
    }
  }
  if (lm.logits) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(lm.logits + (int64_t)row * lm.vocab + col + 64 * q + 4 * sl) =
          make_float4(z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]);
  }
  if (sl == 0) {
    const int nvt = lm.vocab >> 8;
    lm.part_f[(int64_t)row * nvt + vt] = make_float4(m, S, T, bz);
    lm.part_i[(int64_t)row * nvt + vt] = make_int2((int)col + cand, (int)col + bc);
  }
}

constexpr int LM_ZLD = 256 + 4;  // fp32 pitch of the logit tile in LDS

// ---------------------------------------------------------------------------
// Row-resident GEMM for dense weights and few rows (the denoiser's canvas):
// one workgroup of 8 waves holds all (up to 256) rows of a row group for a
// block of BN features, so a weight byte is read once per row group and K
// split.  Wave w covers rows [128 (w / 4), +128) and features
// [NWT 16 (w % 4), +NWT 16) of the block (8 x NWT accumulator tiles, two
// waves per SIMD).  Per 32-wide K chunk a wave reads 8 KiB of activations and
// NWT KiB of weights from LDS for 8 NWT MFMAs.
//
// Both operands go straight from memory into a ring of RG_AHEAD + 1 LDS
// stages with global_load_lds_dwordx4 (lane l of an instruction lands at
// base + 16 l), RG_AHEAD chunks ahead of the MFMAs:
//  * activations: one instruction fills 16 rows x 64 B; the 16-byte column
//    groups of a row are XOR-swizzled by (row / 2) % 4, which keeps the
//    B-operand reads free of bank conflicts;
//  * weights: one instruction moves one packed 16 x 32 tile (1 KiB), already
//    in A-operand lane order.
// Memory counters complete in issue order, so one wait per chunk (for the
// loads issued RG_AHEAD chunks earlier) and one barrier (the other waves'
// parts of that stage) cover both.  Every load is unconditional (out-of-range
// rows and chunks load clamped, in-bounds addresses that are never used),
// which keeps the counts exact; a wave with extra loads in flight only waits
// longer.
//
// Variants (256 features per workgroup):
//  * plain: fp32 partials out_f32[split][row][n] = alpha acc;
//  * LM head: the sampler statistics of each 256-id tile instead.
constexpr int RG_THREADS = 512;
constexpr int RG_ROWS = 256;
constexpr int RG_KC = 32;
constexpr int RG_AHEAD = 3;                          // prefetch distance (chunks)
constexpr int RG_SLOTS = RG_AHEAD + 1;
constexpr int RG_ROW_BYTES = RG_KC * 2;              // 64 B, no padding (swizzled)
constexpr int RG_X_BYTES = RG_ROWS * RG_ROW_BYTES;   // activations of one chunk (16 KiB)
constexpr int RG_XDMA = RG_ROWS / 16 / 8;            // activation instructions per wave per chunk
constexpr int RG_ZROWS = 128;                        // LM head: logit rows staged at a time

template <bool LMHEAD, bool FP8>
struct RgCfg {
  static constexpr int NWT = 4;
  static constexpr int BN = 4 * NWT * 16;                  // features per workgroup
  static constexpr int WTILE = FP8 ? 512 : 1024;           // bytes of a 16 x 32 weight tile
  static constexpr int WDMA = BN / 16 * WTILE / 1024 / 8;  // 1 KiB weight loads per wave per chunk
  static constexpr int LOADS = RG_XDMA + WDMA;             // loads per wave per chunk
  static constexpr int STAGE = RG_X_BYTES + BN / 16 * WTILE;  // activations + weight tiles
  static constexpr int RING = RG_SLOTS * STAGE;
  static constexpr int BODY = LMHEAD && RG_ZROWS * LM_ZLD * 4 > RING ? RG_ZROWS * LM_ZLD * 4 : RING;
  static constexpr int EXTRA = LMHEAD ? RG_ROWS * 4 : 0;  // per-row uniforms
  static constexpr int LDS = BODY + EXTRA;
};

__device__ __forceinline__ int rg_swz(int row) { return (row >> 1) & 3; }

typedef __attribute__((address_space(3))) void lds_void_t;

// Main-loop pieces of the row-resident kernel.  A "group" is two of a wave's
// eight 16-row tiles; its MFMAs read two B fragments.
template <int G>
__device__ __forceinline__ void rg_read_x(const unsigned char* st, int rh, int lane, bf16x8_t (&x)[2]) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int r = rh * 128 + (2 * G + jj) * 16 + (lane & 15);
    x[jj] = *reinterpret_cast<const bf16x8_t*>(st + r * RG_ROW_BYTES + (((lane >> 4) ^ rg_swz(r)) << 4));
  }
}
template <int NWT, bool FP8>
__device__ __forceinline__ void rg_read_w(const unsigned char* st, int cg, int lane, bf16x8_t (&wf)[NWT]) {
#pragma unroll
  for (int i = 0; i < NWT; ++i) {
    if constexpr (FP8)
      wf[i] = fp8x8_to_bf16(*reinterpret_cast<const uint2*>(st + RG_X_BYTES + (cg * NWT + i) * 512 + lane * 8));
    else
      wf[i] = *reinterpret_cast<const bf16x8_t*>(st + RG_X_BYTES + (cg * NWT + i) * 1024 + lane * 16);
  }
}
template <int NWT, int G>
__device__ __forceinline__ void rg_mfma(f32x4_t (&acc)[NWT][8], const bf16x8_t (&wf)[NWT], const bf16x8_t (&x)[2]) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < NWT; ++i)
      acc[i][2 * G + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i], x[jj], acc[i][2 * G + jj], 0, 0, 0);
}

// LM-head epilogue of a 256-row x 256-id block (8 waves; wave w holds rows
// 128 (w / 4) + [0, 128) and ids 64 (w % 4) + [0, 64) in acc): the logits
// z = alpha acc (alpha scale[n] acc for fp8 weights) go through LDS 128 rows
// at a time, then four rows per wave for the sampler statistics.  smem: at
// least RG_ZROWS * LM_ZLD floats, free; u2s: RG_ROWS floats.
template <bool FP8>
__device__ __forceinline__ void rg_lm_epilogue(const GemmArgs& a, const LmArgs& lm, const f32x4_t (&acc)[4][8],
                                               unsigned char* smem, float* u2s, int fb, int row0, int nrows,
                                               uint64_t seed) {
  constexpr int NWT = 4, MW = 8, BN = 256;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rh = wave >> 2, cg = wave & 3;
  if (tid < nrows) u2s[tid] = row_u2_seeded(row0 + tid, seed, lm);  // read after the next barrier
  float* zt = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (rh == half) {
#pragma unroll
      for (int i = 0; i < NWT; ++i) {
        const int col = (cg * NWT + i) * 16 + (lane >> 4) * 4;
        f32x4_t sc = f32x4_t{a.alpha, a.alpha, a.alpha, a.alpha};
        if constexpr (FP8) {
          const float4 w = *reinterpret_cast<const float4*>(a.ws0 + (int64_t)fb * BN + col);
          sc = f32x4_t{a.alpha * w.x, a.alpha * w.y, a.alpha * w.z, a.alpha * w.w};
        }
#pragma unroll
        for (int j = 0; j < MW; ++j) {
          const f32x4_t v = acc[i][j] * sc;
          *reinterpret_cast<float4*>(zt + (j * 16 + (lane & 15)) * LM_ZLD + col) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    __syncthreads();
    for (int rr = wave * 4; rr < RG_ZROWS; rr += 4 * (RG_THREADS / 64)) {
      const int r = half * RG_ZROWS + rr;
      if (r < nrows) {
        const int nr = min(4, nrows - r);
        tile_stats4(zt + rr * LM_ZLD, LM_ZLD, nr, row0 + r, fb, lm, u2s[r + min(lane >> 4, nr - 1)]);
      }
    }
    __syncthreads();
  }
}

template <bool LMHEAD, bool FP8>
__global__ __launch_bounds__(RG_THREADS, 1) void k_rowgemm(GemmArgs a, LmArgs lm) {
  using C = RgCfg<LMHEAD, FP8>;
  constexpr int MW = 8;
  constexpr int NWT = C::NWT;
  // one LDS object (stages / logit tile, then the per-row uniforms or factor
  // ring): a second object makes the compiler wait for every in-flight LDS
  // DMA before each LDS read
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];
  float* extra = reinterpret_cast<float*>(smem + C::BODY);

  const int lb = xcd_logical_block(a.nblocks);
  // order: row group fastest (shares the weights), then feature block (shares
  // the activations of one K split), then split
  const int tile = lb % a.max_tiles;
  const int fb = (lb / a.max_tiles) % a.n_fb;
  const int ks = lb / (a.max_tiles * a.n_fb);
  if (ks >= a.n_split) return;
  const int row0 = tile * RG_ROWS;
  const int nrows = min(RG_ROWS, a.M - row0);
  if (nrows <= 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rh = wave >> 2, cg = wave & 3;
  const int kb = ks * a.k_split;
  const int ke = min(a.K, kb + a.k_split);
  const int nch = (ke - kb) / RG_KC;
  if (nch <= 0) return;

  f32x4_t acc[NWT][MW];
#pragma unroll
  for (int i = 0; i < NWT; ++i)
#pragma unroll
    for (int j = 0; j < MW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  bool wval[NWT];
#pragma unroll
  for (int i = 0; i < NWT; ++i) wval[i] = (fb * (C::BN / 16) + cg * NWT + i) * 16 < a.N;
  // 1 KiB weight loads of this wave: load u = WDMA wave + e moves block tile u
  // (bf16), or tiles 2u and 2u + 1 (fp8, 32 lanes each); tiles past N reload
  // tile 0.  (Fixed-size array: a template-dependent size captured by the
  // lambda below makes hipcc drop the host-side launch stubs of this kernel.)
  const char* wsrc[2];
  static_assert(C::WDMA <= 2, "weight loads per wave per chunk");
  // (a member of C named inside the lambda also drops the launch stubs)
  const int64_t wstep = C::WTILE;
#pragma unroll
  for (int e = 0; e < C::WDMA; ++e) {
    const int u = wave * C::WDMA + e;
    const int ft = fb * (C::BN / 16) + (FP8 ? 2 * u + (lane >> 5) : u);
    const int lofs = FP8 ? (lane & 31) * 16 : lane * 16;
    wsrc[e] = reinterpret_cast<const char*>(a.w0) +
              ((int64_t)(ft * 16 < a.N ? ft : 0) * a.kt_main + (kb >> 5)) * C::WTILE + lofs;
  }
  // activation instruction d of this wave fills rows (wave*RG_XDMA + d)*16 + lane/4,
  // physical column group lane%4 <- logical group (lane%4) ^ swz(row)
  const bf16_t* xsrc[RG_XDMA];
#pragma unroll
  for (int d = 0; d < RG_XDMA; ++d) {
    const int r = (wave * RG_XDMA + d) * 16 + (lane >> 2);
    const int g = (lane & 3) ^ rg_swz(r);
    xsrc[d] = reinterpret_cast<const bf16_t*>(a.act) + (int64_t)(row0 + min(r, nrows - 1)) * a.act_ld + kb + g * 8;
  }

  // chunk c's loads (clamped to the last chunk) into stage c % RG_SLOTS
  auto issue = [&](int c) {
    const int cc = min(c, nch - 1);
    unsigned char* st = smem + (c % RG_SLOTS) * C::STAGE;
#pragma unroll
    for (int d = 0; d < RG_XDMA; ++d)
      __builtin_amdgcn_global_load_lds(xsrc[d] + cc * RG_KC, (lds_void_t*)(st + (wave * RG_XDMA + d) * 1024), 16, 0,
                                       0);
#pragma unroll
    for (int e = 0; e < C::WDMA; ++e)
      __builtin_amdgcn_global_load_lds(wsrc[e] + (int64_t)cc * wstep,
                                       (lds_void_t*)(st + RG_X_BYTES + (wave * C::WDMA + e) * 1024), 16, 0, 0);
  };

  // LM head: each row's seed is loaded before the first chunks and used
  // after the main loop has drained, so no wait for it stalls the pipeline
  uint64_t seed = 0;
  if constexpr (LMHEAD) {
    seed = lm.seeds[(row0 + min(tid, nrows - 1)) / lm.canvas];
    asm volatile("" ::: "memory");  // issue it before the chunk loads
  }
  for (int c = 0; c < RG_AHEAD; ++c) issue(c);
  // Own loads of a chunk done, then a plain barrier: every wave's part of the
  // stage is in LDS.  No fence: it would wait for the loads still in flight;
  // the asm memory clobber keeps the compiler from moving LDS accesses across.
  // Operand reads run one group ahead of the MFMAs, and the wait + barrier
  // for chunk c + 1 come before chunk c's last group, so chunk c + 1's first
  // reads overlap those MFMAs.  lgkmcnt(0) before that barrier: every read of
  // chunk c has completed, so chunk c + 1 + RG_AHEAD may refill its stage.
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((RG_AHEAD - 1) * C::LOADS) : "memory");
  issue(RG_AHEAD);
  bf16x8_t wf[NWT], wn[NWT], xa[2], xb[2];
  rg_read_w<NWT, FP8>(smem, cg, lane, wf);
  rg_read_x<0>(smem, rh, lane, xa);
  // (sched_barrier keeps the compiler from sinking each read next to its use)
  for (int c = 0; c < nch; ++c) {
    const unsigned char* st = smem + (c % RG_SLOTS) * C::STAGE;
    rg_read_x<1>(st, rh, lane, xb);
    __builtin_amdgcn_sched_barrier(0);
    rg_mfma<NWT, 0>(acc, wf, xa);
    rg_read_x<2>(st, rh, lane, xa);
    __builtin_amdgcn_sched_barrier(0);
    rg_mfma<NWT, 1>(acc, wf, xb);
    rg_read_x<3>(st, rh, lane, xb);
    __builtin_amdgcn_sched_barrier(0);
    rg_mfma<NWT, 2>(acc, wf, xa);
    if (c + 1 < nch) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((RG_AHEAD - 1) * C::LOADS)
                   : "memory");
      issue(c + 1 + RG_AHEAD);
      const unsigned char* sn = smem + ((c + 1) % RG_SLOTS) * C::STAGE;
      rg_read_w<NWT, FP8>(sn, cg, lane, wn);
      rg_read_x<0>(sn, rh, lane, xa);
    }
    __builtin_amdgcn_sched_barrier(0);
    rg_mfma<NWT, 3>(acc, wf, xb);
#pragma unroll
    for (int i = 0; i < NWT; ++i) wf[i] = wn[i];
  }
  // drain the clamped prefetches before the LDS is reused or the wave ends
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

  if constexpr (!LMHEAD) {
#pragma unroll
    for (int i = 0; i < NWT; ++i) {
      if (!wval[i]) continue;
      const int n = (fb * (C::BN / 16) + cg * NWT + i) * 16 + (lane >> 4) * 4;
#pragma unroll
      for (int j = 0; j < MW; ++j) {
        const int r = rh * 128 + j * 16 + (lane & 15);
        if (r < nrows) {
          const f32x4_t g = acc[i][j];
          *reinterpret_cast<float4*>(a.out_f32 + (int64_t)ks * a.split_stride + (int64_t)(row0 + r) * a.ldo + n) =
              make_float4(a.alpha * g[0], a.alpha * g[1], a.alpha * g[2], a.alpha * g[3]);
        }
      }
    }
  } else {
    rg_lm_epilogue<FP8>(a, lm, acc, smem, extra, fb, row0, nrows, seed);
  }
}

// Sum of K-split partials, then the epilogue (QKV, GELU, activation store).
__global__ __launch_bounds__(kThreads) void k_split_epilogue(GemmArgs a, const float* part, int n_split,
                                                            int64_t split_stride, int ldp) {
  const int64_t pairs = (int64_t)a.M * (a.N >> 1);
  const int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (p >= pairs) return;
  const int row = (int)(p / (a.N >> 1));
  const int n = (int)(p - (int64_t)row * (a.N >> 1)) * 2;
  constexpr int kMaxS = 16;
  float2 v[kMaxS];
#pragma unroll
  for (int s = 0; s < kMaxS; ++s)
    v[s] = s < n_split ? *reinterpret_cast<const float2*>(part + s * split_stride + (int64_t)row * ldp + n)
                       : make_float2(0.f, 0.f);
  float g0 = v[0].x, g1 = v[0].y;
#pragma unroll
  for (int s = 1; s < kMaxS; ++s) {
    g0 += v[s].x;
    g1 += v[s].y;
  }
  epi_pair<bf16_t>(a, 0, row, n, g0, g1, g0, g1);
}

// Per-(row, tile) statistics straight from fp32 logits (fp32 models and the
// sampler test entry point): one wave per (four rows, tile).
__global__ __launch_bounds__(kThreads) void k_partials_from_logits(const float* logits, int rows, LmArgs lm) {
  const int nvt = lm.vocab >> 8;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int groups = (rows + 3) / 4;
  if (w >= groups * nvt) return;
  const int g = w / nvt, vt = w - g * nvt;
  const int row0 = g * 4, nr = min(4, rows - row0);
  const int my_row = row0 + min((int)(threadIdx.x & 63) >> 4, nr - 1);
  tile_stats4(logits + (int64_t)row0 * lm.vocab + (int64_t)vt * 256, lm.vocab, nr, row0, vt, lm, row_u2(my_row, lm));
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
    float g0 = 0.f, g1 = 0.f, u0 = 0.f, u1 = 0.f;
    for (int k = kb; k < ke; ++k) {
      const float xv = x[k];
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

// Logical E4M3 codes [rows][cols] -> fp8 weight layout: 16 x 32 tiles of 512 B,
// tile (nt, kt) at byte (nt * cols / 32 + kt) * 512, lane l's 8 codes (row
// nt*16 + l%16, k = kt*32 + 8(l/16) ...) at byte 8 l of the tile.
__global__ __launch_bounds__(kThreads) void k_pack_fp8(uint8_t* dst, const uint8_t* src, int64_t rows, int64_t cols) {
  const int64_t kt_n = cols / 32;
  const int64_t tiles = (rows / 16) * kt_n;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tiles) return;
  const int lane = threadIdx.x & 63;
  const int64_t nt = t / kt_n, kt = t - nt * kt_n;
  const int64_t r = nt * 16 + (lane & 15);
  const int64_t c = kt * 32 + (lane >> 4) * 8;
  *reinterpret_cast<uint2*>(dst + t * 512 + lane * 8) = *reinterpret_cast<const uint2*>(src + r * cols + c);
}

// Logical MXFP4 element codes [rows][cols] (one per byte) and block scale
// codes [rows][cols / 32] -> MXFP4 weight layout: 16 x 64 superblocks of
// 544 B, superblock (nt, kb) at byte (nt * cols / 64 + kb) * 544; lane l's 8
// bytes at 8 l: the 8 codes (row nt*16 + l%16, k = kb*64 + 32h + 8(l/16) ...)
// of half h in bytes 4h..4h+3, two per byte, lower k in the low nibble; then
// the 16 rows' two scale codes at 512 + 2 (row) + h.  One wave per superblock.
__global__ __launch_bounds__(kThreads) void k_pack_mxfp4(uint8_t* dst, const uint8_t* codes, const uint8_t* scales,
                                                         int64_t rows, int64_t cols) {
  const int64_t sbn = cols / 64;
  const int64_t nsb = (rows / 16) * sbn;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= nsb) return;
  const int lane = threadIdx.x & 63;
  const int64_t nt = t / sbn, kb = t - nt * sbn;
  const int64_t r = nt * 16 + (lane & 15);
  uint8_t* o = dst + t * 544;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint8_t* src = codes + r * cols + kb * 64 + 32 * h + (lane >> 4) * 8;
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) word |= (uint32_t)((src[2 * q] & 15u) | ((src[2 * q + 1] & 15u) << 4)) << (8 * q);
    *reinterpret_cast<uint32_t*>(o + lane * 8 + 4 * h) = word;
  }
  if (lane < 16) {
    const uint8_t* sr = scales + (nt * 16 + lane) * (cols / 32) + kb * 2;
    o[512 + 2 * lane] = sr[0];
    o[512 + 2 * lane + 1] = sr[1];
  }
}

}  // namespace

// ---------------------------------------------------------------------------
static int round8(int n) { return (n + 7) & ~7; }

template <int BM, int NWT, int KC, bool GEGLU, int WS = 2>
static void launch_t(const GemmArgs& a0, int act, hipStream_t s) {
  GemmArgs a = a0;
  a.nblocks = round8(a.n_split * a.max_tiles * a.n_fb);
  dim3 grid(a.nblocks);
  if (act == ACT_BF16) hipLaunchKernelGGL((k_wsgemm<BM, NWT, KC, GEGLU, ACT_BF16, WF_BF16, WS>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((k_wsgemm<BM, NWT, KC, GEGLU, ACT_F32, WF_BF16, WS>), grid, dim3(kThreads), 0, s, a);
}

// quantised weights (fp8 or MXFP4), bf16 activations
template <int BM, int NWT, int KC, bool GEGLU, int WF, int WS = 2>
static void launch_q(const GemmArgs& a0, hipStream_t s) {
  GemmArgs a = a0;
  a.nblocks = round8(a.n_split * a.max_tiles * a.n_fb);
  hipLaunchKernelGGL((k_wsgemm<BM, NWT, KC, GEGLU, ACT_BF16, WF, WS>), dim3(a.nblocks), dim3(kThreads), 0, s, a);
}

int launch_wsgemm(const GemmArgs& a, int bm, int nwt, int kc, bool geglu, hipStream_t s) {
  if (a.K % kc != 0 || a.k_split % kc != 0 || a.N % 16 != 0) return -1;
  if (a.w_fp8) {
    // fp8 weights: bf16 rows, per-feature scales for every group present
    if (a.act_kind != ACT_BF16 || !a.ws0 || (geglu && !a.ws1)) return -1;
    if (a.w0_alt && (!a.ws0_alt || (geglu && !a.ws1_alt))) return -1;
    // float4 scale reads: 16-byte aligned bases and group strides
    if (a.ws_group_stride % 4 || a.ws_alt_stride % 4 || reinterpret_cast<uintptr_t>(a.ws0) % 16 ||
        reinterpret_cast<uintptr_t>(a.ws1) % 16 || reinterpret_cast<uintptr_t>(a.ws0_alt) % 16 ||
        reinterpret_cast<uintptr_t>(a.ws1_alt) % 16)
      return -1;
    if (bm == 32 && nwt == 1 && kc == 128 && geglu) launch_q<32, 1, 128, true, WF_FP8>(a, s);
    else if (bm == 32 && nwt == 2 && kc == 64 && !geglu) launch_q<32, 2, 64, false, WF_FP8>(a, s);
    else return -2;
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  if (a.w_mx4) {
    // MXFP4 weights: whole 64-wide superblocks per chunk and per K split,
    // every group's K offset on a superblock boundary
    if (a.act_kind != ACT_BF16 || kc % 64 || a.K % 64 || a.k_split % 64 || a.kt_main % 2 || a.kt_alt % 2 ||
        a.kt_off_alt % 2)
      return -1;
    if (bm == 32 && nwt == 1 && kc == 128 && geglu) launch_q<32, 1, 128, true, WF_MX4>(a, s);
    else if (bm == 32 && nwt == 1 && kc == 64 && geglu) launch_q<32, 1, 64, true, WF_MX4>(a, s);
    else if (bm == 32 && nwt == 2 && kc == 64 && !geglu) launch_q<32, 2, 64, false, WF_MX4>(a, s);
    else return -2;
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
#define DG_CASE(BM_, NWT_, KC_, GG_)                                   \
  if (bm == BM_ && nwt == NWT_ && kc == KC_ && geglu == GG_) {         \
    launch_t<BM_, NWT_, KC_, GG_>(a, a.act_kind, s);                   \
    return hipGetLastError() == hipSuccess ? 0 : -5;                   \
  }
  DG_CASE(128, 1, 64, false)
  DG_CASE(64, 1, 64, false)
  DG_CASE(32, 1, 64, true)
  DG_CASE(32, 1, 128, true)
  DG_CASE(64, 1, 128, true)
  DG_CASE(128, 1, 64, true)
  DG_CASE(32, 2, 64, false)
  DG_CASE(32, 1, 64, false)
  DG_CASE(32, 1, 128, false)
  DG_CASE(64, 1, 128, false)
  DG_CASE(64, 2, 64, false)
  DG_CASE(128, 2, 64, false)
#undef DG_CASE
  return -2;
}

__global__ __launch_bounds__(kThreads) void k_rope_table(float2* out, int64_t n, int half, int pos0, int d_head,
                                                        float base) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= n) return;
  const int i = (int)(t / half), j = (int)(t - (int64_t)i * half);
  out[t] = rope_cs(pos0 + i, j, d_head, base);
}

int launch_rope_table(float2* out, int rows, int d_head, int pos0, float rope_base, hipStream_t s) {
  if (rows < 1 || d_head < 2 || d_head % 2) return -1;
  const int64_t n = (int64_t)rows * (d_head / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)DG_CEIL_DIV(n, kThreads)), dim3(kThreads), 0, s, out, n, d_head / 2,
                     pos0, d_head, rope_base);
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

int launch_pack_fp8(uint8_t* dst, const uint8_t* src, int64_t rows, int64_t cols, hipStream_t s) {
  if (rows % 16 || cols % 32) return -1;
  const int64_t tiles = (rows / 16) * (cols / 32);
  hipLaunchKernelGGL(k_pack_fp8, dim3((unsigned)DG_CEIL_DIV(tiles, 4)), dim3(kThreads), 0, s, dst, src, rows, cols);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_pack_mxfp4(uint8_t* dst, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                      hipStream_t s) {
  if (rows % 16 || cols % 64) return -1;
  const int64_t sbs = (rows / 16) * (cols / 64);
  hipLaunchKernelGGL(k_pack_mxfp4, dim3((unsigned)DG_CEIL_DIV(sbs, 4)), dim3(kThreads), 0, s, dst, codes, scales, rows,
                     cols);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_lm_partials_from_logits(const float* logits, int rows, const LmArgs& lm, hipStream_t s) {
  const int64_t waves = (int64_t)((rows + 3) / 4) * (lm.vocab >> 8);
  hipLaunchKernelGGL(k_partials_from_logits, dim3((unsigned)DG_CEIL_DIV(waves, 4)), dim3(kThreads), 0, s,
                     logits, rows, lm);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_rowgemm(const GemmArgs& a0, const LmArgs* lm, hipStream_t s) {
  GemmArgs a = a0;
  const int bn = RgCfg<false, false>::BN;
  // fp8 weights: LM head only, with 16-byte aligned per-feature scales
  if (a.w_fp8 && (!lm || !a.ws0 || reinterpret_cast<uintptr_t>(a.ws0) % 16)) return -1;
  if (a.tiles || a.row_map || a.w1 || a.act_kind != ACT_BF16 || a.M < 1 || a.N % 16 ||
      a.K % RG_KC || a.k_split % RG_KC || a.act_ld % 8)
    return -1;
  if (!lm && (a.epi != EPI_STORE_F32 || !a.out_f32 || a.ldo % 4)) return -1;
  if (lm && a.N % 256) return -1;
  if (a.n_fb != (a.N + bn - 1) / bn || a.n_split < 1 || (int64_t)a.n_split * a.k_split < a.K) return -1;
  a.max_tiles = (a.M + RG_ROWS - 1) / RG_ROWS;
  a.nblocks = round8(a.max_tiles * a.n_fb * a.n_split);
  LmArgs l;
  if (lm) l = *lm;
  else memset(&l, 0, sizeof(l));
  const dim3 grid(a.nblocks), block(RG_THREADS);
  if (lm && a.w_fp8) hipLaunchKernelGGL((k_rowgemm<true, true>), grid, block, 0, s, a, l);
  else if (lm) hipLaunchKernelGGL((k_rowgemm<true, false>), grid, block, 0, s, a, l);
  else hipLaunchKernelGGL((k_rowgemm<false, false>), grid, block, 0, s, a, l);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

__global__ __launch_bounds__(kThreads) void k_geglu_splits(const float* part, int n_split, int64_t split_stride,
                                                          int rows, int N, bf16_t* out, int ldo) {
  const int64_t pairs = (int64_t)rows * (N >> 1);
  const int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (p >= pairs) return;
  const int row = (int)(p / (N >> 1));
  const int n = (int)(p - (int64_t)row * (N >> 1)) * 2;
  const float* pg = part + (int64_t)row * N + n;
  const float* pu = pg + (int64_t)n_split * split_stride;
  float2 g = *reinterpret_cast<const float2*>(pg), u = *reinterpret_cast<const float2*>(pu);
  for (int s = 1; s < n_split; ++s) {
    const float2 gs = *reinterpret_cast<const float2*>(pg + s * split_stride);
    const float2 us = *reinterpret_cast<const float2*>(pu + s * split_stride);
    g.x += gs.x; g.y += gs.y;
    u.x += us.x; u.y += us.y;
  }
  store_act2<bf16_t>(out, (int64_t)row * ldo + n, gelu_tanh(g.x) * u.x, gelu_tanh(g.y) * u.y);
}

int launch_geglu_splits(const float* part, int n_split, int64_t split_stride, int rows, int N, void* out, int ldo,
                        hipStream_t s) {
  if (n_split < 1 || rows < 1 || N % 2 || ldo % 2) return -1;
  const int64_t pairs = (int64_t)rows * (N >> 1);
  hipLaunchKernelGGL(k_geglu_splits, dim3((unsigned)DG_CEIL_DIV(pairs, kThreads)), dim3(kThreads), 0, s, part, n_split,
                     split_stride, rows, N, reinterpret_cast<bf16_t*>(out), ldo);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_split_epilogue(const GemmArgs& a, const float* part, int n_split, int64_t split_stride, int ldp,
                          hipStream_t s) {
  if (n_split < 1 || n_split > 16 || a.N % 2) return -1;
  const int64_t pairs = (int64_t)a.M * (a.N >> 1);
  hipLaunchKernelGGL(k_split_epilogue, dim3((unsigned)DG_CEIL_DIV(pairs, kThreads)), dim3(kThreads), 0, s, a, part,
                     n_split, split_stride, ldp);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
