// Canvas attention: every query of a sequence's canvas attends to the joint
// key list [cached prefix ; canvas].  All prefix keys are visible; canvas key
// j is visible to canvas query i always (denoising) or only when j <= i
// (causal encode).  Grouped-query attention: query head h reads KV head
// h / (n_q / n_kv).  Scale 1/sqrt(d_head).
//
// Keys come from up to two stores: src0 holds keys [0, len0), src1 holds keys
// [len0, len0 + len1) (the denoiser's transient canvas K/V).  K is stored
// [seq][kv_head][row][d_head]; V is stored transposed, [seq][kv_head][d_head][row]
// with a row pitch per store, so that the V^T operand streams as contiguous
// key runs.  In causal mode the canvas keys are the last n keys of src0
// (written there by the QKV epilogue before attention runs).
//
// bf16 path (d_head = 256): one workgroup of 8 waves = one KV head, 128
// query rows (the G query heads sharing that KV head x 128/G queries), one
// KV split.  Tiles of 64 keys are staged in double-buffered LDS (K as rows,
// V^T as rows of 64 keys converted to fp16; the next tile's loads are in
// flight during this tile's MFMAs), and each wave computes S^T = K Q^T (keys down, queries across)
// with v_mfma_f32_16x16x32_bf16, so the exponentiated scores already sit in
// the B-operand layout of O^T = V^T P^T (v_mfma_f32_16x16x32_f16 with P split
// into two fp16 parts, so the product keeps fp32 accuracy; V's bf16 values
// convert to fp16 exactly).  Online softmax in the exp2 domain.  Splits write (m, l, O) partials merged in
// split order.
#include "dg_internal.h"

namespace {

struct AttnArgs {
  const void* q;  // [T][n_q * d]
  int64_t q_ld;
  const void* k0;
  const void* v0;
  const void* k1;
  const void* v1;
  int64_t s0_seq, s0_head;  // element strides of src0 (seq, head); K row stride = d
  int64_t s1_seq, s1_head;
  int32_t vp0, vp1;         // row pitch of the transposed V stores
  int32_t len0, len1;
  int32_t n_prefix;   // keys before the canvas (causal boundary)
  int32_t causal;
  int32_t seq_len;    // queries per sequence
  int32_t n_seq, n_q, n_kv, d;
  int32_t n_split, keys_per_split;
  float scale_log2;   // log2(e) / sqrt(d)
  float* part_o;      // [split][T][n_q][d] unnormalised
  float2* part_ml;    // [split][T][n_q] (m in log2 units, l)
  void* out;          // [T][n_q * d]
};

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t f16x2_bits(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)(*reinterpret_cast<const uint16_t*>(&ha)) | ((uint32_t)(*reinterpret_cast<const uint16_t*>(&hb)) << 16);
}

// 8 bf16 -> 8 fp16 (exact for bf16 values inside fp16's normal range)
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  uint4 r;
  r.x = f16x2_bits(bf2f((bf16_t)(v.x & 0xFFFF)), bf2f((bf16_t)(v.x >> 16)));
  r.y = f16x2_bits(bf2f((bf16_t)(v.y & 0xFFFF)), bf2f((bf16_t)(v.y >> 16)));
  r.z = f16x2_bits(bf2f((bf16_t)(v.z & 0xFFFF)), bf2f((bf16_t)(v.z >> 16)));
  r.w = f16x2_bits(bf2f((bf16_t)(v.w & 0xFFFF)), bf2f((bf16_t)(v.w >> 16)));
  return r;
}

constexpr int ATT_D = 256;
constexpr int ATT_KT = 64;
constexpr int ATT_WAVES = 8;
constexpr int ATT_THREADS = ATT_WAVES * 64;
constexpr int ATT_ROWS = ATT_WAVES * 16;           // query rows per workgroup
constexpr int KS_LD = ATT_D + 8;                   // bf16 pitch of a K row in LDS
constexpr int VT_LD = ATT_KT + 8;                  // fp16 pitch of a V^T row in LDS
constexpr int KS_ELEMS = ATT_KT * KS_LD;
constexpr int VT_ELEMS = ATT_D * VT_LD;
constexpr int ATT_VPT = ATT_KT * ATT_D / 8 / ATT_THREADS;  // 16-byte vectors per thread per tensor

__global__ __launch_bounds__(ATT_THREADS, 1) void k_attn_mfma(AttnArgs a) {
  // two buffers of (K tile, V^T tile): the next tile is loaded while this one is used
  __shared__ __attribute__((aligned(16))) uint16_t sm[2 * (KS_ELEMS + VT_ELEMS)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.n_q / a.n_kv;
  const int qpb = ATT_ROWS / G;  // queries per block
  const int nqb = DG_CEIL_DIV(a.seq_len, qpb);
  int bid = blockIdx.x;
  const int sp = bid % a.n_split;
  bid /= a.n_split;
  const int qb = bid % nqb;
  bid /= nqb;
  const int hk = bid % a.n_kv;
  const int seq = bid / a.n_kv;
  if (seq >= a.n_seq) return;

  const int row0 = wave * 16;            // this wave's 16 rows inside the block
  const int hq = hk * G + row0 / qpb;    // query head
  const int qi0 = qb * qpb + row0 % qpb; // first query index in the sequence
  const int my_q = qi0 + (lane & 15);
  const bool qvalid = my_q < a.seq_len;
  const int64_t tok = (int64_t)seq * a.seq_len + (qvalid ? my_q : 0);

  // Q fragments (B operand of S^T = K Q^T): lane holds q[my_q][32s + 8g .. +8]
  bf16x8_t qf[ATT_D / 32];
  {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) + tok * a.q_ld + (int64_t)hq * ATT_D + (lane >> 4) * 8;
#pragma unroll
    for (int s = 0; s < ATT_D / 32; ++s) {
      uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qp + s * 32) : make_uint4(0, 0, 0, 0);
      qf[s] = *reinterpret_cast<bf16x8_t*>(&v);
    }
  }

  f32x4_t o[ATT_D / 16];
#pragma unroll
  for (int t = 0; t < ATT_D / 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_keys = a.len0 + a.len1;
  const int kb = sp * a.keys_per_split;
  int ke = min(n_keys, kb + a.keys_per_split);
  if (a.causal) ke = min(ke, a.n_prefix + min(a.seq_len, qb * qpb + qpb));  // later keys are masked for all
  const int g4 = (lane >> 4) * 4;

  const bf16_t* kbase0 = reinterpret_cast<const bf16_t*>(a.k0) + (int64_t)seq * a.s0_seq + (int64_t)hk * a.s0_head;
  const bf16_t* vbase0 = reinterpret_cast<const bf16_t*>(a.v0) + (int64_t)seq * a.s0_seq + (int64_t)hk * a.s0_head;
  const bf16_t* kbase1 = reinterpret_cast<const bf16_t*>(a.k1) + (int64_t)seq * a.s1_seq + (int64_t)hk * a.s1_head;
  const bf16_t* vbase1 = reinterpret_cast<const bf16_t*>(a.v1) + (int64_t)seq * a.s1_seq + (int64_t)hk * a.s1_head;

  uint4 kreg[ATT_VPT], vreg[ATT_VPT];
  // K: vector v -> key row v / 32, dims (v % 32) * 8;  V^T: vector v -> dim v / 8, keys (v % 8) * 8
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < ATT_VPT; ++it) {
      const int v = tid + it * ATT_THREADS;
      {
        const int j = k0 + (v >> 5), c8 = (v & 31) * 8;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (j < ke) {
          const bf16_t* kp = j < a.len0 ? kbase0 + (int64_t)j * ATT_D + c8 : kbase1 + (int64_t)(j - a.len0) * ATT_D + c8;
          x = *reinterpret_cast<const uint4*>(kp);
        }
        kreg[it] = x;
      }
      {
        const int dd = v >> 3, j0 = k0 + (v & 7) * 8;
        const bool full = j0 + 8 <= ke;
        const bool in0 = j0 + 8 <= a.len0, in1 = j0 >= a.len0;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (full && in0 && ((j0 | a.vp0) & 7) == 0) {
          x = *reinterpret_cast<const uint4*>(vbase0 + (int64_t)dd * a.vp0 + j0);
        } else if (full && in1 && (((j0 - a.len0) | a.vp1) & 7) == 0) {
          x = *reinterpret_cast<const uint4*>(vbase1 + (int64_t)dd * a.vp1 + (j0 - a.len0));
        } else if (j0 < ke) {
          // tile edge or a store boundary inside these 8 keys: element by element
          uint32_t w[4] = {0, 0, 0, 0};
#pragma nounroll
          for (int e = 0; e < 8; ++e) {
            const int j = j0 + e;
            if (j < ke) {
              const uint32_t b = j < a.len0 ? vbase0[(int64_t)dd * a.vp0 + j] : vbase1[(int64_t)dd * a.vp1 + (j - a.len0)];
              w[e >> 1] |= b << ((e & 1) * 16);
            }
          }
          x = make_uint4(w[0], w[1], w[2], w[3]);
        }
        vreg[it] = x;
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = sm + buf * (KS_ELEMS + VT_ELEMS);
    uint16_t* vt = ks + KS_ELEMS;
#pragma unroll
    for (int it = 0; it < ATT_VPT; ++it) {
      const int v = tid + it * ATT_THREADS;
      *reinterpret_cast<uint4*>(ks + (v >> 5) * KS_LD + (v & 31) * 8) = kreg[it];
      *reinterpret_cast<uint4*>(vt + (v >> 3) * VT_LD + (v & 7) * 8) = bf16x8_to_f16x8(vreg[it]);
    }
  };

  if (kb < ke) {
    load_tile(kb);
    store_tile(0);
  }
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += ATT_KT, buf ^= 1) {
    const bool more = k0 + ATT_KT < ke;
    if (more) load_tile(k0 + ATT_KT);  // in flight during this tile's MFMAs
    const uint16_t* ks = sm + buf * (KS_ELEMS + VT_ELEMS);
    const uint16_t* vt = ks + KS_ELEMS;
    // S^T for four 16-key quarters: lane holds keys 16h + 4g + e, query l%16
    f32x4_t st[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      st[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < ATT_D / 32; ++s) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(ks + (h * 16 + (lane & 15)) * KS_LD + s * 32 + (lane >> 4) * 8);
        st[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], st[h], 0, 0, 0);
      }
    }
    float sv[16];
    float mt = -INFINITY;
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = k0 + h * 16 + g4 + e;
        bool vis = j < ke;
        if (a.causal) vis = vis && (j <= a.n_prefix + my_q);
        const float x = vis ? st[h][e] * a.scale_log2 : -INFINITY;
        sv[h * 4 + e] = x;
        mt = fmaxf(mt, x);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float shift = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - shift);
    m_run = m_new;
    float ps = 0.f;
    float pv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pv[e] = exp2f(sv[e] - shift);
      ps += pv[e];
    }
    l_run = l_run * alpha + ps;
    // P^T operands for the two 32-key k-steps: k index (g, e) -> key
    // 32kk + 4g + e (e < 4) or 32kk + 16 + 4g + (e - 4).  P = P_hi + P_lo in
    // fp16 (relative error ~2^-22): P V is as accurate as an fp32 product.
    f16x8_t pf[2], pl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = pv[(2 * kk + (e >> 2)) * 4 + (e & 3)];
        const _Float16 hi = (_Float16)x;
        pf[kk][e] = hi;
        pl[kk][e] = (_Float16)(x - (float)hi);
      }
#pragma unroll
    for (int t = 0; t < ATT_D / 16; ++t) {
      o[t] *= alpha;
      const uint16_t* vr = vt + (t * 16 + (lane & 15)) * VT_LD;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vr + kk * 32 + g4);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + kk * 32 + 16 + g4);
        uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const f16x8_t vf = *reinterpret_cast<f16x8_t*>(&u);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[kk], o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl[kk], o[t], 0, 0, 0);
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  // lane holds O^T[dh = 16t + 4g + e][query l%16]
  if (a.n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16_t* op = reinterpret_cast<bf16_t*>(a.out) + tok * (int64_t)(a.n_q * ATT_D) + (int64_t)hq * ATT_D;
#pragma unroll
    for (int t = 0; t < ATT_D / 16; ++t) {
      const int d0 = t * 16 + g4;
      const uint32_t lo = (uint32_t)f2bf(o[t][0] * inv) | ((uint32_t)f2bf(o[t][1] * inv) << 16);
      const uint32_t hi = (uint32_t)f2bf(o[t][2] * inv) | ((uint32_t)f2bf(o[t][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + d0) = make_uint2(lo, hi);
    }
  } else {
    const int64_t T = (int64_t)a.n_seq * a.seq_len;
    const int64_t prow = ((int64_t)sp * T + tok) * a.n_q + hq;
    float* pp = a.part_o + prow * ATT_D;
#pragma unroll
    for (int t = 0; t < ATT_D / 16; ++t)
      *reinterpret_cast<float4*>(pp + t * 16 + g4) = make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
    if (lane < 16) a.part_ml[prow] = make_float2(m_run, l_run);
  }
}

// Merge split partials in split order: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <typename TA>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int64_t T = (int64_t)a.n_seq * a.seq_len;
  const int64_t row = blockIdx.x;  // token * n_q + head
  if (row >= T * a.n_q) return;
  constexpr int kMaxS = 16;
  __shared__ float wsp[kMaxS];
  __shared__ float inv_l;
  if (threadIdx.x == 0) {
    float2 ml[kMaxS];
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      ml[s] = s < a.n_split ? a.part_ml[(int64_t)s * T * a.n_q + row] : make_float2(-INFINITY, 0.f);
      M = fmaxf(M, ml[s].x);
    }
    const float sh = M == -INFINITY ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      wsp[s] = exp2f(ml[s].x - sh);
      L += wsp[s] * ml[s].y;
    }
    inv_l = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  for (int dd = threadIdx.x; dd < a.d; dd += blockDim.x) {
    float v[kMaxS];
#pragma unroll
    for (int s = 0; s < kMaxS; ++s)
      v[s] = s < a.n_split ? a.part_o[((int64_t)s * T * a.n_q + row) * a.d + dd] : 0.f;
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) acc += wsp[s] * v[s];
    reinterpret_cast<TA*>(a.out)[row * a.d + dd] = to_act<TA>(acc * inv_l);
  }
}

// Plain path (fp32 models, any d_head <= 256): one wave per (token, head),
// 64 keys per iteration, online softmax.
template <typename TA>
__global__ __launch_bounds__(64) void k_attn_simple(AttnArgs a) {
  __shared__ float qs[256];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int64_t T = (int64_t)a.n_seq * a.seq_len;
  const int64_t row = blockIdx.x;  // token * n_q + head
  if (row >= T * a.n_q) return;
  const int64_t tok = row / a.n_q;
  const int hq = (int)(row - tok * a.n_q);
  const int seq = (int)(tok / a.seq_len), qi = (int)(tok - (int64_t)seq * a.seq_len);
  const int hk = hq / (a.n_q / a.n_kv);
  const int d = a.d;
  for (int i = lane; i < d; i += 64) qs[i] = ld_act<TA>(reinterpret_cast<const TA*>(a.q) + tok * a.q_ld + (int64_t)hq * d + i);
  __syncthreads();
  float oacc[4] = {0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int n_keys = a.len0 + a.len1;
  const float scale = a.scale_log2;
  for (int k0 = 0; k0 < n_keys; k0 += 64) {
    const int j = k0 + lane;
    bool vis = j < n_keys;
    if (a.causal) vis = vis && (j <= a.n_prefix + qi);
    float sc = -INFINITY;
    if (vis) {
      const TA* kp = j < a.len0
                         ? reinterpret_cast<const TA*>(a.k0) + (int64_t)seq * a.s0_seq + (int64_t)hk * a.s0_head + (int64_t)j * d
                         : reinterpret_cast<const TA*>(a.k1) + (int64_t)seq * a.s1_seq + (int64_t)hk * a.s1_head +
                               (int64_t)(j - a.len0) * d;
      float dot = 0.f;
      for (int i = 0; i < d; ++i) dot = fmaf(qs[i], ld_act<TA>(kp + i), dot);
      sc = dot * scale;
    }
    const float mt = wave_max(sc);
    const float m_new = fmaxf(m_run, mt);
    const float shift = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - shift);
    const float p = exp2f(sc - shift);
    l_run = l_run * alpha + wave_sum(p);
    m_run = m_new;
    ps[lane] = p;
    __syncthreads();
    for (int q = 0; q < 4; ++q) {
      const int dd = lane + q * 64;
      if (dd >= d) break;
      float acc = oacc[q] * alpha;
      for (int jj = 0; jj < 64 && k0 + jj < n_keys; ++jj) {
        const int j2 = k0 + jj;
        if (ps[jj] == 0.f) continue;
        const TA* vp = j2 < a.len0
                           ? reinterpret_cast<const TA*>(a.v0) + (int64_t)seq * a.s0_seq + (int64_t)hk * a.s0_head +
                                 (int64_t)dd * a.vp0 + j2
                           : reinterpret_cast<const TA*>(a.v1) + (int64_t)seq * a.s1_seq + (int64_t)hk * a.s1_head +
                                 (int64_t)dd * a.vp1 + (j2 - a.len0);
        acc = fmaf(ps[jj], ld_act<TA>(vp), acc);
      }
      oacc[q] = acc;
    }
    __syncthreads();
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  for (int q = 0; q < 4; ++q) {
    const int dd = lane + q * 64;
    if (dd < d) reinterpret_cast<TA*>(a.out)[tok * (int64_t)a.n_q * d + (int64_t)hq * d + dd] = to_act<TA>(oacc[q] * inv);
  }
}

}  // namespace

// Host launcher.  dtype: 0 = fp32 activations (plain path), 1 = bf16 (MFMA path, d = 256).
int launch_attention(int dtype, const void* q, int64_t q_ld, const void* k0, const void* v0, int64_t s0_seq,
                     int64_t s0_head, int vp0, int len0, const void* k1, const void* v1, int64_t s1_seq,
                     int64_t s1_head, int vp1, int len1, int n_prefix, int causal, int seq_len, int n_seq, int n_q,
                     int n_kv, int d, int n_split, float* part_o, float2* part_ml, void* out, hipStream_t s) {
  AttnArgs a;
  a.q = q; a.q_ld = q_ld;
  a.k0 = k0; a.v0 = v0; a.k1 = k1; a.v1 = v1;
  a.s0_seq = s0_seq; a.s0_head = s0_head; a.s1_seq = s1_seq; a.s1_head = s1_head;
  a.vp0 = vp0; a.vp1 = vp1;
  a.len0 = len0; a.len1 = len1; a.n_prefix = n_prefix; a.causal = causal;
  a.seq_len = seq_len; a.n_seq = n_seq; a.n_q = n_q; a.n_kv = n_kv; a.d = d;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  a.part_o = part_o; a.part_ml = part_ml; a.out = out;
  const int n_keys = len0 + len1;
  if (dtype == 0) {
    a.n_split = 1;
    a.keys_per_split = n_keys;
    hipLaunchKernelGGL(k_attn_simple<float>, dim3((unsigned)((int64_t)n_seq * seq_len * n_q)), dim3(64), 0, s, a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  const int G = n_q / n_kv;
  if (d != ATT_D || (G != 1 && G != 2 && G != 4) || n_q % n_kv) return -2;
  n_split = n_split < 1 ? 1 : n_split;
  int kps = DG_CEIL_DIV(n_keys, n_split);
  kps = DG_CEIL_DIV(kps, ATT_KT) * ATT_KT;
  n_split = DG_CEIL_DIV(n_keys, kps);
  a.n_split = n_split;
  a.keys_per_split = kps;
  const int nqb = DG_CEIL_DIV(seq_len, ATT_ROWS / G);
  const int64_t blocks = (int64_t)n_seq * n_kv * nqb * n_split;
  hipLaunchKernelGGL(k_attn_mfma, dim3((unsigned)blocks), dim3(ATT_THREADS), 0, s, a);
  if (hipGetLastError() != hipSuccess) return -5;
  if (n_split > 1) {
    hipLaunchKernelGGL(k_attn_merge<bf16_t>, dim3((unsigned)((int64_t)n_seq * seq_len * n_q)), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return -5;
  }
  return 0;
}
