// Canvas attention: every query of a sequence's canvas attends to the joint
// key list [cached prefix ; canvas].  All prefix keys are visible; canvas key
// j is visible to canvas query i always (denoising) or only when j <= i
// (causal encode).  Grouped-query attention: query head h reads KV head
// h / (n_q / n_kv).  Scale 1/sqrt(d_head).
//
// Keys come from up to two stores with the same layout
// [seq][kv_head][rows][d_head]: src0 holds keys [0, len0), src1 holds keys
// [len0, len0 + len1) (the denoiser's transient canvas K/V).  In causal mode
// the canvas keys are the last n keys of src0 (written there by the QKV
// epilogue before attention runs).
//
// bf16 path (d_head = 256): one workgroup = one KV head, 64 query rows (the
// G query heads sharing that KV head x 64/G queries), one KV split.  K tiles
// of 32 keys are staged in LDS as rows, V tiles transposed, and each wave
// computes S^T = K Q^T (keys down, queries across) with
// v_mfma_f32_16x16x32_bf16, so that the exponentiated scores already sit in
// the B-operand layout of the next MFMA, O^T = V^T P^T.  Online softmax in the
// exp2 domain.  The P V product runs in fp16 (P in [0, 1] keeps 11
// significant bits instead of bf16's 8; V's bf16 values convert exactly), so
// rounding P is a smaller error than rounding the output.  Splits write
// (m, l, O) partials merged in split order.
#include "dg_internal.h"

namespace {

struct AttnArgs {
  const void* q;  // [T][n_q * d]
  int64_t q_ld;
  const void* k0;
  const void* v0;
  const void* k1;
  const void* v1;
  int64_t s0_seq, s0_head;  // element strides of src0 (seq, head); row stride = d
  int64_t s1_seq, s1_head;
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

__device__ __forceinline__ uint16_t f16_bits(float f) {
  const _Float16 h = (_Float16)f;
  return *reinterpret_cast<const uint16_t*>(&h);
}

constexpr int ATT_D = 256;
constexpr int ATT_KT = 32;
constexpr int KS_LD = ATT_D + 8;   // bf16 pitch of a K row in LDS
constexpr int VT_LD = ATT_KT + 8;  // bf16 pitch of a transposed V row

__global__ __launch_bounds__(256) void k_attn_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t ks[ATT_KT * KS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t vt[ATT_D * VT_LD];  // V^T as fp16 bits
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.n_q / a.n_kv;
  const int qpb = 64 / G;  // queries per block
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
  if (a.causal) ke = min(ke, a.n_prefix + min(a.seq_len, qb * qpb + qpb));  // keys beyond the last query are masked
  const int g4 = (lane >> 4) * 4;

  for (int k0 = kb; k0 < ke; k0 += ATT_KT) {
    __syncthreads();
    // stage K rows and V^T: 32 keys x 256 dims = 1024 vectors of 8 per tensor
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int v = tid + it * 256;
      const int kr = v >> 5, c8 = (v & 31) * 8;
      const int j = k0 + kr;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (j < ke) {
        const bf16_t *kp, *vp;
        if (j < a.len0) {
          const int64_t off = (int64_t)seq * a.s0_seq + (int64_t)hk * a.s0_head + (int64_t)j * ATT_D + c8;
          kp = reinterpret_cast<const bf16_t*>(a.k0) + off;
          vp = reinterpret_cast<const bf16_t*>(a.v0) + off;
        } else {
          const int64_t off = (int64_t)seq * a.s1_seq + (int64_t)hk * a.s1_head + (int64_t)(j - a.len0) * ATT_D + c8;
          kp = reinterpret_cast<const bf16_t*>(a.k1) + off;
          vp = reinterpret_cast<const bf16_t*>(a.v1) + off;
        }
        kv = *reinterpret_cast<const uint4*>(kp);
        vv = *reinterpret_cast<const uint4*>(vp);
      }
      *reinterpret_cast<uint4*>(ks + kr * KS_LD + c8) = kv;
      const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[(c8 + 2 * e) * VT_LD + kr] = f16_bits(bf2f((bf16_t)(w4[e] & 0xFFFF)));
        vt[(c8 + 2 * e + 1) * VT_LD + kr] = f16_bits(bf2f((bf16_t)(w4[e] >> 16)));
      }
    }
    __syncthreads();

    // S^T for two 16-key halves: lane holds keys 16h + 4g + e, query l%16
    f32x4_t st[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      st[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < ATT_D / 32; ++s) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(ks + (h * 16 + (lane & 15)) * KS_LD + s * 32 + (lane >> 4) * 8);
        st[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], st[h], 0, 0, 0);
      }
    }
    float sv[8];
    float mt = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
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
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = exp2f(sv[e] - shift);
      ps += pv[e];
    }
    l_run = l_run * alpha + ps;
    // P^T operand (fp16): k index (g, e) -> key 4g+e (e < 4) or 16+4g+(e-4)
    f16x8_t pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = (_Float16)pv[e];
#pragma unroll
    for (int t = 0; t < ATT_D / 16; ++t) {
      o[t] *= alpha;
      const uint16_t* vr = vt + (t * 16 + (lane & 15)) * VT_LD;
      const uint2 lo = *reinterpret_cast<const uint2*>(vr + g4);
      const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16 + g4);
      uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
      const f16x8_t vf = *reinterpret_cast<f16x8_t*>(&u);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf, o[t], 0, 0, 0);
    }
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
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.part_ml[(int64_t)s * T * a.n_q + row].x);
  const float sh = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float2 ml = a.part_ml[(int64_t)s * T * a.n_q + row];
    L += exp2f(ml.x - sh) * ml.y;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int dd = threadIdx.x; dd < a.d; dd += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
      const int64_t pr = (int64_t)s * T * a.n_q + row;
      acc += exp2f(a.part_ml[pr].x - sh) * a.part_o[pr * a.d + dd];
    }
    reinterpret_cast<TA*>(a.out)[row * a.d + dd] = to_act<TA>(acc * inv);
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
                           ? reinterpret_cast<const TA*>(a.v0) + (int64_t)seq * a.s0_seq + (int64_t)hk * a.s0_head + (int64_t)j2 * d
                           : reinterpret_cast<const TA*>(a.v1) + (int64_t)seq * a.s1_seq + (int64_t)hk * a.s1_head +
                                 (int64_t)(j2 - a.len0) * d;
        acc = fmaf(ps[jj], ld_act<TA>(vp + dd), acc);
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
                     int64_t s0_head, int len0, const void* k1, const void* v1, int64_t s1_seq, int64_t s1_head,
                     int len1, int n_prefix, int causal, int seq_len, int n_seq, int n_q, int n_kv, int d,
                     int n_split, float* part_o, float2* part_ml, void* out, hipStream_t s) {
  AttnArgs a;
  a.q = q; a.q_ld = q_ld;
  a.k0 = k0; a.v0 = v0; a.k1 = k1; a.v1 = v1;
  a.s0_seq = s0_seq; a.s0_head = s0_head; a.s1_seq = s1_seq; a.s1_head = s1_head;
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
  const int nqb = DG_CEIL_DIV(seq_len, 64 / G);
  const int64_t blocks = (int64_t)n_seq * n_kv * nqb * n_split;
  hipLaunchKernelGGL(k_attn_mfma, dim3((unsigned)blocks), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return -5;
  if (n_split > 1) {
    hipLaunchKernelGGL(k_attn_merge<bf16_t>, dim3((unsigned)((int64_t)n_seq * seq_len * n_q)), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return -5;
  }
  return 0;
}
