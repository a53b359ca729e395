// Canvas attention: every query of a sequence's canvas attends to the keys
// [0, n_keys) of its store: the cached prefix followed by the canvas rows
// (the denoiser writes the canvas K/V into the cache rows past the cache
// length, which it does not advance; the causal encode appends there).  All
// prefix keys are visible; canvas key j is visible to canvas query i always
// (denoising) or only when j <= i (causal encode).  Grouped-query attention:
// query head h reads KV head h / (n_q / n_kv).  Scale 1/sqrt(d_head).
//
// K is stored [seq][kv_head][row][d_head]; V is stored transposed,
// [seq][kv_head][d_head][row] with row pitch vp, so that the V^T operand
// streams as contiguous key runs.  bf16 models keep both in bf16.
//
// bf16 path (d_head = 256): one workgroup of 8 waves (two per SIMD) = one KV
// head, 128 query rows (the G query heads sharing that KV head x 128/G
// queries), one KV split; each wave owns 16 query rows.  Tiles of 64
// keys move straight from memory into a double-buffered LDS stage with
// global_load_lds_dwordx4 (K: 512 B per key row, 16-byte column groups
// XOR-swizzled; V^T: 128 B per dimension row, likewise swizzled), one tile
// ahead of the MFMAs.  S^T = K Q^T comes from v_mfma_f32_16x16x32_bf16 with
// the key rows of each 16-row MFMA chosen so that every lane ends up with 8
// consecutive keys per 32-key step: the exponentiated scores are directly
// the B operand of O^T = V^T P^T (the same bf16 MFMA), and the V^T operand is
// one 16-byte read.  P is split into two bf16 parts, hi = bf16(p) and lo =
// bf16(p - hi), two MFMAs each, so the weights keep 2^-18 relative accuracy:
// with a single bf16 P the output over thousands of diffuse keys carries an
// error close to its own bf16 rounding step, and a large share of those
// roundings flip.  Online softmax in the exp2 domain.  Splits write (m, l, O)
// partials merged in split order.
#include "dg_internal.h"

namespace {

struct AttnArgs {
  const void* q;  // [T][n_q * d]
  int64_t q_ld;
  const void* k;  // key store: K [seq][kv_head][row][d], V^T [seq][kv_head][d][row] (pitch vp)
  const void* v;
  int64_t s_seq, s_head;  // element strides of the store (seq, head)
  int32_t vp;             // row pitch of the transposed V store
  int32_t n_keys;         // keys [0, n_keys) per sequence
  int32_t n_prefix;       // keys before the canvas (causal boundary)
  int32_t causal;
  int32_t seq_len;        // queries per sequence
  int32_t n_seq, n_q, n_kv, d;
  int32_t n_split, keys_per_split;
  float scale_log2;       // log2(e) / sqrt(d)
  float* part_o;          // [split][T][n_q][d] unnormalised
  float2* part_ml;        // [split][T][n_q] (m in log2 units, l)
  void* out;              // [T][n_q * d]
};

constexpr int ATT_D = 256;
constexpr int ATT_KT = 64;                  // keys per tile
constexpr int ATT_WAVES = 8;
constexpr int ATT_THREADS = ATT_WAVES * 64;
constexpr int ATT_QT = 1;                   // 16-query MFMA tiles per wave
constexpr int ATT_QW = 16 * ATT_QT;         // query rows per wave
constexpr int ATT_ROWS = ATT_WAVES * ATT_QW; // query rows per workgroup
constexpr int ATT_K_BYTES = ATT_KT * ATT_D * 2;   // 32 KiB
constexpr int ATT_V_BYTES = ATT_D * ATT_KT * 2;   // 32 KiB
constexpr int ATT_STAGE = ATT_K_BYTES + ATT_V_BYTES;
constexpr int ATT_DMA = (ATT_STAGE / 1024) / ATT_WAVES;  // 1 KiB instructions per wave per tile

typedef __attribute__((address_space(3))) void lds_void_t;

// K tile: key row r at r * 512 B; 16-byte group c (dims 8c..8c+7) at physical
// group c ^ fk(r).  The rows sit 512 B apart, all on the same LDS banks, so
// fk alone spreads a read: the 16 lanes a 16-byte read serves at a time
// (gfx950's 64 banks) read 16 rows with 16 distinct fk values.
__device__ __forceinline__ int att_fk(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }
// S^T MFMA (step kk, half hf): row i <-> key 32 kk + 8 (i / 4) + 4 hf + i % 4,
// so lane group g of the output holds keys 32 kk + 8 g + 4 hf + e.
__device__ __forceinline__ int att_krow(int kk, int hf, int i) { return 32 * kk + 8 * (i >> 2) + 4 * hf + (i & 3); }

__global__ __launch_bounds__(ATT_THREADS, 1) void k_attn_mfma(AttnArgs a) {
  static_assert(ATT_ROWS == 128, "workgroup covers 128 query rows");
  __shared__ __attribute__((aligned(1024))) unsigned char sm[2 * ATT_STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.n_q / a.n_kv;
  const int qpb = ATT_ROWS / G;  // queries per head in a workgroup
  const int nqb = DG_CEIL_DIV(a.seq_len, qpb);
  int bid = blockIdx.x;
  const int sp = bid % a.n_split;
  bid /= a.n_split;
  const int qb = bid % nqb;
  bid /= nqb;
  const int hk = bid % a.n_kv;
  const int seq = bid / a.n_kv;
  if (seq >= a.n_seq) return;

  const int row0 = wave * ATT_QW;              // this wave's 32 rows inside the workgroup
  const int hq = hk * G + row0 / qpb;          // query head (qpb is a multiple of 32)
  const int qi0 = qb * qpb + row0 % qpb;       // first query index of the wave
  const int g = lane >> 4, c16 = lane & 15;
  int my_q[ATT_QT];
  bool qvalid[ATT_QT];
  int64_t tok[ATT_QT];
#pragma unroll
  for (int qt = 0; qt < ATT_QT; ++qt) {
    my_q[qt] = qi0 + qt * 16 + c16;
    qvalid[qt] = my_q[qt] < a.seq_len;
    tok[qt] = (int64_t)seq * a.seq_len + (qvalid[qt] ? my_q[qt] : 0);
  }

  // Q fragments (B operand of S^T = K Q^T): q[query][32 s + 8 g .. +8]
  bf16x8_t qf[ATT_QT][ATT_D / 32];
#pragma unroll
  for (int qt = 0; qt < ATT_QT; ++qt) {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) + tok[qt] * a.q_ld + (int64_t)hq * ATT_D + g * 8;
#pragma unroll
    for (int s = 0; s < ATT_D / 32; ++s) {
      uint4 v = qvalid[qt] ? *reinterpret_cast<const uint4*>(qp + s * 32) : make_uint4(0, 0, 0, 0);
      qf[qt][s] = *reinterpret_cast<bf16x8_t*>(&v);
    }
  }

  f32x4_t o[ATT_QT][ATT_D / 16];
  float m_run[ATT_QT], l_run[ATT_QT];
#pragma unroll
  for (int qt = 0; qt < ATT_QT; ++qt) {
#pragma unroll
    for (int t = 0; t < ATT_D / 16; ++t) o[qt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }

  const int kb = sp * a.keys_per_split;
  int ke = min(a.n_keys, kb + a.keys_per_split);
  if (a.causal) ke = min(ke, a.n_prefix + min(a.seq_len, qb * qpb + qpb));  // later keys are masked for all
  const int ntiles = ke > kb ? DG_CEIL_DIV(ke - kb, ATT_KT) : 0;

  const bf16_t* kbase = reinterpret_cast<const bf16_t*>(a.k) + (int64_t)seq * a.s_seq + (int64_t)hk * a.s_head;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + (int64_t)seq * a.s_seq + (int64_t)hk * a.s_head;

  // tile i (clamped to the last one) into stage i & 1.  Instruction n of the
  // workgroup: n < 32 -> K rows 2n, 2n + 1; else V^T rows 8 (n - 32) .. +7.
  // Keys past the store's end load the last key (masked below).
  auto issue = [&](int i) {
    const int ic = min(i, ntiles - 1);
    const int k0 = kb + ic * ATT_KT;
    unsigned char* st = sm + (i & 1) * ATT_STAGE;
    static_assert(ATT_DMA * ATT_WAVES == 64, "32 K and 32 V^T instructions per tile");
    static_assert(ATT_QW % 16 == 0 && (ATT_ROWS / 4) % ATT_QW == 0, "a wave's rows stay in one head");
    if (wave < ATT_WAVES / 2) {  // K
#pragma unroll
      for (int u = 0; u < ATT_DMA; ++u) {
        const int n = wave * ATT_DMA + u;
        const int r = 2 * n + (lane >> 5);
        const int c = (lane & 31) ^ att_fk(r);
        const int j = min(k0 + r, a.n_keys - 1);
        // uniform base + 32-bit byte offset (< 2^31: rows x 512 B): scalar-base addressing
        const uint32_t off = (uint32_t)(j * ATT_D + c * 8) * 2u;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(kbase) + off, (lds_void_t*)(st + n * 1024), 16,
                                         0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < ATT_DMA; ++u) {
        const int n = wave * ATT_DMA + u;
        const int dd = 8 * (n - 32) + (lane >> 3);
        const int c = (lane & 7) ^ (dd & 7);
        const int j = min(k0 + 8 * c, ((a.n_keys - 1) & ~7));
        const uint32_t off = (uint32_t)(dd * a.vp + j) * 2u;  // < 2^31: 256 x pitch x 2 B
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(vbase) + off, (lds_void_t*)(st + n * 1024), 16,
                                         0, 0);
      }
    }
  };

  if (ntiles > 0) issue(0);
  for (int i = 0; i < ntiles; ++i) {
    // tile i's loads are the only ones in flight: wait, then a plain barrier
    // (every wave's part is in LDS; every wave is done with tile i - 1, whose
    // stage the next issue refills).  The asm memory clobber keeps LDS
    // accesses on their side.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (i + 1 < ntiles) issue(i + 1);
    const unsigned char* ks = sm + (i & 1) * ATT_STAGE;
    const unsigned char* vs = ks + ATT_K_BYTES;
    const int k0 = kb + i * ATT_KT;
    if (ke - k0 < ATT_KT) {
      // last, partial tile: its masked keys (P = 0) may sit in rows never
      // written (up to 7 past the store's last row); zero their V^T entries
      // so that 0 * V cannot meet a non-finite value
      const int kv = ke - k0;
      unsigned char* vw = sm + (i & 1) * ATT_STAGE + ATT_K_BYTES;
      for (int e = tid; e < ATT_D * ATT_KT; e += ATT_THREADS) {
        const int dd = e >> 6, kk = e & 63;
        if (kk >= kv)
          *reinterpret_cast<uint16_t*>(vw + dd * 128 + ((((kk >> 3) ^ (dd & 7)) << 4) | ((kk & 7) << 1))) = 0;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // S^T for the four (kk, half) 16-key groups and both query tiles
    f32x4_t st[ATT_QT][4];
    {
      // step by step over the 32-dim slices, the four key groups side by
      // side; the next slice's four K fragments are read before this one's
      // MFMAs (each st[x] still accumulates s = 0, 1, .. in order)
      int kr[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        kr[x] = att_krow(x >> 1, x & 1, c16);
#pragma unroll
        for (int qt = 0; qt < ATT_QT; ++qt) st[qt][x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      bf16x8_t kf[2][4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        kf[0][x] = *reinterpret_cast<const bf16x8_t*>(ks + kr[x] * 512 + ((g ^ att_fk(kr[x])) << 4));
#pragma unroll
      for (int s = 0; s < ATT_D / 32; ++s) {
        if (s + 1 < ATT_D / 32) {
#pragma unroll
          for (int x = 0; x < 4; ++x)
            kf[(s + 1) & 1][x] =
                *reinterpret_cast<const bf16x8_t*>(ks + kr[x] * 512 + ((((s + 1) * 4 + g) ^ att_fk(kr[x])) << 4));
        }
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int qt = 0; qt < ATT_QT; ++qt)
            st[qt][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s & 1][x], qf[qt][s], st[qt][x], 0, 0, 0);
      }
    }
    // schedule (group masks: 0x100 LDS reads, 0x008 MFMAs): the first two
    // slices' reads, then four MFMAs and the next slice's four reads in turn,
    // so that each wait for K fragments covers eight reads, not one or two
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int s = 0; s < 6; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    // online softmax per query column; P^T operands: k index 8 g + e' <-> key 32 kk + 8 g + e'
    // A tile whose 64 keys are all visible to all of the wave's queries needs
    // no per-element mask (every tile but a split's last, and in the causal
    // encode those below the wave's diagonal).
    const bool full = (k0 + ATT_KT <= ke) && (!a.causal || k0 + ATT_KT - 1 <= a.n_prefix + qi0);
    bf16x8_t pf[ATT_QT][2], pl[ATT_QT][2];
#pragma unroll
    for (int qt = 0; qt < ATT_QT; ++qt) {
      float sv[16];
      float mt = -INFINITY;
      if (full) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float xv = st[qt][x][e] * a.scale_log2;
            sv[x * 4 + e] = xv;
            mt = fmaxf(mt, xv);
          }
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = k0 + 32 * (x >> 1) + 8 * g + 4 * (x & 1) + e;
            bool vis = j < ke;
            if (a.causal) vis = vis && (j <= a.n_prefix + my_q[qt]);
            const float xv = vis ? st[qt][x][e] * a.scale_log2 : -INFINITY;
            sv[x * 4 + e] = xv;
            mt = fmaxf(mt, xv);
          }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      // The reference point m_run moves only when the tile's maximum exceeds
      // it by more than 8 (log2 units), so the weights 2^(s - m_run) stay
      // <= 2^8 and the O rescale is rare.  O and l always share the same
      // reference, so O / l is unchanged.
      // (Hardware exp2: arguments <= 8; results below 2^-126 flush to zero.)
      float alpha = 1.f;
      if (mt > m_run[qt] + 8.f) {  // also the first visible key (m_run = -inf)
        alpha = __builtin_amdgcn_exp2f(m_run[qt] - mt);
        m_run[qt] = mt;
      }
      const float shift = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
      float ps = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(sv[x * 4 + e] - shift);
          ps += p;
          const __bf16 hi = (__bf16)p;  // round to nearest even
          const int kk = x >> 1, ep = 4 * (x & 1) + e;
          pf[qt][kk][ep] = hi;
          pl[qt][kk][ep] = (__bf16)(p - (float)hi);
        }
      l_run[qt] = l_run[qt] * alpha + ps;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int t = 0; t < ATT_D / 16; ++t) o[qt][t] *= alpha;
      }
    }
    // O^T += V^T P^T: lane reads V^T[dim 16 t + c16][keys 32 kk + 8 g .. +8]
    {
      // the next dimension tile's two V^T fragments are read before this
      // tile's MFMAs
      bf16x8_t vf[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        vf[0][kk] = *reinterpret_cast<const bf16x8_t*>(vs + c16 * 128 + (((4 * kk + g) ^ (c16 & 7)) << 4));
#pragma unroll
      for (int t = 0; t < ATT_D / 16; ++t) {
        if (t + 1 < ATT_D / 16) {
          const int dn = (t + 1) * 16 + c16;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            vf[(t + 1) & 1][kk] = *reinterpret_cast<const bf16x8_t*>(vs + dn * 128 + (((4 * kk + g) ^ (dn & 7)) << 4));
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int qt = 0; qt < ATT_QT; ++qt) {
            o[qt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[t & 1][kk], pf[qt][kk], o[qt][t], 0, 0, 0);
            o[qt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[t & 1][kk], pl[qt][kk], o[qt][t], 0, 0, 0);
          }
      }
    }
    // schedule: the first three dimension tiles' reads, then the four MFMAs
    // of a tile and the two reads of a later one in turn
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
    for (int t = 0; t < 14; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);
  }
#pragma unroll
  for (int qt = 0; qt < ATT_QT; ++qt) {
    float l = l_run[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (!qvalid[qt]) continue;
    // lane holds O^T[dh = 16t + 4g + e][query c16]
    if (a.n_split == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      bf16_t* op = reinterpret_cast<bf16_t*>(a.out) + tok[qt] * (int64_t)(a.n_q * ATT_D) + (int64_t)hq * ATT_D;
#pragma unroll
      for (int t = 0; t < ATT_D / 16; ++t) {
        const int d0 = t * 16 + 4 * g;
        const uint32_t lo = (uint32_t)f2bf(o[qt][t][0] * inv) | ((uint32_t)f2bf(o[qt][t][1] * inv) << 16);
        const uint32_t hi = (uint32_t)f2bf(o[qt][t][2] * inv) | ((uint32_t)f2bf(o[qt][t][3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + d0) = make_uint2(lo, hi);
      }
    } else {
      const int64_t T = (int64_t)a.n_seq * a.seq_len;
      const int64_t prow = ((int64_t)sp * T + tok[qt]) * a.n_q + hq;
      float* pp = a.part_o + prow * ATT_D;
#pragma unroll
      for (int t = 0; t < ATT_D / 16; ++t)
        *reinterpret_cast<float4*>(pp + t * 16 + 4 * g) = make_float4(o[qt][t][0], o[qt][t][1], o[qt][t][2], o[qt][t][3]);
      if (g == 0) a.part_ml[prow] = make_float2(m_run[qt], l);
    }
  }
}

// Merge split partials in split order: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <typename TA>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  // one wave per (token, head) row, four of the 256 dims per lane; every
  // lane forms the split weights itself (the same few loads, broadcast), and
  // all loads are issued before the first use
  const int64_t T = (int64_t)a.n_seq * a.seq_len;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // token * n_q + head
  if (row >= T * a.n_q) return;
  const int lane = threadIdx.x & 63;
  // splits in passes of kS (all loads of a pass issued before their use);
  // the sums run in split order whatever the pass size
  constexpr int kS = 16;
  const int64_t sstride = T * a.n_q;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto load_pass = [&](int s0, float2 (&ml)[kS], float4 (&v)[kS], bool with_o) {
#pragma unroll
    for (int j = 0; j < kS; ++j) {
      const int64_t pr = (s0 + j) * sstride + row;
      ml[j] = s0 + j < a.n_split ? a.part_ml[pr] : make_float2(-INFINITY, 0.f);
      if (with_o)
        v[j] = s0 + j < a.n_split ? *reinterpret_cast<const float4*>(a.part_o + pr * a.d + 4 * lane)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto add_pass = [&](const float2 (&ml)[kS], const float4 (&v)[kS], float sh) {
    float w[kS];
#pragma unroll
    for (int j = 0; j < kS; ++j) {
      w[j] = exp2f(ml[j].x - sh);
      L += w[j] * ml[j].y;
    }
#pragma unroll
    for (int j = 0; j < kS; ++j) {
      acc.x += w[j] * v[j].x;
      acc.y += w[j] * v[j].y;
      acc.z += w[j] * v[j].z;
      acc.w += w[j] * v[j].w;
    }
  };
  float2 ml[kS];
  float4 v[kS];
  if (a.n_split <= kS) {
    // one pass: the row maxima and the partials are in flight together
    load_pass(0, ml, v, true);
#pragma unroll
    for (int j = 0; j < kS; ++j) M = fmaxf(M, ml[j].x);
    add_pass(ml, v, M == -INFINITY ? 0.f : M);
  } else {
    for (int s0 = 0; s0 < a.n_split; s0 += kS) {
      load_pass(s0, ml, v, false);
#pragma unroll
      for (int j = 0; j < kS; ++j) M = fmaxf(M, ml[j].x);
    }
    const float sh = M == -INFINITY ? 0.f : M;
    for (int s0 = 0; s0 < a.n_split; s0 += kS) {
      load_pass(s0, ml, v, true);
      add_pass(ml, v, sh);
    }
  }
  const float inv_l = L > 0.f ? 1.f / L : 0.f;
  TA* o = reinterpret_cast<TA*>(a.out) + row * a.d + 4 * lane;
  if constexpr (sizeof(TA) == 2) {  // the lane's four bf16 values in one 8-byte store
    const uint32_t lo = (uint32_t)to_act<TA>(acc.x * inv_l) | ((uint32_t)to_act<TA>(acc.y * inv_l) << 16);
    const uint32_t hi = (uint32_t)to_act<TA>(acc.z * inv_l) | ((uint32_t)to_act<TA>(acc.w * inv_l) << 16);
    *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
  } else {
    o[0] = to_act<TA>(acc.x * inv_l);
    o[1] = to_act<TA>(acc.y * inv_l);
    o[2] = to_act<TA>(acc.z * inv_l);
    o[3] = to_act<TA>(acc.w * inv_l);
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
  const int n_keys = a.n_keys;
  const float scale = a.scale_log2;
  for (int k0 = 0; k0 < n_keys; k0 += 64) {
    const int j = k0 + lane;
    bool vis = j < n_keys;
    if (a.causal) vis = vis && (j <= a.n_prefix + qi);
    float sc = -INFINITY;
    if (vis) {
      const TA* kp = reinterpret_cast<const TA*>(a.k) + (int64_t)seq * a.s_seq + (int64_t)hk * a.s_head + (int64_t)j * d;
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
        const TA* vp = reinterpret_cast<const TA*>(a.v) + (int64_t)seq * a.s_seq + (int64_t)hk * a.s_head +
                       (int64_t)dd * a.vp + j2;
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

// Host launcher.  dtype: 0 = fp32 activations (plain path), 1 = bf16 (MFMA
// path: d = 256, K and V^T bf16, vp a multiple of 8).
int launch_attention(int dtype, const void* q, int64_t q_ld, const void* k, const void* v, int64_t s_seq,
                     int64_t s_head, int vp, int n_keys, int n_prefix, int causal, int seq_len, int n_seq, int n_q,
                     int n_kv, int d, int n_split, float* part_o, float2* part_ml, void* out, hipStream_t s) {
  AttnArgs a;
  a.q = q; a.q_ld = q_ld;
  a.k = k; a.v = v; a.s_seq = s_seq; a.s_head = s_head; a.vp = vp;
  a.n_keys = n_keys; a.n_prefix = n_prefix; a.causal = causal;
  a.seq_len = seq_len; a.n_seq = n_seq; a.n_q = n_q; a.n_kv = n_kv; a.d = d;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  a.part_o = part_o; a.part_ml = part_ml; a.out = out;
  if (n_keys < 1) return -1;
  if (dtype == 0) {
    a.n_split = 1;
    a.keys_per_split = n_keys;
    hipLaunchKernelGGL(k_attn_simple<float>, dim3((unsigned)((int64_t)n_seq * seq_len * n_q)), dim3(64), 0, s, a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  const int G = n_q / n_kv;
  if (d != ATT_D || (G != 1 && G != 2 && G != 4) || n_q % n_kv || vp % 8 || vp < n_keys) return -2;
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
    hipLaunchKernelGGL(k_attn_merge<bf16_t>, dim3((unsigned)DG_CEIL_DIV((int64_t)n_seq * seq_len * n_q, 4)), dim3(256), 0,
                       s, a);
    if (hipGetLastError() != hipSuccess) return -5;
  }
  return 0;
}
