// Host side of the C ABI (include/dg.h): argument checks, the workspace plan,
// and the launch sequence of encode / denoise / commit.  Allocates nothing.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/dg.h"
#include "dg_internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMoeBM = 32;        // row tile of the grouped expert GEMMs (bf16)
constexpr int kSimpleBM = 16;     // row tile of the fp32 GEMMs
constexpr int kMaxRoutePairs = 32768;  // (token, slot) pairs of one encode pass
constexpr int kPassTokens = 4096;      // tokens of one encode pass (at most)
constexpr int kMaxStepTokens = 16384;  // canvas tokens (batch x canvas) of one denoising step
constexpr int kMaxSplit = 16;
constexpr int kAttMaxSplit = 32;  // key splits of one attention launch (the merge takes any count)
constexpr int kSelfSplit = 32;   // vocabulary splits of the expected-embedding product (at most)
constexpr int kRowPartRows = 2048;  // rows of the split-epilogue partial buffer (x split)

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Shape {
  int L, d, nq, nkv, dh, E, k, de, ds, V, dsc, dt;
  bool ex8, lm8;  // fp8 expert / LM-head weights
  bool ex4;       // MXFP4 expert weights
  float rope_base, eps;
  int qdim, kvdim, qkv, n_sh, nvt;
  size_t act;  // bytes per activation element
};

Shape shape_of(const dg_model_config* c) {
  Shape s;
  s.L = c->n_layers; s.d = c->d_model; s.nq = c->n_q_heads; s.nkv = c->n_kv_heads; s.dh = c->d_head;
  s.E = c->n_experts; s.k = c->top_k; s.de = c->d_expert; s.ds = c->d_shared; s.V = c->vocab;
  s.dsc = c->d_selfcond; s.dt = c->dtype;
  s.ex8 = c->expert_dtype == DG_DTYPE_FP8_E4M3;
  s.lm8 = c->lm_dtype == DG_DTYPE_FP8_E4M3;
  s.ex4 = c->expert_dtype == DG_DTYPE_MXFP4;
  s.rope_base = c->rope_base; s.eps = c->norm_eps;
  s.qdim = s.nq * s.dh; s.kvdim = s.nkv * s.dh; s.qkv = s.qdim + 2 * s.kvdim;
  s.n_sh = s.de > 0 ? s.ds / s.de : 0;
  s.nvt = s.V / 256;
  s.act = s.dt == DG_DTYPE_BF16 ? 2 : 4;
  return s;
}

int check_config(const dg_model_config* c) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->d_head < 2 ||
      c->n_experts < 1 || c->top_k < 1 || c->top_k > c->n_experts || c->d_expert < 1 || c->d_shared < 1 ||
      c->vocab < 256 || c->d_selfcond < 1)
    return DG_ERR_INVALID_ARG;
  if (c->dtype != DG_DTYPE_F32 && c->dtype != DG_DTYPE_BF16) return DG_ERR_UNSUPPORTED;
  // fp8 weights (experts, LM head) only in bf16 models
  for (int wd : {c->expert_dtype, c->lm_dtype})
    if (wd != c->dtype && !(wd == DG_DTYPE_FP8_E4M3 && c->dtype == DG_DTYPE_BF16) &&
        !(wd == DG_DTYPE_MXFP4 && wd == c->expert_dtype && c->dtype == DG_DTYPE_BF16))
      return DG_ERR_UNSUPPORTED;
  if (c->lm_dtype == DG_DTYPE_MXFP4) return DG_ERR_UNSUPPORTED;
  if (c->expert_dtype == DG_DTYPE_FP8_E4M3 && c->d_model % 128) return DG_ERR_UNSUPPORTED;
  if (c->expert_dtype == DG_DTYPE_MXFP4 && (c->d_model % 64 || c->d_expert % 64 || c->d_shared % 64))
    return DG_ERR_UNSUPPORTED;
  if (c->n_q_heads % c->n_kv_heads || c->d_shared % c->d_expert || c->vocab % 256 || c->d_head % 2 ||
      c->top_k > 16 || c->n_experts > 255 || c->d_head > 256)
    return DG_ERR_UNSUPPORTED;
  if (c->dtype == DG_DTYPE_BF16) {
    const int G = c->n_q_heads / c->n_kv_heads;
    if (c->d_head != 256 || (G != 1 && G != 2 && G != 4) || c->d_model % 64 || c->d_expert % 64 ||
        c->d_shared % 64 || c->d_selfcond % 64 || (c->n_q_heads * c->d_head) % 64 || c->n_experts % 16)
      return DG_ERR_UNSUPPORTED;
  } else {
    if (c->d_model % 2 || c->d_expert % 2 || c->d_selfcond % 2 || c->n_experts % 2) return DG_ERR_UNSUPPORTED;
  }
  return DG_OK;
}

// Token capacity of one pass through the layer stack (the routing sort
// handles up to route_max_tokens() tokens at a time).
int max_tokens(const Shape& s, int batch, int max_canvas) {
  const int route_cap = std::min(kMaxRoutePairs / s.k, route_max_tokens());
  return std::max(std::min(kPassTokens, route_cap), batch * max_canvas);
}

struct Plan {
  int T;        // tokens per pass
  int Tdn;      // denoise tokens
  int att_rows; // attention partial rows (split x tokens)
  int g_rows;   // rows (x the widest N) of the split-epilogue partial buffer
  int64_t o_rows;  // rows (x d_model) of the O-projection K-split partials
  size_t x, n, q, o, att_o, att_ml, o_part, r_part, ids, wts, row_token, inv, offsets, tiles,
      n_tiles, h, Y, lm_f, lm_i, logits, e_part, ebar, hsc, g_part, rcnt, rope, total;
};

// step_only: a plan for denoising steps alone (no encode passes), whose
// buffers hold batch * max_canvas tokens.  Its launches are the same as the
// full plan's for those steps: every dispatch choice reads either the step's
// own sizes or a capacity both plans give the same value at these sizes.
Plan make_plan(const Shape& s, int batch, int max_canvas, bool step_only = false) {
  Plan p;
  p.T = step_only ? batch * max_canvas : max_tokens(s, batch, max_canvas);
  p.Tdn = batch * max_canvas;
  p.att_rows = std::max(4096, kMaxSplit * p.Tdn);
  const size_t T = p.T, Tdn = p.Tdn;
  const size_t rows_moe = T * s.k + (size_t)s.n_sh * T;
  const size_t max_tiles = T * s.k / kSimpleBM + s.E + (size_t)s.n_sh * ((T + kSimpleBM - 1) / kSimpleBM) + 8;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes); return o; };
  p.x = take(T * s.d * 4);
  p.n = take(T * s.d * s.act);
  p.q = take(T * s.qdim * s.act);
  p.o = take(T * s.qdim * s.act);
  p.att_o = take((size_t)p.att_rows * s.nq * s.dh * 4);
  p.att_ml = take((size_t)p.att_rows * s.nq * 8);
  // O-projection partials: up to min(16, o_rows / rows) K splits (16 for a
  // step of at most 2048 tokens under either plan)
  p.o_rows = step_only ? 16 * (int64_t)Tdn : 8 * (int64_t)T;
  p.o_part = take((size_t)p.o_rows * s.d * 4);
  p.r_part = take(16 * T * s.E * 4);  // router K-split partials (up to 16)
  p.ids = take(T * s.k * 4);
  p.wts = take(T * s.k * 4);
  p.row_token = take(rows_moe * 4);
  p.inv = take(T * s.k * 4);
  p.offsets = take((s.E + 1) * 4);
  p.tiles = take(max_tiles * sizeof(GemmTile));
  p.n_tiles = take(4);
  p.h = take(rows_moe * s.de * s.act);
  p.Y = take(rows_moe * s.d * 4);
  p.lm_f = take(Tdn * s.nvt * sizeof(float4));
  p.lm_i = take(Tdn * s.nvt * sizeof(int2));
  p.logits = take(s.dt == DG_DTYPE_F32 ? Tdn * s.V * 4 : 0);
  p.e_part = take(std::max(kMaxSplit, kSelfSplit) * Tdn * s.d * 4);
  p.ebar = take(Tdn * s.d * s.act);
  p.hsc = take(Tdn * s.dsc * s.act);
  // split-epilogue partials: every row a pass or step can hold (a non-store
  // epilogue over the row-resident kernel stages at least M x N fp32 values)
  p.g_rows = std::max(kRowPartRows, std::max(p.T, p.Tdn));
  p.g_part = take((size_t)p.g_rows * std::max(s.qkv, s.dsc) * 4);
  p.rcnt = take((size_t)std::max(1, route_chunk_words((int)T)) * 4);     // routing sort, per-chunk counts
  p.rope = take(T * (s.dh / 2) * sizeof(float2));                         // RoPE (cos, sin) per row and pair
  p.total = off;
  return p;
}

struct Ctx {
  Shape s;
  Plan p;
  char* ws;
  hipStream_t st;
  const dg_weights* w;
  dg_trace* tr = nullptr;
  const int32_t* force_ids = nullptr;  // test path: [n_layers][T][k] expert ids
  float* router_out = nullptr;         // test path: [n_layers][T][E] router logits
  const float* teacher_x = nullptr;    // test path: [n_layers + 1][T][d] residual each layer (and the head) starts from
  float* layer_out = nullptr;          // test path: [n_layers + 1][T][d] embedding output, then each layer's output
  size_t head_row0 = 0;                // first row of the normalised output the LM head reads
  template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
};

// Records a begin/end event pair around a phase when the trace asks for it.
struct Phase {
  const Ctx& c;
  int idx = -1;
  Phase(const Ctx& ctx, int phase) : c(ctx) {
    dg_trace* t = c.tr;
    if (t && (t->mask >> phase & 1u) && t->count + 2 <= t->capacity) {
      idx = t->count;
      t->phase[idx / 2] = phase;
      t->count += 2;
      hipEventRecord((hipEvent_t)t->events[idx], c.st);
    }
  }
  ~Phase() {
    if (idx >= 0) hipEventRecord((hipEvent_t)c.tr->events[idx + 1], c.st);
  }
};

GemmArgs base_args() {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.alpha = 1.0f;
  a.n_split = 1;
  return a;
}

#define DG_TRY(x)                 \
  do {                            \
    const int rc_ = (x);          \
    if (rc_ != 0) return rc_ < 0 ? rc_ : DG_ERR_HIP; \
  } while (0)

// Enough workgroups to keep ~4 waves per SIMD streaming weights.
constexpr int kTargetBlocks = 1024;
// Largest M that takes the weight-streaming kernel for dense products.
constexpr int kWsMaxRows = 512;
// Row-resident GEMM: one 4-wave workgroup per CU; K-split partials of the
// non-store epilogues use at most kRowPartRows rows x N of workspace.
constexpr int kRowTargetBlocks = 256;
constexpr int kRowMaxSplit = 16;
// Non-store epilogues: K splits limited so the fp32 partials stay within this
// many bytes (writing and re-reading them costs more than the extra CUs gain).
constexpr int64_t kRowPartBytes = 32ll << 20;

// Row tile of the grouped expert GEMMs (bf16): 32 rows while the experts see
// a few dozen tokens each (the weight stream bounds them); 64 and 128 once an
// average expert's rows span several tiles, so that each weight fragment a
// wave loads feeds more MFMAs.  fp8 experts keep 32.
int moe_bm(const Shape& s, int T) {
  if (s.ex8 || s.ex4) return kMoeBM;
  const int64_t per_expert = (int64_t)T * s.k / s.E;
  return per_expert >= 512 ? 128 : per_expert >= 128 ? 64 : kMoeBM;
}

int pick_split(int blocks_per_split, int K, int kc, int max_split) {
  int sp = std::max(1, std::min(max_split, (kTargetBlocks + blocks_per_split - 1) / std::max(1, blocks_per_split)));
  while (sp > 1 && (K / kc) < sp) --sp;
  return sp;
}

// K split of the row-resident GEMM: about one workgroup per CU, at most
// max_split, and at least two 64-wide K chunks per split.
int row_split(int M, int N, int K, int max_split) {
  const int base = ((M + 255) / 256) * ((N + 255) / 256);
  int sp = std::max(1, std::min(max_split, (kRowTargetBlocks + base - 1) / base));
  while (sp > 1 && K / 64 < 2 * sp) --sp;
  return sp;
}

// Dense GEMM: out = act[M][K] . W[N][K]^T with the given epilogue.
// EPI_STORE_F32 may split K up to max_split ways (partials at out_f32 +
// split * split_stride; the split count used is returned in *used_split);
// the other epilogues split K through fp32 partials in the workspace and a
// summing epilogue kernel.
int dense_gemm(const Ctx& c, GemmArgs a, int M, int N, int K, int max_split, int* used_split = nullptr) {
  a.M = M; a.N = N; a.K = K;
  a.n_main = 1;
  if (used_split) *used_split = 1;
  // Canvas-sized products (M <= kWsMaxRows): weight-streaming kernel, 64-feature
  // workgroups with 128-wide K chunks.  Many small workgroups keep more loads in
  // flight than the row-resident kernel's 256 x 256 blocks, which at these M
  // leave half the CUs idle or pay for fp32 partials.  Fused epilogues (no K
  // split) take 64-row tiles, which halve the L2 re-reads of the weights; the
  // K-split stores take 32-row tiles, which keep more workgroups per split
  // (measured on the 30-layer step: QKV 42 -> 38 us, O and router faster at 32).
  if (c.s.dt == DG_DTYPE_BF16 && M <= kWsMaxRows && K % 128 == 0 && a.act_kind == ACT_BF16 &&
      a.epi != EPI_GEGLU) {
    const bool store = a.epi == EPI_STORE_F32;
    // A handful of rows (the single-token decode step): a fused epilogue
    // without a K split would run one workgroup per 64 features, too few to
    // keep the weight stream going, so K is split through fp32 partials in the
    // workspace and the summing epilogue kernel applies the epilogue.
    const int64_t part_rows = (int64_t)kRowPartRows * std::max(c.s.qkv, c.s.dsc);
    if (!store && (int64_t)((M + 63) / 64) * ((N + 63) / 64) * 4 <= kTargetBlocks &&
        (int64_t)M * N * kRowMaxSplit <= part_rows) {
      a.kt_main = K / 32;
      a.n_fb = (N + 63) / 64;
      a.max_tiles = (M + 31) / 32;
      a.tile_fastest = 1;
      const int sp = pick_split(a.max_tiles * a.n_fb, K, 128, kRowMaxSplit);
      a.k_split = ((K / 128 + sp - 1) / sp) * 128;
      a.n_split = (K + a.k_split - 1) / a.k_split;
      GemmArgs pa = a;
      pa.epi = EPI_STORE_F32; pa.out_f32 = c.at<float>(c.p.g_part); pa.ldo = N; pa.split_stride = (int64_t)M * N;
      pa.alpha = 1.0f;
      DG_TRY(launch_wsgemm(pa, 32, 1, 128, false, c.st));
      return launch_split_epilogue(a, pa.out_f32, a.n_split, pa.split_stride, N, c.st);
    }
    const int bm = store ? 32 : 64;
    a.kt_main = K / 32;
    a.n_fb = (N + 63) / 64;
    a.max_tiles = (M + bm - 1) / bm;
    a.tile_fastest = 1;
    const int sp = store ? pick_split(a.max_tiles * a.n_fb, K, 128, max_split) : 1;
    a.k_split = ((K / 128 + sp - 1) / sp) * 128;
    a.n_split = (K + a.k_split - 1) / a.k_split;
    if (used_split) *used_split = a.n_split;
    return launch_wsgemm(a, bm, 1, 128, false, c.st);
  }
  if (c.s.dt == DG_DTYPE_BF16 && K % 64 == 0 && a.epi != EPI_GEGLU &&
      a.epi != EPI_RESID) {
    a.kt_main = K / 32;
    a.n_fb = (N + 255) / 256;
    const bool store = a.epi == EPI_STORE_F32;
    // non-store epilogues: the partials must fit the split-epilogue buffer
    const int64_t g_cap = (int64_t)c.p.g_rows * std::max(c.s.qkv, c.s.dsc);
    const int64_t part_cap = std::min<int64_t>(g_cap, kRowPartBytes / 4) / ((int64_t)M * N);
    const int cap = store ? max_split : (int)std::min<int64_t>(kRowMaxSplit, part_cap);
    const int sp = row_split(M, N, K, std::max(1, cap));
    a.k_split = ((K / 64 + sp - 1) / sp) * 64;
    a.n_split = (K + a.k_split - 1) / a.k_split;
    if (store) {
      if (used_split) *used_split = a.n_split;
      return launch_rowgemm(a, nullptr, c.st);
    }
    if ((int64_t)M * N * a.n_split > g_cap) return DG_ERR_UNSUPPORTED;
    GemmArgs pa = a;
    pa.epi = EPI_STORE_F32; pa.out_f32 = c.at<float>(c.p.g_part); pa.ldo = N; pa.split_stride = (int64_t)M * N;
    pa.alpha = 1.0f;
    DG_TRY(launch_rowgemm(pa, nullptr, c.st));
    return launch_split_epilogue(a, pa.out_f32, a.n_split, pa.split_stride, N, c.st);
  }
  if (c.s.dt == DG_DTYPE_BF16) {
    // largest row tile that still gives enough workgroups (weights re-read
    // by the other row tiles of a feature block come from L2: tile_fastest)
    const int nwt = 1;
    a.n_fb = (N + 64 * nwt - 1) / (64 * nwt);
    int bm = 32;
    for (int cand : {128, 64}) {
      if (((M + cand - 1) / cand) * a.n_fb >= kTargetBlocks) { bm = cand; break; }
    }
    a.kt_main = K / 32;
    a.max_tiles = (M + bm - 1) / bm;
    a.tile_fastest = 1;
    int sp = (a.epi == EPI_STORE_F32) ? pick_split(a.max_tiles * a.n_fb, K, 64, max_split) : 1;
    a.k_split = ((K / 64 + sp - 1) / sp) * 64;
    a.n_split = (K + a.k_split - 1) / a.k_split;
    if (used_split) *used_split = a.n_split;
    return launch_wsgemm(a, bm, nwt, 64, a.epi == EPI_GEGLU, c.st);
  }
  a.kt_main = K / 32;  // row pitch of plain fp32 weights is kt_main * 32 = K
  a.max_tiles = (M + kSimpleBM - 1) / kSimpleBM;
  a.n_split = 1;
  a.k_split = K;
  return launch_gemm_simple(a, c.st);
}


// The layer stack over T = n_seq * seq_len tokens whose embeddings are in
// x / n.  causal: encode (k, v appended to the cache at rows L..); else the
// denoiser (canvas k, v kept in the workspace).
// Two segments (`fused`): rows [0, n_seq seq_len) are a committed block
// encoded causally at L (K/V appended at rows [L, L + seq_len)), rows
// [n_seq seq_len, 2 n_seq seq_len) the next block's canvas, bidirectional
// over [cache ; committed block ; canvas] (K/V at rows [L + seq_len, L + 2
// seq_len)).  The projections, routing and experts run over both at once.
int run_layers(const Ctx& c, const dg_kv_cache* cache, int n_seq, int seq_len, int L, bool causal,
               bool need_output = false, bool fused = false) {
  const Shape& s = c.s;
  const int n_segs = fused ? 2 : 1;
  const int Tseg = n_seq * seq_len;
  const int T = n_segs * Tseg;
  const bool bf = s.dt == DG_DTYPE_BF16;
  const int64_t layer_elems = (int64_t)cache->batch * s.nkv * cache->capacity * s.dh;
  const int64_t c_seq = (int64_t)s.nkv * cache->capacity * s.dh, c_head = (int64_t)cache->capacity * s.dh;
  void* xn = c.at<void>(c.p.n);
  // RoPE rotations of this call's positions, formed once for every layer
  for (int seg = 0; seg < n_segs; ++seg)
    DG_TRY(launch_rope_table(c.at<float2>(c.p.rope) + (size_t)seg * seq_len * (s.dh / 2), seq_len, s.dh,
                             L + seg * seq_len, s.rope_base, c.st));
  for (int l = 0; l < s.L; ++l) {
    const dg_layer_weights& lw = c.w->layers[l];
    if (c.teacher_x)  // test path: this layer starts from the given residual
      DG_TRY(launch_set_norm(bf, c.teacher_x + (int64_t)l * T * s.d, c.at<float>(c.p.x), xn, T, s.d, s.eps, c.st));
    char* kc = reinterpret_cast<char*>(cache->k) + (size_t)l * layer_elems * s.act;
    char* vc = reinterpret_cast<char*>(cache->v) + (size_t)l * layer_elems * s.act;
    // q, k, v with RoPE.  With one sequence the two segments are one run of
    // 2 seq_len tokens at positions L.. (rows, cache rows and rotation table
    // all contiguous), so one product covers both (one pass over the
    // weights); with several sequences each segment has its own launch.
    const int qkv_launches = (n_segs == 1 || n_seq == 1) ? 1 : n_segs;
    const int qkv_len = seq_len * n_segs / qkv_launches;  // tokens per sequence and launch
    for (int seg = 0; seg < qkv_launches; ++seg) {
      Phase ph(c, DG_PHASE_QKV);
      GemmArgs a = base_args();
      a.act = c.at<char>(c.p.n) + (size_t)seg * Tseg * s.d * s.act; a.act_ld = s.d;
      a.act_kind = bf ? ACT_BF16 : ACT_F32;
      a.w0 = lw.wqkv;
      a.epi = EPI_QKV;
      QkvEpi& q = a.qkv;
      q.q = c.at<char>(c.p.q) + (size_t)seg * Tseg * s.qdim * s.act;
      q.q_dim = s.qdim; q.kv_dim = s.kvdim; q.d_head = s.dh; q.n_kv = s.nkv;
      // k, v of these tokens go to cache rows [L, L + seq_len): appended by the
      // encoder; scratch rows for the denoiser, which leaves the length as is
      q.k = kc; q.v = vc; q.kv_b_stride = c_seq; q.kv_h_stride = c_head; q.kv_row0 = L + seg * seq_len;
      q.v_pitch = cache->capacity;
      q.seq_len = qkv_len; q.pos0 = L + seg * seq_len; q.rope_base = s.rope_base;
      q.rope = c.at<float2>(c.p.rope) + (size_t)seg * seq_len * (s.dh / 2);
      DG_TRY(dense_gemm(c, a, n_seq * qkv_len, s.qkv, s.d, 1));
    }
    // The causal encode keeps only the K/V rows it appends: past the last
    // layer's QKV nothing reads its output (no LM head follows; the next chunk
    // embeds its own tokens).  The test entry points that record or force
    // per-layer routes, and the AR step (its LM head reads the last layer's
    // normalised output), run the whole layer.
    if (causal && !fused && !need_output && l == s.L - 1 && !c.router_out && !c.force_ids) break;
    // attention (per segment: the second sees the first's K/V rows as context)
    for (int seg = 0; seg < n_segs; ++seg) {
      Phase ph(c, DG_PHASE_ATTN);
      const int L0 = L + seg * seq_len;
      const int n_keys = L0 + seq_len;
      int split = 1;
      if (bf) {
        const int G = s.nq / s.nkv;
        const int base_blocks = n_seq * s.nkv * ((seq_len + 128 / G - 1) / (128 / G));
        split = std::max(1, (256 + base_blocks - 1) / base_blocks);         // ~1 workgroup per CU
        // >= 4 key tiles per split; >= 2 when there are few query blocks
        // (the decode step: 8 workgroups before the split)
        split = std::min(split, std::max(1, (n_keys + 255) / 256 * (base_blocks < 32 ? 2 : 1)));
        split = std::min(split, std::min(kAttMaxSplit, std::max(1, c.p.att_rows / Tseg)));
      }
      const size_t qoff = (size_t)seg * Tseg * s.qdim * s.act;
      DG_TRY(launch_attention(bf, c.at<char>(c.p.q) + qoff, s.qdim, kc, vc, c_seq, c_head, cache->capacity, n_keys,
                              L0, (causal && seg == 0) ? 1 : 0, seq_len, n_seq, s.nq, s.nkv, s.dh, split,
                              c.at<float>(c.p.att_o), c.at<float2>(c.p.att_ml), c.at<char>(c.p.o) + qoff, c.st));
    }
    // O projection (split-K partials), residual, RMSNorm
    {
      Phase ph(c, DG_PHASE_OPROJ);
      GemmArgs a = base_args();
      a.act = c.at<void>(c.p.o); a.act_ld = s.qdim; a.act_kind = bf ? ACT_BF16 : ACT_F32;
      a.w0 = lw.wo;
      a.epi = EPI_STORE_F32; a.out_f32 = c.at<float>(c.p.o_part); a.ldo = s.d; a.split_stride = (int64_t)T * s.d;
      int n_split = 1;
      DG_TRY(dense_gemm(c, a, T, s.d, s.qdim, (int)std::min<int64_t>(16, c.p.o_rows / T), &n_split));
      DG_TRY(launch_resid_norm(bf, c.at<float>(c.p.x), c.at<float>(c.p.o_part), n_split, (int64_t)T * s.d, xn, T, s.d,
                               s.eps, c.st));
    }
    // router logits
    int r_split = 1;
    const int bm = bf ? moe_bm(s, T) : kSimpleBM;
    {
      Phase ph(c, DG_PHASE_ROUTE);
      GemmArgs a = base_args();
      a.act = xn; a.act_ld = s.d; a.act_kind = bf ? ACT_BF16 : ACT_F32;
      a.w0 = lw.wr;
      a.epi = EPI_STORE_F32; a.out_f32 = c.at<float>(c.p.r_part); a.ldo = s.E; a.split_stride = (int64_t)T * s.E;
      DG_TRY(dense_gemm(c, a, T, s.E, s.d, 16, &r_split));
      const int32_t* forced = c.force_ids ? c.force_ids + (int64_t)l * T * s.k : nullptr;
      float* r_out = c.router_out ? c.router_out + (int64_t)l * T * s.E : nullptr;
      DG_TRY(launch_topk(c.at<float>(c.p.r_part), r_split, (int64_t)T * s.E, T, s.E, s.k, forced,
                         c.at<int32_t>(c.p.ids), c.at<float>(c.p.wts), r_out, c.st));
      DG_TRY(launch_route_sort(c.at<int32_t>(c.p.ids), T, s.k, s.E, s.n_sh, bm, c.at<int32_t>(c.p.row_token),
                               c.at<int32_t>(c.p.inv), c.at<int32_t>(c.p.offsets), c.at<GemmTile>(c.p.tiles),
                               c.at<int32_t>(c.p.n_tiles), c.at<int32_t>(c.p.rcnt), c.st));
    }
    const int max_tiles = T * s.k / bm + s.E + s.n_sh * ((T + bm - 1) / bm);
    if (max_tiles >= 65536) return DG_ERR_UNSUPPORTED;  // tile spans hold 16-bit indices
    // experts + shared slices: gate/up with GeGLU
    {
      Phase ph(c, DG_PHASE_MOE_UP);
      GemmArgs a = base_args();
      a.act = xn; a.act_ld = s.d; a.act_kind = bf ? ACT_BF16 : ACT_F32;
      a.row_map = c.at<int32_t>(c.p.row_token);
      a.w0 = lw.ex_g; a.w1 = lw.ex_u; a.w_group_stride = (int64_t)s.de * s.d;
      a.w0_alt = lw.sh_g; a.w1_alt = lw.sh_u; a.w_alt_stride = (int64_t)s.de * s.d;
      a.n_main = s.E; a.kt_main = s.d / 32; a.kt_alt = s.d / 32; a.kt_off_alt = 0;
      a.K = s.d; a.N = s.de;
      a.tiles = c.at<GemmTile>(c.p.tiles); a.n_tiles_dev = c.at<int32_t>(c.p.n_tiles); a.max_tiles = max_tiles;
      a.M = 0;
      a.epi = EPI_GEGLU; a.out_act = c.at<void>(c.p.h); a.ldo = s.de;
      a.n_split = 1; a.k_split = s.d;
      if (s.ex8) {
        a.w_fp8 = 1;
        a.ws0 = lw.ex_g_scale; a.ws1 = lw.ex_u_scale; a.ws_group_stride = s.de;
        a.ws0_alt = lw.sh_g_scale; a.ws1_alt = lw.sh_u_scale; a.ws_alt_stride = s.de;  // slice c: features c*de..
      }
      a.w_mx4 = s.ex4;
      if (bf) {
        a.n_fb = (s.de + 63) / 64;
        // expert by expert, the row tiles of one (expert, feature block)
        // together (same XCD): a hot expert's weight slice comes from HBM
        // once and from L2 for its other tiles, and a tile's activation rows
        // are read again one expert's tile count later, still in L2
        a.group_major = 1;
        const int kc = bm == 128 ? 64 : s.d % 128 == 0 ? 128 : 64;
        const int64_t rows_moe = (int64_t)T * (s.k + s.n_sh);
        // Fewer (token, slot) pairs than experts (the decode step): a dozen
        // row tiles x feature blocks cannot keep the weight stream going, so
        // K is split four ways; gate and up partials go to the workspace and
        // a summing kernel applies the GeGLU.
        const int dsplit = 4;
        if (!s.ex8 && !s.ex4 && (int64_t)T * s.k < s.E && s.d / kc >= dsplit &&
            2 * dsplit * rows_moe * s.de <= (int64_t)c.p.g_rows * std::max(s.qkv, s.dsc)) {
          a.k_split = ((s.d / kc + dsplit - 1) / dsplit) * kc;
          a.n_split = (s.d + a.k_split - 1) / a.k_split;
          a.epi = EPI_GEGLU_PARTS; a.out_f32 = c.at<float>(c.p.g_part); a.ldo = s.de;
          a.split_stride = rows_moe * s.de;
          DG_TRY(launch_wsgemm(a, bm, 1, kc, true, c.st));
          DG_TRY(launch_geglu_splits(a.out_f32, a.n_split, a.split_stride, (int)rows_moe, s.de, c.at<void>(c.p.h), s.de,
                                     c.st));
        } else {
          DG_TRY(launch_wsgemm(a, bm, 1, kc, true, c.st));
        }
      } else {
        DG_TRY(launch_gemm_simple(a, c.st));
      }
    }
    // down projections
    {
      Phase ph(c, DG_PHASE_MOE_DOWN);
      GemmArgs a = base_args();
      a.act = c.at<void>(c.p.h); a.act_ld = s.de; a.act_kind = bf ? ACT_BF16 : ACT_F32;
      a.w0 = lw.ex_d; a.w_group_stride = (int64_t)s.d * s.de;
      a.w0_alt = lw.sh_d; a.w_alt_stride = 0;
      a.n_main = s.E; a.kt_main = s.de / 32; a.kt_alt = s.ds / 32; a.kt_off_alt = s.de / 32;
      a.K = s.de; a.N = s.d;
      a.tiles = c.at<GemmTile>(c.p.tiles); a.n_tiles_dev = c.at<int32_t>(c.p.n_tiles); a.max_tiles = max_tiles;
      a.epi = EPI_STORE_F32; a.out_f32 = c.at<float>(c.p.Y); a.ldo = s.d; a.split_stride = 0;
      a.n_split = 1; a.k_split = s.de;
      if (s.ex8) {
        a.w_fp8 = 1;
        a.ws0 = lw.ex_d_scale; a.ws_group_stride = s.d;
        a.ws0_alt = lw.sh_d_scale; a.ws_alt_stride = 0;  // K slices of one matrix: same output features
      }
      a.w_mx4 = s.ex4;
      if (bf) {
        // fewer (token, slot) pairs than experts (the decode step): one
        // 16-feature tile per wave, twice the workgroups for the few row tiles
        const int nwt = (!s.ex8 && !s.ex4 && (int64_t)T * s.k < s.E) ? 1 : 2;
        a.n_fb = (s.d + 64 * nwt - 1) / (64 * nwt);
        a.group_major = 1;  // expert by expert, as the gate/up launch
        DG_TRY(launch_wsgemm(a, bm, nwt, 64, false, c.st));
      } else {
        DG_TRY(launch_gemm_simple(a, c.st));
      }
    }
    {
      Phase ph(c, DG_PHASE_COMBINE);
      DG_TRY(launch_combine_norm(bf, c.at<float>(c.p.x), c.at<float>(c.p.Y), c.at<int32_t>(c.p.inv),
                                 c.at<float>(c.p.wts), T, s.k, s.n_sh, xn, s.d, s.eps, c.st));
    }
    if (c.layer_out)  // test path: this layer's output residual
      DG_TRY(launch_copy_i32(reinterpret_cast<int32_t*>(c.layer_out + (int64_t)(l + 1) * T * s.d),
                             c.at<int32_t>(c.p.x), T * s.d, c.st));
  }
  return DG_OK;
}

int check_ws(const Plan& p, void* ws, size_t bytes) {
  if (!ws || bytes < p.total) return DG_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return DG_ERR_INVALID_ARG;
  return DG_OK;
}

int check_weights(const dg_model_config* cfg, const dg_weights* w) {
  if (!w || !w->embed || !w->lm_head || !w->layers) return DG_ERR_INVALID_ARG;
  auto aligned = [](const float* p) { return p && reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  if (cfg->lm_dtype == DG_DTYPE_FP8_E4M3 && !aligned(w->lm_head_scale)) return DG_ERR_INVALID_ARG;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dg_layer_weights& L = w->layers[l];
    if (!L.wqkv || !L.wo || !L.wr || !L.sh_g || !L.sh_u || !L.sh_d || !L.ex_g || !L.ex_u || !L.ex_d)
      return DG_ERR_INVALID_ARG;
    if (cfg->expert_dtype == DG_DTYPE_FP8_E4M3 &&
        !(aligned(L.ex_g_scale) && aligned(L.ex_u_scale) && aligned(L.ex_d_scale) && aligned(L.sh_g_scale) &&
          aligned(L.sh_u_scale) && aligned(L.sh_d_scale)))
      return DG_ERR_INVALID_ARG;
  }
  return DG_OK;
}

int check_cache(const dg_model_config* cfg, const dg_kv_cache* c, int batch) {
  if (!c || !c->k || !c->v || c->batch != batch || c->capacity < 1 || c->length < 0 || c->length > c->capacity)
    return DG_ERR_INVALID_ARG;
  // bf16 models: V^T rows are read in 16-byte runs of 8 keys
  if (cfg->dtype == DG_DTYPE_BF16 && c->capacity % 8) return DG_ERR_UNSUPPORTED;
  return DG_OK;
}

// The denoiser writes its canvas K/V into rows [length, length + canvas).
int check_denoise_cache(const dg_model_config* cfg, const dg_kv_cache* c, const dg_canvas* cv) {
  DG_TRY(check_cache(cfg, c, cv->batch));
  if ((int64_t)c->length + cv->canvas > c->capacity) return DG_ERR_KV_CAPACITY;
  return DG_OK;
}

int check_canvas(const dg_canvas* cv, bool outputs) {
  if (!cv || cv->batch < 1 || cv->canvas < 1 || cv->canvas > 1024 || !cv->tokens || !cv->seeds) return DG_ERR_INVALID_ARG;
  if (outputs && (!cv->entropy || !cv->sample || !cv->argmax || !cv->prev_argmax || !cv->accepted || !cv->n_accepted ||
                  !cv->mean_entropy || !cv->stop || !cv->flags))
    return DG_ERR_INVALID_ARG;
  if ((cv->p_side == nullptr) != (cv->p_scale == nullptr)) return DG_ERR_INVALID_ARG;
  return DG_OK;
}

// Embedding + self-conditioning for the canvas tokens -> x, n.
int embed_canvas(const Ctx& c, const dg_canvas* cv, const dg_step_params* p) {
  const Shape& s = c.s;
  const bool bf = s.dt == DG_DTYPE_BF16;
  const int T = cv->batch * cv->canvas;
  const bool ext = cv->sc_probs != nullptr;
  const bool carried = !ext && p->t >= 1 && cv->p_side != nullptr;
  const float* add = nullptr;
  int add_split = 0;
  if (ext || carried) {
    if (!c.w->embed_t || !c.w->sc_up || !c.w->sc_down) return DG_ERR_INVALID_ARG;
    Phase ph(c, DG_PHASE_SELFCOND);
    // expected embedding e_bar = P E (split over the vocabulary)
    GemmArgs a = base_args();
    if (ext) {
      a.act = cv->sc_probs; a.act_kind = ACT_F32;
    } else {
      // carried: the previous step's tempered probabilities (normalised in place by its sampler)
      a.act = cv->p_side; a.act_kind = bf ? ACT_BF16 : ACT_F32;
    }
    a.act_ld = s.V;
    a.w0 = c.w->embed_t;
    a.epi = EPI_STORE_F32; a.out_f32 = c.at<float>(c.p.e_part); a.ldo = s.d; a.split_stride = (int64_t)T * s.d;
    a.M = T; a.N = s.d; a.K = s.V; a.n_main = 1; a.kt_main = s.V / 32;
    int n_split = 1;
    if (bf && !ext) {
      // row-resident kernel: 256-feature blocks (P, 134 MB at 256 rows, is
      // re-read once per feature block), the vocabulary split so that the
      // workgroups fill the CUs in one round (one workgroup per CU)
      a.n_fb = (s.d + 255) / 256;
      const int base = ((T + 255) / 256) * a.n_fb;
      n_split = std::max(1, std::min(kSelfSplit, kRowTargetBlocks / base));
      a.k_split = ((s.V / 32 + n_split - 1) / n_split) * 32;
      n_split = (s.V + a.k_split - 1) / a.k_split;
      a.n_split = n_split;
      DG_TRY(launch_rowgemm(a, nullptr, c.st));
    } else if (bf) {
      const int bm = 128, nwt = 2;
      a.max_tiles = (T + bm - 1) / bm;
      a.n_fb = (s.d + 64 * nwt - 1) / (64 * nwt);
      a.tile_fastest = 1;  // the row tiles of one E^T slice run together: E^T comes from HBM once
      n_split = kMaxSplit;
      a.k_split = ((s.V / 256 + n_split - 1) / n_split) * 256;  // whole 256-wide vocabulary tiles
      n_split = (s.V + a.k_split - 1) / a.k_split;
      a.n_split = n_split;
      DG_TRY(launch_wsgemm(a, bm, nwt, 64, false, c.st));
    } else {
      a.max_tiles = (T + kSimpleBM - 1) / kSimpleBM;
      a.n_split = 1; a.k_split = s.V;
      DG_TRY(launch_gemm_simple(a, c.st));
    }
    DG_TRY(launch_reduce_splits(bf, c.at<float>(c.p.e_part), n_split, (int64_t)T * s.d, (int64_t)T * s.d,
                                c.at<void>(c.p.ebar), c.st));
    GemmArgs u = base_args();
    u.act = c.at<void>(c.p.ebar); u.act_ld = s.d; u.act_kind = bf ? ACT_BF16 : ACT_F32;
    u.w0 = c.w->sc_up;
    u.epi = EPI_GELU; u.out_act = c.at<void>(c.p.hsc); u.ldo = s.dsc;
    DG_TRY(dense_gemm(c, u, T, s.dsc, s.d, 1));
    GemmArgs dn = base_args();
    dn.act = c.at<void>(c.p.hsc); dn.act_ld = s.dsc; dn.act_kind = bf ? ACT_BF16 : ACT_F32;
    dn.w0 = c.w->sc_down;
    // partials in e_part (free again after the reduction above), summed by the embedding kernel
    dn.epi = EPI_STORE_F32; dn.out_f32 = c.at<float>(c.p.e_part); dn.ldo = s.d; dn.split_stride = (int64_t)T * s.d;
    DG_TRY(dense_gemm(c, dn, T, s.d, s.dsc, kMaxSplit, &add_split));
    add = c.at<float>(c.p.e_part);
  }
  Phase ph(c, DG_PHASE_EMBED);
  return launch_embed_norm(bf, cv->tokens, c.w->embed, add, add_split, (int64_t)T * s.d, c.at<float>(c.p.x),
                           c.at<void>(c.p.n), T, s.d, s.eps, c.st);
}

// LM head + sampler statistics of the T rows of the final norm output.
// lm: the statistics' destination and sampler parameters; lm.logits, if set
// (test path), also receives the fp32 logits.
int lm_head_rows(const Ctx& c, int T, LmArgs lm) {
  Phase ph(c, DG_PHASE_LMHEAD);
  const Shape& s = c.s;
  const bool bf = s.dt == DG_DTYPE_BF16;
  float* logits_out = lm.logits;
  lm.part_f = c.at<float4>(c.p.lm_f);
  lm.part_i = c.at<int2>(c.p.lm_i);
  lm.p_side_f32 = !bf;
  lm.vocab = s.V;
  GemmArgs a = base_args();
  a.act = c.at<char>(c.p.n) + c.head_row0 * s.d * s.act; a.act_ld = s.d; a.act_kind = bf ? ACT_BF16 : ACT_F32;
  a.w0 = c.w->lm_head;
  a.alpha = c.w->lm_scale;
  a.M = T; a.N = s.V; a.K = s.d; a.n_main = 1; a.kt_main = s.d / 32;
  if (s.lm8) {
    a.w_fp8 = 1;
    a.ws0 = c.w->lm_head_scale;
  }
  if (bf && s.d % 64 == 0) {
    a.n_fb = s.nvt;
    a.n_split = 1;
    a.k_split = s.d;
    return launch_rowgemm(a, &lm, c.st);
  }
  if (s.lm8 || bf) return DG_ERR_UNSUPPORTED;  // bf16 models have d_model % 64 == 0 (check_config)
  float* z = logits_out ? logits_out : c.at<float>(c.p.logits);
  a.epi = EPI_STORE_F32; a.out_f32 = z; a.ldo = s.V;
  DG_TRY(dense_gemm(c, a, T, s.V, s.d, 1));
  lm.logits = nullptr;
  return launch_lm_partials_from_logits(z, T, lm, c.st);
}

// The canvas LM head: statistics at the step's temperature, the next step's
// self-conditioning input (unless the logits are being captured without it).
int lm_head(const Ctx& c, const dg_canvas* cv, const dg_step_params* p, float* logits_out, bool side = false) {
  LmArgs lm;
  memset(&lm, 0, sizeof(lm));
  lm.p_side = (logits_out && !side) ? nullptr : cv->p_side;
  lm.logits = logits_out;
  lm.inv_tau = 1.0f / dg_temperature(p->t, p->n_steps);
  lm.seeds = cv->seeds;
  lm.canvas = cv->canvas;
  lm.step = p->t;
  lm.block = p->block;
  return lm_head_rows(c, cv->batch * cv->canvas, lm);
}

// One autoregressive decode step: the latest token of each of `batch`
// sequences is encoded causally at row L of its cache (K/V appended) through
// the whole layer stack, the LM head runs on those rows, and the next token
// is their argmax (the sampler's row merge: greedy, ties to the lower id).
int ar_impl(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache, const int32_t* d_tokens,
            int32_t batch, int32_t* d_next, float* d_logits, void* d_ws, size_t ws_bytes, void* stream) {
  DG_TRY(check_config(cfg));
  DG_TRY(check_weights(cfg, w));
  if (!d_tokens || !d_next || batch < 1) return DG_ERR_INVALID_ARG;
  DG_TRY(check_cache(cfg, cache, batch));
  if ((int64_t)cache->length + 1 > cache->capacity) return DG_ERR_KV_CAPACITY;
  Ctx c;
  c.s = shape_of(cfg);
  c.p = make_plan(c.s, batch, 1);
  DG_TRY(check_ws(c.p, d_ws, ws_bytes));
  if ((int64_t)batch * c.s.k > kMaxRoutePairs || batch > route_max_tokens()) return DG_ERR_UNSUPPORTED;
  c.ws = (char*)d_ws;
  c.st = (hipStream_t)stream;
  c.w = w;
  const bool bf = c.s.dt == DG_DTYPE_BF16;
  DG_TRY(launch_embed_norm(bf, d_tokens, w->embed, nullptr, 0, 0, c.at<float>(c.p.x), c.at<void>(c.p.n), batch,
                           c.s.d, c.s.eps, c.st));
  DG_TRY(run_layers(c, cache, batch, 1, cache->length, true, true));
  // The statistics carry a sampling candidate drawn from per-row seeds; the
  // greedy step reads none of it, so the seeds point at workspace words
  // (the routing ids buffer, done with by now).
  LmArgs lm;
  memset(&lm, 0, sizeof(lm));
  lm.logits = d_logits;
  lm.inv_tau = 1.0f;
  lm.seeds = c.at<uint64_t>(c.p.ids);
  lm.canvas = 1;
  DG_TRY(lm_head_rows(c, batch, lm));
  DG_TRY(launch_row_merge(c.at<float4>(c.p.lm_f), c.at<int2>(c.p.lm_i), c.s.nvt, batch, 1, lm.seeds, 0, 0,
                          c.at<float>(c.p.wts), c.at<int32_t>(c.p.inv), d_next, nullptr, c.st));
  cache->length += 1;
  return DG_OK;
}

int sample_and_select(const Ctx& c, dg_canvas* cv, const dg_step_params* p) {
  Phase ph(c, DG_PHASE_SAMPLER);
  const Shape& s = c.s;
  const int T = cv->batch * cv->canvas;
  DG_TRY(launch_row_merge(c.at<float4>(c.p.lm_f), c.at<int2>(c.p.lm_i), s.nvt, T, cv->canvas, cv->seeds, p->t,
                          p->block, cv->entropy, cv->sample, cv->argmax, cv->p_scale, c.st));
  if (cv->p_side) DG_TRY(launch_normalize_side(s.dt == DG_DTYPE_BF16, cv->p_side, cv->p_scale, T, s.V, c.st));
  return launch_select(cv->entropy, cv->sample, cv->argmax, cv->prev_argmax, cv->tokens, cv->accepted, cv->n_accepted,
                       cv->mean_entropy, cv->stop, cv->flags, cv->seeds, cv->batch, cv->canvas, p->t, p->block, s.V,
                       p->adaptive, p->entropy_bound, p->stop_threshold, c.st);
}

int check_step(const dg_step_params* p) {
  if (!p || p->n_steps < 1 || p->t < 0 || p->t >= p->n_steps || p->block < 0) return DG_ERR_INVALID_ARG;
  return DG_OK;
}

}  // namespace

static int encode_impl(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache, const int32_t* d_tokens,
                       int32_t batch, int32_t n_tokens, void* d_ws, size_t ws_bytes, void* stream, dg_trace* trace,
                       const int32_t* force_ids, float* router_out);
static int denoise_impl(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache, dg_canvas* cv,
                        const dg_step_params* p, void* d_ws, size_t ws_bytes, void* stream, dg_trace* trace,
                        const int32_t* force_ids, float* router_out, float* logits_out, bool step_only = false,
                        const float* teacher_x = nullptr, float* layer_out = nullptr);

extern "C" {

float dg_temperature(int32_t t, int32_t n_steps) {
  if (n_steps <= 1) return 0.8f;
  return (float)(0.8 + (0.4 - 0.8) * ((double)t / (double)(n_steps - 1)));
}

size_t dg_workspace_bytes(const dg_model_config* cfg, int32_t batch, int32_t max_canvas) {
  if (check_config(cfg) != DG_OK || batch < 1 || max_canvas < 1) return 0;
  return make_plan(shape_of(cfg), batch, max_canvas).total;
}

int dg_pack_weight_bf16(void* d_dst, const void* d_src, int64_t rows, int64_t cols, void* stream) {
  if (!d_dst || !d_src || rows <= 0 || cols <= 0 || rows % 16 || cols % 32) return DG_ERR_INVALID_ARG;
  return launch_pack_bf16((bf16_t*)d_dst, (const bf16_t*)d_src, rows, cols, 0, (hipStream_t)stream) == 0 ? DG_OK
                                                                                                          : DG_ERR_HIP;
}

int dg_pack_weight_bf16_transposed(void* d_dst, const void* d_src, int64_t rows, int64_t cols, void* stream) {
  if (!d_dst || !d_src || rows <= 0 || cols <= 0 || rows % 16 || cols % 32) return DG_ERR_INVALID_ARG;
  return launch_pack_bf16((bf16_t*)d_dst, (const bf16_t*)d_src, rows, cols, 1, (hipStream_t)stream) == 0 ? DG_OK
                                                                                                          : DG_ERR_HIP;
}

int dg_pack_weight_fp8(void* d_dst, const void* d_src, int64_t rows, int64_t cols, void* stream) {
  if (!d_dst || !d_src || rows <= 0 || cols <= 0 || rows % 16 || cols % 32) return DG_ERR_INVALID_ARG;
  return launch_pack_fp8((uint8_t*)d_dst, (const uint8_t*)d_src, rows, cols, (hipStream_t)stream) == 0 ? DG_OK
                                                                                                      : DG_ERR_HIP;
}

int dg_pack_weight_mxfp4(void* d_dst, const void* d_codes, const void* d_scales, int64_t rows, int64_t cols,
                         void* stream) {
  if (!d_dst || !d_codes || !d_scales || rows <= 0 || cols <= 0 || rows % 16 || cols % 64)
    return DG_ERR_INVALID_ARG;
  return launch_pack_mxfp4((uint8_t*)d_dst, (const uint8_t*)d_codes, (const uint8_t*)d_scales, rows, cols,
                           (hipStream_t)stream) == 0
             ? DG_OK
             : DG_ERR_HIP;
}

int dg_init_canvas(const dg_model_config* cfg, dg_canvas* cv, int32_t block, void* stream) {
  DG_TRY(check_config(cfg));
  if (!cv || !cv->tokens || !cv->seeds || cv->batch < 1 || cv->canvas < 1 || block < 0) return DG_ERR_INVALID_ARG;
  return launch_init_canvas(cv->tokens, cv->seeds, cv->batch, cv->canvas, block, cfg->vocab, (hipStream_t)stream) == 0
             ? DG_OK
             : DG_ERR_HIP;
}

int dg_encode_append(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache, const int32_t* d_tokens,
                     int32_t batch, int32_t n_tokens, void* d_ws, size_t ws_bytes, void* stream) {
  return dg_encode_append_traced(cfg, w, cache, d_tokens, batch, n_tokens, d_ws, ws_bytes, stream, nullptr);
}

int dg_encode_append_traced(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache,
                            const int32_t* d_tokens, int32_t batch, int32_t n_tokens, void* d_ws, size_t ws_bytes,
                            void* stream, dg_trace* trace) {
  return encode_impl(cfg, w, cache, d_tokens, batch, n_tokens, d_ws, ws_bytes, stream, trace, nullptr, nullptr);
}

int dg_test_encode_append(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache,
                          const int32_t* d_tokens, int32_t batch, int32_t n_tokens, const int32_t* d_force_ids,
                          float* d_router_logits, void* d_ws, size_t ws_bytes, void* stream) {
  return encode_impl(cfg, w, cache, d_tokens, batch, n_tokens, d_ws, ws_bytes, stream, nullptr, d_force_ids,
                     d_router_logits);
}

}  // extern "C"

static int encode_impl(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache, const int32_t* d_tokens,
                       int32_t batch, int32_t n_tokens, void* d_ws, size_t ws_bytes, void* stream, dg_trace* trace,
                       const int32_t* force_ids, float* router_out) {
  DG_TRY(check_config(cfg));
  DG_TRY(check_weights(cfg, w));
  if (batch < 1 || n_tokens < 1 || !d_tokens) return DG_ERR_INVALID_ARG;
  DG_TRY(check_cache(cfg, cache, batch));
  if ((int64_t)cache->length + n_tokens > cache->capacity) return DG_ERR_KV_CAPACITY;
  Ctx c;
  c.s = shape_of(cfg);
  c.p = make_plan(c.s, batch, 1);
  DG_TRY(check_ws(c.p, d_ws, ws_bytes));
  const int chunk = std::max(1, std::min(c.p.T, std::min(kMaxRoutePairs / c.s.k, route_max_tokens())) / batch);
  c.ws = (char*)d_ws;
  c.st = (hipStream_t)stream;
  c.w = w;
  c.tr = trace;
  // test path: per-layer routes and router logits are indexed by the token
  // rows of one chunk, so the whole encode must fit in one
  if ((force_ids || router_out) && n_tokens > chunk) return DG_ERR_UNSUPPORTED;
  c.force_ids = force_ids;
  c.router_out = router_out;
  for (int done = 0; done < n_tokens; done += chunk) {
    const int nc = std::min(chunk, n_tokens - done);
    // gather this chunk's tokens [batch][nc] into the workspace token buffer
    int32_t* tok = c.at<int32_t>(c.p.ids);  // reused: ids are rewritten per layer after embedding
    for (int b = 0; b < batch; ++b)
      DG_TRY(launch_copy_i32(tok + b * nc, d_tokens + (int64_t)b * n_tokens + done, nc, c.st));
    DG_TRY(launch_embed_norm(c.s.dt == DG_DTYPE_BF16, tok, w->embed, nullptr, 0, 0, c.at<float>(c.p.x),
                             c.at<void>(c.p.n), batch * nc, c.s.d, c.s.eps, c.st));
    DG_TRY(run_layers(c, cache, batch, nc, cache->length, true));
    cache->length += nc;
  }
  return DG_OK;
}

extern "C" {

int dg_denoise_step(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache, dg_canvas* cv,
                    const dg_step_params* p, void* d_ws, size_t ws_bytes, void* stream) {
  return dg_denoise_step_traced(cfg, w, cache, cv, p, d_ws, ws_bytes, stream, nullptr);
}

int dg_denoise_step_traced(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache, dg_canvas* cv,
                           const dg_step_params* p, void* d_ws, size_t ws_bytes, void* stream, dg_trace* trace) {
  return denoise_impl(cfg, w, cache, cv, p, d_ws, ws_bytes, stream, trace, nullptr, nullptr, nullptr);
}

}  // extern "C"

// Scratch of dg_denoise_step_noalloc: a module global, so every GPU the
// library runs on holds its own copy, allocated when the code object loads
// there and kept until the process ends.  Host code never uses the array's
// name as an address (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and kept in noalloc_ptr[device].
static __device__ __align__(256) unsigned char scratch[DG_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call there).
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DG_ERR_HIP;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (!noalloc_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DG_ERR_HIP;
    noalloc_ptr[dev] = ptr;
  }
  *out = noalloc_ptr[dev];
  return DG_OK;
}
}  // namespace

extern "C" {

int dg_denoise_step_noalloc(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache,
                            dg_canvas* cv, const dg_step_params* p, void* stream) {
  DG_TRY(check_config(cfg));
  DG_TRY(check_canvas(cv, true));
  // the step-only plan of this call must fit the static scratch
  if (make_plan(shape_of(cfg), cv->batch, cv->canvas, true).total > (size_t)DG_NOALLOC_SCRATCH_BYTES)
    return DG_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  DG_TRY(noalloc_scratch(&ws));
  return denoise_impl(cfg, w, cache, cv, p, ws, (size_t)DG_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, nullptr,
                      nullptr, true);
}

int dg_test_denoise_step(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache, dg_canvas* cv,
                         const dg_step_params* p, const int32_t* d_force_ids, float* d_router_logits, float* d_logits,
                         const float* d_teacher_x, float* d_layer_out, void* d_ws, size_t ws_bytes, void* stream) {
  return denoise_impl(cfg, w, cache, cv, p, d_ws, ws_bytes, stream, nullptr, d_force_ids, d_router_logits, d_logits,
                      false, d_teacher_x, d_layer_out);
}

}  // extern "C"

static int denoise_impl(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache, dg_canvas* cv,
                        const dg_step_params* p, void* d_ws, size_t ws_bytes, void* stream, dg_trace* trace,
                        const int32_t* force_ids, float* router_out, float* logits_out, bool step_only,
                        const float* teacher_x, float* layer_out) {
  DG_TRY(check_config(cfg));
  DG_TRY(check_weights(cfg, w));
  DG_TRY(check_canvas(cv, true));
  DG_TRY(check_step(p));
  DG_TRY(check_denoise_cache(cfg, cache, cv));
  Ctx c;
  c.s = shape_of(cfg);
  c.p = make_plan(c.s, cv->batch, cv->canvas, step_only);
  DG_TRY(check_ws(c.p, d_ws, ws_bytes));
  if ((int64_t)cv->batch * cv->canvas > std::min(kMaxStepTokens, route_max_tokens())) return DG_ERR_UNSUPPORTED;
  c.ws = (char*)d_ws;
  c.st = (hipStream_t)stream;
  c.w = w;
  if (trace && (!trace->events || !trace->phase || trace->capacity < 0)) return DG_ERR_INVALID_ARG;
  c.tr = trace;
  c.force_ids = force_ids;
  c.router_out = router_out;
  c.teacher_x = teacher_x;
  c.layer_out = layer_out;
  const int T = cv->batch * cv->canvas;
  DG_TRY(embed_canvas(c, cv, p));
  if (layer_out)  // test path: the embedding (+ self-conditioning) output
    DG_TRY(launch_copy_i32(reinterpret_cast<int32_t*>(layer_out), c.at<int32_t>(c.p.x), T * c.s.d, c.st));
  DG_TRY(run_layers(c, cache, cv->batch, cv->canvas, cache->length, false));
  if (teacher_x)  // test path: the LM head reads the given final residual
    DG_TRY(launch_set_norm(c.s.dt == DG_DTYPE_BF16, teacher_x + (int64_t)c.s.L * T * c.s.d, c.at<float>(c.p.x),
                           c.at<void>(c.p.n), T, c.s.d, c.s.eps, c.st));
  DG_TRY(lm_head(c, cv, p, logits_out, true));
  return sample_and_select(c, cv, p);
}

extern "C" {

int dg_ar_step(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache, const int32_t* d_tokens,
               int32_t batch, int32_t* d_next, void* d_ws, size_t ws_bytes, void* stream) {
  return ar_impl(cfg, w, cache, d_tokens, batch, d_next, nullptr, d_ws, ws_bytes, stream);
}

int dg_test_ar_step(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache, const int32_t* d_tokens,
                    int32_t batch, int32_t* d_next, float* d_logits, void* d_ws, size_t ws_bytes, void* stream) {
  if (!d_logits) return DG_ERR_INVALID_ARG;
  return ar_impl(cfg, w, cache, d_tokens, batch, d_next, d_logits, d_ws, ws_bytes, stream);
}

int dg_commit_block(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache, dg_canvas* cv,
                    const dg_step_params* p, void* d_ws, size_t ws_bytes, void* stream) {
  DG_TRY(check_config(cfg));
  DG_TRY(check_canvas(cv, true));
  DG_TRY(check_step(p));
  if (!cv->committed) return DG_ERR_INVALID_ARG;
  DG_TRY(check_cache(cfg, cache, cv->batch));
  if ((int64_t)cache->length + cv->canvas > cache->capacity) return DG_ERR_KV_CAPACITY;
  const int T = cv->batch * cv->canvas;
  DG_TRY(launch_copy_i32(cv->committed, cv->argmax, T, (hipStream_t)stream));
  DG_TRY(dg_encode_append(cfg, w, cache, cv->committed, cv->batch, cv->canvas, d_ws, ws_bytes, stream));
  return launch_init_canvas(cv->tokens, cv->seeds, cv->batch, cv->canvas, p->block + 1, cfg->vocab,
                            (hipStream_t)stream) == 0
             ? DG_OK
             : DG_ERR_HIP;
}

int dg_commit_and_step(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache, dg_canvas* cv,
                       const dg_step_params* p_commit, const dg_step_params* p_next, void* d_ws, size_t ws_bytes,
                       void* stream) {
  DG_TRY(check_config(cfg));
  DG_TRY(check_weights(cfg, w));
  DG_TRY(check_canvas(cv, true));
  DG_TRY(check_step(p_commit));
  DG_TRY(check_step(p_next));
  if (!cv->committed || p_next->t != 0 || p_next->block != p_commit->block + 1) return DG_ERR_INVALID_ARG;
  if (cv->sc_probs) return DG_ERR_UNSUPPORTED;
  DG_TRY(check_cache(cfg, cache, cv->batch));
  const int C = cv->canvas, Tseg = cv->batch * C;
  // the committed rows are appended, the next canvas's rows follow as scratch
  if ((int64_t)cache->length + 2 * C > cache->capacity) return DG_ERR_KV_CAPACITY;
  Ctx c;
  c.s = shape_of(cfg);
  c.p = make_plan(c.s, cv->batch, C);
  DG_TRY(check_ws(c.p, d_ws, ws_bytes));
  if (2 * Tseg > c.p.T || 2 * Tseg > std::min(kMaxStepTokens, route_max_tokens())) return DG_ERR_UNSUPPORTED;
  c.ws = (char*)d_ws;
  c.st = (hipStream_t)stream;
  c.w = w;
  const bool bf = c.s.dt == DG_DTYPE_BF16;
  DG_TRY(launch_copy_i32(cv->committed, cv->argmax, Tseg, c.st));
  DG_TRY(launch_init_canvas(cv->tokens, cv->seeds, cv->batch, C, p_next->block, cfg->vocab, c.st));
  for (int seg = 0; seg < 2; ++seg)
    DG_TRY(launch_embed_norm(bf, seg == 0 ? cv->committed : cv->tokens, w->embed, nullptr, 0, 0,
                             c.at<float>(c.p.x) + (size_t)seg * Tseg * c.s.d,
                             c.at<char>(c.p.n) + (size_t)seg * Tseg * c.s.d * c.s.act, Tseg, c.s.d, c.s.eps, c.st));
  DG_TRY(run_layers(c, cache, cv->batch, C, cache->length, true, true, true));
  cache->length += C;
  c.head_row0 = Tseg;
  DG_TRY(lm_head(c, cv, p_next, nullptr));
  return sample_and_select(c, cv, p_next);
}

const char* dg_status_string(int status) {
  switch (status) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARG: return "invalid argument";
    case DG_ERR_UNSUPPORTED: return "unsupported configuration";
    case DG_ERR_KV_CAPACITY: return "KV cache capacity exceeded";
    case DG_ERR_WORKSPACE: return "workspace too small";
    case DG_ERR_HIP: return "HIP launch error";
    case DG_ERR_SCRATCH_LIMIT: return "step needs more than the no-allocation scratch (DG_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int dg_test_sample_from_logits(const dg_model_config* cfg, const float* d_logits, dg_canvas* cv,
                               const dg_step_params* p, void* d_ws, size_t ws_bytes, void* stream) {
  DG_TRY(check_config(cfg));
  DG_TRY(check_canvas(cv, true));
  DG_TRY(check_step(p));
  if (!d_logits) return DG_ERR_INVALID_ARG;
  Ctx c;
  c.s = shape_of(cfg);
  c.p = make_plan(c.s, cv->batch, cv->canvas);
  DG_TRY(check_ws(c.p, d_ws, ws_bytes));
  c.ws = (char*)d_ws;
  c.st = (hipStream_t)stream;
  c.w = nullptr;
  LmArgs lm;
  memset(&lm, 0, sizeof(lm));
  lm.part_f = c.at<float4>(c.p.lm_f);
  lm.part_i = c.at<int2>(c.p.lm_i);
  lm.p_side = cv->p_side;
  lm.p_side_f32 = cfg->dtype != DG_DTYPE_BF16;
  lm.inv_tau = 1.0f / dg_temperature(p->t, p->n_steps);
  lm.seeds = cv->seeds;
  lm.canvas = cv->canvas;
  lm.step = p->t;
  lm.block = p->block;
  lm.vocab = c.s.V;
  DG_TRY(launch_lm_partials_from_logits(d_logits, cv->batch * cv->canvas, lm, c.st));
  return sample_and_select(c, cv, p);
}

int dg_test_route_from_logits(const dg_model_config* cfg, const float* d_logits, int32_t T, int32_t* d_ids, float* d_w,
                              int32_t* d_row_token, int32_t* d_inv, int32_t* d_offsets, void* d_ws, size_t ws_bytes,
                              void* stream) {
  DG_TRY(check_config(cfg));
  if (!d_logits || !d_ids || !d_w || !d_row_token || !d_inv || !d_offsets || T < 1) return DG_ERR_INVALID_ARG;
  const Shape s = shape_of(cfg);
  if (T > std::min(kMaxStepTokens, route_max_tokens())) return DG_ERR_UNSUPPORTED;
  const Plan p = make_plan(s, 1, T);
  DG_TRY(check_ws(p, d_ws, ws_bytes));
  char* ws = (char*)d_ws;
  hipStream_t st = (hipStream_t)stream;
  const int bm = s.dt == DG_DTYPE_BF16 ? kMoeBM : kSimpleBM;
  DG_TRY(launch_topk(d_logits, 1, 0, T, s.E, s.k, nullptr, d_ids, d_w, nullptr, st));
  DG_TRY(launch_route_sort(d_ids, T, s.k, s.E, s.n_sh, bm, d_row_token, d_inv, d_offsets,
                           reinterpret_cast<GemmTile*>(ws + p.tiles), reinterpret_cast<int32_t*>(ws + p.n_tiles),
                           reinterpret_cast<int32_t*>(ws + p.rcnt), st));
  return DG_OK;
}

int dg_test_forward_logits(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache, dg_canvas* cv,
                           const dg_step_params* p, const int32_t* d_force_ids, float* d_router_logits,
                           float* d_logits, void* d_ws, size_t ws_bytes, void* stream) {
  DG_TRY(check_config(cfg));
  DG_TRY(check_weights(cfg, w));
  DG_TRY(check_canvas(cv, false));
  DG_TRY(check_step(p));
  DG_TRY(check_denoise_cache(cfg, cache, cv));
  if (!d_logits) return DG_ERR_INVALID_ARG;
  Ctx c;
  c.s = shape_of(cfg);
  c.p = make_plan(c.s, cv->batch, cv->canvas);
  DG_TRY(check_ws(c.p, d_ws, ws_bytes));
  c.ws = (char*)d_ws;
  c.st = (hipStream_t)stream;
  c.w = w;
  if ((int64_t)cv->batch * cv->canvas > std::min(kMaxStepTokens, route_max_tokens())) return DG_ERR_UNSUPPORTED;
  c.force_ids = d_force_ids;
  c.router_out = d_router_logits;
  DG_TRY(embed_canvas(c, cv, p));
  DG_TRY(run_layers(c, cache, cv->batch, cv->canvas, cache->length, false));
  return lm_head(c, cv, p, d_logits);
}

}  // extern "C"
