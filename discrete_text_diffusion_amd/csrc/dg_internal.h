// Host/device shared launch descriptors of the denoising-step kernels.
#pragma once
#include <stdint.h>

#include "dg_common.h"

// One row tile of a (possibly grouped) GEMM: rows [row0, row0 + nrows) of the
// output, all belonging to weight group `group` (an expert, or one of the
// shared expert's virtual slices).  span: (index of the group's first tile in
// the list << 16) | the group's tile count (tile lists hold fewer than 65536
// tiles, a group fewer than 65536).
struct GemmTile {
  int32_t group, row0, nrows, span;
};

enum GemmEpi : int32_t {
  EPI_STORE_F32 = 0,  // out_f32[split][row][n] = alpha * acc
  EPI_RESID = 1,      // out_f32[row][n] += acc
  EPI_GEGLU = 2,      // out_act[row][n] = act(gelu(acc_gate) * acc_up)
  EPI_GELU = 3,       // out_act[row][n] = act(gelu(acc))
  EPI_QKV = 4,        // q/k/v split, RoPE on q and k, activation rounding, k/v to their store
  EPI_STORE_ACT = 5,  // out_act[row][n] = act(alpha * acc)
  EPI_GEGLU_PARTS = 6,  // GeGLU K-split: out_f32[split][row][n] = acc_gate,
                        // out_f32[n_split + split][row][n] = acc_up
};

enum ActKind : int32_t {
  ACT_BF16 = 0,         // bf16 rows
  ACT_F32 = 1,          // fp32 rows, rounded to bf16 when staged (MFMA path)
};

struct QkvEpi {
  void* q;            // [T][q_dim]
  void* k;            // k destination base (cache or canvas store)
  void* v;
  int32_t q_dim, kv_dim, d_head, n_kv;
  int64_t kv_b_stride;  // elements between sequences of the k/v store
  int64_t kv_h_stride;  // elements between kv heads (= capacity * d_head)
  int32_t kv_row0;      // first row written inside each head (cache length for append)
  int32_t v_pitch;      // row pitch of the transposed V store ([d_head][rows] per head)
  int32_t seq_len;      // tokens per sequence in this call
  int32_t pos0;         // absolute position of the first token of each sequence
  float rope_base;
  const float2* rope;   // [seq_len][d_head / 2] RoPE (cos, sin) of positions pos0 + i (launch_rope_table)
};

struct GemmArgs {
  // activations (the MFMA B operand): rows of length >= K
  const void* act;
  int64_t act_ld;
  int32_t act_kind;
  const int32_t* row_map;  // output row -> activation row (null: identity)
  // weights (the MFMA A operand), packed tiles; groups < n_main use w0/w1
  // with w_group_stride, the others use w0_alt/w1_alt.
  const void* w0;
  const void* w1;
  int64_t w_group_stride;
  const void* w0_alt;
  const void* w1_alt;
  int64_t w_alt_stride;
  int32_t n_main;
  // fp8 weights: E4M3 codes in 16 x 32 tiles of 512 B (8 codes per lane, A-operand
  // lane order), each output feature n scaled by an fp32 factor: main group g
  // reads ws0/ws1[g * ws_group_stride + n], alt group c ws0_alt/ws1_alt[c * ws_alt_stride + n]
  int32_t w_fp8;
  // MXFP4 weights: 16 x 64 superblocks of 544 B (E2M1 codes in A-operand lane
  // order, then the 32 E8M0 block scales), see dg_pack_weight_mxfp4
  int32_t w_mx4;
  const float* ws0;
  const float* ws1;
  int64_t ws_group_stride;
  const float* ws0_alt;
  const float* ws1_alt;
  int64_t ws_alt_stride;
  int32_t kt_main;     // 32-wide k tiles per 16-row tile of a main-group matrix
  int32_t kt_alt;      // same for alt groups
  int32_t kt_off_alt;  // alt group c starts at k tile c * kt_off_alt
  int32_t K, N;
  // row tiles
  const GemmTile* tiles;  // null: dense rows [0, M)
  const int32_t* n_tiles_dev;
  int32_t max_tiles;
  int32_t M;
  int32_t n_fb;      // feature blocks
  int32_t n_split;   // K splits
  int32_t k_split;   // K per split (multiple of the K chunk)
  int32_t tile_fastest;
  int32_t group_major;  // grouped GEMMs: blocks ordered (group, feature block, tile of the group)
  int32_t nblocks;   // launched blocks (multiple of 8)
  // epilogue
  int32_t epi;
  float* out_f32;
  int64_t ldo;
  int64_t split_stride;
  void* out_act;
  float alpha;
  QkvEpi qkv;
};

// LM-head epilogue outputs: per (row, 256-id vocabulary tile) statistics.
struct LmArgs {
  float4* part_f;    // [rows][n_vt]: (m_k, S_k, T_k, zmax_k) of a = z / tau
  int2* part_i;      // [rows][n_vt]: (candidate id at u2, argmax id)
  void* p_side;      // [rows][V] exp(a - m_k) in bf16 or fp32 (null: not written)
  int32_t p_side_f32;
  float* logits;     // [rows][V] fp32 z (test path; null: not written)
  float inv_tau;
  const uint64_t* seeds;  // [batch]
  int32_t canvas;         // rows per canvas
  int32_t step, block;
  int32_t vocab;
};

// Launchers
// k_gemm.hip
// RoPE (cos, sin) of pairs j < d_head / 2 at positions pos0 + i, i < rows:
// out[i][j], the angle formed in fp64 (every layer's QKV epilogue reads it).
int launch_rope_table(float2* out, int rows, int d_head, int pos0, float rope_base, hipStream_t s);
int launch_wsgemm(const GemmArgs& a, int bm, int nwt, int kc, bool geglu, hipStream_t s);
// Row-resident GEMM (M rows in groups of 256, 256-feature blocks; 128 with
// scaled activations, whose K and k_split are multiples of 256): fp32
// partials (EPI_STORE_F32), or with lm != null the LM-head statistics.
int launch_rowgemm(const GemmArgs& a, const LmArgs* lm, hipStream_t s);
// Sum of K-split fp32 partials part[s][row][n] (pitch ldp), then a.epi.
// h[row][n] = bf16(gelu(sum of gate partials) * sum of up partials) over the
// EPI_GEGLU_PARTS layout (splits summed in split order)
int launch_geglu_splits(const float* part, int n_split, int64_t split_stride, int rows, int N, void* out, int ldo,
                        hipStream_t s);
int launch_split_epilogue(const GemmArgs& a, const float* part, int n_split, int64_t split_stride, int ldp,
                          hipStream_t s);
int launch_gemm_simple(const GemmArgs& a, hipStream_t s);
int launch_pack_bf16(bf16_t* dst, const bf16_t* src, int64_t rows, int64_t cols, int transposed, hipStream_t s);
int launch_pack_fp8(uint8_t* dst, const uint8_t* src, int64_t rows, int64_t cols, hipStream_t s);
int launch_pack_mxfp4(uint8_t* dst, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                      hipStream_t s);
int launch_lm_partials_from_logits(const float* logits, int rows, const LmArgs& lm, hipStream_t s);
// k_route.hip
int launch_topk(const float* part, int n_split, int64_t split_stride, int T, int E, int k, const int32_t* forced,
                int32_t* ids, float* w, float* r_out, hipStream_t s);
int route_max_tokens();
// int32 words of per-chunk counts the sort needs for T tokens (0: one workgroup)
int route_chunk_words(int T);
int launch_route_sort(const int32_t* ids, int T, int k, int E, int n_sh, int bm, int32_t* row_token, int32_t* inv,
                      int32_t* offsets, GemmTile* tiles, int32_t* n_tiles, int32_t* chunk_counts, hipStream_t s);
// k_attn.hip
int launch_attention(int dtype, const void* q, int64_t q_ld, const void* k, const void* v, int64_t s_seq,
                     int64_t s_head, int vp, int n_keys, int n_prefix, int causal, int seq_len, int n_seq, int n_q,
                     int n_kv, int d, int n_split, float* part_o, float2* part_ml, void* out, hipStream_t s);
// k_misc.hip
int launch_embed_norm(int dtype, const int32_t* tok, const void* emb, const float* add, int n_add, int64_t add_stride,
                      float* x, void* n, int T, int d, float eps, hipStream_t s);
// x = src; n = RMSNorm(x) per row (T rows of d)
int launch_set_norm(int dtype, const float* src, float* x, void* n, int T, int d, float eps, hipStream_t s);
int launch_resid_norm(int dtype, float* x, const float* part, int n_split, int64_t split_stride, void* n, int T, int d,
                      float eps, hipStream_t s);
int launch_combine_norm(int dtype, float* x, const float* Y, const int32_t* inv, const float* w, int T, int k, int n_sh,
                        void* n, int d, float eps, hipStream_t s);
int launch_reduce_splits(int dtype, const float* part, int n_split, int64_t split_stride, int64_t n_elems, void* out,
                         hipStream_t s);
int launch_init_canvas(int32_t* tokens, const uint64_t* seeds, int B, int C, int block, int vocab, hipStream_t s);
int launch_copy_i32(int32_t* dst, const int32_t* src, int n, hipStream_t s);
// k_sampler.hip
int launch_row_merge(const float4* part_f, const int2* part_i, int n_vt, int rows, int C, const uint64_t* seeds,
                     int step, int block, float* H, int32_t* sample, int32_t* argmax, float* p_scale, hipStream_t s);
// p_side *= its (row, 256-id tile) factor, in place (the carried tempered distribution)
int launch_normalize_side(int bf16, void* p, const float* scale, int rows, int vocab, hipStream_t s);
int launch_select(const float* H, const int32_t* sample, const int32_t* argmax, int32_t* prev_argmax, int32_t* tokens,
                  uint8_t* accepted, int32_t* n_accepted, float* mean_entropy, int32_t* stop, uint32_t* flags,
                  const uint64_t* seeds, int B, int C, int step, int block, int vocab, int adaptive, float bound,
                  float threshold, hipStream_t s);
