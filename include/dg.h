/*
 * dg.h — C ABI of the MI355X (gfx950) block-diffusion decoding step.
 *
 * The library runs, on one GPU, the three calls of the generation pipeline
 * described in the DiffusionGemma Technical Report (digest by METAL MEDIA,
 * Figure 4): causal context encoding into a KV cache, one denoising step over
 * a canvas with bidirectional attention inside the canvas plus attention to
 * the cache, and encode & append of a finished canvas.  The sampler follows
 * the DiffusionGemma docs' recommended serving configuration table (Google AI
 * for Developers, DiffusionGemma page): temperature linear 0.8 -> 0.4 over
 * the step budget, lowest-entropy tokens accepted while their summed entropy
 * stays within the 0.1 bound, the rest fully re-noised, adaptive stop when
 * the canvas-mean entropy is under 0.005 and two consecutive argmax
 * predictions agree.  Self-conditioning (LLM-Wiki digest of the PyTorchKR
 * review, key points; report Table 1's self-conditioning MLP) feeds the
 * previous step's distribution back as an expected embedding through a small
 * MLP.
 *
 * Conventions
 *  - Every pointer named d_* or documented "device" is device memory owned by
 *    the caller; host structs are read during the call only.  The library
 *    allocates nothing and keeps no state between calls.
 *  - Calls enqueue work on `stream` (a hipStream_t) and return; results are
 *    valid after the stream is synchronised.  No call synchronises, copies
 *    to the host or records memset nodes, so the sequence of calls of a fixed
 *    number of steps can be captured in a HIP graph.
 *  - Return value: DG_OK (0) or a negative DG_ERR_*.  Argument errors are
 *    found on the host before anything is enqueued; nothing is written then.
 *  - Token ids are int32.  Matrices named [rows][cols] are row-major unless
 *    the "weight layout" is stated (see dg_pack_weight).
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_OK 0
#define DG_ERR_INVALID_ARG (-1)
#define DG_ERR_UNSUPPORTED (-2)
#define DG_ERR_KV_CAPACITY (-3)
#define DG_ERR_WORKSPACE (-4)
#define DG_ERR_HIP (-5)
#define DG_ERR_SCRATCH_LIMIT (-6) /* dg_denoise_step_noalloc: the step needs more scratch than it holds */

#define DG_DTYPE_F32 0
#define DG_DTYPE_BF16 1
#define DG_DTYPE_FP8_E4M3 2 /* weights only: OCP E4M3 codes with per-output-feature fp32 scales */
#define DG_DTYPE_MXFP4 3     /* expert weights only: OCP MXFP4 (E2M1 codes, an E8M0 scale per 32 inputs) */

/* canvas.flags bits (device side) */
#define DG_FLAG_NONFINITE 1u /* some entropy of the step was NaN or infinite */

/* Model shape.  dtype applies to every weight and to activation storage:
 * DG_DTYPE_BF16 models round GEMM inputs (norm outputs, attention output,
 * GeGLU hidden, q/k/v) to bf16 and accumulate in fp32; DG_DTYPE_F32 models
 * round nothing.  Requirements: n_q_heads % n_kv_heads == 0,
 * d_shared % d_expert == 0, vocab % 256 == 0; bf16 models also need
 * d_head == 256, n_q/n_kv in {1, 2, 4}, d_model, d_expert, d_shared,
 * d_selfcond and n_q_heads*d_head multiples of 64, n_experts % 16 == 0.
 * expert_dtype (routed and shared expert matrices) and lm_dtype (LM head)
 * equal dtype, or are DG_DTYPE_FP8_E4M3 in a bf16 model: each stored weight
 * is then an OCP E4M3 code whose value, times the fp32 scale of its output
 * feature, is the weight (dequantised exactly to bf16 inside the kernels,
 * bf16 MFMA, the scale applied to the fp32 sum); fp8 experts need
 * d_model % 128 == 0.  expert_dtype may also be DG_DTYPE_MXFP4 in a bf16
 * model (4-bit expert weights, the counterpart of the NVFP4 kernels of
 * euno.news, "how it was built"; the format is OCP Microscaling Formats
 * v1.0, MXFP4: along each matrix row, every
 * block of 32 consecutive inputs shares one E8M0 scale 2^(e - 127) and each
 * weight is that scale times an FP4 E2M1 element, 0, +-0.5, +-1, +-1.5, +-2,
 * +-3, +-4, +-6): the kernels convert each element times its block scale to
 * bf16, which is exact for scale codes 1..254 (code 0 is read as zero, code
 * 255, NaN, is not a valid input), and feed the bf16 MFMA; MXFP4 experts need
 * d_model, d_expert and d_shared multiples of 64.  Otherwise
 * DG_ERR_UNSUPPORTED. */
typedef struct dg_model_config {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, d_head;
  int32_t n_experts, top_k, d_expert, d_shared, vocab, d_selfcond;
  int32_t dtype;
  float rope_base; /* RoPE base (RoFormer pairing (2j, 2j+1)) */
  float norm_eps;  /* RMSNorm epsilon; gain 1 */
  int32_t expert_dtype, lm_dtype;
} dg_model_config;

/* Weights of one layer, device pointers, each in the weight layout of its
 * logical [out][in] matrix (bf16, or fp8 codes packed by dg_pack_weight_fp8)
 * or plain row-major (fp32):
 *   wqkv [(n_q + 2 n_kv) d_head][d_model]  rows: q heads, then k heads, then v heads
 *   wo   [d_model][n_q d_head]
 *   wr   [n_experts][d_model]              router
 *   sh_g, sh_u [d_shared][d_model]; sh_d [d_model][d_shared]   shared expert (GeGLU)
 *   ex_g, ex_u [n_experts][d_expert][d_model]; ex_d [n_experts][d_model][d_expert]
 *     (each expert's matrix packed separately, experts back to back)
 * fp8 experts: per-output-feature fp32 scales ex_g_scale, ex_u_scale
 * [n_experts][d_expert], ex_d_scale [n_experts][d_model], sh_g_scale,
 * sh_u_scale [d_shared], sh_d_scale [d_model] (16-byte aligned); NULL
 * otherwise.  MXFP4 experts: every expert matrix in the MXFP4 layout of
 * dg_pack_weight_mxfp4 (its block scales inside), the *_scale pointers NULL. */
typedef struct dg_layer_weights {
  const void* wqkv;
  const void* wo;
  const void* wr;
  const void* sh_g;
  const void* sh_u;
  const void* sh_d;
  const void* ex_g;
  const void* ex_u;
  const void* ex_d;
  const float* ex_g_scale;
  const float* ex_u_scale;
  const float* ex_d_scale;
  const float* sh_g_scale;
  const float* sh_u_scale;
  const float* sh_d_scale;
} dg_layer_weights;

typedef struct dg_weights {
  const void* embed;   /* [vocab][d_model] row-major (token gather) */
  const void* embed_t; /* E^T [d_model][vocab] in weight layout (self-conditioning contraction);
                          may be NULL if no step uses self-conditioning */
  const void* lm_head; /* [vocab][d_model] in weight layout (untied head) */
  const void* sc_up;   /* [d_selfcond][d_model] */
  const void* sc_down; /* [d_model][d_selfcond] */
  const dg_layer_weights* layers; /* HOST array of n_layers */
  float lm_scale;      /* logits z = lm_scale * (RMSNorm(x) W_lm^T) */
  const float* lm_head_scale; /* fp8 LM head: [vocab] fp32 per-id scales (16-byte aligned); else NULL */
} dg_weights;

/* KV cache, rows [0, length) valid:
 *   k: [n_layers][batch][n_kv][capacity][d_head]   post-RoPE keys, model dtype
 *   v: [n_layers][batch][n_kv][d_head][capacity]   values, model dtype, stored
 *      transposed so that attention streams contiguous runs of keys per
 *      dimension.
 * bf16 models: capacity a multiple of 8 (else DG_ERR_UNSUPPORTED).
 * Rows [length, capacity) are scratch: the denoiser writes its canvas K/V to
 * rows [length, length + canvas) without changing `length`.
 * `length` is host bookkeeping updated by the appending calls at enqueue time. */
typedef struct dg_kv_cache {
  void* k;
  void* v;
  int32_t batch, capacity, length;
} dg_kv_cache;

/* One batch of canvases (all device pointers unless stated).
 *   tokens       [B][C]  in: the canvas of step t; out: the canvas for t + 1
 *   seeds        [B]     sampler seed per canvas (Philox4x32-10 key)
 *   sc_probs     [B*C][vocab] fp32, optional external self-conditioning input
 *                (normalised probabilities); used whenever non-NULL
 *   p_side       [B*C][vocab] model dtype, and p_scale [vocab/256][B*C] fp32
 *                (tile-major): written by every step, p_side = the step's
 *                tempered distribution softmax(z / tau_t) (formed as
 *                exp(a - m_k) times the per-tile factor exp(m_k - m)/S, which
 *                p_scale keeps), read by the next step (t >= 1) as its
 *                self-conditioning input.  NULL: no self-conditioning carried
 *                between steps.
 *   entropy [B*C] fp32, sample/argmax/prev_argmax [B*C] int32, accepted [B*C]
 *   uint8, n_accepted/stop [B] int32, mean_entropy [B] fp32, flags [B] uint32.
 *   prev_argmax holds the previous step's argmax (read by the stop test at
 *   t >= 1, then overwritten).
 *   committed    [B][C]  out of dg_commit_block: the tokens appended. */
typedef struct dg_canvas {
  int32_t batch, canvas;
  int32_t* tokens;
  const uint64_t* seeds;
  const float* sc_probs;
  void* p_side;
  float* p_scale;
  float* entropy;
  int32_t* sample;
  int32_t* argmax;
  int32_t* prev_argmax;
  uint8_t* accepted;
  int32_t* n_accepted;
  float* mean_entropy;
  int32_t* stop;
  uint32_t* flags;
  int32_t* committed;
} dg_canvas;

/* Step parameters.  t is 0-based within the block's budget of n_steps; the
 * temperature is dg_temperature(t, n_steps).  `block` indexes the canvas
 * within the generation (it is part of the Philox counter).  Use
 * DG_ENTROPY_BOUND / DG_STOP_THRESHOLD for the pages' values. */
typedef struct dg_step_params {
  int32_t t, n_steps, block, adaptive;
  float entropy_bound;
  float stop_threshold;
} dg_step_params;

#define DG_ENTROPY_BOUND 0.1f
#define DG_STOP_THRESHOLD 0.005f

/* Linear temperature schedule 0.8 -> 0.4 over the budget: tau_t =
 * 0.8 + (0.4 - 0.8) t/(n-1) in fp64 rounded once to fp32; 0.8 when n == 1.
 * (DiffusionGemma docs, recommended serving configuration, temperature row;
 * report Figure 9: larger budgets anneal more mildly.) */
float dg_temperature(int32_t t, int32_t n_steps);

/* Workspace bytes for calls on `batch` sequences with at most
 * `max_canvas` canvas tokens per sequence in a denoising step.  Encoding
 * processes its input in chunks that fit the same workspace. */
size_t dg_workspace_bytes(const dg_model_config* cfg, int32_t batch, int32_t max_canvas);

/* Pack a logical row-major bf16 matrix [rows][cols] (device) into the weight
 * layout: 16-row x 32-column tiles of 1 KiB, tile (r/16, c/32) at element
 * offset ((r/16)*(cols/32) + c/32)*512, element (r, c) inside it at
 * (((c%32)/8)*16 + r%16)*8 + c%8.  rows % 16 == 0, cols % 32 == 0.
 * dst and src must not overlap.  fp32 weights are used as given (row-major). */
int dg_pack_weight_bf16(void* d_dst, const void* d_src, int64_t rows, int64_t cols, void* stream);

/* As dg_pack_weight_bf16 for the matrix [rows][cols] whose transpose is
 * given: d_src is row-major [cols][rows] (e.g. the embedding [vocab][d_model]
 * packed as E^T [d_model][vocab] for the self-conditioning contraction). */
int dg_pack_weight_bf16_transposed(void* d_dst, const void* d_src, int64_t rows, int64_t cols, void* stream);

/* Pack logical row-major E4M3 codes [rows][cols] (device, one byte each)
 * into the fp8 weight layout: 16-row x 32-column tiles of 512 B, tile
 * (r/16, c/32) at byte ((r/16)*(cols/32) + c/32)*512, code (r, c) inside it
 * at (((c%32)/8)*16 + r%16)*8 + c%8.  rows % 16 == 0, cols % 32 == 0. */
int dg_pack_weight_fp8(void* d_dst, const void* d_src, int64_t rows, int64_t cols, void* stream);

/* Pack an MXFP4 matrix [rows][cols] into the MXFP4 weight layout.  Inputs
 * (device): d_codes, one E2M1 element code per byte (low 4 bits; OCP MX v1.0
 * FP4 encoding S.EE.M), row-major [rows][cols]; d_scales, the E8M0 scale code
 * of each block of 32 consecutive columns, row-major [rows][cols / 32].
 * Output: superblocks of 16 rows x 64 columns, 544 B each, superblock
 * (r/16, c/64) at byte ((r/16)*(cols/64) + c/64)*544.  Inside one: byte
 * 8l + 4h + q (l = 0..63, h = 0..1, q = 0..3) holds the codes of row r%16 = l%16,
 * columns c%64 = 32h + 8(l/16) + 2q (low nibble) and + 1 (high nibble), i.e.
 * lane l's MFMA A-operand elements of the two 32-column halves; byte
 * 512 + 2(r%16) + h holds the scale code of row r, block (c/32) of half h.
 * Total size rows*cols*17/32 bytes.  rows % 16 == 0, cols % 64 == 0; the
 * buffers must not overlap. */
int dg_pack_weight_mxfp4(void* d_dst, const void* d_codes, const void* d_scales, int64_t rows, int64_t cols,
                         void* stream);

/* Fill canvas->tokens with uniform noise for `block` (Philox stream 0).
 * (euno.news, "what DiffusionGemma does": a canvas starts as random tokens;
 *  report Figure 3: the noise end is the uniform distribution.) */
int dg_init_canvas(const dg_model_config* cfg, dg_canvas* canvas, int32_t block, void* stream);

/* Context encoding / encode & append (report Figure 4, stages 1 and 3):
 * causally encode d_tokens [batch][n_tokens] at positions
 * cache->length .. + n_tokens - 1 of every sequence and append their K, V to
 * the cache; cache->length += n_tokens.  DG_ERR_KV_CAPACITY if the cache
 * would overflow (nothing written). */
int dg_encode_append(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache,
                     const int32_t* d_tokens, int32_t batch, int32_t n_tokens, void* d_ws,
                     size_t ws_bytes, void* stream);

/* One denoising step over the canvases (report Figure 4, stage 2): embedding
 * plus self-conditioning, the layer stack with bidirectional canvas attention
 * over [cache ; canvas] (the canvas K/V go to the cache's scratch rows
 * [length, length + canvas); rows below length are not written; capacity
 * below length + canvas: DG_ERR_KV_CAPACITY), final norm, fused LM head
 * (logits never stored), per-position entropy / sample / argmax, entropy-
 * bounded acceptance, re-noise, stop test.  Writes the canvas outputs.
 * batch * canvas <= 16384 (else DG_ERR_UNSUPPORTED). */
int dg_denoise_step(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache,
                    dg_canvas* canvas, const dg_step_params* p, void* d_ws, size_t ws_bytes,
                    void* stream);

/* Commit (report Figure 4, stage 3; LLM-Wiki key points, block-autoregressive
 * commit): committed = the last step's argmax; encode & append it; then
 * re-noise canvas->tokens for block p->block + 1.  The next step of the new
 * block must use t = 0 (no self-conditioning). */
int dg_commit_block(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache,
                    dg_canvas* canvas, const dg_step_params* p, void* d_ws, size_t ws_bytes,
                    void* stream);

/* dg_commit_block followed by the first denoising step (t = 0) of the next
 * block, in one pass through the layer stack (report Figure 4: stage 3 of
 * one block and stage 2 of the next).  The committed block (the last step's
 * argmax) is encoded causally and appended at rows [L, L + canvas); the
 * canvas is re-noised for p_next->block and denoised over [cache ; committed
 * block ; canvas] (its K/V in the scratch rows [L + canvas, L + 2 canvas)).
 * The weights stream once for both.  Results equal those of the two calls
 * up to floating-point summation order.  Requires p_next->t == 0,
 * p_next->block == p_commit->block + 1 and committed != NULL (else
 * DG_ERR_INVALID_ARG), no sc_probs, 2 * batch * canvas within the
 * workspace's pass size (dg_workspace_bytes(cfg, batch, canvas) holds
 * max(4096, batch * canvas) rows) and 16384 (else DG_ERR_UNSUPPORTED), and
 * capacity >= length + 2 canvas (else DG_ERR_KV_CAPACITY).
 * cache->length += canvas. */
int dg_commit_and_step(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache,
                       dg_canvas* canvas, const dg_step_params* p_commit,
                       const dg_step_params* p_next, void* d_ws, size_t ws_bytes, void* stream);

/* One autoregressive decode step on the same weights (DiffusionGemma
 * Technical Report digest, Figure 11: the single-token AR step the diffusion
 * step's latency is set against).  d_tokens [batch] (device int32, each in
 * [0, vocab)) is the latest token of each sequence; it is encoded causally at
 * position cache->length through every layer, its K/V rows appended, and the
 * LM head runs on those batch rows.  d_next [batch] (device int32) receives
 * the greedy next token, argmax of the logits, ties to the lower id.
 * cache->length += 1 on success.  Workspace: dg_workspace_bytes(cfg, batch, 1).
 * Errors: DG_ERR_INVALID_ARG for null tokens / outputs or batch < 1,
 * DG_ERR_KV_CAPACITY if the cache is full (nothing written),
 * DG_ERR_WORKSPACE if the workspace is short, DG_ERR_UNSUPPORTED above the
 * routing limit (batch * top_k <= 32768). */
int dg_ar_step(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache,
               const int32_t* d_tokens, int32_t batch, int32_t* d_next, void* d_ws,
               size_t ws_bytes, void* stream);

/* dg_denoise_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same inputs, outputs, launches and
 * results as dg_denoise_step with a caller workspace; calls no hipMalloc,
 * hipFree or allocating library routine.  Its scratch is a static device
 * array of DG_NOALLOC_SCRATCH_BYTES (320 MiB) in the library, one per GPU the
 * library runs on, held until the process ends; the call uses the current
 * device's (the stream's device must be the current device).  It holds one
 * step of batch * canvas <= 256 tokens at the pages' full width (d_model
 * 2816, 16/8 heads of 256, 128 experts top-8 + shared, vocab 262144); a step
 * needing more returns DG_ERR_SCRATCH_LIMIT before anything is enqueued.
 * Nothing in the scratch needs to start at zero; every call on one GPU
 * shares its array and leaves its contents, so calls whose work overlaps on
 * one GPU (other streams or threads, before the previous call's work has
 * finished) race: serialise them on one stream.  Other errors as
 * dg_denoise_step. */
#define DG_NOALLOC_SCRATCH_BYTES (320u << 20)
int dg_denoise_step_noalloc(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache,
                            dg_canvas* canvas, const dg_step_params* p, void* stream);

const char* dg_status_string(int status);

/* ---- measurement ---- */

/* Phases of a step whose GPU time can be traced. */
enum {
  DG_PHASE_SELFCOND = 0, /* expected embedding + self-conditioning MLP */
  DG_PHASE_EMBED = 1,    /* token gather + first RMSNorm */
  DG_PHASE_QKV = 2,      /* per layer: QKV projection + RoPE (+ K/V append when encoding) */
  DG_PHASE_ATTN = 3,     /* per layer: canvas attention (+ split merge) */
  DG_PHASE_OPROJ = 4,    /* per layer: O projection + residual + RMSNorm */
  DG_PHASE_ROUTE = 5,    /* per layer: router logits, top-k, segment sort */
  DG_PHASE_MOE_UP = 6,   /* per layer: routed + shared expert gate/up GEMM with GeGLU */
  DG_PHASE_MOE_DOWN = 7, /* per layer: routed + shared expert down GEMM */
  DG_PHASE_COMBINE = 8,  /* per layer: weighted combine + residual + RMSNorm */
  DG_PHASE_LMHEAD = 9,   /* fused LM head with sampler statistics */
  DG_PHASE_SAMPLER = 10, /* row merge, selection, re-noise, stop */
  DG_PHASE_COUNT = 11
};

/* Event trace: for every phase whose bit (1u << phase) is set in `mask`, the
 * call records events[count] before the phase and events[count + 1] after it
 * on the call's stream and stores the phase id in phase[count / 2]; count
 * grows by 2 per traced phase instance until `capacity` events are used
 * (later instances are not traced).  events are hipEvent_t created by the
 * caller; phase is a host array of capacity / 2 ints. */
typedef struct dg_trace {
  void** events;
  int32_t* phase;
  int32_t capacity;
  int32_t count;
  uint32_t mask;
} dg_trace;

/* dg_denoise_step / dg_encode_append with an optional event trace (NULL: none). */
int dg_denoise_step_traced(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache,
                           dg_canvas* canvas, const dg_step_params* p, void* d_ws, size_t ws_bytes,
                           void* stream, dg_trace* trace);
int dg_encode_append_traced(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache,
                            const int32_t* d_tokens, int32_t batch, int32_t n_tokens, void* d_ws,
                            size_t ws_bytes, void* stream, dg_trace* trace);

/* ---- test entry points (same device code as the calls above) ---- */

/* Sampler from given logits d_logits [B*C][vocab] fp32 (the LM head's
 * statistics computed from them), then acceptance, re-noise and stop exactly
 * as in dg_denoise_step. */
int dg_test_sample_from_logits(const dg_model_config* cfg, const float* d_logits, dg_canvas* canvas,
                               const dg_step_params* p, void* d_ws, size_t ws_bytes, void* stream);

/* Routing from given router logits d_logits [T][n_experts] fp32: d_ids/d_w
 * [T][top_k], d_row_token [T*top_k + (d_shared/d_expert)*T], d_inv [T*top_k],
 * d_offsets [n_experts + 1].  T <= 16384 (above 1024 the sort runs in
 * 1024-token chunks); workspace dg_workspace_bytes(cfg, 1, T). */
int dg_test_route_from_logits(const dg_model_config* cfg, const float* d_logits, int32_t T,
                              int32_t* d_ids, float* d_w, int32_t* d_row_token, int32_t* d_inv,
                              int32_t* d_offsets, void* d_ws, size_t ws_bytes, void* stream);

/* Denoiser forward only: writes fp32 logits d_logits [B*C][vocab] of the
 * canvas (with self-conditioning as in dg_denoise_step) and nothing else of
 * the canvas.  d_force_ids (optional, [n_layers][B*C][top_k], rank order)
 * replaces the top-k choice of every layer by the given experts (the gate
 * weights are still the softmax of this run's router logits over them), so
 * that continuous outputs can be compared when a near-tie would flip a route.
 * d_router_logits (optional, [n_layers][B*C][n_experts] fp32) receives every
 * layer's router logits. */
int dg_test_forward_logits(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache,
                           dg_canvas* canvas, const dg_step_params* p, const int32_t* d_force_ids,
                           float* d_router_logits, float* d_logits, void* d_ws, size_t ws_bytes,
                           void* stream);

/* The whole denoising step of dg_denoise_step (every canvas output written:
 * entropy, sample, argmax, accepted set, next tokens, mean entropy, stop,
 * flags, and the carried self-conditioning input p_side / p_scale), with
 * optional test hooks (device pointers, NULL for none):
 *   d_force_ids / d_router_logits: every layer's routing forced / observed as
 *     in dg_test_forward_logits;
 *   d_logits [B*C][vocab] fp32: the logits captured as well;
 *   d_teacher_x [n_layers + 1][B*C][d_model] fp32: teacher forcing, layer l
 *     starts from the residual d_teacher_x[l] (its RMSNorm recomputed)
 *     instead of the previous layer's output, and the LM head reads
 *     d_teacher_x[n_layers]; the canvas K/V of layer l come from that input;
 *   d_layer_out [n_layers + 1][B*C][d_model] fp32: row 0 receives the
 *     embedding output (token embedding plus the self-conditioning term, from
 *     the canvas tokens and the carried or external input), row l + 1 layer
 *     l's output residual.
 * Lets a comparison run the product's carried self-conditioning path and
 * every layer on the oracle's routes and inputs.  Same workspace and errors
 * as dg_denoise_step. */
int dg_test_denoise_step(const dg_model_config* cfg, const dg_weights* w, const dg_kv_cache* cache,
                         dg_canvas* canvas, const dg_step_params* p, const int32_t* d_force_ids,
                         float* d_router_logits, float* d_logits, const float* d_teacher_x, float* d_layer_out,
                         void* d_ws, size_t ws_bytes, void* stream);

/* Causal encode-and-append as in dg_encode_append, with the routing of every
 * layer optionally forced and observed as in dg_test_forward_logits:
 * d_force_ids [n_layers][batch*n_tokens][top_k] (rank order), d_router_logits
 * [n_layers][batch*n_tokens][n_experts] fp32, rows in [batch][position]
 * order.  The whole encode must fit in one internal chunk (batch*n_tokens
 * <= 4096 and batch*n_tokens*top_k <= 32768), else DG_ERR_UNSUPPORTED. */
int dg_test_encode_append(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache,
                          const int32_t* d_tokens, int32_t batch, int32_t n_tokens, const int32_t* d_force_ids,
                          float* d_router_logits, void* d_ws, size_t ws_bytes, void* stream);

/* dg_ar_step that also stores the fp32 logits of the decoded rows in
 * d_logits [batch][vocab] (device, caller-owned, required: null is
 * DG_ERR_INVALID_ARG).  Same workspace, errors and cache update. */
int dg_test_ar_step(const dg_model_config* cfg, const dg_weights* w, dg_kv_cache* cache,
                    const int32_t* d_tokens, int32_t batch, int32_t* d_next, float* d_logits,
                    void* d_ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H_ */
