/*
 * Seeded synthetic inputs for the block-diffusion decoder: weights, tokens,
 * KV-cache fills and Dirichlet rows.  This file holds no step of the decoding
 * method; it only manufactures inputs.  Both the CPU oracle and the GPU path
 * receive exactly the values produced here (or by the device twin in
 * gen_dev.hip, which implements the same definition and is checked against
 * this file bit for bit).
 *
 * Definition (all integer, so host and device agree exactly):
 *   h(seed, tensor, i) = SplitMix64 finaliser applied to
 *       seed + G*(i+1) + H*(tensor+1)      (mod 2^64)
 *     with G = 0x9E3779B97F4A7C15, H = 0xD1B54A32D192ED03 and the finaliser
 *     of Steele, Lea & Flood, "Fast splittable pseudorandom number
 *     generators" (OOPSLA 2014), with the mixing constants of Vigna's
 *     splitmix64.
 *   normal value   = fp32( (sum of the four 16-bit fields of h) - 131070 )
 *                    * scale,   scale = fp32(std / sqrt((65536^2-1)/3))
 *                    (Irwin-Hall sum of 4 uniforms: mean 0, variance std^2,
 *                    support +-3.46 std), then bf16 by round-to-nearest-even
 *                    when a bf16 tensor is asked for.
 *   token          = (hi32(h) * V) >> 32   (exactly uniform when V is 2^b).
 *   uniform in (0,1) = ((h >> 11) + 0.5) * 2^-53.
 *   fp8 weights    = the bf16 normal tensor quantised per output row r:
 *                    s_r = fp32(max_c |w[r][c]| / 448)  (1 if the row is all zero),
 *                    code[r][c] = E4M3 code of fp32(w[r][c] / s_r), rounded to
 *                    nearest even, |x| >= 464 saturating to 448 (OCP FP8 E4M3:
 *                    exponent bias 7, 3 mantissa bits, no infinities).
 *   MXFP4 weights  = the bf16 normal tensor quantised in blocks of 32
 *                    consecutive values of a row (OCP Microscaling Formats
 *                    v1.0): shared exponent E = floor(log2(max |w|)) - 2 (2 is
 *                    the largest E2M1 exponent), clamped to [-127, 127], stored
 *                    as the E8M0 code E + 127; element codes E2M1(w / 2^E)
 *                    (sign, 2 exponent bits with bias 1, 1 mantissa bit:
 *                    0, 0.5, 1, 1.5, 2, 3, 4, 6), rounded to nearest even on
 *                    that grid, |x| > 6 saturating to 6.  An all-zero block
 *                    gets the code 0 and zero elements.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t synth_hash(uint64_t seed, uint64_t tensor, uint64_t i) {
  uint64_t z = seed + 0x9E3779B97F4A7C15ull * (i + 1) + 0xD1B54A32D192ED03ull * (tensor + 1);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline float synth_normal_value(uint64_t z, float scale) {
  int32_t s = (int32_t)(z & 0xFFFF) + (int32_t)((z >> 16) & 0xFFFF) +
              (int32_t)((z >> 32) & 0xFFFF) + (int32_t)(z >> 48) - 131070;
  return (float)s * scale;
}

static inline uint16_t synth_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float synth_scale_for_std(double std) {
  return (float)(std / sqrt((65536.0 * 65536.0 - 1.0) / 3.0));
}

void synth_normal_f32(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, float scale,
                      float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)count; ++j)
    out[j] = synth_normal_value(synth_hash(seed, tensor, start + (uint64_t)j), scale);
}

void synth_normal_bf16(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, float scale,
                       uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)count; ++j)
    out[j] = synth_bf16_rne(synth_normal_value(synth_hash(seed, tensor, start + (uint64_t)j), scale));
}

/* The bf16 values of synth_normal_bf16, widened exactly to double (what an
 * fp64 consumer of bf16 tensors reads). */
void synth_normal_bf16_as_f64(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, float scale,
                              double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)count; ++j) {
    const uint32_t u = (uint32_t)synth_bf16_rne(synth_normal_value(synth_hash(seed, tensor, start + (uint64_t)j), scale)) << 16;
    float f;
    memcpy(&f, &u, 4);
    out[j] = (double)f;
  }
}

/* OCP E4M3 code of x, round to nearest even. */
static inline uint8_t synth_e4m3_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E80000u) return sign | 0x7Eu; /* |x| >= 464 */
  if (a < 0x3C800000u) {                     /* |x| < 2^-6: subnormal grid, step 2^-9 */
    float f;
    memcpy(&f, &a, 4);
    return sign | (uint8_t)nearbyintf(f * 512.0f); /* 8 -> code 0x08, the smallest normal */
  }
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u); /* keep 3 mantissa bits, ties to even */
  return sign | (uint8_t)((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

/* Row-wise fp8 quantisation of the bf16 normal tensor [rows][cols] (element
 * r*cols + c of the tensor's stream). */
void synth_e4m3_rows(uint64_t seed, uint64_t tensor, int64_t rows, int64_t cols, float scale, uint8_t* codes,
                     float* row_scale) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float mx = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
      const uint32_t u = (uint32_t)synth_bf16_rne(synth_normal_value(synth_hash(seed, tensor, (uint64_t)(r * cols + c)), scale)) << 16;
      float w;
      memcpy(&w, &u, 4);
      w = fabsf(w);
      if (w > mx) mx = w;
    }
    const float s = mx > 0.0f ? mx / 448.0f : 1.0f;
    row_scale[r] = s;
    for (int64_t c = 0; c < cols; ++c) {
      const uint32_t u = (uint32_t)synth_bf16_rne(synth_normal_value(synth_hash(seed, tensor, (uint64_t)(r * cols + c)), scale)) << 16;
      float w;
      memcpy(&w, &u, 4);
      codes[r * cols + c] = synth_e4m3_rne(w / s);
    }
  }
}

/* E2M1 code of x (finite), round to nearest even on the grid
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6}: the thresholds are the grid's midpoints, a
 * midpoint going to the neighbour whose code is even; |x| > 6 gives 6. */
static inline uint8_t synth_e2m1_rne(float x) {
  const uint8_t sign = signbit(x) ? 8u : 0u;
  const float a = fabsf(x);
  uint8_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return sign | c;
}

/* MXFP4 form of one block of 32 fp32 values: codes[32] (one E2M1 code per
 * byte) and the E8M0 scale code. */
static void synth_mxfp4_block(const float* w, uint8_t* codes, uint8_t* scale) {
  float mx = 0.0f;
  for (int i = 0; i < 32; ++i)
    if (fabsf(w[i]) > mx) mx = fabsf(w[i]);
  if (mx == 0.0f) {
    *scale = 0;
    for (int i = 0; i < 32; ++i) codes[i] = 0;
    return;
  }
  int e2;
  frexpf(mx, &e2); /* mx = f 2^e2, f in [0.5, 1): floor(log2 mx) = e2 - 1 */
  int E = e2 - 1 - 2;
  if (E < -127) E = -127;
  if (E > 127) E = 127;
  *scale = (uint8_t)(E + 127);
  for (int i = 0; i < 32; ++i) codes[i] = synth_e2m1_rne(ldexpf(w[i], -E));
}

/* MXFP4 form of w[rows][cols] (cols % 32 == 0): codes [rows][cols], scales
 * [rows][cols / 32]. */
void synth_mxfp4_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < cols / 32; ++b)
      synth_mxfp4_block(w + r * cols + b * 32, codes + r * cols + b * 32, scales + r * (cols / 32) + b);
}

/* MXFP4 form of the bf16 normal tensor [rows][cols] (element r*cols + c of
 * the tensor's stream). */
void synth_mxfp4_rows(uint64_t seed, uint64_t tensor, int64_t rows, int64_t cols, float scale, uint8_t* codes,
                      uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float w[32];
    for (int64_t b = 0; b < cols / 32; ++b) {
      for (int i = 0; i < 32; ++i) {
        const uint32_t u =
            (uint32_t)synth_bf16_rne(synth_normal_value(synth_hash(seed, tensor, (uint64_t)(r * cols + b * 32 + i)), scale))
            << 16;
        memcpy(&w[i], &u, 4);
      }
      synth_mxfp4_block(w, codes + r * cols + b * 32, scales + r * (cols / 32) + b);
    }
  }
}

void synth_tokens(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, uint32_t vocab,
                  int32_t* out) {
  for (uint64_t j = 0; j < count; ++j) {
    uint64_t hi = synth_hash(seed, tensor, start + j) >> 32;
    out[j] = (int32_t)((hi * (uint64_t)vocab) >> 32);
  }
}

static inline double synth_uniform(uint64_t seed, uint64_t tensor, uint64_t i) {
  return ((double)(synth_hash(seed, tensor, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Standard normal by Box-Muller from two uniforms (host only; used for the
 * Gamma draws of the Dirichlet rows, never for weights). */
static inline double synth_std_normal(uint64_t seed, uint64_t tensor, uint64_t i) {
  double u1 = synth_uniform(seed, tensor, 2 * i), u2 = synth_uniform(seed, tensor, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* Gamma(alpha, 1) for alpha < 1 by Marsaglia & Tsang (ACM TOMS 2000) on
 * alpha+1 with the U^(1/alpha) boost.  Each draw j uses its own sub-stream
 * (tensor, j) so rows can be generated in parallel. */
static double synth_gamma(uint64_t seed, uint64_t tensor, uint64_t j, double alpha) {
  double a = alpha < 1.0 ? alpha + 1.0 : alpha;
  double d = a - 1.0 / 3.0, c = 1.0 / sqrt(9.0 * d);
  uint64_t sub = 0x5D588B656C078965ull * (j + 1) ^ tensor;
  for (uint64_t it = 0;; ++it) {
    double x = synth_std_normal(seed, sub, 3 * it), v = 1.0 + c * x;
    if (v <= 0.0) continue;
    v = v * v * v;
    double u = synth_uniform(seed, sub, 3 * it + 2);
    if (log(u) < 0.5 * x * x + d - d * v + d * log(v)) {
      double g = d * v;
      if (alpha < 1.0) g *= pow(synth_uniform(seed, sub ^ 0xA5A5A5A5ull, it + 7), 1.0 / alpha);
      return g;
    }
  }
}

/* rows x V Dirichlet(alpha) rows, normalised in fp64, rounded once to fp32. */
void synth_dirichlet_rows(uint64_t seed, uint64_t tensor, int64_t rows, int64_t V, double alpha,
                          float* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    double* g = (double*)malloc((size_t)V * sizeof(double));
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) {
      g[v] = synth_gamma(seed, tensor, (uint64_t)(r * V + v), alpha);
      s += g[v];
    }
    for (int64_t v = 0; v < V; ++v) out[r * V + v] = (float)(g[v] / s);
    free(g);
  }
}
