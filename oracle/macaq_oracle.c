/*
 * CPU oracle for the MACaQ online W4A4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no source with the HIP library.
 *
 * What it computes (sources):
 *   - "MACaQ: Fast, Model Agnostic Calibrated Quantization for Low-Precision
 *     Weights and Activations" (paper card, Abstract): every linear layer is
 *     treated on its own; a per-channel scale and a block-Hadamard transform
 *     are applied online to the layer's activations, the inverse transforms
 *     are absorbed into that layer's weights, and both sides are MXFP4 (W4A4),
 *     with round-to-nearest as the weight rounding that Flip-Refinement later
 *     improves on.
 *   - "MACaQ - Huawei open-sources a 4-bit quantizer ..." (How it works): the
 *     same per-channel scale plus block-Hadamard rotation, the inverse folded
 *     into the weights, nothing crossing a layer boundary.
 *   - MX format (OCP Microscaling Formats v1.0): 32 E2M1 elements share one
 *     E8M0 power-of-two scale; E2M1 magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6.
 *
 * Readings where the pages are silent (each one is a choice, not page text):
 *   - D divides the activations by s_k = sqrt(max_r |x_rk|) over calibration
 *     rows, and multiplies the weight columns by s_k.
 *   - H is the orthonormal Sylvester block-Hadamard S_b / sqrt(b) on
 *     contiguous, aligned b-blocks along K. The 1/sqrt(b) is folded into the
 *     per-channel multipliers on both sides: a_k = c_b / s_k, r_k = c_b * s_k
 *     with c_b = RN32(1/sqrt(b)).
 *   - The transform runs in fp32: one multiply, then butterfly stages of
 *     span h = 1, 2, 4, ..., b/2 in that order, each (u, v) -> (u + v, u - v).
 *     The quantized codes are decided in this precision on both sides.
 *   - MX scale: floor(log2(amax)) - 2 (2 is the largest E2M1 exponent),
 *     clamped to E8M0's lowest value 2^-127; an all-zero block gets 2^-127.
 *   - E2M1 rounding: to nearest, ties to the even code, saturating at 6; the
 *     sign of the input is kept, so a negative value that rounds to 0 gives
 *     code 8.
 *   - Packing: element 2i in the low nibble of byte i, 2i+1 in the high
 *     nibble; scales are one byte per 32 elements, row-major.
 *   - The GEMM over codes accumulates in fp64 (a sum of dyadic products,
 *     exact at the sizes used).
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

/* ------------------------------------------------------------------ */
/* Element access                                                      */
/* ------------------------------------------------------------------ */

/* A bf16 value is the upper half of an fp32; widening is exact. */
static float bf16_to_float(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* dtype 0: bf16 (uint16 bits); dtype 1: fp32 */
static float load_elem(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) return bf16_to_float(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

static int valid_block(int b) { return b == 0 || b == 32 || b == 64 || b == 128; }

/* ------------------------------------------------------------------ */
/* Per-channel scale (calibration) and the folded multipliers          */
/* ------------------------------------------------------------------ */

/* s_k = sqrt(max over calibration rows of |x_rk|), rounded once to fp32;
   a channel that is zero on every calibration row gets s_k = 1. */
int oracle_calibrate(const void* xcal, int dtype, int64_t R, int64_t K, int64_t ld, float* s) {
  if (!xcal || !s || R < 1 || K < 1 || ld < K) return ORACLE_EINVAL;
  for (int64_t k = 0; k < K; ++k) {
    float mx = 0.0f;
    for (int64_t r = 0; r < R; ++r) {
      float v = fabsf(load_elem(xcal, dtype, r * ld + k));
      if (v > mx) mx = v;
    }
    s[k] = (mx == 0.0f) ? 1.0f : sqrtf(mx);
  }
  return ORACLE_OK;
}

/* Calibration variants (the pages leave the form of the calibrated scale
   open): s_k = max_r |x_rk| raised to quarters/4, for quarters 0 (no scale,
   s = 1), 1 (two correctly rounded square roots in turn), 2 (one, as
   oracle_calibrate) or 4 (the maximum itself); 1 for an all-zero channel. */
int oracle_calibrate_pow(const void* xcal, int dtype, int64_t R, int64_t K, int64_t ld, int quarters, float* s) {
  if (quarters != 0 && quarters != 1 && quarters != 2 && quarters != 4) return ORACLE_EINVAL;
  if (!xcal || !s || R < 1 || K < 1 || ld < K) return ORACLE_EINVAL;
  for (int64_t k = 0; k < K; ++k) {
    float mx = 0.0f;
    for (int64_t r = 0; r < R; ++r) {
      float v = fabsf(load_elem(xcal, dtype, r * ld + k));
      if (v > mx) mx = v;
    }
    float v = 1.0f;
    if (mx != 0.0f) {
      if (quarters == 1) v = sqrtf(sqrtf(mx));
      else if (quarters == 2) v = sqrtf(mx);
      else if (quarters == 4) v = mx;
    }
    s[k] = v;
  }
  return ORACLE_OK;
}

/* c_b = RN32(1/sqrt(b)) (1 when b == 0); a_k = RN32(c_b / s_k),
   r_k = RN32(c_b * s_k). Either output may be NULL. */
int oracle_multipliers(const float* s, int64_t K, int b, float* a, float* r) {
  if (!s || K < 1 || !valid_block(b)) return ORACLE_EINVAL;
  float cb = 1.0f;
  if (b > 0) cb = sqrtf(1.0f / (float)b); /* 1/b is exact; sqrtf rounds once */
  for (int64_t k = 0; k < K; ++k) {
    if (a) a[k] = cb / s[k];
    if (r) r[k] = cb * s[k];
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Transform of one row: per-channel multiply, then block-Hadamard      */
/* ------------------------------------------------------------------ */

/* t = S_b (m .* v) on each aligned b-block, in fp32, stages of span
   h = 1, 2, ..., b/2. m == NULL means no multiply; b == 0 means no
   Hadamard. */
static void transform_row(const void* x, int dtype, int64_t row_off, const float* m, int64_t K, int b,
                          float* t) {
  for (int64_t k = 0; k < K; ++k) {
    float v = load_elem(x, dtype, row_off + k);
    t[k] = m ? v * m[k] : v;
  }
  if (b == 0) return;
  for (int64_t base = 0; base < K; base += b) {
    float* blk = t + base;
    for (int h = 1; h < b; h *= 2) {
      for (int i = 0; i < b; ++i) {
        if (i & h) continue;
        float u = blk[i];
        float w = blk[i + h];
        blk[i] = u + w;
        blk[i + h] = u - w;
      }
    }
  }
}

int oracle_transform_rows(const void* x, int dtype, int64_t M, int64_t K, int64_t ld, const float* m, int b,
                          float* t) {
  if (!x || !t || M < 1 || K < 1 || ld < K || !valid_block(b)) return ORACLE_EINVAL;
  if (b > 0 && K % b != 0) return ORACLE_EINVAL;
  for (int64_t r = 0; r < M; ++r) transform_row(x, dtype, r * ld, m, K, b, t + r * K);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* MXFP4 encoding                                                       */
/* ------------------------------------------------------------------ */

/* E2M1 magnitude of each 3-bit code */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Round a non-negative magnitude (already divided by the block scale) to the
   nearest E2M1 magnitude. Between two neighbours the decision is a compare
   with their midpoint, which is exact; a value on the midpoint goes to the
   neighbour with the even code (even mantissa bit). Above 6 saturates. */
static unsigned e2m1_round_magnitude(double u) {
  if (u >= kE2M1[7]) return 7;
  if (!(u >= 0.0)) return 0; /* NaN: inputs must be finite; any code, no crash */
  unsigned c = 0;
  while (c < 6 && !(u < kE2M1[c + 1])) ++c; /* kE2M1[c] <= u < kE2M1[c+1] */
  double mid = 0.5 * (kE2M1[c] + kE2M1[c + 1]);
  if (u < mid) return c;
  if (u > mid) return c + 1;
  return (c % 2 == 0) ? c : c + 1;
}

/* Quantize one 32-element group to (32 codes, 1 E8M0 scale code). */
static void mx_quantize_group(const float* t, uint8_t* code, uint8_t* scale_code) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float v = fabsf(t[i]);
    if (v > amax) amax = v;
  }
  int shared_exp = -127; /* 2^-127 for an all-zero group */
  if (amax > 0.0f) {
    int e;
    frexpf(amax, &e);        /* amax = f * 2^e, f in [0.5, 1) */
    int floor_log2 = e - 1;  /* so 2^floor_log2 <= amax < 2^(floor_log2+1) */
    shared_exp = floor_log2 - 2;
    if (shared_exp < -127) shared_exp = -127;
  }
  *scale_code = (uint8_t)(shared_exp + 127);
  for (int i = 0; i < 32; ++i) {
    /* |t| / 2^shared_exp is exact in double */
    double u = ldexp((double)fabsf(t[i]), -shared_exp);
    unsigned mag = e2m1_round_magnitude(u);
    unsigned sign = signbit(t[i]) ? 1u : 0u;
    code[i] = (uint8_t)((sign << 3) | mag);
  }
}

/* Quantize M rows of x (after the transform with multiplier m and block b) into
   packed codes [M, K/2] and scales [M, K/32]. */
int oracle_quant_rows(const void* x, int dtype, int64_t M, int64_t K, int64_t ld, const float* m, int b,
                      uint8_t* codes, uint8_t* scales) {
  if (!x || !codes || !scales || M < 1 || K < 32 || K % 32 != 0 || ld < K || !valid_block(b))
    return ORACLE_EINVAL;
  if (b > 0 && K % b != 0) return ORACLE_EINVAL;
  float* t = (float*)malloc((size_t)K * sizeof(float));
  uint8_t* c = (uint8_t*)malloc((size_t)K);
  if (!t || !c) {
    free(t);
    free(c);
    return ORACLE_EINVAL;
  }
  for (int64_t r = 0; r < M; ++r) {
    transform_row(x, dtype, r * ld, m, K, b, t);
    for (int64_t g = 0; g < K / 32; ++g) mx_quantize_group(t + 32 * g, c + 32 * g, scales + r * (K / 32) + g);
    for (int64_t i = 0; i < K / 2; ++i)
      codes[r * (K / 2) + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
  }
  free(t);
  free(c);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Dequantization and the GEMM over codes (fp64)                        */
/* ------------------------------------------------------------------ */

static double dequant_elem(const uint8_t* codes, const uint8_t* scales, int64_t K, int64_t row, int64_t k) {
  uint8_t byte = codes[row * (K / 2) + k / 2];
  unsigned c = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
  double mag = kE2M1[c & 7];
  double v = (c & 8) ? -mag : mag;
  int sc = scales[row * (K / 32) + k / 32];
  return ldexp(v, sc - 127);
}

int oracle_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t M, int64_t K, double* out) {
  if (!codes || !scales || !out || M < 1 || K < 32 || K % 32 != 0) return ORACLE_EINVAL;
  for (int64_t r = 0; r < M; ++r)
    for (int64_t k = 0; k < K; ++k) out[r * K + k] = dequant_elem(codes, scales, K, r, k);
  return ORACLE_OK;
}

typedef struct {
  const double* a; /* dequantized A [M, K] */
  const double* w; /* dequantized W' [N, K] */
  double* y;       /* [M, N] */
  int64_t m0, m1, N, K;
} gemm_job;

static void* gemm_worker(void* p) {
  gemm_job* j = (gemm_job*)p;
  for (int64_t m = j->m0; m < j->m1; ++m) {
    const double* ar = j->a + m * j->K;
    for (int64_t n = 0; n < j->N; ++n) {
      const double* wr = j->w + n * j->K;
      double acc = 0.0;
      for (int64_t k = 0; k < j->K; ++k) acc += ar[k] * wr[k];
      j->y[m * j->N + n] = acc;
    }
  }
  return NULL;
}

/* y[m, n] = sum_k dq(A[m, k]) * dq(W'[n, k]) in fp64, rows split over
   `threads` workers (each output is computed the same way by one worker). */
int oracle_gemm_codes(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, const uint8_t* w_codes,
                      const uint8_t* w_scales, int64_t N, int64_t K, double* y, int threads) {
  if (!a_codes || !a_scales || !w_codes || !w_scales || !y || M < 1 || N < 1 || K < 32 || K % 32 != 0)
    return ORACLE_EINVAL;
  if (threads < 1) threads = 1;
  if (threads > M) threads = (int)M;
  double* a = (double*)malloc((size_t)M * K * sizeof(double));
  double* w = (double*)malloc((size_t)N * K * sizeof(double));
  gemm_job* jobs = (gemm_job*)malloc((size_t)threads * sizeof(gemm_job));
  pthread_t* tid = (pthread_t*)malloc((size_t)threads * sizeof(pthread_t));
  if (!a || !w || !jobs || !tid) {
    free(a);
    free(w);
    free(jobs);
    free(tid);
    return ORACLE_EINVAL;
  }
  oracle_dequant_rows(a_codes, a_scales, M, K, a);
  oracle_dequant_rows(w_codes, w_scales, N, K, w);
  for (int i = 0; i < threads; ++i) {
    jobs[i].a = a;
    jobs[i].w = w;
    jobs[i].y = y;
    jobs[i].N = N;
    jobs[i].K = K;
    jobs[i].m0 = M * i / threads;
    jobs[i].m1 = M * (i + 1) / threads;
  }
  int started = 0;
  for (int i = 1; i < threads; ++i)
    if (pthread_create(&tid[i], NULL, gemm_worker, &jobs[i]) == 0) started = i;
    else break;
  gemm_worker(&jobs[0]);
  for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
  for (int i = started + 1; i < threads; ++i) gemm_worker(&jobs[i]); /* any that failed to start */
  free(a);
  free(w);
  free(jobs);
  free(tid);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* The layer: activations through the transform and MXFP4, then the GEMM */
/* ------------------------------------------------------------------ */

/* y = W' . Q(H D x) for M bf16 rows of x; weights already prepared. */
int oracle_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* a, int b,
                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, double* y, int threads) {
  if (!x || !w_codes || !w_scales || !y || M < 1 || N < 1) return ORACLE_EINVAL;
  uint8_t* ac = (uint8_t*)malloc((size_t)M * K / 2);
  uint8_t* as = (uint8_t*)malloc((size_t)M * K / 32);
  if (!ac || !as) {
    free(ac);
    free(as);
    return ORACLE_EINVAL;
  }
  int rc = oracle_quant_rows(x, 0, M, K, ldx, a, b, ac, as);
  if (rc == ORACLE_OK) rc = oracle_gemm_codes(ac, as, M, w_codes, w_scales, N, K, y, threads);
  free(ac);
  free(as);
  return rc;
}

/* Per expert e: rows [off[e], off[e+1]) of x (expert-major order) go
   through expert e's multiplier a[e, :] and weights W'_e [N, K]. Experts
   with no rows are skipped. */
int oracle_linear_grouped(const uint16_t* x, const int32_t* off, int E, int64_t T, int64_t K, const float* a,
                          int b, const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, double* y,
                          int threads) {
  if (!x || !off || !w_codes || !w_scales || !y || E < 1 || T < 0 || N < 1 || K < 32 || K % 32 != 0)
    return ORACLE_EINVAL;
  if (off[0] != 0 || off[E] != T) return ORACLE_EINVAL;
  for (int e = 0; e < E; ++e) {
    if (off[e + 1] < off[e]) return ORACLE_EINVAL;
  }
  for (int e = 0; e < E; ++e) {
    int64_t rows = off[e + 1] - off[e];
    if (rows == 0) continue;
    int rc = oracle_linear(x + (int64_t)off[e] * K, rows, K, K, a ? a + (int64_t)e * K : NULL, b,
                           w_codes + (int64_t)e * N * (K / 2), w_scales + (int64_t)e * N * (K / 32), N,
                           y + (int64_t)off[e] * N, threads);
    if (rc != ORACLE_OK) return rc;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* MoE block around the grouped layer                                   */
/* ------------------------------------------------------------------ */
/*
 * Sources: "MACaQ ..." (paper card, Abstract) treats every linear layer on
 * its own; "MACaQ - Huawei open-sources a 4-bit quantizer ..." (What it is)
 * lists MoE models among those it covers; "Huawei's MACaQ-R beats Unsloth's
 * ..." (the "Changed tensors" item) names the routed experts' three
 * projections, gate, up and down. The pages do not spell out the expert
 * FFN; it is taken as the usual gated one, y = down(SiLU(gate x) * up x),
 * with the token's top-k expert outputs summed with its routing weights.
 * Readings (choices, not page text):
 *   - routing order: the rows of the grouped layers are the (token, slot)
 *     entries sorted by expert, ties by entry index i = t * k + j (stable);
 *     an id outside [0, E) takes no row;
 *   - gate and up projections of one expert are stacked as one weight
 *     matrix [2F, H] whose rows alternate in blocks of 32: rows 64c .. 64c+31
 *     are gate channels 32c .. 32c+31, rows 64c+32 .. 64c+63 up channels
 *     32c .. 32c+31;
 *   - h = SiLU(g) * u with SiLU(g) = g / (1 + exp(-g)), evaluated here in
 *     fp64 on the fp64 GEMM outputs and rounded once to fp32; h then goes
 *     through the down projection's own transform and MXFP4 exactly as an
 *     activation row does (its multiplier a_dn[e], block b);
 *   - each expert's down-projection output row is rounded to bf16 (it is a
 *     layer output), and the combine sums w[t, j] * row over j = 0 .. k-1
 *     in that order (fp64 here).
 */

/* Stable counting sort of the entries by expert. offsets [E+1]; row_token
   [T*k] gets the token of each row (rows past offsets[E] are left alone);
   pos [T*k] gets the row of each entry, or -1 for an id outside [0, E). */
int oracle_moe_route(const int32_t* ids, int64_t T, int k, int E, int32_t* offsets, int32_t* row_token,
                     int32_t* pos) {
  if (!ids || !offsets || !row_token || !pos || T < 0 || k < 1 || E < 1) return ORACLE_EINVAL;
  const int64_t n = T * k;
  int64_t row = 0;
  for (int64_t i = 0; i < n; ++i) pos[i] = -1;
  for (int e = 0; e < E; ++e) {
    offsets[e] = (int32_t)row;
    for (int64_t i = 0; i < n; ++i) {
      if (ids[i] != e) continue;
      row_token[row] = (int32_t)(i / k);
      pos[i] = (int32_t)row;
      ++row;
    }
  }
  offsets[E] = (int32_t)row;
  return ORACLE_OK;
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* h[r, c] = RN32(SiLU(g) * u) from gate/up outputs stacked as above:
   gu [R, 2F] (fp64), h [R, F] (fp32). F % 32 == 0. */
int oracle_silu_mul(const double* gu, int64_t R, int64_t F, float* h) {
  if (!gu || !h || R < 0 || F < 32 || F % 32 != 0) return ORACLE_EINVAL;
  for (int64_t r = 0; r < R; ++r)
    for (int64_t c = 0; c < F; ++c) {
      const int64_t gcol = 64 * (c / 32) + c % 32;
      const double g = gu[r * 2 * F + gcol], u = gu[r * 2 * F + gcol + 32];
      h[r * F + c] = (float)(silu(g) * u);
    }
  return ORACLE_OK;
}

/* bf16 rounding (to nearest, ties to even) of a finite fp64 value, through
   fp32 first as a device would round its fp32 result; returned as a float. */
static float round_bf16_of(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  const uint32_t lsb = (u >> 16) & 1u;
  u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* y[t, :] = sum_j w[t, j] * rows[pos[t*k + j], :] (j ascending, fp64),
   entries with pos < 0 skipped. rows [R, H] fp32 values. */
int oracle_moe_combine(const float* rows, int64_t H, const int32_t* pos, const float* w, int64_t T, int k,
                       double* y) {
  if (!rows || !pos || !w || !y || H < 1 || T < 0 || k < 1) return ORACLE_EINVAL;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) {
        const int32_t r = pos[t * k + j];
        if (r < 0) continue;
        acc += (double)w[t * k + j] * (double)rows[(int64_t)r * H + c];
      }
      y[t * H + c] = acc;
    }
  return ORACLE_OK;
}

/* The block for the tokens with want[t] != 0 (want == NULL: all tokens):
   route, gather each row's token, gate/up through expert e's a_gu[e] and
   stacked weights, SiLU * up, the down projection's transform and MXFP4
   with a_dn[e], the down GEMM, bf16 rows, combine. Rows of tokens not
   wanted are skipped (their y rows are left alone).
   Optional outputs (NULL to skip): dn_codes [T*k, F/2], dn_scales
   [T*k, F/32] (row-major, rows in routing order; rows of unwanted tokens
   left alone). x [T, H] bf16 bits; wgu [E, 2F, H/2] + [E, 2F, H/32];
   wdn [E, H, F/2] + [E, H, F/32]; y [T, H] fp64. */
int oracle_moe_block(const uint16_t* x, int64_t T, int64_t H, const int32_t* ids, const float* w, int k, int E,
                     const float* a_gu, const uint8_t* wgu_codes, const uint8_t* wgu_scales, const float* a_dn,
                     const uint8_t* wdn_codes, const uint8_t* wdn_scales, int64_t F, int b, const uint8_t* want,
                     uint8_t* dn_codes, uint8_t* dn_scales, double* y, int threads) {
  if (!x || !ids || !w || !wgu_codes || !wgu_scales || !wdn_codes || !wdn_scales || !y || T < 1 || k < 1 ||
      E < 1 || H < 32 || H % 32 != 0 || F < 32 || F % 32 != 0 || !valid_block(b))
    return ORACLE_EINVAL;
  if (b > 0 && (H % b != 0 || F % b != 0)) return ORACLE_EINVAL;
  const int64_t n = T * k;
  int32_t* off = (int32_t*)malloc((size_t)(E + 1) * sizeof(int32_t));
  int32_t* row_token = (int32_t*)malloc((size_t)n * sizeof(int32_t));
  int32_t* pos = (int32_t*)malloc((size_t)n * sizeof(int32_t));
  float* rows_out = (float*)calloc((size_t)n * H, sizeof(float));
  int rc = (off && row_token && pos && rows_out) ? ORACLE_OK : ORACLE_EINVAL;
  if (rc == ORACLE_OK) rc = oracle_moe_route(ids, T, k, E, off, row_token, pos);
  for (int e = 0; rc == ORACLE_OK && e < E; ++e) {
    /* this expert's wanted rows */
    int64_t cnt = 0;
    for (int64_t r = off[e]; r < off[e + 1]; ++r)
      if (!want || want[row_token[r]]) ++cnt;
    if (cnt == 0) continue;
    int64_t* idx = (int64_t*)malloc((size_t)cnt * sizeof(int64_t));
    uint16_t* xe = (uint16_t*)malloc((size_t)cnt * H * sizeof(uint16_t));
    double* gu = (double*)malloc((size_t)cnt * 2 * F * sizeof(double));
    float* h = (float*)malloc((size_t)cnt * F * sizeof(float));
    uint8_t* hc = (uint8_t*)malloc((size_t)cnt * F / 2);
    uint8_t* hs = (uint8_t*)malloc((size_t)cnt * F / 32);
    double* ye = (double*)malloc((size_t)cnt * H * sizeof(double));
    if (!idx || !xe || !gu || !h || !hc || !hs || !ye) rc = ORACLE_EINVAL;
    if (rc == ORACLE_OK) {
      int64_t j = 0;
      for (int64_t r = off[e]; r < off[e + 1]; ++r)
        if (!want || want[row_token[r]]) idx[j++] = r;
      for (int64_t i = 0; i < cnt; ++i) memcpy(xe + i * H, x + (int64_t)row_token[idx[i]] * H, (size_t)H * 2);
      rc = oracle_linear(xe, cnt, H, H, a_gu ? a_gu + (int64_t)e * H : NULL, b,
                         wgu_codes + (int64_t)e * 2 * F * (H / 2), wgu_scales + (int64_t)e * 2 * F * (H / 32),
                         2 * F, gu, threads);
    }
    if (rc == ORACLE_OK) rc = oracle_silu_mul(gu, cnt, F, h);
    if (rc == ORACLE_OK)
      rc = oracle_quant_rows(h, 1, cnt, F, F, a_dn ? a_dn + (int64_t)e * F : NULL, b, hc, hs);
    if (rc == ORACLE_OK)
      rc = oracle_gemm_codes(hc, hs, cnt, wdn_codes + (int64_t)e * H * (F / 2),
                             wdn_scales + (int64_t)e * H * (F / 32), H, F, ye, threads);
    if (rc == ORACLE_OK) {
      for (int64_t i = 0; i < cnt; ++i) {
        const int64_t r = idx[i];
        for (int64_t c = 0; c < H; ++c) rows_out[r * H + c] = round_bf16_of(ye[i * H + c]);
        if (dn_codes) memcpy(dn_codes + r * (F / 2), hc + i * (F / 2), (size_t)F / 2);
        if (dn_scales) memcpy(dn_scales + r * (F / 32), hs + i * (F / 32), (size_t)F / 32);
      }
    }
    free(idx);
    free(xe);
    free(gu);
    free(h);
    free(hc);
    free(hs);
    free(ye);
  }
  if (rc == ORACLE_OK) {
    for (int64_t t = 0; t < T; ++t) {
      if (want && !want[t]) continue;
      rc = oracle_moe_combine(rows_out, H, pos + t * k, w + t * k, 1, k, y + t * H);
      if (rc != ORACLE_OK) break;
    }
  }
  free(off);
  free(row_token);
  free(pos);
  free(rows_out);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Flip-Refinement of prepared weights                                  */
/* ------------------------------------------------------------------ */
/*
 * Sources: "MACaQ ..." (paper card, Abstract) improves on round-to-nearest
 * weights with Flip-Refinement, a Hessian-aware coordinate descent that
 * greedily moves single FP4 codes to adjacent representable values; "Huawei's
 * MACaQ-R beats Unsloth's ..." (Why that's still interesting) applies the
 * same idea to existing codes, and (What we found when we compared the
 * files) finds only codes changed, block scales kept. Readings (choices,
 * not page text):
 *   - the objective of output row n is e^T H e with e = w~ - q: w~ the row in
 *     the transformed basis (S_b (r .* w), the fp32 values the quantizer
 *     sees), q its dequantized codes, H = X~^T X~ over calibration rows in
 *     the same basis (x~ = S_b (a .* x), fp32), so that e.x~ is the row's
 *     output error on a calibration row (w~.x~ = w.x);
 *   - a move takes one element from signed E2M1 index m (value
 *     sign(m) LUT[|m|], m in -7..7) to m - 1 or m + 1 at the element's
 *     fixed group scale; it changes the objective by
 *     D = d*d*H[k][k] - 2*d*g[k] (d = the value step, g = H e);
 *   - each step takes the move with the most negative D (ties: lowest k,
 *     then the downward move), and the row stops when no move has D < 0 or
 *     after max_flips moves;
 *   - all of it in fp64 with sums in index order, each term added with one
 *     rounding (fused multiply-add): g[j] = sum over k of e[k] * H[k][j]
 *     (k ascending), H[j][k] = sum over r of x~[r][j] * x~[r][k] (r
 *     ascending; these products are exact); after a move g[j] -= d * H[k][j]
 *     (d is a power of two, so that product is exact too);
 *   - an element that is moved gets its canonical code (m = 0 is code 0);
 *     elements never moved keep their code bits (a -0 stays 0x8).
 */

/* H [K, K] (fp64) of R bf16 calibration rows through multiplier a and the
   block-Hadamard of size b. */
int oracle_hessian(const uint16_t* x, int64_t R, int64_t K, int64_t ldx, const float* a, int b, double* H) {
  if (!x || !H || R < 1 || K < 32 || ldx < K || !valid_block(b)) return ORACLE_EINVAL;
  if (b > 0 && K % b != 0) return ORACLE_EINVAL;
  float* t = (float*)malloc((size_t)R * K * sizeof(float));
  if (!t) return ORACLE_EINVAL;
  for (int64_t r = 0; r < R; ++r) transform_row(x, 0, r * ldx, a, K, b, t + r * K);
  for (int64_t j = 0; j < K; ++j)
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0;
      for (int64_t r = 0; r < R; ++r) acc = fma((double)t[r * K + j], (double)t[r * K + k], acc);
      H[j * K + k] = acc;
    }
  free(t);
  return ORACLE_OK;
}

/* signed E2M1 index of a code: -7..7 (code 8, -0, is index 0) */
static int code_index(unsigned c) { return (c & 8) ? -(int)(c & 7) : (int)(c & 7); }
static unsigned index_code(int m) { return m < 0 ? (8u | (unsigned)(-m)) : (unsigned)m; }
static double index_value(int m) { return m < 0 ? -kE2M1[-m] : kE2M1[m]; }

/* Flip-Refinement of N rows of prepared weights (row-major codes [N, K/2],
   scales [N, K/32], refined in place): W [N, ldw] (dtype 0 bf16, 1 fp32),
   weight multiplier r, block b, H [K, K]. flips[n] (optional) receives the
   number of moves of row n. */
int oracle_flip_refine(const void* W, int dtype, int64_t N, int64_t K, int64_t ldw, const float* r, int b,
                       const double* H, int max_flips, uint8_t* codes, const uint8_t* scales, int32_t* flips) {
  if (!W || !H || !codes || !scales || N < 1 || K < 32 || K % 32 != 0 || ldw < K || !valid_block(b) || max_flips < 0)
    return ORACLE_EINVAL;
  if (b > 0 && K % b != 0) return ORACLE_EINVAL;
  float* wt = (float*)malloc((size_t)K * sizeof(float));
  double* e = (double*)malloc((size_t)K * sizeof(double));
  double* g = (double*)malloc((size_t)K * sizeof(double));
  int* m = (int*)malloc((size_t)K * sizeof(int));
  int* m0 = (int*)malloc((size_t)K * sizeof(int));
  if (!wt || !e || !g || !m || !m0) {
    free(wt); free(e); free(g); free(m); free(m0);
    return ORACLE_EINVAL;
  }
  for (int64_t n = 0; n < N; ++n) {
    uint8_t* crow = codes + n * (K / 2);
    const uint8_t* srow = scales + n * (K / 32);
    transform_row(W, dtype, n * ldw, r, K, b, wt);
    for (int64_t k = 0; k < K; ++k) {
      const unsigned c = (k % 2 == 0) ? (crow[k / 2] & 0xF) : (crow[k / 2] >> 4);
      m[k] = m0[k] = code_index(c);
      e[k] = (double)wt[k] - ldexp(index_value(m[k]), (int)srow[k / 32] - 127);
    }
    for (int64_t j = 0; j < K; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc = fma(e[k], H[k * K + j], acc);
      g[j] = acc;
    }
    int moves = 0;
    while (moves < max_flips) {
      double best = 0.0;
      int64_t bk = -1;
      int bdir = 0;
      for (int64_t k = 0; k < K; ++k) {
        for (int dir = -1; dir <= 1; dir += 2) {
          const int mn = m[k] + dir;
          if (mn < -7 || mn > 7) continue;
          const double d = ldexp(index_value(mn) - index_value(m[k]), (int)srow[k / 32] - 127);
          const double D = d * d * H[k * K + k] - 2.0 * d * g[k];
          if (D < best) {
            best = D;
            bk = k;
            bdir = dir;
          }
        }
      }
      if (bk < 0) break;
      const double d = ldexp(index_value(m[bk] + bdir) - index_value(m[bk]), (int)srow[bk / 32] - 127);
      m[bk] += bdir;
      for (int64_t j = 0; j < K; ++j) g[j] -= d * H[bk * K + j];
      ++moves;
    }
    for (int64_t k = 0; k < K; ++k) {
      if (m[k] == m0[k]) continue;
      const unsigned c = index_code(m[k]);
      uint8_t* byte = crow + k / 2;
      *byte = (k % 2 == 0) ? (uint8_t)((*byte & 0xF0) | c) : (uint8_t)((*byte & 0x0F) | (c << 4));
    }
    if (flips) flips[n] = moves;
  }
  free(wt); free(e); free(g); free(m); free(m0);
  return ORACLE_OK;
}
