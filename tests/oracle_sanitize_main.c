/*
 * Drives every entry point of the CPU oracle on small inputs, including
 * non-finite and overflowing ones and rejected arguments, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py
 * compiles it together with oracle/macaq_oracle.c and runs it). Any
 * out-of-bounds access, leak or undefined operation aborts the run; the
 * checks below add what the oracle promises for such input:
 *   - nothing is read or written outside the arguments, and every call
 *     returns (no hang, no crash);
 *   - no scale code is 255 (E8M0 NaN is never produced);
 *   - a row's codes depend on that row only, and a group's codes on its own
 *     Hadamard block only: finite blocks next to a non-finite or overflowing
 *     one quantize exactly as they do alone;
 *   - invalid arguments are rejected with a non-zero code and nothing written.
 * Test infrastructure; it links only the oracle.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_calibrate(const void* xcal, int dtype, int64_t R, int64_t K, int64_t ld, float* s);
int oracle_calibrate_pow(const void* xcal, int dtype, int64_t R, int64_t K, int64_t ld, int quarters, float* s);
int oracle_multipliers(const float* s, int64_t K, int b, float* a, float* r);
int oracle_transform_rows(const void* x, int dtype, int64_t M, int64_t K, int64_t ld, const float* m, int b,
                          float* t);
int oracle_quant_rows(const void* x, int dtype, int64_t M, int64_t K, int64_t ld, const float* m, int b,
                      uint8_t* codes, uint8_t* scales);
int oracle_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t M, int64_t K, double* out);
int oracle_gemm_codes(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, const uint8_t* w_codes,
                      const uint8_t* w_scales, int64_t N, int64_t K, double* y, int threads);
int oracle_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* a, int b,
                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, double* y, int threads);
int oracle_linear_grouped(const uint16_t* x, const int32_t* off, int E, int64_t T, int64_t K, const float* a,
                          int b, const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, double* y,
                          int threads);
int oracle_moe_route(const int32_t* ids, int64_t T, int k, int E, int32_t* offsets, int32_t* row_token,
                     int32_t* pos);
int oracle_silu_mul(const double* gu, int64_t R, int64_t F, float* h);
int oracle_moe_combine(const float* rows, int64_t H, const int32_t* pos, const float* w, int64_t T, int k,
                       double* y);
int oracle_moe_block(const uint16_t* x, int64_t T, int64_t H, const int32_t* ids, const float* w, int k, int E,
                     const float* a_gu, const uint8_t* wgu_codes, const uint8_t* wgu_scales, const float* a_dn,
                     const uint8_t* wdn_codes, const uint8_t* wdn_scales, int64_t F, int b, const uint8_t* want,
                     uint8_t* dn_codes, uint8_t* dn_scales, double* y, int threads);
int oracle_hessian(const uint16_t* x, int64_t R, int64_t K, int64_t ldx, const float* a, int b, double* H);
int oracle_flip_refine(const void* W, int dtype, int64_t N, int64_t K, int64_t ldw, const float* r, int b,
                       const double* H, int max_flips, uint8_t* codes, const uint8_t* scales, int32_t* flips);

static int failures = 0;
#define CHECK(cond, ...)                        \
  do {                                          \
    if (!(cond)) {                              \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);             \
      fprintf(stderr, "\n");                    \
      ++failures;                               \
    }                                           \
  } while (0)

/* xorshift64*, seeded per test */
static uint64_t rng_state;
static double uniform(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static float normal(void) {
  double u = uniform() + 1e-300, v = uniform();
  return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}

/* bf16 bits of a float by truncation (inputs only need to be bf16 values) */
static uint16_t bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static const float kInf = INFINITY;

/* ------------------------------------------------------------------ */

static void test_quant_non_finite(int b) {
  enum { K = 256, M = 8 };
  const int bb = b > 0 ? b : 1;
  rng_state = 0x9E3779B97F4A7C15ull + (uint64_t)b;
  float x[M * K], m[K];
  for (int i = 0; i < M * K; ++i) x[i] = normal();
  for (int k = 0; k < K; ++k) m[k] = 0.5f + (float)uniform();
  /* row 1: +inf in channel 3; row 2: NaN in channel 40; row 3: -inf at 100;
     row 4: largest finite floats across its first block (the Hadamard sums
     overflow); row 5: NaN and inf everywhere; rows 0, 6, 7 finite */
  x[1 * K + 3] = kInf;
  x[2 * K + 40] = NAN;
  x[3 * K + 100] = -kInf;
  for (int k = 0; k < (b > 0 ? b : 32); ++k) x[4 * K + k] = 3.0e38f;
  for (int k = 0; k < K; ++k) x[5 * K + k] = (k % 2) ? NAN : kInf;
  uint8_t codes[M * K / 2], scales[M * K / 32];
  float t[M * K];
  CHECK(oracle_quant_rows(x, 1, M, K, K, m, b, codes, scales) == 0, "quant_rows b=%d", b);
  CHECK(oracle_transform_rows(x, 1, M, K, K, m, b, t) == 0, "transform_rows b=%d", b);
  for (int i = 0; i < M * K / 32; ++i) CHECK(scales[i] != 255, "scale 255 at %d (b=%d)", i, b);
  /* every finite block quantizes as it does alone (the row with all other
     channels zero), which also covers the finite rows */
  const int bad_ch[M] = {-1, 3, 40, 100, 0, -2, -1, -1}; /* -2: whole row non-finite */
  for (int r = 0; r < M; ++r) {
    if (bad_ch[r] == -2) continue;
    for (int g = 0; g < K / 32; ++g) {
      const int blk0 = (32 * g) / bb * bb, blk1 = blk0 + (bb > 32 ? bb : 32);
      int touched = 0;
      if (bad_ch[r] >= 0) {
        const int lo = (r == 4) ? 0 : bad_ch[r], hi = (r == 4) ? (b > 0 ? b : 32) : bad_ch[r] + 1;
        touched = lo < blk1 && hi > blk0;
      }
      if (touched) continue;
      float alone[K];
      memset(alone, 0, sizeof alone);
      for (int k = blk0; k < blk1; ++k) alone[k] = x[r * K + k];
      uint8_t c1[K / 2], s1[K / 32];
      CHECK(oracle_quant_rows(alone, 1, 1, K, K, m, b, c1, s1) == 0, "alone");
      CHECK(s1[g] == scales[r * K / 32 + g], "row %d group %d scale (b=%d)", r, g, b);
      CHECK(memcmp(c1 + 16 * g, codes + r * K / 2 + 16 * g, 16) == 0, "row %d group %d codes (b=%d)", r, g, b);
    }
  }
  /* bf16 input with the same pattern */
  uint16_t xb[M * K];
  for (int i = 0; i < M * K; ++i) xb[i] = bf16_bits(x[i]);
  CHECK(oracle_quant_rows(xb, 0, M, K, K, m, b, codes, scales) == 0, "quant_rows bf16 b=%d", b);
  for (int i = 0; i < M * K / 32; ++i) CHECK(scales[i] != 255, "bf16 scale 255 at %d (b=%d)", i, b);
  /* multipliers that are non-finite or zero */
  float m2[K];
  for (int k = 0; k < K; ++k) m2[k] = (k % 7 == 0) ? kInf : (k % 11 == 0) ? NAN : (k % 13 == 0) ? 0.0f : m[k];
  CHECK(oracle_quant_rows(x, 1, M, K, K, m2, b, codes, scales) == 0, "quant_rows bad multipliers b=%d", b);
  for (int i = 0; i < M * K / 32; ++i) CHECK(scales[i] != 255, "scale 255 with bad multipliers (b=%d)", b);
}

static void test_calibration(void) {
  enum { R = 5, K = 64 };
  float x[R * K];
  rng_state = 7;
  for (int i = 0; i < R * K; ++i) x[i] = normal();
  x[0 * K + 1] = kInf;
  x[1 * K + 2] = NAN;
  x[2 * K + 3] = -kInf;
  for (int r = 0; r < R; ++r) x[r * K + 4] = 0.0f; /* all-zero channel */
  x[3 * K + 5] = 1e-45f;                           /* subnormal */
  float s[K], a[K], rr[K];
  CHECK(oracle_calibrate(x, 1, R, K, K, s) == 0, "calibrate");
  CHECK(s[4] == 1.0f, "all-zero channel gets 1 (got %g)", s[4]);
  for (int q = 0; q <= 4; ++q) {
    const int rc = oracle_calibrate_pow(x, 1, R, K, K, q, s);
    CHECK((q == 3) ? rc != 0 : rc == 0, "calibrate_pow quarters=%d rc=%d", q, rc);
  }
  CHECK(oracle_calibrate(x, 1, R, K, K, s) == 0, "calibrate");
  const int blocks[5] = {0, 32, 64, 128, 16};
  for (int i = 0; i < 5; ++i) {
    const int rc = oracle_multipliers(s, K, blocks[i], a, rr);
    CHECK((blocks[i] == 16) ? rc != 0 : rc == 0, "multipliers b=%d rc=%d", blocks[i], rc);
  }
  /* fp32 input from the same data as bf16 */
  uint16_t xb[R * K];
  for (int i = 0; i < R * K; ++i) xb[i] = bf16_bits(x[i]);
  CHECK(oracle_calibrate(xb, 0, R, K, K, s) == 0, "calibrate bf16");
}

static void test_dequant_gemm(void) {
  /* every code byte under every scale code, 255 included */
  enum { M = 256, K = 32 * 256 / 32 };
  uint8_t* codes = malloc((size_t)M * K / 2);
  uint8_t* scales = malloc((size_t)M * K / 32);
  double* out = malloc((size_t)M * K * sizeof(double));
  for (int r = 0; r < M; ++r) {
    for (int i = 0; i < K / 2; ++i) codes[r * K / 2 + i] = (uint8_t)(i + r);
    for (int g = 0; g < K / 32; ++g) scales[r * K / 32 + g] = (uint8_t)(r + 31 * g);
  }
  CHECK(oracle_dequant_rows(codes, scales, M, K, out) == 0, "dequant_rows");
  free(out);
  /* GEMM with more threads than rows, and a single row */
  double* y = malloc((size_t)M * M * sizeof(double));
  CHECK(oracle_gemm_codes(codes, scales, 3, codes, scales, 5, K, y, 16) == 0, "gemm 3x5 16 threads");
  CHECK(oracle_gemm_codes(codes, scales, 1, codes, scales, 1, K, y, 1) == 0, "gemm 1x1");
  CHECK(oracle_gemm_codes(codes, scales, 0, codes, scales, 1, K, y, 1) != 0, "gemm M=0 rejected");
  CHECK(oracle_gemm_codes(codes, scales, 4, codes, scales, 4, 48, y, 1) != 0, "gemm K=48 rejected");
  CHECK(oracle_gemm_codes(NULL, scales, 4, codes, scales, 4, K, y, 1) != 0, "gemm NULL rejected");
  free(y);
  free(codes);
  free(scales);
}

static void make_weights(int64_t N, int64_t K, int b, const float* r, uint8_t* wc, uint8_t* ws) {
  float* w = malloc((size_t)N * K * sizeof(float));
  for (int64_t i = 0; i < N * K; ++i) w[i] = 0.02f * normal();
  CHECK(oracle_quant_rows(w, 1, N, K, K, r, b, wc, ws) == 0, "prepare weights");
  free(w);
}

static void test_linear_and_moe(void) {
  enum { T = 9, H = 128, F = 64, E = 4, k = 3 };
  rng_state = 99;
  uint16_t x[T * H];
  for (int i = 0; i < T * H; ++i) x[i] = bf16_bits(normal());
  x[2 * H + 5] = bf16_bits(kInf);
  x[4 * H + 9] = bf16_bits(NAN);
  float a_gu[E * H], a_dn[E * F], r_gu[E * H];
  for (int i = 0; i < E * H; ++i) a_gu[i] = r_gu[i] = 0.5f + (float)uniform();
  for (int i = 0; i < E * F; ++i) a_dn[i] = 0.5f + (float)uniform();
  uint8_t* gc = malloc((size_t)E * 2 * F * H / 2);
  uint8_t* gs = malloc((size_t)E * 2 * F * H / 32);
  uint8_t* dc = malloc((size_t)E * H * F / 2);
  uint8_t* ds = malloc((size_t)E * H * F / 32);
  for (int e = 0; e < E; ++e) {
    make_weights(2 * F, H, 32, r_gu + e * H, gc + (size_t)e * 2 * F * H / 2, gs + (size_t)e * 2 * F * H / 32);
    make_weights(H, F, 32, a_dn + e * F, dc + (size_t)e * H * F / 2, ds + (size_t)e * H * F / 32);
  }
  double y[T * 2 * F];
  CHECK(oracle_linear(x, T, H, H, a_gu, 32, gc, gs, 2 * F, y, 3) == 0, "linear");
  CHECK(oracle_linear(x, T, 48, H, a_gu, 32, gc, gs, 2 * F, y, 3) != 0, "linear K=48 rejected");
  /* grouped: an empty expert in the middle and at the end */
  const int32_t off[E + 1] = {0, 4, 4, T, T};
  double yg[T * H];
  CHECK(oracle_linear_grouped(x, off, E, T, H, a_gu, 32, gc, gs, 2 * F, y, 2) == 0, "linear_grouped");
  const int32_t bad_off[E + 1] = {0, 5, 4, T, T};
  CHECK(oracle_linear_grouped(x, bad_off, E, T, H, a_gu, 32, gc, gs, 2 * F, y, 2) != 0, "decreasing offsets");
  /* routing with ids out of range, and no entries at all */
  int32_t ids[T * k], offsets[E + 1], row_token[T * k], pos[T * k];
  for (int i = 0; i < T * k; ++i) ids[i] = (int32_t)(uniform() * (E + 2)) - 1; /* -1 .. E */
  CHECK(oracle_moe_route(ids, T, k, E, offsets, row_token, pos) == 0, "route");
  CHECK(oracle_moe_route(ids, 0, k, E, offsets, row_token, pos) == 0, "route T=0");
  /* SiLU * up on non-finite and large gate / up values */
  double gu[2 * 64 * 2];
  for (int i = 0; i < 256; ++i) gu[i] = (i % 5 == 0) ? kInf : (i % 5 == 1) ? -kInf : (i % 5 == 2) ? NAN
                                          : (i % 5 == 3) ? -1000.0 : 1000.0;
  float h[2 * 64];
  CHECK(oracle_silu_mul(gu, 2, 64, h) == 0, "silu_mul");
  CHECK(oracle_silu_mul(gu, 2, 48, h) != 0, "silu_mul F=48 rejected");
  /* combine with skipped slots */
  float rows[T * k * H];
  for (int i = 0; i < T * k * H; ++i) rows[i] = normal();
  float w[T * k];
  for (int i = 0; i < T * k; ++i) w[i] = (float)uniform();
  CHECK(oracle_moe_combine(rows, H, pos, w, T, k, yg) == 0, "combine");
  /* the whole block, some tokens only, with bad ids */
  uint8_t want[T];
  for (int t = 0; t < T; ++t) want[t] = (uint8_t)(t % 2);
  uint8_t dnc[T * k * F / 2], dns[T * k * F / 32];
  CHECK(oracle_moe_block(x, T, H, ids, w, k, E, a_gu, gc, gs, a_dn, dc, ds, F, 32, want, dnc, dns, yg, 3) == 0,
        "moe_block");
  CHECK(oracle_moe_block(x, T, H, ids, w, k, E, a_gu, gc, gs, a_dn, dc, ds, F, 32, NULL, NULL, NULL, yg, 1) == 0,
        "moe_block all tokens, no down-input output");
  free(gc);
  free(gs);
  free(dc);
  free(ds);
}

static void test_hessian_flip(void) {
  enum { R = 16, K = 64, N = 4 };
  rng_state = 1234;
  uint16_t x[R * K];
  for (int i = 0; i < R * K; ++i) x[i] = bf16_bits(normal());
  float a[K], r[K];
  for (int i = 0; i < K; ++i) a[i] = r[i] = 1.0f;
  double* H = malloc((size_t)K * K * sizeof(double));
  CHECK(oracle_hessian(x, R, K, K, a, 32, H) == 0, "hessian");
  float W[N * K];
  for (int i = 0; i < N * K; ++i) W[i] = 0.05f * normal();
  uint8_t wc[N * K / 2], ws[N * K / 32];
  int32_t flips[N];
  CHECK(oracle_quant_rows(W, 1, N, K, K, r, 32, wc, ws) == 0, "prepare");
  CHECK(oracle_flip_refine(W, 1, N, K, K, r, 32, H, 50, wc, ws, flips) == 0, "flip_refine");
  CHECK(oracle_flip_refine(W, 1, N, K, K, r, 32, H, -1, wc, ws, flips) != 0, "max_flips < 0 rejected");
  free(H);
}

static void test_rejections(void) {
  float x[64 * 2] = {0}, t[64 * 2];
  uint8_t c[64], s[4];
  memset(t, 0x5A, sizeof t);
  memset(c, 0x5A, sizeof c);
  CHECK(oracle_quant_rows(x, 1, 2, 48, 48, NULL, 0, c, s) != 0, "K=48");
  CHECK(oracle_quant_rows(x, 1, 2, 64, 32, NULL, 0, c, s) != 0, "ld < K");
  CHECK(oracle_quant_rows(x, 1, 2, 64, 64, NULL, 16, c, s) != 0, "b=16");
  CHECK(oracle_quant_rows(x, 1, 1, 96, 96, NULL, 64, c, s) != 0, "K % b");
  CHECK(oracle_quant_rows(NULL, 1, 2, 64, 64, NULL, 0, c, s) != 0, "x NULL");
  CHECK(oracle_transform_rows(x, 1, 0, 64, 64, NULL, 0, t) != 0, "M=0");
  uint8_t untouched[64];
  memset(untouched, 0x5A, sizeof untouched);
  CHECK(memcmp(c, untouched, sizeof c) == 0, "rejected calls wrote codes");
}

int main(void) {
  const int blocks[4] = {0, 32, 64, 128};
  for (int i = 0; i < 4; ++i) test_quant_non_finite(blocks[i]);
  test_calibration();
  test_dequant_gemm();
  test_linear_and_moe();
  test_hessian_flip();
  test_rejections();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle checks passed\n");
  return 0;
}
