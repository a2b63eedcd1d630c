/*
 * Host-side memory and undefined-behaviour check of the C oracle (test
 * infrastructure). Built together with oracle/q4_oracle.c under
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitized.py and run as a child process: every call gets
 * buffers of exactly the size its contract states, allocated one by one, so a
 * read or write past any of them, a use of freed memory or an overflow in the
 * index arithmetic ends the run with the sanitizer's report.
 *
 * The shapes cover the edge cases of each entry point: one group (k = 32),
 * one row, a ragged row count, the model's widths, the last MultiLinear step,
 * tokens outside a table, position 0 and the last cache slot. Invalid
 * arguments must be refused without touching memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_bf16_round(const float* in, int64_t count, uint16_t* out);
int oracle_quantize(const float* w, int64_t n, int64_t k, uint32_t* packed, uint16_t* scales, uint16_t* biases);
int oracle_unpack(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                  uint8_t* q_out, float* w_out);
int oracle_matmul(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                  const uint16_t* biases, int64_t n, int64_t k, double* y);
int oracle_multilinear_step(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                            const uint16_t* biases, int64_t num_steps, int64_t out, int64_t k, int64_t step,
                            double* y);
int oracle_embed_sum(const int32_t* tokens, int64_t frames, int64_t streams, const uint32_t* const* packed,
                     const uint16_t* const* scales, const uint16_t* const* biases, const int64_t* rows,
                     int64_t dim, double* y);
int oracle_rope(const uint16_t* x, int64_t heads, int64_t d, int64_t pos, double theta, uint16_t* out);
int oracle_attn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t heads, int64_t d,
                       int64_t cap, int64_t pos, double* out);
int oracle_rmsnorm(const uint16_t* x, int64_t m, int64_t k, const uint16_t* g, double eps, uint16_t* out);
int oracle_silu_mul(const double* gate, const double* up, int64_t count, double* out);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, in [-1, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}
static void* take(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(3);
  }
  return p;
}
static int failures = 0;
static void expect(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}
static uint16_t* bf16_vector(int64_t count, double amp) {
  float* f = take(sizeof(float) * (size_t)count);
  uint16_t* b = take(sizeof(uint16_t) * (size_t)count);
  for (int64_t i = 0; i < count; ++i) f[i] = (float)(amp * uniform());
  expect(oracle_bf16_round(f, count, b) == 0, "bf16_round");
  free(f);
  return b;
}

/* quantize, unpack and multiply one [n][k] matrix against m rows */
static void product_case(int64_t n, int64_t k, int64_t m) {
  const int64_t nk = n * k;
  float* w = take(sizeof(float) * (size_t)nk);
  for (int64_t i = 0; i < nk; ++i) w[i] = (float)(0.02 * uniform());
  uint32_t* packed = take(sizeof(uint32_t) * (size_t)(nk / 8));
  uint16_t* scales = take(sizeof(uint16_t) * (size_t)(nk / 32));
  uint16_t* biases = take(sizeof(uint16_t) * (size_t)(nk / 32));
  expect(oracle_quantize(w, n, k, packed, scales, biases) == 0, "quantize");
  uint8_t* q = take((size_t)nk);
  float* wh = take(sizeof(float) * (size_t)nk);
  expect(oracle_unpack(packed, scales, biases, n, k, q, wh) == 0, "unpack");
  uint16_t* x = bf16_vector(m * k, 1.0);
  double* y = take(sizeof(double) * (size_t)(m * n));
  expect(oracle_matmul(x, m, packed, scales, biases, n, k, y) == 0, "matmul");
  for (int64_t i = 0; i < m * n; ++i) expect(isfinite(y[i]), "matmul output finite");
  /* a non-finite weight is refused */
  w[nk - 1] = INFINITY;
  expect(oracle_quantize(w, n, k, packed, scales, biases) != 0, "quantize refuses inf");
  free(w), free(packed), free(scales), free(biases), free(q), free(wh), free(x), free(y);
}

static void multilinear_case(int64_t steps, int64_t out, int64_t k, int64_t m) {
  const int64_t rows = steps * out;
  float* w = take(sizeof(float) * (size_t)(rows * k));
  for (int64_t i = 0; i < rows * k; ++i) w[i] = (float)(0.02 * uniform());
  uint32_t* packed = take(sizeof(uint32_t) * (size_t)(rows * k / 8));
  uint16_t* scales = take(sizeof(uint16_t) * (size_t)(rows * k / 32));
  uint16_t* biases = take(sizeof(uint16_t) * (size_t)(rows * k / 32));
  expect(oracle_quantize(w, rows, k, packed, scales, biases) == 0, "quantize stacked");
  uint16_t* x = bf16_vector(m * k, 1.0);
  double* y = take(sizeof(double) * (size_t)(m * out));
  expect(oracle_multilinear_step(x, m, packed, scales, biases, steps, out, k, 0, y) == 0, "multilinear first");
  expect(oracle_multilinear_step(x, m, packed, scales, biases, steps, out, k, steps - 1, y) == 0,
         "multilinear last");
  expect(oracle_multilinear_step(x, m, packed, scales, biases, steps, out, k, steps, y) != 0,
         "multilinear refuses a step past the last");
  free(w), free(packed), free(scales), free(biases), free(x), free(y);
}

static void embed_case(int64_t frames, int64_t streams, int64_t dim) {
  uint32_t** packed = take(sizeof(uint32_t*) * (size_t)streams);
  uint16_t** scales = take(sizeof(uint16_t*) * (size_t)streams);
  uint16_t** biases = take(sizeof(uint16_t*) * (size_t)streams);
  int64_t* rows = take(sizeof(int64_t) * (size_t)streams);
  for (int64_t t = 0; t < streams; ++t) {
    rows[t] = 3 + t % 5;
    float* w = take(sizeof(float) * (size_t)(rows[t] * dim));
    for (int64_t i = 0; i < rows[t] * dim; ++i) w[i] = (float)uniform();
    packed[t] = take(sizeof(uint32_t) * (size_t)(rows[t] * dim / 8));
    scales[t] = take(sizeof(uint16_t) * (size_t)(rows[t] * dim / 32));
    biases[t] = take(sizeof(uint16_t) * (size_t)(rows[t] * dim / 32));
    expect(oracle_quantize(w, rows[t], dim, packed[t], scales[t], biases[t]) == 0, "quantize table");
    free(w);
  }
  int32_t* tokens = take(sizeof(int32_t) * (size_t)(frames * streams));
  for (int64_t i = 0; i < frames * streams; ++i) {
    const int64_t t = i % streams;
    /* every third token lies outside its table (-1 or rows[t]): it adds nothing */
    tokens[i] = (int32_t)(i % 3 == 0 ? (i % 2 ? -1 : rows[t]) : (i * 7) % rows[t]);
  }
  double* y = take(sizeof(double) * (size_t)(frames * dim));
  expect(oracle_embed_sum(tokens, frames, streams, (const uint32_t* const*)packed, (const uint16_t* const*)scales,
                          (const uint16_t* const*)biases, rows, dim, y) == 0,
         "embed_sum");
  for (int64_t t = 0; t < streams; ++t) free(packed[t]), free(scales[t]), free(biases[t]);
  free(packed), free(scales), free(biases), free(rows), free(tokens), free(y);
}

static void attention_case(int64_t heads, int64_t d, int64_t cap) {
  uint16_t* q = bf16_vector(heads * d, 1.0);
  uint16_t* qr = take(sizeof(uint16_t) * (size_t)(heads * d));
  uint16_t* k = bf16_vector(heads * cap * d, 1.0);
  uint16_t* v = bf16_vector(heads * cap * d, 1.0);
  double* out = take(sizeof(double) * (size_t)(heads * d));
  expect(oracle_rope(q, heads, d, 0, 10000.0, qr) == 0, "rope at 0");
  expect(oracle_rope(q, heads, d, cap - 1, 10000.0, qr) == 0, "rope at the last slot");
  expect(oracle_attn_decode(qr, k, v, heads, d, cap, 0, out) == 0, "attention over one position");
  expect(oracle_attn_decode(qr, k, v, heads, d, cap, cap - 1, out) == 0, "attention over the full cache");
  expect(oracle_attn_decode(qr, k, v, heads, d, cap, cap, out) != 0, "attention refuses pos == cap");
  free(q), free(qr), free(k), free(v), free(out);
}

static void norm_case(int64_t m, int64_t k) {
  uint16_t* x = bf16_vector(m * k, 3.0);
  uint16_t* g = bf16_vector(k, 1.0);
  uint16_t* out = take(sizeof(uint16_t) * (size_t)(m * k));
  expect(oracle_rmsnorm(x, m, k, g, 1e-5, out) == 0, "rmsnorm");
  double* a = take(sizeof(double) * (size_t)k);
  double* b = take(sizeof(double) * (size_t)k);
  double* o = take(sizeof(double) * (size_t)k);
  for (int64_t i = 0; i < k; ++i) a[i] = 40.0 * uniform(), b[i] = uniform();
  expect(oracle_silu_mul(a, b, k, o) == 0, "silu_mul");
  free(x), free(g), free(out), free(a), free(b), free(o);
}

int main(void) {
  product_case(1, 32, 1);       /* one group */
  product_case(37, 96, 3);      /* ragged rows, 3 groups */
  product_case(300, 1056, 5);   /* 33 groups */
  product_case(64, 4096, 2);    /* the model's width */
  product_case(16, 11264, 1);   /* the FFN's width */
  multilinear_case(16, 40, 96, 2);
  multilinear_case(4, 64, 1024, 1);
  embed_case(3, 17, 256);
  attention_case(4, 128, 9);
  attention_case(1, 2, 1);
  norm_case(3, 4096);
  norm_case(1, 32);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitized run: ok\n");
  return 0;
}
