/*
 * Reference CPU oracle for the affine 4-bit group-32 quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously-correct
 * statement of what the GPU path must compute. Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it. It
 * shares no code, header, table or constant with the HIP library.
 *
 * What it follows (sources are the web pages the method is taken from):
 *  - "personaplex-edge-q4" model card, Release details table: the format is
 *    affine Q4 with group size 32 and BF16 activations; the parameter count
 *    and the source/packed sizes in that table fix 5 bits per weight, i.e. a
 *    4-bit code plus a 16-bit scale and a 16-bit bias per 32 weights.
 *  - same card, introduction: weights stay packed at inference and feed a
 *    quantized matmul; they are not expanded back to BF16.
 *  - "NVIDIA PersonaPlex 7B on Apple Silicon" (blog translation), section on
 *    the Depformer's per-step weight switching (MultiLinear code figure): the
 *    quantized product takes (x, w, scales, biases) with transpose, i.e.
 *    y = x . W^T with W stored [out, in], groups running along `in`, and a
 *    codebook step s slicing rows [s*out, (s+1)*out) of weight, scales and
 *    biases together.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - quantizer: per group, mn = min, mx = max, scale = fl32(fl32(mx-mn)/15)
 *    with a correctly rounded divide, bias = mn; both stored as bf16 by
 *    round-to-nearest-even; codes are computed against the STORED bf16
 *    scale/bias: q = clamp(rint_half_even(fl32(fl32(w-b')/s')), 0, 15), and
 *    q = 0 for every element when the stored scale is zero;
 *  - min/max scan the group in index order with strict comparisons;
 *  - packing: 8 codes per uint32 along the input dimension, code t of a word
 *    in bits [4t, 4t+4) (low nibble first); scales and biases are two
 *    separate [n][k/32] arrays of bf16 bit patterns;
 *  - dequantized weight w_hat = fl32(s' * q + b') (s'*q is exact, so this is
 *    a single rounding);
 *  - product: y[m][n] = sum_k w_hat[n][k] * x[m][k], summed in double in
 *    natural k order (each product is exact in double).
 *
 * Non-finite inputs are outside the method's domain: every entry point
 * rejects them with a nonzero return code.
 *
 * Built with gcc -O2 -ffp-contract=off -fopenmp (no intrinsics); OpenMP is
 * used only to split output rows across host threads.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NONFINITE 2

/* --- bf16 helpers: a bf16 is the upper 16 bits of an IEEE binary32 --- */

static float bits_to_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t f32_to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

/* Value of a bf16 bit pattern: exact widening to binary32. */
static float bf16_value(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* Round a finite binary32 to bf16, to nearest, ties to even. Dropping the
 * low 16 bits is truncation; adding 0x7FFF plus the kept LSB first turns it
 * into round-half-even (a carry out of the mantissa correctly bumps the
 * exponent). */
static uint16_t bf16_round_nearest_even(float f) {
  uint32_t u = f32_to_bits(f);
  uint32_t kept_lsb = (u >> 16) & 1u;
  u += 0x7FFFu + kept_lsb;
  return (uint16_t)(u >> 16);
}

/* --- quantize + pack --- */

int oracle_version(void) { return 1; }

int oracle_bf16_round(const float* in, int64_t count, uint16_t* out) {
  if (!in || !out || count < 0) return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < count; ++i) {
    if (!isfinite(in[i])) return ORACLE_ERR_NONFINITE;
    out[i] = bf16_round_nearest_even(in[i]);
  }
  return ORACLE_OK;
}

/* Quantize one group of 32 weights; write 32 codes, the stored scale and bias. */
static void quantize_group(const float* w, uint8_t* q, uint16_t* scale_bits, uint16_t* bias_bits) {
  float mn = w[0], mx = w[0];
  for (int i = 1; i < 32; ++i) {
    if (w[i] < mn) mn = w[i];
    if (w[i] > mx) mx = w[i];
  }
  float range = mx - mn;
  float scale = range / 15.0f;
  uint16_t sb = bf16_round_nearest_even(scale);
  uint16_t bb = bf16_round_nearest_even(mn);
  float s_stored = bf16_value(sb);
  float b_stored = bf16_value(bb);
  for (int i = 0; i < 32; ++i) {
    if (s_stored == 0.0f) {
      q[i] = 0;
      continue;
    }
    float t = (w[i] - b_stored) / s_stored;
    float r = rintf(t); /* default rounding mode: nearest, ties to even */
    if (r < 0.0f) r = 0.0f;
    if (r > 15.0f) r = 15.0f;
    q[i] = (uint8_t)r;
  }
  *scale_bits = sb;
  *bias_bits = bb;
}

/* w: fp32 [n][k] row-major, k % 32 == 0.
 * packed: uint32 [n][k/8]; scales, biases: bf16 bits [n][k/32]. */
int oracle_quantize(const float* w, int64_t n, int64_t k, uint32_t* packed, uint16_t* scales,
                    uint16_t* biases) {
  if (!w || !packed || !scales || !biases || n < 0 || k < 0 || k % 32 != 0) return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < n * k; ++i)
    if (!isfinite(w[i])) return ORACLE_ERR_NONFINITE;
  const int64_t groups = k / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < groups; ++g) {
      uint8_t q[32];
      quantize_group(w + r * k + g * 32, q, &scales[r * groups + g], &biases[r * groups + g]);
      for (int j = 0; j < 4; ++j) {
        uint32_t word = 0;
        for (int t = 0; t < 8; ++t) word |= (uint32_t)q[8 * j + t] << (4 * t);
        packed[r * (k / 8) + g * 4 + j] = word;
      }
    }
  }
  return ORACLE_OK;
}

/* --- unpack / dequantize --- */

/* q_out (nullable): uint8 [n][k]; w_out (nullable): fp32 [n][k]. */
int oracle_unpack(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases, int64_t n,
                  int64_t k, uint8_t* q_out, float* w_out) {
  if (!packed || !scales || !biases || n < 0 || k < 0 || k % 32 != 0) return ORACLE_ERR_ARG;
  const int64_t groups = k / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t c = 0; c < k; ++c) {
      uint32_t word = packed[r * (k / 8) + c / 8];
      uint8_t q = (uint8_t)((word >> (4 * (c % 8))) & 0xFu);
      if (q_out) q_out[r * k + c] = q;
      if (w_out) {
        float s = bf16_value(scales[r * groups + c / 32]);
        float b = bf16_value(biases[r * groups + c / 32]);
        w_out[r * k + c] = s * (float)q + b;
      }
    }
  }
  return ORACLE_OK;
}

/* --- quantized product y = x . W_hat^T --- */

/* x: bf16 bits [m][k]; y: double [m][n] (exact-sum reference, before any
 * output rounding). Dequantizes each weight to fp32 and takes a plain dot
 * product accumulated in double. */
int oracle_matmul(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                  const uint16_t* biases, int64_t n, int64_t k, double* y) {
  if (!x || !packed || !scales || !biases || !y || m < 0 || n < 0 || k < 0 || k % 32 != 0)
    return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < m * k; ++i)
    if (!isfinite(bf16_value(x[i]))) return ORACLE_ERR_NONFINITE;
  const int64_t groups = k / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t row = 0; row < m; ++row) {
      double acc = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        uint32_t word = packed[r * (k / 8) + c / 8];
        uint32_t q = (word >> (4 * (c % 8))) & 0xFu;
        float s = bf16_value(scales[r * groups + c / 32]);
        float b = bf16_value(biases[r * groups + c / 32]);
        float w_hat = s * (float)q + b;
        acc += (double)w_hat * (double)bf16_value(x[row * k + c]);
      }
      y[row * n + r] = acc;
    }
  }
  return ORACLE_OK;
}

/* Depformer per-step product: weights hold num_steps blocks of `out` rows
 * ([num_steps*out][k]); step s uses rows [s*out, (s+1)*out) of the packed
 * codes, scales and biases together, then the same product. */
int oracle_multilinear_step(const uint16_t* x, int64_t m, const uint32_t* packed,
                            const uint16_t* scales, const uint16_t* biases, int64_t num_steps,
                            int64_t out, int64_t k, int64_t step, double* y) {
  if (num_steps <= 0 || step < 0 || step >= num_steps || out < 0 || k < 0 || k % 32 != 0)
    return ORACLE_ERR_ARG;
  if (!packed || !scales || !biases) return ORACLE_ERR_ARG;
  const int64_t start = step * out;
  return oracle_matmul(x, m, packed + start * (k / 8), scales + start * (k / 32),
                       biases + start * (k / 32), out, k, y);
}

/* --- packed-embedding gather and stream sum --- */

/* The step's input is the sum of one embedding row per token stream: the
 * text stream and the audio codebook streams are summed into one vector
 * ("NVIDIA PersonaPlex 7B on Apple Silicon", pipeline figure: 17 streams,
 * text plus 8 user plus 8 assistant audio, summed into the temporal
 * transformer), and the embeddings stay packed ("personaplex-edge-q4" model
 * card, introduction). Each stream t has its own table, stored in the packed
 * layout above with rows[t] rows of `dim` values. For frame f:
 *   y[f][d] = sum over t of w_hat_t[tokens[f][t]][d]
 * where a token outside [0, rows[t]) (a stream with no token this frame)
 * adds nothing. Each w_hat is the fp32 dequantized value (exact), summed in
 * double in stream order. tokens: int32 [frames][streams]; y: double
 * [frames][dim]. */
int oracle_embed_sum(const int32_t* tokens, int64_t frames, int64_t streams, const uint32_t* const* packed,
                     const uint16_t* const* scales, const uint16_t* const* biases, const int64_t* rows,
                     int64_t dim, double* y) {
  if (!tokens || !packed || !scales || !biases || !rows || !y || frames < 0 || streams < 1 || dim <= 0 ||
      dim % 32 != 0)
    return ORACLE_ERR_ARG;
  for (int64_t t = 0; t < streams; ++t)
    if (!packed[t] || !scales[t] || !biases[t] || rows[t] < 0) return ORACLE_ERR_ARG;
  const int64_t groups = dim / 32;
  for (int64_t f = 0; f < frames; ++f) {
    for (int64_t d = 0; d < dim; ++d) {
      double acc = 0.0;
      for (int64_t t = 0; t < streams; ++t) {
        const int64_t tok = tokens[f * streams + t];
        if (tok < 0 || tok >= rows[t]) continue;
        uint32_t word = packed[t][tok * (dim / 8) + d / 8];
        uint32_t q = (word >> (4 * (d % 8))) & 0xFu;
        float s = bf16_value(scales[t][tok * groups + d / 32]);
        float b = bf16_value(biases[t][tok * groups + d / 32]);
        float w_hat = s * (float)q + b;
        acc += (double)w_hat;
      }
      y[f * dim + d] = acc;
    }
  }
  return ORACLE_OK;
}

/* --- single-query attention over the KV cache (one decoding step) --- */

/* Rotary position embedding at position pos ("NVIDIA PersonaPlex 7B on Apple
 * Silicon", optimisation list: the RoPE offset is passed to the step as an
 * input; the same page reuses RoPE among the model's parts). The pages do not
 * give the form: the reading is the original rotary embedding, which turns
 * each pair (x[2i], x[2i+1]) of a head by the angle pos * theta^(-2i/D).
 * x: bf16 [heads][D] (D even); out: the rotated values rounded to bf16. */
int oracle_rope(const uint16_t* x, int64_t heads, int64_t d, int64_t pos, double theta, uint16_t* out) {
  if (!x || !out || heads < 0 || d <= 0 || d % 2 != 0 || pos < 0 || !(theta > 0.0)) return ORACLE_ERR_ARG;
  for (int64_t h = 0; h < heads; ++h) {
    for (int64_t i = 0; i < d / 2; ++i) {
      const double angle = (double)pos * pow(theta, -(double)(2 * i) / (double)d);
      const double c = cos(angle), sn = sin(angle);
      const double x0 = (double)bf16_value(x[h * d + 2 * i]);
      const double x1 = (double)bf16_value(x[h * d + 2 * i + 1]);
      /* the rotated pair in double, rounded to fp32, then to bf16 */
      out[h * d + 2 * i] = bf16_round_nearest_even((float)(x0 * c - x1 * sn));
      out[h * d + 2 * i + 1] = bf16_round_nearest_even((float)(x0 * sn + x1 * c));
    }
  }
  return ORACLE_OK;
}

/* Attention of one query per head over positions 0..pos of the cache (the
 * ONNX bundle's README, How to use: the step takes and returns the K and V
 * caches [layers][1][32 heads][T][128] explicitly). For head h:
 *   s_t = (q_h . k_h[t]) / sqrt(D) for t = 0..pos,
 *   out_h = sum_t softmax(s)_t v_h[t],
 * in double. q: bf16 [heads][D] (already rotated); k, v: bf16
 * [heads][cap][D]; out: double [heads][D]. */
int oracle_attn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t heads, int64_t d,
                       int64_t cap, int64_t pos, double* out) {
  if (!q || !k || !v || !out || heads < 0 || d <= 0 || cap <= 0 || pos < 0 || pos >= cap) return ORACLE_ERR_ARG;
  const double scale = 1.0 / sqrt((double)d);
  double* s = (double*)malloc(sizeof(double) * (size_t)(pos + 1));
  if (!s) return ORACLE_ERR_ARG;
  for (int64_t h = 0; h < heads; ++h) {
    double mx = -HUGE_VAL;
    for (int64_t t = 0; t <= pos; ++t) {
      double dot = 0.0;
      for (int64_t i = 0; i < d; ++i)
        dot += (double)bf16_value(q[h * d + i]) * (double)bf16_value(k[(h * cap + t) * d + i]);
      s[t] = dot * scale;
      if (s[t] > mx) mx = s[t];
    }
    double z = 0.0;
    for (int64_t t = 0; t <= pos; ++t) {
      s[t] = exp(s[t] - mx);
      z += s[t];
    }
    for (int64_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int64_t t = 0; t <= pos; ++t) acc += s[t] * (double)bf16_value(v[(h * cap + t) * d + i]);
      out[h * d + i] = acc / z;
    }
  }
  free(s);
  return ORACLE_OK;
}

/* --- the parts of a decoder layer around its linear products --- */

/* RMSNorm of each activation row (the GeekNews summary's audio pipeline and
 * the blog translation's reuse of RMSNorm among the model's parts): for row
 * i of x (bf16 [m][k]) and the norm weight g (bf16 [k]),
 *   inv = 1 / sqrt(sum_j x_j^2 / k + eps),  out_j = bf16((x_j * g_j) * inv)
 * with every operation in double (x_j^2 and x_j * g_j are exact: products of
 * two bf16 values), then rounded to fp32 and to bf16: the normalized row is a
 * bf16 activation like every other. The definition is exact arithmetic;
 * taking the exact product x_j * g_j first leaves one rounding in the scaling. */
int oracle_rmsnorm(const uint16_t* x, int64_t m, int64_t k, const uint16_t* g, double eps, uint16_t* out) {
  if (!x || !g || !out || m < 0 || k <= 0 || !(eps >= 0.0)) return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < m * k; ++i)
    if (!isfinite(bf16_value(x[i]))) return ORACLE_ERR_NONFINITE;
  for (int64_t i = 0; i < m; ++i) {
    double ss = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      const double v = (double)bf16_value(x[i * k + j]);
      ss += v * v;
    }
    const double inv = 1.0 / sqrt(ss / (double)k + eps);
    for (int64_t j = 0; j < k; ++j) {
      const double v = ((double)bf16_value(x[i * k + j]) * (double)bf16_value(g[j])) * inv;
      out[i * k + j] = bf16_round_nearest_even((float)v);
    }
  }
  return ORACLE_OK;
}

/* The gated FFN's product (SwiGLU, reused among the model's parts per the
 * same pages): out_j = silu(gate_j) * up_j, silu(t) = t / (1 + exp(-t)), in
 * double on the exact (double) products. */
int oracle_silu_mul(const double* gate, const double* up, int64_t count, double* out) {
  if (!gate || !up || !out || count < 0) return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < count; ++i) out[i] = gate[i] / (1.0 + exp(-gate[i])) * up[i];
  return ORACLE_OK;
}

/* Threads the OpenMP runtime will use (1 when built without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int t) {
#ifdef _OPENMP
  if (t > 0) omp_set_num_threads(t);
#else
  (void)t;
#endif
}
