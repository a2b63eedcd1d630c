/*
 * q4.h — C ABI of the MI355X (gfx950) affine 4-bit group-32 quantized linear
 * library (libq4.so).
 *
 * The operation: a weight matrix W [out = n][in = k] is stored quantized in
 * groups of 32 consecutive input elements; each group has a bf16 scale s and
 * a bf16 bias b, and each weight a 4-bit code q in 0..15, with
 * w_hat = s*q + b. Activations are bf16. The product is y = x . W_hat^T
 * ("personaplex-edge-q4" model card, introduction and Release details table:
 * affine Q4, group size 32, BF16 activations, weights kept packed at
 * inference; "NVIDIA PersonaPlex 7B on Apple Silicon", Depformer MultiLinear
 * code figure: quantized product with transpose, scales and biases sliced by
 * output rows).
 *
 * STORED LAYOUT, version 1 (q4_layout_version() == 1):
 *   packed : uint32 [n][k/8], row-major. Word j of row r holds the codes of
 *            inputs 8j..8j+7; the code of input 8j+t sits in bits [4t, 4t+4)
 *            (low nibble first). One 16-byte run of 4 words is one group.
 *   scales : uint16 [n][k/32], bf16 bit patterns, row-major.
 *   biases : uint16 [n][k/32], bf16 bit patterns, row-major.
 *   Stored bytes per weight: 1/2 + 2/32 + 2/32 = 5/8.
 * A MultiLinear weight for S codebook steps is one such tensor with
 * n = S*out rows; step s owns rows [s*out, (s+1)*out).
 *
 * CONVENTIONS FOR EVERY ENTRY POINT
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or retains them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call is asynchronous on that stream and performs no host/device
 *     synchronisation and no allocation, so it may be captured into a HIP
 *     graph.
 *   - Arguments are validated on the host before any HIP call; the first
 *     failing check decides the status, and on any error nothing is launched.
 *     Checks, in order: a required pointer is NULL -> Q4_ERR_NULL; a size is
 *     out of range -> Q4_ERR_SHAPE; a pointer is misaligned -> Q4_ERR_ALIGN;
 *     a valid size the kernels do not cover -> Q4_ERR_UNSUPPORTED.
 *   - n == 0 is a valid empty call: nothing is launched and Q4_OK returned.
 *   - k must be a positive multiple of 32.
 *   - Alignment: `w` (fp32 input of q4_pack), `packed`, `x`, and the unpack
 *     outputs must be 16-byte aligned; scales, biases and y need their natural
 *     element alignment.
 *   - A launch failure returns Q4_ERR_HIP; q4_last_hip_error() then gives the
 *     hipError_t value (per calling thread).
 *   - Non-finite weights or activations are outside the method's domain; they
 *     are not checked on the device and give unspecified results.
 *   - Accumulation is fp32; outputs are rounded once (round to nearest even)
 *     when y is bf16. Results are deterministic: no atomics are used in any
 *     reduction.
 *   - No C++ exception crosses this interface. The library is thread-safe.
 */
#ifndef Q4_H
#define Q4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_GROUP 32
#define Q4_MAX_M 16
#define Q4_MAX_K 16384

typedef enum q4_status {
  Q4_OK = 0,
  Q4_ERR_NULL = 1,
  Q4_ERR_SHAPE = 2,
  Q4_ERR_ALIGN = 3,
  Q4_ERR_UNSUPPORTED = 4,
  Q4_ERR_HIP = 5
} q4_status;

typedef enum q4_out_dtype { Q4_OUT_BF16 = 0, Q4_OUT_F32 = 1 } q4_out_dtype;

/* Version of the stored layout described above. Returns 1. */
int q4_layout_version(void);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* q4_status_str(int status);

/* hipError_t of the most recent Q4_ERR_HIP returned on the calling thread
 * (0 if none). */
int q4_last_hip_error(void);

/* Quantize and pack (model card, Release details table: affine Q4, group 32).
 * For each row and each group of 32 inputs: mn/mx = min/max of the group,
 * scale = (mx - mn)/15 in fp32 (correctly rounded), stored scale s' and bias
 * b' = the bf16 (nearest-even) roundings of scale and mn; each code is
 * clamp(rint_half_even((w - b')/s'), 0, 15), or 0 for the whole group when
 * s' == 0. min/max scan the group in index order with strict comparisons.
 *   w      : fp32 [n][k] (input)
 *   packed : uint32 [n][k/8], scales/biases: uint16 [n][k/32] (outputs)
 * Bit-exact with the CPU oracle. */
q4_status q4_pack(const float* w, int64_t n, int64_t k, uint32_t* packed, uint16_t* scales,
                  uint16_t* biases, void* stream);

/* Unpack: recover codes and/or dequantized weights w_hat = s'*q + b' (one
 * rounding to fp32; the product s'*q is exact). Bit-exact with the oracle.
 *   q_out : uint8 [n][k] or NULL;  w_out : fp32 [n][k] or NULL (at least one
 *   must be non-NULL). */
q4_status q4_unpack(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                    int64_t n, int64_t k, uint8_t* q_out, float* w_out, void* stream);

/* Quantized matrix-vector product, one activation row (M = 1):
 *   y[r] = sum_k w_hat[r][k] * x[k]   for r in [0, n)
 * computed per group as s'*(sum q*x) + b'*(sum x) with fp32 accumulation.
 *   x : bf16 [k] (uint16 bit patterns), y : [n] of y_dtype. */
q4_status q4_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                  const uint16_t* biases, int64_t n, int64_t k, void* y, q4_out_dtype y_dtype,
                  void* stream);

/* Small quantized GEMM for M concurrent activation rows (1 <= m <= 16), all
 * sharing one pass over the weights:
 *   y[i][r] = sum_k w_hat[r][k] * x[i][k]
 *   x : bf16 [m][k] row-major, y : [m][n] row-major of y_dtype.
 * m == 1 is the same computation as q4_gemv. Supports k <= Q4_MAX_K. */
q4_status q4_gemm_small(const uint16_t* x, int64_t m, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                        void* y, q4_out_dtype y_dtype, void* stream);

/* Depformer MultiLinear step ("NVIDIA PersonaPlex 7B on Apple Silicon",
 * Depformer section, MultiLinear code figure): the weight holds num_steps
 * blocks of `out` rows ([num_steps*out][k]); step `step` multiplies by rows
 * [step*out, (step+1)*out) of packed, scales and biases together (a pointer
 * offset, no copy), then the same product as q4_gemm_small.
 *   x : bf16 [m][k], y : [m][out]. step must lie in [0, num_steps). */
q4_status q4_multilinear_step(const uint16_t* x, int64_t m, const uint32_t* packed,
                              const uint16_t* scales, const uint16_t* biases, int64_t num_steps,
                              int64_t out, int64_t k, int64_t step, void* y,
                              q4_out_dtype y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Chain executor: an ordered list of GEMV stages run by ONE persistent launch.
 *
 * The per-frame temporal step is such a chain ("NVIDIA PersonaPlex 7B on Apple
 * Silicon", pipeline diagram: 32 layers of width 4096; the layers reuse KV
 * cache, RoPE, SwiGLU and RMSNorm parts per the GeekNews summary's audio
 * pipeline section). Read as a standard decoder layer, the attention input
 * feeds q, k, v, the attention output feeds o, the FFN input feeds gate and
 * up, and the gated product feeds down. A stage is one activation vector x
 * (bf16 [k]) multiplied by one or more matrices that share it:
 *   y_i[r] = sum_k w_hat_i[r][k] * x[k]   for every matrix i of the stage.
 * Stages run in order: no product of stage s+1 starts before every output of
 * stage s is written and visible, so a stage's x may be (the bf16 output of)
 * an earlier stage. Weight bytes of later stages are fetched ahead of that
 * point (weights never depend on activations).
 *
 * Use: describe the chain with host arrays, q4_chain_encode() it into a host
 * buffer of q4_chain_plan_bytes(), copy that buffer to device memory
 * (64-byte aligned), then call q4_chain_run() as often as needed. The plan
 * holds the device pointers given at encode time; it stays valid while those
 * buffers live. Each stage's k must satisfy the q4_gemv limits; every
 * stage needs >= 1 matrix, all of that stage's k. Limits of the executor
 * (Q4_ERR_UNSUPPORTED from q4_chain_encode otherwise): at most 384 stages and
 * 768 matrices per chain (the block copies the plan into LDS), at most 4
 * matrices per stage, k <= 12288, n < 2^22, at most 128
 * units of 4 rows of one matrix per block (n <= 512 x the number of compute
 * units), scales and biases 16-byte aligned, and no stage's output may
 * overlap its own input.
 *
 * Workspace: Q4_CHAIN_WORKSPACE_BYTES of device memory, 128-byte aligned,
 * zero-filled once by the caller before its first use; the executor leaves it
 * ready for the next call. Calls sharing one workspace must not overlap in
 * time (use one workspace per stream). Word 0 of the workspace is a status:
 * 0 = ok, 1 = a wait timed out (the launch ended early, outputs undefined),
 * 2 = the plan buffer is not a valid plan, 3 = a block did not run on the XCD
 * the launch order implies (the barrier's per-XCD counters need it). A
 * nonzero status stays set until the caller clears the workspace again.
 */
#define Q4_CHAIN_WORKSPACE_BYTES 131328 /* 256 + 128 per block, up to 1024 blocks */

typedef struct q4_chain_matrix {
  const uint32_t* packed; /* [n][k/8]  */
  const uint16_t* scales; /* [n][k/32] */
  const uint16_t* biases; /* [n][k/32] */
  void* y;                /* [n] of the chain's output dtype */
  int64_t n;
} q4_chain_matrix;

typedef struct q4_chain_stage {
  const uint16_t* x;      /* bf16 [k], 16-byte aligned */
  int64_t k;
  int32_t first_matrix;   /* index into the matrix array */
  int32_t num_matrices;
} q4_chain_stage;

/* Bytes of the plan buffer for a chain of this size (< 0 on invalid counts). */
int64_t q4_chain_plan_bytes(int32_t num_stages, int32_t num_matrices);

/* Validate the chain (same pointer/shape/alignment rules as q4_gemv for every
 * matrix) and write the plan into host_plan (plan_bytes long). Reads the
 * device's compute-unit count (each block stages its share of a matrix's
 * rows); launches nothing. */
q4_status q4_chain_encode(const q4_chain_stage* stages, int32_t num_stages,
                          const q4_chain_matrix* matrices, int32_t num_matrices,
                          q4_out_dtype y_dtype, void* host_plan, int64_t plan_bytes);

/* Run an encoded chain (device copy of the plan) on `stream`: one launch of one
 * 960-thread block per compute unit, all resident at once (the stage
 * barrier needs that; Q4_ERR_UNSUPPORTED if the kernel cannot fit one block
 * per compute unit or the device has more than 1024 of them). y_dtype must
 * match the dtype the plan was encoded with. Nothing else should occupy the
 * device's compute units during the call: a block that cannot start makes
 * the others' bounded waits expire (status 1) instead of hanging. */
q4_status q4_chain_run(const void* device_plan, q4_out_dtype y_dtype, void* workspace,
                       void* stream);

/* The same chain with m_rows (1..4) activation rows sharing every weight
 * stream: concurrent conversations ("A smaller voice model", Concurrency
 * section: several conversations read one copy of the weights). Each stage's
 * x is bf16 [m_rows][k] and each matrix's y is [m_rows][n] (row-major,
 * contiguous); every row r is the product of that matrix with x row r.
 * m_rows == 1 is q4_chain_encode. With 2..4 rows the executor keeps one
 * activation buffer per block (the next stage's rows are fetched during the
 * stage barrier), which lowers its limits: at most 128 stages, 256 matrices,
 * k <= 11264 and 32 units of 4 rows of one matrix per block
 * (Q4_ERR_UNSUPPORTED otherwise); Q4_ERR_SHAPE if m_rows is out of range. */
q4_status q4_chain_encode_rows(const q4_chain_stage* stages, int32_t num_stages,
                               const q4_chain_matrix* matrices, int32_t num_matrices, int32_t m_rows,
                               q4_out_dtype y_dtype, void* host_plan, int64_t plan_bytes);

/* Run a plan encoded by q4_chain_encode_rows with the same m_rows (a plan
 * encoded for another row count makes the kernel report status 2). */
q4_status q4_chain_run_rows(const void* device_plan, int32_t m_rows, q4_out_dtype y_dtype,
                            void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
