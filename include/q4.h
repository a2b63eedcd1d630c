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
#define Q4_MAX_M 64
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

/* Unpack ("personaplex-edge-q4" model card, Release details table: each
 * weight is a 4-bit code with the bf16 scale and bias of its group of 32):
 * recover codes and/or dequantized weights w_hat = s'*q + b' (one rounding to
 * fp32; the product s'*q is exact). Bit-exact with the oracle.
 *   q_out : uint8 [n][k] or NULL;  w_out : fp32 [n][k] or NULL (at least one
 *   must be non-NULL). */
q4_status q4_unpack(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                    int64_t n, int64_t k, uint8_t* q_out, float* w_out, void* stream);

/* Quantized matrix-vector product, one activation row (M = 1): the decoding
 * step's linear layer run straight from the packed weights ("personaplex-
 * edge-q4" model card, introduction: weights stay packed and feed a quantized
 * matmul; "NVIDIA PersonaPlex 7B on Apple Silicon", Depformer MultiLinear
 * code figure: the product takes x, the packed weight, scales and biases,
 * with the weight transposed):
 *   y[r] = sum_k w_hat[r][k] * x[k]   for r in [0, n)
 * computed per group as s'*(sum q*x) + b'*(sum x) with fp32 accumulation.
 *   x : bf16 [k] (uint16 bit patterns), y : [n] of y_dtype. */
q4_status q4_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                  const uint16_t* biases, int64_t n, int64_t k, void* y, q4_out_dtype y_dtype,
                  void* stream);

/* Small quantized GEMM for M activation rows (1 <= m <= Q4_MAX_M = 64), all
 * sharing one pass over the weights: concurrent conversations ("A smaller
 * voice model", Concurrency section: several conversations served together
 * read one copy of the weights, so their frames cost little more than one)
 * and, for 17..64 rows, prefill ("NVIDIA PersonaPlex 7B on Apple Silicon",
 * optimisation list: the 50-frame voice prompt runs as one batched forward
 * pass instead of single steps):
 *   y[i][r] = sum_k w_hat[r][k] * x[i][k]
 *   x : bf16 [m][k] row-major, y : [m][n] row-major of y_dtype.
 * m == 1 is the same computation as q4_gemv. Supports k <= Q4_MAX_K. */
q4_status q4_gemm_small(const uint16_t* x, int64_t m, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                        void* y, q4_out_dtype y_dtype, void* stream);

/* A batch of independent q4_gemm_small products that share m (5..16 rows) and
 * k, run in one launch: the concurrent conversations of q4_gemm_small ("A
 * smaller voice model", Concurrency section) over many weight matrices, such
 * as every matrix of a decoder step, without one launch per matrix. Product i
 * is y_i = x_i w_hat_i^T exactly as q4_gemm_small computes it (same kernel
 * body and rounding), for item i's x ([m][k] bf16), packed, scales, biases,
 * y ([m][n] of y_dtype) and n >= 1.
 *
 * Use: q4_gemm_batch_encode() the items into a host buffer (2-byte aligned,
 * as any allocated or array buffer is) of q4_gemm_batch_plan_bytes() (it
 * needs the number of row blocks, sum of ceil(n_i / 16), as `blocks`;
 * q4_gemm_batch_blocks() returns it), copy the buffer to device memory
 * (16-byte aligned), then call q4_gemm_batch_run() with both copies as often
 * as needed. The plan holds the device pointers given at encode time and
 * stays valid while those buffers live; the two copies must hold the same
 * bytes. Limits: 1..4096 items (Q4_ERR_SHAPE), at most 2^24 blocks in total
 * and k <= Q4_MAX_K (Q4_ERR_UNSUPPORTED); Q4_ERR_SHAPE also for m outside
 * 5..16 or a plan buffer too small. Outputs may not overlap each other or any
 * input (not checked). Items are not ordered: the products run concurrently. */
typedef struct q4_gemm_batch_item {
  const uint16_t* x;      /* bf16 [m][k], 16-byte aligned */
  const uint32_t* packed; /* [n][k/8]  */
  const uint16_t* scales; /* [n][k/32] */
  const uint16_t* biases; /* [n][k/32] */
  void* y;                /* [m][n] of the batch's output dtype */
  int64_t n;
} q4_gemm_batch_item;

/* Blocks of 16 weight rows over the items (< 0 if items is NULL, count is
 * outside 1..4096 or an n is outside 1..2^30). */
int64_t q4_gemm_batch_blocks(const q4_gemm_batch_item* items, int32_t count);
/* Bytes of the plan buffer for `count` items and `blocks` row blocks (< 0
 * outside the limits above). */
int64_t q4_gemm_batch_plan_bytes(int32_t count, int64_t blocks);
/* Validate every item (q4_gemm_small's pointer and shape rules) and write the
 * plan into host_plan (plan_bytes long). Launches nothing. */
q4_status q4_gemm_batch_encode(const q4_gemm_batch_item* items, int32_t count, int64_t m, int64_t k,
                               q4_out_dtype y_dtype, void* host_plan, int64_t plan_bytes);
/* Run the batch on `stream` (one launch); host_plan is read for the launch
 * shape, device_plan by the kernel. Q4_ERR_SHAPE if host_plan is not an
 * encoded plan, Q4_ERR_ALIGN if device_plan is not 16-byte aligned. */
q4_status q4_gemm_batch_run(const void* host_plan, const void* device_plan, void* stream);

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

/* Packed-embedding gather and stream sum: the step's input vector is the sum
 * of one embedding row per token stream ("NVIDIA PersonaPlex 7B on Apple
 * Silicon", pipeline figure: 17 streams, text + 8 user + 8 assistant audio
 * codebooks, summed into the temporal transformer; "personaplex-edge-q4"
 * model card, introduction: the embeddings stay packed). Each stream t has
 * its own table of `rows` rows of `dim` values in the stored layout above
 * (rows x dim/2 bytes must stay below 2^31). For frame f:
 *   y[f][d] = sum over t of w_hat_t[tokens[f][t]][d]
 * with the dequantized values added in stream order in fp32 and rounded once
 * if y is bf16. A token outside [0, rows_t) (a stream with no token this
 * frame) adds nothing; the device reads no memory for it.
 *   tokens : DEVICE int32 [frames][num_tables]
 *   tables : HOST array of num_tables descriptors (1..Q4_EMBED_MAX_TABLES);
 *            their pointers are device pointers (packed 16-byte aligned)
 *   y      : DEVICE [frames][dim] of y_dtype, 16-byte aligned
 * dim must be a positive multiple of 32. frames == 0 launches nothing. */
#define Q4_EMBED_MAX_TABLES 32
typedef struct q4_embed_table {
  const uint32_t* packed; /* [rows][dim/8] */
  const uint16_t* scales; /* [rows][dim/32] */
  const uint16_t* biases; /* [rows][dim/32] */
  int64_t rows;
} q4_embed_table;

q4_status q4_embed_sum(const int32_t* tokens, int64_t frames, const q4_embed_table* tables, int32_t num_tables,
                       int64_t dim, void* y, q4_out_dtype y_dtype, void* stream);

/* Decode attention for one layer: the step's one query per head attends over
 * the layer's KV cache. The step's q, k and v (bf16 [heads][head_dim]) come
 * from the layer's projections; q and k are turned by the rotary embedding
 * at position pos (the RoPE offset is a step input: "NVIDIA PersonaPlex 7B on
 * Apple Silicon", optimisation list), k and v are written to the caches at
 * pos (the ONNX bundle's README, How to use: the step carries the K and V
 * caches [layers][1][32][T][128] explicitly), then for each head
 *   out_h = softmax_t(q_h . k_h[t] / sqrt(head_dim)) . v_h[t],  t = 0..pos.
 * The rotary embedding turns each pair (x[2i], x[2i+1]) of a head by the
 * angle pos * rope_theta^(-2i/head_dim), computed in fp64 and rounded to fp32
 * and then to bf16 (the rotated q and k are bf16, like every activation).
 *   q, k_new, v_new : DEVICE bf16 [heads][head_dim] (q 16-byte aligned)
 *   k_cache, v_cache: DEVICE bf16 [heads][cap][head_dim], 16-byte aligned;
 *                     row pos is written, rows 0..pos-1 are read
 *   out             : DEVICE [heads][head_dim] of out_dtype
 *   workspace       : DEVICE, 256-byte aligned, >= q4_attn_workspace_bytes()
 *                     bytes, owned by the caller, zero-filled once before its
 *                     first use (the heads' split counters, which every call
 *                     leaves at zero; then the rotated q, bf16 [heads][D],
 *                     and the splits' partial results); calls sharing one
 *                     workspace must not overlap in time
 * head_dim must be 64 or 128 (Q4_ERR_UNSUPPORTED otherwise); 0 <= pos < cap.
 * One launch on `stream` (blocks of a head split the positions; the head's
 * last block to finish adds the splits up); no allocation. */
int64_t q4_attn_workspace_bytes(int64_t heads, int64_t head_dim);
q4_status q4_attn_decode(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache,
                         uint16_t* v_cache, int64_t heads, int64_t head_dim, int64_t cap, int64_t pos,
                         double rope_theta, void* out, q4_out_dtype out_dtype, void* workspace,
                         int64_t workspace_bytes, void* stream);

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
 * Stages run in order as far as memory can tell: a stage that reads what an
 * earlier stage writes (its x, a residual), or writes what an earlier stage
 * reads or writes, starts only after that stage's outputs are written and
 * visible everywhere (a grid barrier, placed by the encoder), so a stage's x
 * may be (the bf16 output of) an earlier stage. Stages with no such
 * dependency run without a barrier between them: each block goes on to its
 * share of the next stage as soon as it has finished its share of the last.
 * Weight bytes of later stages are fetched ahead of either point (weights
 * never depend on activations).
 *
 * Use: describe the chain with host arrays, q4_chain_encode() it into a host
 * buffer of q4_chain_plan_bytes(), copy that buffer to device memory
 * (64-byte aligned), then call q4_chain_run() as often as needed. The plan
 * holds the device pointers given at encode time; it stays valid while those
 * buffers live. Each stage's k must satisfy the q4_gemv limits; every
 * stage needs >= 1 matrix, all of that stage's k. Limits of the executor
 * (Q4_ERR_UNSUPPORTED from q4_chain_encode otherwise): at most 384 stages and
 * 768 matrices per chain (the block copies the plan into LDS), at most 4
 * matrices per stage, k <= 12288, n < 2^22, at most 32
 * units of 4 rows of one matrix per block (n <= 128 x the number of compute
 * units), scales and biases 16-byte aligned, no stage's output may overlap
 * its own input, and no two outputs of one stage may overlap. Outputs of
 * different stages may overlap: the later stage's values are the ones left
 * (the encoder makes the earlier stage's stores complete before its barrier,
 * as it does for outputs a later stage reads).
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

/* The chain with the parts of a decoder layer fused around its products
 * (RMSNorm, the SwiGLU gate and the residual sum are reused parts of the
 * model: GeekNews summary, audio pipeline; "NVIDIA PersonaPlex 7B on Apple
 * Silicon", Mimi reuse section). Each is optional per stage or matrix:
 *  - norm_weight (bf16 [k], may be NULL): the stage's x is replaced by its
 *    RMSNorm before the products: inv = 1/sqrt(sum x^2 / k + norm_eps),
 *    x_j -> bf16((x_j * norm_weight_j) * inv), the product exact, the sum of
 *    squares and the scaling in fp64 (one activation row only: m_rows == 1);
 *  - gated (0 or 1): a stage of exactly two matrices of equal n (gate, up);
 *    its output is silu(gate) * up, silu(t) = t / (1 + exp(-t)), computed in
 *    fp32 from the two fp32 products and written to matrix 0's y (matrix 1's
 *    y is not written and may be NULL);
 *  - residual (per matrix, may be NULL): [m_rows][n] of the chain's output
 *    dtype, added to the matrix's product (after the gate, on a gated stage's
 *    matrix 0) before its one rounding; it may be y itself (in place) and may
 *    be written by an earlier stage of the chain.
 * Every other rule is q4_chain_encode_rows's; in addition a norm weight may
 * not overlap any stage's output, a residual may not overlap another output
 * of its own stage, and a gated stage's matrix 1 takes no residual. */
typedef struct q4_chain_stage_ex {
  const uint16_t* x;           /* bf16 [m_rows][k], 16-byte aligned */
  int64_t k;
  int32_t first_matrix;
  int32_t num_matrices;
  const uint16_t* norm_weight; /* bf16 [k] or NULL, 16-byte aligned */
  double norm_eps;
  int32_t gated;
  int32_t reserved;            /* 0 */
} q4_chain_stage_ex;

typedef struct q4_chain_matrix_ex {
  const uint32_t* packed;
  const uint16_t* scales;
  const uint16_t* biases;
  void* y;
  int64_t n;
  const void* residual;        /* [m_rows][n] of the output dtype, or NULL */
} q4_chain_matrix_ex;

q4_status q4_chain_encode_ex(const q4_chain_stage_ex* stages, int32_t num_stages,
                             const q4_chain_matrix_ex* matrices, int32_t num_matrices, int32_t m_rows,
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
 * stage barrier), which lowers its limits: at most 128 stages, 256 matrices
 * and k <= 11264 (Q4_ERR_UNSUPPORTED otherwise); Q4_ERR_SHAPE if m_rows is out of range. */
q4_status q4_chain_encode_rows(const q4_chain_stage* stages, int32_t num_stages,
                               const q4_chain_matrix* matrices, int32_t num_matrices, int32_t m_rows,
                               q4_out_dtype y_dtype, void* host_plan, int64_t plan_bytes);

/* Run a plan encoded by q4_chain_encode_rows with the same m_rows (a plan
 * encoded for another row count makes the kernel report status 2). */
q4_status q4_chain_run_rows(const void* device_plan, int32_t m_rows, q4_out_dtype y_dtype,
                            void* workspace, void* stream);

/* q4_chain_run_rows without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It performs no allocation at all: the
 * executor's workspace words live in a device-global array of the library
 * (Q4_CHAIN_STATIC_SCRATCH_BYTES per device, held until the process ends;
 * enough for devices of up to 16 XCDs, Q4_ERR_UNSUPPORTED beyond). Every call
 * clears those words, runs the chain, and, if status_out (device uint32, may
 * be NULL) is given, writes the launch's status word there (the values of the
 * workspace status word described above). All calls on one device share the
 * one array: calls that overlap in time on one device race and give undefined
 * results, and must be serialised by the caller (e.g. one stream). Same
 * arguments otherwise as q4_chain_run_rows; the regular entry points are
 * unchanged. */
#define Q4_CHAIN_STATIC_SCRATCH_BYTES 4608
q4_status q4_chain_run_rows_noalloc(const void* device_plan, int32_t m_rows, q4_out_dtype y_dtype,
                                    uint32_t* status_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
