// C ABI of libq4 (declared in include/q4.h): argument validation, launch
// configuration and kernel launches. No allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4.h"
#include "q4_kernels.h"
#include "q4_chain.h"

namespace {

thread_local int g_last_hip_error = 0;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline q4_status launch_status() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return Q4_ERR_HIP;
  }
  return Q4_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kNumCU = 256;

int grid_for_groups(int64_t n_groups) {
  const int64_t blocks = ceil_div(n_groups, 256);
  return static_cast<int>(blocks < 8 * kNumCU * 4 ? (blocks < 1 ? 1 : blocks) : 8 * kNumCU * 4);
}

// ---- GEMV launch: pick the lane split C so that S = ceil(G/C) waves cover
// the input groups with the least idle lanes (ties: wider rows per load).
struct GemvPlan {
  int c;
  int waves;
  int rows_per_block;
  int blocks;
};

// weight rows each lane keeps in flight: 8 for one activation row; 2 when
// up to 4 activation rows hold their slices in registers too
constexpr int gemv_u(int mv) { return mv == 1 ? 8 : 2; }

bool plan_gemv(int64_t n, int64_t G, int mv, GemvPlan* p) {
  int best_c = 0, best_s = 0;
  int64_t best_waste = -1;
  const int cs[4] = {64, 32, 16, 8};
  for (int i = 0; i < 4; ++i) {
    const int c = cs[i];
    const int64_t s = ceil_div(G, c);
    if (s > 16) continue;
    const int64_t waste = s * c - G;
    if (best_waste < 0 || waste < best_waste) {
      best_waste = waste;
      best_c = c;
      best_s = static_cast<int>(s);
    }
  }
  if (best_waste < 0) return false;
  const int rows_iter = (64 / best_c) * gemv_u(mv);
  // Aim for >= 2 blocks per CU; each block covers at least one iteration.
  const int64_t target_blocks = 2 * kNumCU;
  int64_t rpb = ceil_div(n, target_blocks);
  rpb = ceil_div(rpb, rows_iter) * rows_iter;
  if (rpb < rows_iter) rpb = rows_iter;
  // a block's rows are addressed through 32-bit buffer ranges
  const int64_t max_rpb = ((int64_t)INT32_MAX / (G * 16)) / rows_iter * rows_iter;
  if (max_rpb < rows_iter) return false;
  if (rpb > max_rpb) rpb = max_rpb;
  p->c = best_c;
  p->waves = best_s;
  p->rows_per_block = static_cast<int>(rpb);
  p->blocks = static_cast<int>(ceil_div(n, rpb));
  return true;
}

template <int C, int MV>
void launch_gemv_c(const GemvPlan& p, bool f32, const uint16_t* x, int64_t k, const uint32_t* packed,
                   const uint16_t* scales, const uint16_t* biases, int n, int G, void* y,
                   hipStream_t st) {
  const dim3 grid(p.blocks), block(64 * p.waves);
  constexpr int U = gemv_u(MV);
  if (f32)
    hipLaunchKernelGGL((q4k::gemv_kernel<C, U, MV, true>), grid, block, 0, st, x, k, packed, scales,
                       biases, n, G, p.rows_per_block, y, (int64_t)n);
  else
    hipLaunchKernelGGL((q4k::gemv_kernel<C, U, MV, false>), grid, block, 0, st, x, k, packed, scales,
                       biases, n, G, p.rows_per_block, y, (int64_t)n);
}

template <int MV>
q4_status run_gemv_mv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                      const uint16_t* biases, int64_t n, int64_t k, void* y, q4_out_dtype dt,
                      hipStream_t st) {
  const int64_t G = k / 32;
  GemvPlan p;
  if (!plan_gemv(n, G, MV, &p)) return Q4_ERR_UNSUPPORTED;
  const bool f32 = dt == Q4_OUT_F32;
  switch (p.c) {
    case 64: launch_gemv_c<64, MV>(p, f32, x, k, packed, scales, biases, (int)n, (int)G, y, st); break;
    case 32: launch_gemv_c<32, MV>(p, f32, x, k, packed, scales, biases, (int)n, (int)G, y, st); break;
    case 16: launch_gemv_c<16, MV>(p, f32, x, k, packed, scales, biases, (int)n, (int)G, y, st); break;
    default: launch_gemv_c<8, MV>(p, f32, x, k, packed, scales, biases, (int)n, (int)G, y, st); break;
  }
  return launch_status();
}

q4_status run_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                   const uint16_t* biases, int64_t n, int64_t k, void* y, q4_out_dtype dt,
                   hipStream_t st) {
  return run_gemv_mv<1>(x, packed, scales, biases, n, k, y, dt, st);
}

// ---- small GEMM launch (MFMA): S waves of GS groups each, T row tiles of 16.
template <int GS, int T>
void launch_gemm_gs(int waves, bool f32, const uint16_t* x, int m, const uint32_t* packed,
                    const uint16_t* scales, const uint16_t* biases, int n, int G, void* y,
                    hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(ceil_div(n, 16 * T))), block(64 * waves);
  // the waves' partial tiles, then each wave's code staging (2 batches of
  // KB groups x 16 rows per row tile, rows padded by 16 bytes)
  constexpr int KB = q4k::kGemmKB;
  const size_t shmem = static_cast<size_t>(waves) * T * 256 * sizeof(float) +
                       static_cast<size_t>(waves) * 2 * T * 16 * (KB * 4 + 4) * sizeof(uint32_t);
  // (16-byte runs of scales per row when every row's run is 16-byte aligned)
  const bool sb16 = G % 8 == 0 && aligned(scales, 16) && aligned(biases, 16);
  if (f32 && sb16)
    hipLaunchKernelGGL((q4k::gemm_mfma_kernel<GS, T, true, true>), grid, block, shmem, st, x, m, packed,
                       scales, biases, n, G, y);
  else if (f32)
    hipLaunchKernelGGL((q4k::gemm_mfma_kernel<GS, T, true, false>), grid, block, shmem, st, x, m, packed,
                       scales, biases, n, G, y);
  else if (sb16)
    hipLaunchKernelGGL((q4k::gemm_mfma_kernel<GS, T, false, true>), grid, block, shmem, st, x, m, packed,
                       scales, biases, n, G, y);
  else
    hipLaunchKernelGGL((q4k::gemm_mfma_kernel<GS, T, false, false>), grid, block, shmem, st, x, m, packed,
                       scales, biases, n, G, y);
}

// Small GEMM: up to 4 activation rows share one pass of the GEMV kernel
// (each loaded group dequantized once, dotted with every row); more rows go
// to the MFMA kernel, one 16-row tile per group.
q4_status run_gemm_small(const uint16_t* x, int64_t m, const uint32_t* packed,
                         const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                         void* y, q4_out_dtype dt, hipStream_t st) {
  switch (m) {
    case 1: return run_gemv_mv<1>(x, packed, scales, biases, n, k, y, dt, st);
    case 2: return run_gemv_mv<2>(x, packed, scales, biases, n, k, y, dt, st);
    case 3: return run_gemv_mv<3>(x, packed, scales, biases, n, k, y, dt, st);
    case 4: return run_gemv_mv<4>(x, packed, scales, biases, n, k, y, dt, st);
    default: break;
  }
  const int64_t G = k / 32;
  const bool f32 = dt == Q4_OUT_F32;
  constexpr int T = 1;
  // (24 groups per wave would spill registers)
  const int gss[3] = {8, 16, 32};
  for (int i = 0; i < 3; ++i) {
    const int64_t waves = ceil_div(G, gss[i]);
    if (waves > 16) continue;
    switch (gss[i]) {
      case 8: launch_gemm_gs<8, T>((int)waves, f32, x, (int)m, packed, scales, biases, (int)n, (int)G, y, st); break;
      case 16: launch_gemm_gs<16, T>((int)waves, f32, x, (int)m, packed, scales, biases, (int)n, (int)G, y, st); break;
      default: launch_gemm_gs<32, T>((int)waves, f32, x, (int)m, packed, scales, biases, (int)n, (int)G, y, st); break;
    }
    return launch_status();
  }
  return Q4_ERR_UNSUPPORTED;
}

q4_status check_matrix(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                       int64_t n, int64_t k) {
  if (!packed || !scales || !biases) return Q4_ERR_NULL;
  if (n < 0 || k <= 0 || k % 32 != 0 || n > INT32_MAX / 2) return Q4_ERR_SHAPE;
  return Q4_OK;
}

q4_status check_align_matrix(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases) {
  if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(biases, 2)) return Q4_ERR_ALIGN;
  return Q4_OK;
}

q4_status check_product(const uint16_t* x, int64_t m, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                        void* y, q4_out_dtype dt) {
  if (!x || !y) return Q4_ERR_NULL;
  q4_status s = check_matrix(packed, scales, biases, n, k);
  if (s != Q4_OK) return s;
  if (m < 1 || m > Q4_MAX_M) return Q4_ERR_SHAPE;
  if (dt != Q4_OUT_BF16 && dt != Q4_OUT_F32) return Q4_ERR_SHAPE;
  s = check_align_matrix(packed, scales, biases);
  if (s != Q4_OK) return s;
  if (!aligned(x, 16) || !aligned(y, dt == Q4_OUT_F32 ? 4 : 2)) return Q4_ERR_ALIGN;
  if (k > Q4_MAX_K) return Q4_ERR_UNSUPPORTED;
  return Q4_OK;
}

}  // namespace

extern "C" {

int q4_layout_version(void) { return 1; }

const char* q4_status_str(int status) {
  switch (status) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "null pointer";
    case Q4_ERR_SHAPE: return "invalid shape or argument";
    case Q4_ERR_ALIGN: return "misaligned pointer";
    case Q4_ERR_UNSUPPORTED: return "unsupported size";
    case Q4_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int q4_last_hip_error(void) { return g_last_hip_error; }

q4_status q4_pack(const float* w, int64_t n, int64_t k, uint32_t* packed, uint16_t* scales,
                  uint16_t* biases, void* stream) {
  if (!w) return Q4_ERR_NULL;
  q4_status s = check_matrix(packed, scales, biases, n, k);
  if (s != Q4_OK) return s;
  s = check_align_matrix(packed, scales, biases);
  if (s != Q4_OK) return s;
  if (!aligned(w, 16)) return Q4_ERR_ALIGN;
  if (n == 0) return Q4_OK;
  const int64_t ng = n * (k / 32);
  hipLaunchKernelGGL(q4k::pack_kernel, dim3(grid_for_groups(ng)), dim3(256), 0, as_stream(stream), w,
                     ng, packed, scales, biases);
  return launch_status();
}

q4_status q4_unpack(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                    int64_t n, int64_t k, uint8_t* q_out, float* w_out, void* stream) {
  q4_status s = check_matrix(packed, scales, biases, n, k);
  if (s != Q4_OK) return s;
  if (!q_out && !w_out) return Q4_ERR_NULL;
  s = check_align_matrix(packed, scales, biases);
  if (s != Q4_OK) return s;
  if ((q_out && !aligned(q_out, 16)) || (w_out && !aligned(w_out, 16))) return Q4_ERR_ALIGN;
  if (n == 0) return Q4_OK;
  const int64_t ng = n * (k / 32);
  hipLaunchKernelGGL(q4k::unpack_kernel, dim3(grid_for_groups(ng)), dim3(256), 0, as_stream(stream),
                     packed, scales, biases, ng, q_out, w_out);
  return launch_status();
}

q4_status q4_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                  const uint16_t* biases, int64_t n, int64_t k, void* y, q4_out_dtype y_dtype,
                  void* stream) {
  const q4_status s = check_product(x, 1, packed, scales, biases, n, k, y, y_dtype);
  if (s != Q4_OK) return s;
  if (n == 0) return Q4_OK;
  return run_gemv(x, packed, scales, biases, n, k, y, y_dtype, as_stream(stream));
}

q4_status q4_gemm_small(const uint16_t* x, int64_t m, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                        void* y, q4_out_dtype y_dtype, void* stream) {
  const q4_status s = check_product(x, m, packed, scales, biases, n, k, y, y_dtype);
  if (s != Q4_OK) return s;
  if (n == 0) return Q4_OK;
  return run_gemm_small(x, m, packed, scales, biases, n, k, y, y_dtype, as_stream(stream));
}

q4_status q4_multilinear_step(const uint16_t* x, int64_t m, const uint32_t* packed,
                              const uint16_t* scales, const uint16_t* biases, int64_t num_steps,
                              int64_t out, int64_t k, int64_t step, void* y,
                              q4_out_dtype y_dtype, void* stream) {
  if (!x || !y || !packed || !scales || !biases) return Q4_ERR_NULL;
  if (num_steps <= 0 || out < 0 || step < 0 || step >= num_steps) return Q4_ERR_SHAPE;
  if (out > 0 && num_steps > (INT32_MAX / 2) / out) return Q4_ERR_SHAPE;
  const q4_status s = check_product(x, m, packed, scales, biases, out, k, y, y_dtype);
  if (s != Q4_OK) return s;
  if (out == 0) return Q4_OK;
  const int64_t row0 = step * out;
  return run_gemm_small(x, m, packed + row0 * (k / 8), scales + row0 * (k / 32),
                        biases + row0 * (k / 32), out, k, y, y_dtype, as_stream(stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Chain executor host side.
namespace {

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kNumCU;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return kNumCU;
  return cus;
}

// Number of XCDs (chiplets with their own L2) of the current device.
uint32_t device_xcc_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n <= 0) return 1;
  return static_cast<uint32_t>(n);
}

template <int MV>
constexpr size_t chain_lds_bytes() { return sizeof(q4k::ChainLds<MV>); }

// Per device and activation-row count: raise the dynamic-LDS limit of the
// chain kernels once and check that one block fits per compute unit.
template <int MV>
bool chain_ready_rows(int dev) {
  static int state[64] = {0};  // 0 unknown, 1 ready, -1 not possible
  if (dev < 0 || dev >= 64) return false;
  if (state[dev] == 0) {
    constexpr size_t lds = chain_lds_bytes<MV>();
    bool ok = hipFuncSetAttribute(reinterpret_cast<const void*>(&q4k::chain_kernel<MV, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess &&
              hipFuncSetAttribute(reinterpret_cast<const void*>(&q4k::chain_kernel<MV, false>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess;
    int a = 0, b = 0;
    ok = ok &&
         hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, q4k::chain_kernel<MV, true>, 64 * q4k::kChainWaves,
                                                      lds) == hipSuccess &&
         hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, q4k::chain_kernel<MV, false>, 64 * q4k::kChainWaves,
                                                      lds) == hipSuccess &&
         a >= 1 && b >= 1;
    (void)hipGetLastError();
    state[dev] = ok ? 1 : -1;
  }
  return state[dev] == 1;
}

template <int MV>
q4_status launch_chain(const q4k::ChainHeader* plan, q4_out_dtype y_dtype, uint32_t* ws, hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || !chain_ready_rows<MV>(dev)) return Q4_ERR_UNSUPPORTED;
  // One block of 15 waves per compute unit, all resident at once (the stage
  // barrier needs that); bounded waits turn a violation into a status.
  const int cus = device_cu_count();
  if (cus > q4k::kChainMaxBlocks) return Q4_ERR_UNSUPPORTED;
  const uint32_t nxcc = device_xcc_count();
  if (nxcc < 1 || nxcc > q4k::kMaxXcc) return Q4_ERR_UNSUPPORTED;
  const dim3 grid(cus), block(64 * q4k::kChainWaves);
  constexpr size_t lds = chain_lds_bytes<MV>();
  if (y_dtype == Q4_OUT_F32)
    hipLaunchKernelGGL((q4k::chain_kernel<MV, true>), grid, block, lds, st, plan, ws, nxcc);
  else
    hipLaunchKernelGGL((q4k::chain_kernel<MV, false>), grid, block, lds, st, plan, ws, nxcc);
  return launch_status();
}

// Limits of a chain with m activation rows.
struct ChainLimits {
  int tab_stages, tab_mats, stage_units, max_groups;
};
ChainLimits chain_limits(int m) {
  if (m == 1)
    return {q4k::ChainShape<1>::kTabStages, q4k::ChainShape<1>::kTabMats, q4k::ChainShape<1>::kStageUnits,
            q4k::ChainShape<1>::kMaxGroups};
  return {q4k::ChainShape<2>::kTabStages, q4k::ChainShape<2>::kTabMats, q4k::ChainShape<2>::kStageUnits,
          q4k::ChainShape<2>::kMaxGroups};
}
static_assert(q4k::ChainShape<2>::kTabStages == q4k::ChainShape<4>::kTabStages &&
                  q4k::ChainShape<2>::kStageUnits == q4k::ChainShape<4>::kStageUnits &&
                  q4k::ChainShape<2>::kMaxGroups == q4k::ChainShape<4>::kMaxGroups &&
                  q4k::ChainShape<2>::kTabMats == q4k::ChainShape<4>::kTabMats,
              "one set of limits for several activation rows");

// Lanes per row for a stage of G groups: among 64/32/16/8 lanes, the split
// with the fewest idle lanes (ties: more lanes per row) whose padded width
// fits the activation buffer and whose rows per unit (64/lanes) divide every
// matrix's row count.
// A chain stage processes units of 4 rows in chunks of 16 groups per row, so
// its geometry depends on G only: chunks per row CH = ceil(G / 16), with the
// activations padded to 16 * CH groups.
bool plan_stage(int64_t G, int max_groups, int* c_log2, int* CH) {
  const int64_t ch = ceil_div(G, q4k::kChunkGroups);
  if (ch * q4k::kChunkGroups > max_groups) return false;
  *c_log2 = 4;
  *CH = static_cast<int>(ch);
  return true;
}

bool ranges_overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

}  // namespace

extern "C" {

int64_t q4_chain_plan_bytes(int32_t num_stages, int32_t num_matrices) {
  if (num_stages <= 0 || num_matrices <= 0) return -1;
  return static_cast<int64_t>(sizeof(q4k::ChainHeader)) +
         static_cast<int64_t>(num_stages) * sizeof(q4k::ChainStageDesc) +
         static_cast<int64_t>(num_matrices) * sizeof(q4k::ChainMatDesc);
}

q4_status q4_chain_encode_rows(const q4_chain_stage* stages, int32_t num_stages,
                               const q4_chain_matrix* matrices, int32_t num_matrices, int32_t m_rows,
                               q4_out_dtype y_dtype, void* host_plan, int64_t plan_bytes) {
  if (!stages || !matrices || !host_plan) return Q4_ERR_NULL;
  if (num_stages <= 0 || num_matrices <= 0) return Q4_ERR_SHAPE;
  if (m_rows < 1 || m_rows > q4k::kMaxRows) return Q4_ERR_SHAPE;
  const ChainLimits lim = chain_limits(m_rows);
  if (y_dtype != Q4_OUT_BF16 && y_dtype != Q4_OUT_F32) return Q4_ERR_SHAPE;
  const int64_t need = q4_chain_plan_bytes(num_stages, num_matrices);
  if (plan_bytes < need) return Q4_ERR_SHAPE;
  const int64_t ybytes = y_dtype == Q4_OUT_F32 ? 4 : 2;
  int32_t next_matrix = 0;
  for (int32_t s = 0; s < num_stages; ++s) {
    const q4_chain_stage& st = stages[s];
    if (st.num_matrices <= 0 || st.first_matrix != next_matrix ||
        st.first_matrix + (int64_t)st.num_matrices > num_matrices)
      return Q4_ERR_SHAPE;
    next_matrix += st.num_matrices;
    for (int32_t i = 0; i < st.num_matrices; ++i) {
      const q4_chain_matrix& m = matrices[st.first_matrix + i];
      const q4_status c = check_product(st.x, m_rows, m.packed, m.scales, m.biases, m.n, st.k, m.y, y_dtype);
      if (c != Q4_OK) return c;
      if (m.n >= (1 << 22)) return Q4_ERR_UNSUPPORTED;
      // each block stages its rows of a matrix in LDS
      if (ceil_div(ceil_div(m.n, q4k::kUnitRows), device_cu_count()) > lim.stage_units) return Q4_ERR_UNSUPPORTED;
      if (!aligned(m.scales, 16) || !aligned(m.biases, 16)) return Q4_ERR_UNSUPPORTED;
      // a stage may not write its own input
      if (ranges_overlap(st.x, 2 * st.k * m_rows, m.y, ybytes * m.n * m_rows)) return Q4_ERR_UNSUPPORTED;
    }
    int lg, ch;
    if (st.num_matrices > q4k::kMaxMatsPerStage || num_matrices > lim.tab_mats || num_stages > lim.tab_stages ||
        !plan_stage(st.k / 32, lim.max_groups, &lg, &ch))
      return Q4_ERR_UNSUPPORTED;
  }
  if (next_matrix != num_matrices) return Q4_ERR_SHAPE;

  unsigned char* out = static_cast<unsigned char*>(host_plan);
  auto* hdr = reinterpret_cast<q4k::ChainHeader*>(out);
  *hdr = q4k::ChainHeader{};
  hdr->magic = q4k::kChainMagic;
  hdr->num_stages = num_stages;
  hdr->num_mats = num_matrices;
  hdr->out_f32 = y_dtype == Q4_OUT_F32 ? 1 : 0;
  hdr->plan_bytes = static_cast<int32_t>(need);
  hdr->rows = m_rows;
  auto* sd = reinterpret_cast<q4k::ChainStageDesc*>(hdr + 1);
  for (int32_t s = 0; s < num_stages; ++s) {
    const q4_chain_stage& st = stages[s];
    q4k::ChainStageDesc d{};
    d.x = st.x;
    d.G = static_cast<int32_t>(st.k / 32);
    plan_stage(d.G, lim.max_groups, &d.c_log2, &d.CH);
    d.num_mats = st.num_matrices;
    d.mat_begin = st.first_matrix;
    sd[s] = d;
  }
  // Dependencies through memory: a stage whose x overlaps an earlier stage's
  // outputs loads it only after the preceding stage barrier (device-coherent
  // loads), and that earlier stage makes its outputs visible before it
  // arrives at its barrier. Activations no stage writes are prefetched.
  for (int32_t s = 0; s < num_stages; ++s) {
    const q4_chain_stage& st = stages[s];
    for (int32_t t = 0; t < s; ++t) {
      for (int32_t i = 0; i < stages[t].num_matrices; ++i) {
        const q4_chain_matrix& m = matrices[stages[t].first_matrix + i];
        // (a later stage writing x is harmless: x is read before that stage
        // starts, prefetch included)
        if (t < s && ranges_overlap(st.x, 2 * st.k * m_rows, m.y, ybytes * m.n * m_rows)) {
          sd[s].x_internal = 1;
          sd[t].sync_outputs = 1;
        }
      }
    }
  }
  auto* md = reinterpret_cast<q4k::ChainMatDesc*>(sd + num_stages);
  for (int32_t i = 0; i < num_matrices; ++i) {
    q4k::ChainMatDesc d{};
    d.packed = matrices[i].packed;
    d.scales = matrices[i].scales;
    d.biases = matrices[i].biases;
    d.y = matrices[i].y;
    d.n = static_cast<int32_t>(matrices[i].n);
    md[i] = d;
  }
  return Q4_OK;
}

q4_status q4_chain_encode(const q4_chain_stage* stages, int32_t num_stages,
                          const q4_chain_matrix* matrices, int32_t num_matrices,
                          q4_out_dtype y_dtype, void* host_plan, int64_t plan_bytes) {
  return q4_chain_encode_rows(stages, num_stages, matrices, num_matrices, 1, y_dtype, host_plan, plan_bytes);
}

q4_status q4_chain_run_rows(const void* device_plan, int32_t m_rows, q4_out_dtype y_dtype, void* workspace,
                            void* stream) {
  if (!device_plan || !workspace) return Q4_ERR_NULL;
  if (y_dtype != Q4_OUT_BF16 && y_dtype != Q4_OUT_F32) return Q4_ERR_SHAPE;
  if (m_rows < 1 || m_rows > q4k::kMaxRows) return Q4_ERR_SHAPE;
  if (!aligned(device_plan, 64) || !aligned(workspace, 128)) return Q4_ERR_ALIGN;
  const q4k::ChainHeader* plan = static_cast<const q4k::ChainHeader*>(device_plan);
  uint32_t* ws = static_cast<uint32_t*>(workspace);
  switch (m_rows) {
    case 1: return launch_chain<1>(plan, y_dtype, ws, as_stream(stream));
    case 2: return launch_chain<2>(plan, y_dtype, ws, as_stream(stream));
    case 3: return launch_chain<3>(plan, y_dtype, ws, as_stream(stream));
    default: return launch_chain<4>(plan, y_dtype, ws, as_stream(stream));
  }
}

q4_status q4_chain_run(const void* device_plan, q4_out_dtype y_dtype, void* workspace, void* stream) {
  return q4_chain_run_rows(device_plan, 1, y_dtype, workspace, stream);
}

}  // extern "C"
