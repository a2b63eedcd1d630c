// C ABI of libq4 (declared in include/q4.h): argument validation, launch
// configuration and kernel launches. No allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "q4.h"
#include "q4_kernels.h"
#include "q4_chain.h"
#include "q4_attn.h"

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

constexpr int kMaxDevices = 64;
constexpr int kFallbackCU = 256;  // only if the device cannot be queried

// Compute units of the current device, queried once per device (thread-safe).
int device_cu_count() {
  static std::once_flag once[kMaxDevices];
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kFallbackCU;
  }
  std::call_once(once[dev], [dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = kFallbackCU;
    }
    cus[dev].store(n);
  });
  return cus[dev].load();
}

int grid_for_groups(int64_t n_groups) {
  const int64_t blocks = ceil_div(n_groups, 256);
  const int64_t cap = 32 * (int64_t)device_cu_count();
  return static_cast<int>(blocks < cap ? (blocks < 1 ? 1 : blocks) : cap);
}

// ---- GEMV launch: pick the lane split C so that S = ceil(G/C) waves cover
// the input groups with the least idle lanes (ties: wider rows per load).
struct GemvPlan {
  int c;
  int waves;
  int u;  // weight rows each lane keeps in flight
  int rows_per_block;
  int blocks;
};

// A cold GEMV is one memory round trip per block: the launch is fastest when
// every block loads its rows in one go and the blocks are many (measured on a
// 4096x4096 GEMV, graph of launches: 8 rows per lane and 2 blocks per compute
// unit 6.3 us per call, 4 rows and 4 blocks 5.5 us, 2 rows and 8 blocks
// 5.3 us). So with one activation row each lane keeps U = 8, 4 or 2 weight
// rows in flight, the largest that still gives >= 8 blocks per compute unit
// (2 if none does), and a block takes one load per lane and row; with 2..4
// activation rows, whose slices also live in registers, U = 2.
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
  const int rpi = 64 / best_c;  // row slots per wave
  const int64_t cus = device_cu_count();
  int u = 2;
  if (mv == 1) {
    const int cand[3] = {8, 4, 2};
    for (int i = 0; i < 3; ++i) {
      if (ceil_div(n, (int64_t)rpi * cand[i]) >= 8 * cus) {
        u = cand[i];
        break;
      }
    }
  }
  const int64_t rows_iter = (int64_t)rpi * u;
  // a block's rows are addressed through 32-bit buffer ranges
  if (rows_iter * G * 16 > (int64_t)INT32_MAX) return false;
  const int64_t blocks = ceil_div(n, rows_iter);
  if (blocks > (int64_t)INT32_MAX) return false;
  p->c = best_c;
  p->waves = best_s;
  p->u = u;
  p->rows_per_block = static_cast<int>(rows_iter);
  p->blocks = static_cast<int>(blocks);
  return true;
}

template <int C, int U, int MV>
void launch_gemv_cu(const GemvPlan& p, bool f32, const uint16_t* x, int64_t k, const uint32_t* packed,
                    const uint16_t* scales, const uint16_t* biases, int n, int G, void* y, hipStream_t st) {
  const dim3 grid(p.blocks), block(64 * p.waves);
  if (f32)
    hipLaunchKernelGGL((q4k::gemv_kernel<C, U, MV, true>), grid, block, 0, st, x, k, packed, scales,
                       biases, n, G, p.rows_per_block, y, (int64_t)n);
  else
    hipLaunchKernelGGL((q4k::gemv_kernel<C, U, MV, false>), grid, block, 0, st, x, k, packed, scales,
                       biases, n, G, p.rows_per_block, y, (int64_t)n);
}

template <int C, int MV>
void launch_gemv_c(const GemvPlan& p, bool f32, const uint16_t* x, int64_t k, const uint32_t* packed,
                   const uint16_t* scales, const uint16_t* biases, int n, int G, void* y,
                   hipStream_t st) {
  if constexpr (MV == 1) {
    if (p.u == 8) return launch_gemv_cu<C, 8, MV>(p, f32, x, k, packed, scales, biases, n, G, y, st);
    if (p.u == 4) return launch_gemv_cu<C, 4, MV>(p, f32, x, k, packed, scales, biases, n, G, y, st);
  }
  launch_gemv_cu<C, 2, MV>(p, f32, x, k, packed, scales, biases, n, G, y, st);
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

uint32_t device_xcc_count();

// ---- small GEMM launch (MFMA): S waves of GS groups each, T tiles of 16
// weight rows per block. TILED (more than 16 activation rows): every tile of
// 16 rows in the same launch, the tiles of a row block on blocks of one XCD
// (the grid is a whole number of rounds of nxcc row blocks).
template <int T>
constexpr size_t gemm_shmem(int waves) {
  // the waves' partial tiles, then each wave's code staging (2 batches of
  // KB groups x 16 rows per weight tile, rows padded by 16 bytes)
  return static_cast<size_t>(waves) * T * 256 * sizeof(float) +
         static_cast<size_t>(waves) * 2 * T * 16 * (q4k::kGemmKB * 4 + 4) * sizeof(uint32_t);
}
template <int GS, int T, bool TILED>
void launch_gemm_gs(int waves, bool f32, bool sb16, const uint16_t* x, int m, const uint32_t* packed,
                    const uint16_t* scales, const uint16_t* biases, int n, int G, void* y,
                    hipStream_t st) {
  const int mtiles = TILED ? static_cast<int>(ceil_div(m, 16)) : 1;
  // (one XCD if the device cannot be queried: the mapping stays a permutation)
  const int nxcc = TILED ? std::max(1, static_cast<int>(device_xcc_count())) : 1;
  const int64_t nb = ceil_div(n, 16 * T);
  const int64_t blocks = TILED ? ceil_div(nb, nxcc) * nxcc * mtiles : nb;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * waves);
  const size_t shmem = gemm_shmem<T>(waves);
#define Q4_GEMM_LAUNCH(F, S)                                                                                  \
  hipLaunchKernelGGL((q4k::gemm_mfma_kernel<GS, T, F, S, TILED>), grid, block, shmem, st, x, m, packed, scales, \
                     biases, n, G, y, mtiles, nxcc)
  if (f32 && sb16) {
    Q4_GEMM_LAUNCH(true, true);
  } else if (sb16) {
    Q4_GEMM_LAUNCH(false, true);
  } else if constexpr (T == 1) {
    // (two weight tiles per block are only built with 16-byte scale runs:
    // without them the kernel spills)
    if (f32)
      Q4_GEMM_LAUNCH(true, false);
    else
      Q4_GEMM_LAUNCH(false, false);
  }
#undef Q4_GEMM_LAUNCH
}

// Two weight tiles per block (the prefill) take more than the default 64 KB of
// dynamic LDS: raise the limit of those kernels once per device (thread-safe;
// the answer is kept). Without it the prefill runs one tile per block.
template <int GS>
bool prefill_two_tiles_ready() {
  static std::once_flag once[kMaxDevices];
  static std::atomic<bool> ready[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::call_once(once[dev], [dev]() {
    const int lds = static_cast<int>(gemm_shmem<2>(16));
    const bool ok = hipFuncSetAttribute(reinterpret_cast<const void*>(&q4k::gemm_mfma_kernel<GS, 2, true, true, true>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess &&
                    hipFuncSetAttribute(reinterpret_cast<const void*>(&q4k::gemm_mfma_kernel<GS, 2, false, true, true>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
    (void)hipGetLastError();
    ready[dev].store(ok);
  });
  return ready[dev].load();
}

template <int GS>
void launch_gemm(int waves, bool f32, const uint16_t* x, int m, const uint32_t* packed, const uint16_t* scales,
                 const uint16_t* biases, int n, int G, void* y, hipStream_t st) {
  // (16-byte runs of scales per row when every row's run is 16-byte aligned)
  const bool sb16 = G % 8 == 0 && aligned(scales, 16) && aligned(biases, 16);
  if (m <= 16)
    launch_gemm_gs<GS, 1, false>(waves, f32, sb16, x, m, packed, scales, biases, n, G, y, st);
  else if (sb16 && prefill_two_tiles_ready<GS>())
    launch_gemm_gs<GS, 2, true>(waves, f32, sb16, x, m, packed, scales, biases, n, G, y, st);
  else
    launch_gemm_gs<GS, 1, true>(waves, f32, sb16, x, m, packed, scales, biases, n, G, y, st);
}

// Small GEMM: up to 4 activation rows share one pass of the GEMV kernel
// (each loaded group dequantized once, dotted with every row); 5..16 rows go
// to the MFMA kernel, one 16-row tile per group. More rows (prefill, up to
// 64) run the MFMA kernel on every 16-row tile of x in one launch, the tiles
// of a row block on one XCD, where a weight line the first of them reads from
// HBM can serve the others from the XCD's L2; a block then holds two tiles of
// 16 weight rows, so that each activation load serves twice the weights
// (M=50 step 6.20 -> 5.19 ms).
// Groups per wave of the MFMA kernel for a product with G groups: 16 where
// that still makes 8..16 waves, since two such blocks fit a compute unit
// (measured on the step's matrices, k = 4096: M=50 step 5.19 -> 4.76 ms, M=8
// 0.7% faster, M=16 unchanged); otherwise the first of 8, 16 and 32 that
// needs at most 16 waves (24 groups per wave would spill registers). False if
// none does.
bool gemm_plan(int64_t G, int& gs, int& waves) {
  const int64_t w16 = ceil_div(G, 16);
  if (w16 >= 8 && w16 <= 16) {
    gs = 16, waves = static_cast<int>(w16);
    return true;
  }
  for (const int g : {8, 16, 32}) {
    const int64_t w = ceil_div(G, g);
    if (w <= 16) {
      gs = g, waves = static_cast<int>(w);
      return true;
    }
  }
  return false;
}

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
  int gs = 0, waves = 0;
  if (!gemm_plan(G, gs, waves)) return Q4_ERR_UNSUPPORTED;
  switch (gs) {
    case 8: launch_gemm<8>(waves, f32, x, (int)m, packed, scales, biases, (int)n, (int)G, y, st); break;
    case 16: launch_gemm<16>(waves, f32, x, (int)m, packed, scales, biases, (int)n, (int)G, y, st); break;
    default: launch_gemm<32>(waves, f32, x, (int)m, packed, scales, biases, (int)n, (int)G, y, st); break;
  }
  return launch_status();
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

// Plan of a product batch: this header, the items (q4k::GemmBatchItem), then
// each block's item index (uint16).
struct GemmBatchHeader {
  uint32_t magic;
  int32_t count, m, G, blocks, dtype, gs, waves, sb16;
  int32_t reserved[7];
};
static_assert(sizeof(GemmBatchHeader) == 64, "the plan's header layout");
constexpr uint32_t kBatchMagic = 0x51344742u;
constexpr int32_t kBatchMaxItems = 4096;
constexpr int64_t kBatchMaxBlocks = int64_t(1) << 24;
constexpr int64_t batch_owner_offset(int64_t count) {
  return static_cast<int64_t>(sizeof(GemmBatchHeader)) + count * static_cast<int64_t>(sizeof(q4k::GemmBatchItem));
}

template <int GS>
void launch_batch(const GemmBatchHeader& h, const void* device_plan, hipStream_t st) {
  const char* base = static_cast<const char*>(device_plan);
  const auto* items = reinterpret_cast<const q4k::GemmBatchItem*>(base + sizeof(GemmBatchHeader));
  const auto* owner = reinterpret_cast<const uint16_t*>(base + batch_owner_offset(h.count));
  const dim3 grid(static_cast<unsigned>(h.blocks)), block(64 * h.waves);
  const size_t shmem = gemm_shmem<1>(h.waves);
#define Q4_BATCH_LAUNCH(F, S) \
  hipLaunchKernelGGL((q4k::gemm_batch_kernel<GS, F, S>), grid, block, shmem, st, items, owner, h.m, h.G)
  const bool f32 = h.dtype == Q4_OUT_F32;
  if (h.sb16) {
    if (f32)
      Q4_BATCH_LAUNCH(true, true);
    else
      Q4_BATCH_LAUNCH(false, true);
  } else {
    if (f32)
      Q4_BATCH_LAUNCH(true, false);
    else
      Q4_BATCH_LAUNCH(false, false);
  }
#undef Q4_BATCH_LAUNCH
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

int64_t q4_gemm_batch_blocks(const q4_gemm_batch_item* items, int32_t count) {
  if (!items || count < 1 || count > kBatchMaxItems) return -1;
  int64_t blocks = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (items[i].n < 1 || items[i].n > (int64_t(1) << 30)) return -1;
    blocks += ceil_div(items[i].n, 16);
  }
  return blocks;
}

int64_t q4_gemm_batch_plan_bytes(int32_t count, int64_t blocks) {
  if (count < 1 || count > kBatchMaxItems || blocks < 1 || blocks > kBatchMaxBlocks) return -1;
  return ceil_div(batch_owner_offset(count) + 2 * blocks, 16) * 16;
}

q4_status q4_gemm_batch_encode(const q4_gemm_batch_item* items, int32_t count, int64_t m, int64_t k,
                               q4_out_dtype y_dtype, void* host_plan, int64_t plan_bytes) {
  if (!items || !host_plan) return Q4_ERR_NULL;
  if (count < 1 || count > kBatchMaxItems || m < 5 || m > 16) return Q4_ERR_SHAPE;
  bool sb16 = k % 256 == 0;
  for (int32_t i = 0; i < count; ++i) {
    const q4_gemm_batch_item& it = items[i];
    if (it.n < 1 || it.n > (int64_t(1) << 30)) return Q4_ERR_SHAPE;
    const q4_status s = check_product(it.x, m, it.packed, it.scales, it.biases, it.n, k, it.y, y_dtype);
    if (s != Q4_OK) return s;
    sb16 = sb16 && aligned(it.scales, 16) && aligned(it.biases, 16);
  }
  const int64_t blocks = q4_gemm_batch_blocks(items, count);
  if (blocks > kBatchMaxBlocks) return Q4_ERR_UNSUPPORTED;
  if (blocks < 1 || plan_bytes < q4_gemm_batch_plan_bytes(count, blocks)) return Q4_ERR_SHAPE;
  int gs = 0, waves = 0;
  if (!gemm_plan(k / 32, gs, waves)) return Q4_ERR_UNSUPPORTED;

  char* base = static_cast<char*>(host_plan);
  GemmBatchHeader h{};
  h.magic = kBatchMagic;
  h.count = count, h.m = static_cast<int32_t>(m), h.G = static_cast<int32_t>(k / 32);
  h.blocks = static_cast<int32_t>(blocks), h.dtype = static_cast<int32_t>(y_dtype);
  h.gs = gs, h.waves = waves, h.sb16 = sb16 ? 1 : 0;
  std::memcpy(base, &h, sizeof h);
  uint16_t* owner = reinterpret_cast<uint16_t*>(base + batch_owner_offset(count));
  int32_t start = 0;
  for (int32_t i = 0; i < count; ++i) {
    const q4_gemm_batch_item& it = items[i];
    q4k::GemmBatchItem d{it.x, it.packed, it.scales, it.biases, it.y, static_cast<int32_t>(it.n), start};
    std::memcpy(base + sizeof(GemmBatchHeader) + i * sizeof(q4k::GemmBatchItem), &d, sizeof d);
    const int32_t nb = static_cast<int32_t>(ceil_div(it.n, 16));
    for (int32_t b = 0; b < nb; ++b) owner[start + b] = static_cast<uint16_t>(i);
    start += nb;
  }
  return Q4_OK;
}

q4_status q4_gemm_batch_run(const void* host_plan, const void* device_plan, void* stream) {
  if (!host_plan || !device_plan) return Q4_ERR_NULL;
  GemmBatchHeader h;
  std::memcpy(&h, host_plan, sizeof h);
  if (h.magic != kBatchMagic || h.count < 1 || h.count > kBatchMaxItems || h.blocks < 1 ||
      h.blocks > kBatchMaxBlocks || h.m < 5 || h.m > 16 || h.waves < 1 || h.waves > 16 ||
      (h.gs != 8 && h.gs != 16 && h.gs != 32) || (h.dtype != Q4_OUT_BF16 && h.dtype != Q4_OUT_F32))
    return Q4_ERR_SHAPE;
  if (!aligned(device_plan, 16)) return Q4_ERR_ALIGN;
  const hipStream_t st = as_stream(stream);
  switch (h.gs) {
    case 8: launch_batch<8>(h, device_plan, st); break;
    case 16: launch_batch<16>(h, device_plan, st); break;
    default: launch_batch<32>(h, device_plan, st); break;
  }
  return launch_status();
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

q4_status q4_embed_sum(const int32_t* tokens, int64_t frames, const q4_embed_table* tables, int32_t num_tables,
                       int64_t dim, void* y, q4_out_dtype y_dtype, void* stream) {
  if (!tokens || !tables || !y) return Q4_ERR_NULL;
  for (int32_t t = 0; t < num_tables && t < Q4_EMBED_MAX_TABLES; ++t)
    if (!tables[t].packed || !tables[t].scales || !tables[t].biases) return Q4_ERR_NULL;
  if (num_tables < 1 || num_tables > Q4_EMBED_MAX_TABLES || frames < 0 || dim <= 0 || dim % 32 != 0)
    return Q4_ERR_SHAPE;
  if (y_dtype != Q4_OUT_BF16 && y_dtype != Q4_OUT_F32) return Q4_ERR_SHAPE;
  for (int32_t t = 0; t < num_tables; ++t)
    if (tables[t].rows < 1) return Q4_ERR_SHAPE;
  if (!aligned(tokens, 4) || !aligned(y, 16)) return Q4_ERR_ALIGN;
  for (int32_t t = 0; t < num_tables; ++t)
    if (!aligned(tables[t].packed, 16) || !aligned(tables[t].scales, 2) || !aligned(tables[t].biases, 2))
      return Q4_ERR_ALIGN;
  // every table is addressed through 32-bit buffer ranges
  for (int32_t t = 0; t < num_tables; ++t)
    if (tables[t].rows > (int64_t)INT32_MAX / (dim / 2)) return Q4_ERR_UNSUPPORTED;
  if (frames == 0) return Q4_OK;
  const int G = static_cast<int>(dim / 32);
  const int tiles = static_cast<int>(ceil_div(G, 64));
  if (frames > (int64_t)INT32_MAX / tiles) return Q4_ERR_UNSUPPORTED;
  q4k::EmbedTables tabs{};
  for (int32_t t = 0; t < num_tables; ++t) {
    tabs.packed[t] = tables[t].packed;
    tabs.scales[t] = tables[t].scales;
    tabs.biases[t] = tables[t].biases;
    tabs.rows[t] = static_cast<int32_t>(tables[t].rows);
  }
  tabs.count = num_tables;
  const dim3 grid(static_cast<unsigned>(frames * tiles)), block(64);
  if (y_dtype == Q4_OUT_F32)
    hipLaunchKernelGGL((q4k::embed_sum_kernel<true>), grid, block, 0, as_stream(stream), tokens, tabs, G, tiles, y);
  else
    hipLaunchKernelGGL((q4k::embed_sum_kernel<false>), grid, block, 0, as_stream(stream), tokens, tabs, G, tiles, y);
  return launch_status();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode attention host side.
namespace {

// positions per split: enough splits to give every compute unit about four
// blocks, at least 64 positions each, at most kAttnMaxSplits
int attn_splits(int64_t heads, int64_t npos) {
  const int64_t cus = device_cu_count();
  // (about two blocks per compute unit: measured against one and four, from
  // 512 to 16384 positions)
  int64_t splits = ceil_div(2 * cus, heads);
  const int64_t by_len = ceil_div(npos, 64);
  if (splits > by_len) splits = by_len;
  if (splits > q4k::kAttnMaxSplits) splits = q4k::kAttnMaxSplits;
  return static_cast<int>(splits < 1 ? 1 : splits);
}

template <int D>
q4_status launch_attn(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache,
                      uint16_t* v_cache, int heads, int cap, int pos, double theta, void* out, bool f32,
                      unsigned char* ws, hipStream_t st) {
  const int npos = pos + 1;
  const int splits = attn_splits(heads, npos);
  const int chunk = static_cast<int>(ceil_div(npos, splits));
  const dim3 grid(heads, splits), block(q4k::kAttnThreads);
  if (f32)
    hipLaunchKernelGGL((q4k::attn_decode_kernel<D, true>), grid, block, 0, st, q, k_new, v_new, k_cache, v_cache, cap,
                       pos, theta, chunk, splits, ws, out);
  else
    hipLaunchKernelGGL((q4k::attn_decode_kernel<D, false>), grid, block, 0, st, q, k_new, v_new, k_cache, v_cache,
                       cap, pos, theta, chunk, splits, ws, out);
  return launch_status();
}

}  // namespace

extern "C" {

int64_t q4_attn_workspace_bytes(int64_t heads, int64_t head_dim) {
  if (heads < 1 || head_dim < 1) return -1;
  return q4k::attn_ws_part_offset(heads, head_dim) + heads * q4k::kAttnMaxSplits * (head_dim + 2) * 4;
}

q4_status q4_attn_decode(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache,
                         uint16_t* v_cache, int64_t heads, int64_t head_dim, int64_t cap, int64_t pos,
                         double rope_theta, void* out, q4_out_dtype out_dtype, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !out || !workspace) return Q4_ERR_NULL;
  if (heads < 1 || cap < 1 || pos < 0 || pos >= cap || !(rope_theta > 0.0)) return Q4_ERR_SHAPE;
  if (out_dtype != Q4_OUT_BF16 && out_dtype != Q4_OUT_F32) return Q4_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return Q4_ERR_UNSUPPORTED;
  if (workspace_bytes < q4_attn_workspace_bytes(heads, head_dim)) return Q4_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k_new, 4) || !aligned(v_new, 4) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(out, out_dtype == Q4_OUT_F32 ? 4 : 2) || !aligned(workspace, 256))
    return Q4_ERR_ALIGN;
  // positions per split fit the scores' LDS; caches are addressed in 32-bit
  // element counts per head
  if (heads > 65535 || cap > (int64_t)INT32_MAX / head_dim || heads * cap * head_dim > (int64_t)1 << 40)
    return Q4_ERR_UNSUPPORTED;
  // (a split's range is addressed through a 32-bit buffer range)
  const int splits = attn_splits(heads, pos + 1);
  if (ceil_div(pos + 1, splits) * head_dim * 2 > (int64_t)INT32_MAX) return Q4_ERR_UNSUPPORTED;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const bool f32 = out_dtype == Q4_OUT_F32;
  if (head_dim == 128)
    return launch_attn<128>(q, k_new, v_new, k_cache, v_cache, (int)heads, (int)cap, (int)pos, rope_theta, out, f32,
                            ws, as_stream(stream));
  return launch_attn<64>(q, k_new, v_new, k_cache, v_cache, (int)heads, (int)cap, (int)pos, rope_theta, out, f32,
                         ws, as_stream(stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Chain executor host side.
namespace {

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
// chain kernels once and check that one block fits per compute unit (once per
// device, thread-safe; the answer is kept).
template <int MV>
bool chain_ready_rows(int dev) {
  static std::once_flag once[kMaxDevices];
  static std::atomic<bool> ready[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::call_once(once[dev], [dev]() {
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
    ready[dev].store(ok);
  });
  return ready[dev].load();
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

// A chain stage processes units of 4 rows in chunks of 16 groups per row (one
// group per lane, 16 lanes per row), so its geometry depends on G only: chunks
// per row CH = ceil(G / 16), with the activations padded to 16 CH groups.
bool plan_stage(int64_t G, int max_groups, int* CH) {
  const int64_t ch = ceil_div(G, q4k::kChunkGroups);
  if (ch * q4k::kChunkGroups > max_groups) return false;
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

q4_status q4_chain_encode_ex(const q4_chain_stage_ex* stages, int32_t num_stages,
                             const q4_chain_matrix_ex* matrices, int32_t num_matrices, int32_t m_rows,
                             q4_out_dtype y_dtype, void* host_plan, int64_t plan_bytes) {
  if (!stages || !matrices || !host_plan) return Q4_ERR_NULL;
  if (num_stages <= 0 || num_matrices <= 0) return Q4_ERR_SHAPE;
  if (m_rows < 1 || m_rows > q4k::kMaxRows) return Q4_ERR_SHAPE;
  const ChainLimits lim = chain_limits(m_rows);
  if (y_dtype != Q4_OUT_BF16 && y_dtype != Q4_OUT_F32) return Q4_ERR_SHAPE;
  const int64_t need = q4_chain_plan_bytes(num_stages, num_matrices);
  if (plan_bytes < need) return Q4_ERR_SHAPE;
  const int64_t ybytes = y_dtype == Q4_OUT_F32 ? 4 : 2;
  // (a gated stage's matrix 1 writes nothing)
  auto writes = [&](const q4_chain_stage_ex& st, int32_t i) { return !(st.gated && i == 1); };
  int32_t next_matrix = 0;
  for (int32_t s = 0; s < num_stages; ++s) {
    const q4_chain_stage_ex& st = stages[s];
    if (st.num_matrices <= 0 || st.first_matrix != next_matrix ||
        st.first_matrix + (int64_t)st.num_matrices > num_matrices)
      return Q4_ERR_SHAPE;
    next_matrix += st.num_matrices;
    if (st.gated != 0 && st.gated != 1) return Q4_ERR_SHAPE;
    if (st.gated && (st.num_matrices != 2 || matrices[st.first_matrix].n != matrices[st.first_matrix + 1].n))
      return Q4_ERR_SHAPE;
    if (st.norm_weight) {
      if (!(st.norm_eps >= 0.0)) return Q4_ERR_SHAPE;
      if (!aligned(st.norm_weight, 16)) return Q4_ERR_ALIGN;
      if (m_rows != 1) return Q4_ERR_UNSUPPORTED;
    }
    for (int32_t i = 0; i < st.num_matrices; ++i) {
      const q4_chain_matrix_ex& m = matrices[st.first_matrix + i];
      // (matrix 1 of a gated stage has no output: any valid address stands in
      // for its y in the shared checks)
      void* y = writes(st, i) ? m.y : matrices[st.first_matrix].y;
      const q4_status c = check_product(st.x, m_rows, m.packed, m.scales, m.biases, m.n, st.k, y, y_dtype);
      if (c != Q4_OK) return c;
      if (m.residual && !writes(st, i)) return Q4_ERR_SHAPE;
      if (m.residual && !aligned(m.residual, ybytes)) return Q4_ERR_ALIGN;
      if (m.n >= (1 << 22)) return Q4_ERR_UNSUPPORTED;
      // each block stages its rows of a matrix in LDS
      if (ceil_div(ceil_div(m.n, q4k::kUnitRows), device_cu_count()) > lim.stage_units) return Q4_ERR_UNSUPPORTED;
      if (!aligned(m.scales, 16) || !aligned(m.biases, 16)) return Q4_ERR_UNSUPPORTED;
      if (!writes(st, i)) continue;
      // a stage may not write its own input (nor its norm weight)
      if (ranges_overlap(st.x, 2 * st.k * m_rows, m.y, ybytes * m.n * m_rows)) return Q4_ERR_UNSUPPORTED;
      // nor write one output range twice (its blocks store in no fixed order),
      // nor write another matrix's residual
      for (int32_t j = 0; j < st.num_matrices; ++j) {
        if (j == i || !writes(st, j)) continue;
        const q4_chain_matrix_ex& o = matrices[st.first_matrix + j];
        if (j < i && ranges_overlap(o.y, ybytes * o.n * m_rows, m.y, ybytes * m.n * m_rows)) return Q4_ERR_UNSUPPORTED;
        if (o.residual && ranges_overlap(o.residual, ybytes * o.n * m_rows, m.y, ybytes * m.n * m_rows))
          return Q4_ERR_UNSUPPORTED;
      }
    }
    int ch;
    if (st.num_matrices > q4k::kMaxMatsPerStage || num_matrices > lim.tab_mats || num_stages > lim.tab_stages ||
        !plan_stage(st.k / 32, lim.max_groups, &ch))
      return Q4_ERR_UNSUPPORTED;
  }
  if (next_matrix != num_matrices) return Q4_ERR_SHAPE;
  // no stage may write a norm weight
  for (int32_t s = 0; s < num_stages; ++s) {
    if (!stages[s].norm_weight) continue;
    for (int32_t t = 0; t < num_stages; ++t)
      for (int32_t i = 0; i < stages[t].num_matrices; ++i) {
        const q4_chain_matrix_ex& m = matrices[stages[t].first_matrix + i];
        if (writes(stages[t], i) && ranges_overlap(stages[s].norm_weight, 2 * stages[s].k, m.y, ybytes * m.n * m_rows))
          return Q4_ERR_UNSUPPORTED;
      }
  }

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
    const q4_chain_stage_ex& st = stages[s];
    q4k::ChainStageDesc d{};
    d.x = st.x;
    d.G = static_cast<int32_t>(st.k / 32);
    plan_stage(d.G, lim.max_groups, &d.CH);
    d.num_mats = st.num_matrices;
    d.mat_begin = st.first_matrix;
    d.norm = st.norm_weight;
    d.norm_eps = st.norm_eps;
    d.gated = st.gated;
    sd[s] = d;
  }
  // Dependencies through memory, between a stage t and a later stage s:
  //  - s reads what t wrote (s's x or a residual of s overlaps t's outputs):
  //    t makes its outputs visible before it arrives at its barrier; s loads
  //    its x only after the preceding stage barrier (device-coherent loads;
  //    residuals are always read that way, after s's products);
  //  - s writes where t wrote (outputs overlap): t's stores are likewise
  //    complete before its barrier, so s's stores land last;
  //  - s writes where t reads a residual: t's residual reads (and stores)
  //    complete before its barrier.
  // A later stage writing an earlier stage's x is harmless: every block has
  // read that x before it arrives at the barrier that precedes the writes.
  // Activations no stage writes are prefetched.
  auto stage_writes = [&](int32_t t, const void* p, int64_t bytes) {
    for (int32_t i = 0; i < stages[t].num_matrices; ++i) {
      const q4_chain_matrix_ex& m = matrices[stages[t].first_matrix + i];
      if (writes(stages[t], i) && ranges_overlap(p, bytes, m.y, ybytes * m.n * m_rows)) return true;
    }
    return false;
  };
  for (int32_t s = 0; s < num_stages; ++s) {
    const q4_chain_stage_ex& st = stages[s];
    for (int32_t t = 0; t < s; ++t) {
      if (stage_writes(t, st.x, 2 * st.k * m_rows)) {
        sd[s].x_internal = 1;
        sd[t].sync_outputs = 1;
      }
      for (int32_t i = 0; i < st.num_matrices; ++i) {
        const q4_chain_matrix_ex& m = matrices[st.first_matrix + i];
        if (writes(st, i) && stage_writes(t, m.y, ybytes * m.n * m_rows)) sd[t].sync_outputs = 1;
        if (m.residual && stage_writes(t, m.residual, ybytes * m.n * m_rows)) sd[t].sync_outputs = 1;
      }
      for (int32_t i = 0; i < stages[t].num_matrices; ++i) {
        const q4_chain_matrix_ex& m = matrices[stages[t].first_matrix + i];
        if (m.residual && stage_writes(s, m.residual, ybytes * m.n * m_rows)) sd[t].sync_outputs = 1;
      }
    }
  }
  // One activation row: each stage's activations (and a normalized stage's
  // norm weights after them) get a region of the kernel's LDS arena, placed
  // one after another round it; xwait names the last earlier stage whose
  // region overlaps, which must be finished before these activations are
  // staged. Several rows share one buffer.
  {
    const int32_t arena = q4k::ChainShape<1>::kXBuffers * q4k::ChainShape<1>::kVecWords;
    int32_t next = 0;
    for (int32_t t = 0; t < num_stages; ++t) {
      if (m_rows != 1) {
        sd[t].xoff = 0;
        sd[t].xwait = t - 1;
        continue;
      }
      const int32_t size = (stages[t].norm_weight ? 2 : 1) * q4k::kChunkGroups * sd[t].CH * q4k::kXWordsPerGroup;
      if (next + size > arena) next = 0;
      sd[t].xoff = next;
      sd[t].xwait = -1;
      for (int32_t u = t - 1; u >= 0; --u) {
        const int32_t us = (stages[u].norm_weight ? 2 : 1) * q4k::kChunkGroups * sd[u].CH * q4k::kXWordsPerGroup;
        if (sd[u].xoff < next + size && next < sd[u].xoff + us) {
          sd[t].xwait = u;
          break;
        }
      }
      next += size;
    }
  }
  // Grid barriers only where a dependency needs one. Stage s starts without
  // one when, against every stage u since the last barrier, s reads nothing u
  // writes (its x, its residuals), and writes nothing u reads (x, residuals)
  // or writes. Blocks then run through such stages at their own pace: a
  // block's reads of an x or a residual all happen between the barriers that
  // enclose its stage (an x is prefetched at most two stages ahead, and
  // before the barrier that opens its stage completes its loads).
  auto stage_reads = [&](int32_t u, const void* p, int64_t bytes) {
    if (ranges_overlap(stages[u].x, 2 * stages[u].k * m_rows, p, bytes)) return true;
    for (int32_t i = 0; i < stages[u].num_matrices; ++i) {
      const q4_chain_matrix_ex& m = matrices[stages[u].first_matrix + i];
      if (m.residual && ranges_overlap(m.residual, ybytes * m.n * m_rows, p, bytes)) return true;
    }
    return false;
  };
  auto depends = [&](int32_t s, int32_t u) {
    const q4_chain_stage_ex& st = stages[s];
    if (stage_writes(u, st.x, 2 * st.k * m_rows)) return true;
    for (int32_t i = 0; i < st.num_matrices; ++i) {
      const q4_chain_matrix_ex& m = matrices[st.first_matrix + i];
      if (m.residual && stage_writes(u, m.residual, ybytes * m.n * m_rows)) return true;
      if (writes(st, i) && (stage_reads(u, m.y, ybytes * m.n * m_rows) || stage_writes(u, m.y, ybytes * m.n * m_rows)))
        return true;
    }
    return false;
  };
  int32_t barriers = 0;
  for (int32_t s = 1, seg = 0; s < num_stages; ++s) {
    bool need = false;
    for (int32_t u = seg; u < s && !need; ++u) need = depends(s, u);
    if (need) {
      seg = s;
      ++barriers;
    } else {
      sd[s].no_barrier = 1;
    }
  }
  // The grid barrier: the one whose arrivals wait for no round trip where the
  // stretches between barriers are short (below 8 MB of weights on average:
  // the Depformer's 0.7-1.8 MB stages, each reading the last one's output),
  // the L2-flag one for longer stretches.
  {
    double bytes = 0.0;
    for (int32_t s2 = 0; s2 < num_stages; ++s2)
      for (int32_t i = 0; i < stages[s2].num_matrices; ++i)
        bytes += (double)matrices[stages[s2].first_matrix + i].n * (double)stages[s2].k * 0.625;
    hdr->barrier = bytes / (barriers + 1) < 8.0e6 ? q4k::kBarrierCounters : q4k::kBarrierL2Flags;
  }
  auto* md = reinterpret_cast<q4k::ChainMatDesc*>(sd + num_stages);
  for (int32_t i = 0; i < num_matrices; ++i) {
    q4k::ChainMatDesc d{};
    d.packed = matrices[i].packed;
    d.scales = matrices[i].scales;
    d.biases = matrices[i].biases;
    d.y = matrices[i].y;
    d.n = static_cast<int32_t>(matrices[i].n);
    d.residual = matrices[i].residual;
    md[i] = d;
  }
  return Q4_OK;
}

q4_status q4_chain_encode_rows(const q4_chain_stage* stages, int32_t num_stages,
                               const q4_chain_matrix* matrices, int32_t num_matrices, int32_t m_rows,
                               q4_out_dtype y_dtype, void* host_plan, int64_t plan_bytes) {
  if (!stages || !matrices || !host_plan) return Q4_ERR_NULL;
  if (num_stages <= 0 || num_matrices <= 0) return Q4_ERR_SHAPE;
  std::vector<q4_chain_stage_ex> se, me_dummy;
  std::vector<q4_chain_matrix_ex> me;
  try {
    se.resize(static_cast<size_t>(num_stages));
    me.resize(static_cast<size_t>(num_matrices));
  } catch (...) {
    return Q4_ERR_UNSUPPORTED;  // (no exception crosses the interface)
  }
  for (int32_t s = 0; s < num_stages; ++s)
    se[s] = q4_chain_stage_ex{stages[s].x, stages[s].k, stages[s].first_matrix, stages[s].num_matrices, nullptr, 0.0,
                              0, 0};
  for (int32_t i = 0; i < num_matrices; ++i)
    me[i] = q4_chain_matrix_ex{matrices[i].packed, matrices[i].scales, matrices[i].biases, matrices[i].y,
                               matrices[i].n, nullptr};
  return q4_chain_encode_ex(se.data(), num_stages, me.data(), num_matrices, m_rows, y_dtype, host_plan, plan_bytes);
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

// ---------------------------------------------------------------------------
// The chain without a caller workspace. Its workspace words (status, per-XCD
// arrival counters, XCD flags: q4k::kWsWords words, enough for up to
// q4k::kMaxXcc XCDs) live in this device-global array, one copy per device.
// In host code `scratch` names a host-side stand-in, never the device memory:
// the device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is passed to kernels.
static __device__ __align__(256) uint32_t scratch[q4k::kWsWords];

namespace {

constexpr int kScratchWords = q4k::kWsWords;
static_assert(kScratchWords * sizeof(uint32_t) == Q4_CHAIN_STATIC_SCRATCH_BYTES, "scratch size as declared");

struct ScratchSlot {
  std::once_flag once;
  std::atomic<uint32_t*> ptr{nullptr};
  std::atomic<int> err{0};
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (nullptr and the
// hipError_t in *err if it cannot be had).
uint32_t* device_scratch(int dev, int* err) {
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot]() {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      slot.err.store(e != hipSuccess ? static_cast<int>(e) : static_cast<int>(hipErrorInvalidSymbol));
      (void)hipGetLastError();
      return;
    }
    slot.ptr.store(static_cast<uint32_t*>(p));
  });
  *err = slot.err.load();
  return slot.ptr.load();
}

}  // namespace

extern "C" q4_status q4_chain_run_rows_noalloc(const void* device_plan, int32_t m_rows, q4_out_dtype y_dtype,
                                               uint32_t* status_out, void* stream) {
  if (!device_plan) return Q4_ERR_NULL;
  if (y_dtype != Q4_OUT_BF16 && y_dtype != Q4_OUT_F32) return Q4_ERR_SHAPE;
  if (m_rows < 1 || m_rows > q4k::kMaxRows) return Q4_ERR_SHAPE;
  if (!aligned(device_plan, 64) || (status_out && !aligned(status_out, 4))) return Q4_ERR_ALIGN;
  // the array holds the barrier words of up to kMaxXcc XCDs
  const uint32_t nxcc = device_xcc_count();
  if (nxcc < 1 || nxcc > static_cast<uint32_t>(q4k::kMaxXcc)) return Q4_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    g_last_hip_error = static_cast<int>(hipGetLastError());
    return Q4_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return Q4_ERR_UNSUPPORTED;
  int err = 0;
  uint32_t* ws = device_scratch(dev, &err);
  if (!ws) {
    g_last_hip_error = err;
    return Q4_ERR_HIP;
  }
  const hipStream_t st = as_stream(stream);
  // every call starts from cleared words (an earlier call on this device may
  // have ended on a timeout and left them inconsistent)
  hipLaunchKernelGGL(q4k::chain_ws_clear_kernel, dim3(1), dim3(256), 0, st, ws, kScratchWords);
  q4_status s = launch_status();
  if (s != Q4_OK) return s;
  const q4k::ChainHeader* plan = static_cast<const q4k::ChainHeader*>(device_plan);
  switch (m_rows) {
    case 1: s = launch_chain<1>(plan, y_dtype, ws, st); break;
    case 2: s = launch_chain<2>(plan, y_dtype, ws, st); break;
    case 3: s = launch_chain<3>(plan, y_dtype, ws, st); break;
    default: s = launch_chain<4>(plan, y_dtype, ws, st); break;
  }
  if (s != Q4_OK || !status_out) return s;
  hipLaunchKernelGGL(q4k::chain_ws_status_kernel, dim3(1), dim3(64), 0, st, ws, status_out);
  return launch_status();
}
