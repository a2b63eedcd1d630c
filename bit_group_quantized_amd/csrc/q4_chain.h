// Persistent chain executor for ordered stages of quantized GEMVs (gfx950).
// Included by q4_api.hip after q4_kernels.h.
//
// The temporal step is an ordered chain of stages ("NVIDIA PersonaPlex 7B on
// Apple Silicon", pipeline diagram: 32 layers; read as standard decoder
// layers: attention input -> q,k,v; attention output -> o; FFN input ->
// gate,up; gated product -> down). A stage multiplies one activation vector by
// one or more matrices that share it; no product of stage s+1 starts before
// every output of stage s is written and visible.
//
// One launch runs the whole chain with one block per compute unit. At the
// start every block copies the plan into LDS (stage and matrix records, with
// its own share of each stage worked out), so no wave walks the plan in
// device memory afterwards. The waves have two roles that meet only through
// LDS words:
//  - waves 1..kComputeWaves compute. A stage's rows are cut into units of 4
//    rows, dealt to the blocks in contiguous runs; a block's units (or pieces of
//    them, when a stage has few units per block) are its items. A compute
//    wave takes its own item of each stage, then claims further items from a
//    per-stage counter, so waves that run faster take more. A slot is one
//    chunk of an item: 16 groups of 4 rows, one group per lane (16 bytes of
//    codes and the group's scale and bias). Each wave keeps the next
//    kRegRing slots in flight in its registers with buffer loads issued in
//    chain order, across stage boundaries (weights never depend on
//    activations), so the first slots of stage s+1 stream in while the grid
//    synchronises after stage s. The dot products run on the matrix cores
//    against the stage's activations in LDS; finished rows go to LDS.
//  - wave 0, the service wave, waits for the block's compute waves to finish
//    a stage, stores the stage's rows, synchronises the grid between stages,
//    and stages activations into LDS (with one activation row, double
//    buffered: activations no stage writes are fetched a stage ahead).
//    Activations an earlier stage writes, and every stage's with several
//    activation rows (one buffer), are staged by all compute waves together
//    once the buffer is free (after the barrier for the former).
//
// Grid synchronisation is two-level: blocks on one XCD (which share an L2)
// count arrivals with L2 atomics; the last arrival of each XCD raises the
// XCD's flag in device-coherent memory, and every block waits for all XCDs'
// flags. All waits are bounded and report a status in the workspace instead
// of hanging.
#pragma once

namespace q4k {

constexpr uint32_t kChainMagic = 0x34433451u;  // "Q4C4"
#ifndef Q4_CHAIN_COMPUTE_WAVES
#define Q4_CHAIN_COMPUTE_WAVES 14
#endif
constexpr int kServiceWave = 0;
constexpr int kComputeWaves = Q4_CHAIN_COMPUTE_WAVES;  // waves 1..kComputeWaves
constexpr int kChainWaves = 1 + kComputeWaves;
constexpr int kMaxMatsPerStage = 4;
constexpr int kUnitRows = 4;      // rows per unit
constexpr int kMaxPieces = 8;     // pieces a unit's chunks may be cut into
constexpr int kMinPieceChunks = 2;  // chunks a piece keeps at least (shorter pieces cost more to close than they balance)
#ifndef Q4_CHAIN_SPLIT_UNITS
#define Q4_CHAIN_SPLIT_UNITS 8
#endif
constexpr int kSplitUnits = Q4_CHAIN_SPLIT_UNITS;  // units are cut until a stage has this many items
constexpr int kSplitItems = 2 * kSplitUnits;       // (so a cut stage has fewer items than this)
#ifndef Q4_CHAIN_REG_RING
#define Q4_CHAIN_REG_RING 6
#endif
constexpr int kRegRing = Q4_CHAIN_REG_RING;  // slots each compute wave keeps in flight, in registers
static_assert(kRegRing == 4 || kRegRing == 6 || kRegRing == 8 || kRegRing == 12 || kRegRing == 16,
              "register ring depth");
constexpr int kQueueLen = 32;     // claimed items a wave may hold between its loads and its arithmetic
static_assert(kRegRing + 1 <= kQueueLen, "item queue");
constexpr uint32_t kQueueEnd = 0xFFFFFFFFu;
constexpr int kChunkGroups = 16;  // groups of each row per slot
constexpr int kXWordsPerGroup = 20;   // 16 re-paired words + sum + pad (bank spread)
constexpr int kChainMaxBlocks = 1024;
constexpr int kMaxRows = 4;       // activation rows a chain may carry
// Limits and LDS shape of a chain carrying MV activation rows. One row keeps
// two activation buffers (the next stage's activations arrive during the
// current stage) and large plan tables; several rows share one weight stream
// (every MFMA row is one activation row), fill one buffer during the stage
// barrier instead, and take smaller tables so that the rows fit.
template <int MV>
struct ChainShape {
  static_assert(MV >= 1 && MV <= kMaxRows, "activation rows");
  static constexpr int kTabStages = MV == 1 ? 384 : 128;  // stages of a chain (the plan is copied into LDS)
  static constexpr int kTabMats = MV == 1 ? 768 : 256;    // matrices of a chain
  static constexpr int kStageUnits = 32;  // units of one matrix per block and stage
  static constexpr int kXBuffers = MV == 1 ? 2 : 1;
  // With one row the activations of successive stages go to regions of an
  // LDS arena the size of two of the widest, placed one after another round
  // it by the encoder; the service wave stages a stage's activations as soon
  // as the stages that used its region are done, up to kRowBufs - 1 stages
  // ahead of the block's slowest wave, whose rows go to kRowBufs buffers in
  // turn. With several rows one buffer serves every stage.
  static constexpr int kRowBufs = MV == 1 ? 4 : 1;
  static constexpr int kMaxGroups = MV == 1 ? 384 : 352;  // k <= 12288 (11264 with several rows)
  static constexpr int kVecWords = kMaxGroups * kXWordsPerGroup + (MV == 1 ? 0 : 4);  // one row (bank shift)
};
constexpr int kDoneSlots = 4;  // completion counts, by stage mod 4 (no wave runs more than 3 stages ahead)
constexpr int kMaxXcc = 16;
constexpr uint32_t kSpinLimit = 1u << 22;

// Waits between waves of a block sleep (the sleeping wave takes no issue
// slots from the working ones) and are cut short by the producer's wakeup;
// a wakeup that arrives just before the sleep only costs the sleep.
__device__ __forceinline__ void nap() { __builtin_amdgcn_s_sleep(8); }
__device__ __forceinline__ void wake_block() { asm volatile("s_wakeup" ::: "memory"); }
static_assert(kChainWaves <= 16, "chain shape");

struct alignas(16) ChainHeader {
  uint32_t magic;
  int32_t num_stages;
  int32_t num_mats;
  int32_t out_f32;
  int32_t plan_bytes;
  int32_t rows;          // activation rows (1..kMaxRows)
  int32_t barrier;       // grid barrier kind (1 or 2)
  int32_t pad[9];
};
struct alignas(16) ChainStageDesc {
  const uint16_t* x;
  int32_t G;             // groups of 32 inputs
  int32_t CH;            // chunks per row: ceil(G / 16)
  int32_t num_mats;
  int32_t mat_begin;
  int32_t x_internal;    // x is written by an earlier stage of the chain
  int32_t sync_outputs;  // a later stage reads or overwrites this stage's outputs (or a residual it reads)
  const uint16_t* norm;  // RMSNorm weight of x, or null
  double norm_eps;
  int32_t gated;         // outputs silu(matrix 0) * matrix 1, to matrix 0's y
  int32_t no_barrier;    // no grid barrier before this stage (nothing it touches depends on the stages since the last one)
  int32_t xoff;          // word offset of the stage's activations in the LDS arena (one row)
  int32_t xwait;         // the last earlier stage whose arena region overlaps this one's, or -1
};
struct alignas(16) ChainMatDesc {
  const uint32_t* packed;
  const uint16_t* scales;
  const uint16_t* biases;
  void* y;
  int32_t n;
  int32_t pad;
  const void* residual;  // added to the product before the rounding, or null
};
static_assert(sizeof(ChainHeader) == 64 && sizeof(ChainStageDesc) == 64 && sizeof(ChainMatDesc) == 48,
              "descriptor sizes");

// Workspace words: status on its own line; per XCD an arrival counter (L2
// scope, one 128-byte line each); the XCDs' flags (device scope, one line).
constexpr int kWsStatus = 0;  // 0 ok, 1 wait timed out, 2 bad plan, 3 block not on the expected XCD
constexpr int kWsXcnt = 64;                       // + 32 * xcc
constexpr int kWsGflag = kWsXcnt + 32 * kMaxXcc;  // + xcc
constexpr int kWsXcnt2 = kWsGflag + 64;          // + 32 * xcc (64-bit counters of the second barrier)
constexpr int kWsWords = kWsXcnt2 + 32 * kMaxXcc;

// Plan reads go through the constant address space, so that (at wave-uniform
// addresses) they become scalar loads and never enter the vector memory
// pipeline that streams the weights.
#define Q4_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ T cload(const T* p) {
  // the address is wave-uniform; saying so keeps the load scalar even where
  // the compiler cannot prove it
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uintptr_t u = (uintptr_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                      ((uintptr_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
  return *(const Q4_CONST T*)u;
}
// Loads through plan pointers are issued as global (not flat) accesses, which
// count only in the vector-memory counter.
#define Q4_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
  return *(const Q4_GLOBAL T*)p;
}
typedef uint32_t q4_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(const void* p) {
  const q4_u32x4 v = *(const Q4_GLOBAL q4_u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <typename T>
__device__ __forceinline__ T gload_off(const unsigned char* base, uint32_t off) {
  return gload(reinterpret_cast<const T*>(base + off));
}

// device-coherent accesses (all XCDs)
__device__ __forceinline__ uint32_t coh_load(const uint32_t* p) {
  return __hip_atomic_load((const Q4_GLOBAL uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint16_t coh_load16(const uint16_t* p) {
  return __hip_atomic_load((const Q4_GLOBAL uint16_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store((Q4_GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store16(uint16_t* p, uint16_t v) {
  __hip_atomic_store((Q4_GLOBAL uint16_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t coh_load64(const uint64_t* p) {
  return __hip_atomic_load((const Q4_GLOBAL uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// device-coherent add whose result is not waited for
__device__ __forceinline__ void coh_add64_post(uint64_t* p, uint64_t v) {
  (void)__hip_atomic_fetch_add((Q4_GLOBAL uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t coh_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add((Q4_GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// XCD-local arrival counter, updated at the XCD's L2 (coherent for the
// blocks that share that L2).
__device__ __forceinline__ uint32_t l2_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add((Q4_GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// hardware id of the XCD this wave runs on
__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15u;
}

// The plan as one block sees it, copied into LDS at the start of a launch
// (every wave then reads its stages and matrices with LDS latency instead of
// chains of dependent memory loads). Block-specific fields (its units, the
// pieces its units are cut into) are worked out in that copy.
struct StageRec {
  int32_t G, CH, nm, mat_begin;
  int32_t P, total;           // pieces per unit, items of the block
  uint32_t inv_p;             // ceil(2^16 / P): i / P == (i * inv_p) >> 16 for the small i here
  int32_t flags;              // 1 ragged (16 CH > G), 2 x written in the chain, 4 outputs read in the chain,
                              // 8 x normalized (RMSNorm), 16 gated output, 32 no grid barrier before it
  int32_t U[kMaxMatsPerStage];  // the block's units of each matrix
  int32_t U0[kMaxMatsPerStage];  // the first of them
  const uint16_t* x;
  const uint16_t* norm;       // RMSNorm weight (flag 8)
  double norm_eps;
  int32_t xoff, xwait;        // the stage's region of the activation arena (ChainStageDesc)
};
struct MatRec {
  const uint32_t* packed;
  const uint16_t* scales;
  const uint16_t* biases;
  void* y;
  int32_t n, pad;
  const void* residual;
};
static_assert(sizeof(StageRec) == 96 && sizeof(MatRec) == 48, "table records");
constexpr int kStageRagged = 1, kStageXInternal = 2, kStageSyncOut = 4, kStageNorm = 8, kStageGated = 16,
              kStageNoBarrier = 32;

// Shared memory: activations and the plan tables (dynamic LDS), and the words
// that connect the roles (a separate static object).
template <int MV>
struct ChainLds {
  using S = ChainShape<MV>;
  uint32_t x[S::kXBuffers * MV * S::kVecWords];  // activations: a stage's at its offset, row v at v * kVecWords
  StageRec st[S::kTabStages];
  MatRec mt[S::kTabMats];
};
template <int MV>
struct ChainFlags {
  using S = ChainShape<MV>;
  // (buffer s mod kRowBufs for stage s)
  float parts[S::kRowBufs][kSplitItems][kUnitRows][MV];   // partial row sums of the pieces of a stage
  uint32_t pieces_done[S::kRowBufs][kSplitUnits];         // pieces of a unit of the stage finished
  float out[S::kRowBufs][kMaxMatsPerStage][S::kStageUnits][kUnitRows][MV];  // the stage's finished rows
  float res[S::kRowBufs][kMaxMatsPerStage][S::kStageUnits][kUnitRows][MV];  // residuals of those rows, loaded early
  uint32_t done[kDoneSlots];         // completions of the stages s = j mod kDoneSlots by the compute waves
  int32_t x_stage;                   // last stage whose activations are in LDS
  int32_t x_fill;                    // stage whose activations the compute waves stage together
  uint32_t x_filled;                 // compute-wave shares of such stagings done so far
  uint32_t abort;
  uint32_t go;
  uint32_t misfit;                   // a matrix has more units per block than the row staging holds
  uint32_t claim[S::kTabStages];     // items of each stage claimed so far by the block's waves
  uint32_t queue[kComputeWaves][kQueueLen];  // each wave's claimed items, oldest first
  double norm_part[kComputeWaves];   // each compute wave's share of a normalized stage's sum of squares
  uint32_t norm_cnt;                 // shares written so far
  uint32_t any_norm;                 // some stage of the plan is normalized
};

// LDS flag words, accessed through explicit LDS pointers (a volatile access
// through a generic pointer would become a flat access, which also counts in
// the vector-memory counter).
#define Q4_LDS __attribute__((address_space(3)))
// Every lane reads the same word, so the value is wave-uniform; saying so
// keeps the control flow that depends on it scalar.
__device__ __forceinline__ uint32_t lds_get(const uint32_t* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)*(const volatile Q4_LDS uint32_t*)p);
}
__device__ __forceinline__ int32_t lds_geti(const int32_t* p) {
  return __builtin_amdgcn_readfirstlane(*(const volatile Q4_LDS int32_t*)p);
}
__device__ __forceinline__ void lds_put(uint32_t* p, uint32_t v) { *(volatile Q4_LDS uint32_t*)p = v; }
__device__ __forceinline__ void lds_puti(int32_t* p, int32_t v) { *(volatile Q4_LDS int32_t*)p = v; }
__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add((Q4_LDS uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint32_t lds_add_rtn(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add((Q4_LDS uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ int ufl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Stage geometry (wave-uniform).
struct Geo {
  int G, CH, num_mats, mat_begin;
};
__device__ __forceinline__ Geo geo_of(const StageRec& r) {
  Geo g;
  g.G = ufl(r.G);
  g.CH = ufl(r.CH);
  g.num_mats = ufl(r.nm);
  g.mat_begin = ufl(r.mat_begin);
  return g;
}
// a pointer field of a table record, wave-uniform
template <typename T>
__device__ __forceinline__ T* ufl_ptr(T* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return reinterpret_cast<T*>((uintptr_t)(uint32_t)ufl((int)(uint32_t)a) |
                              ((uintptr_t)(uint32_t)ufl((int)(uint32_t)(a >> 32)) << 32));
}

// Units (4 consecutive rows) of a matrix are dealt to the blocks in
// contiguous runs: block b takes units [u0, u0 + count), the first
// nunits % gridDim.x blocks one more than the others (measured ~1% faster on
// the temporal step than dealing units round-robin).
struct BlockRange {
  int u0, count;  // first unit, units of this block
};
__device__ __forceinline__ BlockRange block_range(int nunits) {
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  BlockRange r;
  const int q = nunits / nb, rem = nunits - q * nb;
  r.u0 = b * q + min(b, rem);
  r.count = q + (b < rem ? 1 : 0);
  return r;
}
__device__ __forceinline__ int unit_of(const BlockRange& br, int i) { return br.u0 + i; }


// s_waitcnt immediate that waits for the vector-memory counter only
constexpr int vmcnt_imm(int n) { return 0xF70 | (n & 15) | (((n >> 4) & 3) << 14); }

// ---------------------------------------------------------------- compute

// Lane t of a slot holds row (t & 3) of its unit and group (16 ch + (t >> 2))
// of that row. Sum over the 16 lanes that hold one row (lanes congruent mod
// 4): two rotations within each 16-lane DPP row, then across the four rows.
__device__ __forceinline__ float row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  // (the swaps give every lane the same two addends, its own and its
  // partner's, so both lanes of a pair hold the same sum)
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One slot in a lane's registers: its 16 bytes of codes and its group's bf16
// scale and bias (zero-extended).
struct Slot {
  uint4 w;
  uint32_t s, b;
};

typedef short mfma_bf16x4 __attribute__((ext_vector_type(4)));
typedef float mfma_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ mfma_bf16x4 as_bf16x4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(mfma_bf16x4, make_uint2(lo, hi));
}

// The lane's group term of a slot, scale * (codes . activations) + bias * (sum
// of activations), with the dot product on the matrix cores. The 4x4x4 bf16
// MFMA works on 16 independent 4x4 blocks; block b (lanes 4b..4b+3)
// multiplies A (4 rows x 4 inputs, row i from lane 4b+i) by B (4 inputs x 4
// columns, column j from lane 4b+j), and lane 4b+j receives column j of the
// product, row i in register i. Here B column j is lane 4b+j's own dequantized
// codes (exact small integers in bf16) and every lane supplies its group's
// activations as A, so register 0 of each lane accumulates exactly its own
// group's sum of code x activation in fp32: two MFMAs per 8 codes, codes and
// activations in the same re-paired input order. xg: the group's 16
// re-paired activation words and their sum (LDS).
// With MV activation rows, lane 4b+i supplies row min(i, MV - 1) as A row i,
// so register i accumulates activation row i against the lane's codes: MV
// rows cost the same 8 MFMAs. xg is then the lane's own A row's group and
// xrow the distance between rows in LDS (the group sums of every row are
// read from there), vown the row the lane supplies.
template <int MV>
__device__ __forceinline__ void slot_terms(const Slot& d, const uint32_t* xg, int xrow, int vown, bool live,
                                           float (&term)[MV]) {
  const uint4 x0 = *reinterpret_cast<const uint4*>(xg + 0);
  const uint4 x1 = *reinterpret_cast<const uint4*>(xg + 4);
  const uint4 x2 = *reinterpret_cast<const uint4*>(xg + 8);
  const uint4 x3 = *reinterpret_cast<const uint4*>(xg + 12);
  const uint32_t ws[4] = {d.w.x, d.w.y, d.w.z, d.w.w};
  const uint32_t xp[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                           x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
  mfma_f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t q02, q46, q13, q57;
    word_to_bf16_pairs(ws[t], q02, q46, q13, q57);
    c = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_bf16x4(xp[4 * t], xp[4 * t + 1]), as_bf16x4(q02, q46), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_bf16x4(xp[4 * t + 2], xp[4 * t + 3]), as_bf16x4(q13, q57), c, 0, 0, 0);
  }
  // lanes past G in a ragged last chunk weigh zero
  const float sc = __uint_as_float(live ? d.s << 16 : 0u);
  const float bi = __uint_as_float(live ? d.b << 16 : 0u);
  if constexpr (MV == 1) {
    term[0] = fmaf(sc, c[0], bi * __uint_as_float(xg[16]));
  } else {
    // (row i's sum sits at the same place of row i's activations; vown is
    // the row this lane supplies)
    const uint32_t* x_row0 = xg - vown * xrow;
#pragma unroll
    for (int i = 0; i < MV; ++i) term[i] = fmaf(sc, c[i], bi * __uint_as_float(x_row0[i * xrow + 16]));
  }
}

// Lanes 0..3 leave the 4 rows of local unit u of matrix mi of the stage in
// LDS; the service wave stores them. Compute waves issue no global stores at
// all, so that every step of their loop issues exactly the same loads.
template <int MV>
__device__ __forceinline__ void stage_rows(ChainFlags<MV>& F, int s, int mi, int u, int lane, const float (&v)[MV]) {
  if (lane < kUnitRows) {
#pragma unroll
    for (int i = 0; i < MV; ++i) *(volatile Q4_LDS float*)&F.out[s % ChainShape<MV>::kRowBufs][mi][u][lane][i] = v[i];
  }
}

// a wait timed out: the service wave reports it
template <int MV>
__device__ __forceinline__ void compute_fail(ChainFlags<MV>& F) {
  if ((threadIdx.x & 63) == 0) lds_put(&F.abort, 2u);
  wake_block();
}

// Work of one block in one stage. The stage's matrices, in order, contribute
// U[mi] units each (the block's share); every unit is cut into P
// pieces of consecutive chunks, piece p covering chunks [p CH / P,
// (p + 1) CH / P). Item i of the stage is (matrix, unit, piece) in that
// order. Compute wave w takes item w of every stage, then claims further items
// one at a time from a counter per stage (a wave that runs faster takes more
// of them); it runs its items in the order it took them. P grows (up
// to 8, and not past CH) while the stage holds fewer than 3 items per compute
// wave, so a cut stage has fewer than 3 kComputeWaves units and fewer than
// 6 kComputeWaves items.
struct StageInfo {
  int s, G, CH, nm, mat_begin, P, total;
  uint32_t inv_p;  // ceil(2^16 / P): i / P == (i * inv_p) >> 16 for the small i here
  bool ragged;     // 16 CH > G: the last chunk has lanes past the row end
  int U[kMaxMatsPerStage];
};
// Fill the block's record of a stage (one lane per stage, at the start of a
// launch). Returns false if a matrix has more units per block than the LDS
// staging of rows holds.
template <int MV>
__device__ __forceinline__ bool build_stage_rec(StageRec& r, const ChainStageDesc* sd, const ChainMatDesc* mats) {
  r.G = sd->G;
  r.CH = sd->CH;
  r.nm = sd->num_mats;
  r.mat_begin = sd->mat_begin;
  r.x = sd->x;
  r.flags = (r.CH * kChunkGroups != r.G ? kStageRagged : 0) | (sd->x_internal ? kStageXInternal : 0) |
            (sd->sync_outputs ? kStageSyncOut : 0) | (sd->norm ? kStageNorm : 0) | (sd->gated ? kStageGated : 0) |
            (sd->no_barrier ? kStageNoBarrier : 0);
  r.norm = sd->norm;
  r.norm_eps = sd->norm_eps;
  r.xoff = MV == 1 ? sd->xoff : 0;
  r.xwait = MV == 1 ? sd->xwait : -1;
  int units = 0;
  bool fits = true;
  for (int mi = 0; mi < kMaxMatsPerStage; ++mi) {
    const int nunits = mi < r.nm ? (mats[r.mat_begin + mi].n + kUnitRows - 1) / kUnitRows : 0;
    const BlockRange br = block_range(nunits);
    r.U[mi] = br.count;
    r.U0[mi] = br.u0;
    // (block 0 has the most units; every block takes the same decision)
    fits = fits && (nunits + (int)gridDim.x - 1) / (int)gridDim.x <= ChainShape<MV>::kStageUnits;
    units += r.U[mi];
  }
  int P = 1;
  // (a cut stage has fewer than kSplitUnits units and, since P stops growing
  // once units * P reaches kSplitUnits, fewer than 2 kSplitUnits items)
  while (P < kMaxPieces && r.CH >= kMinPieceChunks * (P + 1) && units * P < kSplitUnits) ++P;
  r.P = P;
  r.inv_p = (65536u + (uint32_t)P - 1u) / (uint32_t)P;
  r.total = units * P;
  return fits;
}
template <int MV>
__device__ __forceinline__ int stage_flags(const ChainLds<MV>& L, int s) { return ufl(L.st[s].flags); }
template <int MV>
__device__ __forceinline__ const uint16_t* stage_x(const ChainLds<MV>& L, int s) { return ufl_ptr(L.st[s].x); }
// the LDS region of stage s's activations (and, after them, a normalized
// stage's norm weights)
template <int MV>
__device__ __forceinline__ uint32_t* stage_xbuf(ChainLds<MV>& L, int s) { return L.x + ufl(L.st[s].xoff); }
template <int MV>
__device__ __forceinline__ void stage_info(StageInfo& si, const ChainLds<MV>& L, int s) {
  const StageRec& r = L.st[s];
  si.s = s;
  si.G = ufl(r.G);
  si.CH = ufl(r.CH);
  si.nm = ufl(r.nm);
  si.mat_begin = ufl(r.mat_begin);
  si.ragged = (ufl(r.flags) & kStageRagged) != 0;
  si.P = ufl(r.P);
  si.inv_p = (uint32_t)ufl((int)r.inv_p);
  si.total = ufl(r.total);
#pragma unroll
  for (int mi = 0; mi < kMaxMatsPerStage; ++mi) si.U[mi] = ufl(r.U[mi]);
}
struct Item {
  int mi, u, p, ca, cb;
};
__device__ __forceinline__ void decode_item(const StageInfo& si, int i, Item& it) {
  it.mi = 0;
#pragma unroll
  for (int mi = 0; mi < kMaxMatsPerStage - 1; ++mi) {
    const int n = si.U[it.mi] * si.P;
    if (i >= n) {
      i -= n;
      ++it.mi;
    }
  }
  it.mi = ufl(it.mi);
  it.u = ufl((int)(((uint32_t)i * si.inv_p) >> 16));
  it.p = ufl(i - it.u * si.P);
  it.ca = ufl((int)(((uint32_t)(it.p * si.CH) * si.inv_p) >> 16));
  it.cb = ufl((int)(((uint32_t)((it.p + 1) * si.CH) * si.inv_p) >> 16));
}

// cache-policy bits of a buffer load: sc1, the device-coherent load (as the
// agent-scope atomic loads above are issued); nt, the streaming hint, for the
// weight codes, which are read once (measured on the temporal step: 2% faster;
// the same hint on scales and biases, whose cache lines serve four
// consecutive chunks, is 3.5% slower)
constexpr int kAuxSc1 = 16;
constexpr int kAuxNt = 2;
#ifndef Q4_CHAIN_WEIGHT_AUX
#define Q4_CHAIN_WEIGHT_AUX 2
#endif
constexpr int kWeightAux = Q4_CHAIN_WEIGHT_AUX;  // policy of the weight-code loads
// Buffer descriptor of a raw byte range: loads at offsets at or past nbytes
// return zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}

// The slot a compute wave loads next: item i of stage si (the last item the
// wave claimed) and its next chunk. Loads go through buffer descriptors of the
// item's unit's codes, scales and biases, sized to the rows that exist: lanes
// that run past a ragged row's end read the next row (given zero weight) or,
// past the matrix, zeros. Wave-uniform except the lane offsets.
struct LoadCursor {
  StageInfo si;
  int i;                                 // current item
  int left;                              // its slots not yet loaded
  __amdgpu_buffer_rsrc_t rw, rs, rb;     // the unit's codes, scales, biases
  uint32_t vw, vs;                       // lane offsets of the next slot
  uint32_t lw, ls;                       // lane offsets of chunk 0 (per stage)
  bool done;                             // no slots left in the chain
  uint32_t qh;                           // items the wave has claimed
  bool fresh;                            // no item of this stage taken yet
};

// Lane (row r = t & 3, col c = t >> 2) loads the 16 bytes of codes of group
// 16 ch + c of row r of the unit, and that group's scale and bias: chunk ch
// adds 256 (codes) and 32 (scales) bytes to the lane's offset in the unit.
__device__ __forceinline__ void lc_lanes(LoadCursor& lc, int lane) {
  const int G = lc.si.G;
  const int row = lane & 3, col = lane >> 2;
  // (24-bit products: a full 32-bit multiply-add would be a 64-bit one whose
  // unused high half can alias a register with a load in flight)
  const uint32_t e = __umul24((uint32_t)row, (uint32_t)G) + (uint32_t)col;
  lc.lw = e * 16u;
  lc.ls = e * 2u;
}
// set up item lc.i of stage lc.si
template <int MV>
__device__ __forceinline__ void lc_item(LoadCursor& lc, const ChainLds<MV>& L) {
  Item it;
  decode_item(lc.si, lc.i, it);
  const MatRec& mr = L.mt[lc.si.mat_begin + it.mi];
  const int n = ufl(mr.n);
  const int gu = ufl(L.st[lc.si.s].U0[it.mi]) + it.u;  // (the block's units are consecutive)
  const uint32_t rows = (uint32_t)min(kUnitRows, n - gu * kUnitRows);
  const uint32_t row_w = (uint32_t)lc.si.G * 16u, row_s = (uint32_t)lc.si.G * 2u;
  lc.rw = byte_range(reinterpret_cast<const unsigned char*>(ufl_ptr(mr.packed)) + (uint64_t)gu * kUnitRows * row_w, rows * row_w);
  lc.rs = byte_range(reinterpret_cast<const unsigned char*>(ufl_ptr(mr.scales)) + (uint64_t)gu * kUnitRows * row_s, rows * row_s);
  lc.rb = byte_range(reinterpret_cast<const unsigned char*>(ufl_ptr(mr.biases)) + (uint64_t)gu * kUnitRows * row_s, rows * row_s);
  lc.vw = lc.lw + (uint32_t)it.ca * 256u;
  lc.vs = lc.ls + (uint32_t)it.ca * 32u;
  lc.left = ufl(it.cb - it.ca);
}
// claim the wave's next item (through the stages) and queue it for the
// arithmetic, or queue the end
template <int MV>
__device__ __forceinline__ void lc_next_item(LoadCursor& lc, const ChainLds<MV>& L, ChainFlags<MV>& F, int num_stages, int cw,
                                             int lane) {
  while (true) {
    // a wave's first item of a stage is its own (item cw); the rest are
    // claimed in turn
    uint32_t item = (uint32_t)cw;
    if (lc.fresh) {
      lc.fresh = false;
    } else if (lc.si.total <= kComputeWaves) {
      item = (uint32_t)lc.si.total;  // every item of the stage is some wave's own: none to claim
    } else {
      if (lane == 0) item = lds_add_rtn(&F.claim[lc.si.s], 1u);
      item = kComputeWaves + (uint32_t)ufl((int)item);
    }
    uint32_t code;
    if (item < (uint32_t)lc.si.total) {
      lc.i = (int)item;
      code = ((uint32_t)lc.si.s << 16) | item;
    } else if (lc.si.s + 1 >= num_stages) {
      // nothing left: empty ranges, whose loads return zeros without
      // touching memory
      lc.done = true;
      lc.rw = lc.rs = lc.rb = byte_range(nullptr, 0u);
      lc.left = 0x7FFFFFFF;
      code = kQueueEnd;
    } else {
      stage_info(lc.si, L, lc.si.s + 1);
      lc_lanes(lc, lane);
      lc.fresh = true;
      continue;
    }
    if (lane == 0) lds_put(&F.queue[cw][lc.qh % kQueueLen], code);
    lc.qh = (uint32_t)ufl((int)(lc.qh + 1u));
    if (!lc.done) lc_item(lc, L);
    return;
  }
}
// Issue the loads of the cursor's slot into d and advance (every step issues
// the same three loads, which lets the compiler wait for exactly the slot it
// is about to use).
template <int MV>
__device__ __forceinline__ void lc_load(LoadCursor& lc, Slot& d, int lane, const ChainLds<MV>& L, ChainFlags<MV>& F,
                                        int num_stages, int cw) {
  const q4_u32x4 w =
      __builtin_bit_cast(q4_u32x4, __builtin_amdgcn_raw_buffer_load_b128(lc.rw, (int)lc.vw, 0, kWeightAux));
  d.w = make_uint4(w.x, w.y, w.z, w.w);
  d.s = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(lc.rs, (int)lc.vs, 0, 0);
  d.b = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(lc.rb, (int)lc.vs, 0, 0);
  lc.vw += 256u;
  lc.vs += 32u;
  lc.left = ufl(lc.left - 1);
  if (lc.left == 0) lc_next_item(lc, L, F, num_stages, cw, lane);
}

// One compute wave's share of staging stage t's activations (the layout
// service_load_x writes): group e of the MV rows' 16 CH padded groups goes to
// wave e / 64 mod kComputeWaves. Used where the waves would otherwise wait
// for one wave to stage them alone: with one activation buffer (several
// rows), and for activations an earlier stage wrote (loaded after the grid
// barrier, COH: device-coherent loads). Every load goes through a range-checked
// buffer descriptor (groups past G read zero), so that all of them are in flight together.
template <int MV, bool COH>
__device__ __forceinline__ void fill_x_share(const Geo& g, const void* x, uint32_t* buf, int cw, int lane) {
  constexpr int kPer = 1;  // groups per lane in flight (two would crowd the registers of the slots in flight)
  constexpr int kSpan = kComputeWaves * 64;
  const int gpad = kChunkGroups * g.CH;
  const int total = MV * gpad;
  const __amdgpu_buffer_rsrc_t rx = byte_range(x, (uint32_t)(MV * g.G * 64));
  for (int base = cw * 64; base < total; base += kPer * kSpan) {
    q4_u32x4 q[kPer][4];
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int e = base + p * kSpan + lane;
      int v = 0;
#pragma unroll
      for (int r = 1; r < MV; ++r) v += e >= r * gpad ? 1 : 0;
      const int grp = e - v * gpad;
      const uint32_t off = (e < total && grp < g.G) ? (uint32_t)((v * g.G + grp) * 64) : 0xFFFFFF00u;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        q[p][j] = __builtin_bit_cast(q4_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16 * j), 0,
                                                                                     COH ? kAuxSc1 : 0));
    }
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int e = base + p * kSpan + lane;
      int v = 0;
#pragma unroll
      for (int r = 1; r < MV; ++r) v += e >= r * gpad ? 1 : 0;
      const int grp = e - v * gpad;
      if (e < total) {
        uint32_t* dst = buf + v * ChainShape<MV>::kVecWords + grp * kXWordsPerGroup;
        float xs = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 e4 = make_uint4(q[p][j].x, q[p][j].y, q[p][j].z, q[p][j].w);
          uint32_t p02, p46, p13, p57;
          x_to_pairs(e4, p02, p46, p13, p57);
          *reinterpret_cast<uint4*>(dst + 4 * j) = make_uint4(p02, p46, p13, p57);
          xs += x_sum8(e4);
        }
        dst[16] = __float_as_uint(xs);
      }
    }
  }
}

// Sum over a wave, in fp64, in a fixed order: within each row of 16 lanes by
// DPP rotations (every lane ends with its row's total), then the four rows'
// totals (read from lanes 0, 16, 32, 48) as (r0 + r1) + (r2 + r3).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double lane_f64(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = __dadd_rn(v, dpp_f64<0x128>(v));  // row_ror:8
  v = __dadd_rn(v, dpp_f64<0x124>(v));  // row_ror:4
  v = __dadd_rn(v, dpp_f64<0x122>(v));  // row_ror:2
  v = __dadd_rn(v, dpp_f64<0x121>(v));  // row_ror:1
  return __dadd_rn(__dadd_rn(lane_f64(v, 0), lane_f64(v, 16)), __dadd_rn(lane_f64(v, 32), lane_f64(v, 48)));
}

// One compute wave's share of staging a normalized stage's activations (one
// activation row; RMSNorm in front of the products, the normalization of the
// model's layers). Two lanes share a group: lane (cw, lane) takes half
// (64 cw + lane) & 1 of group (64 cw + lane) >> 1, 16 values; every group of
// the padded row has its lanes (2 * 16 CH <= 768 < 64 kComputeWaves).
//  1. The lane loads its 16 values and their 16 norm weights and parks both,
//     raw, in their slots: the values in the stage's activation region, the
//     weights in the same layout right after it (the encoder gives a
//     normalized stage a region twice the size).
//     The squares (exact in fp32) are summed in fp64; the wave's sum goes to
//     LDS and, once all kComputeWaves shares are there, every wave adds them
//     in wave order, so every block forms the same total.
//  2. inv = 1 / sqrt(total / k + eps) in fp64; each value becomes
//     (x * gamma) * inv, the product x * gamma exact in fp32 and the scaling
//     in fp64, rounded to fp32 and then to bf16 (the normalized row is a bf16
//     activation), re-paired in place. The group sum adds the four 8-value
//     sums in the order the plain staging adds them.
// Groups past G stay zero. nfill counts the normalized stagings this wave has
// taken part in (the LDS count of shares runs on across stages). Returns false
// if the wait for the other waves' shares timed out or the block is aborting.
// Only phase 1 holds loaded registers; the spin between holds none.
__device__ __forceinline__ bool fill_x_norm(const Geo& g, const void* x, const uint16_t* gamma, double eps,
                                            uint32_t* buf, uint32_t* gbuf, int cw, int lane, ChainFlags<1>& F,
                                            uint32_t& nfill) {
  const int gpad = kChunkGroups * g.CH;
  const int grp = (cw * 64 + lane) >> 1;
  const int half = lane & 1;
  const bool live = grp < g.G;
  const bool slot = grp < gpad;
  uint32_t* dst = buf + grp * kXWordsPerGroup + 8 * half;
  uint32_t* gdst = gbuf + grp * kXWordsPerGroup + 8 * half;
  {
    const __amdgpu_buffer_rsrc_t rx = byte_range(x, (uint32_t)(g.G * 64));
    const __amdgpu_buffer_rsrc_t rg = byte_range(gamma, (uint32_t)(g.G * 64));
    const uint32_t off = live ? (uint32_t)(grp * 64 + 32 * half) : 0xFFFFFF00u;
    q4_u32x4 q[2], gm[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      q[j] = __builtin_bit_cast(q4_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16 * j), 0, kAuxSc1));
      gm[j] = __builtin_bit_cast(q4_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, (int)(off + 16 * j), 0, 0));
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t w4[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float lo = bf16_to_f32(w4[h] & 0xFFFFu), hi = bf16_to_f32(w4[h] >> 16);
        ss = __dadd_rn(ss, (double)(lo * lo));
        ss = __dadd_rn(ss, (double)(hi * hi));
      }
    }
    if (slot) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        *reinterpret_cast<uint4*>(dst + 4 * j) = make_uint4(q[j].x, q[j].y, q[j].z, q[j].w);
        *reinterpret_cast<uint4*>(gdst + 4 * j) = make_uint4(gm[j].x, gm[j].y, gm[j].z, gm[j].w);
      }
    }
    ss = wave_sum_f64(ss);
    if (lane == 0) *(volatile Q4_LDS double*)&F.norm_part[cw] = ss;
  }
  compiler_fence();
  lds_wait();
  if (lane == 0) lds_add(&F.norm_cnt, 1u);
  wake_block();
  ++nfill;
  uint32_t spins = 0;
  while ((int)(lds_get(&F.norm_cnt) - (uint32_t)kComputeWaves * nfill) < 0) {
    nap();
    if (lds_get(&F.abort) != 0u || ++spins > kSpinLimit) return false;
  }
  compiler_fence();
  double tot = 0.0;
  for (int w = 0; w < kComputeWaves; ++w) tot = __dadd_rn(tot, *(volatile Q4_LDS double*)&F.norm_part[w]);
  const double inv = __ddiv_rn(1.0, __dsqrt_rn(__dadd_rn(__ddiv_rn(tot, (double)(g.G * 32)), eps)));
  float part[2] = {0.f, 0.f};
  if (slot) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 xw = *reinterpret_cast<const uint4*>(dst + 4 * j);
      const uint4 gw = *reinterpret_cast<const uint4*>(gdst + 4 * j);
      const uint32_t w4[4] = {xw.x, xw.y, xw.z, xw.w};
      const uint32_t g4[4] = {gw.x, gw.y, gw.z, gw.w};
      uint32_t nv[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float tlo = bf16_to_f32(w4[h] & 0xFFFFu) * bf16_to_f32(g4[h] & 0xFFFFu);
        const float thi = bf16_to_f32(w4[h] >> 16) * bf16_to_f32(g4[h] >> 16);
        nv[h] = live ? ((uint32_t)f32_to_bf16_rne(__double2float_rn(__dmul_rn((double)tlo, inv))) |
                        ((uint32_t)f32_to_bf16_rne(__double2float_rn(__dmul_rn((double)thi, inv))) << 16))
                     : 0u;
      }
      const uint4 e4 = make_uint4(nv[0], nv[1], nv[2], nv[3]);
      uint32_t p02, p46, p13, p57;
      x_to_pairs(e4, p02, p46, p13, p57);
      *reinterpret_cast<uint4*>(dst + 4 * j) = make_uint4(p02, p46, p13, p57);
      part[j] = x_sum8(e4);
    }
  }
  // group sum ((s0 + s1) + s2) + s3, s2 and s3 from the odd lane of the pair
  const float s2 = __shfl_xor(part[0], 1, 64), s3 = __shfl_xor(part[1], 1, 64);
  if (slot && half == 0) dst[16] = __float_as_uint(((part[0] + part[1]) + s2) + s3);
  return true;
}

// NORM: the plan has normalized stages. The staging code those need is
// large and is inlined at every place a wave can change stage, so plans
// without them run a body compiled without it (its code then stays small).
template <int MV, bool OUT_F32, bool NORM>
__device__ __forceinline__ void compute_body(int num_stages, int cw, ChainLds<MV>& L, ChainFlags<MV>& F,
                                             uint32_t* ws) {
  using S = ChainShape<MV>;
  const int lane = threadIdx.x & 63;
  const int col = lane >> 2;
  const int vown = (lane & 3) < MV ? (lane & 3) : MV - 1;  // the activation row this lane supplies
  LoadCursor lc;
  lc.done = false;
  lc.qh = 0;
  lc.fresh = true;
  stage_info(lc.si, L, 0);
  lc_lanes(lc, lane);
  lc_next_item(lc, L, F, num_stages, cw, lane);
  Slot d[kRegRing];  // slots k .. k + kRegRing - 1 in flight (indexed only by unrolled constants)
#pragma unroll
  for (int j = 0; j < kRegRing; ++j) lc_load(lc, d[j], lane, L, F, num_stages, cw);

  StageInfo si;      // the stage being computed (si.s == num_stages: done)
  int i = 0;         // the item being computed
  uint32_t qt = 0;   // items taken from the wave's queue
  Item it;
  int left = 0;      // its slots not yet computed
  int gch = 0;       // first group of its next chunk
  const uint32_t* x0 = nullptr;  // group col of chunk 0 of the lane's activation row
  float acc[MV];
#pragma unroll
  for (int v = 0; v < MV; ++v) acc[v] = 0.f;
  bool stop = false;  // a wait timed out or another wave failed: finish without waiting
  uint32_t nfill = 0;  // normalized stagings this wave has taken part in

  // stage si.s may start once the service wave has published it: its
  // activations are in LDS, and every wave of the grid has finished the
  // stages it depends on
  auto enter_stage = [&]() {
    uint32_t spins = 0;
    bool filled = false;
    while (!stop && lds_geti(&F.x_stage) < si.s) {
      if (!filled && lds_geti(&F.x_fill) == si.s) {
        // the service wave asks the compute waves to stage these activations
        compiler_fence();
        const Geo g = geo_of(L.st[si.s]);
        uint32_t* buf = stage_xbuf(L, si.s);
        const int fl = stage_flags(L, si.s);
        if constexpr (MV == 1) {
          // (one activation row: the service wave stages activations no stage
          // writes, except a normalized stage's; the compute waves stage those
          // and the ones written in the chain, always with coherent loads)
          if (NORM && (fl & kStageNorm)) {
            if (!fill_x_norm(g, stage_x(L, si.s), ufl_ptr(L.st[si.s].norm), L.st[si.s].norm_eps, buf,
                             buf + kChunkGroups * g.CH * kXWordsPerGroup, cw, lane, F, nfill))
              stop = true;
          } else {
            fill_x_share<MV, true>(g, stage_x(L, si.s), buf, cw, lane);
          }
        } else {
          if (fl & kStageXInternal)
            fill_x_share<MV, true>(g, stage_x(L, si.s), buf, cw, lane);
          else
            fill_x_share<MV, false>(g, stage_x(L, si.s), buf, cw, lane);
        }
        compiler_fence();
        if (lane == 0) lds_add(&F.x_filled, 1u);
        wake_block();
        filled = true;
        continue;
      }
      nap();
      stop = lds_get(&F.abort) != 0u || ++spins > kSpinLimit;
    }
    compiler_fence();
    x0 = stage_xbuf(L, si.s) + vown * S::kVecWords + col * kXWordsPerGroup;
  };
  // move to the wave's next claimed item, closing the stages it leaves (every
  // stage is counted once, after the wave's rows of it are in LDS) and
  // entering the next ones
  // after the wave's item ends: take its next item from the queue (code; the
  // stage it belongs to is s_next). Stages between are entered one by one
  // (the wave takes its share of any staging of their activations) and
  // counted done; the stage being left was counted done already, before the
  // refill (end_stage_early).
  auto next_item = [&](uint32_t code, int s_next) {
    bool left_counted = true;
    while (si.s < s_next) {
      if (!left_counted) {
        compiler_fence();
        if (lane == 0) lds_add(&F.done[si.s % kDoneSlots], 1u);
        wake_block();
      }
      left_counted = false;
      if (si.s + 1 >= num_stages) {
        si.s = num_stages;
        return;
      }
      stage_info(si, L, si.s + 1);
      enter_stage();
    }
    i = (int)(code & 0xFFFFu);
    decode_item(si, i, it);
    left = ufl(it.cb - it.ca);
    gch = ufl(it.ca * kChunkGroups);
  };
  // the wave's next item as the load cursor queued it; if it lies in a later
  // stage, the current stage is counted done here: its rows are in LDS
  auto end_stage_early = [&](uint32_t& code) {
    code = lds_get(&F.queue[cw][qt % kQueueLen]);
    qt = (uint32_t)ufl((int)(qt + 1u));
    const int s_next = code == kQueueEnd ? num_stages : (int)(code >> 16);
    if (si.s < s_next) {
      compiler_fence();
      if (lane == 0) lds_add(&F.done[si.s % kDoneSlots], 1u);
      wake_block();
    }
    return s_next;
  };
  // the item's partial row sums are complete: a whole unit's rows go to LDS;
  // a piece's go to its place, and the wave that completes a unit's last
  // piece adds the pieces up in piece order
  auto end_item = [&]() {
    float tot[MV];
#pragma unroll
    for (int v = 0; v < MV; ++v) {
      tot[v] = row_sum(acc[v]);
      acc[v] = 0.f;
    }
    if (si.P == 1) {
      stage_rows(F, si.s, it.mi, it.u, lane, tot);
      return;
    }
    // pieces of unit j of the stage are items j P .. j P + P - 1
    const int j = ufl((int)(((uint32_t)i * si.inv_p) >> 16));
    const int rb = si.s % S::kRowBufs;
    if (lane < kUnitRows) {
#pragma unroll
      for (int v = 0; v < MV; ++v) *(volatile Q4_LDS float*)&F.parts[rb][i][lane][v] = tot[v];
    }
    compiler_fence();
    uint32_t old = 0;
    if (lane == 0) old = lds_add_rtn(&F.pieces_done[rb][j], 1u);
    old = (uint32_t)__builtin_amdgcn_readfirstlane((int)old);
    if (old == (uint32_t)si.P - 1u) {
      compiler_fence();
      float sum[MV];
#pragma unroll
      for (int v = 0; v < MV; ++v) sum[v] = 0.f;
      for (int p = 0; p < si.P; ++p) {
#pragma unroll
        for (int v = 0; v < MV; ++v) sum[v] += *(volatile Q4_LDS float*)&F.parts[rb][j * si.P + p][lane & 3][v];
      }
      stage_rows(F, si.s, it.mi, it.u, lane, sum);
      if (lane == 0) lds_put(&F.pieces_done[rb][j], 0u);
    }
  };
  // consume the slot in d (the current item's next chunk), then refill d
  // with the slot kRegRing further on
  // (an item that ends the wave's part of a stage is closed and the stage
  // counted done before the refill, so that the block's last wave reports a
  // short stage without first walking the load cursor to its next item; the
  // next stage is entered after the refill, so that the refill is in flight
  // during the stage barrier)
  auto step = [&](Slot& d) {
    // lanes past G (only in the last chunk of a ragged row) weigh zero
    const bool live = !si.ragged || gch + col < si.G;
    float term[MV];
    slot_terms<MV>(d, x0 + gch * kXWordsPerGroup, S::kVecWords, vown, live, term);
#pragma unroll
    for (int v = 0; v < MV; ++v) acc[v] += term[v];
    gch = ufl(gch + kChunkGroups);
    left = ufl(left - 1);
    const bool item_end = left == 0;
    uint32_t code = 0;
    int s_next = 0;
    if (item_end) {
      end_item();
      s_next = end_stage_early(code);
    }
    lc_load(lc, d, lane, L, F, num_stages, cw);
    if (item_end) next_item(code, s_next);
  };

  stage_info(si, L, 0);
  enter_stage();
  {
    const uint32_t code = lds_get(&F.queue[cw][qt % kQueueLen]);
    qt = (uint32_t)ufl((int)(qt + 1u));
    const int s_next = code == kQueueEnd ? num_stages : (int)(code >> 16);
    // (stages before the wave's first item: entered and counted done in turn)
    while (si.s < s_next) {
      compiler_fence();
      if (lane == 0) lds_add(&F.done[si.s % kDoneSlots], 1u);
      wake_block();
      if (si.s + 1 >= num_stages) {
        si.s = num_stages;
        break;
      }
      stage_info(si, L, si.s + 1);
      enter_stage();
    }
    if (si.s < num_stages) {
      i = (int)(code & 0xFFFFu);
      decode_item(si, i, it);
      left = ufl(it.cb - it.ca);
      gch = ufl(it.ca * kChunkGroups);
    }
  }
  // (the steps are written out, with one exit test after the last: every
  // path round the loop then issues the same loads in the same order, which
  // keeps the compiler's count of loads in flight exact. Steps past the
  // wave's last item change nothing: left never returns to zero, the loads
  // read empty ranges and the x reads stay inside the last stage's buffer.)
  while (true) {
    step(d[0]);
    step(d[1]);
    step(d[2]);
#if Q4_CHAIN_REG_RING >= 6
    step(d[3]);
    step(d[4]);
#endif
#if Q4_CHAIN_REG_RING >= 8
    step(d[5]);
    step(d[6]);
#endif
#if Q4_CHAIN_REG_RING >= 12
    step(d[7]);
    step(d[8]);
    step(d[9]);
    step(d[10]);
#endif
#if Q4_CHAIN_REG_RING >= 16
    step(d[11]);
    step(d[12]);
    step(d[13]);
    step(d[14]);
#endif
    step(d[kRegRing - 1]);
    if (si.s >= num_stages || stop) break;
  }
  if (stop && lds_get(&F.abort) == 0u) compute_fail(F);
}

template <int MV, bool OUT_F32>
__device__ __forceinline__ void compute_run(int num_stages, int cw, ChainLds<MV>& L, ChainFlags<MV>& F,
                                            uint32_t* ws) {
  if constexpr (MV == 1) {
    if (lds_get(&F.any_norm) != 0u)
      compute_body<MV, OUT_F32, true>(num_stages, cw, L, F, ws);
    else
      compute_body<MV, OUT_F32, false>(num_stages, cw, L, F, ws);
  } else {
    compute_body<MV, OUT_F32, false>(num_stages, cw, L, F, ws);
  }
  // loads still in flight (the refills past the wave's last slot, or an
  // aborted wave's) complete before the wave ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---------------------------------------------------------------- service

// A stage's activations are staged into an LDS buffer re-paired, with group
// sums; groups past G up to 16 CH are zero. The service wave stages
// activations no stage writes (the compute waves stage the others, after the
// barrier: fill_x_share), kXBatch groups per lane at a time: xb_issue starts a batch's loads into registers, xb_store
// writes the batch to LDS once they are in (MV activation rows [MV][k] in
// memory; row v goes to dst_buf + v * kVecWords).
constexpr int kXBatch = 3;
struct XBatch {
  q4_u32x4 q[kXBatch][4];
};
template <int MV>
__device__ __forceinline__ int xb_row(int e, int gpad) {
  int v = 0;
#pragma unroll
  for (int r = 1; r < MV; ++r) v += e >= r * gpad ? 1 : 0;
  return v;
}
// Buffer loads with 32-bit offsets (the base stays in scalar registers); a
// lane past the rows' groups reads zeros.
template <int MV>
__device__ __forceinline__ void xb_issue(const Geo& g, const void* x, int base, XBatch& xb) {
  const int lane = threadIdx.x & 63;
  const int gpad = kChunkGroups * g.CH;
  const int total = MV * gpad;
  const __amdgpu_buffer_rsrc_t rx = byte_range(x, (uint32_t)(MV * g.G * 64));
#pragma unroll
  for (int b = 0; b < kXBatch; ++b) {
    if (base + 64 * b >= total) break;  // (no load for a batch past the rows' groups)
    const int e = base + 64 * b + lane;
    const int v = xb_row<MV>(e, gpad);
    const int grp = e - v * gpad;
    const uint32_t off = (e < total && grp < g.G) ? (uint32_t)((v * g.G + grp) * 64) : 0xFFFFFF00u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xb.q[b][j] = __builtin_bit_cast(q4_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16 * j), 0, 0));
  }
}
template <int MV>
__device__ __forceinline__ void xb_store(const Geo& g, int base, const XBatch& xb, uint32_t* dst_buf) {
  const int lane = threadIdx.x & 63;
  const int gpad = kChunkGroups * g.CH;
  const int total = MV * gpad;
#pragma unroll
  for (int b = 0; b < kXBatch; ++b) {
    if (base + 64 * b >= total) break;
    const int e = base + 64 * b + lane;
    const int v = xb_row<MV>(e, gpad);
    const int grp = e - v * gpad;
    if (e < total) {
      // (groups past G are zero)
      uint32_t* dst = dst_buf + v * ChainShape<MV>::kVecWords + grp * kXWordsPerGroup;
      float xs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 e4 = make_uint4(xb.q[b][j].x, xb.q[b][j].y, xb.q[b][j].z, xb.q[b][j].w);
        uint32_t p02, p46, p13, p57;
        x_to_pairs(e4, p02, p46, p13, p57);
        *reinterpret_cast<uint4*>(dst + 4 * j) = make_uint4(p02, p46, p13, p57);
        xs += x_sum8(e4);
      }
      dst[16] = __float_as_uint(xs);
    }
  }
}
// the batches from group index `from` on, then wait for the LDS writes
template <int MV>
__device__ __forceinline__ void service_load_x(const Geo& g, const void* x, uint32_t* dst_buf, int from = 0) {
  const int total = MV * kChunkGroups * g.CH;
  for (int base = from; base < total; base += 64 * kXBatch) {
    XBatch xb;
    xb_issue<MV>(g, x, base, xb);
    xb_store<MV>(g, base, xb, dst_buf);
  }
  lds_wait();
}

struct GridSync {
  uint32_t xcc;
  uint32_t per;      // blocks on this XCD
  uint32_t present;  // mask of XCDs that hold blocks
  uint32_t epoch;
  uint32_t nxcc;
};

template <int MV>
__device__ __forceinline__ bool service_fail(uint32_t* ws, ChainFlags<MV>& F, uint32_t code) {
  if ((threadIdx.x & 63) == 0) {
    coh_store(ws + kWsStatus, code);
    lds_put(&F.abort, 1u);
  }
  wake_block();
  return false;
}

// Two grid barriers; the plan names the one its launches use (the encoder
// picks by stage size). Each keeps its own words of the workspace, which run
// on across launches of that kind.
//  1. Blocks of one XCD count arrivals with an L2 atomic; the XCD's last
//     arrival stores the XCD's epoch flag device-coherently; every block polls
//     the flags (one line). Best for large stages (the temporal step's).
//  2. Each XCD has a 64-bit arrival counter (in its own 128-byte line),
//     incremented with a posted system-scope add that no block waits for;
//     every block polls the counters with one lane per XCD. No arrival waits
//     for an atomic's round trip, which pays where stages are short (the
//     Depformer's: 7% faster per frame, 6% slower on the temporal step).
constexpr int kBarrierL2Flags = 1;
constexpr int kBarrierCounters = 2;
__device__ __forceinline__ uint64_t* xcd_counter(uint32_t* ws, uint32_t x) {
  return reinterpret_cast<uint64_t*>(ws + kWsXcnt2 + 32 * x);
}

// Start of a launch. The hardware deals the blocks of a launch round-robin
// over the device's nxcc XCDs, so block b runs on XCD b % nxcc (checked: a
// block on any other XCD reports status 3). The barrier's words continue from
// earlier launches of its kind on this workspace:
//  1. the XCD's flag holds the last completed epoch, and it cannot move before
//     every block of this XCD has arrived at the first barrier of this
//     launch, so every block of the XCD reads the same value here;
//  2. every such launch has the same blocks per XCD and completes all its
//     barriers, so the counter of XCD x holds per_x * E arrivals, E the
//     barriers completed so far, plus fewer than per_x arrivals of this
//     launch's first barrier (which cannot complete before this block
//     arrives): E is the counter divided by per_x.
template <int BAR, int MV>
__device__ __forceinline__ bool service_start(uint32_t* ws, ChainFlags<MV>& F, GridSync& gs, uint32_t nxcc) {
  const uint32_t nb = gridDim.x;
  gs.xcc = blockIdx.x % nxcc;
  if (xcc_id() != gs.xcc) return service_fail(ws, F, 3u);
  gs.per = nb / nxcc + (gs.xcc < nb % nxcc ? 1u : 0u);
  gs.present = nxcc >= 32u ? 0xFFFFFFFFu : ((1u << (nxcc < nb ? nxcc : nb)) - 1u);
  gs.nxcc = nxcc;
  if constexpr (BAR == kBarrierCounters)
    gs.epoch = (uint32_t)(coh_load64(xcd_counter(ws, gs.xcc)) / gs.per);
  else
    gs.epoch = coh_load(ws + kWsGflag + gs.xcc);
  return true;
}

// Grid barrier in two halves: work issued between arrive and wait overlaps
// the wait.
template <int BAR>
__device__ __forceinline__ void service_arrive(uint32_t* ws, GridSync& gs) {
  const int lane = threadIdx.x & 63;
  const uint32_t e = ++gs.epoch;
  if constexpr (BAR == kBarrierCounters) {
    if (lane == 0) coh_add64_post(xcd_counter(ws, gs.xcc), 1u);
  } else {
    uint32_t old = 0;
    if (lane == 0) old = l2_add(ws + kWsXcnt + 32 * gs.xcc, 1u);
    old = __shfl(old, 0);
    if ((old + 1u) % gs.per == 0u && lane == 0) coh_store(ws + kWsGflag + gs.xcc, e);
  }
}
template <int BAR, int MV>
__device__ __forceinline__ bool service_wait(uint32_t* ws, ChainFlags<MV>& F, GridSync& gs) {
  const int lane = threadIdx.x & 63;
  const uint32_t e = gs.epoch;
  const bool watch = lane < kMaxXcc && ((gs.present >> lane) & 1u);
  const uint32_t nb = gridDim.x;
  const uint64_t per_x = nb / gs.nxcc + ((uint32_t)lane < nb % gs.nxcc ? 1u : 0u);
  const uint64_t target = per_x * (uint64_t)e;
  uint32_t spins = 0;
  while (true) {
    bool mine = true;
    if (watch) {
      if constexpr (BAR == kBarrierCounters)
        mine = coh_load64(xcd_counter(ws, (uint32_t)lane)) >= target;
      else
        mine = (int)(coh_load(ws + kWsGflag + lane) - e) >= 0;
    }
    if (__all(mine)) break;
    if (++spins > kSpinLimit || coh_load(ws + kWsStatus) != 0u) return service_fail(ws, F, 1u);
  }
  return true;
}

// Store stage s's rows from LDS: entry (mi, u, r) is row 4 unit + r of the
// stage's matrix mi, for the block's local unit u.
// With MV activation rows the outputs are [MV][n].
// A gated stage stores silu(matrix 0) * matrix 1 as matrix 0's output; a
// matrix with a residual adds it (staged by service_load_res) before the one
// rounding.
template <int MV, bool OUT_F32>
__device__ __forceinline__ void service_store(const ChainLds<MV>& L, int s, ChainFlags<MV>& F) {
  const int lane = threadIdx.x & 63;
  const Geo g = geo_of(L.st[s]);
  const bool gated = (stage_flags(L, s) & kStageGated) != 0;
  for (int mi = 0; mi < (gated ? 1 : g.num_mats); ++mi) {
    const MatRec& mr = L.mt[g.mat_begin + mi];
    const int n = ufl(mr.n);
    const BlockRange br = {ufl(L.st[s].U0[mi]), ufl(L.st[s].U[mi])};  // (block_range of the unit count)
    void* y = ufl_ptr(mr.y);
    const void* res = ufl_ptr(mr.residual);
    for (int e = lane; e < br.count * kUnitRows; e += 64) {
      const int u = e >> 2, r = e & 3;
      const int orow = unit_of(br, u) * kUnitRows + r;
      if (orow < n) {
#pragma unroll
        for (int v = 0; v < MV; ++v) {
          float val = *(volatile Q4_LDS float*)&F.out[s % ChainShape<MV>::kRowBufs][mi][u][r][v];
          if (gated) {
            const float up = *(volatile Q4_LDS float*)&F.out[s % ChainShape<MV>::kRowBufs][1][u][r][v];
            val = val / (1.0f + expf(-val)) * up;
          }
          if (res) val += *(volatile Q4_LDS float*)&F.res[s % ChainShape<MV>::kRowBufs][mi][u][r][v];
          if constexpr (OUT_F32) {
            coh_store(static_cast<uint32_t*>(y) + (int64_t)v * n + orow, __float_as_uint(val));
          } else {
            coh_store16(static_cast<uint16_t*>(y) + (int64_t)v * n + orow, f32_to_bf16_rne(val));
          }
        }
      }
    }
  }
}

// The residuals of the rows this block stores in stage s, into LDS, as soon
// as the stage starts (device-coherent loads: a stage before s that writes
// them has made its outputs visible before a grid barrier that precedes s; a
// later stage that overwrites them is separated from s by a barrier), so that
// the stores at the end of the stage do not wait for them.
template <int MV, bool OUT_F32>
__device__ __forceinline__ void service_load_res(const ChainLds<MV>& L, int s, ChainFlags<MV>& F) {
  const int lane = threadIdx.x & 63;
  const Geo g = geo_of(L.st[s]);
  const bool gated = (stage_flags(L, s) & kStageGated) != 0;
  for (int mi = 0; mi < (gated ? 1 : g.num_mats); ++mi) {
    const MatRec& mr = L.mt[g.mat_begin + mi];
    const void* res = ufl_ptr(mr.residual);
    if (!res) continue;
    const int n = ufl(mr.n);
    const BlockRange br = {ufl(L.st[s].U0[mi]), ufl(L.st[s].U[mi])};  // (block_range of the unit count)
    for (int e = lane; e < br.count * kUnitRows; e += 64) {
      const int u = e >> 2, r = e & 3;
      const int orow = unit_of(br, u) * kUnitRows + r;
      if (orow < n) {
#pragma unroll
        for (int v = 0; v < MV; ++v) {
          float val;
          if constexpr (OUT_F32)
            val = __uint_as_float(coh_load(static_cast<const uint32_t*>(res) + (int64_t)v * n + orow));
          else
            val = bf16_to_f32(coh_load16(static_cast<const uint16_t*>(res) + (int64_t)v * n + orow));
          *(volatile Q4_LDS float*)&F.res[s % ChainShape<MV>::kRowBufs][mi][u][r][v] = val;
        }
      }
    }
  }
}

template <int MV, bool OUT_F32, int BAR>
__device__ __forceinline__ void service_run(int num_stages, ChainLds<MV>& L, ChainFlags<MV>& F, uint32_t* ws,
                                            uint32_t nxcc) {
  using S = ChainShape<MV>;
  constexpr bool kAhead = S::kXBuffers == 2;  // activations staged ahead into the arena
  GridSync gs;
  if (!service_start<BAR>(ws, F, gs, nxcc)) return;
  int fills = 0;  // stagings shared with the compute waves so far
  // (a normalized stage's activations are always staged by the compute
  // waves together: the norm needs every group's sum of squares)
  auto wait_filled = [&]() {
    uint32_t fspins = 0;
    while ((int)(lds_get(&F.x_filled) - (uint32_t)(kComputeWaves * fills)) < 0) {
      nap();
      if (lds_get(&F.abort) != 0u || ++fspins > kSpinLimit) {
        service_fail(ws, F, 1u);
        return false;
      }
    }
    return true;
  };
  // This wave stages the activations no stage writes (prefetchable), except a
  // normalized stage's; the compute waves stage the others together when the
  // stage opens. A prefetchable stage that needs no grid barrier is published
  // as soon as its activations are in LDS and every stage before it is
  // published (early): the block's waves that have finished the stages
  // before it go on at once, while the others finish.
  auto prefetchable = [&](int t) {
    return kAhead && t < num_stages && !(stage_flags(L, t) & (kStageXInternal | kStageNorm));
  };
  auto early = [&](int t) { return prefetchable(t) && (stage_flags(L, t) & kStageNoBarrier) != 0; };
  auto publish = [&](int t) {
    compiler_fence();
    if ((threadIdx.x & 63) == 0) lds_puti(&F.x_stage, t);
    wake_block();
    service_load_res<MV, OUT_F32>(L, t, F);
  };
  auto stage = [&](int t) { service_load_x<MV>(geo_of(L.st[t]), stage_x(L, t), stage_xbuf(L, t)); };
  if (stage_flags(L, 0) & kStageNorm) {
    if ((threadIdx.x & 63) == 0) lds_puti(&F.x_fill, 0);
    wake_block();
    ++fills;
    if (!wait_filled()) return;
  } else {
    stage(0);
  }
  int published = 0;  // the last stage published
  int staged = 0;     // the last stage whose activations are in LDS (or staged when it opens)
  publish(0);
  // After every compute wave has finished stage done_s and its rows are
  // stored: publish what is staged and needs no barrier, then stage the next
  // prefetchable stages whose arena region no unfinished stage uses and whose
  // row buffer is free (stage t - kRowBufs stored), publishing as it goes.
  auto run_ahead = [&](int done_s) {
    while (published < staged && early(published + 1)) publish(++published);
    while (staged + 1 < num_stages && prefetchable(staged + 1) && ufl(L.st[staged + 1].xwait) <= done_s &&
           staged + 1 - S::kRowBufs <= done_s) {
      stage(++staged);
      if (published == staged - 1 && early(staged)) publish(++published);
    }
  };
  run_ahead(-1);
  // Outputs a later stage reads, stored since the last grid barrier: the next
  // barrier waits for their stores before arriving.
  bool unsynced = false;
  for (int s = 0; s < num_stages; ++s) {
    uint32_t spins = 0;
    // every compute wave has finished stage s (no wave runs kDoneSlots
    // stages ahead of the slowest, so the count of stage s's slot holds no
    // completions of later stages yet)
    while ((int)(lds_get(&F.done[s % kDoneSlots]) - (uint32_t)(kComputeWaves * (s / kDoneSlots + 1))) < 0) {
      nap();
      if (lds_get(&F.abort) != 0u || ++spins > kSpinLimit) {
        service_fail(ws, F, 1u);
        return;
      }
    }
    compiler_fence();
    if (s + 1 >= num_stages) {
      service_store<MV, OUT_F32>(L, s, F);
      break;
    }
    const bool sync_out = (stage_flags(L, s) & kStageSyncOut) != 0;
    // Stage s + 1 runs already (published early: no barrier between), or it
    // waits for this transition: a grid barrier, or activations staged by the
    // compute waves together. Stage s + 1 needs no grid barrier where nothing
    // it reads or writes depends on the stages since the last one (the
    // encoder checks).
    const bool ahead = published > s;
    const bool barrier = !ahead && (stage_flags(L, s + 1) & kStageNoBarrier) == 0;
    if (!barrier) {
      service_store<MV, OUT_F32>(L, s, F);
      unsynced = unsynced || sync_out;
    } else if (sync_out || unsynced) {
      // outputs read by a later stage must be visible before the barrier
      service_store<MV, OUT_F32>(L, s, F);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      service_arrive<BAR>(ws, gs);
      unsynced = false;
    } else {
      // arrive first: the stores then overlap the wait instead of delaying
      // the arrival
      service_arrive<BAR>(ws, gs);
      service_store<MV, OUT_F32>(L, s, F);
    }
    if (!ahead) {
      const bool internal = (stage_flags(L, s + 1) & kStageXInternal) != 0;
      const bool norm = (stage_flags(L, s + 1) & kStageNorm) != 0;
      // The compute waves stage the next activations together where they
      // would otherwise wait for this wave to do it alone: with one buffer
      // (the block's compute waves have all finished stage s, so it is free),
      // for activations written in the chain (after the barrier), and for a
      // normalized stage.
      const bool shared_fill = !kAhead || internal || norm;
      compiler_fence();
      if (shared_fill && !internal) {
        if ((threadIdx.x & 63) == 0) lds_puti(&F.x_fill, s + 1);
        wake_block();
      }
      // (activations this wave stages, not yet staged because their region
      // was in use until now: loaded while the barrier completes)
      if (!shared_fill && staged < s + 1) stage(staged = s + 1);
      if (barrier && !service_wait<BAR>(ws, F, gs)) return;
      if (shared_fill) {
        if (internal) {
          if ((threadIdx.x & 63) == 0) lds_puti(&F.x_fill, s + 1);
          wake_block();
        }
        ++fills;
        if (!wait_filled()) return;
      }
      publish(published = s + 1);
      if (staged < s + 1) staged = s + 1;
    }
    run_ahead(s);
  }
}

// ---------------------------------------------------------------- kernel

template <int MV, bool OUT_F32>
__global__ void __launch_bounds__(64 * kChainWaves) __attribute__((amdgpu_waves_per_eu((kChainWaves + 3) / 4, (kChainWaves + 3) / 4)))
chain_kernel(const ChainHeader* __restrict__ plan, uint32_t* __restrict__ ws, uint32_t nxcc) {
  using S = ChainShape<MV>;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  __shared__ ChainFlags<MV> F;
  ChainLds<MV>& L = *reinterpret_cast<ChainLds<MV>*>(lds_raw);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  if (threadIdx.x < ChainShape<MV>::kRowBufs * kSplitUnits) (&F.pieces_done[0][0])[threadIdx.x] = 0u;
  for (int e = threadIdx.x; e < S::kTabStages; e += blockDim.x) F.claim[e] = 0u;
  if (threadIdx.x == 0) {
    for (int j = 0; j < kDoneSlots; ++j) F.done[j] = 0u;
    F.x_stage = -1;
    F.x_fill = -1;
    F.x_filled = 0u;
    F.abort = 0u;
    F.misfit = 0u;
    F.norm_cnt = 0u;
    F.any_norm = 0u;
    // the plan must be one this library encoded, and fit the LDS tables
    const int ns = cload(&plan->num_stages), nm = cload(&plan->num_mats);
    const bool ok = coh_load(ws + kWsStatus) == 0u && cload(&plan->magic) == kChainMagic && ns > 0 &&
                    ns <= S::kTabStages && nm > 0 && nm <= S::kTabMats && cload(&plan->rows) == MV &&
                    (cload(&plan->barrier) == kBarrierL2Flags || cload(&plan->barrier) == kBarrierCounters) &&
                    gridDim.x <= (unsigned)kChainMaxBlocks && nxcc >= 1u && nxcc <= (unsigned)kMaxXcc;
    F.go = ok ? 1u : 0u;
    if (!ok && blockIdx.x == 0 && coh_load(ws + kWsStatus) == 0u) coh_store(ws + kWsStatus, 2u);
  }
  __syncthreads();
  if (F.go == 0u) return;
  const int num_stages = cload(&plan->num_stages);
  const int num_mats = cload(&plan->num_mats);
  const ChainStageDesc* stages = reinterpret_cast<const ChainStageDesc*>(plan + 1);
  const ChainMatDesc* mats = reinterpret_cast<const ChainMatDesc*>(stages + num_stages);
  // the plan into LDS, one lane per stage and per matrix
  for (int s = threadIdx.x; s < num_stages; s += blockDim.x) {
    if (!build_stage_rec<MV>(L.st[s], stages + s, mats)) lds_put(&F.misfit, 1u);
    if (L.st[s].flags & kStageNorm) lds_put(&F.any_norm, 1u);
  }
  for (int m = threadIdx.x; m < num_mats; m += blockDim.x) {
    MatRec r;
    r.packed = mats[m].packed;
    r.scales = mats[m].scales;
    r.biases = mats[m].biases;
    r.y = mats[m].y;
    r.n = mats[m].n;
    r.pad = 0;
    r.residual = mats[m].residual;
    L.mt[m] = r;
  }
  __syncthreads();
  if (F.misfit != 0u) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && coh_load(ws + kWsStatus) == 0u) coh_store(ws + kWsStatus, 2u);
    return;
  }

  if (wave == kServiceWave) {
    if (cload(&plan->barrier) == kBarrierCounters)
      service_run<MV, OUT_F32, kBarrierCounters>(num_stages, L, F, ws, nxcc);
    else
      service_run<MV, OUT_F32, kBarrierL2Flags>(num_stages, L, F, ws, nxcc);
  } else {
    compute_run<MV, OUT_F32>(num_stages, wave - 1, L, F, ws);
  }
}

// Set-up and read-out of a chain workspace that lives in a device-global
// array (the entry point for callers that cannot allocate): clear its words
// before a launch, and copy the launch's status word out after it.
__global__ void __launch_bounds__(256) chain_ws_clear_kernel(uint32_t* __restrict__ ws, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) ws[i] = 0u;
}
__global__ void __launch_bounds__(64) chain_ws_status_kernel(const uint32_t* __restrict__ ws,
                                                             uint32_t* __restrict__ status_out) {
  if (threadIdx.x == 0) status_out[0] = coh_load(ws + kWsStatus);
}

}  // namespace q4k
