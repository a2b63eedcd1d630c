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
// One launch runs the whole chain with one block per compute unit. The waves
// have two roles that meet only through LDS counters:
//  - waves 1..kComputeWaves compute. Each owns a ring of kRingSlots slot
//    buffers in LDS; a slot is 64 lanes x one 16-byte group of codes plus
//    those 64 groups' scales and biases. A wave walks its share of every
//    stage's rows in chain order and keeps the next kRingSlots slots in
//    flight with loads that write straight into its ring, so its own vector
//    memory counter says when a slot has landed. It forms the dequantized dot
//    products with the stage's activations (in LDS), reduces each row over its
//    lanes and stores the row's output. The loads run ahead across stage
//    boundaries: the first slots of stage s+1 stream in while the grid
//    synchronises after stage s.
//  - wave 0, the service wave, synchronises the grid between stages and
//    stages activations into LDS (double buffered: the next stage's
//    activations are fetched during the current stage unless an earlier stage
//    of the chain writes them).
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
#define Q4_CHAIN_COMPUTE_WAVES 12
#endif
#ifndef Q4_CHAIN_RING_SLOTS
#define Q4_CHAIN_RING_SLOTS 6
#endif
constexpr int kServiceWave = 0;
constexpr int kComputeWaves = Q4_CHAIN_COMPUTE_WAVES;  // waves 1..kComputeWaves
constexpr int kChainWaves = 1 + kComputeWaves;
constexpr int kRingSlots = Q4_CHAIN_RING_SLOTS;  // slot buffers per compute wave = slots in flight ahead of it
constexpr int kSlotBytes = 1280;    // 64 lanes x 16 B codes, then 64 bf16 scales, then 64 bf16 biases
constexpr int kMaxMatsPerStage = 4;
constexpr int kChainMaxGroups = 384;  // k <= 12288
constexpr int kChainMaxCH = 12;
constexpr int kXWordsPerGroup = 20;   // 16 re-paired words + sum + pad (bank spread)
constexpr int kChainMaxBlocks = 1024;
constexpr int kMaxXcc = 16;
constexpr uint32_t kSpinLimit = 1u << 22;
static_assert(kChainWaves <= 16 && kRingSlots >= 2 && 2 * kRingSlots <= 63, "chain shape");

struct alignas(16) ChainHeader {
  uint32_t magic;
  int32_t num_stages;
  int32_t num_mats;
  int32_t out_f32;
  int32_t plan_bytes;
  int32_t pad[11];
};
struct alignas(16) ChainStageDesc {
  const uint16_t* x;
  int32_t G;             // groups of 32 inputs
  int32_t c_log2;        // lanes per row = 1 << c_log2
  int32_t CH;            // chunks per row: ceil(G / lanes per row)
  int32_t num_mats;
  int32_t mat_begin;
  int32_t x_internal;    // x is written by an earlier stage of the chain
  int32_t sync_outputs;  // a later stage reads this stage's outputs
  int32_t pad[7];
};
struct alignas(16) ChainMatDesc {
  const uint32_t* packed;
  const uint16_t* scales;
  const uint16_t* biases;
  void* y;
  int32_t n;
  int32_t pad[3];
};
static_assert(sizeof(ChainHeader) == 64 && sizeof(ChainStageDesc) == 64 && sizeof(ChainMatDesc) == 48,
              "descriptor sizes");

// Workspace words: status on its own line; per XCD an arrival counter (L2
// scope, one 128-byte line each); the XCDs' flags (device scope, one line).
constexpr int kWsStatus = 0;  // 0 ok, 1 wait timed out, 2 bad plan, 3 block not on the expected XCD
constexpr int kWsXcnt = 64;                       // + 32 * xcc
constexpr int kWsGflag = kWsXcnt + 32 * kMaxXcc;  // + xcc
constexpr int kWsWords = kWsGflag + 64;

// Plan reads go through the constant address space, so that (at wave-uniform
// addresses) they become scalar loads and never enter the vector memory
// pipeline that streams the weights.
#define Q4_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ T cload(const T* p) {
  return *(const Q4_CONST T*)p;
}
// Loads through plan pointers are issued as global (not flat) accesses, which
// count only in the vector-memory counter.
#define Q4_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
  return *(const Q4_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ T gload_off(const unsigned char* base, uint32_t off) {
  return gload(reinterpret_cast<const T*>(base + off));
}

// device-coherent accesses (all XCDs)
__device__ __forceinline__ uint32_t coh_load(const uint32_t* p) {
  return __hip_atomic_load((const Q4_GLOBAL uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t coh_load64(const uint64_t* p) {
  return __hip_atomic_load((const Q4_GLOBAL uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store((Q4_GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store16(uint16_t* p, uint16_t v) {
  __hip_atomic_store((Q4_GLOBAL uint16_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Shared memory: activations and slot rings (dynamic LDS) and the flag words
// that connect the roles (a separate static object).
struct ChainLds {
  uint32_t x[2][kChainMaxGroups * kXWordsPerGroup];          // activations, double buffered
  unsigned char ring[kComputeWaves][kRingSlots][kSlotBytes];  // slot buffers
};
struct ChainFlags {
  uint32_t done_total;               // stage completions of all compute waves
  int32_t x_stage;                   // last stage whose activations are in LDS
  uint32_t abort;
  uint32_t go;
};

// LDS flag words, accessed through explicit LDS pointers (a volatile access
// through a generic pointer would become a flat access, which also counts in
// the vector-memory counter).
#define Q4_LDS __attribute__((address_space(3)))
__device__ __forceinline__ uint32_t lds_get(const uint32_t* p) { return *(const volatile Q4_LDS uint32_t*)p; }
__device__ __forceinline__ int32_t lds_geti(const int32_t* p) { return *(const volatile Q4_LDS int32_t*)p; }
__device__ __forceinline__ void lds_put(uint32_t* p, uint32_t v) { *(volatile Q4_LDS uint32_t*)p = v; }
__device__ __forceinline__ void lds_puti(int32_t* p, int32_t v) { *(volatile Q4_LDS int32_t*)p = v; }
__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add((Q4_LDS uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ int ufl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Stage geometry (wave-uniform).
struct Geo {
  int G, clog, LPR, RPI, CH, num_mats, mat_begin;
};
__device__ __forceinline__ Geo geo_of(const ChainStageDesc* sd) {
  Geo g;
  g.G = cload(&sd->G);
  g.clog = cload(&sd->c_log2);
  g.LPR = 1 << g.clog;
  g.RPI = 64 >> g.clog;
  g.CH = cload(&sd->CH);
  g.num_mats = cload(&sd->num_mats);
  g.mat_begin = cload(&sd->mat_begin);
  return g;
}

// Units (RPI consecutive rows) of a matrix: block b owns a contiguous range
// (sizes differ by at most one unit over the grid), and deals it round-robin
// to its compute waves: local unit i goes to compute wave i % kComputeWaves.
struct BlockRange {
  int u0, count;
};
__device__ __forceinline__ BlockRange block_range(int nunits) {
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  const int per = nunits / nb, rem = nunits - per * nb;
  BlockRange r;
  r.u0 = b * per + (b < rem ? b : rem);
  r.count = per + (b < rem ? 1 : 0);
  return r;
}

// s_waitcnt immediate that waits for the vector-memory counter only
constexpr int vmcnt_imm(int n) { return 0xF70 | (n & 15) | (((n >> 4) & 3) << 14); }

// ---------------------------------------------------------------- compute

// Sum over the LPR lanes of a row slot with DPP adds; the total lands in the
// slot's last lane (lane % LPR == LPR - 1).
__device__ __forceinline__ float dpp_sum(float v, int LPR) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));  // xor 1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  // xor 2
  if (LPR >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half-row mirror
  if (LPR >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  if (LPR >= 32) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row bcast 15
  if (LPR >= 64) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row bcast 31
  return v;
}

// One slot's operands, read from LDS: the lane's 16 bytes of codes, its
// group's bf16 scale and bias (as fp32 bit patterns), and the group's
// re-paired activations and their sum.
struct SlotRegs {
  uint4 w;
  uint32_t sv, bv;
  uint4 x0, x1, x2, x3;
  uint32_t xs;
};
__device__ __forceinline__ void read_slot(const unsigned char* slot, const uint32_t* xg, int lane, uint32_t sb_off,
                                          SlotRegs& r) {
  r.w = *reinterpret_cast<const uint4*>(slot + lane * 16);
  r.sv = (uint32_t)*reinterpret_cast<const uint16_t*>(slot + 1024 + sb_off) << 16;
  r.bv = (uint32_t)*reinterpret_cast<const uint16_t*>(slot + 1152 + sb_off) << 16;
  r.x0 = *reinterpret_cast<const uint4*>(xg + 0);
  r.x1 = *reinterpret_cast<const uint4*>(xg + 4);
  r.x2 = *reinterpret_cast<const uint4*>(xg + 8);
  r.x3 = *reinterpret_cast<const uint4*>(xg + 12);
  r.xs = xg[16];
}
__device__ __forceinline__ float slot_dot(const SlotRegs& r, bool live, float acc) {
  uint32_t xp[16];
  xp[0] = r.x0.x; xp[1] = r.x0.y; xp[2] = r.x0.z; xp[3] = r.x0.w;
  xp[4] = r.x1.x; xp[5] = r.x1.y; xp[6] = r.x1.z; xp[7] = r.x1.w;
  xp[8] = r.x2.x; xp[9] = r.x2.y; xp[10] = r.x2.z; xp[11] = r.x2.w;
  xp[12] = r.x3.x; xp[13] = r.x3.y; xp[14] = r.x3.z; xp[15] = r.x3.w;
  const float sc = __uint_as_float(live ? r.sv : 0u);
  const float bi = __uint_as_float(live ? r.bv : 0u);
  return fmaf(sc, group_dot(r.w, xp), fmaf(bi, __uint_as_float(r.xs), acc));
}

__device__ __forceinline__ void compute_fail(uint32_t* ws, ChainFlags& F) {
  if ((threadIdx.x & 63) == 0) {
    coh_store(ws + kWsStatus, 1u);
    lds_put(&F.abort, 1u);
  }
}

// Direct-to-LDS load of 16 bytes per active lane: lane t's bytes land at LDS
// byte address lds + 16 t. The LDS base goes in M0, which the compiler never
// allocates. The load is issued from assembly so that the compiler does not
// hold later LDS reads behind it; every read of a slot buffer is preceded by
// an explicit wait on the vector memory counter instead.
__device__ __forceinline__ void dma16_s(const unsigned char* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma16_v(const unsigned char* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(lds) : "memory");
}

// The next slot a compute wave loads: its position in chain order (stage,
// matrix, the wave's local unit, chunk), the unit's addresses and the stage's
// per-lane offsets. All fields but the lane offsets are wave-uniform.
struct LoadCursor {
  int s, m, m_end, i, count, ch, CH, LPR, clog;
  uint32_t unit_w, unit_s;           // bytes of codes / of scales per unit
  const unsigned char *pw, *ps, *pb;  // current unit's codes, scales, biases
  uint32_t lw, lw_last, ls, ls_last;  // lane offsets (chunk 0 / last chunk)
};

// Slot loads: 64 lanes x 16 bytes of codes, and 16 lanes x 16 bytes holding
// the slot's 64 bf16 scales (lanes 0..7) and biases (lanes 8..15) (G % 8 == 0,
// so a 16-byte piece never straddles a row end). Lane (srow, c) reads group
// (srow, ch*LPR + c) of its unit; the last chunk carries its column in the
// offset, so that in a ragged row (LPR*CH > G) lanes past G read group 0 of
// their own row instead (they are given zero weight).
__device__ __forceinline__ void lc_stage(LoadCursor& lc, const ChainStageDesc* stages, int lane) {
  const Geo g = geo_of(stages + lc.s);
  lc.CH = g.CH;
  lc.LPR = g.LPR;
  lc.clog = g.clog;
  lc.unit_w = (uint32_t)(g.RPI * g.G) * 16u;
  lc.unit_s = (uint32_t)(g.RPI * g.G) * 2u;
  const int c = lane & (g.LPR - 1);
  const int srow = lane >> g.clog;
  const int last_col = (g.CH - 1) * g.LPR + c;
  lc.lw = (uint32_t)(srow * g.G + c) * 16u;
  lc.lw_last = (uint32_t)(srow * g.G + (last_col < g.G ? last_col : 0)) * 16u;
  const int lpr8 = g.LPR >> 3;
  const int sj = lane & 7;
  const int s_row = sj / lpr8, s_col = (sj - s_row * lpr8) * 8;
  const int s_last_col = (g.CH - 1) * g.LPR + s_col;
  lc.ls = (uint32_t)(s_row * g.G + s_col) * 2u;
  lc.ls_last = (uint32_t)(s_row * g.G + (s_last_col < g.G ? s_last_col : 0)) * 2u;
  lc.m = g.mat_begin;
  lc.m_end = g.mat_begin + g.num_mats;
}
__device__ __forceinline__ void lc_mat(LoadCursor& lc, const ChainMatDesc* mats, int cw) {
  const BlockRange br = block_range(cload(&mats[lc.m].n) >> (6 - lc.clog));
  lc.i = cw;
  lc.count = br.count;
  lc.ch = 0;
  const uint64_t u = (uint64_t)(br.u0 + cw);
  lc.pw = reinterpret_cast<const unsigned char*>(cload(&mats[lc.m].packed)) + u * lc.unit_w;
  lc.ps = reinterpret_cast<const unsigned char*>(cload(&mats[lc.m].scales)) + u * lc.unit_s;
  lc.pb = reinterpret_cast<const unsigned char*>(cload(&mats[lc.m].biases)) + u * lc.unit_s;
}
// move to the first position at or after the cursor that holds a slot of this
// wave (lc.s == num_stages: none left)
__device__ __forceinline__ void lc_seek(LoadCursor& lc, const ChainStageDesc* stages, const ChainMatDesc* mats,
                                        int num_stages, int cw, int lane) {
  while (lc.s < num_stages && lc.i >= lc.count) {
    if (++lc.m < lc.m_end) {
      lc_mat(lc, mats, cw);
    } else if (++lc.s < num_stages) {
      lc_stage(lc, stages, lane);
      lc_mat(lc, mats, cw);
    }
  }
}
__device__ __forceinline__ void lc_issue(LoadCursor& lc, uint32_t dst, int lane, const ChainStageDesc* stages,
                                         const ChainMatDesc* mats, int num_stages, int cw) {
  const bool last = lc.ch == lc.CH - 1;
  const uint32_t ow = last ? lc.lw_last : lc.lw + (uint32_t)(lc.ch * lc.LPR) * 16u;
  const uint32_t os = last ? lc.ls_last : lc.ls + (uint32_t)(lc.ch * lc.LPR) * 2u;
  dma16_s(lc.pw, ow, dst);
  if (lane < 16) dma16_v((lane >= 8 ? lc.pb : lc.ps) + os, dst + 1024u);
  if (++lc.ch == lc.CH) {
    lc.ch = 0;
    lc.i += kComputeWaves;
    lc.pw += (uint64_t)lc.unit_w * kComputeWaves;
    lc.ps += (uint64_t)lc.unit_s * kComputeWaves;
    lc.pb += (uint64_t)lc.unit_s * kComputeWaves;
    lc_seek(lc, stages, mats, num_stages, cw, lane);
  }
}

// Wait until every slot load older than the newest `younger` slots is
// complete (two loads per slot; the counter completes in issue order).
__device__ __forceinline__ void wait_slots(uint32_t younger) {
  if (younger == (uint32_t)(kRingSlots - 2)) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (kRingSlots - 2)));
  } else if (younger == (uint32_t)(kRingSlots - 1)) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (kRingSlots - 1)));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  compiler_fence();
}

// Compute wave cw: consumes its slots in the order it loads them. Per pair of
// chunks it waits for both slots, reads them (and the activations) from LDS,
// refills the two freed buffers with the slots kRingSlots further on, and
// only then does the arithmetic.
template <bool OUT_F32>
__device__ __forceinline__ void compute_body(const ChainStageDesc* stages, const ChainMatDesc* mats, int num_stages,
                                             int cw, ChainLds& L, ChainFlags& F, uint32_t* ws) {
  const int lane = threadIdx.x & 63;
  const uint32_t ring = (uint32_t)ufl((int)(uint32_t)(uintptr_t)(Q4_LDS unsigned char*)&L.ring[cw][0][0]);
  const unsigned char* myring = &L.ring[cw][0][0];
  LoadCursor lc;
  lc.s = 0;
  lc_stage(lc, stages, lane);
  lc_mat(lc, mats, cw);
  lc_seek(lc, stages, mats, num_stages, cw, lane);
  uint32_t issued = 0, k = 0;  // slots issued / consumed
  int ipos = 0, kpos = 0;      // their ring positions
  for (; issued < (uint32_t)kRingSlots && lc.s < num_stages; ++issued) {
    lc_issue(lc, ring + (uint32_t)ipos * kSlotBytes, lane, stages, mats, num_stages, cw);
    ipos = ipos + 1 == kRingSlots ? 0 : ipos + 1;
  }
  for (int s = 0; s < num_stages; ++s) {
    const Geo g = geo_of(stages + s);
    const bool sync_out = cload(&stages[s].sync_outputs) != 0;
    const int c = lane & (g.LPR - 1);
    const int srow = lane >> g.clog;
    const uint32_t sb_off = (uint32_t)(srow * g.LPR + c) * 2u;  // lane's bf16 in the slot's scales/biases
    {  // activations of stage s
      uint32_t spins = 0;
      while (lds_geti(&F.x_stage) < s) {
        __builtin_amdgcn_s_sleep(1);
        if (lds_get(&F.abort) != 0u) return;
        if (++spins > kSpinLimit) {
          compute_fail(ws, F);
          return;
        }
      }
    }
    compiler_fence();
    const uint32_t* xb = L.x[s & 1];
    for (int mi = 0; mi < g.num_mats; ++mi) {
      const int m = g.mat_begin + mi;
      const BlockRange br = block_range(cload(&mats[m].n) >> (6 - g.clog));
      void* y = cload(&mats[m].y);
      for (int i = cw; i < br.count; i += kComputeWaves) {
        float acc = 0.f;
        for (int ch = 0; ch < g.CH; ch += 2) {
          const int n2 = g.CH - ch >= 2 ? 2 : 1;
          wait_slots(issued - (k + (uint32_t)n2));
          const int kpos1 = kpos + 1 == kRingSlots ? 0 : kpos + 1;
          SlotRegs r0, r1;
          read_slot(myring + kpos * kSlotBytes, xb + (ch * g.LPR + c) * kXWordsPerGroup, lane, sb_off, r0);
          if (n2 == 2) read_slot(myring + kpos1 * kSlotBytes, xb + ((ch + 1) * g.LPR + c) * kXWordsPerGroup, lane, sb_off, r1);
          lds_wait();  // the reads are complete: the buffers may be refilled
          compiler_fence();
          for (int j = 0; j < n2; ++j) {
            if (lc.s < num_stages) {
              lc_issue(lc, ring + (uint32_t)ipos * kSlotBytes, lane, stages, mats, num_stages, cw);
              ipos = ipos + 1 == kRingSlots ? 0 : ipos + 1;
              ++issued;
            }
          }
          acc = slot_dot(r0, ch * g.LPR + c < g.G, acc);  // lanes past G in a ragged last chunk weigh zero
          if (n2 == 2) acc = slot_dot(r1, (ch + 1) * g.LPR + c < g.G, acc);
          k += (uint32_t)n2;
          kpos = n2 == 2 ? (kpos1 + 1 == kRingSlots ? 0 : kpos1 + 1) : kpos1;
        }
        const float tot = dpp_sum(acc, g.LPR);
        if (c == g.LPR - 1) {
          const int row = (br.u0 + i) * g.RPI + srow;
          if constexpr (OUT_F32) {
            coh_store(static_cast<uint32_t*>(y) + row, __float_as_uint(tot));
          } else {
            coh_store16(static_cast<uint16_t*>(y) + row, f32_to_bf16_rne(tot));
          }
        }
      }
    }
    // stage done; outputs read by a later stage must be visible first
    if (sync_out) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    compiler_fence();
    if (lane == 0) lds_add(&F.done_total, 1u);
  }
}
template <bool OUT_F32>
__device__ __forceinline__ void compute_run(const ChainStageDesc* stages, const ChainMatDesc* mats, int num_stages,
                                            int cw, ChainLds& L, ChainFlags& F, uint32_t* ws) {
  compute_body<OUT_F32>(stages, mats, num_stages, cw, L, F, ws);
  // no load into this block's LDS may outlive the wave (an aborted wave may
  // leave some in flight)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---------------------------------------------------------------- service

// Load a stage's activations into an LDS buffer, re-paired, with group sums;
// groups past G up to LPR*CH are zero. Coherent loads when an earlier stage of
// this launch wrote them.
__device__ __forceinline__ void service_load_x(const Geo& g, const void* x, bool coherent, uint32_t* dst_buf) {
  const int lane = threadIdx.x & 63;
  const int gpad = g.LPR * g.CH;
  const uint64_t* x64 = static_cast<const uint64_t*>(x);
  for (int grp = lane; grp < gpad; grp += 64) {
    uint32_t* dst = dst_buf + grp * kXWordsPerGroup;
    if (grp < g.G) {
      uint64_t q[8];
      if (coherent) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = coh_load64(x64 + (int64_t)grp * 8 + i);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = gload(x64 + (int64_t)grp * 8 + i);
      }
      float xs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 e;
        e.x = (uint32_t)q[2 * j];
        e.y = (uint32_t)(q[2 * j] >> 32);
        e.z = (uint32_t)q[2 * j + 1];
        e.w = (uint32_t)(q[2 * j + 1] >> 32);
        uint32_t p02, p46, p13, p57;
        x_to_pairs(e, p02, p46, p13, p57);
        *reinterpret_cast<uint4*>(dst + 4 * j) = make_uint4(p02, p46, p13, p57);
        xs += x_sum8(e);
      }
      dst[16] = __float_as_uint(xs);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(dst + 4 * j) = make_uint4(0u, 0u, 0u, 0u);
      dst[16] = 0u;
    }
  }
  lds_wait();
}

struct GridSync {
  uint32_t xcc;
  uint32_t per;      // blocks on this XCD
  uint32_t present;  // mask of XCDs that hold blocks
  uint32_t epoch;
};

__device__ __forceinline__ bool service_fail(uint32_t* ws, ChainFlags& F, uint32_t code) {
  if ((threadIdx.x & 63) == 0) {
    coh_store(ws + kWsStatus, code);
    lds_put(&F.abort, 1u);
  }
  return false;
}

// Start of a launch. The hardware deals the blocks of a launch round-robin
// over the device's nxcc XCDs, so block b runs on XCD b % nxcc (checked: a
// block on any other XCD reports status 3). The XCD's counters continue from
// earlier launches: the exchange flag holds the last completed epoch, and it
// cannot move before every block of this XCD has arrived at the first
// barrier of this launch, so every block of the XCD reads the same value here.
__device__ __forceinline__ bool service_start(uint32_t* ws, ChainFlags& F, GridSync& gs, uint32_t nxcc) {
  const uint32_t nb = gridDim.x;
  gs.xcc = blockIdx.x % nxcc;
  if (xcc_id() != gs.xcc) return service_fail(ws, F, 3u);
  gs.per = nb / nxcc + (gs.xcc < nb % nxcc ? 1u : 0u);
  gs.present = nxcc >= 32u ? 0xFFFFFFFFu : ((1u << (nxcc < nb ? nxcc : nb)) - 1u);
  // (unlike an L2 atomic on one line for every block of the XCD, reading the
  // flag does not serialise)
  gs.epoch = coh_load(ws + kWsGflag + gs.xcc);
  return true;
}

// Grid barrier: arrive on this XCD's L2 counter; the XCD's last arrival
// publishes the XCD's flag device-wide; every block waits until all XCDs'
// flags (one 64-byte line) carry this epoch.
__device__ __forceinline__ bool service_barrier(uint32_t* ws, ChainFlags& F, GridSync& gs) {
  const int lane = threadIdx.x & 63;
  const uint32_t e = ++gs.epoch;
  uint32_t old = 0;
  if (lane == 0) old = l2_add(ws + kWsXcnt + 32 * gs.xcc, 1u);
  old = __shfl(old, 0);
  if ((old + 1u) % gs.per == 0u && lane == 0) coh_store(ws + kWsGflag + gs.xcc, e);
  uint32_t spins = 0;
  while (true) {
    bool mine = true;
    if (lane < kMaxXcc && ((gs.present >> lane) & 1u)) mine = (int)(coh_load(ws + kWsGflag + lane) - e) >= 0;
    if (__all(mine)) break;
    if (++spins > kSpinLimit || coh_load(ws + kWsStatus) != 0u) return service_fail(ws, F, 1u);
  }
  return true;
}

__device__ __forceinline__ void service_run(const ChainStageDesc* stages, int num_stages, ChainLds& L,
                                            ChainFlags& F, uint32_t* ws, uint32_t nxcc) {
  GridSync gs;
  if (!service_start(ws, F, gs, nxcc)) return;
  service_load_x(geo_of(stages), cload(&stages[0].x), false, L.x[0]);
  if (num_stages > 1 && cload(&stages[1].x_internal) == 0)
    service_load_x(geo_of(stages + 1), cload(&stages[1].x), false, L.x[1]);
  compiler_fence();
  if ((threadIdx.x & 63) == 0) lds_puti(&F.x_stage, 0);
  for (int s = 0; s < num_stages; ++s) {
    uint32_t spins = 0;
    while ((int)(lds_get(&F.done_total) - (uint32_t)(kComputeWaves * (s + 1))) < 0) {
      __builtin_amdgcn_s_sleep(1);
      if (lds_get(&F.abort) != 0u) return;
      if (++spins > kSpinLimit) {
        service_fail(ws, F, 1u);
        return;
      }
    }
    if (s + 1 >= num_stages) break;
    if (!service_barrier(ws, F, gs)) return;
    if (cload(&stages[s + 1].x_internal) != 0)
      service_load_x(geo_of(stages + s + 1), cload(&stages[s + 1].x), true, L.x[(s + 1) & 1]);
    compiler_fence();
    if ((threadIdx.x & 63) == 0) lds_puti(&F.x_stage, s + 1);
    // every compute wave has finished stage s, so its buffer is free
    if (s + 2 < num_stages && cload(&stages[s + 2].x_internal) == 0)
      service_load_x(geo_of(stages + s + 2), cload(&stages[s + 2].x), false, L.x[s & 1]);
  }
}

// ---------------------------------------------------------------- kernel

template <bool OUT_F32>
__global__ void __launch_bounds__(64 * kChainWaves) __attribute__((amdgpu_waves_per_eu((kChainWaves + 3) / 4, (kChainWaves + 3) / 4)))
chain_kernel(const ChainHeader* __restrict__ plan, uint32_t* __restrict__ ws, uint32_t nxcc) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  __shared__ ChainFlags F;
  ChainLds& L = *reinterpret_cast<ChainLds*>(lds_raw);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  if (threadIdx.x == 0) {
    F.done_total = 0u;
    F.x_stage = -1;
    F.abort = 0u;
    // the plan must be one this library encoded
    const bool ok = coh_load(ws + kWsStatus) == 0u && cload(&plan->magic) == kChainMagic &&
                    cload(&plan->num_stages) > 0 && cload(&plan->num_mats) > 0 &&
                    gridDim.x <= (unsigned)kChainMaxBlocks && nxcc >= 1u && nxcc <= (unsigned)kMaxXcc;
    F.go = ok ? 1u : 0u;
    if (!ok && blockIdx.x == 0 && coh_load(ws + kWsStatus) == 0u) coh_store(ws + kWsStatus, 2u);
  }
  __syncthreads();
  if (F.go == 0u) return;
  const int num_stages = cload(&plan->num_stages);
  const ChainStageDesc* stages = reinterpret_cast<const ChainStageDesc*>(plan + 1);
  const ChainMatDesc* mats = reinterpret_cast<const ChainMatDesc*>(stages + num_stages);

  if (wave == kServiceWave) {
    service_run(stages, num_stages, L, F, ws, nxcc);
  } else {
    compute_run<OUT_F32>(stages, mats, num_stages, wave - 1, L, F, ws);
  }
}

}  // namespace q4k
