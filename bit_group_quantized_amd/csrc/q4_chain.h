// Persistent chain executor for ordered stages of quantized GEMVs (gfx950).
// Included by q4_api.hip after q4_kernels.h.
//
// The temporal step is an ordered chain of stages ("NVIDIA PersonaPlex 7B on
// Apple Silicon", pipeline diagram: 32 layers; read as standard decoder
// layers: attention input -> q,k,v; attention output -> o; FFN input ->
// gate,up; gated product -> down). A stage multiplies one activation vector by
// one or more matrices that share it and may consume the previous stage's
// outputs, so its products may not start before every output of the previous
// stage is written and visible.
//
// One launch runs the whole chain, one block of 16 waves per compute unit:
//  - 15 compute waves only stream weights and do arithmetic. The rows of a
//    stage are cut into units of RPI rows (C lanes per row, one 32-input group
//    per lane and chunk, CH chunks per row) dealt round-robin to every compute
//    wave of the grid. A wave's units of a stage form rounds of at most
//    kSlots 16-byte loads per lane; two rounds are always in flight (double
//    buffer), across stage boundaries, because weights never depend on
//    activations. Activations come from LDS; finished rows are handed to LDS
//    as (row, value) records.
//  - 1 service wave owns everything with device-wide ordering: it writes the
//    records to global memory with device-coherent stores, waits for them,
//    raises the block's flag (one 128-byte line per block holding a running
//    barrier count), waits until block 0 has gathered every flag and
//    published the count, and loads the next stage's activations with
//    device-coherent loads into LDS. Keeping these off the compute waves
//    matters because a wave's vector-memory counter completes in order: a
//    compute wave waiting on a coherent load or store would also wait for all
//    weight loads it issued before.
//  - compute and service waves meet at two block barriers per stage (outputs
//    handed over; next activations ready). Waits on other blocks are bounded
//    and report a timeout in the workspace instead of hanging.
#pragma once

namespace q4k {

constexpr uint32_t kChainMagic = 0x48433451u;  // "Q4CH"
constexpr int kChainWaves = 12;
constexpr int kComputeWaves = 11;
constexpr int kServiceWave = 11;
constexpr int kSlots = 6;              // 16-byte loads per lane per round
constexpr int kMaxMatsPerStage = 4;
constexpr int kMaxRecPerWave = 64;     // finished rows per compute wave per stage
constexpr int kMaxGroups = 512;        // k <= 16384
constexpr int kXWordsPerGroup = 20;    // 16 re-paired words + sum + pad (bank spread)
constexpr int kPlanLdsBytes = 96 * 1024;
constexpr int kChainMaxBlocks = 1024;
constexpr uint32_t kBarrierSpinLimit = 1u << 21;

struct alignas(16) ChainHeader {
  uint32_t magic;
  int32_t num_stages;
  int32_t num_mats;
  int32_t out_f32;
  int32_t plan_bytes;
  int32_t max_rows;  // largest stage row count
  int32_t pad[10];
};
struct alignas(16) ChainStageDesc {
  const uint16_t* x;
  int32_t G;        // groups of 32 inputs
  int32_t c_log2;   // lanes per row = 1 << c_log2
  int32_t CH;       // chunks per row (ceil(G / C) <= kSlots)
  int32_t UPR;      // units per round = kSlots / CH
  int32_t nrows;    // rows of all matrices of the stage
  int32_t num_mats;
  int32_t mat_begin;
  int32_t row_off[kMaxMatsPerStage + 1];  // first row of each matrix; [num_mats] = nrows
  int32_t pad[2];
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

// workspace words: status on its own 128-byte line, then one flag word per
// block (dense, so a wave reads all flags with a few wide loads)
constexpr int kWsStatus = 0;  // 0 ok, 1 barrier timeout, 2 bad plan
constexpr int kWsFlags = 64;  // block b's flag at kWsFlags + b

// Pointers read from the plan are generic; loads through them must be issued
// as global (not flat) accesses, which count only in the vector-memory
// counter and let the weight loads stay in flight.
#define Q4_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
  return *(const Q4_GLOBAL T*)p;
}

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

// Shared-memory layout of the chain kernel (dynamic LDS).
struct ChainLds {
  uint32_t x[kMaxGroups * kXWordsPerGroup];          // re-paired activations + group sums
  uint32_t rec_row[kComputeWaves][kMaxRecPerWave];   // (matrix << 24) | local row
  float rec_val[kComputeWaves][kMaxRecPerWave];
  int32_t rec_count[kComputeWaves];
  int32_t ok;
  int32_t pad[16 - ((kComputeWaves + 1) % 16)];
  unsigned char plan[kPlanLdsBytes];
};

// Uniform (per-wave) reads of plan fields held in LDS.
__device__ __forceinline__ int u32r(const int32_t* p) { return __builtin_amdgcn_readfirstlane(*p); }
__device__ __forceinline__ const void* ptrr(const void* const* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(*p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// Per-stage geometry (wave-uniform).
struct StageView {
  int idx;
  int G, C, clog, CH, UPR, RPI, num_mats, mat_begin;
};

__device__ __forceinline__ StageView stage_view(const ChainStageDesc* stages, int s) {
  StageView v;
  const ChainStageDesc* sd = stages + s;
  v.idx = s;
  v.G = u32r(&sd->G);
  v.clog = u32r(&sd->c_log2);
  v.C = 1 << v.clog;
  v.CH = u32r(&sd->CH);
  v.UPR = u32r(&sd->UPR);
  v.RPI = 64 >> v.clog;
  v.num_mats = u32r(&sd->num_mats);
  v.mat_begin = u32r(&sd->mat_begin);
  return v;
}

// Position in the work sequence: stage s, matrix m (absolute index), round r
// of that matrix. A matrix's units (RPI consecutive rows) are dealt
// round-robin to every compute wave of the grid; a wave takes its units of a
// matrix UPR at a time (one round). Every matrix has >= 1 round per wave so
// that every wave walks the same sequence.
struct Cursor {
  StageView v;
  int m, r, nrounds, nunits;
  bool valid;
};

__device__ __forceinline__ void cursor_matrix(Cursor& c, const ChainMatDesc* mats, int wct) {
  const int n = u32r(&mats[c.m].n);
  c.nunits = n >> (6 - c.v.clog);  // matrices hold whole units (n % RPI == 0)
  const int per_wave = (c.nunits + wct - 1) / wct;
  c.nrounds = max(1, (per_wave + c.v.UPR - 1) / c.v.UPR);
  c.r = 0;
}

__device__ __forceinline__ Cursor cursor_stage(const ChainStageDesc* stages, const ChainMatDesc* mats,
                                               int num_stages, int s, int wct) {
  Cursor c;
  c.valid = s < num_stages;
  if (!c.valid) return c;
  c.v = stage_view(stages, s);
  c.m = c.v.mat_begin;
  cursor_matrix(c, mats, wct);
  return c;
}

// true when the cursor sits on the last round of its stage
__device__ __forceinline__ bool cursor_stage_end(const Cursor& c) {
  return c.r + 1 >= c.nrounds && c.m + 1 >= c.v.mat_begin + c.v.num_mats;
}

__device__ __forceinline__ void cursor_advance(Cursor& c, const ChainStageDesc* stages, const ChainMatDesc* mats,
                                               int num_stages, int wct) {
  if (++c.r < c.nrounds) return;
  if (++c.m < c.v.mat_begin + c.v.num_mats) {
    cursor_matrix(c, mats, wct);
    return;
  }
  c = cursor_stage(stages, mats, num_stages, c.v.idx + 1, wct);
}

// Issue-side state of the stage being issued: per-lane byte offsets (all
// non-negative) of the lane's group relative to group 0 of the unit's first
// row. Chunk ch < CH-1 adds ch*C groups through the uniform base; the last
// chunk carries its column in the lane offset, so that in a ragged row
// (C*CH > G) the lanes past G read group 0 of their own row instead. Their
// activations are zero, so the weights they read do not count.
struct LaneOffsets {
  uint32_t lw, lw_last;    // packed
  uint32_t ls, ls_last;    // scales / biases: byte offset of the aligned word holding the lane's bf16
  uint32_t sel, sel_last;  // which half of that word (byte selector for bf16_half_to_f32)
};

__device__ __forceinline__ LaneOffsets lane_offsets(const StageView& v) {
  const int lane = threadIdx.x & 63;
  const int c = lane & (v.C - 1);
  const int slot_row = lane >> v.clog;
  const uint32_t grp = (uint32_t)(slot_row * v.G + c);
  const int last_col = (v.CH - 1) * v.C + c;
  const uint32_t grp_last = (uint32_t)(slot_row * v.G + (last_col < v.G ? last_col : 0));
  LaneOffsets o;
  o.lw = grp * 16u;
  o.lw_last = grp_last * 16u;
  // G is even and the arrays are 4-byte aligned, so a group's parity decides
  // the half of its 32-bit word
  o.ls = (grp & ~1u) * 2u;
  o.ls_last = (grp_last & ~1u) * 2u;
  o.sel = (grp & 1u) ? kSelHiHalf : kSelLoHalf;
  o.sel_last = (grp_last & 1u) ? kSelHiHalf : kSelLoHalf;
  return o;
}

struct RoundBuf {
  uint4 w[kSlots];
  uint32_t s[kSlots];
  uint32_t b[kSlots];
};

template <typename T>
__device__ __forceinline__ T gload_off(const unsigned char* base, uint32_t off) {
  return gload(reinterpret_cast<const T*>(base + off));
}

// Issue the weight loads of one round: slot jj*CH+ch is chunk ch of unit jj.
// All kSlots*3 loads are issued unconditionally (units past the matrix
// re-read unit 0 and are skipped at compute time), so every round issues the
// same loads in the same order and the compiler's load counting stays exact.
template <int CH>
__device__ __forceinline__ void round_issue(const Cursor& cu, const ChainMatDesc* mats, const LaneOffsets& lo,
                                            int gw, int wct, RoundBuf& buf) {
  constexpr int UPR = kSlots / CH;
  const StageView& v = cu.v;
  const unsigned char* pk = static_cast<const unsigned char*>(ptrr(reinterpret_cast<const void* const*>(&mats[cu.m].packed)));
  const unsigned char* sc = static_cast<const unsigned char*>(ptrr(reinterpret_cast<const void* const*>(&mats[cu.m].scales)));
  const unsigned char* bi = static_cast<const unsigned char*>(ptrr(reinterpret_cast<const void* const*>(&mats[cu.m].biases)));
#pragma unroll
  for (int jj = 0; jj < UPR; ++jj) {
    int unit = gw + (cu.r * UPR + jj) * wct;
    unit = unit < cu.nunits ? unit : 0;
    const int64_t row_g = (int64_t)unit * v.RPI * v.G;  // group index of the unit's first row
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      const int i = jj * CH + ch;
      const bool last = ch == CH - 1;
      const int64_t gbase = row_g + (last ? 0 : ch * v.C);
      const u32x4_t t = gload_off<u32x4_t>(pk + gbase * 16, last ? lo.lw_last : lo.lw);
      buf.w[i] = make_uint4(t.x, t.y, t.z, t.w);
      buf.s[i] = gload_off<uint32_t>(sc + gbase * 2, last ? lo.ls_last : lo.ls);
      buf.b[i] = gload_off<uint32_t>(bi + gbase * 2, last ? lo.ls_last : lo.ls);
    }
  }
}

// Sum over the C lanes of a row slot with DPP adds; the total lands in the
// slot's last lane (lane % C == C - 1).
__device__ __forceinline__ float dpp_sum(float v, int C) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));  // xor 1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  // xor 2
  if (C >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half-row mirror
  if (C >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  if (C >= 32) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row bcast 15
  if (C >= 64) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row bcast 31
  return v;
}

template <int CH>
__device__ __forceinline__ void round_compute(const Cursor& cu, const LaneOffsets& lo, int gw, int wct,
                                              const RoundBuf& buf, ChainLds& L, int cw) {
  constexpr int UPR = kSlots / CH;
  const StageView& v = cu.v;
  if (gw + cu.r * UPR * wct >= cu.nunits) return;  // no rows for this wave in this round
  const int lane = threadIdx.x & 63;
  const int c = lane & (v.C - 1);
  const int slot_row = lane >> v.clog;
  int cnt = u32r(&L.rec_count[cw]);
#pragma unroll
  for (int jj = 0; jj < UPR; ++jj) {
    const int unit = gw + (cu.r * UPR + jj) * wct;
    if (unit < cu.nunits) {  // wave-uniform
      float acc = 0.f;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const int i = jj * CH + ch;
        const uint32_t* xg = L.x + (ch * v.C + c) * kXWordsPerGroup;  // padded groups hold zeros
        uint32_t xp[16];
        const uint4 a0 = *reinterpret_cast<const uint4*>(xg + 0);
        const uint4 a1 = *reinterpret_cast<const uint4*>(xg + 4);
        const uint4 a2 = *reinterpret_cast<const uint4*>(xg + 8);
        const uint4 a3 = *reinterpret_cast<const uint4*>(xg + 12);
        xp[0] = a0.x; xp[1] = a0.y; xp[2] = a0.z; xp[3] = a0.w;
        xp[4] = a1.x; xp[5] = a1.y; xp[6] = a1.z; xp[7] = a1.w;
        xp[8] = a2.x; xp[9] = a2.y; xp[10] = a2.z; xp[11] = a2.w;
        xp[12] = a3.x; xp[13] = a3.y; xp[14] = a3.z; xp[15] = a3.w;
        const float xsum = __uint_as_float(xg[16]);
        const uint32_t sel = ch == CH - 1 ? lo.sel_last : lo.sel;
        acc = fmaf(bf16_half_to_f32(buf.s[i], sel), group_dot(buf.w[i], xp),
                   fmaf(bf16_half_to_f32(buf.b[i], sel), xsum, acc));
      }
      const float tot = dpp_sum(acc, v.C);
      if (c == v.C - 1) {
        L.rec_row[cw][cnt + slot_row] = ((uint32_t)cu.m << 22) | (uint32_t)(unit * v.RPI + slot_row);
        L.rec_val[cw][cnt + slot_row] = tot;
      }
      cnt += v.RPI;
    }
  }
  if (lane == 0) L.rec_count[cw] = cnt;
}

__device__ __forceinline__ void dispatch_issue(const Cursor& cu, const ChainMatDesc* mats, const LaneOffsets& lo,
                                               int gw, int wct, RoundBuf& b) {
  switch (cu.v.CH) {
    case 1: round_issue<1>(cu, mats, lo, gw, wct, b); break;
    case 2: round_issue<2>(cu, mats, lo, gw, wct, b); break;
    case 3: round_issue<3>(cu, mats, lo, gw, wct, b); break;
    case 4: round_issue<4>(cu, mats, lo, gw, wct, b); break;
    case 5: round_issue<5>(cu, mats, lo, gw, wct, b); break;
    default: round_issue<6>(cu, mats, lo, gw, wct, b); break;
  }
}

__device__ __forceinline__ void dispatch_compute(const Cursor& cu, const LaneOffsets& lo, int gw, int wct,
                                                 const RoundBuf& b, ChainLds& L, int cw) {
  switch (cu.v.CH) {
    case 1: round_compute<1>(cu, lo, gw, wct, b, L, cw); break;
    case 2: round_compute<2>(cu, lo, gw, wct, b, L, cw); break;
    case 3: round_compute<3>(cu, lo, gw, wct, b, L, cw); break;
    case 4: round_compute<4>(cu, lo, gw, wct, b, L, cw); break;
    case 5: round_compute<5>(cu, lo, gw, wct, b, L, cw); break;
    default: round_compute<6>(cu, lo, gw, wct, b, L, cw); break;
  }
}

// ---- service wave helpers (all 64 lanes of the service wave call these)

// Load stage s's activations (device-coherent) into LDS, re-paired, with group
// sums; groups past G up to the padded count are zero.
__device__ __forceinline__ void service_load_x(const StageView& v, const void* x, ChainLds& L) {
  const int lane = threadIdx.x & 63;
  const int gpad = v.C * v.CH;
  const uint64_t* x64 = static_cast<const uint64_t*>(x);
  for (int g = lane; g < gpad; g += 64) {
    uint32_t* dst = L.x + g * kXWordsPerGroup;
    if (g < v.G) {
      uint64_t q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = coh_load64(x64 + (int64_t)g * 8 + i);
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
}

template <bool OUT_F32>
__device__ __forceinline__ void service_store_records(const ChainMatDesc* mats, ChainLds& L) {
  const int lane = threadIdx.x & 63;
  for (int w = 0; w < kComputeWaves; ++w) {
    const int cnt = L.rec_count[w];
    for (int i = lane; i < cnt; i += 64) {
      const uint32_t code = L.rec_row[w][i];
      const ChainMatDesc& md = mats[code >> 22];
      const int row = (int)(code & 0x3FFFFFu);
      const float val = L.rec_val[w][i];
      if constexpr (OUT_F32) {
        coh_store(static_cast<uint32_t*>(md.y) + row, __float_as_uint(val));
      } else {
        coh_store16(static_cast<uint16_t*>(md.y) + row, f32_to_bf16_rne(val));
      }
    }
  }
}

// Cross-block stage barrier, service wave only: raise this block's flag to
// `epoch`, then read every block's flag (four per lane per poll) until all
// have reached it. One memory round trip after the last block arrives.
// Returns false on timeout or a reported error (then the status word is set).
__device__ __forceinline__ bool service_barrier(uint32_t* ws, uint32_t epoch) {
  const int lane = threadIdx.x & 63;
  const int nb = gridDim.x;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's output stores are complete
  if (lane == 0) coh_store(ws + kWsFlags + blockIdx.x, epoch);
  const uint64_t* f64 = reinterpret_cast<const uint64_t*>(ws + kWsFlags);
  bool ok = true;
  uint32_t spins = 0;
  while (true) {
    bool mine = true;
    for (int b4 = lane; 4 * b4 < nb; b4 += 64) {
      const uint64_t a = coh_load64(f64 + 2 * b4);
      const uint64_t c = coh_load64(f64 + 2 * b4 + 1);
      const uint32_t f[4] = {(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)c, (uint32_t)(c >> 32)};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * b4 + j < nb && (int)(f[j] - epoch) < 0) mine = false;
    }
    if (__all(mine)) break;
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kBarrierSpinLimit || coh_load(ws + kWsStatus) != 0u) {
      ok = false;
      break;
    }
  }
  if (!ok && lane == 0) coh_store(ws + kWsStatus, 1u);
  return ok;
}

template <bool OUT_F32>
__global__ void __launch_bounds__(768) chain_kernel(const ChainHeader* __restrict__ plan_g,
                                                      uint32_t* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  ChainLds& L = *reinterpret_cast<ChainLds*>(lds_raw);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = threadIdx.x & 63;

  if (coh_load(ws + kWsStatus) != 0u) return;  // earlier failure: workspace must be cleared
  if (plan_g->magic != kChainMagic || plan_g->plan_bytes > kPlanLdsBytes) {
    if (blockIdx.x == 0 && threadIdx.x == 0) coh_store(ws + kWsStatus, 2u);
    return;
  }
  // copy the plan into LDS
  {
    const int words = plan_g->plan_bytes / 16;
    const uint4* src = reinterpret_cast<const uint4*>(plan_g);
    uint4* dst = reinterpret_cast<uint4*>(L.plan);
    for (int i = threadIdx.x; i < words; i += blockDim.x) dst[i] = src[i];
  }
  if (threadIdx.x < kComputeWaves) L.rec_count[threadIdx.x] = 0;
  if (threadIdx.x == 0) L.ok = 1;
  __syncthreads();
  const ChainHeader* plan = reinterpret_cast<const ChainHeader*>(L.plan);
  const int num_stages = plan->num_stages;
  const ChainStageDesc* stages = reinterpret_cast<const ChainStageDesc*>(plan + 1);
  const ChainMatDesc* mats = reinterpret_cast<const ChainMatDesc*>(stages + num_stages);
  const int wct = kComputeWaves * gridDim.x;  // compute waves in the grid
  // each compute wave must be able to hold its rows of any stage as records
  // (a wave's rows of one matrix: at most n/(wct*RPI) + 1 units of RPI <= 8 rows)
  if (plan->max_rows > (kMaxRecPerWave - 8 * kMaxMatsPerStage) * wct) {
    if (blockIdx.x == 0 && threadIdx.x == 0) coh_store(ws + kWsStatus, 2u);
    return;
  }

  if (wave == kServiceWave) {
    // running barrier count, equal in all blocks after a completed launch
    uint32_t epoch = coh_load(ws + kWsFlags + blockIdx.x);
    service_load_x(stage_view(stages, 0), ptrr(reinterpret_cast<const void* const*>(&stages[0].x)), L);
    __syncthreads();  // S2 of stage 0: activations ready
    for (int s = 0; s < num_stages; ++s) {
      __syncthreads();  // S1: compute waves finished stage s, records complete
      service_store_records<OUT_F32>(mats, L);
      if (s + 1 < num_stages) {
        const bool ok = service_barrier(ws, ++epoch);
        if (lane < kComputeWaves) L.rec_count[lane] = 0;
        if (ok) service_load_x(stage_view(stages, s + 1), ptrr(reinterpret_cast<const void* const*>(&stages[s + 1].x)), L);
        else if (lane == 0) L.ok = 0;
        __syncthreads();  // S2: next activations ready (or abort)
        if (!ok) return;
      }
    }
    return;
  }

  // ---- compute waves
  const int cw = wave;
  const int gw = cw * gridDim.x + blockIdx.x;
  RoundBuf bufA, bufB;
  // issue cursor runs two rounds ahead of the compute cursor
  Cursor ic = cursor_stage(stages, mats, num_stages, 0, wct);
  LaneOffsets lo = lane_offsets(ic.v);
  int lo_stage = 0;
  Cursor cc = ic;
  for (int k = 0; k < 2; ++k) {
    RoundBuf& b = k == 0 ? bufA : bufB;
    if (ic.valid) {
      if (ic.v.idx != lo_stage) { lo = lane_offsets(ic.v); lo_stage = ic.v.idx; }
      dispatch_issue(ic, mats, lo, gw, wct, b);
      cursor_advance(ic, stages, mats, num_stages, wct);
    }
  }
  __syncthreads();  // S2 of stage 0
  LaneOffsets clo = lane_offsets(cc.v);  // offsets of the stage being computed
  bool running = true;
  while (running) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      RoundBuf& b = k == 0 ? bufA : bufB;
      dispatch_compute(cc, clo, gw, wct, b, L, cw);
      const bool stage_end = cursor_stage_end(cc);
      if (stage_end) __syncthreads();  // S1: hand the stage's records to the service wave
      // refill this buffer two rounds ahead (after S1 at a stage end, so a
      // wait on older loads cannot delay the hand-over)
      if (ic.valid) {
        if (ic.v.idx != lo_stage) { lo = lane_offsets(ic.v); lo_stage = ic.v.idx; }
        dispatch_issue(ic, mats, lo, gw, wct, b);
        cursor_advance(ic, stages, mats, num_stages, wct);
      }
      if (stage_end) {
        if (cc.v.idx + 1 >= num_stages) { running = false; break; }
        __syncthreads();  // S2: next stage's activations ready
        if (L.ok == 0) { running = false; break; }
      }
      cursor_advance(cc, stages, mats, num_stages, wct);
      if (stage_end) clo = lane_offsets(cc.v);
    }
  }
}

}  // namespace q4k
