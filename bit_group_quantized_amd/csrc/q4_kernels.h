// Device code of libq4: gfx950 (CDNA4) kernels for the affine 4-bit group-32
// quantized linear layer. Included by q4_api.hip only.
//
// Format (model card "personaplex-edge-q4", Release details table: affine Q4,
// group size 32, BF16 activations): a group of 32 inputs is one 16-byte run of
// four uint32 words, code of input 8j+t in bits [4t, 4t+4) of word j; one bf16
// scale and one bf16 bias per group in two separate [n][k/32] arrays.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Code unpacking. A byte holding c in 0..15 read as OCP e4m3 is exactly
// c * 2^-9 (c < 8: subnormal c/8 * 2^-6; c >= 8: (1 + (c-8)/8) * 2^-6), so the
// gfx950 scaled fp8->bf16 conversion with scale 2^9 yields the integer c as an
// exact bf16. Masking the word with 0x0F0F0F0F puts codes 0,2,4,6 of the word
// in bytes 0..3; shifting by 4 first gives codes 1,3,5,7.
// Output pairs (low half first): (c0,c2) (c4,c6) (c1,c3) (c5,c7).
__device__ __forceinline__ void word_to_bf16_pairs(uint32_t w, uint32_t& p02, uint32_t& p46,
                                                   uint32_t& p13, uint32_t& p57) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  p02 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false));
  p46 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true));
  p13 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false));
  p57 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true));
}

// Eight bf16 activations x0..x7 (as loaded: four uint32 (x0,x1) (x2,x3)
// (x4,x5) (x6,x7)) re-paired to match word_to_bf16_pairs.
__device__ __forceinline__ void x_to_pairs(uint4 e, uint32_t& p02, uint32_t& p46, uint32_t& p13,
                                           uint32_t& p57) {
  p02 = (e.x & 0xFFFFu) | (e.y << 16);
  p46 = (e.z & 0xFFFFu) | (e.w << 16);
  p13 = (e.x >> 16) | (e.y & 0xFFFF0000u);
  p57 = (e.z >> 16) | (e.w & 0xFFFF0000u);
}

__device__ __forceinline__ float x_sum8(uint4 e) {
  return ((bf16_to_f32(e.x & 0xFFFFu) + bf16_to_f32(e.x >> 16)) +
          (bf16_to_f32(e.y & 0xFFFFu) + bf16_to_f32(e.y >> 16))) +
         ((bf16_to_f32(e.z & 0xFFFFu) + bf16_to_f32(e.z >> 16)) +
          (bf16_to_f32(e.w & 0xFFFFu) + bf16_to_f32(e.w >> 16)));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// sum_{t<32} c_t * x_t for one group: 16 packed bf16 dot products, fp32 sum.
__device__ __forceinline__ float group_dot(uint4 w, const uint32_t (&xp)[16]) {
  float acc = 0.f;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t q02, q46, q13, q57;
    word_to_bf16_pairs(ws[j], q02, q46, q13, q57);
    acc = dot2(q02, xp[4 * j + 0], acc);
    acc = dot2(q46, xp[4 * j + 1], acc);
    acc = dot2(q13, xp[4 * j + 2], acc);
    acc = dot2(q57, xp[4 * j + 3], acc);
  }
  return acc;
}

// bf16 bit pattern -> fp32, taken from either half of a 32-bit word: the
// selector keeps bytes (lo) or (hi) of the word as the upper half and zeroes
// the lower half. Scales and biases are fetched as the aligned 32-bit word
// holding the wanted bf16: on gfx950 whole-word loads stream at full rate
// while 2-byte loads do not.
constexpr uint32_t kSelLoHalf = 0x01000C0Cu;
constexpr uint32_t kSelHiHalf = 0x03020C0Cu;
__device__ __forceinline__ float bf16_half_to_f32(uint32_t word, uint32_t sel) {
  return __uint_as_float(__builtin_amdgcn_perm(0u, word, sel));
}

// Load the bf16 at p (2-byte aligned) through its aligned 32-bit word; returns
// the value as fp32.
__device__ __forceinline__ float load_bf16_word(const uint16_t* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(a & ~(uintptr_t)3);
  return bf16_half_to_f32(w, (a & 2) ? kSelHiHalf : kSelLoHalf);
}

template <bool OUT_F32>
__device__ __forceinline__ void store_out(void* y, int64_t idx, float v) {
  if constexpr (OUT_F32) {
    static_cast<float*>(y)[idx] = v;
  } else {
    static_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
  }
}

// ---------------------------------------------------------------------------
// Quantize + pack: one thread per group of 32.
__global__ void __launch_bounds__(256) pack_kernel(const float* __restrict__ w, int64_t n_groups,
                                                    uint32_t* __restrict__ packed,
                                                    uint16_t* __restrict__ scales,
                                                    uint16_t* __restrict__ biases) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n_groups; idx += stride) {
    const float4* src = reinterpret_cast<const float4*>(w + idx * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 t = src[i];
      v[4 * i + 0] = t.x;
      v[4 * i + 1] = t.y;
      v[4 * i + 2] = t.z;
      v[4 * i + 3] = t.w;
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
      if (v[i] < mn) mn = v[i];
      if (v[i] > mx) mx = v[i];
    }
    const float scale = (mx - mn) / 15.0f;  // IEEE division (correctly rounded)
    const uint16_t sb = f32_to_bf16_rne(scale);
    const uint16_t bb = f32_to_bf16_rne(mn);
    const float s = bf16_to_f32(sb);
    const float b = bf16_to_f32(bb);
    uint32_t words[4] = {0u, 0u, 0u, 0u};
    if (s != 0.0f) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        float r = rintf((v[i] - b) / s);
        r = fminf(fmaxf(r, 0.0f), 15.0f);
        words[i >> 3] |= (uint32_t)r << (4 * (i & 7));
      }
    }
    reinterpret_cast<uint4*>(packed)[idx] = make_uint4(words[0], words[1], words[2], words[3]);
    scales[idx] = sb;
    biases[idx] = bb;
  }
}

// Unpack: one thread per group; codes as bytes and/or w_hat = s*q + b.
__global__ void __launch_bounds__(256) unpack_kernel(const uint32_t* __restrict__ packed,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ biases,
                                                      int64_t n_groups, uint8_t* __restrict__ q_out,
                                                      float* __restrict__ w_out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n_groups; idx += stride) {
    const uint4 wd = reinterpret_cast<const uint4*>(packed)[idx];
    const uint32_t ws[4] = {wd.x, wd.y, wd.z, wd.w};
    if (q_out) {
      uint32_t bytes[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = ws[j] & 0x0F0F0F0Fu;         // codes 0,2,4,6
        const uint32_t hi = (ws[j] >> 4) & 0x0F0F0F0Fu;  // codes 1,3,5,7
        // interleave to input order c0 c1 c2 c3 | c4 c5 c6 c7
        bytes[2 * j] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
        bytes[2 * j + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
      }
      uint4* dst = reinterpret_cast<uint4*>(q_out + idx * 32);
      dst[0] = make_uint4(bytes[0], bytes[1], bytes[2], bytes[3]);
      dst[1] = make_uint4(bytes[4], bytes[5], bytes[6], bytes[7]);
    }
    if (w_out) {
      const float s = bf16_to_f32(scales[idx]);
      const float b = bf16_to_f32(biases[idx]);
      float4* dst = reinterpret_cast<float4*>(w_out + idx * 32);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float4 t;
        const uint32_t word = ws[i >> 1];
        const int sh = (i & 1) * 16;
        t.x = fmaf(s, (float)((word >> (sh + 0)) & 0xFu), b);
        t.y = fmaf(s, (float)((word >> (sh + 4)) & 0xFu), b);
        t.z = fmaf(s, (float)((word >> (sh + 8)) & 0xFu), b);
        t.w = fmaf(s, (float)((word >> (sh + 12)) & 0xFu), b);
        dst[i] = t;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// GEMV against MV activation rows (MV = 1: the GEMV; up to 4 rows share one
// weight stream).
//
// Mapping: a wave is split into 64/C row slots of C lanes; lane (slot, c) of
// wave w owns group g = w*C + c of the input dimension for every row it
// visits, so its 32 activations of each of the MV rows live in 16 registers
// each (re-paired bf16) for the whole kernel and the weight stream needs no
// shared memory. A block has S = ceil(G/C) waves covering all groups; each
// load instruction of a wave reads C consecutive 16-byte groups of one row per
// slot (C*16 contiguous bytes). Each lane handles U weight rows per iteration
// (U independent loads in flight), dequantizes each loaded group once and
// takes its dot product with every activation row, reduces each partial over
// its C lanes with butterfly shuffles, and the S waves' partials are added in
// fixed order through LDS.
template <int C, int U, int MV, bool OUT_F32>
__global__ void __launch_bounds__(1024) gemv_kernel(const uint16_t* __restrict__ x, int64_t x_stride,
                                                     const uint32_t* __restrict__ packed,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint16_t* __restrict__ biases, int n,
                                                     int G, int rows_per_block,
                                                     void* __restrict__ y, int64_t y_stride) {
  constexpr int RPI = 64 / C;   // row slots per wave
  constexpr int ROWS = RPI * U; // weight rows per iteration
  __shared__ float red[16][ROWS * MV];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c = lane % C;
  const int slot = lane / C;
  const int g = wave * C + c;
  const bool gv = g < G;

  const int row_begin = blockIdx.x * rows_per_block;
  const int row_end = min(n, row_begin + rows_per_block);
  const int64_t wpr = (int64_t)G * 4;  // words per row
  // with one activation row, the first iteration's weight loads go out
  // before the activation loads, so the two memory round trips overlap (with
  // more rows the registers held across the activation loads cost more than
  // the overlap gains)
  // Loads go through buffer descriptors of the block's rows: a lane past the
  // last row or past G gets an offset outside the range and reads zeros, so
  // every lane issues the same loads with no branch (a branch whose other
  // side zeroes the same registers makes the compiler wait for each load
  // before the next one is issued).
  const int nrows = max(0, row_end - row_begin);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(packed + (int64_t)row_begin * wpr), 0, (int)(nrows * wpr * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales + (int64_t)row_begin * G), 0, (int)(nrows * G * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(biases + (int64_t)row_begin * G), 0, (int)(nrows * G * 2), 0x00020000);
  uint4 wv[U];
  float sv[U], bv[U];
  auto load_rows = [&](int r0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int lr = r0 - row_begin + u * RPI + slot;  // row within the block
      const bool ok = gv && lr < nrows;
      const uint32_t ow = ok ? (uint32_t)(lr * wpr + 4 * g) * 4u : 0xFFFFFFF0u;
      const uint32_t os = ok ? (uint32_t)(lr * G + g) * 2u : 0xFFFFFFF0u;
      typedef uint32_t v4u __attribute__((ext_vector_type(4)));
      const v4u w = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)ow, 0, 0));
      wv[u] = make_uint4(w.x, w.y, w.z, w.w);
      sv[u] = bf16_to_f32((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)os, 0, 0));
      bv[u] = bf16_to_f32((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, (int)os, 0, 0));
    }
  };
  if constexpr (MV == 1) load_rows(row_begin);

  uint32_t xp[MV][16];
  float xsum[MV];
#pragma unroll
  for (int v = 0; v < MV; ++v) {
    xsum[v] = 0.f;
    if (gv) {
      const uint4* xs = reinterpret_cast<const uint4*>(x + v * x_stride + (int64_t)g * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 e = xs[j];
        x_to_pairs(e, xp[v][4 * j + 0], xp[v][4 * j + 1], xp[v][4 * j + 2], xp[v][4 * j + 3]);
        xsum[v] += x_sum8(e);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) xp[v][j] = 0u;
    }
  }

  for (int r0 = row_begin; r0 < row_end; r0 += ROWS) {
    if (MV != 1 || r0 != row_begin) load_rows(r0);
    float part[U][MV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int v = 0; v < MV; ++v) part[u][v] = fmaf(sv[u], group_dot(wv[u], xp[v]), bv[u] * xsum[v]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
#pragma unroll
        for (int off = C / 2; off > 0; off >>= 1) part[u][v] += __shfl_xor(part[u][v], off, 64);
      }
    }
    if (c == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int v = 0; v < MV; ++v) red[wave][v * ROWS + u * RPI + slot] = part[u][v];
      }
    }
    __syncthreads();
    // (a block may have fewer threads than ROWS * MV outputs)
    for (int idx = threadIdx.x; idx < ROWS * MV; idx += blockDim.x) {
      const int rr = idx % ROWS;
      const int v = idx / ROWS;
      float s = 0.f;
      for (int w2 = 0; w2 < nwaves; ++w2) s += red[w2][idx];
      const int row = r0 + rr;
      if (row < row_end) store_out<OUT_F32>(y, v * y_stride + row, s);
    }
    __syncthreads();
  }
}

// groups per batch of weight loads in the small-GEMM MFMA kernel
#ifndef Q4_GEMM_KB
#define Q4_GEMM_KB 4
#endif
constexpr int kGemmKB = Q4_GEMM_KB;

// ---------------------------------------------------------------------------
// Small GEMM, M in [5, 16] activation rows, on MFMA.
//
// One v_mfma_f32_16x16x32_bf16 covers exactly one group (32 inputs) for 16
// activation rows (A operand, zero-padded past m) and 16 weight rows (B
// operand = the 32 codes as exact bf16 integers). The group's scale and bias
// are applied to the fp32 tile afterwards, D*s + b*X_g, where the group sums
// X_g come from a second MFMA against a B of ones. Lane l of the MFMA holds
// A/B k-block l/16 (8 inputs = one packed word) for row l%16 and receives the
// outputs D[4*(l/16)+i][l%16], i < 4. The 8 inputs of a k-block use the same
// re-pairing on both operands, so the contraction is unchanged.
//
// A block has S waves; wave w owns groups [w*GS, (w+1)*GS) and keeps its
// activation tile in registers; the block walks T tiles of 16 weight rows and
// the S waves' tiles are summed in fixed order through LDS.
// More than 16 activation rows (a prompt's frames, up to 64) run as mtiles
// tiles of 16 rows in the same launch, one block per (row block, tile). The
// tiles of a row block go to blocks that the dispatcher deals to the same
// XCD (it deals blocks to the nxcc XCDs in turn), so that the row block's
// weights, read from HBM by the first of them, can be served from that XCD's
// L2 to the others (measured: M=50 step 8.04 -> 6.20 ms against one launch
// per tile).
// SB16: G is a multiple of 8, so a row's scales (and biases) of the wave's GS
// groups are 16-byte aligned runs, loaded once per row with 16-byte loads
// (GS / 8 per row) instead of one 2-byte load per group and batch: 16 rows
// per load either way, so that cuts the cache lines looked up per wave by 8.
// The product's body for block `bid` of its grid (the kernels below pass
// their own block index, or a block's index within one product of a batch).
template <int GS, int T, bool OUT_F32, bool SB16, bool TILED>
__device__ __forceinline__ void gemm_mfma_body(int bid, const uint16_t* __restrict__ x, int m,
                                               const uint32_t* __restrict__ packed,
                                               const uint16_t* __restrict__ scales,
                                               const uint16_t* __restrict__ biases, int n, int G,
                                               void* __restrict__ y, int mtiles, int nxcc) {
  extern __shared__ float red_dyn[];  // [nwaves][T][4][64], then each wave's code staging
  int rblk = bid, tile = 0;
  if constexpr (TILED) {
    const int b = bid, span = nxcc * mtiles;
    rblk = (b / span) * nxcc + b % nxcc;
    tile = (b / nxcc) % mtiles;
    if (rblk * 16 * T >= n) return;  // (past the last row block: the grid is a whole number of XCD rounds)
  }
  const int nbase = rblk * 16 * T;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int r16 = lane & 15;
  const int kb = lane >> 4;
  const int g0 = wave * GS;
  const int gcount = max(0, min(G - g0, GS));
  const int64_t K = (int64_t)G * 32;
  if constexpr (TILED) {
    x += (int64_t)tile * 16 * K;
    m = min(16, m - 16 * tile);
  }

  // All loads go through buffer descriptors: lanes past m, G or n get an
  // offset outside the range and read zeros, so the loads carry no branch
  // and the compiler can keep many in flight.
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, (int)(m * K * 2), 0x00020000);
  // Activations are loaded a whole cache line per row: the load for the
  // wave's groups gi, gi + 1 and half h covers rows 8 h .. 8 h + 7, 128
  // contiguous bytes each (8 lines per load instead of 16 for one group of
  // all 16 rows), and passes through the LDS staging area into the MFMA
  // layout (x_unpack, below).
  auto x_line = [&](int gi, int h) {
    const int row = 8 * h + (lane >> 3);
    const int seg = lane & 7;  // 16 bytes: group gi + seg / 4, inputs 8 (seg % 4) ..
    const int g = gi + (seg >> 2);
    const bool ok = g < gcount && row < m;
    const uint32_t off = ok ? (uint32_t)(((int64_t)row * K + (int64_t)(g0 + g) * 32 + 8 * (seg & 3)) * 2)
                            : 0xFFFFFFF0u;
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0));
  };
  auto x_pairs = [](const u32x4_t e4) {
    uint32_t p02, p46, p13, p57;
    x_to_pairs(make_uint4(e4.x, e4.y, e4.z, e4.w), p02, p46, p13, p57);
    return u32x4_t{p02, p46, p13, p57};
  };
  // Up to 16 groups per wave keep their activation tile in registers for the
  // whole kernel; wider waves load it with each batch of weights instead
  // (holding 24 or 32 tiles would spill).
  constexpr bool kXReg = GS <= 16;
  u32x4_t a[kXReg ? GS : 1];
  // (the register tile's loads: j covers groups 2 (j / 2), + 1, half j % 2;
  // unpacked before the first batch)
  constexpr int kXLoads = kXReg ? GS : 1;
  u32x4_t xr[kXLoads];
  if constexpr (kXReg) {
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) xr[j] = x_line(2 * (j >> 1), j & 1);
  }
  const u32x4_t ones = u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = zero;

  const int64_t wpr = (int64_t)G * 4;
  const int tile_rows = max(0, min(16 * T, n - nbase));
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(packed + (int64_t)nbase * wpr), 0, (int)(tile_rows * wpr * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales + (int64_t)nbase * G), 0, (int)(tile_rows * G * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(biases + (int64_t)nbase * G), 0, (int)(tile_rows * G * 2), 0x00020000);
  // Weight loads in batches of KB groups, one batch ahead of the arithmetic
  // (written out so that every wait is for exactly the batch in use); groups
  // past this wave's share read zeros (scale and bias 0: no term).
  constexpr int KB = kGemmKB;
  static_assert(GS % KB == 0, "group batches");
  // Codes are loaded 16 bytes (one group of one row) per lane, lanes along a
  // row's consecutive groups, and passed through a per-wave LDS staging area
  // to the lanes whose MFMA operand they are (lane (row, kb) needs word kb of
  // each group of its row). Staging rows are padded by 16 bytes so that the
  // 64 word reads hit 64 different banks.
  constexpr int kPieces = 16 * KB;                       // 16-byte pieces per batch and row tile
  constexpr int kPerLane = (kPieces + 63) / 64;
  constexpr int kRowWords = KB * 4 + 4;
  uint32_t* stage = reinterpret_cast<uint32_t*>(red_dyn + nwaves * T * 256) + wave * (2 * T * 16 * kRowWords);
  u32x4_t wq[2][T][kPerLane];
  uint32_t sb[2][T][SB16 ? 1 : KB], bb[2][T][SB16 ? 1 : KB];
  constexpr int kSW = SB16 ? GS / 8 : 1;  // 16-byte runs of scales per row and wave
  u32x4_t sw[T][kSW], bw[T][kSW];
  if constexpr (SB16) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int c = 0; c < kSW; ++c) {
        // (past the wave's groups or the row tile: zeros, or groups weighed zero below)
        const int lr = 16 * t + r16;
        const uint32_t os = g0 + 8 * c < G ? (uint32_t)((lr * G + g0 + 8 * c) * 2) : 0xFFFFFFF0u;
        sw[t][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)os, 0, 0));
        bw[t][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)os, 0, 0));
      }
    }
  }
  // two groups' activations of 16 rows (the loads of halves 0 and 1) into
  // the MFMA layout, re-paired: rows of 8 segments padded to 36 words
  auto x_unpack = [&](const u32x4_t lo, const u32x4_t hi, u32x4_t& a0, u32x4_t& a1) {
    constexpr int kXRow = 36;
    static_assert(16 * kXRow <= 2 * T * 16 * kRowWords, "two groups fit the staging area");
    *reinterpret_cast<u32x4_t*>(stage + (lane >> 3) * kXRow + (lane & 7) * 4) = lo;
    *reinterpret_cast<u32x4_t*>(stage + (8 + (lane >> 3)) * kXRow + (lane & 7) * 4) = hi;
    a0 = x_pairs(*reinterpret_cast<const u32x4_t*>(stage + r16 * kXRow + kb * 4));
    a1 = x_pairs(*reinterpret_cast<const u32x4_t*>(stage + r16 * kXRow + (4 + kb) * 4));
  };
  static_assert(KB % 2 == 0 && GS % 2 == 0, "activations go in pairs of groups");
  u32x4_t xb[2][kXReg ? 1 : KB];
  auto load_batch = [&](int i0, int buf) {
#pragma unroll
    for (int ii = 0; ii < KB; ++ii) {
      if constexpr (!kXReg) xb[buf][ii] = x_line(i0 + 2 * (ii >> 1), ii & 1);
      if constexpr (!SB16) {
        const bool gok = i0 + ii < gcount;
        const int g = g0 + i0 + ii;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int lr = 16 * t + r16;  // row within the tile (the range ends at n)
          const uint32_t os = gok ? (uint32_t)((lr * G + g) * 2) : 0xFFFFFFF0u;
          sb[buf][t][ii] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)os, 0, 0);
          bb[buf][t][ii] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, (int)os, 0, 0);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        const int pc = lane + 64 * j;
        const int prow = pc / KB, pg = pc % KB;
        const bool ok = pc < kPieces && i0 + pg < gcount;
        const uint32_t ow = ok ? (uint32_t)(((16 * t + prow) * wpr + 4 * (g0 + i0 + pg)) * 4) : 0xFFFFFFF0u;
        wq[buf][t][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)ow, 0, 0));
      }
    }
  };
  load_batch(0, 0);
#pragma unroll
  for (int i0 = 0; i0 < GS; i0 += KB) {
    const int buf = (i0 / KB) & 1;
    if (i0 + KB < GS) load_batch(i0 + KB, buf ^ 1);
    // (the staging area is free here: the batch's codes go in below, and a
    // wave's LDS accesses complete in order)
    if (kXReg && i0 == 0) {
#pragma unroll
      for (int p = 0; p < kXLoads / 2; ++p) x_unpack(xr[2 * p], xr[2 * p + 1], a[2 * p], a[2 * p + 1]);
    }
    u32x4_t ab[kXReg ? 1 : KB];
    if constexpr (!kXReg) {
#pragma unroll
      for (int p = 0; p < KB / 2; ++p) x_unpack(xb[buf][2 * p], xb[buf][2 * p + 1], ab[2 * p], ab[2 * p + 1]);
    }
    // this batch's codes into the staging area, then each lane's words out
    // (a wave's LDS accesses complete in order)
    uint32_t* sbuf = stage + buf * (T * 16 * kRowWords);
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        const int pc = lane + 64 * j;
        if (pc < kPieces)
          *reinterpret_cast<u32x4_t*>(sbuf + (t * 16 + pc / KB) * kRowWords + (pc % KB) * 4) = wq[buf][t][j];
      }
    }
#pragma unroll
    for (int ii = 0; ii < KB; ++ii) {
      u32x4_t ai;
      if constexpr (kXReg) {
        ai = a[i0 + ii];
      } else {
        ai = ab[ii];
      }
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, ai);
      const f32x4_t xg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, ones), zero, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        uint32_t q02, q46, q13, q57;
        word_to_bf16_pairs(sbuf[(t * 16 + r16) * kRowWords + ii * 4 + kb], q02, q46, q13, q57);
        const u32x4_t bq = u32x4_t{q02, q46, q13, q57};
        const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bq), zero, 0, 0, 0);
        float s, b;
        if constexpr (SB16) {
          // group gi of the wave: half gi % 2 of word (gi % 8) / 2 of run gi / 8;
          // groups past the wave's share weigh zero
          const int gi = i0 + ii;
          const uint32_t ws = sw[t][gi / 8][(gi % 8) / 2], wb = bw[t][gi / 8][(gi % 8) / 2];
          const bool gok = gi < gcount;
          s = gok ? __uint_as_float(gi % 2 ? ws & 0xFFFF0000u : ws << 16) : 0.f;
          b = gok ? __uint_as_float(gi % 2 ? wb & 0xFFFF0000u : wb << 16) : 0.f;
        } else {
          s = bf16_to_f32(sb[buf][t][ii]);
          b = bf16_to_f32(bb[buf][t][ii]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t][j] = fmaf(s, d[j], fmaf(b, xg[j], acc[t][j]));
      }
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) red_dyn[((wave * T + t) * 4 + j) * 64 + lane] = acc[t][j];
  __syncthreads();
  for (int idx = threadIdx.x; idx < T * 256; idx += blockDim.x) {
    float s = 0.f;
    for (int w2 = 0; w2 < nwaves; ++w2) s += red_dyn[w2 * T * 256 + idx];
    const int l = idx & 63;
    const int j = (idx >> 6) & 3;
    const int t = idx >> 8;
    const int mi = 4 * (l >> 4) + j;
    const int row = nbase + 16 * t + (l & 15);
    if (mi < m && row < n) store_out<OUT_F32>(y, (int64_t)(16 * tile + mi) * n + row, s);
  }
}

template <int GS, int T, bool OUT_F32, bool SB16, bool TILED>
__global__ void __launch_bounds__(1024) gemm_mfma_kernel(const uint16_t* __restrict__ x, int m,
                                                          const uint32_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ biases,
                                                          int n, int G, void* __restrict__ y, int mtiles,
                                                          int nxcc) {
  gemm_mfma_body<GS, T, OUT_F32, SB16, TILED>(blockIdx.x, x, m, packed, scales, biases, n, G, y, mtiles, nxcc);
}

// A batch of independent products of one shape class (same m <= 16 rows, same
// k) in one launch: each product's blocks follow the last one's, so the grid
// has no gap between products. `owner` gives each block its product.
struct GemmBatchItem {
  const uint16_t* x;
  const uint32_t* packed;
  const uint16_t* scales;
  const uint16_t* biases;
  void* y;
  int32_t n;
  int32_t block_start;  // its first block in the grid
};
static_assert(sizeof(GemmBatchItem) == 48, "the plan's item layout");

template <int GS, bool OUT_F32, bool SB16>
__global__ void __launch_bounds__(1024) gemm_batch_kernel(const GemmBatchItem* __restrict__ items,
                                                          const uint16_t* __restrict__ owner, int m, int G) {
  const GemmBatchItem* it = items + owner[blockIdx.x];
  gemm_mfma_body<GS, 1, OUT_F32, SB16, false>(static_cast<int>(blockIdx.x) - it->block_start, it->x, m,
                                              it->packed, it->scales, it->biases, it->n, G, it->y, 1, 1);
}

// ---------------------------------------------------------------------------
// Packed-embedding gather and stream sum: the step's input vector is the sum
// of one packed embedding row per token stream ("NVIDIA PersonaPlex 7B on
// Apple Silicon", pipeline figure: 17 streams summed; "personaplex-edge-q4"
// model card, introduction: embeddings stay packed).
//
// Lane g of a block owns group g of a frame's output row (32 values in
// registers); it gathers that group of every stream's row, kEmbedBatch
// streams' loads in flight at a time, and adds the dequantized values in
// stream order in fp32. Every load goes through a buffer descriptor of the
// whole table: a token outside [0, rows) gets an offset past the range and
// reads zeros (code 0, scale 0, bias 0: nothing added).
constexpr int kEmbedMaxTables = 32;
constexpr int kEmbedBatch = 17;  // the model's 17 streams: one round of loads
struct EmbedTables {
  const uint32_t* packed[kEmbedMaxTables];
  const uint16_t* scales[kEmbedMaxTables];
  const uint16_t* biases[kEmbedMaxTables];
  int32_t rows[kEmbedMaxTables];
  int32_t count;
};

template <bool OUT_F32>
__global__ void __launch_bounds__(64) embed_sum_kernel(const int32_t* __restrict__ tokens, EmbedTables tabs,
                                                       int G, int tiles, void* __restrict__ y) {
  const int f = blockIdx.x / tiles;
  const int g = (blockIdx.x - f * tiles) * 64 + threadIdx.x;
  const bool gv = g < G;
  const int nt = tabs.count;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  for (int t0 = 0; t0 < nt; t0 += kEmbedBatch) {
    uint4 w[kEmbedBatch];
    uint32_t sv[kEmbedBatch], bv[kEmbedBatch];
#pragma unroll
    for (int b = 0; b < kEmbedBatch; ++b) {
      const int t = t0 + b;
      int tok = -1, rows = 0;
      const uint32_t* pk = nullptr;
      const uint16_t* sc = nullptr;
      const uint16_t* bi = nullptr;
      if (t < nt) {
        tok = tokens[(int64_t)f * nt + t];
        rows = tabs.rows[t];
        pk = tabs.packed[t];
        sc = tabs.scales[t];
        bi = tabs.biases[t];
      }
      const bool ok = gv && tok >= 0 && tok < rows;
      const uint32_t e = ok ? (uint32_t)tok * (uint32_t)G + (uint32_t)g : 0u;
      const __amdgpu_buffer_rsrc_t rw =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(pk), 0, rows * G * 16, 0x00020000);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sc), 0, rows * G * 2, 0x00020000);
      const __amdgpu_buffer_rsrc_t rb =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(bi), 0, rows * G * 2, 0x00020000);
      const u32x4_t v = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? (int)(e * 16u) : (int)0xFFFFFFF0, 0, 0));
      w[b] = make_uint4(v.x, v.y, v.z, v.w);
      sv[b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, ok ? (int)(e * 2u) : (int)0xFFFFFFF0, 0, 0);
      bv[b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, ok ? (int)(e * 2u) : (int)0xFFFFFFF0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < kEmbedBatch; ++b) {
      // w_hat = s * q + b: the product is exact, so the fma rounds once
      const float sc = bf16_to_f32(sv[b]), bi = bf16_to_f32(bv[b]);
      const uint32_t ws[4] = {w[b].x, w[b].y, w[b].z, w[b].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[8 * j + n] += fmaf(sc, (float)((ws[j] >> (4 * n)) & 0xFu), bi);
    }
  }
  if (!gv) return;
  const int64_t base = ((int64_t)f * G + g) * 32;
  if constexpr (OUT_F32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(y) + base);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
  } else {
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + base);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t p[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        p[h] = (uint32_t)f32_to_bf16_rne(acc[8 * i + 2 * h]) | ((uint32_t)f32_to_bf16_rne(acc[8 * i + 2 * h + 1]) << 16);
      dst[i] = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
}

}  // namespace q4k
