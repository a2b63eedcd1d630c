// Decode attention over the KV cache for one layer (gfx950). Included by
// q4_api.hip after q4_kernels.h.
//
// One decoding step of a layer takes the step's q, k and v (32 heads x 128,
// bf16), turns q and k by the rotary embedding at the step's position (the
// RoPE offset, a step input: "NVIDIA PersonaPlex 7B on Apple Silicon",
// optimisation list), appends k and v to the layer's caches at that position
// (the ONNX bundle's README, How to use: the step carries the K and V caches
// [layers][1][32][T][128] explicitly), and attends with the one query per
// head over cache positions 0..pos: softmax(q . k / sqrt(D)) . v.
//
// One launch, attn_decode_kernel: block (head, split) takes a contiguous
// range of positions.
//  - It issues the loads of its first batch of key and value rows at once
//    (16-byte pieces, D/8 lanes per position, kAttnBatch positions per lane),
//    and meanwhile its first wave turns q (and, in the block that holds
//    position pos, the new k) by the rotary embedding: the angle
//    pos * theta^(-2i/D), its cosine and sine and the rotated pair in fp64
//    with explicit rounding, then fp32, then bf16 -- the same roundings as a
//    plain double implementation. That block writes the new cache rows and
//    uses the new key and value from LDS (no other block reads them).
//  - Scores, a running maximum and the exp-weighted value sums per group of
//    positions (online softmax over the batches, fixed order), then the
//    groups combined in group order: the split's (max, sum, weighted values)
//    go to the workspace with device-coherent stores.
//  - The head's last split to finish (a device-scope counter per head)
//    rescales the splits to their common maximum, adds them in split order,
//    writes the output and resets the counter.
// Every sum runs in a fixed order: results are deterministic.
#pragma once

namespace q4k {

constexpr int kAttnMaxSplits = 64;
constexpr int kAttnThreads = 256;
constexpr int kAttnBatch = 8;  // positions per lane whose loads are in flight together

// Workspace: the heads' split counters (zero between calls), the rotated q
// (bf16 [heads][D], written by split 0 of each head), then the splits'
// partials [heads][kAttnMaxSplits][D + 2] floats: {max, sum, D values}.
__host__ __device__ constexpr int64_t attn_ws_q_offset(int64_t heads) { return ((heads * 4 + 255) / 256) * 256; }
__host__ __device__ constexpr int64_t attn_ws_part_offset(int64_t heads, int64_t d) {
  return attn_ws_q_offset(heads) + ((heads * d * 2 + 255) / 256) * 256;
}

__device__ __forceinline__ uint32_t attn_counter_add(uint32_t* p) {
  return __hip_atomic_fetch_add((Q4_GLOBAL uint32_t*)p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(kAttnThreads) attn_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, int cap, int pos, double theta, int chunk,
    int splits, unsigned char* __restrict__ ws, void* __restrict__ out) {
  constexpr int kC = D / 8;                  // 16-byte pieces per row (lanes per position)
  constexpr int kR = kAttnThreads / kC;      // groups of positions (one position per group and step)
  constexpr int kB = kAttnBatch;             // positions per lane per batch
  static_assert(kC == 16 || kC == 8, "head width 128 or 64");
  static_assert(D <= kAttnThreads && kAttnMaxSplits <= kAttnThreads, "one lane per value");
  __shared__ float q_s[D];
  __shared__ uint32_t knew_s[D / 2], vnew_s[D / 2];   // the new position's rotated key and value (bf16 pairs)
  __shared__ float g_m[kR], g_l[kR];
  __shared__ float g_acc[kR][D];
  __shared__ float c_f[kAttnMaxSplits];
  __shared__ float c_sum;
  __shared__ uint32_t is_last;
  const int h = blockIdx.x, s = blockIdx.y;
  const int t = threadIdx.x, c = t % kC, r = t / kC;
  const int npos = pos + 1;
  const int lo = min(npos, s * chunk), hi = min(npos, lo + chunk);
  const int n = hi - lo;
  const bool owns_new = pos >= lo && pos < hi;
  const uint16_t* kh = k_cache + (int64_t)h * cap * D;
  const uint16_t* vh = v_cache + (int64_t)h * cap * D;
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
  float* part = reinterpret_cast<float*>(ws + attn_ws_part_offset(gridDim.x, D));

  // the cache rows of the range, through buffer descriptors of exactly the
  // range (position lo + p for p = p0 + b kR + r; a lane past the range
  // reads zeros, with no branch, so all its loads are in flight together;
  // the new position's row is read too but not used), with the streaming
  // hint (each row is read once per step: 5% faster at 4096 positions)
  const __amdgpu_buffer_rsrc_t rk = byte_range(kh + (int64_t)lo * D, (uint32_t)(n * D * 2));
  const __amdgpu_buffer_rsrc_t rv = byte_range(vh + (int64_t)lo * D, (uint32_t)(n * D * 2));
  uint4 kv[kB], vv[kB];
  auto load_batch = [&](int p0) {
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int p = p0 + b * kR + r;
      const uint32_t off = p < n ? (uint32_t)(p * D + 8 * c) * 2u : 0xFFFFFF00u;
      kv[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)off, 0, kAuxNt));
      vv[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)off, 0, kAuxNt));
    }
  };
  load_batch(0);

  // rotary embedding (first wave, one lane per pair) while the loads are out
  if (t < D / 2) {
    const int i = t;
    const double angle = __dmul_rn((double)pos, pow(theta, -(double)(2 * i) / (double)D));
    const double cs = cos(angle), sn = sin(angle);
    auto turn = [&](const uint16_t* src) {
      const double x0 = (double)bf16_to_f32(src[2 * i]), x1 = (double)bf16_to_f32(src[2 * i + 1]);
      const double r0 = __dsub_rn(__dmul_rn(x0, cs), __dmul_rn(x1, sn));
      const double r1 = __dadd_rn(__dmul_rn(x0, sn), __dmul_rn(x1, cs));
      return (uint32_t)f32_to_bf16_rne(__double2float_rn(r0)) |
             ((uint32_t)f32_to_bf16_rne(__double2float_rn(r1)) << 16);
    };
    const uint32_t qp = turn(q + (int64_t)h * D);
    q_s[2 * i] = bf16_to_f32(qp & 0xFFFFu);
    q_s[2 * i + 1] = bf16_to_f32(qp >> 16);
    if (s == 0) reinterpret_cast<uint32_t*>(ws + attn_ws_q_offset(gridDim.x))[(int64_t)h * (D / 2) + i] = qp;
    if (owns_new) {
      const uint32_t kp = turn(k_new + (int64_t)h * D);
      const uint32_t vp = (uint32_t)v_new[(int64_t)h * D + 2 * i] | ((uint32_t)v_new[(int64_t)h * D + 2 * i + 1] << 16);
      knew_s[i] = kp;
      vnew_s[i] = vp;
      const int64_t row = ((int64_t)h * cap + pos) * D;
      reinterpret_cast<uint32_t*>(k_cache + row)[i] = kp;
      reinterpret_cast<uint32_t*>(v_cache + row)[i] = vp;
    }
  }
  __syncthreads();
  float qf[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qf[j] = q_s[8 * c + j];
  const float scale = 1.0f / sqrtf((float)D);

  // online softmax of the group's positions, batch by batch
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int p0 = 0; p0 < n; p0 += kR * kB) {
    if (p0 > 0) load_batch(p0);
    float sc[kB];
    float mb = -INFINITY;
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int p = p0 + b * kR + r;
      const bool is_new = lo + p == pos;
      uint4 kw4 = kv[b];
      if (is_new) kw4 = make_uint4(knew_s[4 * c], knew_s[4 * c + 1], knew_s[4 * c + 2], knew_s[4 * c + 3]);
      const uint32_t kw[4] = {kw4.x, kw4.y, kw4.z, kw4.w};
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dot = fmaf(qf[2 * j], bf16_to_f32(kw[j] & 0xFFFFu), dot);
        dot = fmaf(qf[2 * j + 1], bf16_to_f32(kw[j] >> 16), dot);
      }
#pragma unroll
      for (int off = kC / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
      sc[b] = p < n ? dot * scale : -INFINITY;
      mb = fmaxf(mb, sc[b]);
    }
    const float m_new = fmaxf(m, mb);
    if (m_new != -INFINITY) {
      const float corr = m == -INFINITY ? 0.f : expf(m - m_new);
      l *= corr;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= corr;
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const int p = p0 + b * kR + r;
        const float e = sc[b] == -INFINITY ? 0.f : expf(sc[b] - m_new);
        uint4 vw4 = vv[b];
        if (lo + p == pos) vw4 = make_uint4(vnew_s[4 * c], vnew_s[4 * c + 1], vnew_s[4 * c + 2], vnew_s[4 * c + 3]);
        const uint32_t vw[4] = {vw4.x, vw4.y, vw4.z, vw4.w};
        l += e;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] = fmaf(e, bf16_to_f32(vw[j] & 0xFFFFu), acc[2 * j]);
          acc[2 * j + 1] = fmaf(e, bf16_to_f32(vw[j] >> 16), acc[2 * j + 1]);
        }
      }
      m = m_new;
    }
  }
  // the groups, combined in group order
  if (c == 0) {
    g_m[r] = m;
    g_l[r] = l;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) g_acc[r][8 * c + j] = acc[j];
  __syncthreads();
  float* mine = part + ((int64_t)h * kAttnMaxSplits + s) * (D + 2);
  if (t < D) {
    float M = -INFINITY;
    for (int g = 0; g < kR; ++g) M = fmaxf(M, g_m[g]);
    float A = 0.f, L = 0.f;
    for (int g = 0; g < kR; ++g) {
      const float f = g_m[g] == -INFINITY ? 0.f : expf(g_m[g] - M);
      A = fmaf(g_acc[g][t], f, A);
      L = fmaf(g_l[g], f, L);
    }
    coh_store(reinterpret_cast<uint32_t*>(mine) + 2 + t, __float_as_uint(A));
    if (t == 0) {
      coh_store(reinterpret_cast<uint32_t*>(mine), __float_as_uint(M));
      coh_store(reinterpret_cast<uint32_t*>(mine) + 1, __float_as_uint(L));
    }
  }
  // every store of this split is complete before the head's counter moves
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0) is_last = attn_counter_add(counters + h) == (uint32_t)(splits - 1) ? 1u : 0u;
  __syncthreads();
  if (is_last == 0u) return;
  // the head's last split: all splits' partials, rescaled to their common
  // maximum and added in split order (device-coherent loads, all of a lane's
  // in flight together)
  const float* hp = part + (int64_t)h * kAttnMaxSplits * (D + 2);
  const __amdgpu_buffer_rsrc_t rp = byte_range(hp, (uint32_t)(splits * (D + 2) * 4));
  __shared__ float c_m[kAttnMaxSplits], c_l[kAttnMaxSplits];
  if (t < splits) {
    c_m[t] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rp, t * (D + 2) * 4, 0, kAuxSc1));
    c_l[t] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rp, (t * (D + 2) + 1) * 4, 0, kAuxSc1));
  }
  __syncthreads();
  if (t == 0) {
    float M = -INFINITY;
    for (int i = 0; i < splits; ++i) M = fmaxf(M, c_m[i]);
    float L = 0.f;
    for (int i = 0; i < splits; ++i) {
      const float f = c_m[i] == -INFINITY ? 0.f : expf(c_m[i] - M);
      L = fmaf(c_l[i], f, L);
      c_f[i] = f;
    }
    c_sum = L;
    coh_store(counters + h, 0u);
  }
  __syncthreads();
  if (t < D) {
    float A = 0.f;
    for (int i0 = 0; i0 < splits; i0 += 16) {
      float v[16];
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        // (splits past the last read zeros: outside the range)
        const uint32_t off = i0 + b < splits ? (uint32_t)(((i0 + b) * (D + 2) + 2 + t) * 4) : 0xFFFFFF00u;
        v[b] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rp, (int)off, 0, kAuxSc1));
      }
#pragma unroll
      for (int b = 0; b < 16; ++b)
        if (i0 + b < splits) A = fmaf(v[b], c_f[i0 + b], A);
    }
    store_out<OUT_F32>(out, (int64_t)h * D + t, A / c_sum);
  }
}

}  // namespace q4k
