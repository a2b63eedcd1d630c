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
// Three launches:
//  - attn_rope_kernel: one lane per (head, pair): the angle pos *
//    theta^(-2i/D), its cosine and sine and the rotated pair in fp64 with
//    explicit rounding (no contraction), then fp32, then bf16 -- the same
//    roundings as a plain double implementation; q goes to the workspace, k
//    and v to the caches;
//  - attn_partial_kernel: block (head, split) takes a contiguous range of
//    positions: the scores q . k of its range into LDS (16 lanes per position,
//    one 16-byte load each), their maximum, exp(s - max) and sum, then the
//    exp-weighted sum of the value rows; its (max, sum, weighted values)
//    go to the workspace;
//  - attn_combine_kernel: per head, the splits rescaled to their common
//    maximum and added in split order.
// Every sum runs in a fixed order: results are deterministic.
#pragma once

namespace q4k {

constexpr int kAttnMaxSplits = 64;
constexpr int kAttnThreads = 256;
constexpr int kAttnBatch = 8;  // positions per lane whose loads are in flight together

template <int D>
__global__ void __launch_bounds__(D / 2) attn_rope_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
                                                        const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_cache,
                                                        uint16_t* __restrict__ v_cache, int cap, int pos, double theta,
                                                        uint16_t* __restrict__ q_rot) {
  const int h = blockIdx.x, i = threadIdx.x;
  const double angle = __dmul_rn((double)pos, pow(theta, -(double)(2 * i) / (double)D));
  const double c = cos(angle), s = sin(angle);
  auto turn = [&](const uint16_t* src, uint16_t* dst) {
    const double x0 = (double)bf16_to_f32(src[2 * i]), x1 = (double)bf16_to_f32(src[2 * i + 1]);
    const double r0 = __dsub_rn(__dmul_rn(x0, c), __dmul_rn(x1, s));
    const double r1 = __dadd_rn(__dmul_rn(x0, s), __dmul_rn(x1, c));
    dst[2 * i] = f32_to_bf16_rne(__double2float_rn(r0));
    dst[2 * i + 1] = f32_to_bf16_rne(__double2float_rn(r1));
  };
  turn(q + (int64_t)h * D, q_rot + (int64_t)h * D);
  const int64_t row = ((int64_t)h * cap + pos) * D;
  turn(k_new + (int64_t)h * D, k_cache + row);
  v_cache[row + 2 * i] = v_new[(int64_t)h * D + 2 * i];
  v_cache[row + 2 * i + 1] = v_new[(int64_t)h * D + 2 * i + 1];
}

// Partial of split s of head h over positions [lo, hi): ws_part[h][s] =
// {max, sum of exp, D weighted values}. chunk: positions per split.
template <int D>
__global__ void __launch_bounds__(kAttnThreads) attn_partial_kernel(const uint16_t* __restrict__ q_rot,
                                                                  const uint16_t* __restrict__ k_cache,
                                                                  const uint16_t* __restrict__ v_cache, int cap,
                                                                  int npos, int chunk, int splits,
                                                                  float* __restrict__ ws_part) {
  constexpr int kC = D / 8;                  // 16-byte pieces per row (lanes per position)
  constexpr int kR = kAttnThreads / kC;      // positions per block-wide step
  static_assert(kC == 16 || kC == 8, "head width 128 or 64");
  extern __shared__ float sm[];              // scores [chunk], then [kR][D] partial sums
  __shared__ float red[kAttnThreads / 64];
  const int h = blockIdx.x, s = blockIdx.y;
  const int t = threadIdx.x, c = t % kC, r = t / kC;
  const int lo = min(npos, s * chunk), hi = min(npos, lo + chunk);
  const int n = hi - lo;
  float* part = ws_part + ((int64_t)h * splits + s) * (D + 2);
  const float scale = 1.0f / sqrtf((float)D);
  // the lane's 8 query values
  const uint4 qv = *reinterpret_cast<const uint4*>(q_rot + (int64_t)h * D + 8 * c);
  const float qf[8] = {bf16_to_f32(qv.x & 0xFFFFu), bf16_to_f32(qv.x >> 16), bf16_to_f32(qv.y & 0xFFFFu),
                       bf16_to_f32(qv.y >> 16),    bf16_to_f32(qv.z & 0xFFFFu), bf16_to_f32(qv.z >> 16),
                       bf16_to_f32(qv.w & 0xFFFFu), bf16_to_f32(qv.w >> 16)};
  const uint16_t* kh = k_cache + (int64_t)h * cap * D;
  const uint16_t* vh = v_cache + (int64_t)h * cap * D;
  float* scores = sm;
  // scores of the range (the kC lanes of a position are consecutive lanes of
  // one wave: a shuffle sum over them), kAttnBatch positions' loads in flight
  // per lane
  for (int p0 = 0; p0 < n; p0 += kR * kAttnBatch) {
    uint4 kv[kAttnBatch];
#pragma unroll
    for (int b = 0; b < kAttnBatch; ++b) {
      const int p = p0 + b * kR + r;
      kv[b] = p < n ? *reinterpret_cast<const uint4*>(kh + (int64_t)(lo + p) * D + 8 * c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < kAttnBatch; ++b) {
      const int p = p0 + b * kR + r;
      const uint32_t kw[4] = {kv[b].x, kv[b].y, kv[b].z, kv[b].w};
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dot = fmaf(qf[2 * j], bf16_to_f32(kw[j] & 0xFFFFu), dot);
        dot = fmaf(qf[2 * j + 1], bf16_to_f32(kw[j] >> 16), dot);
      }
#pragma unroll
      for (int off = kC / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
      if (p < n && c == 0) scores[p] = dot * scale;
    }
  }
  __syncthreads();
  // maximum, then exp(s - max) in place and its sum (fixed orders)
  float mx = -INFINITY;
  for (int p = t; p < n; p += kAttnThreads) mx = fmaxf(mx, scores[p]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < kAttnThreads / 64; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float sum = 0.f;
  for (int p = t; p < n; p += kAttnThreads) {
    const float e = expf(scores[p] - mx);
    scores[p] = e;
    sum += e;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if ((t & 63) == 0) red[t >> 6] = sum;
  __syncthreads();
  // exp-weighted value rows: lane (r, c) takes positions r, r + kR, ... and
  // its 8 dims; the kR partial rows are added in order through LDS
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int p0 = r; p0 < n; p0 += kR * kAttnBatch) {
    uint4 vv[kAttnBatch];
#pragma unroll
    for (int b = 0; b < kAttnBatch; ++b) {
      const int p = p0 + b * kR;
      vv[b] = p < n ? *reinterpret_cast<const uint4*>(vh + (int64_t)(lo + p) * D + 8 * c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < kAttnBatch; ++b) {
      const int p = p0 + b * kR;
      const float w = p < n ? scores[p] : 0.f;
      const uint32_t vw[4] = {vv[b].x, vv[b].y, vv[b].z, vv[b].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = fmaf(w, bf16_to_f32(vw[j] & 0xFFFFu), acc[2 * j]);
        acc[2 * j + 1] = fmaf(w, bf16_to_f32(vw[j] >> 16), acc[2 * j + 1]);
      }
    }
  }
  float* rows = sm + chunk;
#pragma unroll
  for (int j = 0; j < 8; ++j) rows[r * D + 8 * c + j] = acc[j];
  __syncthreads();
  if (t < D) {
    float v = 0.f;
    for (int rr = 0; rr < kR; ++rr) v += rows[rr * D + t];
    part[2 + t] = v;
  }
  if (t == 0) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnThreads / 64; ++w) l += red[w];
    part[0] = n > 0 ? mx : -INFINITY;
    part[1] = l;
  }
}

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(D) attn_combine_kernel(const float* __restrict__ ws_part, int splits,
                                                       void* __restrict__ out) {
  static_assert(D >= kAttnMaxSplits, "one lane per split");
  __shared__ float sm_m[kAttnMaxSplits], sm_f[kAttnMaxSplits], sm_l[kAttnMaxSplits];
  __shared__ float sm_red[2];
  const int h = blockIdx.x, d = threadIdx.x;
  const float* part = ws_part + (int64_t)h * splits * (D + 2);
  // every split's maximum and sum at once, one lane each
  if (d < splits) {
    sm_m[d] = part[d * (D + 2)];
    sm_l[d] = part[d * (D + 2) + 1];
  }
  __syncthreads();
  if (d == 0) {
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, sm_m[s]);
    float L = 0.f;
    for (int s = 0; s < splits; ++s) {
      // (an empty split holds -inf and adds nothing)
      const float f = sm_m[s] == -INFINITY ? 0.f : expf(sm_m[s] - M);
      sm_f[s] = f;
      L = fmaf(sm_l[s], f, L);
    }
    sm_red[0] = L;
  }
  __syncthreads();
  float acc = 0.f;
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) v[b] = s0 + b < splits ? part[(s0 + b) * (D + 2) + 2 + d] : 0.f;
#pragma unroll
    for (int b = 0; b < 8; ++b)
      if (s0 + b < splits) acc = fmaf(v[b], sm_f[s0 + b], acc);
  }
  store_out<OUT_F32>(out, (int64_t)h * D + d, acc / sm_red[0]);
}

}  // namespace q4k
