// Measurement support (not part of the quantized-product library): a plain
// HBM stream-read kernel that bounds what any kernel reading the same number
// of bytes can reach on this device. Each lane sums 16-byte loads over a
// grid-stride range with several loads in flight, one word per block goes
// out (so the loads cannot be dropped). Built as libq4_ceiling.so; the
// benchmark times it beside the kernels it reports.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL, bool NT>
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  // UNROLL independent 16-byte loads per lane in flight per round
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if constexpr (NT) {
        v[u] = __builtin_nontemporal_load(src + i + u * stride);
      } else {
        v[u] = src[i + u * stride];
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per block: lanes fold their sums through shared memory
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, 16-byte aligned) from device memory `src`
// with `blocks` blocks of 256 threads, `unroll` (1, 2, 4 or 8) loads per lane
// in flight, plain (nontemporal = 0) or streaming-hinted (1) loads; out:
// device uint32 [blocks]. Returns 0, or nonzero on a bad argument or a launch
// error.
int q4_stream_read(const void* src, int64_t bytes, uint32_t* out, int blocks, int unroll, int nontemporal,
                   void* stream) {
  if (!src || !out || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(src);
  const int64_t n16 = bytes / 16;
#define Q4_STREAM_CASE(U)                                                                                     \
  case U:                                                                                                     \
    if (nontemporal)                                                                                          \
      hipLaunchKernelGGL((stream_read_kernel<U, true>), dim3(blocks), dim3(256), 0, st, p, n16, out);       \
    else                                                                                                      \
      hipLaunchKernelGGL((stream_read_kernel<U, false>), dim3(blocks), dim3(256), 0, st, p, n16, out);      \
    break;
  switch (unroll) {
    Q4_STREAM_CASE(1)
    Q4_STREAM_CASE(2)
    Q4_STREAM_CASE(4)
    Q4_STREAM_CASE(8)
    default: return 1;
  }
#undef Q4_STREAM_CASE
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
