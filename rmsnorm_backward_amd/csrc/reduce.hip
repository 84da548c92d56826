// reduce.hip -- kernel B launches (fixed-order sum over row groups), the
// copy probe used for counter calibration, and the triad probe that measures
// the streaming ceiling kernel A is judged against.
#include "nb_device.hpp"
#include "nb_launch.hpp"
#include "norm_bwd.h"

namespace nb {

// A plain grid-stride 16-byte copy (measurement aid only).
__global__ __launch_bounds__(256)
void copy_probe_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

// Streaming ceiling for kernel A's access mix: two operands read and one
// written, all with 16-byte non-temporal accesses, as kernel A streams x and
// dy in and dx out. c = a + b on 32-bit words (the add only makes the store
// depend on both loads). Thread t of block b handles vectors
// i = (b * 256 * U) + t + u * 256 + k * (grid * 256 * U) for u < U: a
// workgroup's U loads per operand are each 4 KiB contiguous, issued before
// any add. Every access is at i < n16.
template <int U>
__global__ __launch_bounds__(256)
void triad_probe_kernel(const u32x4* __restrict__ a, const u32x4* __restrict__ b,
                        u32x4* __restrict__ c, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  for (; i + (int64_t)(U - 1) * 256 < n16; i += stride) {
    u32x4 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      va[u] = __builtin_nontemporal_load(a + i + u * 256);
      vb[u] = __builtin_nontemporal_load(b + i + u * 256);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(va[u] + vb[u], c + i + u * 256);
  }
  // the part of this thread's last stride that holds fewer than U vectors
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = i + (int64_t)u * 256;
    if (j < n16) c[j] = a[j] + b[j];
  }
}

hipError_t launch_reduce(int wgrad_dtype, const float* ws, int64_t G, int N, void* dgamma,
                         void* dbeta, int accumulate, int ws_stream, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kReduceCols - 1) / kReduceCols), dbeta ? 2u : 1u);
  const dim3 block(kReduceWaves * 64);
  switch (wgrad_dtype) {
    case NORM_BWD_F32:
      hipLaunchKernelGGL(reduce_partials_kernel<TF32>, grid, block, 0, stream, ws, G, N, dgamma,
                         dbeta, accumulate, ws_stream);
      break;
    case NORM_BWD_F16:
      hipLaunchKernelGGL(reduce_partials_kernel<TF16>, grid, block, 0, stream, ws, G, N, dgamma,
                         dbeta, accumulate, ws_stream);
      break;
    case NORM_BWD_BF16:
      hipLaunchKernelGGL(reduce_partials_kernel<TBF16>, grid, block, 0, stream, ws, G, N, dgamma,
                         dbeta, accumulate, ws_stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_triad(const void* a, const void* b, void* c, size_t bytes, int grid,
                        int unroll, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const u32x4* pa = static_cast<const u32x4*>(a);
  const u32x4* pb = static_cast<const u32x4*>(b);
  u32x4* pc = static_cast<u32x4*>(c);
  const dim3 g((unsigned)grid), blk(256);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(triad_probe_kernel<1>, g, blk, 0, stream, pa, pb, pc, n16); break;
    case 2: hipLaunchKernelGGL(triad_probe_kernel<2>, g, blk, 0, stream, pa, pb, pc, n16); break;
    case 4: hipLaunchKernelGGL(triad_probe_kernel<4>, g, blk, 0, stream, pa, pb, pc, n16); break;
    case 8: hipLaunchKernelGGL(triad_probe_kernel<8>, g, blk, 0, stream, pa, pb, pc, n16); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nb
