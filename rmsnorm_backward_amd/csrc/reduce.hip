// reduce.hip -- kernel B launches (fixed-order sum over row groups) and the
// copy probe used for bandwidth and counter calibration.
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

}  // namespace nb
