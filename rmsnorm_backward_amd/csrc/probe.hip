// probe.hip -- the streaming probe under a chosen cache policy (measurement
// aid): which load and store cache-policy bits let a 2-read:1-write stream
// move fastest on this part.
#include "nb_device.hpp"
#include "nb_launch.hpp"
#include "norm_bwd.h"

namespace nb {

// c = a + b on 32-bit words through raw buffer resources over `bytes` bytes,
// with load cache policy LP and store cache policy SP (the aux operand of
// the buffer builtins: bit 0 sc0, bit 1 nt, bit 4 sc1). One pass: workgroup
// b covers bytes [b * 4096 * U, (b + 1) * 4096 * U); thread t loads the
// vectors at t * 16 + u * 4096 of it for u < U, all before any store. The
// host guarantees bytes is a multiple of 4096 * U and below 2^32, so every
// offset is inside the resource.
template <int LP, int SP, int U>
__global__ __launch_bounds__(256)
void triad_policy_kernel(const void* a, const void* b, void* c, uint32_t bytes) {
  const __amdgpu_buffer_rsrc_t ra = row_rsrc(a, bytes), rb = row_rsrc(b, bytes);
  const __amdgpu_buffer_rsrc_t rc = row_rsrc(c, bytes);
  const uint32_t base = blockIdx.x * 4096u * U + threadIdx.x * 16u;
  u32x4 va[U], vb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    va[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, base + u * 4096u, 0, LP);
    vb[u] = __builtin_amdgcn_raw_buffer_load_b128(rb, base + u * 4096u, 0, LP);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    __builtin_amdgcn_raw_buffer_store_b128(va[u] + vb[u], rc, base + u * 4096u, 0, SP);
}

namespace {

template <int LP, int SP>
hipError_t launch_lp_sp(const void* a, const void* b, void* c, uint32_t bytes, int unroll,
                        hipStream_t s) {
  const dim3 grid(bytes / (4096u * (uint32_t)unroll)), blk(256);
  switch (unroll) {
    case 1: hipLaunchKernelGGL((triad_policy_kernel<LP, SP, 1>), grid, blk, 0, s, a, b, c, bytes); break;
    case 2: hipLaunchKernelGGL((triad_policy_kernel<LP, SP, 2>), grid, blk, 0, s, a, b, c, bytes); break;
    case 4: hipLaunchKernelGGL((triad_policy_kernel<LP, SP, 4>), grid, blk, 0, s, a, b, c, bytes); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int LP>
hipError_t launch_lp(const void* a, const void* b, void* c, uint32_t bytes, int unroll, int sp,
                     hipStream_t s) {
  switch (sp) {
    case 0: return launch_lp_sp<LP, 0>(a, b, c, bytes, unroll, s);
    case 1: return launch_lp_sp<LP, 1>(a, b, c, bytes, unroll, s);
    case 2: return launch_lp_sp<LP, 2>(a, b, c, bytes, unroll, s);
    case 3: return launch_lp_sp<LP, 3>(a, b, c, bytes, unroll, s);
    case 16: return launch_lp_sp<LP, 16>(a, b, c, bytes, unroll, s);
    case 17: return launch_lp_sp<LP, 17>(a, b, c, bytes, unroll, s);
    case 18: return launch_lp_sp<LP, 18>(a, b, c, bytes, unroll, s);
    case 19: return launch_lp_sp<LP, 19>(a, b, c, bytes, unroll, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_triad_policy(const void* a, const void* b, void* c, uint32_t bytes, int unroll,
                               int lp, int sp, hipStream_t s) {
  switch (lp) {
    case 0: return launch_lp<0>(a, b, c, bytes, unroll, sp, s);
    case 1: return launch_lp<1>(a, b, c, bytes, unroll, sp, s);
    case 2: return launch_lp<2>(a, b, c, bytes, unroll, sp, s);
    case 3: return launch_lp<3>(a, b, c, bytes, unroll, sp, s);
    case 16: return launch_lp<16>(a, b, c, bytes, unroll, sp, s);
    case 17: return launch_lp<17>(a, b, c, bytes, unroll, sp, s);
    case 18: return launch_lp<18>(a, b, c, bytes, unroll, sp, s);
    case 19: return launch_lp<19>(a, b, c, bytes, unroll, sp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nb
