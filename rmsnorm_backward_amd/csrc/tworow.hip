// tworow.hip -- launches of kernel A's two-rows-per-wave instantiations
// (nb_tworow.hpp): rows that 32 lanes of 16-byte vectors cover exactly, with
// saved statistics.
#include "nb_launch.hpp"
#include "nb_tworow.hpp"

namespace nb {

template <class Tg, int KIND, int C, int NACC, bool WSNT>
hipError_t launch_tworow_one(const LaunchA& a) {
  // a.P rows in flight: P / 2 waves of two rows each
  hipLaunchKernelGGL((dx_partials_tworow_kernel<KIND, Tg, C, NACC, WSNT>), dim3(a.grid),
                     dim3(a.threads), a.lds, a.stream, a.x, a.dy, a.gamma, a.mean, a.rstd, a.dx,
                     a.ws, a.M, a.N, a.ldx, a.ldy, a.ldo, a.G, a.P / 2);
  return hipGetLastError();
}

template <class Tg, int KIND, int NACC>
hipError_t launch_tworow_by_chunks(const LaunchA& a) {
  switch (a.chunks) {
    case 1:
      return a.ws_stream ? launch_tworow_one<Tg, KIND, 1, NACC, true>(a)
                         : launch_tworow_one<Tg, KIND, 1, NACC, false>(a);
    case 3:
      return a.ws_stream ? launch_tworow_one<Tg, KIND, 3, NACC, true>(a)
                         : launch_tworow_one<Tg, KIND, 3, NACC, false>(a);
    default:
      return hipErrorInvalidValue;
  }
}

template <class Tg>
hipError_t launch_tworow(const LaunchA& a) {
  if (a.recompute || !a.vec_full || a.S != 1 || a.P < 2 || a.P % 2 != 0 ||
      a.threads != 32 * a.P || a.threads > kTwoRowMaxThreads)
    return hipErrorInvalidValue;
  if (a.kind == 0)
    return a.nacc == 2 ? launch_tworow_by_chunks<Tg, kLayerNorm, 2>(a)
                       : launch_tworow_by_chunks<Tg, kLayerNorm, 1>(a);
  return a.nacc == 2 ? launch_tworow_by_chunks<Tg, kRmsNorm, 2>(a)
                     : launch_tworow_by_chunks<Tg, kRmsNorm, 1>(a);
}

hipError_t launch_a_tworow_f32(const LaunchA& a) { return launch_tworow<TF32>(a); }
hipError_t launch_a_tworow_f16(const LaunchA& a) { return launch_tworow<TF16>(a); }
hipError_t launch_a_tworow_bf16(const LaunchA& a) { return launch_tworow<TBF16>(a); }

}  // namespace nb
