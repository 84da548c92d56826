// nb_launch_a.hpp -- maps a validated plan onto one kernel A instantiation.
// Included by exactly one translation unit per I/O element type.
#pragma once

#include "nb_device.hpp"
#include "nb_launch.hpp"

namespace nb {

template <class Tg, int NACC, bool FULL>
constexpr int lane_elem_limit() {
  return !FULL ? 8 : (Tg::kBytes == 4 ? 16 : (NACC == 2 ? 32 : 64));
}

template <class Tg, int KIND, int NACC, int VEC, int C>
hipError_t launch_one(const LaunchA& a) {
  hipLaunchKernelGGL((dx_partials_kernel<KIND, Tg, VEC, C, NACC>), dim3(a.grid), dim3(a.threads),
                     a.lds, a.stream, a.x, a.dy, a.gamma, a.mean, a.rstd, a.dx, a.ws, a.M, a.N,
                     a.G, a.R, a.S, a.P);
  return hipGetLastError();
}

template <class Tg, int KIND, int NACC, bool FULL>
hipError_t launch_by_chunks(const LaunchA& a) {
  constexpr int VEC = FULL ? 16 / Tg::kBytes : 1;
  constexpr int LIM = lane_elem_limit<Tg, NACC, FULL>();
  switch (a.chunks) {
    case 1: return launch_one<Tg, KIND, NACC, VEC, 1>(a);
    case 2:
      if constexpr (VEC * 2 <= LIM) return launch_one<Tg, KIND, NACC, VEC, 2>(a);
      break;
    case 4:
      if constexpr (VEC * 4 <= LIM) return launch_one<Tg, KIND, NACC, VEC, 4>(a);
      break;
    case 8:
      if constexpr (VEC * 8 <= LIM) return launch_one<Tg, KIND, NACC, VEC, 8>(a);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <class Tg, int KIND, int NACC>
hipError_t launch_by_vec(const LaunchA& a) {
  return a.vec_full ? launch_by_chunks<Tg, KIND, NACC, true>(a)
                    : launch_by_chunks<Tg, KIND, NACC, false>(a);
}

template <class Tg>
hipError_t launch_a_impl(const LaunchA& a) {
  if (a.kind == 0) {
    return a.nacc == 2 ? launch_by_vec<Tg, kLayerNorm, 2>(a) : launch_by_vec<Tg, kLayerNorm, 1>(a);
  }
  return a.nacc == 2 ? launch_by_vec<Tg, kRmsNorm, 2>(a) : launch_by_vec<Tg, kRmsNorm, 1>(a);
}

}  // namespace nb
