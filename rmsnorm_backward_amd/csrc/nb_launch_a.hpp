// nb_launch_a.hpp -- maps a validated plan onto one kernel A instantiation,
// and a forward launch onto one forward-kernel instantiation. Included by the
// per-element-type translation units (kernel A with saved statistics and the
// forward in kernels_<type>.hip, recompute mode in kernels_<type>_recompute.hip).
#pragma once

#include "nb_device.hpp"
#include "nb_forward.hpp"
#include "nb_launch.hpp"

namespace nb {

template <class Tg, int NACC, bool FULL>
constexpr int lane_elem_limit() {
  return !FULL ? 8 : (Tg::kBytes == 4 ? 16 : (NACC == 2 ? 32 : 64));
}

template <class Tg, int KIND, bool RECOMP, int NACC, int VEC, int C, bool WSNT, int MAXT>
hipError_t launch_bounded(const LaunchA& a) {
  hipLaunchKernelGGL((dx_partials_kernel<KIND, RECOMP, Tg, VEC, C, NACC, WSNT, MAXT>),
                     dim3(a.grid), dim3(a.threads), a.lds, a.stream, a.x, a.dy, a.gamma, a.mean,
                     a.rstd, a.dx, a.ws, a.M, a.N, a.ldx, a.ldy, a.ldo, a.G, a.R, a.S, a.P, a.eps);
  return hipGetLastError();
}

// Workgroups of at most 512 threads take the 512-thread-bound instantiation
// where one exists (has_narrow_bound) when their groups are long enough for
// its steady-state loop (at least 5 full iterations of P rows, the ring
// being 3 deep); short groups keep the 1024-thread-bound kernel (1151 x 8192
// fp16 LayerNorm, 4 or 5 rows per group: 20.9 us against 21.6 us).
template <class Tg, int KIND, bool RECOMP, int NACC, int VEC, int C, bool WSNT>
hipError_t launch_one_policy(const LaunchA& a) {
  if constexpr (has_narrow_bound<RECOMP, Tg, VEC, C, NACC>()) {
    if (a.threads <= 512 && a.R >= (int64_t)5 * a.P + 1)
      return launch_bounded<Tg, KIND, RECOMP, NACC, VEC, C, WSNT, 512>(a);
  }
  return launch_bounded<Tg, KIND, RECOMP, NACC, VEC, C, WSNT, max_threads_for<VEC, C>()>(a);
}

// The non-temporal partials store exists for 16-byte vector rows only (the
// one-element-per-lane path serves unaligned rows and keeps cached stores).
template <class Tg, int KIND, bool RECOMP, int NACC, int VEC, int C>
hipError_t launch_one(const LaunchA& a) {
  if constexpr (VEC > 1) {
    if (a.ws_stream) return launch_one_policy<Tg, KIND, RECOMP, NACC, VEC, C, true>(a);
  }
  return launch_one_policy<Tg, KIND, RECOMP, NACC, VEC, C, false>(a);
}

template <class Tg, int KIND, bool RECOMP, int NACC, bool FULL>
hipError_t launch_by_chunks(const LaunchA& a) {
  constexpr int VEC = FULL ? 16 / Tg::kBytes : 1;
  constexpr int LIM = lane_elem_limit<Tg, NACC, FULL>();
  switch (a.chunks) {
    case 1: return launch_one<Tg, KIND, RECOMP, NACC, VEC, 1>(a);
    case 2:
      if constexpr (VEC * 2 <= LIM) return launch_one<Tg, KIND, RECOMP, NACC, VEC, 2>(a);
      break;
    case 4:
      if constexpr (VEC * 4 <= LIM) return launch_one<Tg, KIND, RECOMP, NACC, VEC, 4>(a);
      break;
    case 8:
      if constexpr (VEC * 8 <= LIM) return launch_one<Tg, KIND, RECOMP, NACC, VEC, 8>(a);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <class Tg, int KIND, bool RECOMP, int NACC>
hipError_t launch_by_vec(const LaunchA& a) {
  return a.vec_full ? launch_by_chunks<Tg, KIND, RECOMP, NACC, true>(a)
                    : launch_by_chunks<Tg, KIND, RECOMP, NACC, false>(a);
}

// Kernel A with saved statistics (RECOMP = false) or recomputing them from x
// (RECOMP = true); each is instantiated in its own translation unit.
template <class Tg, bool RECOMP>
hipError_t launch_a_impl(const LaunchA& a) {
  if (a.kind == 0) {
    return a.nacc == 2 ? launch_by_vec<Tg, kLayerNorm, RECOMP, 2>(a)
                       : launch_by_vec<Tg, kLayerNorm, RECOMP, 1>(a);
  }
  return a.nacc == 2 ? launch_by_vec<Tg, kRmsNorm, RECOMP, 2>(a)
                     : launch_by_vec<Tg, kRmsNorm, RECOMP, 1>(a);
}

template <class Tg, int KIND, int VEC, int C, bool BETA>
hipError_t launch_fwd_one(const LaunchF& f) {
  hipLaunchKernelGGL((norm_fwd_kernel<KIND, Tg, VEC, C, BETA>), dim3(f.grid), dim3(f.threads), 0,
                     f.stream, f.x, f.gamma, f.beta, f.y, f.mean, f.rstd, f.M, f.N, f.eps, f.S,
                     f.P);
  return hipGetLastError();
}

template <class Tg, int KIND, bool FULL, bool BETA>
hipError_t launch_fwd_by_chunks(const LaunchF& f) {
  constexpr int VEC = FULL ? 16 / Tg::kBytes : 1;
  constexpr int LIM = lane_elem_limit<Tg, 1, FULL>();
  switch (f.chunks) {
    case 1: return launch_fwd_one<Tg, KIND, VEC, 1, BETA>(f);
    case 2:
      if constexpr (VEC * 2 <= LIM) return launch_fwd_one<Tg, KIND, VEC, 2, BETA>(f);
      break;
    case 4:
      if constexpr (VEC * 4 <= LIM) return launch_fwd_one<Tg, KIND, VEC, 4, BETA>(f);
      break;
    case 8:
      if constexpr (VEC * 8 <= LIM) return launch_fwd_one<Tg, KIND, VEC, 8, BETA>(f);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <class Tg, int KIND, bool BETA>
hipError_t launch_fwd_by_vec(const LaunchF& f) {
  return f.vec_full ? launch_fwd_by_chunks<Tg, KIND, true, BETA>(f)
                    : launch_fwd_by_chunks<Tg, KIND, false, BETA>(f);
}

template <class Tg>
hipError_t launch_f_impl(const LaunchF& f) {
  const bool beta = f.beta != nullptr;
  if (f.kind == 0)
    return beta ? launch_fwd_by_vec<Tg, kLayerNorm, true>(f) : launch_fwd_by_vec<Tg, kLayerNorm, false>(f);
  return beta ? launch_fwd_by_vec<Tg, kRmsNorm, true>(f) : launch_fwd_by_vec<Tg, kRmsNorm, false>(f);
}

}  // namespace nb
