// tworow.hip -- launches of the two-rows-per-wave instantiations
// (nb_tworow.hpp): kernel A with saved or recomputed statistics, and the
// forward, for rows that 32 lanes of 16-byte vectors cover exactly.
#include "nb_launch.hpp"
#include "nb_tworow.hpp"

namespace nb {

template <class Tg, int KIND, bool RECOMP, int C, int NACC, bool WSNT>
hipError_t launch_tworow_one(const LaunchA& a) {
  // a.P rows in flight: P / 2 waves of two rows each
  hipLaunchKernelGGL((dx_partials_tworow_kernel<KIND, RECOMP, Tg, C, NACC, WSNT>), dim3(a.grid),
                     dim3(a.threads), a.lds, a.stream, a.x, a.dy, a.gamma, a.mean, a.rstd, a.dx,
                     a.ws, a.M, a.N, a.ldx, a.ldy, a.ldo, a.G, a.P / 2, a.eps);
  return hipGetLastError();
}

template <class Tg, int KIND, bool RECOMP, int NACC>
hipError_t launch_tworow_by_chunks(const LaunchA& a) {
  switch (a.chunks) {
    case 1:
      return a.ws_stream ? launch_tworow_one<Tg, KIND, RECOMP, 1, NACC, true>(a)
                         : launch_tworow_one<Tg, KIND, RECOMP, 1, NACC, false>(a);
    case 3:
      return a.ws_stream ? launch_tworow_one<Tg, KIND, RECOMP, 3, NACC, true>(a)
                         : launch_tworow_one<Tg, KIND, RECOMP, 3, NACC, false>(a);
    default:
      return hipErrorInvalidValue;
  }
}

template <class Tg, int KIND, bool RECOMP>
hipError_t launch_tworow_by_nacc(const LaunchA& a) {
  return a.nacc == 2 ? launch_tworow_by_chunks<Tg, KIND, RECOMP, 2>(a)
                     : launch_tworow_by_chunks<Tg, KIND, RECOMP, 1>(a);
}

template <class Tg>
hipError_t launch_tworow(const LaunchA& a) {
  if (!a.vec_full || a.S != 1 || a.P < 2 || a.P % 2 != 0 || a.threads != 32 * a.P ||
      a.threads > kTwoRowMaxThreads)
    return hipErrorInvalidValue;
  if (a.kind == 0)
    return a.recompute ? launch_tworow_by_nacc<Tg, kLayerNorm, true>(a)
                       : launch_tworow_by_nacc<Tg, kLayerNorm, false>(a);
  return a.recompute ? launch_tworow_by_nacc<Tg, kRmsNorm, true>(a)
                     : launch_tworow_by_nacc<Tg, kRmsNorm, false>(a);
}

template <class Tg, int KIND, int C, bool BETA>
hipError_t launch_fwd_tworow_one(const LaunchF& f) {
  // f.P waves of two rows each
  hipLaunchKernelGGL((norm_fwd_tworow_kernel<KIND, Tg, C, BETA>), dim3(f.grid), dim3(f.threads),
                     0, f.stream, f.x, f.gamma, f.beta, f.y, f.mean, f.rstd, f.M, f.N, f.eps,
                     f.P);
  return hipGetLastError();
}

template <class Tg, int KIND, bool BETA>
hipError_t launch_fwd_tworow_by_chunks(const LaunchF& f) {
  switch (f.chunks) {
    case 1: return launch_fwd_tworow_one<Tg, KIND, 1, BETA>(f);
    case 3: return launch_fwd_tworow_one<Tg, KIND, 3, BETA>(f);
    default: return hipErrorInvalidValue;
  }
}

template <class Tg>
hipError_t launch_fwd_tworow(const LaunchF& f) {
  if (!f.vec_full || f.S != 1 || f.P < 1 || f.threads != 64 * f.P ||
      f.threads > kTwoRowMaxThreads || f.N != f.chunks * 32 * (16 / Tg::kBytes))
    return hipErrorInvalidValue;
  const bool beta = f.beta != nullptr;
  if (f.kind == 0)
    return beta ? launch_fwd_tworow_by_chunks<Tg, kLayerNorm, true>(f)
                : launch_fwd_tworow_by_chunks<Tg, kLayerNorm, false>(f);
  return beta ? launch_fwd_tworow_by_chunks<Tg, kRmsNorm, true>(f)
              : launch_fwd_tworow_by_chunks<Tg, kRmsNorm, false>(f);
}

hipError_t launch_a_tworow_f32(const LaunchA& a) { return launch_tworow<TF32>(a); }
hipError_t launch_a_tworow_f16(const LaunchA& a) { return launch_tworow<TF16>(a); }
hipError_t launch_a_tworow_bf16(const LaunchA& a) { return launch_tworow<TBF16>(a); }
hipError_t launch_f_tworow_f32(const LaunchF& f) { return launch_fwd_tworow<TF32>(f); }
hipError_t launch_f_tworow_f16(const LaunchF& f) { return launch_fwd_tworow<TF16>(f); }
hipError_t launch_f_tworow_bf16(const LaunchF& f) { return launch_fwd_tworow<TBF16>(f); }

}  // namespace nb
