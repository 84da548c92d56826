// rowloop.hip -- launches of the wide-row kernels: rows held in the
// registers of one workgroup (chunks 4 or 8) or streamed by the row loop.
#include "nb_launch.hpp"
#include "nb_rowloop.hpp"

namespace nb {

namespace {

template <class Tg, int KIND, bool RECOMP, int VEC>
hipError_t launch_l_one(const LaunchL& l) {
  hipLaunchKernelGGL((dx_rowloop_kernel<KIND, RECOMP, Tg, VEC>), dim3((unsigned)l.grid),
                     dim3(kRowWaves * 64), 0, l.stream, l.x, l.dy, l.gamma, l.mean, l.rstd, l.dx,
                     l.mean_out, l.rstd_out, l.M, l.N, l.ldx, l.ldy, l.ldo, l.eps);
  return hipGetLastError();
}

template <class Tg, int KIND, bool RECOMP, int C>
hipError_t launch_lr_one(const LaunchL& l) {
  hipLaunchKernelGGL((dx_rowreg_kernel<KIND, RECOMP, Tg, 16 / Tg::kBytes, C>),
                     dim3((unsigned)l.grid), dim3(kRowWaves * 64), 0, l.stream, l.x, l.dy,
                     l.gamma, l.mean, l.rstd, l.dx, l.mean_out, l.rstd_out, l.M, l.N, l.ldx,
                     l.ldy, l.ldo, l.eps);
  return hipGetLastError();
}

template <class Tg, int KIND, bool RECOMP>
hipError_t launch_l_vec(const LaunchL& l) {
  if (!l.vec_full) return launch_l_one<Tg, KIND, RECOMP, 1>(l);
  switch (l.chunks) {
    case 0: return launch_l_one<Tg, KIND, RECOMP, 16 / Tg::kBytes>(l);
    case 4: return launch_lr_one<Tg, KIND, RECOMP, 4>(l);
    case 8:
      // LayerNorm recompute does not fit at 8 chunks (the planner never asks)
      if constexpr (!(RECOMP && KIND == kLayerNorm)) return launch_lr_one<Tg, KIND, RECOMP, 8>(l);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <class Tg>
hipError_t launch_l_impl(const LaunchL& l) {
  if (l.kind == 0)
    return l.recompute ? launch_l_vec<Tg, kLayerNorm, true>(l)
                       : launch_l_vec<Tg, kLayerNorm, false>(l);
  return l.recompute ? launch_l_vec<Tg, kRmsNorm, true>(l) : launch_l_vec<Tg, kRmsNorm, false>(l);
}

template <class Tg, int KIND, int VEC, bool BETA>
hipError_t launch_fl_one(const LaunchF& f) {
  hipLaunchKernelGGL((fwd_rowloop_kernel<KIND, Tg, VEC, BETA>), dim3((unsigned)f.grid),
                     dim3(kRowWaves * 64), 0, f.stream, f.x, f.gamma, f.beta, f.y, f.mean,
                     f.rstd, f.M, (int64_t)f.N, f.eps);
  return hipGetLastError();
}

template <class Tg, int KIND, int C, bool BETA>
hipError_t launch_flr_one(const LaunchF& f) {
  hipLaunchKernelGGL((fwd_rowreg_kernel<KIND, Tg, 16 / Tg::kBytes, C, BETA>),
                     dim3((unsigned)f.grid), dim3(kRowWaves * 64), 0, f.stream, f.x, f.gamma,
                     f.beta, f.y, f.mean, f.rstd, f.M, (int64_t)f.N, f.eps);
  return hipGetLastError();
}

template <class Tg, int KIND, bool BETA>
hipError_t launch_fl_vec(const LaunchF& f) {
  if (!f.vec_full) return launch_fl_one<Tg, KIND, 1, BETA>(f);
  switch (f.chunks) {
    case 0: return launch_fl_one<Tg, KIND, 16 / Tg::kBytes, BETA>(f);
    case 4: return launch_flr_one<Tg, KIND, 4, BETA>(f);
    case 8:
      // LayerNorm with beta does not fit at 8 chunks (the planner never asks)
      if constexpr (!(BETA && KIND == kLayerNorm)) return launch_flr_one<Tg, KIND, 8, BETA>(f);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <class Tg>
hipError_t launch_fl_impl(const LaunchF& f) {
  const bool beta = f.beta != nullptr;
  if (f.kind == 0)
    return beta ? launch_fl_vec<Tg, kLayerNorm, true>(f) : launch_fl_vec<Tg, kLayerNorm, false>(f);
  return beta ? launch_fl_vec<Tg, kRmsNorm, true>(f) : launch_fl_vec<Tg, kRmsNorm, false>(f);
}

}  // namespace

hipError_t launch_fl_f32(const LaunchF& f) { return launch_fl_impl<TF32>(f); }
hipError_t launch_fl_f16(const LaunchF& f) { return launch_fl_impl<TF16>(f); }
hipError_t launch_fl_bf16(const LaunchF& f) { return launch_fl_impl<TBF16>(f); }

hipError_t launch_l_f32(const LaunchL& l) { return launch_l_impl<TF32>(l); }
hipError_t launch_l_f16(const LaunchL& l) { return launch_l_impl<TF16>(l); }
hipError_t launch_l_bf16(const LaunchL& l) { return launch_l_impl<TBF16>(l); }

}  // namespace nb
