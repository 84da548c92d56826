// rowloop.hip -- launches of the wide-row dx kernel.
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

template <class Tg, int KIND, bool RECOMP>
hipError_t launch_l_vec(const LaunchL& l) {
  return l.vec_full ? launch_l_one<Tg, KIND, RECOMP, 16 / Tg::kBytes>(l)
                    : launch_l_one<Tg, KIND, RECOMP, 1>(l);
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

template <class Tg, int KIND, bool BETA>
hipError_t launch_fl_vec(const LaunchF& f) {
  return f.vec_full ? launch_fl_one<Tg, KIND, 16 / Tg::kBytes, BETA>(f)
                    : launch_fl_one<Tg, KIND, 1, BETA>(f);
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
