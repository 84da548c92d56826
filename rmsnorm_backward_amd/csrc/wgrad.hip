// wgrad.hip -- launches of the column-walk weight-gradient kernel.
#include "nb_launch.hpp"
#include "nb_wgrad.hpp"

namespace nb {

namespace {

template <class Tg, int KIND, int VEC, int NACC>
hipError_t launch_w_one(const LaunchW& w) {
  hipLaunchKernelGGL((wgrad_colwalk_kernel<KIND, Tg, VEC, NACC>), dim3((unsigned)w.grid),
                     dim3(kWgradWaves * 64), 0, w.stream, w.x, w.dy, w.mean, w.rstd, w.M, w.N,
                     w.ldx, w.ldy, w.lpr, w.dgamma, w.dbeta, w.out_dtype, w.accumulate);
  return hipGetLastError();
}

template <class Tg, int KIND, int NACC>
hipError_t launch_w_vec(const LaunchW& w) {
  return w.vec_full ? launch_w_one<Tg, KIND, 16 / Tg::kBytes, NACC>(w)
                    : launch_w_one<Tg, KIND, 1, NACC>(w);
}

template <class Tg>
hipError_t launch_w_impl(const LaunchW& w) {
  if (w.kind == 0)
    return w.nacc == 2 ? launch_w_vec<Tg, kLayerNorm, 2>(w) : launch_w_vec<Tg, kLayerNorm, 1>(w);
  return w.nacc == 2 ? launch_w_vec<Tg, kRmsNorm, 2>(w) : launch_w_vec<Tg, kRmsNorm, 1>(w);
}

}  // namespace

hipError_t launch_w_f32(const LaunchW& w) { return launch_w_impl<TF32>(w); }
hipError_t launch_w_f16(const LaunchW& w) { return launch_w_impl<TF16>(w); }
hipError_t launch_w_bf16(const LaunchW& w) { return launch_w_impl<TBF16>(w); }

}  // namespace nb
