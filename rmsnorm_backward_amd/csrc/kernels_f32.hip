// kernels_f32.hip -- kernel A and forward-kernel instantiations for one I/O
// element type.
#include "nb_launch_a.hpp"

namespace nb {
hipError_t launch_a_f32(const LaunchA& a) {
  if (a.rows_per_wave == 2) return launch_a_tworow_f32(a);
  return a.recompute ? launch_a_recompute_f32(a) : launch_a_impl<TF32, false>(a);
}
hipError_t launch_f_f32(const LaunchF& f) {
  if (f.rows_per_wave == 2) return launch_f_tworow_f32(f);
  return launch_f_impl<TF32>(f);
}
}  // namespace nb
