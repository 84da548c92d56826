// kernels_f16.hip -- kernel A and forward-kernel instantiations for one I/O
// element type.
#include "nb_launch_a.hpp"

namespace nb {
hipError_t launch_a_f16(const LaunchA& a) {
  if (a.rows_per_wave == 2) return launch_a_tworow_f16(a);
  return a.recompute ? launch_a_recompute_f16(a) : launch_a_impl<TF16, false>(a);
}
hipError_t launch_f_f16(const LaunchF& f) {
  if (f.rows_per_wave == 2) return launch_f_tworow_f16(f);
  return launch_f_impl<TF16>(f);
}
}  // namespace nb
