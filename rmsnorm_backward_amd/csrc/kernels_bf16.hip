// kernels_bf16.hip -- kernel A and forward-kernel instantiations for one I/O
// element type.
#include "nb_launch_a.hpp"

namespace nb {
hipError_t launch_a_bf16(const LaunchA& a) {
  if (a.rows_per_wave == 2) return launch_a_tworow_bf16(a);
  return a.recompute ? launch_a_recompute_bf16(a) : launch_a_impl<TBF16, false>(a);
}
hipError_t launch_f_bf16(const LaunchF& f) {
  if (f.rows_per_wave == 2) return launch_f_tworow_bf16(f);
  return launch_f_impl<TBF16>(f);
}
}  // namespace nb
