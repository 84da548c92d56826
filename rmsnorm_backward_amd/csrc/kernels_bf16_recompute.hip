// kernels_bf16_recompute.hip -- kernel A instantiations that recompute the
// per-row statistics from x, for one I/O element type.
#include "nb_launch_a.hpp"

namespace nb {
hipError_t launch_a_recompute_bf16(const LaunchA& a) { return launch_a_impl<TBF16, true>(a); }
}  // namespace nb
