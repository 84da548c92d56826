// kernels_f16.hip -- kernel A instantiations for one I/O element type.
#include "nb_launch_a.hpp"

namespace nb {
hipError_t launch_a_f16(const LaunchA& a) { return launch_a_impl<TF16>(a); }
}  // namespace nb
