// kernels_bf16.hip -- kernel A instantiations for one I/O element type.
#include "nb_launch_a.hpp"

namespace nb {
hipError_t launch_a_bf16(const LaunchA& a) { return launch_a_impl<TBF16>(a); }
}  // namespace nb
