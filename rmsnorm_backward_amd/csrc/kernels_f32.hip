// kernels_f32.hip -- kernel A instantiations for one I/O element type.
#include "nb_launch_a.hpp"

namespace nb {
hipError_t launch_a_f32(const LaunchA& a) { return launch_a_impl<TF32>(a); }
}  // namespace nb
