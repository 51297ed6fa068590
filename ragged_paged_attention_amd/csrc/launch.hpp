// launch.hpp -- host-side entry points of the kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace ra {

hipError_t launch_generic(const Params &p, hipStream_t stream);
bool generic_supports(int D);

}  // namespace ra
