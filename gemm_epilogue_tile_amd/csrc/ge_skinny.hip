// ge_skinny.hip -- small-M weight-streaming kernel (placeholder until written).
#include "ge_launch.hpp"

namespace ge {
bool skinny_supported(const Problem &) { return false; }
hipError_t launch_skinny(const Problem &, int, hipStream_t) { return hipErrorInvalidValue; }
const char *skinny_kernel_name(const Problem &) { return "none"; }
}  // namespace ge
