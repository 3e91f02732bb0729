// ge_tile.hip -- large-tile bf16 MFMA kernel (placeholder until written).
#include "ge_launch.hpp"

namespace ge {
bool tile_supported(const Problem &) { return false; }
hipError_t launch_tile(const Problem &, int, hipStream_t) { return hipErrorInvalidValue; }
const char *tile_kernel_name(const Problem &) { return "none"; }
}  // namespace ge
