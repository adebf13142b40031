// Born and PCT attention forward on complex64 with fp32 matrix cores.
#include "cattn_internal.h"

namespace cattn {

bool supports_f32_mfma(const Problem &) { return false; }
hipError_t launch_f32_mfma(const Problem &) { return hipErrorNotSupported; }

}  // namespace cattn
