// Born-rule attention forward on bf16 planes with gfx950 matrix cores.
#include "cattn_internal.h"

namespace cattn {

bool supports_born_bf16_mfma(const Problem &) { return false; }
hipError_t launch_born_bf16_mfma(const Problem &) { return hipErrorNotSupported; }

}  // namespace cattn
