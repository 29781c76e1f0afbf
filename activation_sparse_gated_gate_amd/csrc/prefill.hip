// prefill.hip -- token-selective prefill (placeholder until the kernels land).
#include <hip/hip_runtime.h>

#include "dev_common.h"

namespace sffn {

hipError_t launch_prefill_select(const PrefillSelectCall &) { return hipErrorNotSupported; }
hipError_t launch_prefill_forward(const PrefillForwardCall &) { return hipErrorNotSupported; }

}  // namespace sffn
