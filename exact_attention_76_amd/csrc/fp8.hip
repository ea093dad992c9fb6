// fp8.hip -- FP8 e4m3 forward pass and pre-pass (not yet built: both report "not supported").
#include <hip/hip_runtime.h>

#include "internal.h"

namespace attn {

hipError_t launch_fwd_fp8(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fp8_prepare(const PrepareArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace attn
