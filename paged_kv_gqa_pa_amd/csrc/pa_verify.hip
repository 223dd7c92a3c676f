// Multi-token (speculative verify) attention -- not built yet.
#include "pa_kernels.h"

namespace pa {

bool verify_supported(int, int, int, int, int) { return false; }

hipError_t launch_verify_pass1(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
