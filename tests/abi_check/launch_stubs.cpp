// Host-only stand-ins for the kernel launchers, so that the C ABI layer
// (gdn_api.cpp) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven without a GPU.  Each counts its calls
// and touches no argument pointer.
#include <hip/hip_runtime.h>

#include "gdn_kernels.hpp"

long g_launches = 0;

namespace gdn {
int64_t bwd_checkpoint_blocks(int64_t T) { return (T + 15) / 16; }
hipError_t launch_backward(const BwdArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_chunk_fwd(const ChunkArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gates(const GateArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_output_gate(const NormArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_short_conv(const ConvArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_state_copy(const float*, float*, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace gdn
