// Host-only stand-ins for the kernel launchers of libstepq.so, so that the
// host side (layout creation, argument checks, status strings) can be built
// with g++ and the address / undefined-behaviour sanitizers and exercised on a
// machine without a GPU.  Every launcher reports a failed launch; the
// argument checks under test return before any launcher is reached.
#include "../../quantized_recurrent_state_packed_amd/csrc/stepq_internal.hpp"

namespace stepq {

size_t mixed_lds_bytes(int D, int max_tile_words) {
  return static_cast<size_t>(max_tile_words + D) * sizeof(uint32_t) + 16384;
}
hipError_t launch_decode_step(const Tables&, const StepArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_readout(const Tables&, const StepArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_pack(const Tables&, const PackArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_unpack(const Tables&, const PackArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace stepq
