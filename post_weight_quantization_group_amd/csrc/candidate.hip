// Candidate-set solver for gfx950 (placeholder until the kernel lands).
#include "device.h"
#include "launch.h"

namespace cqk {
hipError_t launch_candidate(const CandArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace cqk
