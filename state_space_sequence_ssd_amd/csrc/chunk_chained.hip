// Placeholder: the chained one-kernel path is not built yet.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

bool chunk_chained_fits(const Problem&) { return false; }

hipError_t launch_chunk_chained(const Problem&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace ssd
