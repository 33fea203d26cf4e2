// Chunked-prefill paged attention (MFMA); not built yet.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

bool prefill_supported(int, int, int) { return false; }

hipError_t launch_prefill_chunk(const PrefillArgs &, int, int, int, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pa
