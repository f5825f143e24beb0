// Chunked-prefill attention over paged K/V (bf16 MFMA). Placeholder until the
// MFMA kernel lands: reports every configuration as not built.
#include "device.h"

namespace pa {

bool prefill_supported(int, int, int, int) { return false; }

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
