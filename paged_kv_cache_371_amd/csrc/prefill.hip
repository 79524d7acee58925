// MFMA prefill kernel for multi-row requests (placeholder until built).
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

bool prefill_supported(int, int) { return false; }
int prefill_rows_per_tile(int, int) { return 1; }
hipError_t launch_prefill(int, int, const PrefillArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pa
