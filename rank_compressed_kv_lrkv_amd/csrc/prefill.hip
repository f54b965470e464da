// LRKV causal prefill (bf16 MFMA).  Placeholder until the MFMA kernel lands:
// reports every shape as unsupported, so lrkv_prefill returns LRKV_ERR_SHAPE.
#include "lrkv_internal.h"

namespace lrkv {

bool prefill_supported(int, int, int, int) { return false; }
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace lrkv
