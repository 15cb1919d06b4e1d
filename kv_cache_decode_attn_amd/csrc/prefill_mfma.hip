// bf16 MFMA prefill kernel (filled in by the tiled implementation).
#include "launch.h"

namespace kvattn {

bool prefill_mfma_supports(const PrefillLaunch&) { return false; }

int launch_prefill_mfma(const PrefillLaunch&, hipStream_t) { return KVATTN_EUNSUPPORTED; }

}  // namespace kvattn
