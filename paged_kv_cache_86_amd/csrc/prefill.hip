// Prefix-hit paged prefill (placeholder until the MFMA kernel lands).
#include "common.h"
#include "kernels.h"

namespace pa {
int launch_paged_prefill(const PrefillArgs&, int, hipStream_t) { return -3; }
}  // namespace pa
