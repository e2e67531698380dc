// MFMA kernel placeholder: not built yet.
#include "e2a_internal.hpp"

namespace e2a {
bool mfma_supported(int, int, int, int) { return false; }
size_t mfma_packed_weight_bytes(int, int) { return 0; }
e2a_status launch_attention_mfma(const AttnPlan&, hipStream_t) {
  return fail(E2A_ERR_UNSUPPORTED, "MFMA kernel not built");
}
}  // namespace e2a
