// MFMA attention kernels for the MI355X shapes (placeholder until the
// kernels land: every case takes the generic path).
#include "attention.hpp"

namespace csa {

bool mfma_attn_supported(const AttnParams&) { return false; }

int launch_mfma_attn(const AttnParams&, int, int, hipStream_t) {
  return fail(CSA_ERR_UNSUPPORTED, "MFMA attention path not built");
}

size_t mfma_attn_ws_bytes(const csa_attn_desc*, int, int, int, int64_t, int) { return 0; }

}  // namespace csa
