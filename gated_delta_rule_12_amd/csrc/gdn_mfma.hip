// MFMA kernels (bf16, gfx950) — not built yet: every case runs the VALU family.
#include "gdn_internal.h"
#include "../../include/gdn.h"

namespace gdn {

bool mfma_supported(int64_t, int64_t, int, int, int) { return false; }
WsLayout mfma_layout(const Problem&, const Split&) { return WsLayout{}; }
hipError_t mfma_forward(const Problem&, const Split&, char*, hipStream_t) {
    return hipErrorInvalidValue;
}

}  // namespace gdn
