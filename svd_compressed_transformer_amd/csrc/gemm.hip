// bf16 MFMA path for prefill-sized M (placeholder until the tiled kernel lands).
#include "kernels.h"

namespace fsvd {
fsvd_status_t launch_gemm(const GemmArgs&, int, hipStream_t) {
    return fail(FSVD_ERR_UNSUPPORTED, "MFMA path not built yet");
}
}  // namespace fsvd
