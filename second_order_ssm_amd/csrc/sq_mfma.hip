// MFMA kernels of the 2Mamba chunked forward (bf16 inputs, d = 64).
#include "device_common.h"
#include "internal.h"

namespace twm {

bool mfma_sq_supported(const FwdArgs&) { return false; }
size_t mfma_sq_workspace(const FwdArgs&) { return 0; }
int mfma_sq_fwd(const FwdArgs&) { return TWOMAMBA_ERR_UNSUPPORTED; }

}  // namespace twm
