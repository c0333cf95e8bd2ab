// MFMA kernel of the 2Mamba-E forward (bf16 inputs, d = 64).
#include "device_common.h"
#include "internal.h"

namespace twm {

bool mfma_exp_supported(const FwdArgs&) { return false; }
int mfma_exp_fwd(const FwdArgs&) { return TWOMAMBA_ERR_UNSUPPORTED; }

}  // namespace twm
