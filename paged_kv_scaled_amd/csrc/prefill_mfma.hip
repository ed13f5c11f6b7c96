// Prefill attention on bf16/fp16 MFMA (placeholder until the MFMA kernel lands).
#include "common.h"
#include "kernels.h"

namespace pkv {

bool prefill_mfma_supported(int, int) { return false; }

hipError_t launch_prefill_mfma(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv
