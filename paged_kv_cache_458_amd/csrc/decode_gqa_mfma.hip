// Grouped-query decode on the MFMA units (placeholder until the kernel lands: every case runs on VALU).
#include "pa_kernels.h"

namespace pa {

bool gqa_mfma_supported(int, int, int) { return false; }

hipError_t launch_decode_gqa_mfma(const DecodeArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pa
