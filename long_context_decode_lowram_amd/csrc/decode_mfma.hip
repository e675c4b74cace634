// bf16 MFMA decode kernel (placeholder until the fused kernel lands).
#include "kernels.hpp"

namespace lowram {

bool mfma_supported(const DecodeParams&, int, int, int) { return false; }
int mfma_blocks_per_split() { return 1; }
hipError_t launch_decode_mfma(const DecodeParams&, int, int, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace lowram
