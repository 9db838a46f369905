// Whole-workgroup MFMA kernel for 256-class slices (placeholder until implemented).
#include "fq_internal.h"
namespace fq {
bool mfma_wide_supports(const Problem&) { return false; }
hipError_t launch_mfma_wide(const Problem&, const Buffers&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fq
