// Matrix-core (MFMA) kernels of the GQA decode step for gfx950.
#include "device_common.h"
#include "internal.h"

namespace gqa {

const bool kHaveMfmaQk = false;
const bool kHaveMfmaAll = false;

hipError_t launch_attend_mfma_qk(const AttnArgs&, const Plan&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attend_mfma_all(const AttnArgs&, const Plan&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gqa
