// gdr2_bwd.hip -- gate-aware backward of the chunked Gated Delta Rule-2 layer (gfx950).
#include "gdr2_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {
hipError_t bwd_dispatch(int, int, int, const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdr2
