// bwd_bf16.hip -- bf16 attention backward on CDNA4 matrix cores (gfx950).
#include "cp_kernels.h"

namespace cpattn {

hipError_t launch_bwd_bf16(const BwdLaunch &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace cpattn
