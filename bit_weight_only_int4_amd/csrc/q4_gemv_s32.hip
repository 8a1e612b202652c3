// q4_gemv_s32.hip -- the fp32 GEMV kernels for fp32 scales.
#include "q4_gemv_kernels.h"

namespace q4 {
template hipError_t launch_gemv_kernels<float>(const GemvParams&, const GemvLaunch&, hipStream_t);
}  // namespace q4
