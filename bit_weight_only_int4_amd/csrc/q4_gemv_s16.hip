// q4_gemv_s16.hip -- the fp32 GEMV kernels for binary16 scales (q4f16_1 weights).
#include "q4_gemv_kernels.h"

namespace q4 {
template hipError_t launch_gemv_kernels<_Float16>(const GemvParams&, const GemvLaunch&, hipStream_t);
}  // namespace q4
