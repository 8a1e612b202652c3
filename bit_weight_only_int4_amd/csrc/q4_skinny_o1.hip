// q4_skinny_o1.hip -- the few-row MFMA GEMM kernels for nibble order 1
// (qcs4w: even k in the high nibble).
#include "q4_skinny_kernels.h"

namespace q4 {
template hipError_t launch_skinny_kernels<1>(const GemmParams&, const SkinnyPlan&, bool,
                                              hipStream_t);
}  // namespace q4
