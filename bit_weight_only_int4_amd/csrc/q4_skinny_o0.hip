// q4_skinny_o0.hip -- the few-row MFMA GEMM kernels for nibble order 0
// (q4gsw: even k in the low nibble).
#include "q4_skinny_kernels.h"

namespace q4 {
template hipError_t launch_skinny_kernels<0>(const GemmParams&, const SkinnyPlan&, bool,
                                              hipStream_t);
}  // namespace q4
