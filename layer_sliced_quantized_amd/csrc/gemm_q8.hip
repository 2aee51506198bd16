// Instantiations of the batched int8-MFMA products for Q8_0.
#include "gemm_kernel.h"

namespace slq {
template hipError_t gemm_inst<QT_Q8, EPI_STORE>(const Packed&, int, Act, NormIn, GemvOut, int, int, hipStream_t);
template hipError_t gemm_inst<QT_Q8, EPI_SWIGLU>(const Packed&, int, Act, NormIn, GemvOut, int, int, hipStream_t);
template hipError_t gemm_inst<QT_Q8, EPI_RESID>(const Packed&, int, Act, NormIn, GemvOut, int, int, hipStream_t);
}  // namespace slq
