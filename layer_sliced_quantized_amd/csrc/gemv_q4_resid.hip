// Instantiation of the streaming GEMV for Q4_0 weights, epilogue RESID.
#include "gemv_kernel.h"

namespace slq {
template hipError_t gemv_inst<QT_Q4, EPI_RESID>(const Packed&, int, Act, NormIn, GemvOut, int, int, hipStream_t);
}  // namespace slq
