// Instantiation of the streaming GEMV for Q8_0 weights, epilogue SWIGLU.
#include "gemv_kernel.h"

namespace slq {
template hipError_t gemv_inst<QT_Q8, EPI_SWIGLU>(const Packed&, int, Act, NormIn, GemvOut, int, int, hipStream_t);
}  // namespace slq
