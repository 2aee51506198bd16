// Dispatch of the batched int8-MFMA products (instantiations: gemm_q4.hip, gemm_q8.hip).
#include "gemm_kernel.h"

namespace slq {

hipError_t launch_gemm(const Packed& W, int T, Act x, NormIn nin, GemvOut out, int ksplit, int waves,
                       hipStream_t s) {
  const bool q4 = W.qt == QT_Q4;
  switch (out.kind) {
    case EPI_STORE: return q4 ? gemm_inst<QT_Q4, EPI_STORE>(W, T, x, nin, out, ksplit, waves, s)
                              : gemm_inst<QT_Q8, EPI_STORE>(W, T, x, nin, out, ksplit, waves, s);
    case EPI_SWIGLU: return q4 ? gemm_inst<QT_Q4, EPI_SWIGLU>(W, T, x, nin, out, ksplit, waves, s)
                               : gemm_inst<QT_Q8, EPI_SWIGLU>(W, T, x, nin, out, ksplit, waves, s);
    case EPI_RESID: return q4 ? gemm_inst<QT_Q4, EPI_RESID>(W, T, x, nin, out, ksplit, waves, s)
                              : gemm_inst<QT_Q8, EPI_RESID>(W, T, x, nin, out, ksplit, waves, s);
  }
  return hipErrorInvalidValue;
}

bool gemm_usable(int qt, int T, int waves) { return gemm_fits(qt, T, waves); }

int gemm_min_tokens(int qt, int waves) { return qt == QT_Q8 ? 2 : waves <= 4 ? 4 : 8; }

}  // namespace slq
