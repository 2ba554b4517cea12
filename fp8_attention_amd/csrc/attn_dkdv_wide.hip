// dK/dV for d_qk = d_v = 256 in a translation unit of its own, compiled with the
// compiler's default MFMA register form (one wave per SIMD: accumulators in AGPRs).
#include "attn_dkdv.h"

namespace dm {

hipError_t launch_dkdv_256_256(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc,
                               Operand dos, const float* lse, const float* delta, float* dk, float* dv, double* ps,
                               double* pa, hipStream_t s) {
  return launch_dkdv_t<256, 256>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, ps, pa, s);
}

}  // namespace dm
