// dQ for d_qk = 192, d_v = 128 and d_qk = d_v = 256 in a translation unit of its own,
// compiled with the compiler's default MFMA register form (see build.py).
#include "attn_dq.h"

namespace dm {

hipError_t launch_dq_192_128(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                             const float* lse, const float* delta, float* dq, double* ps, double* pa, double* pc,
                             hipStream_t s) {
  launch_dq_t<192, 128>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  return hipGetLastError();
}

hipError_t launch_dq_256_256(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                             const float* lse, const float* delta, float* dq, double* ps, double* pa, double* pc,
                             hipStream_t s) {
  launch_dq_t<256, 256>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  return hipGetLastError();
}

}  // namespace dm
