// dQ launch dispatch (the kernel is in attn_dq.h).
#include "attn_dq.h"

namespace dm {

hipError_t launch_dq(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                     const float* lse, const float* delta, float* dq, double* ps, double* pa, double* pc,
                     hipStream_t s) {
  if (d.dqk == 64 && d.dv == 64) launch_dq_t<64, 64>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  else if (d.dqk == 128 && d.dv == 128) launch_dq_t<128, 128>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  else if (d.dqk == 192 && d.dv == 128) return launch_dq_192_128(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  else if (d.dqk == 256 && d.dv == 256) return launch_dq_256_256(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  else if (d.dqk == 64 && d.dv == 128) launch_dq_t<64, 128>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  else if (d.dqk == 128 && d.dv == 64) launch_dq_t<128, 64>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  else if (d.dqk == 192 && d.dv == 64) launch_dq_t<192, 64>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dm
