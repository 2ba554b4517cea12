// dK/dV launch dispatch and the two-kernel backward (the generic dK/dV kernel is in
// attn_dkdv.h, the d_qk = d_v = 128 one in attn_dkdv128.hip, dQ in attn_dq.h).
#include "attn_dkdv.h"

namespace dm {

hipError_t launch_dkdv(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc, Operand dos,
                       const float* lse, const float* delta, float* dk, float* dv, double* ps, double* pa,
                       hipStream_t s) {
  if (d.dqk == 64 && d.dv == 64) return launch_dkdv_t<64, 64>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, ps, pa, s);
  if (d.dqk == 128 && d.dv == 128)
    return launch_dkdv_d128(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, ps, pa, nullptr, 1, s);
  if (d.dqk == 192 && d.dv == 128)
    return launch_dkdv_t<192, 128>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, ps, pa, s);
  if (d.dqk == 64 && d.dv == 128)
    return launch_dkdv_t<64, 128>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, ps, pa, s);
  if (d.dqk == 128 && d.dv == 64)
    return launch_dkdv_t<128, 64>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, ps, pa, s);
  if (d.dqk == 192 && d.dv == 64)
    return launch_dkdv_t<192, 64>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, ps, pa, s);
  if (d.dqk == 256 && d.dv == 256)
    return launch_dkdv_256_256(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, ps, pa, s);
  return hipErrorInvalidValue;
}

int dkdv_head_split(const AttnDims& d) { return d.dqk == 128 && d.dv == 128 ? dkdv_d128_head_split(d) : 1; }

hipError_t launch_dkdv_split(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc,
                             Operand dos, const float* lse, const float* delta, float* dk, float* dv, float* ws,
                             hipStream_t s) {
  const int hs = dkdv_head_split(d);
  if (hs == 1) return launch_dkdv(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, nullptr, nullptr, s);
  return launch_dkdv_d128(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, nullptr, nullptr, ws, hs, s);
}

hipError_t launch_bwd(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand ks, Operand vc, Operand doc,
                      Operand dos, const float* lse, const float* delta, float* dq, float* dk, float* dv,
                      double* ps, double* pa, hipStream_t s) {
  hipError_t e = launch_dkdv(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, nullptr, nullptr, s);
  if (e != hipSuccess) return e;
  return launch_dq(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, nullptr, s);
}

__global__ void fill_zero_kernel(uint64_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 8;
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint64_t*>(p), n);
  return hipGetLastError();
}

}  // namespace dm
