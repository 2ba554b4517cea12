// Test-only probe of the scaled FP8 matrix instructions the attention kernels use,
// for measuring how they accumulate.  Not part of libdm.
//
// One wave per tile.  For the 32x32x64 form a tile is C[32][32] = C_in + A B^T with
// A [32][K] and B [32][K] (B given as rows, as every kernel holds its operands),
// taken in K/64 chained instructions; for the 16x16x128 form C[16][16] with A, B
// [16][K] in K/128 chained instructions.  Codes are FP8 bytes in the format given
// per operand (0 = E4M3, 1 = E5M2); the scale of element k of a row is
// 2^(e - 127) with e = the row's exponent byte for block k / 32.  The operands reach
// the instruction through the same wrappers and lane layouts as in the kernels
// (dm_common.h).  All indexing stays inside [ntiles * rows * K] for codes,
// [ntiles * rows * K / 32] for exponents and [ntiles * rows * rows] for C.
#include <stdint.h>

#include "dm_common.h"

namespace {

using dm::v16f;
using dm::v4f;
using dm::v4i;
using dm::v8i;

__device__ __forceinline__ v4i load16(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }

template <int FA, int FB>
__global__ __launch_bounds__(64) void probe32(const uint8_t* a, const uint8_t* ea, const uint8_t* b,
                                              const uint8_t* eb, const float* c_in, float* out, int K) {
  const int lane = threadIdx.x, R = lane & 31, h = lane >> 5;
  const int64_t t = blockIdx.x;
  const uint8_t* ar = a + (t * 32 + R) * K;
  const uint8_t* br = b + (t * 32 + R) * K;
  const uint8_t* ear = ea + (t * 32 + R) * (K / 32);
  const uint8_t* ebr = eb + (t * 32 + R) * (K / 32);
  v16f acc;
  // register v of lane (R, h) holds row 8(v/4) + 4h + v%4, column R
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = c_in[t * 1024 + (8 * (v / 4) + 4 * h + v % 4) * 32 + R];
  for (int k0 = 0; k0 < K; k0 += 64) {
    const v8i av = dm::cat(load16(ar + k0 + 16 * h), load16(ar + k0 + 32 + 16 * h));
    const v8i bv = dm::cat(load16(br + k0 + 16 * h), load16(br + k0 + 32 + 16 * h));
    acc = dm::mfma<FA, FB>(av, bv, acc, ear[k0 / 32 + h], ebr[k0 / 32 + h]);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) out[t * 1024 + (8 * (v / 4) + 4 * h + v % 4) * 32 + R] = acc[v];
}

template <int FA, int FB>
__global__ __launch_bounds__(64) void probe16(const uint8_t* a, const uint8_t* ea, const uint8_t* b,
                                              const uint8_t* eb, const float* c_in, float* out, int K) {
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  const int64_t t = blockIdx.x;
  const uint8_t* ar = a + (t * 16 + n) * K;
  const uint8_t* br = b + (t * 16 + n) * K;
  const uint8_t* ear = ea + (t * 16 + n) * (K / 32);
  const uint8_t* ebr = eb + (t * 16 + n) * (K / 32);
  v4f acc;
  // register i of lane (n, g) holds row 4g + i, column n
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = c_in[t * 256 + (4 * g + i) * 16 + n];
  for (int k0 = 0; k0 < K; k0 += 128) {
    const v8i av = dm::cat(load16(ar + k0 + 16 * g), load16(ar + k0 + 64 + 16 * g));
    const v8i bv = dm::cat(load16(br + k0 + 16 * g), load16(br + k0 + 64 + 16 * g));
    acc = dm::mfma16<FA, FB>(av, bv, acc, ear[k0 / 32 + g], ebr[k0 / 32 + g]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) out[t * 256 + (4 * g + i) * 16 + n] = acc[i];
}

template <int FA, int FB>
hipError_t go(int form, const uint8_t* a, const uint8_t* ea, const uint8_t* b, const uint8_t* eb, const float* c,
              float* out, int ntiles, int K, hipStream_t s) {
  if (form == 32)
    hipLaunchKernelGGL((probe32<FA, FB>), dim3(ntiles), dim3(64), 0, s, a, ea, b, eb, c, out, K);
  else
    hipLaunchKernelGGL((probe16<FA, FB>), dim3(ntiles), dim3(64), 0, s, a, ea, b, eb, c, out, K);
  return hipGetLastError();
}

}  // namespace

// form: 32 (v_mfma_scale_f32_32x32x64_f8f6f4) or 16 (v_mfma_scale_f32_16x16x128_f8f6f4).
// fa, fb: 0 = E4M3, 1 = E5M2.  K: a positive multiple of 64 (form 32) or 128 (form 16).
// Returns 0 on success, 1 on invalid arguments (nothing launched), 2 on a launch error.
extern "C" int mfma_acc_probe(int form, int fa, int fb, const uint8_t* a, const uint8_t* ea, const uint8_t* b,
                              const uint8_t* eb, const float* c_in, float* out, int ntiles, int K,
                              hipStream_t stream) {
  if ((form != 32 && form != 16) || fa < 0 || fa > 1 || fb < 0 || fb > 1 || ntiles < 1 || K < 1) return 1;
  if (K % (form == 32 ? 64 : 128) != 0) return 1;
  if (!a || !ea || !b || !eb || !c_in || !out) return 1;
  hipError_t e;
  if (fa == 0 && fb == 0) e = go<dm::E4M3, dm::E4M3>(form, a, ea, b, eb, c_in, out, ntiles, K, stream);
  else if (fa == 0) e = go<dm::E4M3, dm::E5M2>(form, a, ea, b, eb, c_in, out, ntiles, K, stream);
  else if (fb == 0) e = go<dm::E5M2, dm::E4M3>(form, a, ea, b, eb, c_in, out, ntiles, K, stream);
  else e = go<dm::E5M2, dm::E5M2>(form, a, ea, b, eb, c_in, out, ntiles, K, stream);
  return e == hipSuccess ? 0 : 2;
}
