// Row correction delta in three modes.
//
// stale / dO-matched: delta_i = sum_k x_ik O_ik with x = dO (bf16, before its
//   cast) or x = dO^<c> (decoded E5M2 codes times block scales).  One pass over
//   O and x with 16-byte loads; bound by HBM bandwidth.
// matched (Delta-Matching): delta_i = sum_j P_ij dP^_ij with P = exp(S - LSE)
//   recomputed in FP32 and dP^ = dO^<c> V^<c>^T on FP8 matrix cores.  Same tiling
//   as the forward: 4 waves x 32 queries, 128-key chunks staged in LDS; the S^T
//   and dP^T tiles share one layout (query per lane pair, 16 keys per lane), so
//   the product and its row sum stay in registers until one pair reduction.
#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

// ---------------------------------------------------------------------------
// stale / dO-matched
// ---------------------------------------------------------------------------
template <int DV, bool MATCHED_DO>
__global__ __launch_bounds__(256) void delta_rows_kernel(const float* __restrict__ o, const uint16_t* __restrict__ dob,
                                                         const uint8_t* __restrict__ doc, const float* __restrict__ docs,
                                                         float* __restrict__ delta, int64_t nrows, int L, int Lp) {
  constexpr int LPR = DV / 8;          // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;       // rows per workgroup pass
  const int sub = threadIdx.x % LPR;
  // the loop bound is uniform over the workgroup, so every lane of a row group
  // reaches the shuffles together; rows past the end contribute nothing
  for (int64_t base = (int64_t)blockIdx.x * RPB; base < nrows; base += (int64_t)gridDim.x * RPB) {
    const int64_t row = base + threadIdx.x / LPR;
    const bool live = row < nrows;
    float acc = 0.f;
    if (live) {
      const float* op = o + row * DV + 8 * sub;
      v4f o0 = *reinterpret_cast<const v4f*>(op);
      v4f o1 = *reinterpret_cast<const v4f*>(op + 4);
      float x[8];
      if constexpr (!MATCHED_DO) {
        v4i w = *reinterpret_cast<const v4i*>(dob + row * DV + 8 * sub);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = __uint_as_float((uint32_t)w[i] << 16);
          x[2 * i + 1] = __uint_as_float((uint32_t)w[i] & 0xffff0000u);
        }
      } else {
        const int64_t head = row / L, i = row % L;
        const int64_t prow = head * Lp + i;
        uint2 cw = *reinterpret_cast<const uint2*>(doc + prow * DV + 8 * sub);
        const float sc = docs[prow * (DV / kBlock) + (8 * sub) / kBlock];
        x[0] = __builtin_amdgcn_cvt_f32_bf8((int)cw.x, 0) * sc;
        x[1] = __builtin_amdgcn_cvt_f32_bf8((int)cw.x, 1) * sc;
        x[2] = __builtin_amdgcn_cvt_f32_bf8((int)cw.x, 2) * sc;
        x[3] = __builtin_amdgcn_cvt_f32_bf8((int)cw.x, 3) * sc;
        x[4] = __builtin_amdgcn_cvt_f32_bf8((int)cw.y, 0) * sc;
        x[5] = __builtin_amdgcn_cvt_f32_bf8((int)cw.y, 1) * sc;
        x[6] = __builtin_amdgcn_cvt_f32_bf8((int)cw.y, 2) * sc;
        x[7] = __builtin_amdgcn_cvt_f32_bf8((int)cw.y, 3) * sc;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(x[i], o0[i], fmaf(x[4 + i], o1[i], acc));
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (live && sub == 0) delta[row] = acc;
  }
}

hipError_t launch_delta_rows(const AttnDims& d, int mode, const float* o, const uint16_t* dob, Operand doc,
                             float* delta, hipStream_t s) {
  const int64_t nrows = (int64_t)d.B * d.Hq * d.L;
  const int lpr = d.dv / 8, rpb = 256 / lpr;
  int64_t blocks = (nrows + rpb - 1) / rpb;
  if (blocks > 256 * 32) blocks = 256 * 32;
  const bool m = mode == 1;
  if (d.dv == 128) {
    if (m) hipLaunchKernelGGL((delta_rows_kernel<128, true>), dim3(blocks), dim3(256), 0, s, o, dob, doc.codes, doc.scales, delta, nrows, d.L, d.Lp);
    else hipLaunchKernelGGL((delta_rows_kernel<128, false>), dim3(blocks), dim3(256), 0, s, o, dob, doc.codes, doc.scales, delta, nrows, d.L, d.Lp);
  } else {
    if (m) hipLaunchKernelGGL((delta_rows_kernel<64, true>), dim3(blocks), dim3(256), 0, s, o, dob, doc.codes, doc.scales, delta, nrows, d.L, d.Lp);
    else hipLaunchKernelGGL((delta_rows_kernel<64, false>), dim3(blocks), dim3(256), 0, s, o, dob, doc.codes, doc.scales, delta, nrows, d.L, d.Lp);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// matched
// ---------------------------------------------------------------------------
template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void delta_matched_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ kc,
    const float* __restrict__ kcs, const uint8_t* __restrict__ vc, const float* __restrict__ vcs,
    const uint8_t* __restrict__ doc, const float* __restrict__ docs, const float* __restrict__ lse,
    float* __restrict__ delta, int Hq, int Hkv, int L, int Lp, float sigma) {
  constexpr int KS = DQK / 64, VS = DV / 64;
  constexpr int KB = DQK / 32, VB = DV / 32;
  constexpr int KROW = DQK + 16, VROW = DV + 16;
  __shared__ __attribute__((aligned(16))) uint8_t sK[kChunk * KROW];
  __shared__ __attribute__((aligned(16))) float sKs[kChunk * KB];
  __shared__ __attribute__((aligned(16))) uint8_t sV[kChunk * VROW];
  __shared__ __attribute__((aligned(16))) float sVs[kChunk * VB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int R = lane & 31, h = lane >> 5;
  const int nqt = Lp / kChunk;
  const int qt = CAUSAL ? (nqt - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int hk = hq / (Hq / Hkv);
  const int q0 = qt * kChunk;
  const int qi = q0 + 32 * w + R;
  const int64_t qhead = (int64_t)b * Hq + hq, khead = (int64_t)b * Hkv + hk;
  const uint8_t* Qc = qc + qhead * Lp * DQK;
  const float* Qcs = qcs + qhead * Lp * KB;
  const uint8_t* dOc = doc + qhead * Lp * DV;
  const float* dOcs = docs + qhead * Lp * VB;
  const uint8_t* Kc = kc + khead * Lp * DQK;
  const float* Kcs = kcs + khead * Lp * KB;
  const uint8_t* Vc = vc + khead * Lp * DV;
  const float* Vcs = vcs + khead * Lp * VB;

  v8i qb[KS], db[VS];
  int qsc[KS], dsc[VS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint8_t* p = Qc + (int64_t)qi * DQK + 64 * ks;
    qb[ks] = cat(*reinterpret_cast<const v4i*>(p + 16 * h), *reinterpret_cast<const v4i*>(p + 32 + 16 * h));
    qsc[ks] = e8m0(Qcs[(int64_t)qi * KB + 2 * ks + h]);
  }
#pragma unroll
  for (int ks = 0; ks < VS; ++ks) {
    const uint8_t* p = dOc + (int64_t)qi * DV + 64 * ks;
    db[ks] = cat(*reinterpret_cast<const v4i*>(p + 16 * h), *reinterpret_cast<const v4i*>(p + 32 + 16 * h));
    dsc[ks] = e8m0(dOcs[(int64_t)qi * VB + 2 * ks + h]);
  }
  const float c2 = sigma * kLog2e;
  const float l2 = (qi < L) ? lse[qhead * L + qi] * kLog2e : 0.f;
  double acc = 0.0;                              // FP32 per chunk, FP64 across chunks
  const int nchunks = CAUSAL ? (qt + 1) : nqt;
  const int krow_a = pair_row(R);
  for (int c = 0; c < nchunks; ++c) {
    const int k0 = c * kChunk;
    __syncthreads();
    for (int i = tid; i < kChunk * DQK / 16; i += 256) {
      const int row = (i * 16) / DQK, col = (i * 16) % DQK;
      *reinterpret_cast<v4i*>(sK + row * KROW + col) = *reinterpret_cast<const v4i*>(Kc + (int64_t)(k0 + row) * DQK + col);
    }
    for (int i = tid; i < kChunk * KB / 4; i += 256)
      *reinterpret_cast<v4f*>(sKs + 4 * i) = *reinterpret_cast<const v4f*>(Kcs + (int64_t)k0 * KB + 4 * i);
    for (int i = tid; i < kChunk * DV / 16; i += 256) {
      const int row = (i * 16) / DV, col = (i * 16) % DV;
      *reinterpret_cast<v4i*>(sV + row * VROW + col) = *reinterpret_cast<const v4i*>(Vc + (int64_t)(k0 + row) * DV + col);
    }
    for (int i = tid; i < kChunk * VB / 4; i += 256)
      *reinterpret_cast<v4f*>(sVs + 4 * i) = *reinterpret_cast<const v4f*>(Vcs + (int64_t)k0 * VB + 4 * i);
    __syncthreads();
    if (CAUSAL && k0 > q0 + 32 * w + 31) continue;
    const bool need_mask = (k0 + kChunk > L) || (CAUSAL && k0 + kChunk - 1 > q0 + 32 * w);
    float cacc = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int krow = 32 * t + krow_a;
      v16f s = v16f{}, dp = v16f{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint8_t* p = sK + krow * KROW + 64 * ks;
        v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
        s = mfma<E4M3, E4M3>(a, qb[ks], s, e8m0(sKs[krow * KB + 2 * ks + h]), qsc[ks]);
      }
#pragma unroll
      for (int ks = 0; ks < VS; ++ks) {
        const uint8_t* p = sV + krow * VROW + 64 * ks;
        v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
        dp = mfma<E4M3, E5M2>(a, db[ks], dp, e8m0(sVs[krow * VB + 2 * ks + h]), dsc[ks]);
      }
      if (need_mask) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = k0 + 32 * t + 16 * h + v;
          if (kk >= L || (CAUSAL && kk > qi)) s[v] = -INFINITY;
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[v], c2, -l2));
        cacc = fmaf(p, dp[v], cacc);
      }
    }
    acc += (double)cacc;
  }
  acc = pair_sum_d(acc);
  if (qi < L && h == 0) delta[qhead * L + qi] = (float)acc;
}

template <int DQK, int DV>
static void launch_dm_t(const AttnDims& d, Operand doc, Operand q, Operand k, Operand v, const float* lse,
                        float* delta, hipStream_t s) {
  dim3 grid(d.Lp / kChunk, d.Hq, d.B);
  if (d.causal)
    hipLaunchKernelGGL((delta_matched_kernel<DQK, DV, true>), grid, dim3(256), 0, s, q.codes, q.scales, k.codes,
                       k.scales, v.codes, v.scales, doc.codes, doc.scales, lse, delta, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
  else
    hipLaunchKernelGGL((delta_matched_kernel<DQK, DV, false>), grid, dim3(256), 0, s, q.codes, q.scales, k.codes,
                       k.scales, v.codes, v.scales, doc.codes, doc.scales, lse, delta, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
}

hipError_t launch_delta_matched(const AttnDims& d, Operand doc, Operand q, Operand k, Operand v, const float* lse,
                                float* delta, hipStream_t s) {
  if (d.dqk == 64 && d.dv == 64) launch_dm_t<64, 64>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 128 && d.dv == 128) launch_dm_t<128, 128>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 192 && d.dv == 128) launch_dm_t<192, 128>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 64 && d.dv == 128) launch_dm_t<64, 128>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 128 && d.dv == 64) launch_dm_t<128, 64>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 192 && d.dv == 64) launch_dm_t<192, 64>(d, doc, q, k, v, lse, delta, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dm
