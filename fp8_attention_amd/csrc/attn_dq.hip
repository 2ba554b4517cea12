// dQ of block-scaled FP8 attention (query-stationary), with the row-sum probes.
//
// Workgroup = 4 waves = 128 queries (32 per wave); grid = (query tiles, Hq, B).
// The wave's Q^<c> and dO^<c> rows sit in registers as the B operands of
// S^T = K Q^T and dP^T = V dO^T, so both score tiles come out with one query per
// lane pair and 16 keys per lane.  Per 128-key chunk (K^<c>, V^<c>, K^<s> staged
// in LDS): P = exp(S - LSE), dS = P (dP^ - delta) in FP32; dS is cast to E5M2 in
// 32-key blocks in registers (the lane pair holds a whole block) and is already
// the B operand of dQ^T += K^<s>^T dS^<k>^T.  Each dQ row is written once, so
// dQ needs no atomics and is bitwise deterministic.  The pre-cast row sums of dS
// and of |P dP^| (the probes) are plain register sums here.
#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

template <int DQK, int DV, bool CAUSAL, bool PROBE>
__global__ __launch_bounds__(256, 2) void dq_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ kc,
    const float* __restrict__ kcs, const uint8_t* __restrict__ vc, const float* __restrict__ vcs,
    const uint8_t* __restrict__ kst, const float* __restrict__ ksts, const uint8_t* __restrict__ doc,
    const float* __restrict__ docs, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dq, double* __restrict__ psum, double* __restrict__ pabs, int Hq, int Hkv, int L, int Lp,
    float sigma) {
  constexpr int KS = DQK / 64, VS = DV / 64, KB = DQK / 32, VB = DV / 32;
  constexpr int NCT = DQK / 32;                 // 32-channel tiles of dQ^T
  constexpr int KROW = DQK + 16, VROW = DV + 16, TROW = kChunk + 16;
  __shared__ __attribute__((aligned(16))) uint8_t sK[kChunk * KROW];
  __shared__ __attribute__((aligned(16))) float sKs[kChunk * KB];
  __shared__ __attribute__((aligned(16))) uint8_t sV[kChunk * VROW];
  __shared__ __attribute__((aligned(16))) float sVs[kChunk * VB];
  __shared__ __attribute__((aligned(16))) uint8_t sKt[DQK * TROW];
  __shared__ __attribute__((aligned(16))) float sKts[DQK * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int R = lane & 31, h = lane >> 5;
  const int nqt = Lp / kChunk;
  const int qt = CAUSAL ? (nqt - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int hk = hq / (Hq / Hkv);
  const int q0 = qt * kChunk;
  const int qi = q0 + 32 * w + R;
  const int LB = Lp / kBlock;
  const int64_t qhead = (int64_t)b * Hq + hq, khead = (int64_t)b * Hkv + hk;
  const uint8_t* Kc = kc + khead * Lp * DQK;
  const float* Kcs = kcs + khead * Lp * KB;
  const uint8_t* Vc = vc + khead * Lp * DV;
  const float* Vcs = vcs + khead * Lp * VB;
  const uint8_t* Kt = kst + khead * DQK * Lp;
  const float* Kts = ksts + khead * DQK * LB;

  v8i qb[KS], db[VS];
  int qsc[KS], dsc[VS];
  {
    const uint8_t* p = qc + (qhead * Lp + qi) * DQK;
    const float* ps = qcs + (qhead * Lp + qi) * KB;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qb[ks] = cat(*reinterpret_cast<const v4i*>(p + 64 * ks + 16 * h), *reinterpret_cast<const v4i*>(p + 64 * ks + 32 + 16 * h));
      qsc[ks] = e8m0(ps[2 * ks + h]);
    }
    const uint8_t* pd = doc + (qhead * Lp + qi) * DV;
    const float* pds = docs + (qhead * Lp + qi) * VB;
#pragma unroll
    for (int ks = 0; ks < VS; ++ks) {
      db[ks] = cat(*reinterpret_cast<const v4i*>(pd + 64 * ks + 16 * h), *reinterpret_cast<const v4i*>(pd + 64 * ks + 32 + 16 * h));
      dsc[ks] = e8m0(pds[2 * ks + h]);
    }
  }
  const float c2 = sigma * kLog2e;
  const float l2 = qi < L ? lse[qhead * L + qi] * kLog2e : INFINITY;   // pad rows: P = 0
  const float del = qi < L ? delta[qhead * L + qi] : 0.f;
  double rsum = 0.0, rabs = 0.0;                // probes: FP32 per chunk, FP64 across chunks
  v16f acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = v16f{};

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
    for (int i = tid; i < DQK * kChunk / 16; i += 256) {
      const int row = i / (kChunk / 16), col = (i % (kChunk / 16)) * 16;
      *reinterpret_cast<v4i*>(sKt + row * TROW + col) = *reinterpret_cast<const v4i*>(Kt + (int64_t)row * Lp + k0 + col);
    }
    for (int i = tid; i < DQK; i += 256)
      *reinterpret_cast<v4f*>(sKts + 4 * i) = *reinterpret_cast<const v4f*>(Kts + (int64_t)i * LB + k0 / kBlock);
    __syncthreads();
    if (CAUSAL && k0 > q0 + 32 * w + 31) continue;   // every key of the chunk is masked for this wave
    const bool need_mask = (k0 + kChunk > L) || (CAUSAL && k0 + kChunk - 1 > q0 + 32 * w);

    v8i dsb[2];
    int dssc[2] = {0, 0};
    float csum = 0.f, cabs = 0.f;
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
      float am = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[v], c2, -l2));
        const float d = p * (dp[v] - del);
        if constexpr (PROBE) {
          csum += d;
          cabs += fabsf(p * dp[v]);
        }
        s[v] = d;                                    // s now holds dS
        am = fmaxf(am, fabsf(d));
      }
      am = pair_max(am);
      const int k = scale_exp<E5M2>(am);
      const float sc = exp2i(k);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        dsb[t >> 1][4 * (t & 1) + g] = (int)pack4s<E5M2>(s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3], sc);
      if ((t & 1) == h) dssc[t >> 1] = k + 127;
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int ch = 32 * ct + R;
        const uint8_t* p = sKt + ch * TROW + 64 * st;
        v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
        acc[ct] = mfma<E4M3, E5M2>(a, dsb[st], acc[ct], e8m0(sKts[ch * 4 + 2 * st + h]), dssc[st]);
      }
    if constexpr (PROBE) {
      rsum += (double)csum;
      rabs += (double)cabs;
    }
  }

  if constexpr (PROBE) {
    rsum = pair_sum_d(rsum);
    rabs = pair_sum_d(rabs);
  }
  if (qi < L) {
    float* row = dq + (qhead * L + qi) * DQK + 4 * h;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        v4f r = {sigma * acc[ct][4 * a], sigma * acc[ct][4 * a + 1], sigma * acc[ct][4 * a + 2],
                 sigma * acc[ct][4 * a + 3]};
        *reinterpret_cast<v4f*>(row + 32 * ct + 8 * a) = r;
      }
    if constexpr (PROBE) {
      if (h == 0) {
        psum[qhead * L + qi] = rsum;
        pabs[qhead * L + qi] = rabs;
      }
    }
  }
}

template <int DQK, int DV, bool CAUSAL, bool PROBE>
static void launch_dq_t4(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                         const float* lse, const float* delta, float* dq, double* ps, double* pa, hipStream_t s) {
  dim3 grid(d.Lp / kChunk, d.Hq, d.B);
  hipLaunchKernelGGL((dq_kernel<DQK, DV, CAUSAL, PROBE>), grid, dim3(256), 0, s, qc.codes, qc.scales, kc.codes,
                     kc.scales, vc.codes, vc.scales, ks.codes, ks.scales, doc.codes, doc.scales, lse, delta, dq, ps,
                     pa, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
}

template <int DQK, int DV>
static void launch_dq_t(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                        const float* lse, const float* delta, float* dq, double* ps, double* pa, hipStream_t s) {
  if (d.causal) {
    if (ps) launch_dq_t4<DQK, DV, true, true>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
    else launch_dq_t4<DQK, DV, true, false>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
  } else {
    if (ps) launch_dq_t4<DQK, DV, false, true>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
    else launch_dq_t4<DQK, DV, false, false>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
  }
}

hipError_t launch_dq(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                     const float* lse, const float* delta, float* dq, double* ps, double* pa, hipStream_t s) {
  if (d.dqk == 64 && d.dv == 64) launch_dq_t<64, 64>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
  else if (d.dqk == 128 && d.dv == 128) launch_dq_t<128, 128>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
  else if (d.dqk == 192 && d.dv == 128) launch_dq_t<192, 128>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
  else if (d.dqk == 64 && d.dv == 128) launch_dq_t<64, 128>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
  else if (d.dqk == 128 && d.dv == 64) launch_dq_t<128, 64>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
  else if (d.dqk == 192 && d.dv == 64) launch_dq_t<192, 64>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dm
