// Backward of block-scaled FP8 attention on gfx950 matrix cores.
//
// Key-stationary: workgroup = 4 waves = 128 keys (32 per wave), grid = (key
// tiles, Hkv, B).  A workgroup walks the query heads of its KV group and, for
// each, the query blocks of 64 that can see its keys.  Per step:
//   Q^<c>, dO^<c> (row operands), Q^<s>, dO^<s> (sequence-blocked, transposed),
//   LSE and delta of the 64 queries are staged in LDS;
//   S = Q K^T and dP^ = dO V^T come out with one key per lane pair and 16
//   queries per lane (scaled FP8 MFMA, FP32 accumulate);
//   P = exp(S - LSE), dS = P * (dP^ - delta) in FP32;
//   P^<q> and dS^<q> (32-query blocks) are cast in registers -- the lane pair
//   already holds a whole block -- and feed dV^T += dO^T P^<q>, dK^T += Q^T dS^<q>;
//   dS is transposed through LDS so that a lane pair holds 32 keys of one query,
//   cast to dS^<k> (32-key blocks), and dQ^T = K^T dS^<k>^T over the workgroup's
//   128 keys is added to dq with FP32 atomics.
// dK and dV accumulate in registers over every query head of the group and are
// written once (no atomics).
#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

constexpr int kBQ = 64;          // queries per step
constexpr int kTP = 36;          // LDS pitch (floats) of the dS transpose rows

template <int DQK, int DV>
struct BwdSmem {
  static constexpr int QROW = DQK + 16, VROW = DV + 16, TROW = kBQ + 16, KROW = 128 + 16;
  uint8_t q[kBQ * QROW];
  uint8_t dO[kBQ * VROW];
  uint8_t qt[DQK * TROW];
  uint8_t dOt[DV * TROW];
  uint8_t dsk[kBQ * KROW];
  float qsc[kBQ * (DQK / 32)];
  float dOsc[kBQ * (DV / 32)];
  float qtsc[DQK * 2];
  float dOtsc[DV * 2];
  int dsksc[kBQ * 4];
  float lse[kBQ];
  float del[kBQ];
  float pabs[kBQ];                 // probe: per-query sum_j |P dP^| over the workgroup's keys
  float tr[4 * kBQ * kTP];
  uint8_t kt[DQK * KROW];          // K^<s> rows (channels) over the workgroup's 128 keys
  float ktsc[DQK * 4];
};

template <int DQK, int DV, bool CAUSAL, bool PROBE>
__global__ __launch_bounds__(256) void bwd_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ qs,
    const float* __restrict__ qss, const uint8_t* __restrict__ kc, const float* __restrict__ kcs,
    const uint8_t* __restrict__ kst, const float* __restrict__ ksts, const uint8_t* __restrict__ vc,
    const float* __restrict__ vcs, const uint8_t* __restrict__ doc, const float* __restrict__ docs,
    const uint8_t* __restrict__ dos, const float* __restrict__ doss, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    double* __restrict__ psum, double* __restrict__ pabs, int Hq, int Hkv, int L, int Lp, float sigma) {
  constexpr int KS = DQK / 64, VS = DV / 64, KB = DQK / 32, VB = DV / 32;
  constexpr int NKT = DQK / 32, NVT = DV / 32;
  using SM = BwdSmem<DQK, DV>;
  __shared__ __attribute__((aligned(16))) SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int R = lane & 31, h = lane >> 5;
  const int k0 = blockIdx.x * 128;
  const int hk = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int key = k0 + 32 * w + R;                   // this lane's key (column of S tiles)
  const int64_t khead = (int64_t)b * Hkv + hk;
  const int LB = Lp / kBlock;

  // resident key-side operands
  v8i kb[KS], vb[VS];
  int ksc[KS], vsc[VS];
  {
    const uint8_t* kp = kc + (khead * Lp + key) * DQK;
    const float* kps = kcs + (khead * Lp + key) * KB;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kb[s] = cat(*reinterpret_cast<const v4i*>(kp + 64 * s + 16 * h), *reinterpret_cast<const v4i*>(kp + 64 * s + 32 + 16 * h));
      ksc[s] = e8m0(kps[2 * s + h]);
    }
    const uint8_t* vp = vc + (khead * Lp + key) * DV;
    const float* vps = vcs + (khead * Lp + key) * VB;
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      vb[s] = cat(*reinterpret_cast<const v4i*>(vp + 64 * s + 16 * h), *reinterpret_cast<const v4i*>(vp + 64 * s + 32 + 16 * h));
      vsc[s] = e8m0(vps[2 * s + h]);
    }
  }
  // K^<s> rows (channels) over the workgroup's 128 keys, staged once in LDS for dQ
  for (int i = tid; i < DQK * 8; i += 256) {
    const int r = i / 8, c = (i % 8) * 16;
    *reinterpret_cast<v4i*>(sm.kt + r * SM::KROW + c) = *reinterpret_cast<const v4i*>(kst + (khead * DQK + r) * Lp + k0 + c);
  }
  for (int i = tid; i < DQK; i += 256)
    *reinterpret_cast<v4f*>(sm.ktsc + 4 * i) = *reinterpret_cast<const v4f*>(ksts + (khead * DQK + i) * LB + k0 / kBlock);

  v16f dkacc[NKT], dvacc[NVT];
#pragma unroll
  for (int i = 0; i < NKT; ++i) dkacc[i] = v16f{};
#pragma unroll
  for (int i = 0; i < NVT; ++i) dvacc[i] = v16f{};

  const float c2 = sigma * kLog2e;
  const int arow = pair_row(R);
  const int qstart = CAUSAL ? k0 : 0;
  for (int hh = 0; hh < G; ++hh) {
    const int hq = hk * G + hh;
    const int64_t qhead = (int64_t)b * Hq + hq;
    for (int q0 = qstart; q0 < Lp; q0 += kBQ) {
      __syncthreads();
      // ---- stage the query-side operands of this step
      for (int i = tid; i < kBQ * DQK / 16; i += 256) {
        const int r = (i * 16) / DQK, c = (i * 16) % DQK;
        *reinterpret_cast<v4i*>(sm.q + r * SM::QROW + c) = *reinterpret_cast<const v4i*>(qc + (qhead * Lp + q0 + r) * DQK + c);
      }
      for (int i = tid; i < kBQ * DV / 16; i += 256) {
        const int r = (i * 16) / DV, c = (i * 16) % DV;
        *reinterpret_cast<v4i*>(sm.dO + r * SM::VROW + c) = *reinterpret_cast<const v4i*>(doc + (qhead * Lp + q0 + r) * DV + c);
      }
      for (int i = tid; i < DQK * kBQ / 16; i += 256) {
        const int r = i / (kBQ / 16), c = (i % (kBQ / 16)) * 16;
        *reinterpret_cast<v4i*>(sm.qt + r * SM::TROW + c) = *reinterpret_cast<const v4i*>(qs + (qhead * DQK + r) * Lp + q0 + c);
      }
      for (int i = tid; i < DV * kBQ / 16; i += 256) {
        const int r = i / (kBQ / 16), c = (i % (kBQ / 16)) * 16;
        *reinterpret_cast<v4i*>(sm.dOt + r * SM::TROW + c) = *reinterpret_cast<const v4i*>(dos + (qhead * DV + r) * Lp + q0 + c);
      }
      for (int i = tid; i < kBQ * KB; i += 256) sm.qsc[i] = qcs[(qhead * Lp + q0) * KB + i];
      for (int i = tid; i < kBQ * VB; i += 256) sm.dOsc[i] = docs[(qhead * Lp + q0) * VB + i];
      for (int i = tid; i < DQK * 2; i += 256) sm.qtsc[i] = qss[(qhead * DQK + i / 2) * LB + q0 / kBlock + (i & 1)];
      for (int i = tid; i < DV * 2; i += 256) sm.dOtsc[i] = doss[(qhead * DV + i / 2) * LB + q0 / kBlock + (i & 1)];
      if (tid < kBQ) {
        const int q = q0 + tid;
        sm.lse[tid] = q < L ? lse[qhead * L + q] * kLog2e : INFINITY;
        sm.del[tid] = q < L ? delta[qhead * L + q] : 0.f;
        if constexpr (PROBE) sm.pabs[tid] = 0.f;
      }
      __syncthreads();

      // ---- S and dP^ tiles: lane (key R, h), register v <-> query 32*tq + 16*h + v
      v16f s[2], dp[2];
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const int r = 32 * tq + arow;
        s[tq] = v16f{};
        dp[tq] = v16f{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint8_t* p = sm.q + r * SM::QROW + 64 * ks;
          v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
          s[tq] = mfma<E4M3, E4M3>(a, kb[ks], s[tq], e8m0(sm.qsc[r * KB + 2 * ks + h]), ksc[ks]);
        }
#pragma unroll
        for (int ks = 0; ks < VS; ++ks) {
          const uint8_t* p = sm.dO + r * SM::VROW + 64 * ks;
          v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
          dp[tq] = mfma<E5M2, E4M3>(a, vb[ks], dp[tq], e8m0(sm.dOsc[r * VB + 2 * ks + h]), vsc[ks]);
        }
      }
      // ---- P and dS (FP32); masked entries are exact zeros
      const bool need_mask = (k0 + 128 > L) || (CAUSAL && q0 < k0 + 128);
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qq = 32 * tq + 16 * h + 4 * g;
          const v4f l4 = *reinterpret_cast<const v4f*>(sm.lse + qq);
          const v4f d4 = *reinterpret_cast<const v4f*>(sm.del + qq);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * g + e;
            float x = s[tq][v];
            if (need_mask && (key >= L || (CAUSAL && key > q0 + qq + e))) x = -INFINITY;
            const float p = __builtin_amdgcn_exp2f(fmaf(x, c2, -l4[e]));
            s[tq][v] = p;                                   // s now holds P
            dp[tq][v] = p * (dp[tq][v] - d4[e]);            // dp now holds dS
          }
        }
      }
      // ---- dV^T += dO^<s>^T P^<q>
      {
        v8i pq;
        int psc = 0;
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) {
          float am = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) am = fmaxf(am, s[tq][v]);
          am = pair_max(am);
          const int k = scale_exp<E4M3>(am);
          const float inv = exp2i(-k);
#pragma unroll
          for (int g = 0; g < 4; ++g)
            pq[4 * tq + g] = (int)pack4<E4M3>(s[tq][4 * g] * inv, s[tq][4 * g + 1] * inv, s[tq][4 * g + 2] * inv,
                                              s[tq][4 * g + 3] * inv);
          if (tq == h) psc = k + 127;
        }
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
          const uint8_t* p = sm.dOt + (32 * ct + R) * SM::TROW;
          v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
          dvacc[ct] = mfma<E5M2, E4M3>(a, pq, dvacc[ct], e8m0(sm.dOtsc[(32 * ct + R) * 2 + h]), psc);
        }
      }
      // ---- dK^T += Q^<s>^T dS^<q>
      {
        v8i dsq;
        int dsc = 0;
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) {
          float am = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) am = fmaxf(am, fabsf(dp[tq][v]));
          am = pair_max(am);
          const int k = scale_exp<E5M2>(am);
          const float inv = exp2i(-k);
#pragma unroll
          for (int g = 0; g < 4; ++g)
            dsq[4 * tq + g] = (int)pack4<E5M2>(dp[tq][4 * g] * inv, dp[tq][4 * g + 1] * inv, dp[tq][4 * g + 2] * inv,
                                               dp[tq][4 * g + 3] * inv);
          if (tq == h) dsc = k + 127;
        }
#pragma unroll
        for (int ct = 0; ct < NKT; ++ct) {
          const uint8_t* p = sm.qt + (32 * ct + R) * SM::TROW;
          v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
          dkacc[ct] = mfma<E4M3, E5M2>(a, dsq, dkacc[ct], e8m0(sm.qtsc[(32 * ct + R) * 2 + h]), dsc);
        }
      }
      // ---- dS transpose through LDS: row = query of the step, column = key of the wave
      {
        float* tw = sm.tr + w * kBQ * kTP;
#pragma unroll
        for (int tq = 0; tq < 2; ++tq)
#pragma unroll
          for (int v = 0; v < 16; ++v) tw[(32 * tq + 16 * h + v) * kTP + R] = dp[tq][v];
        if constexpr (PROBE) {
          // |P dP^| = |dS + P delta|, summed over this wave's keys into the step's per-query slots
#pragma unroll
          for (int tq = 0; tq < 2; ++tq)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int qq = 32 * tq + 16 * h + v;
              atomicAdd(&sm.pabs[qq], fabsf(dp[tq][v] + s[tq][v] * sm.del[qq]));
            }
        }
      }
      __syncthreads();
      {
        const float* tw = sm.tr + w * kBQ * kTP;
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) {
          const int qq = 32 * tq + R;                  // query of this lane pair
          float x[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v4f t4 = *reinterpret_cast<const v4f*>(tw + qq * kTP + 16 * h + 4 * g);
            x[4 * g] = t4[0]; x[4 * g + 1] = t4[1]; x[4 * g + 2] = t4[2]; x[4 * g + 3] = t4[3];
          }
          float am = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) am = fmaxf(am, fabsf(x[v]));
          am = pair_max(am);
          const int k = scale_exp<E5M2>(am);
          const float inv = exp2i(-k);
          v4i cw;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            cw[g] = (int)pack4<E5M2>(x[4 * g] * inv, x[4 * g + 1] * inv, x[4 * g + 2] * inv, x[4 * g + 3] * inv);
          *reinterpret_cast<v4i*>(sm.dsk + qq * SM::KROW + 32 * w + 16 * h) = cw;
          if (h == 0) sm.dsksc[qq * 4 + w] = k + 127;
          if constexpr (PROBE) {
            float rs = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) rs += x[v];
            rs = pair_sum(rs);
            const int q = q0 + qq;
            if (h == 0 && q < L) atomicAdd(psum + qhead * L + q, (double)rs);
            if (w == 0 && h == 0 && q < L) atomicAdd(pabs + qhead * L + q, (double)sm.pabs[qq]);
          }
        }
      }
      __syncthreads();
      // ---- dQ = dS^<k> K^<s> over the workgroup's 128 keys, added to dq.  The output
      // tile has 32 consecutive channels across the lanes of each register, so each
      // atomic instruction covers two 128-byte row segments; rows past L add zero to
      // row L-1 so that no lane branches around the matrix instructions.
      for (int t = w; t < 2 * NKT; t += 4) {
        const int ct = t >> 1, tq = t & 1;
        const int qq = 32 * tq + R;
        v16f acc = v16f{};
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint8_t* pa = sm.dsk + qq * SM::KROW + 64 * st;
          const uint8_t* pb = sm.kt + (32 * ct + R) * SM::KROW + 64 * st;
          v8i a = cat(lds_read16(pa + 16 * h), lds_read16(pa + 32 + 16 * h));
          v8i bb = cat(lds_read16(pb + 16 * h), lds_read16(pb + 32 + 16 * h));
          acc = mfma<E5M2, E4M3>(a, bb, acc, sm.dsksc[qq * 4 + 2 * st + h],
                                 e8m0(sm.ktsc[(32 * ct + R) * 4 + 2 * st + h]));
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = q0 + 32 * tq + 8 * (v >> 2) + 4 * h + (v & 3);
          const int qc = q < L ? q : L - 1;
          atomicAdd(dq + (qhead * L + qc) * DQK + 32 * ct + R, q < L ? sigma * acc[v] : 0.f);
        }
      }
    }
  }
  // ---- dK, dV written once per key
  if (key < L) {
    float* dkr = dk + (khead * L + key) * DQK + 4 * h;
    float* dvr = dv + (khead * L + key) * DV + 4 * h;
#pragma unroll
    for (int ct = 0; ct < NKT; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        v4f r = {sigma * dkacc[ct][4 * a], sigma * dkacc[ct][4 * a + 1], sigma * dkacc[ct][4 * a + 2],
                 sigma * dkacc[ct][4 * a + 3]};
        *reinterpret_cast<v4f*>(dkr + 32 * ct + 8 * a) = r;
      }
#pragma unroll
    for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        v4f r = {dvacc[ct][4 * a], dvacc[ct][4 * a + 1], dvacc[ct][4 * a + 2], dvacc[ct][4 * a + 3]};
        *reinterpret_cast<v4f*>(dvr + 32 * ct + 8 * a) = r;
      }
  }
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

template <int DQK, int DV, bool CAUSAL, bool PROBE>
static void launch_bwd_t4(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand ks, Operand vc, Operand doc,
                          Operand dos, const float* lse, const float* delta, float* dq, float* dk, float* dv,
                          double* ps, double* pa, hipStream_t s) {
  dim3 grid(d.Lp / 128, d.Hkv, d.B);
  hipLaunchKernelGGL((bwd_kernel<DQK, DV, CAUSAL, PROBE>), grid, dim3(256), 0, s, qc.codes, qc.scales, qs.codes,
                     qs.scales, kc.codes, kc.scales, ks.codes, ks.scales, vc.codes, vc.scales, doc.codes, doc.scales,
                     dos.codes, dos.scales, lse, delta, dq, dk, dv, ps, pa, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
}

template <int DQK, int DV>
static void launch_bwd_t(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand ks, Operand vc, Operand doc,
                         Operand dos, const float* lse, const float* delta, float* dq, float* dk, float* dv,
                         double* ps, double* pa, hipStream_t s) {
  const bool probe = ps != nullptr;
  if (d.causal) {
    if (probe) launch_bwd_t4<DQK, DV, true, true>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
    else launch_bwd_t4<DQK, DV, true, false>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
  } else {
    if (probe) launch_bwd_t4<DQK, DV, false, true>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
    else launch_bwd_t4<DQK, DV, false, false>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
  }
}

hipError_t launch_bwd(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand ks, Operand vc, Operand doc,
                      Operand dos, const float* lse, const float* delta, float* dq, float* dk, float* dv,
                      double* ps, double* pa, hipStream_t s) {
  hipError_t e = launch_fill_zero(dq, (int64_t)d.B * d.Hq * d.L * d.dqk * 4, s);
  if (e != hipSuccess) return e;
  if (ps) {
    if ((e = launch_fill_zero(ps, (int64_t)d.B * d.Hq * d.L * 8, s)) != hipSuccess) return e;
    if ((e = launch_fill_zero(pa, (int64_t)d.B * d.Hq * d.L * 8, s)) != hipSuccess) return e;
  }
  if (d.dqk == 64 && d.dv == 64) launch_bwd_t<64, 64>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
  else if (d.dqk == 128 && d.dv == 128) launch_bwd_t<128, 128>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
  else if (d.dqk == 192 && d.dv == 128) launch_bwd_t<192, 128>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
  else if (d.dqk == 64 && d.dv == 128) launch_bwd_t<64, 128>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
  else if (d.dqk == 128 && d.dv == 64) launch_bwd_t<128, 64>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
  else if (d.dqk == 192 && d.dv == 64) launch_bwd_t<192, 64>(d, qc, qs, kc, ks, vc, doc, dos, lse, delta, dq, dk, dv, ps, pa, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dm
