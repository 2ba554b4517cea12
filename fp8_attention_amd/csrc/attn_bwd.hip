// dK and dV of block-scaled FP8 attention (key-stationary).
//
// Workgroup = 8 waves = 128 keys x 64 queries per step; grid = (key tiles, Hkv,
// B).  Wave w = (key group kg = w % 4, query half qh = w / 4) owns keys
// 32kg..32kg+31 and, in each step, queries 32qh..32qh+31 of the step's 64.  A
// workgroup walks the query heads of its KV group and, for each, the query
// blocks of 64 that can see its keys.  Per step:
//   A  S = Q K^T and dP^ = dO V^T for the wave's 32x32 tile (scaled FP8 MFMA;
//      one key per lane pair, 16 queries per lane); P = exp(S - LSE) and
//      dS = P (dP^ - delta) in FP32; the 32-query block casts P^<q> (E4M3) and
//      dS^<q> (E5M2) happen in registers and the codes go to LDS for the
//      partner wave of the other query half;
//   B  dV^T += dO^<s>^T P^<q> and dK^T += Q^<s>^T dS^<q> over the 64 queries,
//      each wave taking half of the channel tiles of its key group.
// The next step's query-side operands are loaded into registers while the
// current step computes.  dK and dV accumulate in registers over every query
// head of the group and are written once (no atomics).  dQ is computed by the
// query-stationary kernel in attn_dq.hip.
#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

constexpr int kBQ = 64;          // queries per step
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

template <int DQK, int DV>
struct BwdSmem {
  static constexpr int QROW = DQK + 16, VROW = DV + 16, TROW = kBQ + 16;
  uint8_t q[kBQ * QROW];                 // Q^<c> rows of the step
  uint8_t dO[kBQ * VROW];                // dO^<c> rows
  uint8_t qt[DQK * TROW];                // Q^<s>: channel rows over the step's 64 queries
  uint8_t dOt[DV * TROW];                // dO^<s>
  v4i pc[4 * 2 * 64];                    // P^<q> codes per (key group, query half, lane)
  v4i dc[4 * 2 * 64];                    // dS^<q> codes
  int psc[4 * 2 * 64];                   // their E8M0 scales
  int dsc[4 * 2 * 64];
  float qsc[kBQ * (DQK / 32)];
  float dOsc[kBQ * (DV / 32)];
  float qtsc[DQK * 2];
  float dOtsc[DV * 2];
  float lse[kBQ];
  float del[kBQ];
};

// K^<c> and V^<c> rows of the workgroup's 128 keys, read from LDS as the B
// operands of S and dP^ (keeps the wave well under 256 VGPRs).
template <int DQK, int DV>
struct KVTile {
  static constexpr int KROW = DQK + 16, VROW = DV + 16;
  uint8_t k[128 * KROW];
  uint8_t v[128 * VROW];
  float ksc[128 * (DQK / 32)];
  float vsc[128 * (DV / 32)];
};

// Register staging of one step's query-side operands (loaded a step ahead).
template <int DQK, int DV>
struct Prefetch {
  static constexpr int NQ = (kBQ * DQK / 16 + kThreads - 1) / kThreads;   // 16-byte pieces per thread
  static constexpr int NV = (kBQ * DV / 16 + kThreads - 1) / kThreads;
  v4i q[NQ], qt[NQ], dO[NV], dOt[NV];
  float qsc, dOsc, qtsc, dOtsc, lse, del;
};

template <int DQK, int DV>
__device__ __forceinline__ void prefetch(Prefetch<DQK, DV>& pf, int tid, int64_t qhead, int q0, int L, int Lp,
                                         const uint8_t* qc, const float* qcs, const uint8_t* qs, const float* qss,
                                         const uint8_t* doc, const float* docs, const uint8_t* dos,
                                         const float* doss, const float* lse, const float* delta) {
  using P = Prefetch<DQK, DV>;
  const int LB = Lp / kBlock;
#pragma unroll
  for (int j = 0; j < P::NQ; ++j) {
    const int i = tid + j * kThreads;
    if (i < kBQ * DQK / 16) {
      const int r = (i * 16) / DQK, c = (i * 16) % DQK;
      pf.q[j] = *reinterpret_cast<const v4i*>(qc + (qhead * Lp + q0 + r) * DQK + c);
      const int rt = i / (kBQ / 16), ct = (i % (kBQ / 16)) * 16;
      pf.qt[j] = *reinterpret_cast<const v4i*>(qs + (qhead * DQK + rt) * Lp + q0 + ct);
    }
  }
#pragma unroll
  for (int j = 0; j < P::NV; ++j) {
    const int i = tid + j * kThreads;
    if (i < kBQ * DV / 16) {
      const int r = (i * 16) / DV, c = (i * 16) % DV;
      pf.dO[j] = *reinterpret_cast<const v4i*>(doc + (qhead * Lp + q0 + r) * DV + c);
      const int rt = i / (kBQ / 16), ct = (i % (kBQ / 16)) * 16;
      pf.dOt[j] = *reinterpret_cast<const v4i*>(dos + (qhead * DV + rt) * Lp + q0 + ct);
    }
  }
  if (tid < kBQ * DQK / 32) pf.qsc = qcs[(qhead * Lp + q0) * (DQK / 32) + tid];
  if (tid < kBQ * DV / 32) pf.dOsc = docs[(qhead * Lp + q0) * (DV / 32) + tid];
  if (tid < DQK * 2) pf.qtsc = qss[(qhead * DQK + tid / 2) * LB + q0 / kBlock + (tid & 1)];
  if (tid < DV * 2) pf.dOtsc = doss[(qhead * DV + tid / 2) * LB + q0 / kBlock + (tid & 1)];
  if (tid < kBQ) {
    const int q = q0 + tid;
    pf.lse = q < L ? lse[qhead * L + q] * kLog2e : INFINITY;
    pf.del = q < L ? delta[qhead * L + q] : 0.f;
  }
}

template <int DQK, int DV>
__device__ __forceinline__ void commit(const Prefetch<DQK, DV>& pf, BwdSmem<DQK, DV>& sm, int tid) {
  using P = Prefetch<DQK, DV>;
  using SM = BwdSmem<DQK, DV>;
#pragma unroll
  for (int j = 0; j < P::NQ; ++j) {
    const int i = tid + j * kThreads;
    if (i < kBQ * DQK / 16) {
      const int r = (i * 16) / DQK, c = (i * 16) % DQK;
      *reinterpret_cast<v4i*>(sm.q + r * SM::QROW + c) = pf.q[j];
      const int rt = i / (kBQ / 16), ct = (i % (kBQ / 16)) * 16;
      *reinterpret_cast<v4i*>(sm.qt + rt * SM::TROW + ct) = pf.qt[j];
    }
  }
#pragma unroll
  for (int j = 0; j < P::NV; ++j) {
    const int i = tid + j * kThreads;
    if (i < kBQ * DV / 16) {
      const int r = (i * 16) / DV, c = (i * 16) % DV;
      *reinterpret_cast<v4i*>(sm.dO + r * SM::VROW + c) = pf.dO[j];
      const int rt = i / (kBQ / 16), ct = (i % (kBQ / 16)) * 16;
      *reinterpret_cast<v4i*>(sm.dOt + rt * SM::TROW + ct) = pf.dOt[j];
    }
  }
  if (tid < kBQ * DQK / 32) sm.qsc[tid] = pf.qsc;
  if (tid < kBQ * DV / 32) sm.dOsc[tid] = pf.dOsc;
  if (tid < DQK * 2) sm.qtsc[tid] = pf.qtsc;
  if (tid < DV * 2) sm.dOtsc[tid] = pf.dOtsc;
  if (tid < kBQ) {
    sm.lse[tid] = pf.lse;
    sm.del[tid] = pf.del;
  }
}

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void dkdv_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ qs,
    const float* __restrict__ qss, const uint8_t* __restrict__ kc, const float* __restrict__ kcs,
    const uint8_t* __restrict__ vc, const float* __restrict__ vcs, const uint8_t* __restrict__ doc,
    const float* __restrict__ docs, const uint8_t* __restrict__ dos, const float* __restrict__ doss,
    const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv,
    int Hq, int Hkv, int L, int Lp, float sigma) {
  constexpr int KS = DQK / 64, VS = DV / 64, KB = DQK / 32, VB = DV / 32;
  constexpr int NKT = DQK / 32, NVT = DV / 32;
  constexpr int NKW = NKT / 2, NVW = NVT / 2;     // channel tiles of dK^T / dV^T per wave
  using SM = BwdSmem<DQK, DV>;
  using KV = KVTile<DQK, DV>;
  __shared__ __attribute__((aligned(16))) SM sm;
  __shared__ __attribute__((aligned(16))) KV kv;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int kg = w & 3, qh = w >> 2;
  const int R = lane & 31, h = lane >> 5;
  const int k0 = blockIdx.x * 128;
  const int hk = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int key = k0 + 32 * kg + R;                  // this lane's key (column of S tiles)
  const int kr = 32 * kg + R;                        // its row in the workgroup's K/V tiles
  const int64_t khead = (int64_t)b * Hkv + hk;

  // the workgroup's K^<c> and V^<c> rows, staged once
  for (int i = tid; i < 128 * DQK / 16; i += kThreads) {
    const int r = (i * 16) / DQK, c = (i * 16) % DQK;
    *reinterpret_cast<v4i*>(kv.k + r * KV::KROW + c) = *reinterpret_cast<const v4i*>(kc + (khead * Lp + k0 + r) * DQK + c);
  }
  for (int i = tid; i < 128 * DV / 16; i += kThreads) {
    const int r = (i * 16) / DV, c = (i * 16) % DV;
    *reinterpret_cast<v4i*>(kv.v + r * KV::VROW + c) = *reinterpret_cast<const v4i*>(vc + (khead * Lp + k0 + r) * DV + c);
  }
  for (int i = tid; i < 128 * KB; i += kThreads) kv.ksc[i] = kcs[(khead * Lp + k0) * KB + i];
  for (int i = tid; i < 128 * VB; i += kThreads) kv.vsc[i] = vcs[(khead * Lp + k0) * VB + i];

  v16f dkacc[NKW], dvacc[NVW];
#pragma unroll
  for (int i = 0; i < NKW; ++i) dkacc[i] = v16f{};
#pragma unroll
  for (int i = 0; i < NVW; ++i) dvacc[i] = v16f{};

  const float c2 = sigma * kLog2e;
  const int arow = 32 * qh + pair_row(R);
  const int qstart = CAUSAL ? k0 : 0;
  const int nsteps = (Lp - qstart) / kBQ;
  const int total = G * nsteps;

  Prefetch<DQK, DV> pf;
  prefetch<DQK, DV>(pf, tid, (int64_t)b * Hq + hk * G, qstart, L, Lp, qc, qcs, qs, qss, doc, docs, dos, doss, lse,
                    delta);
  commit<DQK, DV>(pf, sm, tid);
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int hh = it / nsteps;
    const int q0 = qstart + (it - hh * nsteps) * kBQ;
    if (it + 1 < total) {
      const int hn = (it + 1) / nsteps;
      prefetch<DQK, DV>(pf, tid, (int64_t)b * Hq + hk * G + hn, qstart + (it + 1 - hn * nsteps) * kBQ, L, Lp, qc,
                        qcs, qs, qss, doc, docs, dos, doss, lse, delta);
    }

    // ---- A: S and dP^ tiles; lane (key R, h), register v <-> query 32*qh + 16*h + v
    v16f s = v16f{}, dp = v16f{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint8_t* p = sm.q + arow * SM::QROW + 64 * ks;
      const uint8_t* pk = kv.k + kr * KV::KROW + 64 * ks;
      v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
      v8i bk = cat(lds_read16(pk + 16 * h), lds_read16(pk + 32 + 16 * h));
      s = mfma<E4M3, E4M3>(a, bk, s, e8m0(sm.qsc[arow * KB + 2 * ks + h]), e8m0(kv.ksc[kr * KB + 2 * ks + h]));
    }
#pragma unroll
    for (int ks = 0; ks < VS; ++ks) {
      const uint8_t* p = sm.dO + arow * SM::VROW + 64 * ks;
      const uint8_t* pv = kv.v + kr * KV::VROW + 64 * ks;
      v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
      v8i bv = cat(lds_read16(pv + 16 * h), lds_read16(pv + 32 + 16 * h));
      dp = mfma<E5M2, E4M3>(a, bv, dp, e8m0(sm.dOsc[arow * VB + 2 * ks + h]), e8m0(kv.vsc[kr * VB + 2 * ks + h]));
    }
    const bool need_mask = (k0 + 128 > L) || (CAUSAL && q0 < k0 + 128);
    const int qb = 32 * qh + 16 * h;               // first step-query of this lane's 16
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const v4f l4 = *reinterpret_cast<const v4f*>(sm.lse + qb + 4 * g);
      const v4f d4 = *reinterpret_cast<const v4f*>(sm.del + qb + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * g + e;
        float x = s[v];
        if (need_mask && (key >= L || (CAUSAL && key > q0 + qb + v))) x = -INFINITY;
        const float p = __builtin_amdgcn_exp2f(fmaf(x, c2, -l4[e]));
        s[v] = p;                                   // s now holds P
        dp[v] = p * (dp[v] - d4[e]);                // dp now holds dS
      }
    }
    {
      // P^<q>, dS^<q>: this wave's 32 queries form one block per key (lane pair)
      float am = 0.f, dm = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        am = fmaxf(am, s[v]);
        dm = fmaxf(dm, fabsf(dp[v]));
      }
      am = pair_max(am);
      dm = pair_max(dm);
      const int kp = scale_exp<E4M3>(am), kd = scale_exp<E5M2>(dm);
      const float sp = exp2i(kp), sd = exp2i(kd);
      v4i pw, dw;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        pw[g] = (int)pack4s<E4M3>(s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3], sp);
        dw[g] = (int)pack4s<E5M2>(dp[4 * g], dp[4 * g + 1], dp[4 * g + 2], dp[4 * g + 3], sd);
      }
      const int slot = (kg * 2 + qh) * 64 + lane;
      sm.pc[slot] = pw;
      sm.dc[slot] = dw;
      sm.psc[slot] = kp + 127;
      sm.dsc[slot] = kd + 127;
    }
    __syncthreads();

    // ---- B: dV^T and dK^T over the step's 64 queries (both query halves of key group kg)
    {
      const int s0 = (kg * 2 + 0) * 64 + lane, s1 = (kg * 2 + 1) * 64 + lane;
      const v8i pq = cat(sm.pc[s0], sm.pc[s1]);
      const v8i dsq = cat(sm.dc[s0], sm.dc[s1]);
      const int psc = sm.psc[(kg * 2 + h) * 64 + lane];
      const int dsc = sm.dsc[(kg * 2 + h) * 64 + lane];
#pragma unroll
      for (int m = 0; m < NVW; ++m) {
        const int ch = 32 * (qh + 2 * m) + R;
        const uint8_t* p = sm.dOt + ch * SM::TROW;
        v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
        dvacc[m] = mfma<E5M2, E4M3>(a, pq, dvacc[m], e8m0(sm.dOtsc[ch * 2 + h]), psc);
      }
#pragma unroll
      for (int m = 0; m < NKW; ++m) {
        const int ch = 32 * (qh + 2 * m) + R;
        const uint8_t* p = sm.qt + ch * SM::TROW;
        v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
        dkacc[m] = mfma<E4M3, E5M2>(a, dsq, dkacc[m], e8m0(sm.qtsc[ch * 2 + h]), dsc);
      }
    }
    __syncthreads();
    // every read of this step's staging buffers is done: the next step's operands go in
    if (it + 1 < total) {
      commit<DQK, DV>(pf, sm, tid);
      __syncthreads();
    }
  }

  // ---- dK, dV written once per key: wave (kg, qh) holds channel tiles qh, qh+2, ...
  if (key < L) {
    float* dkr = dk + (khead * L + key) * DQK + 4 * h;
    float* dvr = dv + (khead * L + key) * DV + 4 * h;
#pragma unroll
    for (int m = 0; m < NKW; ++m)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        v4f r = {sigma * dkacc[m][4 * a], sigma * dkacc[m][4 * a + 1], sigma * dkacc[m][4 * a + 2],
                 sigma * dkacc[m][4 * a + 3]};
        *reinterpret_cast<v4f*>(dkr + 32 * (qh + 2 * m) + 8 * a) = r;
      }
#pragma unroll
    for (int m = 0; m < NVW; ++m)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        v4f r = {dvacc[m][4 * a], dvacc[m][4 * a + 1], dvacc[m][4 * a + 2], dvacc[m][4 * a + 3]};
        *reinterpret_cast<v4f*>(dvr + 32 * (qh + 2 * m) + 8 * a) = r;
      }
  }
}

template <int DQK, int DV>
static void launch_dkdv_t(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc,
                          Operand dos, const float* lse, const float* delta, float* dk, float* dv, hipStream_t s) {
  dim3 grid(d.Lp / 128, d.Hkv, d.B);
  if (d.causal)
    hipLaunchKernelGGL((dkdv_kernel<DQK, DV, true>), grid, dim3(kThreads), 0, s, qc.codes, qc.scales, qs.codes,
                       qs.scales, kc.codes, kc.scales, vc.codes, vc.scales, doc.codes, doc.scales, dos.codes,
                       dos.scales, lse, delta, dk, dv, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
  else
    hipLaunchKernelGGL((dkdv_kernel<DQK, DV, false>), grid, dim3(kThreads), 0, s, qc.codes, qc.scales, qs.codes,
                       qs.scales, kc.codes, kc.scales, vc.codes, vc.scales, doc.codes, doc.scales, dos.codes,
                       dos.scales, lse, delta, dk, dv, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
}

hipError_t launch_bwd(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand ks, Operand vc, Operand doc,
                      Operand dos, const float* lse, const float* delta, float* dq, float* dk, float* dv,
                      double* ps, double* pa, hipStream_t s) {
  if (d.dqk == 64 && d.dv == 64) launch_dkdv_t<64, 64>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, s);
  else if (d.dqk == 128 && d.dv == 128) launch_dkdv_t<128, 128>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, s);
  else if (d.dqk == 192 && d.dv == 128) launch_dkdv_t<192, 128>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, s);
  else if (d.dqk == 64 && d.dv == 128) launch_dkdv_t<64, 128>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, s);
  else if (d.dqk == 128 && d.dv == 64) launch_dkdv_t<128, 64>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, s);
  else if (d.dqk == 192 && d.dv == 64) launch_dkdv_t<192, 64>(d, qc, qs, kc, vc, doc, dos, lse, delta, dk, dv, s);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dq(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, s);
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
