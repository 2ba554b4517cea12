// Backward of block-scaled FP8 attention on gfx950 matrix cores.
//
// Key-stationary: workgroup = 8 waves = 128 keys x 64 queries per step; grid =
// (key tiles, Hkv, B).  Wave w = (key group kg = w % 4, query half qh = w / 4)
// owns keys 32kg..32kg+31 and, in each step, queries 32qh..32qh+31 of the
// step's 64.  A workgroup walks the query heads of its KV group and, for each,
// the query blocks of 64 that can see its keys.  Per step:
//   A  S = Q K^T and dP^ = dO V^T for the wave's 32x32 tile (scaled FP8 MFMA;
//      one key per lane pair, 16 queries per lane); P = exp(S - LSE) and
//      dS = P (dP^ - delta) in FP32; the 32-query block casts P^<q> (E4M3) and
//      dS^<q> (E5M2) happen in registers; codes go to LDS for the partner wave
//      of the other query half, dS (FP32) goes to an LDS transpose buffer;
//   B  dV^T += dO^<s>^T P^<q> and dK^T += Q^<s>^T dS^<q> over the 64 queries,
//      each wave taking half of the channel tiles of its key group; the dS
//      transpose is read back one query per lane pair and cast along keys
//      (dS^<k>, E5M2);
//   C  dQ = dS^<k> K^<s> over the 128 keys, one output tile per wave, added to
//      dq with coalesced FP32 atomics.
// The next step's query-side operands are loaded into registers while the
// current step computes.  dK and dV accumulate in registers over every query
// head of the group and are written once.
#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

constexpr int kBQ = 64;          // queries per step
constexpr int kTP = 36;          // LDS pitch (floats) of the dS transpose rows
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

template <int DQK, int DV>
struct BwdSmem {
  static constexpr int QROW = DQK + 16, VROW = DV + 16, TROW = kBQ + 16, KROW = 128 + 16;
  uint8_t q[kBQ * QROW];                 // Q^<c> rows of the step
  uint8_t dO[kBQ * VROW];                // dO^<c> rows
  uint8_t qt[DQK * TROW];                // Q^<s>: channel rows over the step's 64 queries
  uint8_t dOt[DV * TROW];                // dO^<s>
  uint8_t dsk[kBQ * KROW];               // dS^<k> codes: 64 queries x 128 keys
  uint8_t kt[DQK * KROW];                // K^<s>: channel rows over the workgroup's 128 keys
  v4i pc[4 * 2 * 64];                    // P^<q> codes per (key group, query half, lane)
  v4i dc[4 * 2 * 64];                    // dS^<q> codes
  int psc[4 * 2 * 64];                   // their E8M0 scales
  int dsc[4 * 2 * 64];
  float qsc[kBQ * (DQK / 32)];
  float dOsc[kBQ * (DV / 32)];
  float qtsc[DQK * 2];
  float dOtsc[DV * 2];
  float ktsc[DQK * 4];
  int dsksc[kBQ * 4];
  float lse[kBQ];
  float del[kBQ];
  float pabs[kBQ];                       // probe: per-query sum_j |P dP^| over the workgroup's keys
  float tr[4 * kBQ * kTP];               // dS transpose, one 64 x 32 slab per key group
};

// V^<c> rows of the workgroup's 128 keys, kept in LDS (instead of registers) when
// the LDS budget allows it (d_qk <= 128), to keep the wave under 256 VGPRs.
template <int DV, bool ON>
struct VTile {
  static constexpr int ROW = DV + 16;
  uint8_t v[ON ? 128 * ROW : 16];
  float vsc[ON ? 128 * (DV / 32) : 4];
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

template <int DQK, int DV, bool PROBE>
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
    if constexpr (PROBE) sm.pabs[tid] = 0.f;
  }
}

template <int DQK, int DV, bool CAUSAL, bool PROBE>
__global__ __launch_bounds__(kThreads) void bwd_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ qs,
    const float* __restrict__ qss, const uint8_t* __restrict__ kc, const float* __restrict__ kcs,
    const uint8_t* __restrict__ kst, const float* __restrict__ ksts, const uint8_t* __restrict__ vc,
    const float* __restrict__ vcs, const uint8_t* __restrict__ doc, const float* __restrict__ docs,
    const uint8_t* __restrict__ dos, const float* __restrict__ doss, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    double* __restrict__ psum, double* __restrict__ pabs, int Hq, int Hkv, int L, int Lp, float sigma) {
  constexpr int KS = DQK / 64, VS = DV / 64, KB = DQK / 32, VB = DV / 32;
  constexpr int NKT = DQK / 32, NVT = DV / 32;
  constexpr int NKW = NKT / 2, NVW = NVT / 2;     // channel tiles of dK^T / dV^T per wave
  using SM = BwdSmem<DQK, DV>;
  constexpr bool VLDS = DQK <= 128;
  using VT = VTile<DV, VLDS>;
  __shared__ __attribute__((aligned(16))) SM sm;
  __shared__ __attribute__((aligned(16))) VT vt;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int kg = w & 3, qh = w >> 2;
  const int R = lane & 31, h = lane >> 5;
  const int k0 = blockIdx.x * 128;
  const int hk = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int key = k0 + 32 * kg + R;                  // this lane's key (column of S tiles)
  const int64_t khead = (int64_t)b * Hkv + hk;
  const int LB = Lp / kBlock;

  // resident key-side operands (B operands of S and dP^)
  v8i kb[KS], vb[VLDS ? 1 : VS];
  int ksc[KS], vsc[VLDS ? 1 : VS];
  {
    const uint8_t* kp = kc + (khead * Lp + key) * DQK;
    const float* kps = kcs + (khead * Lp + key) * KB;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kb[s] = cat(*reinterpret_cast<const v4i*>(kp + 64 * s + 16 * h), *reinterpret_cast<const v4i*>(kp + 64 * s + 32 + 16 * h));
      ksc[s] = e8m0(kps[2 * s + h]);
    }
    if constexpr (!VLDS) {
      const uint8_t* vp = vc + (khead * Lp + key) * DV;
      const float* vps = vcs + (khead * Lp + key) * VB;
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        vb[s] = cat(*reinterpret_cast<const v4i*>(vp + 64 * s + 16 * h), *reinterpret_cast<const v4i*>(vp + 64 * s + 32 + 16 * h));
        vsc[s] = e8m0(vps[2 * s + h]);
      }
    }
  }
  if constexpr (VLDS) {
    for (int i = tid; i < 128 * DV / 16; i += kThreads) {
      const int r = (i * 16) / DV, c = (i * 16) % DV;
      *reinterpret_cast<v4i*>(vt.v + r * VT::ROW + c) = *reinterpret_cast<const v4i*>(vc + (khead * Lp + k0 + r) * DV + c);
    }
    for (int i = tid; i < 128 * VB; i += kThreads) vt.vsc[i] = vcs[(khead * Lp + k0) * VB + i];
  }
  // K^<s> rows (channels) over the workgroup's 128 keys, staged once for dQ
  for (int i = tid; i < DQK * 8; i += kThreads) {
    const int r = i / 8, c = (i % 8) * 16;
    *reinterpret_cast<v4i*>(sm.kt + r * SM::KROW + c) = *reinterpret_cast<const v4i*>(kst + (khead * DQK + r) * Lp + k0 + c);
  }
  for (int i = tid; i < DQK; i += kThreads)
    *reinterpret_cast<v4f*>(sm.ktsc + 4 * i) = *reinterpret_cast<const v4f*>(ksts + (khead * DQK + i) * LB + k0 / kBlock);

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
  commit<DQK, DV, PROBE>(pf, sm, tid);
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int hh = it / nsteps;
    const int q0 = qstart + (it - hh * nsteps) * kBQ;
    const int64_t qhead = (int64_t)b * Hq + hk * G + hh;
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
      v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
      s = mfma<E4M3, E4M3>(a, kb[ks], s, e8m0(sm.qsc[arow * KB + 2 * ks + h]), ksc[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < VS; ++ks) {
      const uint8_t* p = sm.dO + arow * SM::VROW + 64 * ks;
      v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
      if constexpr (VLDS) {
        const int kr = 32 * kg + R;
        const uint8_t* pv = vt.v + kr * VT::ROW + 64 * ks;
        v8i bv = cat(lds_read16(pv + 16 * h), lds_read16(pv + 32 + 16 * h));
        dp = mfma<E5M2, E4M3>(a, bv, dp, e8m0(sm.dOsc[arow * VB + 2 * ks + h]), e8m0(vt.vsc[kr * VB + 2 * ks + h]));
      } else {
        dp = mfma<E5M2, E4M3>(a, vb[ks], dp, e8m0(sm.dOsc[arow * VB + 2 * ks + h]), vsc[ks]);
      }
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
      const float ip = exp2i(-kp), id = exp2i(-kd);
      v4i pw, dw;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        pw[g] = (int)pack4<E4M3>(s[4 * g] * ip, s[4 * g + 1] * ip, s[4 * g + 2] * ip, s[4 * g + 3] * ip);
        dw[g] = (int)pack4<E5M2>(dp[4 * g] * id, dp[4 * g + 1] * id, dp[4 * g + 2] * id, dp[4 * g + 3] * id);
      }
      const int slot = (kg * 2 + qh) * 64 + lane;
      sm.pc[slot] = pw;
      sm.dc[slot] = dw;
      sm.psc[slot] = kp + 127;
      sm.dsc[slot] = kd + 127;
      float* tw = sm.tr + kg * kBQ * kTP;
#pragma unroll
      for (int v = 0; v < 16; ++v) tw[(qb + v) * kTP + R] = dp[v];
      if constexpr (PROBE) {
        // |P dP^| = |dS + P delta|, summed over the keys into the step's per-query slots
#pragma unroll
        for (int v = 0; v < 16; ++v) atomicAdd(&sm.pabs[qb + v], fabsf(dp[v] + s[v] * sm.del[qb + v]));
      }
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
    {
      // dS^<k>: lane pair (query 32qh + R) reads the 32 keys of group kg
      const int qq = 32 * qh + R;
      const float* tw = sm.tr + kg * kBQ * kTP + qq * kTP + 16 * h;
      float x[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4f t4 = *reinterpret_cast<const v4f*>(tw + 4 * g);
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
      *reinterpret_cast<v4i*>(sm.dsk + qq * SM::KROW + 32 * kg + 16 * h) = cw;
      if (h == 0) sm.dsksc[qq * 4 + kg] = k + 127;
      if constexpr (PROBE) {
        float rs = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) rs += x[v];
        rs = pair_sum(rs);
        // branch-free: every lane adds, pad rows and the second lane of each pair add zero
        const int q = q0 + qq;
        const int qcl = q < L ? q : L - 1;
        const bool own = h == 0 && q < L;
        atomicAdd(psum + qhead * L + qcl, own ? (double)rs : 0.0);
        atomicAdd(pabs + qhead * L + qcl, own && kg == 0 ? (double)sm.pabs[qq] : 0.0);
      }
    }
    __syncthreads();

    // ---- C: dQ = dS^<k> K^<s> over the workgroup's 128 keys, added to dq.  The output
    // tile has 32 consecutive channels across the lanes of each register, so each
    // atomic instruction covers two 128-byte row segments; rows past L add zero to
    // row L-1 so that no lane branches around the matrix instructions.
    // The staging buffers are free now: the next step's operands go in first.
    if (it + 1 < total) commit<DQK, DV, PROBE>(pf, sm, tid);
    for (int t = w; t < 2 * NKT; t += kWaves) {
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
        const int qcl = q < L ? q : L - 1;
        atomicAdd(dq + (qhead * L + qcl) * DQK + 32 * ct + R, q < L ? sigma * acc[v] : 0.f);
      }
    }
    __syncthreads();
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
  hipLaunchKernelGGL((bwd_kernel<DQK, DV, CAUSAL, PROBE>), grid, dim3(kThreads), 0, s, qc.codes, qc.scales, qs.codes,
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
