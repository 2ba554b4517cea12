// dQ of block-scaled FP8 attention (query-stationary), with the row-sum probes.
//
// Workgroup = 8 waves = 256 queries (32 per wave; 4 waves when d_qk + d_v > 256);
// a 1-D grid over (query tile, Hq, B) with the query tile slowest, so the longest
// causal tiles start first.
// The wave's Q^<c> and dO^<c> rows sit in registers as the B operands of
// S^T = K Q^T and dP^T = V dO^T, so both score tiles come out with one query per
// lane pair and 16 keys per lane.  Per 128-key chunk (64 keys when d = 256) and
// 32-key tile:
// P = exp(S - LSE), dS = P (dP^ - delta) in FP32; dS is cast to E5M2 in 32-key
// blocks in registers (the lane pair holds a whole block) and is already the B
// operand of dQ^T += K^<s>^T dS^<k>^T.  Each dQ row is written once, so dQ needs
// no atomics and is bitwise deterministic.  The pre-cast row sums of dS and of
// |P dP^| (the probes) are plain register sums here; the PROBE instance runs the
// arithmetic of the plain one unchanged (same waves, same products, same casts),
// so its dQ is bit for bit the plain instance's and its sums are those of the dS
// that instance casts.
// K^<c>, V^<c> and K^<s> chunks arrive in double-buffered LDS by direct
// global->LDS loads issued one chunk ahead; one barrier per chunk.
#pragma once
#include <type_traits>

#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

// waves per workgroup (32 queries each): 8 (two per SIMD); head dims beyond
// d_qk + d_v = 256 (192/128: spills at two waves per SIMD and runs 25% faster at one;
// 256/256) run one wave per SIMD with the full register file (accumulators in AGPRs)
template <int DQK, int DV> constexpr int dq_waves() { return DQK + DV > 256 ? 4 : 8; }
// keys per LDS chunk: 128, or 64 when d_qk = d_v = 256 (two chunks of K^<c>, V^<c>
// and K^<s> at 128 keys would not fit in LDS)
template <int DQK, int DV> constexpr int dq_chunk() { return DQK + DV > 384 ? 64 : 128; }

template <int DQK, int DV, int NW, int CK>
struct DqLds {
  static constexpr int KB = DQK / 32, VB = DV / 32;
  // K part: K^<c> rows [CK][DQK] (swizzled) + scales [CK][KB]
  static constexpr int K = CK * DQK, KS = CK * KB * 4, KPART = K + KS;
  // V part: V^<c> rows [CK][DV] + scales [CK][VB], K^<s> rows [DQK][CK] + scales [DQK][4]
  // (the aligned group of four 32-key blocks that holds the chunk's blocks)
  static constexpr int V = CK * DV, VS = CK * VB * 4, T = DQK * CK, TS = DQK * 16;
  static constexpr int OFF_VS = V, OFF_T = V + VS, OFF_TS = V + VS + T, VPART = V + VS + T + TS;
  static constexpr int OFF_VP = 2 * KPART;                      // V parts follow the two K parts
  static constexpr int BYTES = 2 * KPART + 2 * VPART;
  static constexpr int NJK = KPART / 1024, NJV = VPART / 1024;
  static constexpr int NJKW = (NJK + NW - 1) / NW, NJVW = (NJV + NW - 1) / NW;
  static_assert(K % 1024 == 0 && KS % 1024 == 0 && V % 1024 == 0 && VS % 1024 == 0 && T % 1024 == 0 &&
                TS % 1024 == 0, "whole 1 KB loads");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int DQK, int DV, bool CAUSAL, bool PROBE>
__global__ __launch_bounds__((64 * dq_waves<DQK, DV>())) void dq_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ kc,
    const float* __restrict__ kcs, const uint8_t* __restrict__ vc, const float* __restrict__ vcs,
    const uint8_t* __restrict__ kst, const float* __restrict__ ksts, const uint8_t* __restrict__ doc,
    const float* __restrict__ docs, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dq, double* __restrict__ psum, double* __restrict__ pabs, double* __restrict__ pcast, int Hq,
    int Hkv, int L, int Lp,
    float sigma) {
  constexpr int kDqWaves = dq_waves<DQK, DV>(), kDqQ = 32 * kDqWaves;
  constexpr int CK = dq_chunk<DQK, DV>(), NTL = CK / 32, NST = CK / 64;   // key tiles, 64-key halves
  using C = DqLds<DQK, DV, kDqWaves, CK>;
  constexpr int KS = DQK / 64, VS = DV / 64, KB = DQK / 32, VB = DV / 32;
  constexpr int NCT = DQK / 32;                 // 32-channel tiles of dQ^T
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int R = lane & 31, h = lane >> 5;
  const int nqt = (Lp + kDqQ - 1) / kDqQ;
  const QueryItem item = query_item((int)blockIdx.x, nqt, Hq, Hkv, (int)gridDim.x / (nqt * Hq));
  const int qt = CAUSAL ? (nqt - 1 - item.tr) : item.tr;  // longest causal tiles first
  const int hq = item.hq, b = item.b;
  const int hk = hq / (Hq / Hkv);
  const int q0 = qt * kDqQ;
  const int qw = q0 + 32 * w;
  const bool live = qw < Lp;
  const int qi = qw + R;
  const int LB = Lp / kBlock;
  const int64_t qhead = (int64_t)b * Hq + hq, khead = (int64_t)b * Hkv + hk;
  const uint8_t* Kc = kc + khead * Lp * DQK;
  const float* Kcs = kcs + khead * Lp * KB;
  const uint8_t* Vc = vc + khead * Lp * DV;
  const float* Vcs = vcs + khead * Lp * VB;
  const uint8_t* Kt = kst + khead * DQK * Lp;
  const float* Kts = ksts + khead * DQK * LB;

  // ---- direct-load source offsets of this lane (relative to the chunk), loop invariant
  int ko[C::NJKW], vo[C::NJVW];
#pragma unroll
  for (int i = 0; i < C::NJKW; ++i) {
    const int pb = (w + kDqWaves * i) * 1024 + 16 * lane;
    if (pb < C::K) {
      const int r = pb / DQK, c = (pb % DQK) / 16;
      ko[i] = r * DQK + 16 * tile_slot<DQK>(r, c);
    } else {
      ko[i] = pb - C::K;
    }
  }
#pragma unroll
  for (int i = 0; i < C::NJVW; ++i) {
    const int pb = (w + kDqWaves * i) * 1024 + 16 * lane;
    int off;
    if (pb < C::OFF_VS) {
      const int r = pb / DV, c = (pb % DV) / 16;
      off = r * DV + 16 * tile_slot<DV>(r, c);
    } else if (pb < C::OFF_T) {
      off = pb - C::OFF_VS;
    } else if (pb < C::OFF_TS) {
      const int p = pb - C::OFF_T, r = p / CK;              // 1024 / CK channel rows of CK B per load
      off = (lane / (CK / 16)) * Lp + 16 * tile_slot<CK>(r, lane % (CK / 16));
    } else {
      off = lane * LB * 4;                                  // channel 64j + lane, 16 B (4 key blocks)
    }
    vo[i] = off;
  }
  auto issue_k = [&](int cc, int buf) {       // K^<c> chunk cc -> K part buf
#pragma unroll
    for (int i = 0; i < C::NJKW; ++i) {
      const int j = w + kDqWaves * i;
      if (j >= C::NJK) continue;
      const int jb = j * 1024;
      const uint8_t* base = jb < C::K ? Kc + (int64_t)cc * CK * DQK
                                      : reinterpret_cast<const uint8_t*>(Kcs + (int64_t)cc * CK * KB);
      dma16(base + ko[i], lds + buf * C::KPART + jb);
    }
  };
  auto issue_v = [&](int cc, int buf) {       // V^<c>, K^<s> chunk cc -> V part buf
#pragma unroll
    for (int i = 0; i < C::NJVW; ++i) {
      const int j = w + kDqWaves * i;
      if (j >= C::NJV) continue;
      const int jb = j * 1024;
      const uint8_t* base;
      if (jb < C::OFF_VS) base = Vc + (int64_t)cc * CK * DV;
      else if (jb < C::OFF_T) base = reinterpret_cast<const uint8_t*>(Vcs + (int64_t)cc * CK * VB);
      else if (jb < C::OFF_TS) base = Kt + (int64_t)((jb - C::OFF_T) / CK) * Lp + cc * CK;
      else base = reinterpret_cast<const uint8_t*>(Kts + (int64_t)(64 * ((jb - C::OFF_TS) / 1024)) * LB +
                                                   ((cc * (CK / kBlock)) & ~3));
      dma16(base + vo[i], lds + C::OFF_VP + buf * C::VPART + jb);
    }
  };

  v8i qb[KS], db[VS];
  int qsc[KS], dsc[VS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (live) {
      const uint8_t* p = qc + (qhead * Lp + qi) * DQK + 64 * ks;
      qb[ks] = cat(*reinterpret_cast<const v4i*>(p + 16 * h), *reinterpret_cast<const v4i*>(p + 32 + 16 * h));
      qsc[ks] = e8m0(qcs[(qhead * Lp + qi) * KB + 2 * ks + h]);
    } else {
      qb[ks] = v8i{};
      qsc[ks] = 127;
    }
  }
#pragma unroll
  for (int ks = 0; ks < VS; ++ks) {
    if (live) {
      const uint8_t* p = doc + (qhead * Lp + qi) * DV + 64 * ks;
      db[ks] = cat(*reinterpret_cast<const v4i*>(p + 16 * h), *reinterpret_cast<const v4i*>(p + 32 + 16 * h));
      dsc[ks] = e8m0(docs[(qhead * Lp + qi) * VB + 2 * ks + h]);
    } else {
      db[ks] = v8i{};
      dsc[ks] = 127;
    }
  }
  const int kr = pair_row(R);
  int kro[KS][2], vro[VS][2], tro[NST][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) kro[ks][e] = kr * DQK + 16 * tile_slot<DQK>(kr, 4 * ks + 2 * e + h);
#pragma unroll
  for (int ks = 0; ks < VS; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) vro[ks][e] = kr * DV + 16 * tile_slot<DV>(kr, 4 * ks + 2 * e + h);
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int e = 0; e < 2; ++e) tro[st][e] = R * CK + 16 * tile_slot<CK>(R, 4 * st + 2 * e + h);

  const float c2 = sigma * kLog2e;
  const float l2 = (live && qi < L) ? lse[qhead * L + qi] * kLog2e : INFINITY;   // pad rows: P = 0
  const float del = (live && qi < L) ? delta[qhead * L + qi] : 0.f;
  // -delta in every accumulator slot: the dP^ products of the narrow-head instances start
  // from it, so dP^ - delta comes out of the matrix core (one rounding instead of two)
  v16f ndel16;
#pragma unroll
  for (int v = 0; v < 16; ++v) ndel16[v] = -del;
  double rsum = 0.0, rabs = 0.0, rcast = 0.0;   // probes: FP32 per chunk, FP64 across chunks
  v16f acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = v16f{};

  const int kmax = CAUSAL ? min(qi, L - 1) : L - 1;       // last key this lane's query sees
  const int qlast = min(q0 + kDqQ, Lp) - 1;
  const int nchunks = CAUSAL ? (qlast / CK + 1) : Lp / CK;
  const int wlast = CAUSAL ? min(nchunks - 1, (qw + 31) / CK) : nchunks - 1;

  auto score_tile = [&](int buf, int t) -> v16f {
    const uint8_t* bb = lds + buf * C::KPART;
    const float* ksr = reinterpret_cast<const float*>(bb + C::K) + (32 * t + kr) * KB;
    v16f a_ = v16f{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint8_t* p = bb + 32 * t * DQK;
      const v8i a = cat(lds_read16(p + kro[ks][0]), lds_read16(p + kro[ks][1]));
      a_ = mfma<E4M3, E4M3>(a, qb[ks], a_, e8m0(ksr[2 * ks + h]), qsc[ks]);
    }
    return a_;
  };

  // one chunk of work for this wave; MASK instantiates the causal / ragged mask
  auto chunk = [&](int c, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = c * CK;
    const uint8_t* vp = lds + C::OFF_VP + (c & 1) * C::VPART;
    const float* tsp = reinterpret_cast<const float*>(vp + C::OFF_TS);
    const int tb = (c * (CK / kBlock)) & 3;        // the chunk's first block within the staged four
    v8i dsb[NST];
    int dssc[NST] = {};
    float csum = 0.f, cabs = 0.f, ccast = 0.f;
    constexpr bool PIPE = DQK <= 128 && DV <= 128;
    // dP^T tile t of chunk c
    auto dp_tile = [&](int t) -> v16f {
      const float* vsr = reinterpret_cast<const float*>(vp + C::OFF_VS) + (32 * t + kr) * VB;
      v16f dp_ = PIPE ? ndel16 : v16f{};             // PIPE: the product accumulates onto -delta
#pragma unroll
      for (int ks = 0; ks < VS; ++ks) {
        const uint8_t* p = vp + 32 * t * DV;
        const v8i a = cat(lds_read16(p + vro[ks][0]), lds_read16(p + vro[ks][1]));
        dp_ = mfma<E4M3, E5M2>(a, db[ks], dp_, e8m0(vsr[2 * ks + h]), dsc[ks]);
      }
      return dp_;
    };
    // d_qk, d_v <= 128: the next tile's dP^ products go to the matrix core between
    // this tile's S products and its FP32 work, so that work waits less for them (16
    // more registers; wider heads would spill)
    v16f dp_nx = v16f{};
    if constexpr (PIPE) dp_nx = dp_tile(0);
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      v16f dp, sc_;
      if constexpr (PIPE) {
        dp = dp_nx;
        sc_ = score_tile(c & 1, t);
        if (t + 1 < NTL) dp_nx = dp_tile(t + 1);
      } else {
        dp = dp_tile(t);
        sc_ = score_tile(c & 1, t);
      }
      if constexpr (MASK) {
        // key k0 + 32t + 16h + v is visible iff it is <= kmax, i.e. iff v <= lim
        const int lim = kmax - (k0 + 32 * t + 16 * h);
#pragma unroll
        for (int v = 0; v < 16; ++v) sc_[v] = v > lim ? -INFINITY : sc_[v];
      }
      float am = 0.f;
      v16f d;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc_[v], c2, -l2));
        d[v] = PIPE ? p * dp[v] : p * (dp[v] - del);
        if constexpr (PROBE) {
          csum += d[v];
          cabs += fabsf(p * (PIPE ? dp[v] + del : dp[v]));   // PIPE: dp holds dP^ - delta
        }
        am = fmaxf(am, fabsf(d[v]));
      }
      am = pair_max(am);
      const int k = scale_exp<E5M2>(am);
      const float sc = exp2i(k);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        dsb[t >> 1][4 * (t & 1) + g] = (int)pack4s<E5M2>(d[4 * g], d[4 * g + 1], d[4 * g + 2], d[4 * g + 3], sc);
      if ((t & 1) == h) dssc[t >> 1] = k + 127;
      if constexpr (PROBE) {
        // the row's sum after the cast: the decoded E5M2 codes of this tile times its scale
        float cs = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int code = dsb[t >> 1][4 * (t & 1) + g];
          cs += __builtin_amdgcn_cvt_f32_bf8(code, 0) + __builtin_amdgcn_cvt_f32_bf8(code, 1) +
                __builtin_amdgcn_cvt_f32_bf8(code, 2) + __builtin_amdgcn_cvt_f32_bf8(code, 3);
        }
        ccast += cs * sc;
      }
      if (t & 1) {
        // dS^<k> of key half st complete: dQ^T += K^<s>^T dS^<k>^T over those 64 keys
        const int st = t >> 1;
        // raised wave priority while this wave issues its dQ products, so they reach the
        // matrix core ahead of the other wave's FP32 work (about 1% at 8K; same arithmetic)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const uint8_t* p = vp + C::OFF_T + 32 * ct * CK;
          const v8i a = cat(lds_read16(p + tro[st][0]), lds_read16(p + tro[st][1]));
          const v4f x = *reinterpret_cast<const v4f*>(tsp + (32 * ct + R) * 4);   // 4 key blocks of the channel
          float xs;
          if constexpr (CK == 128) xs = h ? x[2 * st + 1] : x[2 * st];
          else xs = x[tb + h];
          acc[ct] = mfma<E4M3, E5M2>(a, dsb[st], acc[ct], e8m0(xs), dssc[st]);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      __builtin_amdgcn_sched_barrier(0);        // one key tile in flight at a time (register budget)
    }
    if constexpr (PROBE) {
      rsum += (double)csum;
      rabs += (double)cabs;
      rcast += (double)ccast;
    }
  };
  auto sync_and_issue = [&](int c) {
    wait_vmem();
    __syncthreads();                             // chunk c landed; the other buffers are free
    if (c + 1 < nchunks) {
      issue_k(c + 1, (c + 1) & 1);
      issue_v(c + 1, (c + 1) & 1);
    }
  };

  // Chunks before nfull need no mask for any wave of the workgroup (all their keys
  // precede every query of the tile and lie below L); the rest take the masked body.
  // Two loops keep the mask code out of the main loop's register allocation.
  const int nfull = min(CAUSAL ? q0 / CK : nchunks, L / CK);
  issue_k(0, 0);
  issue_v(0, 0);
  int c = 0;
  for (; c < nfull; ++c) {
    sync_and_issue(c);
    if (live) chunk(c, std::false_type{});
  }
  for (; c < nchunks; ++c) {
    sync_and_issue(c);
    if (live && c <= wlast) chunk(c, std::true_type{});
  }

  if (!live) return;
  if constexpr (PROBE) {
    rsum = pair_sum_d(rsum);
    rabs = pair_sum_d(rabs);
    rcast = pair_sum_d(rcast);
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
        if (pcast) pcast[qhead * L + qi] = rcast;
      }
    }
  }
}

template <int DQK, int DV, bool CAUSAL, bool PROBE>
static void launch_dq_t4(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                         const float* lse, const float* delta, float* dq, double* ps, double* pa, double* pc,
                         hipStream_t s) {
  constexpr int kDqQ = 32 * dq_waves<DQK, DV>();
  dim3 grid((unsigned)((d.Lp + kDqQ - 1) / kDqQ) * d.Hq * d.B);
  hipLaunchKernelGGL((dq_kernel<DQK, DV, CAUSAL, PROBE>), grid, dim3(2 * kDqQ), 0, s, qc.codes, qc.scales, kc.codes,
                     kc.scales, vc.codes, vc.scales, ks.codes, ks.scales, doc.codes, doc.scales, lse, delta, dq, ps,
                     pa, pc, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
}

template <int DQK, int DV>
static void launch_dq_t(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                        const float* lse, const float* delta, float* dq, double* ps, double* pa, double* pc,
                         hipStream_t s) {
  if (d.causal) {
    if (ps) launch_dq_t4<DQK, DV, true, true>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
    else launch_dq_t4<DQK, DV, true, false>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  } else {
    if (ps) launch_dq_t4<DQK, DV, false, true>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
    else launch_dq_t4<DQK, DV, false, false>(d, qc, kc, ks, vc, doc, lse, delta, dq, ps, pa, pc, s);
  }
}

// dQ launcher for d_qk = 192, d_v = 128, compiled in its own translation unit
// (attn_dq_wide.hip) with the compiler's default MFMA register form.
hipError_t launch_dq_192_128(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                             const float* lse, const float* delta, float* dq, double* ps, double* pa, double* pc,
                             hipStream_t s);
// ... and for d_qk = d_v = 256 (one wave per SIMD: accumulators in AGPRs)
hipError_t launch_dq_256_256(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                             const float* lse, const float* delta, float* dq, double* ps, double* pa, double* pc,
                             hipStream_t s);

}  // namespace dm
