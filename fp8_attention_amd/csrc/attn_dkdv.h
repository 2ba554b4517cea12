// dK and dV of block-scaled FP8 attention (key-stationary).
//
// Workgroup = 8 waves over 128 keys (4 waves over 64 keys when d = 256, one per
// SIMD): key group kg = w % 4 owns keys
// k0+32kg .. k0+32kg+31, and the two waves of a key group split the outputs --
// role 0 accumulates dV, role 1 accumulates dK -- so each wave carries one set
// of accumulators and two waves share every SIMD.  A 1-D grid over (key tile,
// Hkv, B) with key tiles slowest starts the long causal tiles first.  The
// workgroup walks the query heads of its KV group and, for each, the 64-query
// steps that can see its keys.  Per step, for two 32-query tiles:
//   dV waves: S^T = Q K^T, P = exp(S - LSE), P^<q> (E4M3, 32-query blocks);
//   dK waves: S^T, dP^T = dO V^T, dS = P (dP^ - delta), dS^<q> (E5M2);
// (one key per lane pair, 16 queries per lane), and the two tiles' codes side by
// side are exactly the B operands of dV^T += dO^<s>^T P^<q> and
// dK^T += Q^<s>^T dS^<q> over the step's 64 queries -- nothing passes between
// waves.  S is recomputed by both waves of a key group: 25% more matrix work
// for half the accumulator registers.
// K^<c>/V^<c> of the workgroup's keys sit in LDS for the whole kernel; the
// query-side tiles of step i+1 (Q^<c>, dO^<c> rows, Q^<s>, dO^<s> channel rows,
// their scales) arrive in a second LDS buffer by direct global->LDS loads issued
// during step i, with LSE and delta through registers; one barrier per step.  dK
// and dV accumulate in registers over every query head of the group and are
// written once (no atomics).  dQ is computed by the query-stationary kernel in
// attn_dq.h.
//
// The PROBE instance runs the same arithmetic and its dK waves also return, per
// query row, the sum over keys of the FP32 dS they cast and of |P dP^| (the
// zero-row-sum property of matched delta, section 03 of the Delta-Matching
// project page), reduced across the wave's 32 keys and added to the caller's FP64
// rows atomically.
#pragma once
#include <type_traits>

#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

constexpr int kBQ = 64;          // queries per step

template <int DQK, int DV>
struct DkdvCfg {
  // key groups of 32 keys: 4 (two waves per SIMD); 2 when d_qk = d_v = 256, whose
  // 256-channel accumulators and K/V operand rows take a whole register file
  static constexpr int NKG = DQK + DV > 384 ? 2 : 4;
  static constexpr int NW = 2 * NKG;                     // a dV wave and a dK wave per key group
  static constexpr int NT = 64 * NW;
  static constexpr int KT = 32 * NKG;                    // keys per workgroup
  static constexpr int KB = DQK / 32, VB = DV / 32;
  static constexpr int pad1k(int x) { return (x + 1023) / 1024 * 1024; }
  // resident K/V tile
  static constexpr int K_OFF = 0, V_OFF = KT * DQK, KS_OFF = V_OFF + KT * DV, VS_OFF = KS_OFF + KT * KB * 4;
  static constexpr int KV_BYTES = VS_OFF + KT * VB * 4;
  // one step's query-side stage (regions padded to whole 1 KB direct loads)
  static constexpr int QC = 0;                                   // Q^<c> rows [64][DQK], swizzled
  static constexpr int DOC = QC + pad1k(kBQ * DQK);             // dO^<c> rows [64][DV]
  static constexpr int QS = DOC + pad1k(kBQ * DV);              // Q^<s> channel rows [DQK][64]
  static constexpr int DOS = QS + pad1k(DQK * kBQ);             // dO^<s> [DV][64]
  static constexpr int QCS = DOS + pad1k(DV * kBQ);             // Q^<c> scales [64][KB], query lane order
  static constexpr int DOCS = QCS + pad1k(kBQ * KB * 4);        // dO^<c> scales [64][VB], lane order
  static constexpr int NDMA = (DOCS + pad1k(kBQ * VB * 4)) / 1024;   // direct loads per step
  static constexpr int QSS = NDMA * 1024;                        // Q^<s> scales [DQK][2]   (register path)
  static constexpr int DOSS = QSS + DQK * 2 * 4;                 // dO^<s> scales [DV][2]
  static constexpr int LSE = DOSS + DV * 2 * 4;                  // LSE * log2(e) [64]
  static constexpr int DEL = LSE + kBQ * 4;                      // delta [64]
  static constexpr int STAGE = pad1k(DEL + kBQ * 4);
  static constexpr int NSMALL = DQK * 2 + DV * 2 + 2 * kBQ;      // floats through registers per step
  static constexpr int NSR = (NSMALL + NT - 1) / NT;
  static constexpr int NDW = (NDMA + NW - 1) / NW;               // direct loads per wave
  // The resident tile is read only once, into registers, before the first step; when
  // it and two stages do not fit side by side the stages reuse its space.
  static constexpr bool ALIAS = KV_BYTES + 2 * STAGE > 160 * 1024;
  static constexpr int STAGE_OFF = ALIAS ? 0 : KV_BYTES;
  static constexpr int BYTES = ALIAS ? (KV_BYTES > 2 * STAGE ? KV_BYTES : 2 * STAGE) : KV_BYTES + 2 * STAGE;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int DQK, int DV, bool CAUSAL, bool PROBE>
__global__ __launch_bounds__((DkdvCfg<DQK, DV>::NT)) void dkdv_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ qs,
    const float* __restrict__ qss, const uint8_t* __restrict__ kc, const float* __restrict__ kcs,
    const uint8_t* __restrict__ vc, const float* __restrict__ vcs, const uint8_t* __restrict__ doc,
    const float* __restrict__ docs, const uint8_t* __restrict__ dos, const float* __restrict__ doss,
    const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv,
    double* __restrict__ psum, double* __restrict__ pabs, int Hq, int Hkv, int L, int Lp, float sigma) {
  using C = DkdvCfg<DQK, DV>;
  constexpr int NW = C::NW, NT = C::NT, KT = C::KT, KB = C::KB, VB = C::VB;
  constexpr int KS = DQK / 64, VS = DV / 64, NKT = DQK / 32, NVT = DV / 32;
  constexpr int NACC = NKT > NVT ? NKT : NVT;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::BYTES];
  uint8_t* const stage0 = lds + C::STAGE_OFF;
  // LDS byte address of the array: direct-load targets are formed as this plus an
  // offset (converting the stage pointers themselves trips the compiler when the
  // d = 256 instance inlines the issue code)
  const uint32_t lds_addr0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int R = lane & 31, h = lane >> 5;
  const int nkt = (Lp + KT - 1) / KT;
  const int nhb = Hkv * (int)(gridDim.x / (nkt * Hkv));    // Hkv * B
  const int hk = (int)blockIdx.x % nhb % Hkv, b = (int)blockIdx.x % nhb / Hkv;
  const int k0 = ((int)blockIdx.x / nhb) * KT;            // key tiles slowest: long causal tiles first
  const int G = Hq / Hkv;
  const int kg = w & (C::NKG - 1), role = w / C::NKG;   // role 0: dV, role 1: dK
  const int kw0 = k0 + 32 * kg;                      // this wave's first key
  const int key = kw0 + R;                           // this lane's key (column of the S^T tiles)
  const int LB = Lp / kBlock;
  const int64_t khead = (int64_t)b * Hkv + hk;

  // ---- resident K^<c>, V^<c> rows of the workgroup's keys (rows past Lp are zero)
  for (int i = tid; i < KT * DQK / 16; i += NT) {
    const int r = (i * 16) / DQK, c = ((i * 16) % DQK) / 16;
    v4i x = v4i{};
    if (k0 + r < Lp) x = *reinterpret_cast<const v4i*>(kc + (khead * Lp + k0 + r) * DQK + 16 * c);
    *reinterpret_cast<v4i*>(lds + C::K_OFF + r * DQK + 16 * tile_slot<DQK>(r, c)) = x;
  }
  for (int i = tid; i < KT * DV / 16; i += NT) {
    const int r = (i * 16) / DV, c = ((i * 16) % DV) / 16;
    v4i x = v4i{};
    if (k0 + r < Lp) x = *reinterpret_cast<const v4i*>(vc + (khead * Lp + k0 + r) * DV + 16 * c);
    *reinterpret_cast<v4i*>(lds + C::V_OFF + r * DV + 16 * tile_slot<DV>(r, c)) = x;
  }
  for (int i = tid; i < KT * KB; i += NT)
    reinterpret_cast<float*>(lds + C::KS_OFF)[i] = (k0 + i / KB < Lp) ? kcs[(khead * Lp + k0) * KB + i] : 1.f;
  for (int i = tid; i < KT * VB; i += NT)
    reinterpret_cast<float*>(lds + C::VS_OFF)[i] = (k0 + i / VB < Lp) ? vcs[(khead * Lp + k0) * VB + i] : 1.f;

  // ---- per-lane source offsets of this wave's direct loads (loop invariant)
  int doff[C::NDW];
#pragma unroll
  for (int i = 0; i < C::NDW; ++i) {
    const int j = w + NW * i;
    const int pb = j * 1024 + 16 * lane;             // stage byte this lane fills
    int off = 0;
    if (pb < C::DOC) {
      const int p = pb - C::QC, r = p / DQK, c = (p % DQK) / 16;
      off = r < kBQ ? r * DQK + 16 * tile_slot<DQK>(r, c) : -1;
    } else if (pb < C::QS) {
      const int p = pb - C::DOC, r = p / DV, c = (p % DV) / 16;
      off = r < kBQ ? r * DV + 16 * tile_slot<DV>(r, c) : -1;
    } else if (pb < C::DOS) {
      const int p = pb - C::QS, r = p / 64, c = (p % 64) / 16;   // r: channel within the instruction's 16
      off = r < DQK ? (r % 16) * Lp + 16 * tile_slot<64>(r, c) : -1;
    } else if (pb < C::QCS) {
      const int p = pb - C::DOS, r = p / 64, c = (p % 64) / 16;
      off = r < DV ? (r % 16) * Lp + 16 * tile_slot<64>(r, c) : -1;
    } else if (pb < C::DOCS) {
      const int p = pb - C::QCS, pos = p / (4 * KB), within = p % (4 * KB);
      off = pos < kBQ ? ((pos & ~31) + pair_row(pos & 31)) * 4 * KB + within : -1;
    } else {
      const int p = pb - C::DOCS, pos = p / (4 * VB), within = p % (4 * VB);
      off = pos < kBQ ? ((pos & ~31) + pair_row(pos & 31)) * 4 * VB + within : -1;
    }
    doff[i] = off;
  }
  // issue the direct loads of step (qhead, q0) into stage buffer st
  auto issue_stage = [&](int64_t qhead, int q0, uint8_t* st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::NDW; ++i) {
      const int j = w + NW * i;
      if (j >= C::NDMA) continue;
      const int jb = j * 1024;
      const uint8_t* base;
      if (jb < C::DOC) base = qc + (qhead * Lp + q0) * DQK;
      else if (jb < C::QS) base = doc + (qhead * Lp + q0) * DV;
      else if (jb < C::DOS) base = qs + (qhead * DQK + (jb - C::QS) / 64) * (int64_t)Lp + q0;
      else if (jb < C::QCS) base = dos + (qhead * DV + (jb - C::DOS) / 64) * (int64_t)Lp + q0;
      else if (jb < C::DOCS) base = reinterpret_cast<const uint8_t*>(qcs + (qhead * Lp + q0) * KB);
      else base = reinterpret_cast<const uint8_t*>(docs + (qhead * Lp + q0) * VB);
      if (doff[i] >= 0) {
        if constexpr (C::ALIAS) dma16_at(base + doff[i], lds_addr0 + (uint32_t)(st - lds) + jb);
        else dma16(base + doff[i], st + jb);
      }
    }
  };
  // the step's small items (Q^<s>, dO^<s> scales of its two query blocks, LSE, delta) via registers
  float smallv[C::NSR];
  auto load_small = [&](int64_t qhead, int q0) {
#pragma unroll
    for (int i = 0; i < C::NSR; ++i) {
      const int e = tid + NT * i;
      float x = 0.f;
      if (e < DQK * 2) {
        x = qss[(qhead * DQK + e / 2) * LB + q0 / kBlock + (e & 1)];
      } else if (e < DQK * 2 + DV * 2) {
        const int f = e - DQK * 2;
        x = doss[(qhead * DV + f / 2) * LB + q0 / kBlock + (f & 1)];
      } else if (e < DQK * 2 + DV * 2 + kBQ) {
        const int q = q0 + e - DQK * 2 - DV * 2;
        x = q < L ? lse[qhead * L + q] * kLog2e : INFINITY;    // padded queries: P = 0
      } else if (e < C::NSMALL) {
        const int q = q0 + e - DQK * 2 - DV * 2 - kBQ;
        x = q < L ? -delta[qhead * L + q] : 0.f;            // negated: the dP^ products start from it
      }
      smallv[i] = x;
    }
  };
  auto store_small = [&](uint8_t* st) {
#pragma unroll
    for (int i = 0; i < C::NSR; ++i) {
      const int e = tid + NT * i;
      if (e < C::NSMALL) reinterpret_cast<float*>(st + C::QSS)[e] = smallv[i];
    }
  };

  // The two roles run role-specialised copies of the step loop (wave-uniform choice), so
  // neither carries the other's code; both execute the same barriers.
  auto run = [&](auto role_tag) {
  constexpr bool DK = decltype(role_tag)::value;
  v16f acc[NACC];                                    // dV^T (role 0) or dK^T (role 1) channel tiles
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = v16f{};

  const float c2 = sigma * kLog2e;
  const int qstart = CAUSAL ? k0 : 0;
  const int nsteps = qstart < Lp ? (Lp - qstart) / kBQ : 0;
  const int total = G * nsteps;
  const int64_t qhead0 = (int64_t)b * Hq + (int64_t)hk * G;
  const int prow = pair_row(R);
  // LDS read offsets of this lane.  Each tile map depends only on row bits that a
  // 32-row (or 32-channel) step leaves unchanged, so tiles j / channel tiles ct
  // are plain immediate offsets from these.
  int oq[KS][2], od[VS][2], ok[KS][2], ov[VS][2], ot[2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      oq[ks][e] = prow * DQK + 16 * tile_slot<DQK>(prow, 4 * ks + 2 * e + h);
      ok[ks][e] = (32 * kg + R) * DQK + 16 * tile_slot<DQK>(R, 4 * ks + 2 * e + h);
    }
#pragma unroll
  for (int ks = 0; ks < VS; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      od[ks][e] = prow * DV + 16 * tile_slot<DV>(prow, 4 * ks + 2 * e + h);
      ov[ks][e] = (32 * kg + R) * DV + 16 * tile_slot<DV>(R, 4 * ks + 2 * e + h);
    }
#pragma unroll
  for (int e = 0; e < 2; ++e) ot[e] = R * kBQ + 16 * tile_slot<64>(R, 2 * e + h);

  if constexpr (!C::ALIAS) {
    if (total > 0) {
      issue_stage(qhead0, qstart, stage0);
      load_small(qhead0, qstart);
      store_small(stage0);
    }
  }
  // this wave's K^<c> (and for dK, V^<c>) rows as register-resident B operands
  // (lane R = key, K-slots = channels), read once after the resident tile is written
  __syncthreads();
  v8i kb[KS], vb[VS];
  int ksc[KS], vsc[VS];
  {
    const float* ksr = reinterpret_cast<const float*>(lds + C::KS_OFF) + (32 * kg + R) * KB;
    const float* vsr = reinterpret_cast<const float*>(lds + C::VS_OFF) + (32 * kg + R) * VB;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kb[ks] = cat(lds_read16(lds + C::K_OFF + ok[ks][0]), lds_read16(lds + C::K_OFF + ok[ks][1]));
      ksc[ks] = e8m0(ksr[2 * ks + h]);
    }
#pragma unroll
    for (int ks = 0; ks < VS; ++ks) {
      if constexpr (DK) {
        vb[ks] = cat(lds_read16(lds + C::V_OFF + ov[ks][0]), lds_read16(lds + C::V_OFF + ov[ks][1]));
        vsc[ks] = e8m0(vsr[2 * ks + h]);
      } else {
        vb[ks] = v8i{};
        vsc[ks] = 127;
      }
    }
  }
  if constexpr (C::ALIAS) {
    __syncthreads();                                 // every wave holds its rows: the tile's space is free
    if (total > 0) {
      issue_stage(qhead0, qstart, stage0);
      load_small(qhead0, qstart);
      store_small(stage0);
    }
  }
  // one step; MASK instantiates the causal / padded-key mask (kept out of the main loop)
  auto step = [&](int it, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int hh = it / nsteps;
    const int q0 = qstart + (it - hh * nsteps) * kBQ;
    uint8_t* const st = stage0 + (it & 1) * C::STAGE;
    uint8_t* const stn = stage0 + ((it + 1) & 1) * C::STAGE;
    wait_vmem();
    __syncthreads();                               // step it staged; buffer (it+1)&1 free
    const bool more = it + 1 < total;
    if (more) {
      const int hn = (it + 1) / nsteps;
      const int qn = qstart + (it + 1 - hn * nsteps) * kBQ;
      issue_stage(qhead0 + hn, qn, stn);
      load_small(qhead0 + hn, qn);
    }

    if (kw0 < L && (!CAUSAL || q0 + kBQ - 1 >= kw0)) {
      const bool need_mask = MASK && ((kw0 + 32 > L) || (CAUSAL && q0 < kw0 + 31));
      v4i code[2];
      int scl[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // S^T (and dP^T) for queries 32j .. 32j+31 of the step (rows in pair_row order)
        const uint8_t* qt = st + C::QC + 32 * j * DQK;
        const float* qsr = reinterpret_cast<const float*>(st + C::QCS) + (32 * j + R) * KB;
        v16f s = v16f{}, dp = v16f{};
        // lane (key R, h), register v <-> step query 32j + 16h + v
        const float* l2p = reinterpret_cast<const float*>(st + C::LSE) + 32 * j + 16 * h;
        const float* ndlp = reinterpret_cast<const float*>(st + C::DEL) + 32 * j + 16 * h;   // -delta
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const v8i a = cat(lds_read16(qt + oq[ks][0]), lds_read16(qt + oq[ks][1]));
          s = mfma<E4M3, E4M3>(a, kb[ks], s, e8m0(qsr[2 * ks + h]), ksc[ks]);
        }
        if constexpr (DK) {
          const uint8_t* dt = st + C::DOC + 32 * j * DV;
          const float* dsr = reinterpret_cast<const float*>(st + C::DOCS) + (32 * j + R) * VB;
          // dP^ - delta comes out of the products (not for d_qk = 192: no registers to spare)
          if constexpr (DQK != 192) {
#pragma unroll
            for (int v = 0; v < 16; ++v) dp[v] = ndlp[v];
          }
#pragma unroll
          for (int ks = 0; ks < VS; ++ks) {
            const v8i a = cat(lds_read16(dt + od[ks][0]), lds_read16(dt + od[ks][1]));
            dp = mfma<E5M2, E4M3>(a, vb[ks], dp, e8m0(dsr[2 * ks + h]), vsc[ks]);
          }
        }
        if (need_mask) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int q = q0 + 32 * j + 16 * h + v;
            if (key >= L || (CAUSAL && key > q)) s[v] = -INFINITY;
          }
        }
        float am = 0.f;
        if constexpr (!DK) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v4f l4 = *reinterpret_cast<const v4f*>(l2p + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p = __builtin_amdgcn_exp2f(fmaf(s[4 * g + e], c2, -l4[e]));
              s[4 * g + e] = p;                     // s now holds P
              am = fmaxf(am, p);
            }
          }
          am = pair_max(am);
          const int k = scale_exp<E4M3>(am);
          const float sc = exp2i(k);
#pragma unroll
          for (int g = 0; g < 4; ++g) code[j][g] = (int)pack4s<E4M3>(s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3], sc);
          scl[j] = k + 127;
        } else {
          float av[PROBE ? 16 : 1];                 // probe: |P dP^|
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v4f l4 = *reinterpret_cast<const v4f*>(l2p + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 4 * g + e;
              const float p = __builtin_amdgcn_exp2f(fmaf(s[v], c2, -l4[e]));
              const float d = DQK != 192 ? p * dp[v] : p * (dp[v] + ndlp[v]);
              if constexpr (PROBE) av[v] = fabsf(p * (DQK != 192 ? dp[v] - ndlp[v] : dp[v]));
              dp[v] = d;                            // dp now holds dS
              am = fmaxf(am, fabsf(d));
            }
          }
          if constexpr (PROBE) {
            // sums over the wave's 32 keys (lanes R of half h); lane R < 16 then holds those
            // of query 32j + 16h + R of the step
            float rs[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) rs[v] = dp[v];
            const float r = group_sum_scatter<16, 32>(rs, lane);
            const float a = group_sum_scatter<16, 32>(av, lane);
            const int q = q0 + 32 * j + 16 * h + R;
            if (R < 16 && q < L) {
              const int64_t row = (qhead0 + hh) * L + q;
              unsafeAtomicAdd(psum + row, (double)r);
              unsafeAtomicAdd(pabs + row, (double)a);
            }
          }
          am = pair_max(am);
          const int k = scale_exp<E5M2>(am);
          const float sc = exp2i(k);
#pragma unroll
          for (int g = 0; g < 4; ++g)
            code[j][g] = (int)pack4s<E5M2>(dp[4 * g], dp[4 * g + 1], dp[4 * g + 2], dp[4 * g + 3], sc);
          scl[j] = k + 127;
        }
      }

      // dV^T += dO^<s>^T P^<q> (role 0) or dK^T += Q^<s>^T dS^<q> (role 1) over the step's 64
      // queries.  B operand: lane (key R, h) holds queries 16h.. of tile 0 and of tile 1.
      const v8i bq = cat(code[0], code[1]);
      const int bsc = h ? scl[1] : scl[0];
      if constexpr (!DK) {
        const float* dossr = reinterpret_cast<const float*>(st + C::DOSS);
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
          const int ch = 32 * ct + R;
          const uint8_t* p = st + C::DOS + 32 * ct * kBQ;
          const v8i a = cat(lds_read16(p + ot[0]), lds_read16(p + ot[1]));
          acc[ct] = mfma<E5M2, E4M3>(a, bq, acc[ct], e8m0(dossr[2 * ch + h]), bsc);
        }
      } else {
        const float* qssr = reinterpret_cast<const float*>(st + C::QSS);
#pragma unroll
        for (int ct = 0; ct < NKT; ++ct) {
          const int ch = 32 * ct + R;
          const uint8_t* p = st + C::QS + 32 * ct * kBQ;
          const v8i a = cat(lds_read16(p + ot[0]), lds_read16(p + ot[1]));
          acc[ct] = mfma<E4M3, E5M2>(a, bq, acc[ct], e8m0(qssr[2 * ch + h]), bsc);
        }
      }
    }
    if (more) store_small(stn);
  };
  // per head: the steps that can need a mask (the first KT/kBQ for causal, all when the
  // tile holds padded keys), then the rest in a loop without mask code
  const int nmask = (k0 + KT > L) ? nsteps : (CAUSAL ? min(nsteps, KT / kBQ) : 0);
  for (int hh = 0, it = 0; hh < G; ++hh) {
    for (int i = 0; i < nmask; ++i, ++it) step(it, std::true_type{});
    for (int i = nmask; i < nsteps; ++i, ++it) step(it, std::false_type{});
  }

  // ---- dK, dV written once per key: register v of channel tile ct <-> channel 32ct + 8(v/4) + 4h + v%4
  if (key < L) {
    if constexpr (DK) {
      float* dkr = dk + (khead * L + key) * DQK + 4 * h;
#pragma unroll
      for (int ct = 0; ct < NKT; ++ct)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          v4f r = {sigma * acc[ct][4 * a], sigma * acc[ct][4 * a + 1], sigma * acc[ct][4 * a + 2],
                   sigma * acc[ct][4 * a + 3]};
          *reinterpret_cast<v4f*>(dkr + 32 * ct + 8 * a) = r;
        }
    } else {
      float* dvr = dv + (khead * L + key) * DV + 4 * h;
#pragma unroll
      for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          v4f r = {acc[ct][4 * a], acc[ct][4 * a + 1], acc[ct][4 * a + 2], acc[ct][4 * a + 3]};
          *reinterpret_cast<v4f*>(dvr + 32 * ct + 8 * a) = r;
        }
    }
  }
  };
  if (role) run(std::true_type{});
  else run(std::false_type{});
}

template <int DQK, int DV>
inline hipError_t launch_dkdv_t(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc,
                                Operand dos, const float* lse, const float* delta, float* dk, float* dv, double* ps,
                                double* pa, hipStream_t s) {
  using C = DkdvCfg<DQK, DV>;
  if ((ps == nullptr) != (pa == nullptr)) return hipErrorInvalidValue;
  dim3 grid((unsigned)((d.Lp + C::KT - 1) / C::KT) * d.Hkv * d.B);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(C::NT), 0, s, qc.codes, qc.scales, qs.codes, qs.scales, kc.codes, kc.scales,
                       vc.codes, vc.scales, doc.codes, doc.scales, dos.codes, dos.scales, lse, delta, dk, dv, ps, pa,
                       d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
  };
  if (ps) {
    // the probe rows are sums over every key tile: start them from zero
    const int64_t bytes = (int64_t)d.B * d.Hq * d.L * (int64_t)sizeof(double);
    hipError_t e = launch_fill_zero(ps, bytes, s);
    if (e == hipSuccess) e = launch_fill_zero(pa, bytes, s);
    if (e != hipSuccess) return e;
    if (d.causal) go(dkdv_kernel<DQK, DV, true, true>);
    else go(dkdv_kernel<DQK, DV, false, true>);
  } else {
    if (d.causal) go(dkdv_kernel<DQK, DV, true, false>);
    else go(dkdv_kernel<DQK, DV, false, false>);
  }
  return hipGetLastError();
}

}  // namespace dm
