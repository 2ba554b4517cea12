// Forward of block-scaled FP8 attention on gfx950 matrix cores.
//
// Workgroup = 8 waves = 256 queries (32 per wave, 2 waves per SIMD; 4 waves, one
// per SIMD, when d_v = 256); a 1-D grid
// over (query tile of 256, Hq, B) with the query tile slowest, so the longest
// causal tiles are dispatched first.  Each wave keeps its queries' Q^<c> codes in
// registers as the B operand of S^T = K Q^T, so the score tile comes out with
// one query per lane pair (R, R+32) and 16 keys per lane -- exactly the
// B-operand layout the P V product needs, so the probabilities are cast to E4M3
// in registers and fed to the next instruction without any lane exchange.
//
// Per 128-key chunk c:
//   mu  = max(mu, chunk row max)   (exact running max, once per chunk);
//   P'  = exp2(S*sigma*log2e - mu*sigma*log2e); l += sum P' (FP32 per chunk,
//         FP64 across chunks);
//   P'^ = E4M3 cast per 32-key block; the block amax is exp2 of the block's raw
//         score max (exp2 is monotone and computed by the same instructions);
//   O^T = O^T * exp(mu_old - mu) (skipped when no row maximum moved) + V^T P'^^T.
// Epilogue: O = O^T / l, LSE = sigma*mu + ln l.
//
// Software pipeline: the scores of chunk c+1 are computed while chunk c's
// softmax runs -- as soon as a 32-key tile of chunk c has been exponentiated and
// cast, its registers receive that tile of chunk c+1 from the matrix cores -- and
// the P V product of chunk c overlaps the row maxima of chunk c+1.  K^<c> chunks
// (double-buffered) and V^<s> chunks (double-buffered) reach LDS through direct
// global->LDS loads issued a full iteration before use; one barrier per chunk.
#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

// waves per workgroup (32 queries each): two per SIMD; with d_v = 256 the O^T
// accumulators alone fill half the register file, so one per SIMD
template <int DQK, int DV> constexpr int fwd_waves() { return DV > 128 ? 4 : 8; }

template <int DQK, int DV>
struct FwdLds {
  static constexpr int NW = fwd_waves<DQK, DV>();
  static constexpr int KB = DQK / 32;
  static constexpr int K = kChunk * DQK;               // one K^<c> chunk, rows swizzled
  static constexpr int V = DV * kChunk;                // one V^<s> chunk (channel rows), swizzled
  static constexpr int KS = kChunk * KB * 4;           // K scales of a chunk
  static constexpr int VS = DV * 4 * 4;                // V scales of a chunk (4 key blocks per channel)
  static constexpr int OFF_V = 2 * K, OFF_KS = OFF_V + 2 * V, OFF_VS = OFF_KS + 2 * KS;
  static constexpr int BYTES = OFF_VS + 2 * VS;
  // direct-load instructions (1 KB each) per chunk and region
  static constexpr int NK = K / 1024, NV = V / 1024, NKS = KS / 1024, NVS = VS / 1024;
  static constexpr int NKW = (NK + NW - 1) / NW, NVW = (NV + NW - 1) / NW;
  static_assert(K % 1024 == 0 && V % 1024 == 0 && KS % 1024 == 0 && VS % 1024 == 0, "whole 1 KB loads");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__((64 * fwd_waves<DQK, DV>())) void fwd_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ kc,
    const float* __restrict__ kcs, const uint8_t* __restrict__ vs, const float* __restrict__ vss,
    float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int L, int Lp, float sigma) {
  using C = FwdLds<DQK, DV>;
  constexpr int kFwdWaves = C::NW, kFwdQ = 32 * kFwdWaves;
  constexpr int KS = DQK / 64;      // 64-channel steps of QK^T
  constexpr int NCT = DV / 32;      // 32-channel tiles of O^T
  constexpr int KB = DQK / 32;      // channel blocks per K row
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int R = lane & 31, h = lane >> 5;
  const int nqt = (Lp + kFwdQ - 1) / kFwdQ;
  const QueryItem item = query_item((int)blockIdx.x, nqt, Hq, Hkv, (int)gridDim.x / (nqt * Hq));
  const int qt = CAUSAL ? (nqt - 1 - item.tr) : item.tr;  // longest causal tiles first
  const int hq = item.hq, b = item.b;
  const int hk = hq / (Hq / Hkv);
  const int q0 = qt * kFwdQ;
  const int qw = q0 + 32 * w;                 // first query of this wave
  const bool live = qw < Lp;                  // waves past the padded length only help load
  const int qi = qw + R;

  const int64_t qhead = (int64_t)b * Hq + hq, khead = (int64_t)b * Hkv + hk;
  const uint8_t* Kc = kc + khead * Lp * DQK;
  const float* Kcs = kcs + khead * Lp * KB;
  const uint8_t* Vs = vs + khead * DV * Lp;
  const float* Vss = vss + khead * DV * (Lp / kBlock);

  // ---- direct-load source offsets of this lane (loop invariant) ----
  int koff[C::NKW], voff[C::NVW];
#pragma unroll
  for (int i = 0; i < C::NKW; ++i) {
    const int p = (w + kFwdWaves * i) * 1024 + 16 * lane;
    const int r = p / DQK, slot = (p % DQK) / 16;
    koff[i] = r * DQK + 16 * tile_slot<DQK>(r, slot);
  }
#pragma unroll
  for (int i = 0; i < C::NVW; ++i) {
    const int r = 8 * (w + kFwdWaves * i) + (lane >> 3);   // 8 channel rows of 128 B per load
    voff[i] = (lane >> 3) * Lp + 16 * tile_slot<kChunk>(r, lane & 7);
  }
  auto issue_k = [&](int cc, int buf) {       // K^<c> chunk cc (codes + scales) -> K buffer buf
    const uint8_t* src = Kc + (int64_t)cc * kChunk * DQK;
#pragma unroll
    for (int i = 0; i < C::NKW; ++i) {
      const int j = w + kFwdWaves * i;
      if (j < C::NK) dma16(src + koff[i], lds + buf * C::K + j * 1024);
    }
    if constexpr (C::NKS + C::NVS <= kFwdWaves) {  // one scale load per wave
      if (w < C::NKS)
        dma16(reinterpret_cast<const uint8_t*>(Kcs + (int64_t)cc * kChunk * KB) + w * 1024 + 16 * lane,
              lds + C::OFF_KS + buf * C::KS + w * 1024);
    } else {                                     // scale load j of the chunk on wave j % NW
#pragma unroll
      for (int j = 0; j < C::NKS; ++j)
        if (j % kFwdWaves == w)
          dma16(reinterpret_cast<const uint8_t*>(Kcs + (int64_t)cc * kChunk * KB) + j * 1024 + 16 * lane,
                lds + C::OFF_KS + buf * C::KS + j * 1024);
    }
  };
  auto issue_v = [&](int cc, int buf) {       // V^<s> chunk cc (codes + scales) -> V buffer buf
#pragma unroll
    for (int i = 0; i < C::NVW; ++i) {
      const int j = w + kFwdWaves * i;
      if (j < C::NV) dma16(Vs + (int64_t)8 * j * Lp + cc * kChunk + voff[i], lds + C::OFF_V + buf * C::V + j * 1024);
    }
    // V scales: load j covers channels 64j .. 64j+63, 16 B (4 key blocks) each
    if constexpr (C::NKS + C::NVS <= kFwdWaves) {
      if (w >= C::NKS && w < C::NKS + C::NVS) {
        const int j = w - C::NKS;
        dma16(Vss + (int64_t)(64 * j + lane) * (Lp / kBlock) + cc * (kChunk / kBlock),
              lds + C::OFF_VS + buf * C::VS + j * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::NVS; ++j)
        if ((C::NKS + j) % kFwdWaves == w)
          dma16(Vss + (int64_t)(64 * j + lane) * (Lp / kBlock) + cc * (kChunk / kBlock),
                lds + C::OFF_VS + buf * C::VS + j * 1024);
    }
  };

  v8i qb[KS];
  int qsc[KS];
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

  // LDS read offsets of this lane: K rows in pair_row order, V rows natural
  const int kr = pair_row(R);
  int kro[KS][2], vro[2][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kro[ks][0] = kr * DQK + 16 * tile_slot<DQK>(kr, 4 * ks + h);
    kro[ks][1] = kr * DQK + 16 * tile_slot<DQK>(kr, 4 * ks + 2 + h);
  }
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    vro[st][0] = R * kChunk + 16 * tile_slot<kChunk>(R, 4 * st + h);
    vro[st][1] = R * kChunk + 16 * tile_slot<kChunk>(R, 4 * st + 2 + h);
  }

  const float c2 = sigma * kLog2e;
  float mu = -INFINITY;
  double l = 0.0;                                // FP32 per chunk, FP64 across chunks
  v16f oacc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) oacc[ct] = v16f{};

  const int qlast = min(q0 + kFwdQ, Lp) - 1;
  const int nchunks = CAUSAL ? (qlast / kChunk + 1) : Lp / kChunk;
  // last chunk this wave needs (its other chunks are fully masked)
  const int wlast = CAUSAL ? min(nchunks - 1, (qw + 31) / kChunk) : nchunks - 1;

  // scores of K tile t (32 keys) of the chunk in K buffer buf
  auto score_tile = [&](int buf, int t) -> v16f {
    const uint8_t* sK = lds + buf * C::K + 32 * t * DQK;
    const float* sKs = reinterpret_cast<const float*>(lds + C::OFF_KS + buf * C::KS) + (32 * t + kr) * KB;
    v16f acc = v16f{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      v8i a = cat(lds_read16(sK + kro[ks][0]), lds_read16(sK + kro[ks][1]));
      acc = mfma<E4M3, E4M3>(a, qb[ks], acc, e8m0(sKs[2 * ks + h]), qsc[ks]);
    }
    return acc;
  };

  issue_k(0, 0);
  issue_v(0, 0);
  if (nchunks > 1) issue_k(1, 1);
  wait_vmem();
  __syncthreads();
  v16f s[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) s[t] = live ? score_tile(0, t) : v16f{};

  for (int c = 0; c < nchunks; ++c) {
    const int k0 = c * kChunk;
    wait_vmem();
    __syncthreads();                             // K(c+1), V(c) landed; K buffer c%2 and V buffer (c+1)%2 free
    if (c + 2 < nchunks) issue_k(c + 2, c & 1);
    if (c + 1 < nchunks) issue_v(c + 1, (c + 1) & 1);
    if (!live || c > wlast) continue;

    if ((k0 + kChunk > L) || (CAUSAL && k0 + kChunk - 1 > qw)) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = k0 + 32 * t + 16 * h + v;
          if (kk >= L || (CAUSAL && kk > qi)) s[t][v] = -INFINITY;
        }
    }
    // block maxima of the raw scores; exp2 is monotone, so the block amax of P' is
    // exp2 of the block max, computed by the same instructions as that element
    float bm[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bm[t] = pair_max(max16(s[t]));
    const float mx = fmaxf(fmaxf(bm[0], bm[1]), fmaxf(bm[2], bm[3]));
    const float mu_new = fmaxf(mu, mx);
    const float m2 = (mu_new == -INFINITY) ? 0.f : mu_new * c2;
    // exactly 1 when no maximum moved (the fused mu*c2 - m2 would otherwise leave the
    // product's rounding error, and an exp2 of it that can miss 1 by an ulp)
    const float alpha = mu_new == mu ? 1.f : __builtin_amdgcn_exp2f(mu * c2 - m2);
    mu = mu_new;
    l *= (double)alpha;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) oacc[ct] *= alpha;
    }

    v8i pb[2];
    int psc[2] = {0, 0};
    float lc = 0.f;
    const int nb = (c + 1) & 1;
    // K^<c> operand rows of the next chunk's tiles, read one tile ahead of their
    // products so the LDS latency hides behind this chunk's softmax (K buffer nb
    // landed before the barrier above).  Not at d_qk = 192: its three operand
    // pairs would spill at two waves per SIMD.
    constexpr bool KPRE = DQK != 192;
    v8i kpre[KPRE ? KS : 1];
    if constexpr (KPRE) {
      const uint8_t* sK = lds + nb * C::K;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kpre[ks] = cat(lds_read16(sK + kro[ks][0]), lds_read16(sK + kro[ks][1]));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float am = __builtin_amdgcn_exp2f(fmaf(bm[t], c2, -m2));
      const int k = scale_exp<E4M3>(am);
      const float sc = exp2i(k);
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(fmaf(s[t][v], c2, -m2));
      float ls = p[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) ls += p[v];
      lc += ls;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        pb[t >> 1][4 * (t & 1) + g] = (int)pack4s<E4M3>(p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3], sc);
      if ((t & 1) == h) psc[t >> 1] = k + 127;
      // tile t of chunk c+1 into the registers just freed (computed unconditionally:
      // past this wave's last chunk the result is simply never used)
      if constexpr (KPRE) {
        const float* sKs = reinterpret_cast<const float*>(lds + C::OFF_KS + nb * C::KS) + (32 * t + kr) * KB;
        v16f acc = v16f{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma<E4M3, E4M3>(kpre[ks], qb[ks], acc, e8m0(sKs[2 * ks + h]), qsc[ks]);
        s[t] = acc;
        if (t + 1 < 4) {
          const uint8_t* sK = lds + nb * C::K + 32 * (t + 1) * DQK;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) kpre[ks] = cat(lds_read16(sK + kro[ks][0]), lds_read16(sK + kro[ks][1]));
        }
      } else {
        s[t] = score_tile(nb, t);
      }
    }

    const uint8_t* sV = lds + C::OFF_V + (c & 1) * C::V;
    const float* sVs = reinterpret_cast<const float*>(lds + C::OFF_VS + (c & 1) * C::VS);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint8_t* vp = sV + 32 * ct * kChunk;
        v8i a = cat(lds_read16(vp + vro[st][0]), lds_read16(vp + vro[st][1]));
        oacc[ct] = mfma<E4M3, E4M3>(a, pb[st], oacc[ct], e8m0(sVs[(32 * ct + R) * 4 + 2 * st + h]), psc[st]);
      }
    l += (double)lc;
  }

  if (!live) return;
  l = pair_sum_d(l);
  if (qi < L) {
    const float inv_l = (float)(1.0 / l);
    float* orow = o + (qhead * L + qi) * DV;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        v4f r = {oacc[ct][4 * a] * inv_l, oacc[ct][4 * a + 1] * inv_l, oacc[ct][4 * a + 2] * inv_l,
                 oacc[ct][4 * a + 3] * inv_l};
        *reinterpret_cast<v4f*>(orow + 32 * ct + 8 * a + 4 * h) = r;
      }
    if (h == 0) lse[qhead * L + qi] = (float)((double)mu * sigma + log(l));
  }
}

template <int DQK, int DV>
static void launch_fwd_t(const AttnDims& d, Operand q, Operand k, Operand v, float* o, float* lse, hipStream_t s) {
  constexpr int NW = fwd_waves<DQK, DV>();
  dim3 grid((unsigned)((d.Lp + 32 * NW - 1) / (32 * NW)) * d.Hq * d.B);
  if (d.causal)
    hipLaunchKernelGGL((fwd_kernel<DQK, DV, true>), grid, dim3(64 * NW), 0, s, q.codes, q.scales, k.codes,
                       k.scales, v.codes, v.scales, o, lse, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
  else
    hipLaunchKernelGGL((fwd_kernel<DQK, DV, false>), grid, dim3(64 * NW), 0, s, q.codes, q.scales, k.codes,
                       k.scales, v.codes, v.scales, o, lse, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
}

hipError_t launch_fwd(const AttnDims& d, Operand q, Operand k, Operand v, float* o, float* lse, hipStream_t s) {
  if (d.dqk == 64 && d.dv == 64) launch_fwd_t<64, 64>(d, q, k, v, o, lse, s);
  else if (d.dqk == 128 && d.dv == 128) launch_fwd_t<128, 128>(d, q, k, v, o, lse, s);
  else if (d.dqk == 192 && d.dv == 128) launch_fwd_t<192, 128>(d, q, k, v, o, lse, s);
  else if (d.dqk == 64 && d.dv == 128) launch_fwd_t<64, 128>(d, q, k, v, o, lse, s);
  else if (d.dqk == 128 && d.dv == 64) launch_fwd_t<128, 64>(d, q, k, v, o, lse, s);
  else if (d.dqk == 192 && d.dv == 64) launch_fwd_t<192, 64>(d, q, k, v, o, lse, s);
  else if (d.dqk == 256 && d.dv == 256) launch_fwd_t<256, 256>(d, q, k, v, o, lse, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dm
