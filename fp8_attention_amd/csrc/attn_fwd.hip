// Forward of block-scaled FP8 attention on gfx950 matrix cores.
//
// Workgroup = 4 waves = 128 queries (32 per wave); grid = (query tiles, Hq, B).
// Each wave keeps its queries' Q^<c> codes in registers as the B operand of
// S^T = K Q^T, so the score tile comes out with one query per lane pair
// (R, R+32) and 16 keys per lane -- exactly the B-operand layout the P V
// product needs, so the probabilities are cast to E4M3 in registers and fed
// to the next instruction without any lane exchange.  Per 128-key chunk:
//   K^<c> [128 x d_qk] and V^<s> [d_v x 128] codes + scales are staged in LDS
//   with 16-byte loads;
//   S^T = K Q^T (scaled FP8 MFMA, FP32 accumulate);
//   mu  = max(mu, chunk row max)   (exact running max, once per chunk);
//   P'  = exp2(S*sigma*log2e - mu*sigma*log2e); l += sum P' (FP32, unquantized);
//   P'^ = E4M3 cast per 32-key block (amax over the lane pair);
//   O^T = O^T * exp(mu_old - mu) + V^T P'^^T   (scaled FP8 MFMA).
// Epilogue: O = O^T / l, LSE = sigma*mu + ln l.
#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const uint8_t* __restrict__ qc, const float* __restrict__ qcs,
                                                  const uint8_t* __restrict__ kc, const float* __restrict__ kcs,
                                                  const uint8_t* __restrict__ vs, const float* __restrict__ vss,
                                                  float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv,
                                                  int L, int Lp, float sigma) {
  constexpr int KS = DQK / 64;      // 64-channel steps of QK^T
  constexpr int NCT = DV / 32;      // 32-channel tiles of O^T
  constexpr int KB = DQK / 32;      // channel blocks per K row
  constexpr int KROW = DQK + 16;    // LDS pitch (bytes) of a K row
  constexpr int VROW = kChunk + 16; // LDS pitch (bytes) of a V^T row (128 keys)
  __shared__ __attribute__((aligned(16))) uint8_t sK[kChunk * KROW];
  __shared__ __attribute__((aligned(16))) float sKs[kChunk * KB];
  __shared__ __attribute__((aligned(16))) uint8_t sV[DV * VROW];
  __shared__ __attribute__((aligned(16))) float sVs[DV * 4];

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
  const uint8_t* Kc = kc + khead * Lp * DQK;
  const float* Kcs = kcs + khead * Lp * KB;
  const uint8_t* Vs = vs + khead * DV * Lp;
  const float* Vss = vss + khead * DV * (Lp / kBlock);

  v8i qb[KS];
  int qsc[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint8_t* p = Qc + (int64_t)qi * DQK + 64 * ks;
    qb[ks] = cat(*reinterpret_cast<const v4i*>(p + 16 * h), *reinterpret_cast<const v4i*>(p + 32 + 16 * h));
    qsc[ks] = e8m0(Qcs[(int64_t)qi * KB + 2 * ks + h]);
  }

  const float c2 = sigma * kLog2e;
  float mu = -INFINITY;
  double l = 0.0;                                // FP32 per chunk, FP64 across chunks
  v16f oacc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) oacc[ct] = v16f{};

  const int nchunks = CAUSAL ? (qt + 1) : nqt;
  const int krow_a = pair_row(R);
  for (int c = 0; c < nchunks; ++c) {
    const int k0 = c * kChunk;
    __syncthreads();
    // stage K^<c> rows k0..k0+127 and V^<s> columns k0..k0+127
#pragma unroll
    for (int i = tid; i < kChunk * DQK / 16; i += 256) {
      const int row = (i * 16) / DQK, col = (i * 16) % DQK;
      *reinterpret_cast<v4i*>(sK + row * KROW + col) =
          *reinterpret_cast<const v4i*>(Kc + (int64_t)(k0 + row) * DQK + col);
    }
    for (int i = tid; i < kChunk * KB / 4; i += 256)
      *reinterpret_cast<v4f*>(sKs + 4 * i) = *reinterpret_cast<const v4f*>(Kcs + (int64_t)k0 * KB + 4 * i);
#pragma unroll
    for (int i = tid; i < DV * kChunk / 16; i += 256) {
      const int row = i / (kChunk / 16), col = (i % (kChunk / 16)) * 16;
      *reinterpret_cast<v4i*>(sV + row * VROW + col) =
          *reinterpret_cast<const v4i*>(Vs + (int64_t)row * Lp + k0 + col);
    }
    for (int i = tid; i < DV; i += 256)
      *reinterpret_cast<v4f*>(sVs + 4 * i) = *reinterpret_cast<const v4f*>(Vss + (int64_t)i * (Lp / kBlock) + k0 / kBlock);
    __syncthreads();
    if (CAUSAL && k0 > q0 + 32 * w + 31) continue;   // every key of the chunk is masked for this wave

    v16f s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = v16f{};
      const int krow = 32 * t + krow_a;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint8_t* p = sK + krow * KROW + 64 * ks;
        v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
        s[t] = mfma<E4M3, E4M3>(a, qb[ks], s[t], e8m0(sKs[krow * KB + 2 * ks + h]), qsc[ks]);
      }
    }
    const bool need_mask = (k0 + kChunk > L) || (CAUSAL && k0 + kChunk - 1 > q0 + 32 * w);
    if (need_mask) {
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
    for (int t = 0; t < 4; ++t) {
      float m = s[t][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) m = fmaxf(m, s[t][v]);
      bm[t] = pair_max(m);
    }
    const float mx = fmaxf(fmaxf(bm[0], bm[1]), fmaxf(bm[2], bm[3]));
    const float mu_new = fmaxf(mu, mx);
    const float m2 = (mu_new == -INFINITY) ? 0.f : mu_new * c2;
    const float alpha = __builtin_amdgcn_exp2f(mu * c2 - m2);
    mu = mu_new;
    l *= (double)alpha;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) oacc[ct] *= alpha;
    }

    v8i pb[2];
    int psc[2] = {0, 0};
    float lc = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float am = __builtin_amdgcn_exp2f(fmaf(bm[t], c2, -m2));
      const int k = scale_exp<E4M3>(am);
      const float inv = exp2i(-k);
      float ls = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float p4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p4[e] = __builtin_amdgcn_exp2f(fmaf(s[t][4 * g + e], c2, -m2));
          ls += p4[e];
        }
        pb[t >> 1][4 * (t & 1) + g] = (int)pack4<E4M3>(p4[0] * inv, p4[1] * inv, p4[2] * inv, p4[3] * inv);
      }
      lc += ls;
      if ((t & 1) == h) psc[t >> 1] = k + 127;
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int vrow = 32 * ct + R;
        const uint8_t* p = sV + vrow * VROW + 64 * st;
        v8i a = cat(lds_read16(p + 16 * h), lds_read16(p + 32 + 16 * h));
        oacc[ct] = mfma<E4M3, E4M3>(a, pb[st], oacc[ct], e8m0(sVs[vrow * 4 + 2 * st + h]), psc[st]);
      }
    l += (double)lc;
  }

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
  dim3 grid(d.Lp / kChunk, d.Hq, d.B);
  if (d.causal)
    hipLaunchKernelGGL((fwd_kernel<DQK, DV, true>), grid, dim3(256), 0, s, q.codes, q.scales, k.codes, k.scales,
                       v.codes, v.scales, o, lse, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
  else
    hipLaunchKernelGGL((fwd_kernel<DQK, DV, false>), grid, dim3(256), 0, s, q.codes, q.scales, k.codes, k.scales,
                       v.codes, v.scales, o, lse, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
}

hipError_t launch_fwd(const AttnDims& d, Operand q, Operand k, Operand v, float* o, float* lse, hipStream_t s) {
  if (d.dqk == 64 && d.dv == 64) launch_fwd_t<64, 64>(d, q, k, v, o, lse, s);
  else if (d.dqk == 128 && d.dv == 128) launch_fwd_t<128, 128>(d, q, k, v, o, lse, s);
  else if (d.dqk == 192 && d.dv == 128) launch_fwd_t<192, 128>(d, q, k, v, o, lse, s);
  else if (d.dqk == 64 && d.dv == 128) launch_fwd_t<64, 128>(d, q, k, v, o, lse, s);
  else if (d.dqk == 128 && d.dv == 64) launch_fwd_t<128, 64>(d, q, k, v, o, lse, s);
  else if (d.dqk == 192 && d.dv == 64) launch_fwd_t<192, 64>(d, q, k, v, o, lse, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dm
