// Row correction delta in three modes.
//
// stale / dO-matched: delta_i = sum_k x_ik O_ik with x = dO (bf16, before its
//   cast) or x = dO^<c> (decoded E5M2 codes times block scales).  One pass over
//   O and x with 16-byte loads; bound by HBM bandwidth.
// matched (Delta-Matching): delta_i = sum_j P_ij dP^_ij / sum_j P_ij with
//   P = exp(S - LSE) recomputed in FP32 and dP^ = dO^<c> V^<c>^T on FP8 matrix
//   cores.  The denominator is 1 in exact arithmetic (P is the softmax); with P
//   rebuilt from the FP32-rounded LSE it drifts from 1 by up to ~1e-5 on long,
//   near-saturated rows, and dividing by the sum the dQ kernel reproduces bit for
//   bit (same products, same exp2) keeps sum_j dS_ij = 0 in the kernels' own
//   arithmetic, which is the property the correction exists for.  Same tiling
//   as the forward: 8 waves x 32 queries, 128-key chunks streamed through LDS;
//   the S^T and dP^T tiles share one layout (query per lane pair, 16 keys per
//   lane), so the product and its row sum stay in registers until one pair
//   reduction.
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
  if (d.dv == 256) {
    if (m) hipLaunchKernelGGL((delta_rows_kernel<256, true>), dim3(blocks), dim3(256), 0, s, o, dob, doc.codes, doc.scales, delta, nrows, d.L, d.Lp);
    else hipLaunchKernelGGL((delta_rows_kernel<256, false>), dim3(blocks), dim3(256), 0, s, o, dob, doc.codes, doc.scales, delta, nrows, d.L, d.Lp);
  } else if (d.dv == 128) {
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
// waves per workgroup (32 queries each): two per SIMD; one per SIMD when
// d_qk = d_v = 256, whose Q, dO rows and score tiles fill more than half the file
template <int DQK, int DV> constexpr int delta_waves() { return DQK + DV > 384 ? 4 : 8; }
// Up to d_qk + d_v = 256 a lean form keeps one score tile live at a time and fits in
// 128 VGPRs, so two workgroups share a CU (four waves per SIMD, 72 KB of LDS each) and
// the waves interleave their MFMA and softmax work: 8% faster than prefetching the next
// chunk's tiles at two waves per SIMD on large grids (8K, 64K), slower on small ones
// (4K: two unequal causal tiles per CU), so the launcher picks it for grids of at least
// four workgroups per CU.  Wider heads would spill at 128 and only have the prefetching
// form, which overlaps within the wave instead.
template <int DQK, int DV> constexpr bool delta_lean_ok() { return DQK + DV <= 256; }

template <int DQK, int DV>
struct DeltaLds {
  static constexpr int NW = delta_waves<DQK, DV>();
  static constexpr int KB = DQK / 32, VB = DV / 32;
  static constexpr int K = kChunk * DQK, V = kChunk * DV;      // K^<c>, V^<c> rows of a chunk, swizzled
  static constexpr int KS = kChunk * KB * 4, VS = kChunk * VB * 4;
  static constexpr int BUF = K + V + KS + VS;                  // one chunk
  static constexpr int OFF_V = K, OFF_KS = K + V, OFF_VS = K + V + KS;
  static constexpr int NJ = BUF / 1024;                        // direct loads per chunk
  static constexpr int NJW = (NJ + NW - 1) / NW;
  static_assert(K % 1024 == 0 && V % 1024 == 0 && KS % 1024 == 0 && VS % 1024 == 0, "whole 1 KB loads");
  static_assert(2 * BUF <= 160 * 1024, "LDS budget");
};

// Workgroup = 8 waves = 256 queries (4 waves = 128 when d = 256); 1-D grid over (query tile, Hq, B), query
// tile slowest and the longest causal tiles first.  Per 128-key chunk and 32-key tile:
// S^T = K Q^T and dP^T = V dO^T (lane pair = query, 16 keys per lane), then
// delta += sum P * dP^ with P = exp2(S sigma log2e - LSE log2e).  K^<c> / V^<c>
// chunks are double-buffered in LDS via direct global->LDS loads.  Two loop forms
// (LEAN): one tile live at four waves per SIMD, or the tiles of
// chunk c+1 computed as soon as tile t of chunk c has been consumed.  Both accumulate
// in the same order, so they give the same bits.
template <int DQK, int DV, bool CAUSAL, bool LEAN>
__global__ __launch_bounds__((64 * delta_waves<DQK, DV>()), (LEAN ? 4 : 1)) void delta_matched_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ kc,
    const float* __restrict__ kcs, const uint8_t* __restrict__ vc, const float* __restrict__ vcs,
    const uint8_t* __restrict__ doc, const float* __restrict__ docs, const float* __restrict__ lse,
    float* __restrict__ delta, int Hq, int Hkv, int L, int Lp, float sigma) {
  using C = DeltaLds<DQK, DV>;
  constexpr int kDelWaves = C::NW, kDelQ = 32 * kDelWaves;
  constexpr int KS = DQK / 64, VS = DV / 64;
  constexpr int KB = DQK / 32, VB = DV / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int R = lane & 31, h = lane >> 5;
  const int nqt = (Lp + kDelQ - 1) / kDelQ;
  const QueryItem item = query_item((int)blockIdx.x, nqt, Hq, Hkv, (int)gridDim.x / (nqt * Hq));
  const int qt = CAUSAL ? (nqt - 1 - item.tr) : item.tr;  // longest causal tiles first
  const int hq = item.hq, b = item.b;
  const int hk = hq / (Hq / Hkv);
  const int q0 = qt * kDelQ;
  const int qw = q0 + 32 * w;
  const bool live = qw < Lp;
  const int qi = qw + R;
  const int64_t qhead = (int64_t)b * Hq + hq, khead = (int64_t)b * Hkv + hk;
  const uint8_t* Kc = kc + khead * Lp * DQK;
  const float* Kcs = kcs + khead * Lp * KB;
  const uint8_t* Vc = vc + khead * Lp * DV;
  const float* Vcs = vcs + khead * Lp * VB;

  // direct-load source offsets (relative to the chunk) of this lane, loop invariant
  int soff[C::NJW];
#pragma unroll
  for (int i = 0; i < C::NJW; ++i) {
    const int pb = (w + kDelWaves * i) * 1024 + 16 * lane;
    int off = 0;
    if (pb < C::OFF_V) {
      const int r = pb / DQK, c = (pb % DQK) / 16;
      off = r * DQK + 16 * tile_slot<DQK>(r, c);
    } else if (pb < C::OFF_KS) {
      const int p = pb - C::OFF_V, r = p / DV, c = (p % DV) / 16;
      off = r * DV + 16 * tile_slot<DV>(r, c);
    } else if (pb < C::OFF_VS) {
      off = pb - C::OFF_KS;
    } else {
      off = pb - C::OFF_VS;
    }
    soff[i] = off;
  }
  auto issue = [&](int cc, int buf) {         // chunk cc -> buffer buf
#pragma unroll
    for (int i = 0; i < C::NJW; ++i) {
      const int j = w + kDelWaves * i;
      if (j >= C::NJ) continue;
      const int jb = j * 1024;
      const uint8_t* base;
      if (jb < C::OFF_V) base = Kc + (int64_t)cc * kChunk * DQK;
      else if (jb < C::OFF_KS) base = Vc + (int64_t)cc * kChunk * DV;
      else if (jb < C::OFF_VS) base = reinterpret_cast<const uint8_t*>(Kcs + (int64_t)cc * kChunk * KB);
      else base = reinterpret_cast<const uint8_t*>(Vcs + (int64_t)cc * kChunk * VB);
      dma16(base + soff[i], lds + buf * C::BUF + jb);
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
  int kro[KS][2], vro[VS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) kro[ks][e] = kr * DQK + 16 * tile_slot<DQK>(kr, 4 * ks + 2 * e + h);
#pragma unroll
  for (int ks = 0; ks < VS; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) vro[ks][e] = kr * DV + 16 * tile_slot<DV>(kr, 4 * ks + 2 * e + h);

  const float c2 = sigma * kLog2e;
  const float l2 = (live && qi < L) ? lse[qhead * L + qi] * kLog2e : 0.f;
  double acc = 0.0, psum = 0.0;                  // FP32 per chunk, FP64 across chunks
  const int qlast = min(q0 + kDelQ, Lp) - 1;
  const int nchunks = CAUSAL ? (qlast / kChunk + 1) : Lp / kChunk;
  const int wlast = CAUSAL ? min(nchunks - 1, (qw + 31) / kChunk) : nchunks - 1;

  // S^T and dP^T tiles of key tile t of the chunk in buffer buf
  auto tiles = [&](int buf, int t, v16f& s, v16f& dp) {
    const uint8_t* bb = lds + buf * C::BUF;
    const float* ks_ = reinterpret_cast<const float*>(bb + C::OFF_KS) + (32 * t + kr) * KB;
    const float* vs_ = reinterpret_cast<const float*>(bb + C::OFF_VS) + (32 * t + kr) * VB;
    s = v16f{};
    dp = v16f{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint8_t* p = bb + 32 * t * DQK;
      const v8i a = cat(lds_read16(p + kro[ks][0]), lds_read16(p + kro[ks][1]));
      s = mfma<E4M3, E4M3>(a, qb[ks], s, e8m0(ks_[2 * ks + h]), qsc[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < VS; ++ks) {
      const uint8_t* p = bb + C::OFF_V + 32 * t * DV;
      const v8i a = cat(lds_read16(p + vro[ks][0]), lds_read16(p + vro[ks][1]));
      dp = mfma<E4M3, E5M2>(a, db[ks], dp, e8m0(vs_[2 * ks + h]), dsc[ks]);
    }
  };

  issue(0, 0);
  if (nchunks > 1) issue(1, 1);
  if constexpr (LEAN) {
    // one tile at a time; chunk c+1 is loaded while chunk c is consumed
    for (int c = 0; c < nchunks; ++c) {
      const int k0 = c * kChunk;
      wait_vmem();
      __syncthreads();                           // chunk c landed; buffer (c+1)%2 free
      if (c >= 1 && c + 1 < nchunks) issue(c + 1, (c + 1) & 1);
      if (!live || c > wlast) continue;
      const bool mask = (k0 + kChunk > L) || (CAUSAL && k0 + kChunk - 1 > qw);
      const int lim = (CAUSAL ? min(qi, L - 1) : L - 1) - (k0 + 16 * h);   // key k0+32t+16h+v visible iff 32t+v <= lim
      float cacc = 0.f, pc = 0.f;
#pragma unroll 1
      for (int t = 0; t < 4; ++t) {
        v16f s, dp;
        tiles(c & 1, t, s, dp);
        if (mask) {
#pragma unroll
          for (int v = 0; v < 16; ++v) s[v] = (32 * t + v > lim) ? -INFINITY : s[v];
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[v], c2, -l2));
          cacc = fmaf(p, dp[v], cacc);
          pc += p;
        }
      }
      acc += (double)cacc;
      psum += (double)pc;
    }
  } else {
  wait_vmem();
  __syncthreads();
  v16f s[4], dp[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (live) tiles(0, t, s[t], dp[t]);
    else s[t] = dp[t] = v16f{};
  }
  for (int c = 0; c < nchunks; ++c) {
    const int k0 = c * kChunk;
    wait_vmem();
    __syncthreads();                             // chunk c+1 landed; buffer c%2 free
    if (c + 2 < nchunks) issue(c + 2, c & 1);
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
    float cacc = 0.f, pc = 0.f;
    const int nb = (c + 1) & 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[t][v], c2, -l2));
        cacc = fmaf(p, dp[t][v], cacc);
        pc += p;
      }
      // tile t of chunk c+1 (unused past this wave's last chunk)
      tiles(nb, t, s[t], dp[t]);
    }
    acc += (double)cacc;
    psum += (double)pc;
  }
  }
  if (!live) return;
  acc = pair_sum_d(acc);
  psum = pair_sum_d(psum);
  // divided by the row's own sum of P (see the header)
  if (qi < L && h == 0) delta[qhead * L + qi] = psum > 0.0 ? (float)(acc / psum) : 0.f;
}

template <int DQK, int DV>
static void launch_dm_t(const AttnDims& d, Operand doc, Operand q, Operand k, Operand v, const float* lse,
                        float* delta, hipStream_t s) {
  constexpr int NW = delta_waves<DQK, DV>();
  const unsigned nblk = (unsigned)((d.Lp + 32 * NW - 1) / (32 * NW)) * d.Hq * d.B;
  int ncu = 256;
  {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  }
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(64 * NW), 0, s, q.codes, q.scales, k.codes, k.scales, v.codes,
                       v.scales, doc.codes, doc.scales, lse, delta, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
  };
  if constexpr (delta_lean_ok<DQK, DV>()) {
    if (nblk >= 4u * (unsigned)ncu) {
      if (d.causal) go(delta_matched_kernel<DQK, DV, true, true>);
      else go(delta_matched_kernel<DQK, DV, false, true>);
      return;
    }
  }
  if (d.causal) go(delta_matched_kernel<DQK, DV, true, false>);
  else go(delta_matched_kernel<DQK, DV, false, false>);
}

hipError_t launch_delta_matched(const AttnDims& d, Operand doc, Operand q, Operand k, Operand v, const float* lse,
                                float* delta, hipStream_t s) {
  if (d.dqk == 64 && d.dv == 64) launch_dm_t<64, 64>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 128 && d.dv == 128) launch_dm_t<128, 128>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 192 && d.dv == 128) launch_dm_t<192, 128>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 64 && d.dv == 128) launch_dm_t<64, 128>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 128 && d.dv == 64) launch_dm_t<128, 64>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 192 && d.dv == 64) launch_dm_t<192, 64>(d, doc, q, k, v, lse, delta, s);
  else if (d.dqk == 256 && d.dv == 256) launch_dm_t<256, 256>(d, doc, q, k, v, lse, delta, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dm
