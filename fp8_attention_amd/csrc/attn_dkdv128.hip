// dK and dV of block-scaled FP8 attention for d_qk = d_v = 128 (key-stationary),
// on the 16x16x128 scaled matrix instruction.
//
// Workgroup = 8 waves over 128 keys; wave w owns keys k0+16w .. k0+16w+15 and
// forms every product for them, so S, P, dP and dS exist once per (query, key)
// pair.  A 1-D grid over (key tile, Hkv, B) with key tiles slowest starts the
// long causal tiles first.  The workgroup walks the query heads of its KV group
// and, for each, the 128-query steps that can see its keys.  Per step and wave:
//   8 tiles of 16 queries:  S = Q^<c> K^<c>T,  dP^ = dO^<c> V^<c>T  (one instruction each),
//                           P = exp(S - LSE),  dS = P (dP^ - delta);
//   P^<q> (E4M3) and dS^<q> (E5M2) in 32-query blocks;
//   dV^T += dO^<s>T P^<q>,  dK^T += Q^<s>T dS^<q>  (8 channel tiles each, contraction
//   over the step's 128 queries).
// Row m of S tile t is step query qrow(t, m); with that order the 32 results of a
// lane over the 8 tiles are exactly its 32 K-slots of the dV/dK operand, in slot
// order, and every 32-query scale block is split over one lane pair (l, l^16).
// So the codes never leave their lane: per block, one pair max and one exchange
// that hands the block's scale to the lane that supplies it.
//
// The query-side tiles of step i+1 (Q^<c>, dO^<c> rows, Q^<s>, dO^<s> channel
// rows and all four scale arrays) arrive in the other half of a double LDS
// buffer by direct global->LDS loads issued during step i, one per S tile (issued
// all at once, they stall the waves behind them); LSE and delta come through registers.  One barrier per step.  dK and dV accumulate in
// registers over every query head of the group and are written once.
//
// Head split (small grids): with HS > 1 the G query heads of a KV group are dealt to
// HS workgroups per key tile (heads [hp*G/HS, (hp+1)*G/HS)), so a grid of one key tile
// per CU still spreads its long causal tiles; each part writes its raw dV^T and dK^T
// sums to a workspace and dkdv_reduce_kernel adds the parts in a fixed order.
//
// The PROBE instance runs the same arithmetic and also returns, per query row,
// the sum over keys of the FP32 dS it casts and of |P dP^| (section 03 of the
// Delta-Matching project page: matched delta makes the rows of dS sum to zero up
// to FP32 rounding before the cast).  Each wave reduces its 16 keys across lanes
// and adds its partial sums to the caller's FP64 rows atomically.
#include <type_traits>

#include "dm_common.h"
#include "dm_internal.h"

namespace dm {
namespace {

constexpr int kD = 128;                  // d_qk = d_v
constexpr int kNW = 8, kNT = 64 * kNW;
constexpr int kKT = 16 * kNW;            // keys per workgroup
constexpr int kQT = 128;                 // queries per step
// one step's stage (bytes).  Q^<c>/dO^<c> rows and their scales are stored in
// tile order: LDS row 16t+m holds step query qrow(t, m).
constexpr int kQC = 0;                   // Q^<c> [128 rows][128], chunks swizzled by tile_slot<128>
constexpr int kDOC = kQC + kQT * kD;     // dO^<c> rows
constexpr int kQS = kDOC + kQT * kD;     // Q^<s> [128 channels][128 queries], swizzled
constexpr int kDOS = kQS + kD * kQT;     // dO^<s>
constexpr int kQCS = kDOS + kD * kQT;    // Q^<c> scales [128 rows][4 blocks] fp32
constexpr int kDOCS = kQCS + kQT * 16;   // dO^<c> scales
constexpr int kQSS = kDOCS + kQT * 16;   // Q^<s> scales [128 channels][4 query blocks]
constexpr int kDOSS = kQSS + kD * 16;    // dO^<s> scales
constexpr int kLSE = kDOSS + kD * 16;    // LSE * log2(e) [128], then delta [128]
constexpr int kSTAGE = kLSE + 2 * kQT * 4;
static_assert(2 * kSTAGE <= 160 * 1024, "LDS budget");

// step query of row m of S tile t (see the header comment)
__device__ __forceinline__ int qrow(int t, int m) { return 64 * (t >> 2) + 16 * (m >> 2) + 4 * (t & 3) + (m & 3); }

}  // namespace

template <bool CAUSAL, bool PROBE>
__global__ __launch_bounds__(kNT) void dkdv_d128_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qcs, const uint8_t* __restrict__ qs,
    const float* __restrict__ qss, const uint8_t* __restrict__ kc, const float* __restrict__ kcs,
    const uint8_t* __restrict__ vc, const float* __restrict__ vcs, const uint8_t* __restrict__ doc,
    const float* __restrict__ docs, const uint8_t* __restrict__ dos, const float* __restrict__ doss,
    const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv,
    double* __restrict__ psum, double* __restrict__ pabs, float* __restrict__ part, int HS, int Hq, int Hkv, int L,
    int Lp, float sigma) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kSTAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n = lane & 15, g = lane >> 4;              // key column / lane group of the 16x16 tiles
  const int nkt = Lp / kKT;
  const int nhb = Hkv * (int)(gridDim.x / (nkt * Hkv * HS));    // Hkv * B
  const int hk = (int)blockIdx.x % nhb % Hkv, b = (int)blockIdx.x % nhb / Hkv;
  const int rest = (int)blockIdx.x / nhb;                 // key tile (slowest: long causal tiles first), head part
  const int k0 = (rest / HS) * kKT, hp = rest % HS;
  const int G = Hq / Hkv;
  const int hbeg = hp * (G / HS), hend = hbeg + G / HS;  // this workgroup's query heads of the group
  const int kw0 = k0 + 16 * w;                       // this wave's first key
  const int key = kw0 + n;                           // this lane's key
  const int LB = Lp / kBlock;
  const int64_t khead = (int64_t)b * Hkv + hk;
  const int64_t qhead0 = (int64_t)b * Hq + (int64_t)hk * G;

  // this wave's K^<c>, V^<c> rows as B operands (key n, channel chunks g and 4+g)
  v8i kb, vb;
  int ksc, vsc;
  {
    const int64_t kr = khead * Lp + key;
    kb = cat(*reinterpret_cast<const v4i*>(kc + kr * kD + 16 * g), *reinterpret_cast<const v4i*>(kc + kr * kD + 64 + 16 * g));
    vb = cat(*reinterpret_cast<const v4i*>(vc + kr * kD + 16 * g), *reinterpret_cast<const v4i*>(vc + kr * kD + 64 + 16 * g));
    ksc = e8m0(kcs[kr * (kD / kBlock) + g]);
    vsc = e8m0(vcs[kr * (kD / kBlock) + g]);
  }

  // ---- direct loads: per wave two 1 KB pieces of each 16 KB tile and one piece of the scales
  uint32_t orow[2], ochan[2];                        // per-lane source offsets (loop invariant)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * (w + 8 * i) + (lane >> 3);     // LDS row this lane fills
    const int chunk = tile_slot<kD>(r, lane & 7);    // global 16-byte chunk of that slot
    orow[i] = qrow(r >> 4, r & 15) * kD + 16 * chunk;
    ochan[i] = r * Lp + 16 * chunk;
  }
  const int sel = w >> 1;                            // 0 Q^<c>, 1 dO^<c>, 2 Q^<s>, 3 dO^<s> scales
  const int srow = 64 * (w & 1) + lane;
  const uint32_t oscale = sel < 2 ? qrow(srow >> 4, srow & 15) * 16 : srow * LB * 4;
  const uint8_t* const sbase = reinterpret_cast<const uint8_t*>(sel == 0 ? qcs : sel == 1 ? docs : sel == 2 ? qss : doss);
  const int sdst = kQCS + 1024 * w;
  // base pointers of one step's loads (wave-uniform)
  struct Src {
    const uint8_t *q, *d, *qs, *ds, *sc;
  };
  auto sources = [&](int64_t qhead, int q0) {
    const int64_t rowb = (qhead * Lp + q0) * kD;
    const int64_t chb = qhead * kD * (int64_t)Lp + q0;
    Src r;
    r.q = qc + rowb;
    r.d = doc + rowb;
    r.qs = qs + chb;
    r.ds = dos + chb;
    r.sc = sbase + (sel < 2 ? rowb / 8 : qhead * kD * (int64_t)LB * 4 + q0 / 8);
    return r;
  };
  // one of the step's nine direct loads of this wave (part is a constant after unrolling)
  auto issue_part = [&](int part, const Src& sr, uint8_t* st) {
    if (part == 8) {
      dma16s(sr.sc, oscale, st + sdst);
      return;
    }
    const int i = part >> 2, which = part & 3;
    const int dst = 1024 * (w + 8 * i);
    if (which == 0) dma16s(sr.q, orow[i], st + kQC + dst);
    else if (which == 1) dma16s(sr.d, orow[i], st + kDOC + dst);
    else if (which == 2) dma16s(sr.qs, ochan[i], st + kQS + dst);
    else dma16s(sr.ds, ochan[i], st + kDOS + dst);
  };
  auto issue = [&](const Src& sr, uint8_t* st) {
#pragma unroll
    for (int part = 0; part < 9; ++part) issue_part(part, sr, st);
  };
  // LSE (in log2 units) and delta of the step's queries through registers (threads
  // 0-127 and 128-255; the others load an in-range value they do not store).  The
  // load is unconditional and its value is first used when it is stored at the end
  // of the step, so its latency hides behind the step (a select next to the load
  // made the compiler put the load in a branch and wait for it at once).
  float smallx = 0.f;
  bool smallpad = false;
  auto load_small = [&](int64_t qhead, int q0) {
    const int q = q0 + (tid & (kQT - 1));
    smallx = (tid < kQT ? lse : delta)[qhead * L + min(q, L - 1)];
    smallpad = q >= L;
  };
  auto store_small = [&](uint8_t* st) {
    const bool is_lse = tid < kQT;
    // LSE in log2 units, and delta negated: it is the accumulator input of the dP^ product
    const float v = smallpad ? (is_lse ? INFINITY : 0.f) : (is_lse ? smallx * kLog2e : -smallx);  // padded: P = 0
    if (tid < 2 * kQT) reinterpret_cast<float*>(st + kLSE)[tid] = v;
  };

  v4f accv[kD / 16], acck[kD / 16];                  // dV^T, dK^T channel tiles: reg i <-> channel 16ct+4g+i
#pragma unroll
  for (int i = 0; i < kD / 16; ++i) accv[i] = acck[i] = v4f{};

  const float c2 = sigma * kLog2e;
  const int qstart = CAUSAL ? k0 : 0;
  const int nsteps = (Lp - qstart) / kQT;
  uint8_t* const stage0 = lds;
  issue(sources(qhead0 + hbeg, qstart), stage0);
  load_small(qhead0 + hbeg, qstart);
  store_small(stage0);

  // LDS read offsets of this lane's operand row (row n of a 16-row tile, chunks g and 4+g)
  const int ra0 = n * 128 + 16 * tile_slot<kD>(n, g);
  const int ra1 = n * 128 + 16 * tile_slot<kD>(n, 4 + g);

  // step i of query head hh (running index it); the loads issued during it are those
  // of the next step, or again this step's after the last one (never read)
  auto step = [&](int it, int hh, int i, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int q0 = qstart + i * kQT;
    uint8_t* const st = stage0 + (it & 1) * kSTAGE;
    uint8_t* const stn = stage0 + ((it + 1) & 1) * kSTAGE;
    wait_vmem();
    __syncthreads();                               // step it staged; the other buffer is free
    const bool head_end = i + 1 == nsteps;
    const bool more = !(head_end && hh + 1 == hend);
    const int64_t nqh = qhead0 + hh + (head_end && more ? 1 : 0);
    const int nq0 = !more ? q0 : head_end ? qstart : q0 + kQT;
    const Src nx = sources(nqh, nq0);
    load_small(nqh, nq0);
    if (kw0 >= L) issue(nx, stn);

    if (kw0 < L) {
      uint32_t pc[8], dc[8];                       // P^<q>, dS^<q> codes: dword t <-> S tile t
      int kp[2], kd[2];                            // scale exponents of the lane's lo / hi blocks
      const float* lsep = reinterpret_cast<const float*>(st + kLSE) + 16 * g;
      const float* ndelp = lsep + kQT;               // -delta
      const float* qcsp = reinterpret_cast<const float*>(st + kQCS) + 4 * n + g;
      const float* docsp = reinterpret_cast<const float*>(st + kDOCS) + 4 * n + g;
      // S and dP^ of tile t (and the next step's direct load that goes with it)
      auto tile_mm = [&](int t, v4f& s, v4f& dp) {
        issue_part(t + (t == 0 ? 8 : 0), nx, stn);     // next step's loads, spread over the tiles
        if (t == 0) issue_part(0, nx, stn);
        const v8i aq = cat(lds_read16(st + kQC + 2048 * t + ra0), lds_read16(st + kQC + 2048 * t + ra1));
        s = mfma16<E4M3, E4M3>(aq, kb, v4f{}, e8m0(qcsp[64 * t]), ksc);
        const v8i ad = cat(lds_read16(st + kDOC + 2048 * t + ra0), lds_read16(st + kDOC + 2048 * t + ra1));
        // dP^ - delta: the product accumulates onto -delta of the tile's four query rows
        const v4f nd4 = *reinterpret_cast<const v4f*>(ndelp + 64 * (t >> 2) + 4 * (t & 3));
        dp = mfma16<E5M2, E4M3>(ad, vb, nd4, e8m0(docsp[64 * t]), vsc);
      };
      // software pipeline: the products of tile t+1 are issued before the FP32 work on
      // tile t, so that work does not wait for the matrix core
      v4f s_nx, dp_nx;
      tile_mm(0, s_nx, dp_nx);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // tiles 4hf .. 4hf+3: lane (n, g) holds queries 64hf + 16g + 4tt + i
        float pv[16], sv[16];
        float av[PROBE ? 16 : 1];                  // probe: |P dP^| (dP^ = the accumulator plus delta)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int t = 4 * hf + tt;
          const v4f s = s_nx, dp = dp_nx;
          if (t + 1 < 8) tile_mm(t + 1, s_nx, dp_nx);
          const v4f l4 = *reinterpret_cast<const v4f*>(lsep + 64 * hf + 4 * tt);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = s[i];
            if constexpr (MASK) {
              const int q = q0 + 64 * hf + 16 * g + 4 * tt + i;
              if (key >= L || (CAUSAL && key > q)) x = -INFINITY;
            }
            const float p = __builtin_amdgcn_exp2f(fmaf(x, c2, -l4[i]));
            pv[4 * tt + i] = p;
            sv[4 * tt + i] = p * dp[i];
            if constexpr (PROBE) {
              const v4f n4 = *reinterpret_cast<const v4f*>(ndelp + 64 * hf + 4 * tt);
              av[4 * tt + i] = fabsf(p * (dp[i] - n4[i]));
            }
          }
        }
        if constexpr (PROBE) {
          // sums over the wave's 16 keys (the 16 lanes of group g); lane n then holds
          // those of query 64hf + 16g + n and adds them to the row totals
          float rs[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) rs[k] = sv[k];
          const float r = group_sum_scatter<16, 16>(rs, lane);
          const float a = group_sum_scatter<16, 16>(av, lane);
          const int q = q0 + 64 * hf + 16 * g + n;
          if (q < L) {
            const int64_t row = (qhead0 + hh) * L + q;
            unsafeAtomicAdd(psum + row, (double)r);
            unsafeAtomicAdd(pabs + row, (double)a);
          }
        }
        // block maxima: the lane's 16 values and its partner's (l ^ 16) form one 32-query block
        float mp = fmaxf(fmaxf(pv[0], pv[1]), pv[2]);
        float md = fmaxf(fmaxf(fabsf(sv[0]), fabsf(sv[1])), fabsf(sv[2]));
#pragma unroll
        for (int v = 3; v < 15; v += 2) {
          mp = fmaxf(fmaxf(mp, pv[v]), pv[v + 1]);
          md = fmaxf(fmaxf(md, fabsf(sv[v])), fabsf(sv[v + 1]));
        }
        mp = pair16_max(fmaxf(mp, pv[15]));
        md = pair16_max(fmaxf(md, fabsf(sv[15])));
        kp[hf] = scale_exp<E4M3>(mp);
        kd[hf] = scale_exp<E5M2>(md);
        const float sp = exp2i(kp[hf]), sd = exp2i(kd[hf]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          pc[4 * hf + tt] = pack4s<E4M3>(pv[4 * tt], pv[4 * tt + 1], pv[4 * tt + 2], pv[4 * tt + 3], sp);
          dc[4 * hf + tt] = pack4s<E5M2>(sv[4 * tt], sv[4 * tt + 1], sv[4 * tt + 2], sv[4 * tt + 3], sd);
        }
      }
      // Lane group g supplies the scale of K-block g (queries 32g..32g+31).  Its own
      // blocks are g/2 (lo) and 2+g/2 (hi): groups 0 and 3 hold theirs; group 1 takes
      // block 1 from group 3 and group 2 takes block 2 from group 0 (lanes l ^ 32).
      auto supply = [&](const int* k) {
        const uint32_t x = (uint32_t)(g == 0 ? k[1] : k[0]);
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        const int other = (int)(g == 1 ? r[1] : r[0]);
        return (g == 0 ? k[0] : g == 3 ? k[1] : other) + 127;
      };
      const int sup_p = supply(kp), sup_d = supply(kd);
      v8i bp, bd;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bp[i] = (int)pc[i];
        bd[i] = (int)dc[i];
      }
      // dV^T += dO^<s>T P^<q>,  dK^T += Q^<s>T dS^<q>: A = channel rows 16ct+n, query chunks g, 4+g
      const float* dossp = reinterpret_cast<const float*>(st + kDOSS) + 4 * n + g;
      const float* qssp = reinterpret_cast<const float*>(st + kQSS) + 4 * n + g;
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct) {
        const v8i a = cat(lds_read16(st + kDOS + 2048 * ct + ra0), lds_read16(st + kDOS + 2048 * ct + ra1));
        accv[ct] = mfma16<E5M2, E4M3>(a, bp, accv[ct], e8m0(dossp[64 * ct]), sup_p);
      }
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct) {
        const v8i a = cat(lds_read16(st + kQS + 2048 * ct + ra0), lds_read16(st + kQS + 2048 * ct + ra1));
        acck[ct] = mfma16<E4M3, E5M2>(a, bd, acck[ct], e8m0(qssp[64 * ct]), sup_d);
      }
    }
    store_small(stn);
  };
  // per head: the diagonal step for causal (all steps when the tile holds padded
  // keys) with the mask, then the rest in a loop without mask code
  const int nmask = (k0 + kKT > L) ? nsteps : (CAUSAL ? 1 : 0);
  for (int hh = hbeg, it = 0; hh < hend; ++hh) {
    for (int i = 0; i < nmask; ++i, ++it) step(it, hh, i, std::true_type{});
    for (int i = nmask; i < nsteps; ++i, ++it) step(it, hh, i, std::false_type{});
  }

  wait_vmem();                                     // the last step's (unused) loads
  // ---- dK, dV written once per key: lane (n, g), register i of tile ct <-> channel 16ct + 4g + i
  if (key < L) {
    if (HS == 1) {
      float* dkr = dk + (khead * L + key) * kD + 4 * g;
      float* dvr = dv + (khead * L + key) * kD + 4 * g;
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct) {
        *reinterpret_cast<v4f*>(dvr + 16 * ct) = accv[ct];
        *reinterpret_cast<v4f*>(dkr + 16 * ct) = sigma * acck[ct];
      }
    } else {
      // part hp: [B*Hkv][L][dV^T sums (128) | dK^T sums (128)], unscaled
      float* pr = part + (((int64_t)hp * nhb + khead) * L + key) * (2 * kD) + 4 * g;
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct) {
        *reinterpret_cast<v4f*>(pr + 16 * ct) = accv[ct];
        *reinterpret_cast<v4f*>(pr + kD + 16 * ct) = acck[ct];
      }
    }
  }
}

// dV = sum of the HS parts' dV^T sums, dK = sigma * sum of their dK^T sums, parts added in
// order 0, 1, ... (deterministic).  One thread per 4 channels of one key row.
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* __restrict__ part, float* __restrict__ dk,
                                                         float* __restrict__ dv, int64_t nrows, int HS,
                                                         float sigma) {
  const int64_t n4 = nrows * (kD / 4);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / (kD / 4);
    const int c = (int)(i % (kD / 4)) * 4;
    v4f sv = *reinterpret_cast<const v4f*>(part + row * (2 * kD) + c);
    v4f sk = *reinterpret_cast<const v4f*>(part + row * (2 * kD) + kD + c);
    for (int p = 1; p < HS; ++p) {
      const float* pr = part + ((int64_t)p * nrows + row) * (2 * kD);
      sv += *reinterpret_cast<const v4f*>(pr + c);
      sk += *reinterpret_cast<const v4f*>(pr + kD + c);
    }
    *reinterpret_cast<v4f*>(dv + row * kD + c) = sv;
    *reinterpret_cast<v4f*>(dk + row * kD + c) = sigma * sk;
  }
}

int dkdv_d128_head_split(const AttnDims& d) {
  // deal the heads of a KV group to more workgroups while the grid is under
  // kSplitTarget workgroups (four per CU of MI355X's 256; one workgroup of this
  // kernel's LDS size runs on a CU at a time).  The grid stays under 2 * kSplitTarget,
  // so the partial sums take under 2 * kSplitTarget * 128 KiB = 256 MiB.
  constexpr int64_t kSplitTarget = 1024;
  const int G = d.Hq / d.Hkv;
  const int64_t nwg = (int64_t)(d.Lp / kKT) * d.Hkv * d.B;
  int hs = 1;
  while (G % (2 * hs) == 0 && nwg * hs < kSplitTarget) hs *= 2;
  return hs;
}

int64_t dkdv_d128_workspace_bytes(const AttnDims& d, int hs) {
  return hs > 1 ? (int64_t)hs * d.B * d.Hkv * d.L * 2 * kD * (int64_t)sizeof(float) : 0;
}

hipError_t launch_dkdv_d128(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc,
                            Operand dos, const float* lse, const float* delta, float* dk, float* dv, double* ps,
                            double* pa, float* ws, int hs, hipStream_t s) {
  if (d.dqk != kD || d.dv != kD || d.Lp % kKT != 0 || (ps == nullptr) != (pa == nullptr)) return hipErrorInvalidValue;
  if (hs < 1 || (d.Hq / d.Hkv) % hs != 0 || (hs > 1 && (ws == nullptr || ps != nullptr))) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(d.Lp / kKT) * d.Hkv * d.B * hs);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kNT), 0, s, qc.codes, qc.scales, qs.codes, qs.scales, kc.codes, kc.scales,
                       vc.codes, vc.scales, doc.codes, doc.scales, dos.codes, dos.scales, lse, delta, dk, dv, ps, pa,
                       ws, hs, d.Hq, d.Hkv, d.L, d.Lp, d.sigma);
  };
  if (ps) {
    // the probe rows are sums over every key tile: start them from zero
    const int64_t bytes = (int64_t)d.B * d.Hq * d.L * (int64_t)sizeof(double);
    hipError_t e = launch_fill_zero(ps, bytes, s);
    if (e == hipSuccess) e = launch_fill_zero(pa, bytes, s);
    if (e != hipSuccess) return e;
    if (d.causal) go(dkdv_d128_kernel<true, true>);
    else go(dkdv_d128_kernel<false, true>);
  } else {
    if (d.causal) go(dkdv_d128_kernel<true, false>);
    else go(dkdv_d128_kernel<false, false>);
    if (hs > 1) {
      const int64_t nrows = (int64_t)d.B * d.Hkv * d.L;
      int64_t blocks = (nrows * (kD / 4) + 255) / 256;
      if (blocks > 4096) blocks = 4096;
      hipLaunchKernelGGL(dkdv_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ws, dk, dv, nrows, hs,
                         d.sigma);
    }
  }
  return hipGetLastError();
}

}  // namespace dm
