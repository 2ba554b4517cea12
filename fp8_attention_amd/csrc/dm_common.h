// Device helpers shared by the gfx950 kernels of libdm.
//
// Scaled FP8 matrix-core instruction (v_mfma_scale_f32_32x32x64_f8f6f4) lane
// layout, as used throughout (lane l, R = l % 32, h = l / 32):
//   A (32 x 64, row R): bytes 0..15 hold K-slots 16h+0..15 (K-block 0),
//                       bytes 16..31 hold K-slots 32+16h+0..15 (K-block 1);
//   B (64 x 32, col R): the same K-slot assignment;
//   the E8M0 scale of (row R, K-block kb) comes from lane R + 32*kb, i.e. lane
//   (R, h) supplies the scale of K-block h;
//   C (32 x 32): register v of lane l holds row 8*(v/4) + 4*h + v%4, column R.
// A K-block of 32 slots therefore spans the first (or second) 16 bytes of the
// two lanes R and R+32, and one 32-element quantization block maps onto one
// K-block when each lane of the pair holds 16 of its elements.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBlock = 32;     // elements per scale block
constexpr int kChunk = 128;    // keys per running-max update / tile length
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum Fmt : int { E4M3 = 0, E5M2 = 1 };

// Fmax = 1.75 * 2^emax_shift: 448 = 1.75*2^8 (E4M3), 57344 = 1.75*2^15 (E5M2).
template <int F> struct FmtTraits;
template <> struct FmtTraits<E4M3> { static constexpr int emax = 8; };
template <> struct FmtTraits<E5M2> { static constexpr int emax = 15; };

// Smallest integer k with amax <= Fmax * 2^k, clamped to [-126, 127].
// amax = 1.m * 2^e:  k = e - emax when 1.m <= 1.75, else e - emax + 1.
// amax == 0 or subnormal gives e = -127 and clamps to -126.
template <int F>
__device__ __forceinline__ int scale_exp(float amax) {
  uint32_t b = __float_as_uint(amax);
  int e = (int)((b >> 23) & 0xff) - 127;
  int k = e - FmtTraits<F>::emax + ((b & 0x7fffff) > 0x600000u ? 1 : 0);
  return min(max(k, -126), 127);
}

__device__ __forceinline__ float exp2i(int k) {        // 2^k, k in [-126, 127]
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

// Pack four floats (already divided by the block scale, |x| <= Fmax) into one
// dword of FP8 codes, byte i = code of x_i.  Round to nearest even.
template <int F>
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  uint32_t w;
  if constexpr (F == E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0u, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return w;
}

typedef short v2s __attribute__((ext_vector_type(2)));

// Same packing with the block scale applied by the convert itself:
// v_cvt_scalef32_pk_{fp8,bf8}_f32 rounds x / scale to nearest even (checked
// bit for bit against the format definitions), which saves the multiply.
template <int F>
__device__ __forceinline__ uint32_t pack4s(float a, float b, float c, float d, float scale) {
  // both halves are written below; starting from a's bits spares a register copy
  v2s w = __builtin_bit_cast(v2s, a);
  if constexpr (F == E4M3) {
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, scale, true);
  } else {
    w = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w, a, b, scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w, c, d, scale, true);
  }
  return __builtin_bit_cast(uint32_t, w);
}

// The other lane of a (l, l^32) pair: returns {x_lo_lane, x_hi_lane} ordered
// so that max/sum of the two gives the pair reduction on both lanes.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ double pair_sum_d(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const double a = __longlong_as_double(((uint64_t)rh[0] << 32) | rl[0]);
  const double b = __longlong_as_double(((uint64_t)rh[1] << 32) | rl[1]);
  return a + b;
}

template <int FA, int FB>
__device__ __forceinline__ v16f mfma(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

// 16x16x128 form: lane (n, g = l/16) holds row/column n; its bytes 0-15 are
// K-slots 16g..16g+15 and bytes 16-31 K-slots 64+16g..64+16g+15, and it supplies
// the scale of K-block g (slots 32g..32g+31).  Result register i of lane (n, g)
// is row 4g+i, column n.
template <int FA, int FB>
__device__ __forceinline__ v4f mfma16(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

// Maximum over the lane pair (l, l^16).
__device__ __forceinline__ float pair16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum of the 16 accumulator values of one lane (max3 chain).
__device__ __forceinline__ float max16(const v16f& x) {
  float m = fmaxf(fmaxf(x[0], x[1]), x[2]);
#pragma unroll
  for (int v = 3; v < 15; v += 2) m = fmaxf(fmaxf(m, x[v]), x[v + 1]);
  return fmaxf(m, x[15]);
}

// Sum of x[0..NV) over each group of W consecutive lanes, scattered: afterwards the
// lane with (lane % NV) == k holds the group's sum of x[k] (every value of x is
// overwritten).  A reduce-scatter butterfly: log2(W / NV) full exchanges, then one
// halving exchange per remaining lane bit, NV - 1 shuffles in all.
template <int NV, int W>
__device__ __forceinline__ float group_sum_scatter(float (&x)[NV], int lane) {
  static_assert(NV >= 1 && NV <= W && (NV & (NV - 1)) == 0 && (W & (W - 1)) == 0 && W <= 64, "powers of two");
#pragma unroll
  for (int m = W / 2; m >= NV; m >>= 1)
#pragma unroll
    for (int j = 0; j < NV; ++j) x[j] += __shfl_xor(x[j], m, W);
#pragma unroll
  for (int m = NV / 2; m >= 1; m >>= 1) {
    const bool hi = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < m; ++j) {
      const float send = hi ? x[j] : x[j + m];
      const float keep = hi ? x[j + m] : x[j];
      x[j] = keep + __shfl_xor(send, m, W);
    }
  }
  return x[0];
}

// E8M0 byte of a float32 power-of-two scale (its biased exponent).
__device__ __forceinline__ int e8m0(float s) { return (int)(__float_as_uint(s) >> 23); }

// Row index (within a 32-row MFMA tile) of the operand row that should hold
// element 16*h + v of the lane pair (R, R+32) after the product: a C-layout
// row 8a + 4b + c is loaded from element 16b + 4a + c.
__device__ __forceinline__ int pair_row(int r) {
  return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

__device__ __forceinline__ v8i cat(const v4i& lo, const v4i& hi) {
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

__device__ __forceinline__ v4i lds_read16(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// ---------------------------------------------------------------------------
// LDS tiles filled by direct global->LDS loads (global_load_lds_dwordx4: lane l
// of one instruction writes 16 bytes at LDS base + 16*l, from its own global
// address).  The 16-byte chunks of each tile row are XOR-permuted by a function
// of the row index so that the matrix-operand reads (16 bytes per lane, rows in
// pair_row order or natural order) run at full LDS rate.  The permutations were
// chosen by timing ds_read_b128 on gfx950 for these access patterns; the plain
// layout of a 128-byte-row tile runs several times slower.
// ---------------------------------------------------------------------------
// Slot (16-byte position within the row) of logical chunk c of tile row `row`,
// for rows of RB bytes.  Each map is an involution on the row's chunks.
template <int RB>
__device__ __forceinline__ int tile_slot(int row, int c) {
  if constexpr (RB == 128) {
    return c ^ ((row >> 1) & 7);
  } else if constexpr (RB == 64) {
    return c ^ ((row >> 2) & 3);
  } else if constexpr (RB == 256) {
    // a row spans all 64 banks; XOR with a 4-bit function of the row that takes 16
    // distinct values on any 16 rows read together, in natural or pair_row order
    return c ^ ((row & 15) ^ (((row >> 4) & 1) << 3));
  } else {
    static_assert(RB == 192, "tile rows of 64, 128, 192 or 256 bytes");
    const int f = ((row >> 2) & 1) | (((row ^ (row >> 3)) & 1) << 1);
    return c < 8 ? (c ^ f) : 8 + ((c - 8) ^ f);
  }
}

// Work item (query-tile rank tr, query head hq, batch b) of workgroup bid in a 1-D
// grid of nqt * Hq * nb query-stationary workgroups.  Workgroups are dealt to the
// 8 XCDs in turn (bid % 8), each with its own L2: when the (batch, KV group) units
// divide evenly, XCD x takes whole units, one after another, so the query heads
// that share a K/V stream and all their query tiles run behind one L2.  Within a
// unit tr runs fastest over the heads and slowest over tiles, so with tr mapped to
// the longest causal tiles first the long work starts early.
struct QueryItem {
  int tr, hq, b;
};
__device__ __forceinline__ QueryItem query_item(int bid, int nqt, int Hq, int Hkv, int nb) {
  const int G = Hq / Hkv, NG = nb * Hkv;
  if (NG % 8 == 0) {
    const int per = G * nqt;                   // workgroups of one (batch, KV group)
    const int s = bid / 8, gi = (bid % 8) * (NG / 8) + s / per, r = s % per;
    return {r / G, (gi % Hkv) * G + r % G, gi / Hkv};
  }
  const int nhb = Hq * nb;
  return {bid / nhb, bid % nhb % Hq, bid % nhb / Hq};
}

typedef __attribute__((address_space(3))) void lds_void;
// One 16-byte-per-lane direct load to the LDS byte address lds_addr (wave-uniform).
__device__ __forceinline__ void dma16_at(const void* g, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}
// Issued from inline assembly rather than __builtin_amdgcn_global_load_lds: with the
// builtin in a kernel the compiler turns every LDS wait into lgkmcnt(0), so reads
// prefetched for the next tile are waited for together with the current ones.  The
// hardware tracks these loads with VM_CNT only; every kernel waits for them
// explicitly (wait_vmem) before the barrier that publishes a buffer.  M0 (the LDS
// address) is an operand bound to that register, so the compiler writes it; the
// nop is the wait state required between the M0 write and the load that uses it.
__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_base) {
  dma16_at(g, (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds_base));
}
// The same load in the SADDR form: a wave-uniform 64-bit base (SGPRs) plus a
// 32-bit unsigned per-lane byte offset, so a loop that keeps its per-lane offsets
// spends no vector instructions on addresses; with a wave-uniform LDS destination
// the M0 write is scalar too.  A vector instruction that writes an SGPR (a lane
// read) needs five wait states before a memory instruction reads that SGPR, and
// the compiler cannot see that the assembly reads its base, so the nop provides
// them whatever instruction wrote the base or M0 last.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint8_t* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds_base));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(m0) : "memory");
}
// wait for this wave's outstanding global loads (including direct-to-LDS ones)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace dm
