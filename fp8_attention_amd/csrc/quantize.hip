// Block-scaled FP8 quantization (bf16/f32 -> E4M3/E5M2 codes + float32 power-of-two
// scales, one per 32 elements).  Bound by HBM bandwidth: every input byte is read
// once and every code/scale written once, with 16-byte accesses.
#include "dm_common.h"
#include "dm_internal.h"

namespace dm {

template <typename T> __device__ __forceinline__ void load8(const T* p, float* v);
template <> __device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  v4i w = *reinterpret_cast<const v4i*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float((uint32_t)w[i] << 16);
    v[2 * i + 1] = __uint_as_float((uint32_t)w[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float* v) {
  v4f a = *reinterpret_cast<const v4f*>(p);
  v4f b = *reinterpret_cast<const v4f*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

__device__ __forceinline__ float quad_max(float x) {
  // max over the 4 consecutive lanes of a quad (DPP quad_perm [1,0,3,2] then [2,3,0,1])
  float y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x = fmaxf(x, y);
  y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  return fmaxf(x, y);
}

// Blocks along the contiguous axis.  Four lanes share a 32-element block, eight
// elements each.  Grid-stride over groups of 8 elements of the padded output.
template <typename T, int F>
__global__ __launch_bounds__(256) void quantize_cols_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                            int64_t rows_out, int64_t n8, uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // every lane of a quad walks the same sequence of blocks, so the DPP partners exist
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g - (threadIdx.x & 3) < n8; g += stride) {
    const bool live = g < n8;
    const int64_t e0 = g * 8;                      // element index in the padded output
    const int64_t c = e0 % cols;
    const int64_t r = (e0 / cols) % rows_out;
    const int64_t b = e0 / (cols * rows_out);
    float v[8];
    if (live && r < rows) {
      load8<T>(x + (b * rows + r) * cols + c, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
    am = quad_max(am);
    const int k = scale_exp<F>(am);
    const float inv = exp2i(-k);                   // exact; keeps subnormal inputs exact too
    uint32_t w0 = pack4<F>(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    uint32_t w1 = pack4<F>(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    if (live) {
      uint2 o;
      o.x = w0;
      o.y = w1;
      *reinterpret_cast<uint2*>(codes + e0) = o;
      if ((threadIdx.x & 3) == 0) scales[e0 / kBlock] = exp2i(k);
    }
  }
}

// Blocks along rows, output transposed.  A workgroup takes a tile of 128 rows x
// 64 columns, stages it in LDS as float (column-major), then each of the 256
// threads quantizes one (column, 32-row block) and writes 32 contiguous codes.
// Row index bits 3-5 are XORed with bits 3-5 of the column: the eight lanes that
// stage one row (columns 8 apart) then write eight different bank groups, and each
// column's rows stay in contiguous 8-float chunks for the 16-byte reads.
constexpr int kTR = 128, kTC = 64;
__device__ __forceinline__ int tile_pos(int col, int row) { return col * kTR + (row ^ (col & 0x38)); }

template <typename T, int F>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                            int64_t rows_out, uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
  __shared__ float tile[kTC * kTR];
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.x * kTR;
  const int64_t c0 = (int64_t)blockIdx.y * kTC;
  const int t = threadIdx.x;
  // load: 128 rows x 64 cols = 1024 groups of 8 columns; 4 passes of 256 threads
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int gi = p * 256 + t;
    const int rr = gi >> 3;          // 0..127
    const int cc = (gi & 7) * 8;     // 0..56
    float v[8];
    const int64_t r = r0 + rr, c = c0 + cc;
    if (r < rows && c < cols) {
      load8<T>(x + (b * rows + r) * cols + c, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[tile_pos(cc + i, rr)] = v[i];
  }
  __syncthreads();
  const int cc = t >> 2, blk = t & 3;
  const int64_t c = c0 + cc;
  const int64_t r = r0 + blk * kBlock;
  if (c >= cols || r >= rows_out) return;
  float v[32];
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    v4f q = *reinterpret_cast<const v4f*>(tile + tile_pos(cc, blk * kBlock + i));
    v[i] = q[0]; v[i + 1] = q[1]; v[i + 2] = q[2]; v[i + 3] = q[3];
    am = fmaxf(am, fmaxf(fmaxf(fabsf(q[0]), fabsf(q[1])), fmaxf(fabsf(q[2]), fabsf(q[3]))));
  }
  const int k = scale_exp<F>(am);
  const float inv = exp2i(-k);                     // exact; keeps subnormal inputs exact too
  v4i o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0[i] = (int)pack4<F>(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
    o1[i] = (int)pack4<F>(v[16 + 4 * i] * inv, v[17 + 4 * i] * inv, v[18 + 4 * i] * inv, v[19 + 4 * i] * inv);
  }
  uint8_t* dst = codes + (b * cols + c) * rows_out + r;
  *reinterpret_cast<v4i*>(dst) = o0;
  *reinterpret_cast<v4i*>(dst + 16) = o1;
  scales[(b * cols + c) * (rows_out / kBlock) + r / kBlock] = exp2i(k);
}

template <typename T, int F>
static hipError_t launch_quantize_t(const void* x, int64_t batch, int64_t rows, int64_t cols, int64_t rows_out,
                                    int axis, uint8_t* codes, float* scales, hipStream_t s) {
  if (axis == 0) {
    const int64_t n8 = batch * rows_out * cols / 8;
    int64_t blocks = (n8 + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((quantize_cols_kernel<T, F>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const T*>(x), rows, cols, rows_out, n8, codes, scales);
  } else {
    dim3 grid((unsigned)((rows_out + kTR - 1) / kTR), (unsigned)((cols + kTC - 1) / kTC), (unsigned)batch);
    hipLaunchKernelGGL((quantize_rows_kernel<T, F>), grid, dim3(256), 0, s, static_cast<const T*>(x), rows, cols,
                       rows_out, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols, int64_t rows_out,
                           int axis, int fmt, uint8_t* codes, float* scales, hipStream_t s) {
  if (dtype == 0) {
    return fmt == 0 ? launch_quantize_t<uint16_t, E4M3>(x, batch, rows, cols, rows_out, axis, codes, scales, s)
                    : launch_quantize_t<uint16_t, E5M2>(x, batch, rows, cols, rows_out, axis, codes, scales, s);
  }
  return fmt == 0 ? launch_quantize_t<float, E4M3>(x, batch, rows, cols, rows_out, axis, codes, scales, s)
                  : launch_quantize_t<float, E5M2>(x, batch, rows, cols, rows_out, axis, codes, scales, s);
}

}  // namespace dm
