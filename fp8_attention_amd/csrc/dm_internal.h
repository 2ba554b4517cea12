// Internal launcher declarations shared by the API translation unit and the
// kernel translation units of libdm.  Shapes reaching these functions have
// already been validated by the API layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dm {

struct AttnDims {
  int B, Hq, Hkv, L, Lp, dqk, dv, causal;
  float sigma;
};

struct Operand {
  const uint8_t* codes;
  const float* scales;
};

hipError_t launch_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols, int64_t rows_out,
                           int axis, int fmt, uint8_t* codes, float* scales, hipStream_t s);

hipError_t launch_fwd(const AttnDims& d, Operand q_c, Operand k_c, Operand v_s, float* o, float* lse, hipStream_t s);

hipError_t launch_delta_rows(const AttnDims& d, int mode, const float* o, const uint16_t* do_bf16, Operand do_c,
                             float* delta, hipStream_t s);
hipError_t launch_delta_matched(const AttnDims& d, Operand do_c, Operand q_c, Operand k_c, Operand v_c,
                                const float* lse, float* delta, hipStream_t s);

hipError_t launch_bwd(const AttnDims& d, Operand q_c, Operand q_s, Operand k_c, Operand k_s, Operand v_c,
                      Operand do_c, Operand do_s, const float* lse, const float* delta, float* dq, float* dk,
                      float* dv, double* probe_sum, double* probe_abs, hipStream_t s);

// ps, pa: the dK/dV kernel's row-sum probes (pre-cast sum of dS, sum of |P dP^|), both
// null or both set; they are zeroed and then accumulated over key tiles
hipError_t launch_dkdv(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc, Operand dos,
                       const float* lse, const float* delta, float* dk, float* dv, double* ps, double* pa,
                       hipStream_t s);

// d_qk = d_v = 128 form of launch_dkdv (attn_dkdv128.hip).  hs > 1 deals the query heads of
// each KV group to hs workgroups per key tile, with their partial sums in ws
// (dkdv_d128_workspace_bytes(d, hs) bytes) and a reduction kernel after; hs must divide
// Hq / Hkv and excludes the probes.
hipError_t launch_dkdv_d128(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc,
                            Operand dos, const float* lse, const float* delta, float* dk, float* dv, double* ps,
                            double* pa, float* ws, int hs, hipStream_t s);
// head split the d = 128 kernel takes for a shape (1: none) and its workspace bytes
int dkdv_d128_head_split(const AttnDims& d);
int64_t dkdv_d128_workspace_bytes(const AttnDims& d, int hs);
// the head split launch_dkdv_split uses for d (1 for head dims without a split form)
int dkdv_head_split(const AttnDims& d);
// launch_dkdv with the head split dkdv_head_split(d) and its partial sums in ws
// (dkdv_d128_workspace_bytes(d, dkdv_head_split(d)) bytes; may be null when that is 0)
hipError_t launch_dkdv_split(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc,
                             Operand dos, const float* lse, const float* delta, float* dk, float* dv, float* ws,
                             hipStream_t s);
// d_qk = d_v = 256 form of launch_dkdv (attn_dkdv_wide.hip)
hipError_t launch_dkdv_256_256(const AttnDims& d, Operand qc, Operand qs, Operand kc, Operand vc, Operand doc,
                               Operand dos, const float* lse, const float* delta, float* dk, float* dv, double* ps,
                               double* pa, hipStream_t s);

// ps, pa, pc: the row-sum probes (pre-cast sum of dS, sum of |P dP^|, sum of the
// decoded dS^<k>); ps and pa both null or both set, pc only with them
hipError_t launch_dq(const AttnDims& d, Operand qc, Operand kc, Operand ks, Operand vc, Operand doc,
                     const float* lse, const float* delta, float* dq, double* ps, double* pa, double* pc,
                     hipStream_t s);

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t s);

}  // namespace dm
