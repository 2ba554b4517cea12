// C ABI of libdm: argument validation (pure host code, no HIP call before it
// passes) and dispatch to the kernel launchers; the fixed scratch of the
// allocation-free dK/dV call.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "dm_attn.h"
#include "dm_internal.h"

// Scratch of dm_attn_bwd_dkdv_noalloc: the head split's partial sums, for callers that
// cannot allocate.  Each device the library runs on holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol); it uses the device address hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[DM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device; null until the first call on that device

// The device address of the current device's scratch, looked up once per device (with
// that device current).  Null on failure.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dm_status check_shape(const dm_attn_shape* s) {
  if (!s) return DM_ERR_NULL;
  if (s->batch < 1 || s->heads_q < 1 || s->heads_kv < 1 || s->seqlen < 0) return DM_ERR_SHAPE;
  // per-lane load offsets within one head are 32-bit (up to 128 rows of Lp bytes)
  if (s->batch > 65535 || s->heads_q > 65535 || s->seqlen > DM_MAX_SEQLEN) return DM_ERR_SHAPE;
  if (s->heads_q % s->heads_kv != 0) return DM_ERR_SHAPE;
  // every kernel grid is one-dimensional over (sequence tile of 128, head, batch)
  if ((int64_t)s->batch * s->heads_q * ((s->seqlen + 127) / 128) > INT32_MAX) return DM_ERR_SHAPE;
  // d_qk in {64, 128, 192} with d_v in {64, 128}, or d_qk = d_v = 256
  const bool wide = s->d_qk == 256 && s->d_v == 256;
  if (!wide && s->d_qk != 64 && s->d_qk != 128 && s->d_qk != 192) return DM_ERR_SHAPE;
  if (!wide && s->d_v != 64 && s->d_v != 128) return DM_ERR_SHAPE;
  if (s->causal != 0 && s->causal != 1) return DM_ERR_SHAPE;
  if (!(s->softmax_scale > 0.f) || !isfinite(s->softmax_scale)) return DM_ERR_SHAPE;
  return DM_OK;
}

dm_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return DM_ERR_NULL;
  for (const void* p : ps)
    if (!aligned16(p)) return DM_ERR_ALIGN;
  return DM_OK;
}

dm_status check_operand(const dm_fp8_operand& op) { return check_ptrs({op.codes, op.scales}); }

dm::AttnDims dims_of(const dm_attn_shape* s) {
  dm::AttnDims d;
  d.B = s->batch;
  d.Hq = s->heads_q;
  d.Hkv = s->heads_kv;
  d.L = s->seqlen;
  d.Lp = (int)dm_padded_len(s->seqlen);
  d.dqk = s->d_qk;
  d.dv = s->d_v;
  d.causal = s->causal;
  d.sigma = s->softmax_scale;
  return d;
}

dm::Operand op(const dm_fp8_operand& o) { return dm::Operand{o.codes, o.scales}; }

dm_status hip_status(hipError_t e) { return e == hipSuccess ? DM_OK : DM_ERR_HIP; }

}  // namespace

extern "C" {

int64_t dm_padded_len(int64_t L) {
  if (L < 0) return -1;
  return (L + 127) / 128 * 128;
}

const char* dm_status_string(dm_status s) {
  switch (s) {
    case DM_OK: return "DM_OK";
    case DM_ERR_NULL: return "DM_ERR_NULL: a required pointer is NULL";
    case DM_ERR_SHAPE: return "DM_ERR_SHAPE: unsupported or inconsistent sizes";
    case DM_ERR_ALIGN: return "DM_ERR_ALIGN: a pointer is not 16-byte aligned";
    case DM_ERR_ENUM: return "DM_ERR_ENUM: an enum argument is out of range";
    case DM_ERR_HIP: return "DM_ERR_HIP: the HIP runtime reported an error";
    case DM_ERR_WORKSPACE:
      return "DM_ERR_WORKSPACE: the workspace (or the fixed scratch of the allocation-free call) is smaller than "
             "this shape needs";
  }
  return "unknown dm_status";
}

dm_status dm_quantize_blockfp8(const void* x, dm_dtype dtype, int64_t batch, int64_t rows, int64_t cols,
                               int64_t rows_out, dm_block_axis axis, dm_fp8_format fmt, uint8_t* codes,
                               float* scales, hipStream_t stream) {
  if ((int)dtype != DM_BF16 && (int)dtype != DM_F32) return DM_ERR_ENUM;
  if ((int)axis != DM_AXIS_COLS && (int)axis != DM_AXIS_ROWS) return DM_ERR_ENUM;
  if ((int)fmt != DM_E4M3 && (int)fmt != DM_E5M2) return DM_ERR_ENUM;
  if (batch < 1 || rows < 0 || cols < 32 || cols % 32 != 0 || rows_out < rows) return DM_ERR_SHAPE;
  if (batch > 65535 || rows_out > ((int64_t)1 << 36) || cols > (1 << 20)) return DM_ERR_SHAPE;
  if (axis == DM_AXIS_ROWS && rows_out % 32 != 0) return DM_ERR_SHAPE;
  dm_status st = check_ptrs({x, codes, scales});
  if (st != DM_OK) return st;
  if (rows_out == 0) return DM_OK;
  return hip_status(dm::launch_quantize(x, (int)dtype, batch, rows, cols, rows_out, (int)axis, (int)fmt, codes,
                                        scales, stream));
}

dm_status dm_attn_fwd(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand k_c, dm_fp8_operand v_s,
                      float* o, float* lse, hipStream_t stream) {
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  if ((st = check_operand(q_c)) != DM_OK || (st = check_operand(k_c)) != DM_OK ||
      (st = check_operand(v_s)) != DM_OK || (st = check_ptrs({o, lse})) != DM_OK)
    return st;
  if (shape->seqlen == 0) return DM_OK;
  return hip_status(dm::launch_fwd(dims_of(shape), op(q_c), op(k_c), op(v_s), o, lse, stream));
}

dm_status dm_attn_delta(const dm_attn_shape* shape, dm_delta_mode mode, const float* o, const uint16_t* do_bf16,
                        dm_fp8_operand do_c, dm_fp8_operand q_c, dm_fp8_operand k_c, dm_fp8_operand v_c,
                        const float* lse, float* delta, hipStream_t stream) {
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  if ((int)mode != DM_DELTA_STALE && (int)mode != DM_DELTA_DO_MATCHED && (int)mode != DM_DELTA_MATCHED)
    return DM_ERR_ENUM;
  if ((st = check_ptrs({delta})) != DM_OK) return st;
  if (mode == DM_DELTA_STALE) {
    if ((st = check_ptrs({o, do_bf16})) != DM_OK) return st;
  } else if (mode == DM_DELTA_DO_MATCHED) {
    if ((st = check_ptrs({o})) != DM_OK || (st = check_operand(do_c)) != DM_OK) return st;
  } else {
    if ((st = check_operand(do_c)) != DM_OK || (st = check_operand(q_c)) != DM_OK ||
        (st = check_operand(k_c)) != DM_OK || (st = check_operand(v_c)) != DM_OK ||
        (st = check_ptrs({lse})) != DM_OK)
      return st;
  }
  if (shape->seqlen == 0) return DM_OK;
  const dm::AttnDims d = dims_of(shape);
  if (mode == DM_DELTA_MATCHED)
    return hip_status(dm::launch_delta_matched(d, op(do_c), op(q_c), op(k_c), op(v_c), lse, delta, stream));
  return hip_status(dm::launch_delta_rows(d, (int)mode, o, do_bf16, op(do_c), delta, stream));
}

dm_status dm_attn_bwd(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s, dm_fp8_operand k_c,
                      dm_fp8_operand k_s, dm_fp8_operand v_c, dm_fp8_operand do_c, dm_fp8_operand do_s,
                      const float* lse, const float* delta, float* dq, float* dk, float* dv,
                      double* probe_rowsum_ds, double* probe_rowsum_abs_pdp, hipStream_t stream) {
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  const dm_fp8_operand ops[7] = {q_c, q_s, k_c, k_s, v_c, do_c, do_s};
  for (const auto& x : ops)
    if ((st = check_operand(x)) != DM_OK) return st;
  if ((st = check_ptrs({lse, delta, dq, dk, dv})) != DM_OK) return st;
  if ((probe_rowsum_ds == nullptr) != (probe_rowsum_abs_pdp == nullptr)) return DM_ERR_NULL;
  if (probe_rowsum_ds && (st = check_ptrs({probe_rowsum_ds, probe_rowsum_abs_pdp})) != DM_OK) return st;
  if (shape->seqlen == 0) return DM_OK;
  return hip_status(dm::launch_bwd(dims_of(shape), op(q_c), op(q_s), op(k_c), op(k_s), op(v_c), op(do_c),
                                   op(do_s), lse, delta, dq, dk, dv, probe_rowsum_ds, probe_rowsum_abs_pdp, stream));
}

dm_status dm_attn_bwd_dkdv(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s, dm_fp8_operand k_c,
                           dm_fp8_operand v_c, dm_fp8_operand do_c, dm_fp8_operand do_s, const float* lse,
                           const float* delta, float* dk, float* dv, hipStream_t stream) {
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  const dm_fp8_operand ops[6] = {q_c, q_s, k_c, v_c, do_c, do_s};
  for (const auto& x : ops)
    if ((st = check_operand(x)) != DM_OK) return st;
  if ((st = check_ptrs({lse, delta, dk, dv})) != DM_OK) return st;
  if (shape->seqlen == 0) return DM_OK;
  return hip_status(dm::launch_dkdv(dims_of(shape), op(q_c), op(q_s), op(k_c), op(v_c), op(do_c), op(do_s), lse,
                                    delta, dk, dv, nullptr, nullptr, stream));
}

dm_status dm_attn_bwd_dkdv_workspace_size(const dm_attn_shape* shape, int64_t* bytes) {
  if (bytes == nullptr) return DM_ERR_NULL;
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  const dm::AttnDims d = dims_of(shape);
  *bytes = shape->seqlen == 0 ? 0 : dm::dkdv_d128_workspace_bytes(d, dm::dkdv_head_split(d));
  return DM_OK;
}

dm_status dm_attn_bwd_dkdv_ws(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s, dm_fp8_operand k_c,
                              dm_fp8_operand v_c, dm_fp8_operand do_c, dm_fp8_operand do_s, const float* lse,
                              const float* delta, float* dk, float* dv, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream) {
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  const dm_fp8_operand ops[6] = {q_c, q_s, k_c, v_c, do_c, do_s};
  for (const auto& x : ops)
    if ((st = check_operand(x)) != DM_OK) return st;
  if ((st = check_ptrs({lse, delta, dk, dv})) != DM_OK) return st;
  if (shape->seqlen == 0) return DM_OK;
  const dm::AttnDims d = dims_of(shape);
  const int64_t need = dm::dkdv_d128_workspace_bytes(d, dm::dkdv_head_split(d));
  if (need > 0) {
    if (workspace == nullptr) return DM_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return DM_ERR_ALIGN;
    if (workspace_bytes < need) return DM_ERR_WORKSPACE;
  }
  return hip_status(dm::launch_dkdv_split(d, op(q_c), op(q_s), op(k_c), op(v_c), op(do_c), op(do_s), lse, delta, dk,
                                          dv, static_cast<float*>(workspace), stream));
}

dm_status dm_attn_bwd_dkdv_noalloc(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s,
                                   dm_fp8_operand k_c, dm_fp8_operand v_c, dm_fp8_operand do_c, dm_fp8_operand do_s,
                                   const float* lse, const float* delta, float* dk, float* dv, hipStream_t stream) {
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  const dm_fp8_operand ops[6] = {q_c, q_s, k_c, v_c, do_c, do_s};
  for (const auto& x : ops)
    if ((st = check_operand(x)) != DM_OK) return st;
  if ((st = check_ptrs({lse, delta, dk, dv})) != DM_OK) return st;
  if (shape->seqlen == 0) return DM_OK;
  const dm::AttnDims d = dims_of(shape);
  const int64_t need = dm::dkdv_d128_workspace_bytes(d, dm::dkdv_head_split(d));
  if (need > (int64_t)DM_NOALLOC_SCRATCH_BYTES) return DM_ERR_WORKSPACE;
  float* ws = nullptr;
  if (need > 0) {
    ws = static_cast<float*>(device_scratch());
    if (ws == nullptr) return DM_ERR_HIP;
  }
  return hip_status(dm::launch_dkdv_split(d, op(q_c), op(q_s), op(k_c), op(v_c), op(do_c), op(do_s), lse, delta, dk,
                                          dv, ws, stream));
}

dm_status dm_attn_bwd_dkdv_probes(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s,
                                  dm_fp8_operand k_c, dm_fp8_operand v_c, dm_fp8_operand do_c, dm_fp8_operand do_s,
                                  const float* lse, const float* delta, float* dk, float* dv, double* probe_rowsum_ds,
                                  double* probe_rowsum_abs_pdp, hipStream_t stream) {
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  const dm_fp8_operand ops[6] = {q_c, q_s, k_c, v_c, do_c, do_s};
  for (const auto& x : ops)
    if ((st = check_operand(x)) != DM_OK) return st;
  if ((st = check_ptrs({lse, delta, dk, dv, probe_rowsum_ds, probe_rowsum_abs_pdp})) != DM_OK) return st;
  if (shape->seqlen == 0) return DM_OK;
  return hip_status(dm::launch_dkdv(dims_of(shape), op(q_c), op(q_s), op(k_c), op(v_c), op(do_c), op(do_s), lse,
                                    delta, dk, dv, probe_rowsum_ds, probe_rowsum_abs_pdp, stream));
}

dm_status dm_attn_bwd_dq(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand k_c, dm_fp8_operand k_s,
                         dm_fp8_operand v_c, dm_fp8_operand do_c, const float* lse, const float* delta, float* dq,
                         double* probe_rowsum_ds, double* probe_rowsum_abs_pdp, hipStream_t stream) {
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  const dm_fp8_operand ops[5] = {q_c, k_c, k_s, v_c, do_c};
  for (const auto& x : ops)
    if ((st = check_operand(x)) != DM_OK) return st;
  if ((st = check_ptrs({lse, delta, dq})) != DM_OK) return st;
  if ((probe_rowsum_ds == nullptr) != (probe_rowsum_abs_pdp == nullptr)) return DM_ERR_NULL;
  if (probe_rowsum_ds && (st = check_ptrs({probe_rowsum_ds, probe_rowsum_abs_pdp})) != DM_OK) return st;
  if (shape->seqlen == 0) return DM_OK;
  return hip_status(dm::launch_dq(dims_of(shape), op(q_c), op(k_c), op(k_s), op(v_c), op(do_c), lse, delta, dq,
                                  probe_rowsum_ds, probe_rowsum_abs_pdp, nullptr, stream));
}

dm_status dm_attn_bwd_dq_probes(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand k_c,
                                dm_fp8_operand k_s, dm_fp8_operand v_c, dm_fp8_operand do_c, const float* lse,
                                const float* delta, float* dq, double* probe_rowsum_ds, double* probe_rowsum_abs_pdp,
                                double* probe_rowsum_ds_cast, hipStream_t stream) {
  dm_status st = check_shape(shape);
  if (st != DM_OK) return st;
  const dm_fp8_operand ops[5] = {q_c, k_c, k_s, v_c, do_c};
  for (const auto& x : ops)
    if ((st = check_operand(x)) != DM_OK) return st;
  if ((st = check_ptrs({lse, delta, dq, probe_rowsum_ds, probe_rowsum_abs_pdp, probe_rowsum_ds_cast})) != DM_OK)
    return st;
  if (shape->seqlen == 0) return DM_OK;
  return hip_status(dm::launch_dq(dims_of(shape), op(q_c), op(k_c), op(k_s), op(v_c), op(do_c), lse, delta, dq,
                                  probe_rowsum_ds, probe_rowsum_abs_pdp, probe_rowsum_ds_cast, stream));
}

}  // extern "C"
