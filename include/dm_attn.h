/*
 * dm_attn.h -- C ABI of the block-scaled FP8 attention library (libdm) for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes FlashAttention-style attention forward and backward
 * with every matmul on FP8 operands carrying one power-of-two scale per 32
 * elements of the contraction axis, and the softmax row correction delta in
 * the three forms discussed on the Delta-Matching project page ("Delta-
 * Matching for reliable FP8 attention training"):
 *   stale       delta_i = sum_k dO_ik O_ik      (section 01, "What changes in
 *               FP8?": the saved-output shortcut with dO before its cast);
 *   dO-matched  delta_i = sum_k dO^_ik O_ik     (section 03, the variant that
 *               matches only dO);
 *   matched     delta_i = sum_j P_ij dP^_ij     (section 03, Delta-Matching:
 *               P the FP32 softmax, dP^ the FP32 product of the FP8 operands).
 *
 * Conventions shared by every call
 * --------------------------------
 * - All pointers are device pointers, except the dm_attn_shape pointer, which
 *   is a host pointer read before the call returns.  The caller allocates and
 *   owns every buffer; the library allocates nothing and keeps no pointer
 *   after a call returns.  (The one exception is the fixed device scratch of
 *   dm_attn_bwd_dkdv_noalloc, a static array of DM_NOALLOC_SCRATCH_BYTES on
 *   each device, and its per-device address kept from the first such call.)
 * - Every call only enqueues work on `stream` and returns.  The status covers
 *   host-side argument checks and the launch itself (hipGetLastError); a
 *   device-side fault surfaces at the caller's next synchronisation.
 * - A call that returns an error enqueues nothing.
 * - Logical layouts are row-major.  B = batch, Hq / Hkv = query / KV heads,
 *   L = sequence length, Lp = dm_padded_len(L) (L rounded up to 128).
 * - FP8 codes are OCP E4M3FN (DM_E4M3) or OCP E5M2 (DM_E5M2) bytes.  Scales
 *   are float32 powers of two, one per 32 codes along the contraction axis of
 *   the matmul the operand feeds.  The scale of a block is 2^k with the
 *   smallest integer k such that amax <= Fmax * 2^k (Fmax = 448 for E4M3,
 *   57344 for E5M2), k clamped to [-126, 127]; codes are x / 2^k rounded to
 *   nearest, ties to even.  An all-zero block has scale 2^-126.
 * - Operand naming: X<c> is X quantized in blocks along its channel axis,
 *   codes [B][H][Lp][d], scales [B][H][Lp][d/32].  X<s> is X quantized in
 *   blocks along the sequence axis and stored transposed so blocks are
 *   contiguous: codes [B][H][d][Lp], scales [B][H][d][Lp/32].  Positions at
 *   or beyond L hold zero codes (dm_quantize_blockfp8 writes them).
 * - Formats per operand: Q, K, V and the probabilities in E4M3; dO and dS in
 *   E5M2.
 * - Supported head dims: d_qk in {64, 128, 192} with d_v in {64, 128}, and
 *   d_qk = d_v = 256 (the head geometry of the larger models of the
 *   Delta-Matching page, section 04 "What changes as the model gets larger?").
 *   Other pairs return DM_ERR_SHAPE.
 *   Hq must be a multiple of Hkv (GQA: query head h reads KV head h/(Hq/Hkv)).
 *   softmax_scale must be positive and finite.  B, Hq, Hkv >= 1 and
 *   0 <= L <= DM_MAX_SEQLEN (the kernels address up to 128 rows of one head's
 *   sequence-major operand with 32-bit offsets); L == 0 is a no-op.
 * - Pointers must be 16-byte aligned (DM_ERR_ALIGN otherwise).
 * - Calls are reentrant; apart from that scratch the library has no global
 *   state.
 */
#ifndef DM_ATTN_H
#define DM_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest supported sequence length (2^24). */
#define DM_MAX_SEQLEN (1 << 24)

/* Size of the fixed per-device scratch of dm_attn_bwd_dkdv_noalloc (128 MiB). */
#define DM_NOALLOC_SCRATCH_BYTES (128u << 20)

typedef enum {
  DM_OK = 0,
  DM_ERR_NULL = 1,   /* a required pointer is NULL */
  DM_ERR_SHAPE = 2,  /* unsupported or inconsistent sizes */
  DM_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned */
  DM_ERR_ENUM = 4,   /* an enum argument is out of range */
  DM_ERR_HIP = 5,    /* the HIP runtime reported an error at launch */
  DM_ERR_WORKSPACE = 6 /* a workspace is smaller than the shape needs */
} dm_status;

typedef enum { DM_E4M3 = 0, DM_E5M2 = 1 } dm_fp8_format;
typedef enum { DM_BF16 = 0, DM_F32 = 1 } dm_dtype;
typedef enum { DM_AXIS_COLS = 0, DM_AXIS_ROWS = 1 } dm_block_axis;
typedef enum { DM_DELTA_STALE = 0, DM_DELTA_DO_MATCHED = 1, DM_DELTA_MATCHED = 2 } dm_delta_mode;

/* One FP8 operand: codes and their float32 block scales (device pointers). */
typedef struct {
  const uint8_t* codes;
  const float* scales;
} dm_fp8_operand;

typedef struct {
  int32_t batch, heads_q, heads_kv, seqlen, d_qk, d_v, causal;
  float softmax_scale; /* sigma: S = sigma * Q K^T; usually 1/sqrt(d_qk) */
} dm_attn_shape;

/* L rounded up to a multiple of 128: the padded sequence length of every
 * quantized attention operand.  Returns -1 for L < 0. */
int64_t dm_padded_len(int64_t L);

/* Human-readable name of a status code (static storage). */
const char* dm_status_string(dm_status s);

/*
 * Block-quantize x to FP8 (the operands of section 01, "What changes in FP8?":
 * decoded FP8 values including their block scales).
 *   x       [batch][rows][cols], bf16 (DM_BF16) or float32 (DM_F32), finite.
 *   axis == DM_AXIS_COLS: blocks of 32 consecutive columns (cols % 32 == 0);
 *           codes [batch][rows_out][cols], scales [batch][rows_out][cols/32].
 *   axis == DM_AXIS_ROWS: blocks of 32 consecutive rows, output transposed;
 *           rows_out % 32 == 0; codes [batch][cols][rows_out],
 *           scales [batch][cols][rows_out/32].
 *   rows_out >= rows; rows in [rows, rows_out) are written as zero codes with
 *   scale 2^-126.  On both axes cols must be a positive multiple of 32 (at most
 *   2^20), batch <= 65535 and rows_out <= 2^36; otherwise DM_ERR_SHAPE.
 *   Output is bit-exact with the rule above.
 */
dm_status dm_quantize_blockfp8(const void* x, dm_dtype dtype, int64_t batch, int64_t rows,
                               int64_t cols, int64_t rows_out, dm_block_axis axis,
                               dm_fp8_format fmt, uint8_t* codes, float* scales,
                               hipStream_t stream);

/*
 * Forward (section 01, "Write down softmax backward" and "What changes in
 * FP8?"): S = sigma * Q^<c> K^<c>^T in FP32 (causal: keys j <= i), online
 * softmax in FP32 whose running row maximum mu is updated once per chunk of
 * 128 keys, P' = exp(S - mu) cast to E4M3 in 32-key blocks, O_acc rescaled and
 * accumulated with P'^ V^<s> in FP32, l summed from the unquantized P'.
 *   q_c [B][Hq][Lp][d_qk] E4M3, k_c [B][Hkv][Lp][d_qk] E4M3,
 *   v_s [B][Hkv][d_v][Lp] E4M3 (sequence blocks).
 *   o   [B][Hq][L][d_v] float32 (O = O_acc / l), written for rows < L.
 *   lse [B][Hq][L] float32, natural-log log-sum-exp of sigma*S rows.
 */
dm_status dm_attn_fwd(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand k_c,
                      dm_fp8_operand v_s, float* o, float* lse, hipStream_t stream);

/*
 * Row correction delta [B][Hq][L] float32 (section 01 "Why can we reuse the
 * forward output?" and section 03 "Does matching the backward operands fix
 * it?").
 *   DM_DELTA_STALE:      needs o [B][Hq][L][d_v] float32 and do_bf16
 *                        [B][Hq][L][d_v] (bf16 bits, dO before its cast).
 *   DM_DELTA_DO_MATCHED: needs o and do_c (dO^<c>, E5M2).
 *   DM_DELTA_MATCHED:    needs do_c, q_c, k_c, v_c (V^<c>, E4M3 channel
 *                        blocks) and lse from dm_attn_fwd; recomputes
 *                        P = exp(S - LSE) in FP32 and dP^ = dO^<c> V^<c>^T on
 *                        FP8 matrix cores, tile by tile.
 *   Arguments a mode does not use may be NULL.
 */
dm_status dm_attn_delta(const dm_attn_shape* shape, dm_delta_mode mode, const float* o,
                        const uint16_t* do_bf16, dm_fp8_operand do_c, dm_fp8_operand q_c,
                        dm_fp8_operand k_c, dm_fp8_operand v_c, const float* lse, float* delta,
                        hipStream_t stream);

/*
 * Backward (section 01 "Write down softmax backward"; five FP8 matmuls per
 * section 03): per tile P = exp(S - LSE) (FP32), dV += P^<q>^T dO^<s>,
 * dP^ = dO^<c> V^<c>^T, dS = P * (dP^ - delta) (FP32), dQ += sigma dS^<k> K^<s>,
 * dK += sigma dS^<q>^T Q^<s>; P^<q> is P cast to E4M3 in 32-query blocks,
 * dS^<k> / dS^<q> are dS cast to E5M2 in 32-key / 32-query blocks.  dK and dV
 * are summed over the query heads of each KV group.
 *   q_c, q_s [B][Hq]...; k_c, k_s, v_c [B][Hkv]...; do_c, do_s [B][Hq]...
 *   lse, delta [B][Hq][L] float32.
 *   dq [B][Hq][L][d_qk], dk [B][Hkv][L][d_qk], dv [B][Hkv][L][d_v] float32,
 *   fully overwritten.
 *   probe_rowsum_ds, probe_rowsum_abs_pdp: optional [B][Hq][L] double
 *   outputs (NULL to skip): sum_j dS_ij of the FP32 dS before its casts, and
 *   sum_j |P_ij dP^_ij|.  Either both NULL or both non-NULL.
 */
dm_status dm_attn_bwd(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s,
                      dm_fp8_operand k_c, dm_fp8_operand k_s, dm_fp8_operand v_c,
                      dm_fp8_operand do_c, dm_fp8_operand do_s, const float* lse,
                      const float* delta, float* dq, float* dk, float* dv,
                      double* probe_rowsum_ds, double* probe_rowsum_abs_pdp, hipStream_t stream);

/*
 * The two independent halves of dm_attn_bwd, for callers that time them apart
 * or run them on two streams (same arguments, same results; neither reads what
 * the other writes).  dm_attn_bwd is dm_attn_bwd_dkdv followed by
 * dm_attn_bwd_dq on one stream.
 *   dm_attn_bwd_dkdv: dK and dV (key-stationary; the section 03 products
 *     P^<q>^T dO^<s> and dS^<q>^T Q^<s>); needs q_c, q_s, k_c, v_c, do_c, do_s.
 *   dm_attn_bwd_dq: dQ and the optional row-sum probes (query-stationary; the
 *     product dS^<k> K^<s>); needs q_c, k_c, k_s, v_c, do_c.
 * Errors as for dm_attn_bwd.
 */
dm_status dm_attn_bwd_dkdv(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s,
                           dm_fp8_operand k_c, dm_fp8_operand v_c, dm_fp8_operand do_c,
                           dm_fp8_operand do_s, const float* lse, const float* delta, float* dk,
                           float* dv, hipStream_t stream);
dm_status dm_attn_bwd_dq(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand k_c,
                         dm_fp8_operand k_s, dm_fp8_operand v_c, dm_fp8_operand do_c,
                         const float* lse, const float* delta, float* dq,
                         double* probe_rowsum_ds, double* probe_rowsum_abs_pdp, hipStream_t stream);

/*
 * dm_attn_bwd_dkdv for grids too small to fill the chip (section 03's dK and dV
 * products, as for dm_attn_bwd_dkdv).  The dK/dV kernel keeps one tile of keys
 * and sums over every query head of its KV group; when the shape has too few key
 * tiles to occupy every compute unit several times over, the query heads of each
 * KV group are dealt to 2, 4, ... workgroups per key tile, each writes its partial
 * dK and dV sums to the workspace, and a second kernel adds the parts in a fixed
 * order.  Results are deterministic; they may differ from dm_attn_bwd_dkdv's in
 * the last bits (FP32 sums taken in another order) and meet the same accuracy.
 *   dm_attn_bwd_dkdv_workspace_size: *bytes (host pointer) = the workspace the
 *     shape needs; 0 when it takes no split (head dims other than d_qk = d_v =
 *     128, or grids that are already large).  Depends on the shape only and is
 *     under 256 MiB for every shape.
 *   dm_attn_bwd_dkdv_ws: workspace is a device buffer of workspace_bytes bytes,
 *     16-byte aligned, owned by the caller, contents undefined on entry and on
 *     return (NULL allowed when the size is 0).  DM_ERR_WORKSPACE when
 *     workspace_bytes is below the size; other errors as for dm_attn_bwd.  Calls
 *     that share a workspace must not overlap.
 */
dm_status dm_attn_bwd_dkdv_workspace_size(const dm_attn_shape* shape, int64_t* bytes);
dm_status dm_attn_bwd_dkdv_ws(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s,
                              dm_fp8_operand k_c, dm_fp8_operand v_c, dm_fp8_operand do_c,
                              dm_fp8_operand do_s, const float* lse, const float* delta, float* dk,
                              float* dv, void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * dm_attn_bwd_dkdv_ws for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * head split's partial sums go to a static scratch array of
 * DM_NOALLOC_SCRATCH_BYTES that each device holds from the library's first use
 * of it until the process ends.  Same arguments as dm_attn_bwd_dkdv minus the
 * workspace; dK and dV are bit for bit those of dm_attn_bwd_dkdv_ws.
 *   - Never calls hipMalloc, hipFree or an allocating routine.  The first call on
 *     a device looks up that device's scratch address (hipGetSymbolAddress) with
 *     the current device; stream and buffers must belong to the current device.
 *   - DM_ERR_WORKSPACE when dm_attn_bwd_dkdv_workspace_size exceeds
 *     DM_NOALLOC_SCRATCH_BYTES (nothing enqueued; use dm_attn_bwd_dkdv_ws then).
 *   - The scratch needs no clearing: every call writes every byte it reads.  All
 *     calls on one device share it, so calls that overlap in time on one device
 *     (other streams, other threads) race and give wrong results; serialize them.
 *   - Other errors as for dm_attn_bwd; DM_ERR_HIP also when the scratch address
 *     cannot be obtained.
 */
dm_status dm_attn_bwd_dkdv_noalloc(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s,
                                   dm_fp8_operand k_c, dm_fp8_operand v_c, dm_fp8_operand do_c,
                                   dm_fp8_operand do_s, const float* lse, const float* delta, float* dk,
                                   float* dv, hipStream_t stream);

/*
 * dm_attn_bwd_dkdv with the row-sum probes of the dS that the dK/dV kernel itself
 * computes and casts (section 03 "Does matching the backward operands fix it?":
 * with matched delta the rows of dS sum to zero up to FP32 rounding before dS is
 * cast to FP8).  dK and dV are bit for bit those of dm_attn_bwd_dkdv.
 *   probe_rowsum_ds:      [B][Hq][L] double, sum_j dS_ij of the FP32 dS before its
 *                         E5M2 cast along queries (the dK operand);
 *   probe_rowsum_abs_pdp: [B][Hq][L] double, sum_j |P_ij dP^_ij|.
 * Both are required (non-NULL, 16-byte aligned) and fully overwritten: the call
 * zeroes them, then adds FP32 partial sums over groups of 16 or 32 keys to them
 * with FP64 atomics, so the last bits may differ from run to run.  Other errors as
 * for dm_attn_bwd.
 */
dm_status dm_attn_bwd_dkdv_probes(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand q_s,
                                  dm_fp8_operand k_c, dm_fp8_operand v_c, dm_fp8_operand do_c,
                                  dm_fp8_operand do_s, const float* lse, const float* delta, float* dk,
                                  float* dv, double* probe_rowsum_ds, double* probe_rowsum_abs_pdp,
                                  hipStream_t stream);

/*
 * dm_attn_bwd_dq with a third row-sum probe (section 03 "Does matching the
 * backward operands fix it?": Delta-Matching makes the row sums of dS vanish up
 * to FP32 rounding before dS is cast to FP8, and the cast then adds a row-sum
 * residual of its own, which the page compares between stale delta and
 * Delta-Matching):
 *   probe_rowsum_ds, probe_rowsum_abs_pdp: as for dm_attn_bwd_dq;
 *   probe_rowsum_ds_cast: [B][Hq][L] double, sum_j dS^<k>_ij, the dS that enters
 *   the dQ product after its E5M2 cast in 32-key blocks (decoded codes times the
 *   block scales), summed in FP32 per 128 keys and FP64 across them.
 * dq as for dm_attn_bwd_dq.  All three probe pointers are required (non-NULL,
 * 16-byte aligned); other errors as for dm_attn_bwd.
 */
dm_status dm_attn_bwd_dq_probes(const dm_attn_shape* shape, dm_fp8_operand q_c, dm_fp8_operand k_c,
                                dm_fp8_operand k_s, dm_fp8_operand v_c, dm_fp8_operand do_c,
                                const float* lse, const float* delta, float* dq,
                                double* probe_rowsum_ds, double* probe_rowsum_abs_pdp,
                                double* probe_rowsum_ds_cast, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DM_ATTN_H */
