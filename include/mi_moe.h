/*
 * mi_moe.h -- C ABI of the MI355X (gfx950) routed-MoE hot path.
 *
 * Operations (sources are cited by page title and section):
 *   - mi_grouped_mm_bf16      ragged per-expert grouped GEMM
 *                             (flashinfer.grouped_mm.grouped_mm_bf16, formula)
 *   - mi_grouped_mm_swiglu    FC1: gate/up grouped GEMM + SwiGLU epilogue
 *                             (prims_ts_fp4_block_scale_moe, gemm1 parameters)
 *   - mi_moe_fc2_lora_delta   FC2 LoRA delta of a routed MoE
 *                             (flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta, formula)
 *   - mi_moe_fc1_lora_delta   FC1 (gate/up) LoRA delta, one row per routed slot: the
 *                             gemm1_lora_delta the delta page's description names
 *   - mi_moe_fc2_finalize_lora  the MoE finalize (routing-weighted combine of the FC2
 *                             rows) with that delta added, in one pass
 *                             (bgmv_moe_gemm2_lora_delta, description and return value)
 *   - mi_moe_route_permutation  routing output -> expert-sorted permutation
 *                             (bgmv_moe_gemm2_lora_delta and grouped_mm_bf16, parameters)
 *   - mi_moe_permute_rows     token rows -> permuted rows (the FC1 input)
 *   - mi_grouped_mm_nvfp4     ragged grouped GEMM with NVFP4 operands
 *                             (grouped_mm_bf16 formula, mm_nvfp4_lora operand format)
 *   - mi_mm_nvfp4_lora        NVFP4 GEMM with an fp32 LoRA epilogue, raw and prepared
 *                             (flashinfer.gemm.mm_nvfp4_lora, formula and the two bullets)
 *   - mi_prepare_lora_fold    the prepared-path fold
 *                             (flashinfer.gemm.prepare_nvfp4_lora_adapter, description and `out=`)
 *   - mi_nvfp4_dequant_bf16   NVFP4 -> bf16 dequantisation with the GEMM's own decoder
 *   - mi_fp4_quantize         bf16/fp16/fp32 -> NVFP4 codes + UE4M3 scales, the producer of
 *                             the NVFP4 operands (mm_nvfp4_lora, the paragraph after the
 *                             formula, and its alpha parameter)
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or retains them and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on that stream and returns; nothing is read
 *     back to the host.  Results are valid once the stream reaches the work.
 *   - Arguments are validated on the host BEFORE any HIP call.  A violation
 *     returns MI_EINVAL (or MI_EUNSUPPORTED for a valid but unimplemented
 *     dtype/shape) and mi_last_error() names the violated requirement; nothing
 *     is enqueued.  MI_EHIP means a HIP launch error (message from HIP).
 *   - Device-resident index data (m_indptr, ids, permutations) is not read on
 *     the host; kernels clamp/skip out-of-range values so they stay memory-safe.
 *   - Calls are thread-safe; the error message is thread-local.
 *   - Row-major layouts; "bf16" is IEEE binary32 truncated to its top 16 bits
 *     (rounding, where a result is produced, is to nearest even).
 */
#ifndef MI_MOE_H
#define MI_MOE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MI_API __attribute__((visibility("default")))
#else
#define MI_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MI_OK = 0,
  MI_EINVAL = 1,        /* invalid argument: maps to ValueError */
  MI_EUNSUPPORTED = 2,  /* valid request this build does not implement */
  MI_EHIP = 3           /* HIP runtime error while enqueueing */
} mi_status;

typedef enum { MI_BF16 = 0, MI_F16 = 1, MI_F32 = 2 } mi_dtype;

/* Message of the last failing call on this thread ("" after success). */
MI_API const char* mi_last_error(void);

/* ABI version of this library (bumped on any signature change). */
MI_API int mi_abi_version(void);

/*
 * Ragged grouped GEMM (flashinfer.grouped_mm.grouped_mm_bf16, formula and
 * parameters): for every expert e with s = m_indptr[e], t = m_indptr[e+1],
 *     out[s:t, :] = a[s:t, :] @ b[e]^T
 * accumulated in fp32 and rounded once to out_dtype.
 *
 *   a         [m_rows, k] of ab_dtype (MI_BF16 or MI_F16: "bf16 or fp16" in the
 *             parameter list)
 *   b         [batch, n, k] of ab_dtype  (K-major: row j of b[e] is output column j)
 *   m_indptr  int32 [batch + 1], device, non-decreasing, 0 <= values <= m_rows;
 *             read on the device only -- empty groups are skipped, no padding
 *   out       [m_rows, n] of out_dtype (MI_BF16, MI_F16 or MI_F32), 16-byte
 *             aligned; only rows [m_indptr[0], m_indptr[batch]) are written, the
 *             rest untouched
 * Requirements: m_rows >= 0, batch >= 1, n % 256 == 0, k % 64 == 0 (the
 * device-walk backend's shape rule on the page), k >= 64.  k >= 4194304 (2^22)
 * returns MI_EUNSUPPORTED: the kernels address a 512-row panel of b through
 * one 32-bit buffer range.
 */
MI_API mi_status mi_grouped_mm_bf16(const void* a, int64_t m_rows, int64_t k,
                             mi_dtype ab_dtype, const void* b, int64_t batch,
                             int64_t n, const int32_t* m_indptr,
                             void* out, mi_dtype out_dtype, void* stream);

/*
 * FC1 of a routed MoE: the gate/up grouped GEMM with its SwiGLU activation in
 * the epilogue (flashinfer.fused_moe.prims_ts_fp4_block_scale_moe, parameters
 * gemm1_weights, gemm1_alpha, gemm1_beta, gemm1_clamp_limit, activation_type;
 * the ragged product of flashinfer.grouped_mm.grouped_mm_bf16, formula).  For
 * every expert e and row t in [m_indptr[e], m_indptr[e+1]):
 *   h = a[t] @ b[e]^T (+ fc1_delta[t])            fp32, [2I]
 *   g = min(h[0:I], limit[e]);  u = clamp(h[I:2I], -limit[e], limit[e])
 *   out[t] = g * sigmoid(alpha[e] * g) * (u + beta[e])      rounded once
 * which is silu(gate) * up with the defaults (alpha 1, beta 0, no limit).
 *   a          ab_dtype [m_rows, k] (the permuted FC1 input)
 *   b          ab_dtype [batch, 2*inter_size, k]: rows 0..I-1 gate, I..2I-1 up
 *   m_indptr   int32 [batch + 1], device, non-decreasing (clamped into [0, m_rows])
 *   fc1_delta  bf16 [m_rows, 2*inter_size] added before the activation (the FC1
 *              LoRA delta), or NULL; 8-byte aligned
 *   alpha, beta, limit  fp32 [batch] each, or NULL for the default
 *   out        out_dtype [m_rows, inter_size] (MI_BF16, MI_F16 or MI_F32), 16-byte
 *              aligned; rows outside the groups are untouched
 * Requirements: 1 <= batch <= 1024, inter_size % 128 == 0, k % 64 == 0.
 */
MI_API mi_status mi_grouped_mm_swiglu(const void* a, int64_t m_rows, int64_t k, mi_dtype ab_dtype,
                               const void* b, int64_t batch, int64_t inter_size,
                               const int32_t* m_indptr, const void* fc1_delta, const float* alpha,
                               const float* beta, const float* limit, void* out,
                               mi_dtype out_dtype, void* stream);

/*
 * FC2 LoRA delta of a routed MoE (flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta,
 * formula and parameters):
 *     delta[t] = scale * sum_j w[t,j] * B_down[l,e] @ (A_down[l,e] @ act[perm[t*top_k+j]])
 * with e = topk_ids[t,j], w = topk_weights[t,j], l = lora_ids[t].
 *
 *   act          lora_dtype [padded_rows, inter_size]  permuted post-activation rows;
 *                lora_dtype (MI_BF16 or MI_F16, "bf16/fp16" in the parameter list) is
 *                also the element type of both LoRA banks.  May be NULL when
 *                padded_rows == 0 (every slot is then inactive and nothing is read)
 *   expanded_idx_to_permuted_idx  int32 [num_tokens * top_k]; < 0 = inactive slot
 *   w_ptr_a      int64 [num_experts]: byte address (16-byte aligned) of A_down[0,e], a [rank, inter_size]
 *                block; adapter l starts lora_stride_a ELEMENTS later
 *   w_ptr_b      int64 [num_experts]: byte address (16-byte aligned) of B_down[0,e], a [hidden, rank]
 *                block; adapter l starts lora_stride_b ELEMENTS later
 *   topk_ids     int32 [num_tokens, top_k];  topk_weights fp32 [num_tokens, top_k]
 *   lora_ids     int32 [num_tokens]; < 0 = no adapter.  Ids >= num_adapters, slots
 *                whose permuted row is >= padded_rows and expert ids outside
 *                [0, num_experts) are treated as inactive (memory safety only;
 *                they are caller errors).
 *   out          out_dtype [num_tokens, hidden]; EVERY element is written (+0 for
 *                tokens without adapter or without an active slot)
 *   workspace    device scratch of at least mi_moe_fc2_lora_delta_workspace_size()
 *                bytes, 256-byte aligned; contents need no initialisation
 * The intermediate A_down @ act is fp32 and reaches the second product with ~16
 * (bf16) or ~22 (fp16, after a per-slot power-of-two scaling) significant bits;
 * the result is rounded once.
 * Requirements: lora_dtype MI_BF16 or MI_F16; out_dtype MI_BF16, MI_F16 or MI_F32; rank % 8 == 0,
 * 8 <= rank <= 128; inter_size % 8 == 0; hidden % 128 == 0; 1 <= top_k <= 32;
 * lora strides multiples of 8; num_experts <= 512.
 */
MI_API size_t mi_moe_fc2_lora_delta_workspace_size(int64_t num_tokens, int64_t top_k,
                                            int64_t num_experts, int64_t num_adapters,
                                            int64_t rank);
MI_API mi_status mi_moe_fc2_lora_delta(const void* act, int64_t padded_rows, int64_t inter_size,
                                const int32_t* expanded_idx_to_permuted_idx,
                                const int64_t* w_ptr_a, int64_t lora_stride_a,
                                const int64_t* w_ptr_b, int64_t lora_stride_b,
                                const int32_t* topk_ids, const float* topk_weights,
                                const int32_t* lora_ids,
                                int64_t num_tokens, int64_t top_k, int64_t num_experts,
                                int64_t num_adapters, int64_t rank, int64_t hidden_size,
                                mi_dtype lora_dtype, float scale, mi_dtype out_dtype,
                                void* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * mi_moe_fc2_lora_delta for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and result, with the workspace taken from a
 * fixed array inside the library instead of a caller buffer.  The array holds
 * MI_DELTA_SCRATCH_BYTES (32 MiB) on every GPU the library runs on, until the
 * process ends; its device address is looked up once per device
 * (hipGetSymbolAddress) on the first call there, with that device current.
 * The call allocates nothing and clears nothing (the kernels write every
 * scratch entry they read).  Problems whose
 * mi_moe_fc2_lora_delta_workspace_size() exceeds the array return
 * MI_EUNSUPPORTED.  Every call on one GPU uses the same array: calls that
 * overlap on one device (different streams, or threads without ordering)
 * race and give undefined results.
 */
#define MI_DELTA_SCRATCH_BYTES (32u << 20)
MI_API mi_status mi_moe_fc2_lora_delta_noalloc(const void* act, int64_t padded_rows,
                                        int64_t inter_size,
                                        const int32_t* expanded_idx_to_permuted_idx,
                                        const int64_t* w_ptr_a, int64_t lora_stride_a,
                                        const int64_t* w_ptr_b, int64_t lora_stride_b,
                                        const int32_t* topk_ids, const float* topk_weights,
                                        const int32_t* lora_ids, int64_t num_tokens,
                                        int64_t top_k, int64_t num_experts,
                                        int64_t num_adapters, int64_t rank,
                                        int64_t hidden_size, mi_dtype lora_dtype, float scale,
                                        mi_dtype out_dtype, void* out, void* stream);

/*
 * FC1 (gate/up) LoRA delta of a routed MoE: the gemm1_lora_delta that
 * flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta (description) says FC1 runs
 * with.  The pages give no formula for it; this library computes the FC1
 * counterpart of the FC2 formula, one row per routed slot, with no routing
 * weight and no combine:
 *     out[p] = scale * B_up[l,e] @ (A_up[l,e] @ act[p])      p = perm[t*top_k+j]
 * with e = topk_ids[t,j], l = lora_ids[t], act the permuted FC1 input (the rows
 * the FC1 GEMM multiplies).  The result is the fc1_delta of
 * mi_grouped_mm_swiglu, added before the activation.
 *   act          lora_dtype [padded_rows, hidden_size], 16-byte aligned
 *   perm         int32 [num_tokens * top_k]; < 0 = inactive slot
 *   w_ptr_a      int64 [num_experts]: byte address of A_up[0,e], a [rank, hidden_size]
 *                block; adapter l starts lora_stride_a ELEMENTS later (16-byte aligned)
 *   w_ptr_b      int64 [num_experts]: byte address of B_up[0,e], an [out_features, rank]
 *                block; adapter l starts lora_stride_b ELEMENTS later (16-byte aligned)
 *   topk_ids     int32 [num_tokens, top_k];  lora_ids int32 [num_tokens], < 0 = none
 *   out          out_dtype [padded_rows, out_features] (MI_BF16, MI_F16 or MI_F32),
 *                16-byte aligned.  Row p of every slot with p in [0, padded_rows) is
 *                written: the delta, or +0 when the token has no adapter (id outside
 *                [0, num_adapters)) or the expert lies outside [0, num_experts).
 *                Rows no slot points at are untouched.
 *   workspace    at least mi_moe_fc1_lora_delta_workspace_size() bytes, 256-byte
 *                aligned, no initialisation needed
 * Rounding: the intermediate A_up @ act is fp32, carried as bf16 (or scaled fp16)
 * hi + lo into the second product; one rounding to out_dtype.
 * Requirements: as for mi_moe_fc2_lora_delta with hidden_size in the role of
 * inter_size and out_features in the role of hidden_size (out_features % 128 ==
 * 0); two slots pointing at the same row leave one of their deltas there.
 */
MI_API size_t mi_moe_fc1_lora_delta_workspace_size(int64_t num_tokens, int64_t top_k,
                                            int64_t num_experts, int64_t num_adapters,
                                            int64_t rank);
MI_API mi_status mi_moe_fc1_lora_delta(const void* act, int64_t padded_rows, int64_t hidden_size,
                                const int32_t* expanded_idx_to_permuted_idx,
                                const int64_t* w_ptr_a, int64_t lora_stride_a,
                                const int64_t* w_ptr_b, int64_t lora_stride_b,
                                const int32_t* topk_ids, const int32_t* lora_ids,
                                int64_t num_tokens, int64_t top_k, int64_t num_experts,
                                int64_t num_adapters, int64_t rank, int64_t out_features,
                                mi_dtype lora_dtype, float scale, mi_dtype out_dtype,
                                void* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * MoE finalize with the FC2 LoRA delta added (flashinfer.fused_moe.
 * bgmv_moe_gemm2_lora_delta, description and return value: the delta is
 * combined over the experts and added to the MoE output after the combine):
 *     out[t] = sum_j w[t,j] * fc2[perm[t*top_k+j]] + delta[t]
 * with delta[t] exactly as mi_moe_fc2_lora_delta defines it.  The sum is
 * formed in fp32 (delta first, then the slots in order) and rounded once to
 * out_dtype; the delta is never rounded on its own.
 *   fc2          fc2_dtype [padded_rows, hidden_size]: the FC2 grouped-GEMM output in
 *                permuted row order (MI_BF16, MI_F16 or MI_F32), 16-byte aligned;
 *                not read (and may be NULL) when padded_rows == 0
 *   perm, topk_weights: as for the delta; a slot whose permuted row is < 0 or
 *                >= padded_rows is not routed here and contributes nothing (to the
 *                combine and to the delta); every other slot's row is combined with
 *                its weight, whatever its expert id
 *   everything else and the validation: as for mi_moe_fc2_lora_delta (its
 *   messages name that operation).  Tokens without an adapter get the combine
 *   alone.  num_adapters == 0 gives the plain combine.
 *   workspace    at least mi_moe_fc2_lora_delta_workspace_size(...) bytes.  With
 *                mi_moe_fc2_finalize_workspace_size(...) bytes (room for an fp32
 *                [num_tokens, hidden_size] delta) the call runs in two passes --
 *                the delta to the workspace, then a combine that reads whole FC2
 *                rows -- which is faster; both give bitwise the same output.
 */
MI_API size_t mi_moe_fc2_finalize_workspace_size(int64_t num_tokens, int64_t top_k,
                                          int64_t num_experts, int64_t num_adapters,
                                          int64_t rank, int64_t hidden_size);
MI_API mi_status mi_moe_fc2_finalize_lora(const void* fc2, mi_dtype fc2_dtype, const void* act,
                                   int64_t padded_rows, int64_t inter_size,
                                   const int32_t* expanded_idx_to_permuted_idx,
                                   const int64_t* w_ptr_a, int64_t lora_stride_a,
                                   const int64_t* w_ptr_b, int64_t lora_stride_b,
                                   const int32_t* topk_ids, const float* topk_weights,
                                   const int32_t* lora_ids, int64_t num_tokens, int64_t top_k,
                                   int64_t num_experts, int64_t num_adapters, int64_t rank,
                                   int64_t hidden_size, mi_dtype lora_dtype, float scale,
                                   mi_dtype out_dtype, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Routing output -> the expert-sorted permutation that the grouped GEMM, the
 * delta and the finalize consume (flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta,
 * parameter expanded_idx_to_permuted_idx: expanded index t*top_k+j -> permuted
 * row, negative when inactive; flashinfer.grouped_mm.grouped_mm_bf16, parameter
 * m_indptr: cumulative rows per group).  The permuted order is a stable sort of
 * the slots by expert id: expert e owns rows m_indptr[e] .. m_indptr[e+1]-1 and,
 * inside it, the slots keep their expanded order.  A slot whose id is outside
 * [0, num_experts) is not routed here: its entry is -1 and it takes no row.
 * The result is deterministic (bit-identical on every run).
 *   topk_ids      int32 [num_tokens, top_k], device
 *   m_indptr      int32 [num_experts + 1], device, written (m_indptr[0] = 0)
 *   expanded_idx_to_permuted_idx  int32 [num_tokens * top_k], device, written
 *   permuted_idx_to_expanded_idx  int32 [num_tokens * top_k] or NULL: entry p is
 *                 the expanded index at permuted row p for p < m_indptr[E], -1 after
 *   workspace     device scratch of mi_moe_route_workspace_size(num_tokens*top_k,
 *                 num_experts) bytes; its contents are not kept between calls
 * Requirements: top_k >= 1, num_tokens >= 0, num_tokens*top_k < 2^31,
 * 1 <= num_experts <= 1024; the output arrays may not alias topk_ids or each
 * other.  num_tokens == 0 writes m_indptr = 0 only.
 */
MI_API size_t mi_moe_route_workspace_size(int64_t num_slots, int64_t num_experts);
MI_API mi_status mi_moe_route_permutation(const int32_t* topk_ids, int64_t num_tokens,
                                   int64_t top_k, int64_t num_experts, int32_t* m_indptr,
                                   int32_t* expanded_idx_to_permuted_idx,
                                   int32_t* permuted_idx_to_expanded_idx, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * The FC1 input in permuted row order: out[perm[t*top_k+j]] = x[t] for every
 * slot whose entry lies in [0, out_rows); other rows of out are untouched
 * (flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta, parameter
 * expanded_idx_to_permuted_idx, read in the gathering direction).  A byte copy:
 * any element type, rows of row_bytes bytes.
 *   x     [num_tokens, row_bytes] bytes, 16-byte aligned, device
 *   perm  int32 [num_tokens * top_k], device (e.g. from mi_moe_route_permutation)
 *   out   [out_rows, row_bytes] bytes, 16-byte aligned, device; may not alias x
 * Requirements: row_bytes > 0 and a multiple of 16, top_k >= 1,
 * 0 <= num_tokens*top_k < 2^31, out_rows >= 0.  Two slots with the same row
 * (an invalid permutation) leave one of the token rows there.
 */
MI_API mi_status mi_moe_permute_rows(const void* x, int64_t num_tokens, int64_t row_bytes,
                              const int32_t* perm, int64_t top_k, void* out, int64_t out_rows,
                              void* stream);

/*
 * NVFP4 GEMM with a BF16 LoRA correction (flashinfer.gemm.mm_nvfp4_lora):
 *   raw      : out = bf16( alpha*acc + lora_scale*(d @ lora_b^T) [+ bias] )
 *   prepared : out = bf16( alpha*(acc + d @ b_folded^T) [+ bias] )
 *   off      : out = bf16( alpha*acc [+ bias] )
 * acc = dequant(a) @ dequant(b)^T accumulated in fp32; one rounding to bf16.
 *
 *   a, b        uint8 [m, k/2], [n, k/2]: E2M1 codes, a pair in each byte, element 2i in
 *               the low nibble
 *   a_sf, b_sf  UE4M3 scales, one per 16 elements along k, 128x4-tiled with rows
 *               padded to 128 (tile = 128 rows x 4 scale columns = 512 bytes,
 *               tiles row-block major; inside: (r%32)*16 + ((r%128)/32)*4 + c%4);
 *               a_sf_bytes / b_sf_bytes give the buffer sizes (larger is fine)
 *   alpha       fp32 device scalar (element 0 used)
 *   d           bf16 [m, rank] or NULL;  rank = d's column count
 *   lora_b      raw path: bf16 [n, rank];  lora_scale fp32 device scalar.
 *               lora_scale == NULL -> adapter off even if d / lora_b are given.
 *               *lora_scale == 0 (read on the device) -> the adapter-off program
 *               path, bitwise identical to the off call.
 *   b_folded    prepared path: bf16 [n, rank] from mi_prepare_lora_fold, with its
 *               fold_flags word; bit 0 set (zero adapter) -> the off path.
 *   bias        bf16 [n] or NULL, summed in fp32, then the one rounding
 *   out         bf16 [m, n]
 * Requirements: m >= 1, n >= 1, k % 256 == 0 (k >= 256); rank % 8 == 0 and
 * 8 <= rank <= 128 when an adapter is given; not both adapter forms; a prepared
 * adapter needs d; scale buffers large enough for the padded layout.
 */
MI_API mi_status mi_mm_nvfp4_lora(const uint8_t* a, const uint8_t* b,
                           const uint8_t* a_sf, size_t a_sf_bytes,
                           const uint8_t* b_sf, size_t b_sf_bytes,
                           const float* alpha, int64_t m, int64_t n, int64_t k,
                           const void* d, int64_t rank,
                           const void* lora_b, const float* lora_scale,
                           const void* b_folded, const uint32_t* fold_flags,
                           const void* bias, void* out, void* stream);

/*
 * NVFP4 grouped GEMM: the ragged per-expert walk of flashinfer.grouped_mm.
 * grouped_mm_bf16 (formula) with FP4 expert weights in the operand format of
 * flashinfer.gemm.mm_nvfp4_lora (parameters a, b, a_sf, b_sf, alpha) -- the
 * weight format the FP4 fused-MoE page names for its experts:
 *   out[m_indptr[e]:m_indptr[e+1]] = alpha[e] * dequant(a[...]) @ dequant(b[e])^T
 * acc in fp32, one rounding to out_dtype; rows outside [m_indptr[0],
 * m_indptr[batch]) are not written.
 *   a         uint8 [m_rows, k/2] codes (element 2i in the low nibble), device
 *   a_sf      UE4M3 scales of a in the 128x4 layout over all m_rows rows (rows
 *             padded to 128), a_sf_bytes its size (larger is fine)
 *   b         uint8 [batch, n, k/2] codes
 *   b_sf      batch consecutive 128x4 scale buffers, each for [n, k/16] scales
 *             (ceil(n/128) * ceil(k/64) * 512 bytes apiece); b_sf_bytes the total
 *   m_indptr  int32 [batch + 1], device, non-decreasing (clamped into [0, m_rows])
 *   alpha     fp32 [batch], device: each expert's base scale
 *   out       out_dtype (MI_BF16 or MI_F32) [m_rows, n]
 * Requirements: 1 <= batch <= 1024, n % 256 == 0, k % 256 == 0 (k >= 256),
 * a and b 16-byte aligned, scale buffers 4-byte aligned, a's codes, a's scales
 * and one expert's codes below 4 GiB each.  m_rows == 0 is a no-op.
 */
MI_API mi_status mi_grouped_mm_nvfp4(const uint8_t* a, const uint8_t* a_sf, size_t a_sf_bytes,
                              int64_t m_rows, int64_t k, const uint8_t* b, const uint8_t* b_sf,
                              size_t b_sf_bytes, int64_t batch, int64_t n,
                              const int32_t* m_indptr, const float* alpha, void* out,
                              mi_dtype out_dtype, void* stream);

/*
 * The prepared-path fold (flashinfer.gemm.prepare_nvfp4_lora_adapter):
 *   ratio       = fp32 division, round to nearest even: *lora_scale / alpha[0]
 *   b_folded[i] = bf16_rne(fp32(lora_b[i]) * ratio)        (IEEE, subnormals kept)
 *   fold_flags[0] = (*lora_scale == 0) ? 1 : 0              (bit 0: zero adapter)
 * Everything happens on the device (no host read), so the same call is the
 * in-place refold.  alpha == 0 is NOT checked here (it folds to Inf/NaN); the
 * eager prepare checks it with its one documented host read.
 *   lora_b bf16 [n, rank]; b_folded bf16 [n, rank] (may not alias lora_b);
 *   lora_scale, alpha fp32 device scalars; fold_flags uint32 [1].
 */
MI_API mi_status mi_prepare_lora_fold(const void* lora_b, int64_t n, int64_t rank,
                               const float* lora_scale, const float* alpha,
                               void* b_folded, uint32_t* fold_flags, void* stream);

/*
 * Dequantise an NVFP4 matrix with the GEMM's own in-register decoder:
 * out[r, j] = E2M1(code[r, j]) * UE4M3(scale of (r, j/16)) as bf16 (exact).
 *   codes uint8 [rows, k/2]; sf as for mi_mm_nvfp4_lora; out bf16 [rows, k].
 * Requirements: rows >= 1, k % 64 == 0.
 */
MI_API mi_status mi_nvfp4_dequant_bf16(const uint8_t* codes, const uint8_t* sf, size_t sf_bytes,
                                int64_t rows, int64_t k, void* out, void* stream);

/*
 * NVFP4 quantiser: the producer of the operands mi_mm_nvfp4_lora and
 * mi_grouped_mm_nvfp4 take (flashinfer.gemm.mm_nvfp4_lora, the paragraph after
 * the formula: the layout fp4_quantize() writes; parameter alpha: the base
 * scale divided by the two operands' global scales).  The pages do not spell
 * out its steps; for every row and every block of 16 consecutive elements x_i
 * along k, with g = global_scale[matrix], each step an IEEE fp32 operation
 * rounded to nearest even:
 *   amax = max |x_i|;   s = (amax * g) / 6
 *   sf   = the UE4M3 code nearest to s, ties to the even code, >= 448 -> 0x7E
 *   r    = g / value(sf), or 0 when value(sf) == 0
 *   code = the E2M1 code nearest to x_i * r, ties to the even code, magnitudes
 *          above 6 -> 6, sign bit = sign of x_i * r
 * so dequant(codes, sf) / g approximates x (at most value(sf) / g per element).
 *   x             x_dtype (MI_BF16, MI_F16 or MI_F32) [batch, rows, k], 16-byte aligned
 *   global_scale  fp32 [batch], device: g of each matrix
 *   codes         uint8 [batch, rows, k/2], element 2i in the low nibble; 4-byte aligned
 *   sf            batch consecutive 128x4 scale buffers (as for mi_mm_nvfp4_lora), each
 *                 ceil(rows/128) * (k/64) * 512 bytes; padding rows are written as 0;
 *                 sf_bytes the total size (larger is fine); 4-byte aligned
 * Requirements: batch >= 1, rows >= 0 (0 is a no-op), k % 64 == 0, k >= 64.
 */
MI_API mi_status mi_fp4_quantize(const void* x, int64_t batch, int64_t rows, int64_t k,
                          mi_dtype x_dtype, const float* global_scale, uint8_t* codes,
                          uint8_t* sf, size_t sf_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MI_MOE_H */
