/*
 * mxmoe.h -- C ABI of the MI355X (gfx950) MXFP8 Mixture-of-Experts expert path.
 *
 * The path: quantize bf16 activations, weights and gradients to MXFP8
 * (rowwise and columnwise), permute tokens by expert while they stay in
 * MXFP8, and run the block-scaled grouped GEMMs of the expert forward, dgrad
 * and wgrad.  Sources: the engineering.fyi digest "1.5x faster MoE training
 * on Blackwell with MXFP8 kernels built from scratch" (Overview, Key
 * Questions Answered: microscaling and block-scaled matrix multiplies), and
 * pytorch/ao PR #3203 (stacked-PR list: separate MXFP8 quantize and
 * dequantize kernels, an e8m0 -> fp32 scale decode; "Next steps": an MXFP8
 * token shuffle and a scaled grouped GEMM taking pre-quantized tensors).
 *
 * Format (OCP MX v1.0): blocks of 32 consecutive elements share one E8M0
 * scale byte (value 2^(byte-127); byte 0 is 2^-127); elements are E4M3
 * codes (bias 7, max 448, NaN = 0x7F/0xFF).  Scale exponent of a block =
 * floor(log2(amax)) - 8 clamped to [-127, 127] (all-zero block -> byte 0);
 * element code = round-to-nearest-even of x / 2^scale, saturating at 448.
 *
 * Layouts (device memory, caller-owned):
 *   bf16 tensors      uint16 bit patterns, row-major
 *   MX tensor viewed as a matrix of R rows (batch entries stacked) and C
 *   columns, blocks of 32 along C:
 *     codes   q uint8 [R, C] row-major
 *     scales  s uint8 [P, R, 4], P = ceil(C / 128) panels of 128 columns:
 *             byte of (row r, block b) at ((b / 4) * R + r) * 4 + b % 4, so
 *             one GEMM k step reads consecutive rows' scales as consecutive
 *             dwords; bytes past the last block (C % 128 != 0) are zero.
 *             4-byte aligned.  Written "scales [R, C]" below.
 *   rowwise MX of [R, C]      q [R, C],  scales [R, C]
 *   columnwise MX of [R, C]   stored transposed: q [C, R], scales [C, R]
 *                             (blocks are 32 consecutive rows of one column)
 *   expert weights    W [E, N, K] (K contiguous); W^T colwise [E, K, N]
 *   grouped rows      rows of expert e are [off[e], off[e+1]) of an M_cap-row
 *                     buffer; off has E+1 int32 entries in device memory.
 *
 * Conventions:
 *   - Every call validates its host-side arguments first and returns a
 *     status (MX_OK or a negative MX_E* code) without touching the GPU when
 *     they are invalid.  Valid calls enqueue kernels on `stream` (a
 *     hipStream_t; NULL = the default stream) and return without waiting;
 *     MX_EHIP reports a launch failure.
 *   - The library allocates nothing and keeps no global state; all buffers
 *     are passed in.  Calls are thread-safe; calls on one stream are ordered.
 *   - Device-side contents are trusted for meaning but never for memory
 *     safety: out-of-range expert ids are ignored, group offsets are clamped
 *     to [0, M_cap] and made monotone before use.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* mx_stream_t; /* a hipStream_t */

enum {
  MX_OK = 0,
  MX_EINVAL = -1,       /* a null pointer, a bad size or alignment, a bad dtype */
  MX_EUNSUPPORTED = -2, /* a valid request outside the sizes this library implements */
  MX_EHIP = -3          /* the HIP runtime reported an error at launch */
};

enum { MX_OUT_BF16 = 0, MX_OUT_F32 = 1 };

/* Human-readable name of a status code (static storage). */
const char* mx_status_string(int status);

/*
 * MXFP8 quantize (digest "Key Questions Answered": a scale per fine-grained
 * sub-block; PR #3203 stacked list: MXFP8 quantization kernel).
 *
 *   x        bf16 [batch, rows, cols]
 *   gather   optional int32 [rows_out] (batch must be 1): output row r is
 *            source row gather[r], or an all-zero row when gather[r] < 0;
 *            entries >= rows also give zero rows.  Without a gather, output
 *            row r is source row r for r < rows and zero after.
 *   rows_out rows of the quantized output (per batch item)
 *   row_q/row_s  rowwise result: codes [batch, rows_out, cols], scales
 *            [batch * rows_out, cols]; or both NULL to skip it
 *   col_q/col_s  columnwise result stored transposed: codes [batch, cols,
 *            rows_out], scales [batch * cols, rows_out]; or both NULL
 * One kernel reads x once and writes every requested output.  Requires
 * cols % 32 == 0; rows_out % 32 == 0 when a columnwise output is asked for;
 * at least one output.  Expert groups laid out at multiples of 32 with zero
 * pad rows (as mx_permute's src_row gives) never share a columnwise block.
 */
int mx_quantize(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, const int32_t* gather,
                int64_t rows_out, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, uint8_t* col_s,
                mx_stream_t stream);

/*
 * MXFP8 dequantize (PR #3203 stacked list: MXFP8 dequantization kernel and
 * the e8m0 -> fp32 scale decode).  y = RNE_bf16(decode(q) * 2^(s-127)),
 * bf16 subnormals kept, overflow to Inf, NaN codes or scale 255 -> NaN.
 *   q uint8 [rows, cols], s scales [rows, cols] (blocks along cols),
 *   y bf16 [rows, cols].  A columnwise tensor is dequantized as the
 *   [cols, rows] matrix it is stored as.  Requires cols % 32 == 0.
 */
int mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, uint16_t* y,
                  mx_stream_t stream);

/* Bytes of device workspace mx_permute needs for these sizes. */
size_t mx_permute_workspace_size(int64_t tokens, int32_t topk, int32_t num_experts);

/*
 * MXFP8 token permute (PR #3203 "Next steps": a token shuffle that stays in
 * MXFP8; TransformerEngine issue #556, first maintainer reply: fp8 data
 * moves as bytes as long as its scales move with it).
 *
 *   q, s          rowwise MX tokens: codes [tokens, cols], scales [tokens, cols]
 *                 (both NULL, with q_out/s_out NULL: metadata only)
 *   expert_ids    int32 [tokens, topk]; flat pair i = t*topk + j
 *   capacity_rows rows of the permuted buffers, >= tokens*topk + 31*num_experts
 *   q_out, s_out  codes [capacity_rows, cols], scales [capacity_rows, cols]
 *   group_offsets int32 [num_experts+1]: expert e owns rows [off[e], off[e+1]);
 *                 every group is padded to a multiple of 32 rows
 *   dst_row       int32 [tokens*topk]: permuted row of pair i (-1 if its id
 *                 is out of range)
 *   src_row       int32 [capacity_rows]: source token of each permuted row,
 *                 -1 for pad rows and rows past the last group
 *   workspace     >= mx_permute_workspace_size(...) bytes of device memory
 * Rows of one expert keep the order of their flat pair index (stable), so
 * the result is deterministic.  Pad rows get codes 0x00 and scales 0x00.
 * Each token's code row and scale bytes are read once and written to its
 * topk rows.  Requires num_experts <= 16384 (MX_EUNSUPPORTED above); q and
 * q_out 16-byte aligned, s and s_out 4-byte aligned.
 */
int mx_permute(const uint8_t* q, const uint8_t* s, int64_t tokens, int64_t cols, const int32_t* expert_ids,
               int32_t topk, int32_t num_experts, int64_t capacity_rows, uint8_t* q_out, uint8_t* s_out,
               int32_t* group_offsets, int32_t* dst_row, int32_t* src_row, void* workspace,
               size_t workspace_bytes, mx_stream_t stream);

/*
 * mx_permute for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, results and checks without `workspace`.  The routing
 * tables live in a library-owned device array of
 * MX_PERMUTE_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held until the
 * process ends; its address is looked up on the first call on each device
 * (hipGetSymbolAddress, no allocation).  Requests whose
 * mx_permute_workspace_size exceeds it return MX_EUNSUPPORTED (use
 * mx_permute then).  All calls on one GPU share that array: calls that
 * overlap in time on one GPU (different streams, or threads without
 * ordering) race and must not be issued; calls on one stream are ordered
 * and safe.  Nothing is carried from one call to the next (every table entry
 * is written before it is read).
 */
#define MX_PERMUTE_NOALLOC_SCRATCH_BYTES (4u << 20)
int mx_permute_noalloc(const uint8_t* q, const uint8_t* s, int64_t tokens, int64_t cols, const int32_t* expert_ids,
                       int32_t topk, int32_t num_experts, int64_t capacity_rows, uint8_t* q_out, uint8_t* s_out,
                       int32_t* group_offsets, int32_t* dst_row, int32_t* src_row, mx_stream_t stream);

/*
 * Block-scaled grouped GEMMs (digest "Key Questions Answered": block-scaled
 * MMA; PR #3203 "Next steps": grouped GEMM on pre-quantized tensors).  All
 * three are C[m, n] = sum_k A[m, k] B[n, k] with both operands contiguous
 * along k and the E8M0 scales applied inside the CDNA4 scaled MFMA;
 * accumulation in fp32.  out_dtype is MX_OUT_BF16 (RNE) or MX_OUT_F32.
 * Sizes: n % 32 == 0, k % 32 == 0, m_cap >= 0, num_groups >= 1.
 *
 * Scales are in the panel layout above, of the whole operand matrix
 * (b_s of W [E, n, k] is scales [E * n, k]).
 * fwd:   a = X_perm rowwise [m_cap, k], b = W rowwise [E, n, k],
 *        out Y [m_cap, n].  Rows of group e multiply W_e; rows outside every
 *        group are not written.
 * dgrad: a = dY rowwise [m_cap, n_c], b = W^T colwise [E, k_o, n_c]
 *        (same call shape as fwd with n = k_o, k = n_c), out dX [m_cap, k_o].
 * wgrad: a = dY^T colwise [n, m_cap], b = X^T colwise [k, m_cap],
 *        out dW [E, n, k]; group e contracts over columns
 *        [off[e], off[e+1]) (multiples of 32, m_cap % 32 == 0); an empty
 *        group writes an exact zero dW_e.
 */
int mx_grouped_gemm_fwd(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                        const int32_t* group_offsets, int32_t num_groups, int64_t m_cap, int64_t n, int64_t k,
                        void* out, int32_t out_dtype, mx_stream_t stream);

int mx_grouped_gemm_dgrad(const uint8_t* dy_q, const uint8_t* dy_s, const uint8_t* wt_q, const uint8_t* wt_s,
                          const int32_t* group_offsets, int32_t num_groups, int64_t m_cap, int64_t n_out,
                          int64_t k_contract, void* dx, int32_t out_dtype, mx_stream_t stream);

int mx_grouped_gemm_wgrad(const uint8_t* dyt_q, const uint8_t* dyt_s, const uint8_t* xt_q, const uint8_t* xt_s,
                          const int32_t* group_offsets, int32_t num_groups, int64_t m_cap, int64_t n, int64_t k,
                          void* dw, int32_t out_dtype, mx_stream_t stream);

/*
 * SwiGLU glue of the expert FFN with the requantize of its result fused in.
 * The expert computation stays in MXFP8 between the GEMMs (digest "Key
 * Questions Answered"; PR #3203 "Next steps": the grouped GEMM takes
 * pre-quantized operands), so the activation goes straight from the gate/up
 * GEMM output to the MX operands of the down GEMM (rowwise, along F) and of
 * its wgrad (columnwise, along the rows).
 *
 *   h      bf16 [rows, 2F]: gate g in columns [0, F), up u in [F, 2F)
 *   a      optional bf16 [rows, F]: A = RNE_bf16(silu(g) * u), silu(g) =
 *          g / (1 + e^-g), computed in fp32
 *   row_q/row_s  rowwise MX of A: codes [rows, F], scales [rows, F]; or NULL
 *   col_q/col_s  columnwise MX of A stored transposed: codes [F, rows],
 *          scales [F, rows]; or NULL (then rows % 32 == 0 is not required)
 * The MX results are exactly the quantize of the bf16 A (whether or not a is
 * written).  Requires F % 32 == 0, rows % 32 == 0 with a columnwise output,
 * at least one output; h 16-byte aligned.  Rows of zeros (the pad rows of a
 * grouped buffer) give zero codes and zero scales.
 */
int mx_swiglu_quantize(const uint16_t* h, int64_t rows, int64_t F, uint16_t* a, uint8_t* row_q, uint8_t* row_s,
                       uint8_t* col_q, uint8_t* col_s, mx_stream_t stream);

/*
 * SwiGLU backward with the requantize of dH fused in (the dgrad operand of
 * the gate/up GEMM rowwise along 2F, its wgrad operand columnwise).
 *   h   bf16 [rows, 2F] (as in the forward), da bf16 [rows, F]
 *   dh  optional bf16 [rows, 2F] = [dg | du], fp32 math, one RNE rounding:
 *       dg = dA u s (1 + g (1 - s)), du = dA silu(g), s = 1 / (1 + e^-g)
 *   row_q/row_s  rowwise MX of dH [rows, 2F]; col_q/col_s columnwise MX of dH
 *       stored transposed [2F, rows]; either pair may be NULL.
 * Same requirements as mx_swiglu_quantize.
 */
int mx_swiglu_bwd_quantize(const uint16_t* h, const uint16_t* da, int64_t rows, int64_t F, uint16_t* dh,
                           uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, uint8_t* col_s, mx_stream_t stream);

/*
 * Weighted unpermute-combine (the step after the down GEMM; the inverse of
 * the MXFP8 token shuffle of PR #3203 "Next steps").
 *   y        bf16 [y_rows, H]: permuted rows (e.g. the down GEMM output)
 *   dst_row  int32 [tokens * topk] from mx_permute
 *   weights  fp32 [tokens, topk], or NULL for all ones (then this is the
 *            backward of the permute: dX[t] = sum_j dX_perm[dst_row[t k + j]])
 *   out      bf16 [tokens, H]: out[t] = RNE_bf16(sum_j w[t,j] y[dst_row[t k + j]]),
 *            accumulated in fp32 with fused multiply-adds, j ascending
 * A dst_row entry outside [0, y_rows) contributes nothing.  Requires
 * H % 32 == 0, topk >= 1; y and out 16-byte aligned.
 */
int mx_combine(const uint16_t* y, int64_t y_rows, int64_t H, const int32_t* dst_row, const float* weights,
               int64_t tokens, int32_t topk, uint16_t* out, mx_stream_t stream);

/*
 * Backward of the weighted combine with the quantize of the permuted
 * gradient fused in (the dgrad operand of the down GEMM rowwise along H,
 * its wgrad operand columnwise along the rows).
 *   dout     bf16 [tokens, H]; weights fp32 [tokens, topk]
 *   dst_row  int32 [tokens * topk], src_row int32 [rows] from mx_permute
 *   dy       optional bf16 [rows, H]: dY[dst_row[i]] = RNE_bf16(fl32(w[i] *
 *            dOut[i / topk])) (one fp32 product); rows no pair maps to are 0
 *   row_q/row_s  rowwise MX of dY [rows, H]; col_q/col_s columnwise MX of dY
 *            stored transposed [H, rows]; either pair may be NULL.
 * Row r finds its pair as the j with dst_row[src_row[r] * topk + j] == r; a
 * row without one is zero.  Requires H % 32 == 0, topk >= 1, rows % 32 == 0
 * with a columnwise output; dout 16-byte aligned.  With tokens == 0, dout,
 * weights and dst_row may be NULL (every row is zero).
 */
int mx_combine_bwd_quantize(const uint16_t* dout, const float* weights, const int32_t* dst_row,
                            const int32_t* src_row, int64_t tokens, int32_t topk, int64_t rows, int64_t H, uint16_t* dy,
                            uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, uint8_t* col_s, mx_stream_t stream);

/*
 * Router: top-k expert choice with softmax weights, in front of mx_permute.
 * The pages give no router formula (digest "Overview": an MXFP8 MoE layer);
 * the reading: a token's experts are its k largest logits, equal logits to
 * the lower expert id, in decreasing order; the weights are the softmax of
 * the k chosen logits (fp32, renormalised over the chosen experts).
 *   logits      fp32 [tokens, num_experts]
 *   expert_ids  int32 [tokens, topk] (the layout mx_permute takes)
 *   weights     fp32 [tokens, topk] (the layout mx_combine takes)
 * Requires 1 <= topk <= num_experts; num_experts <= 1024 and topk <= 64
 * (else MX_EUNSUPPORTED).  NaN logits are outside the contract.
 */
int mx_route_topk(const float* logits, int64_t tokens, int32_t num_experts, int32_t topk, int32_t* expert_ids,
                  float* weights, mx_stream_t stream);

/*
 * Router backward through the weighted combine: with out[t] = sum_j w[t,j]
 * y[dst_row[t topk + j]],
 *   dw[t,j]          = <dout[t], y[dst_row[t topk + j]]>  (fp32 [tokens, topk])
 *   dlogits[t, e]    = w[t,j] (dw[t,j] - sum_i w[t,i] dw[t,i]) for e = expert_ids[t,j],
 *                      0 for experts not chosen  (fp32 [tokens, num_experts])
 *   dout bf16 [tokens, H]; y bf16 [y_rows, H] (the combine's input rows);
 *   dst_row int32 [tokens * topk]; weights fp32 [tokens, topk].
 * Either output may be NULL (not both); expert_ids is needed with dlogits.
 * fp32 accumulation.  Requires H % 32 == 0, topk <= 64; dout and y 16-byte
 * aligned.  A dst_row entry outside [0, y_rows) contributes nothing.
 */
int mx_router_bwd(const uint16_t* dout, const uint16_t* y, int64_t y_rows, int64_t H, const int32_t* dst_row,
                  const int32_t* expert_ids, const float* weights, int64_t tokens, int32_t num_experts, int32_t topk,
                  float* dw, float* dlogits, mx_stream_t stream);

/*
 * BF16 baseline of the expert step: the same permute and grouped GEMMs with
 * bf16 operands, so the MXFP8 path can be timed against the BF16 MoE layer
 * the digest page compares with (Overview and Key Statistics & Figures: the
 * MoE-layer speedup of MXFP8 over BF16).
 *
 * mx_bf16_gather: row gather and/or transpose of bf16 tensors.
 *   x         bf16 [batch, rows, cols]
 *   gather    optional int32 [rows_out] (batch must be 1): output row r is
 *             source row gather[r], or a zero row when gather[r] < 0 or
 *             >= rows.  Without a gather, output row r is source row r for
 *             r < rows and zero after (rows_out >= rows).
 *   out_rows  bf16 [batch, rows_out, cols], or NULL
 *   out_cols  the same rows transposed, bf16 [batch, cols, rows_out], or NULL
 * The permute of the BF16 step is mx_permute with NULL tensors (routing
 * metadata only) followed by this call with gather = src_row.  Requires
 * cols % 32 == 0, rows_out % 32 == 0, at least one output, 16-byte aligned
 * buffers.  Bit-exact copies (no arithmetic).
 */
int mx_bf16_gather(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, const int32_t* gather,
                   int64_t rows_out, uint16_t* out_rows, uint16_t* out_cols, mx_stream_t stream);

/*
 * BF16 grouped GEMMs: the three NT products of mx_grouped_gemm_fwd / dgrad /
 * wgrad with bf16 operands (no scales), fp32 accumulation, bf16 (RNE) or
 * fp32 output; same groups, shapes, limits and pad-row behaviour.
 *   fwd:   a = X_perm bf16 [m_cap, k], b = W bf16 [E, n, k], out [m_cap, n]
 *   dgrad: a = dY bf16 [m_cap, n_c], b = W^T bf16 [E, k_o, n_c], out [m_cap, k_o]
 *   wgrad: a = dY^T bf16 [n, m_cap], b = X_perm^T bf16 [k, m_cap], out [E, n, k]
 * Operands must be 16-byte aligned.
 */
int mx_bf16_grouped_gemm_fwd(const uint16_t* a, const uint16_t* b, const int32_t* group_offsets, int32_t num_groups,
                             int64_t m_cap, int64_t n, int64_t k, void* out, int32_t out_dtype, mx_stream_t stream);

int mx_bf16_grouped_gemm_dgrad(const uint16_t* dy, const uint16_t* wt, const int32_t* group_offsets,
                               int32_t num_groups, int64_t m_cap, int64_t n_out, int64_t k_contract, void* dx,
                               int32_t out_dtype, mx_stream_t stream);

int mx_bf16_grouped_gemm_wgrad(const uint16_t* dyt, const uint16_t* xt, const int32_t* group_offsets,
                               int32_t num_groups, int64_t m_cap, int64_t n, int64_t k, void* dw, int32_t out_dtype,
                               mx_stream_t stream);

/*
 * Measurement helpers (not part of the MXFP8 path): the ceilings the
 * benchmark reports its roofline fractions against, next to the published
 * peaks.
 *
 * mx_ceiling_copy: a streaming copy of `bytes` (a multiple of 4096; src
 *   and dst 16-byte aligned device buffers that do not overlap), 16-byte
 *   non-temporal loads and stores, one per thread -- the HBM read + write
 *   rate an HBM-bound kernel can reach.
 * mx_ceiling_tile_pattern: the memory traffic of a quantize that writes
 *   both orientations, without its arithmetic: x [rows, cols] bf16 is read
 *   in 128 x 128 tiles as the tile quantizer reads it, and each tile is
 *   written as 1 byte per element to row_out [rows, cols] (row-major, 128
 *   bytes per tile row) and to col_out [cols, rows] (column-major, 128
 *   bytes per tile column); 4 * rows * cols bytes moved, the fused row+col
 *   quantize's traffic minus its scale bytes.  rows and cols multiples of
 *   128; the three device buffers 16-byte aligned and not overlapping.
 * mx_ceiling_mfma: `workgroups` workgroups of 256 threads, each wave running
 *   `iters` rounds of 16 independent V_MFMA_SCALE_F32_32X32X64_F8F6F4 on
 *   register operands in the grouped GEMM's register pattern (4 A and 4 B
 *   fragments, one wave per SIMD); random_operands != 0 fills them with
 *   random E4M3 codes and scale bytes (the switching power of real data,
 *   which lowers the clock the part sustains), 0 with near-constant codes.
 *   It performs workgroups * 4 * iters * 16 * 131072 FLOPs and writes one
 *   float per thread to out [workgroups * 256].
 */
int mx_ceiling_copy(const void* src, void* dst, int64_t bytes, mx_stream_t stream);
int mx_ceiling_tile_pattern(const void* x, void* row_out, void* col_out, int64_t rows, int64_t cols,
                            mx_stream_t stream);
int mx_ceiling_mfma(float* out, int32_t workgroups, int32_t iters, int32_t random_operands, mx_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXMOE_H */
