/*
 * awq_w4a16.h - C ABI of the fused AWQ W4A16 linear for AMD Instinct MI355X (gfx950).
 *
 *   y[M, N] = x[M, K] . W[K, N] + bias[N],
 *   W[k, n] = (q[k, n] - z[k / g, n]) * s[k / g, n]
 *
 * The weights arrive in the AWQ "GEMM" checkpoint layout, consumed as stored:
 *   qweight  int32 [K, N/8]  row-major; bits 4i..4i+3 of word (k, c) hold the
 *                            code of column 8c + ORDER[i], ORDER = {0,2,4,6,1,3,5,7}
 *                            (tensref.org "AWQ" format page, Reader; GPTQModel wiki
 *                            "AWQ", section "Saved formats and packing")
 *   qzeros   int32 [G, N/8]  zero codes packed the same way; subtracted as stored,
 *                            never plus one (format page, rule AWQ-005)
 *   scales   fp16  [G, N]    row k / g scales input row k (format page, Reader)
 *   bias     fp16  [N]       optional (format page, tensor table)
 *   x        fp16  [M, K]    activations, row-major
 *   y        fp16  [M, N]    output, row-major
 * with g = group_size and G = K / g; group_size == -1 means one group spanning all
 * K rows, G = 1 (GPTQModel wiki "AWQ", section "Group quantization and zero points").
 *
 * Conventions shared by every entry point:
 *   - Pointers to tensor data are DEVICE pointers of the current HIP device; fp16
 *     tensors are passed as raw 16-bit storage (IEEE binary16).
 *   - The caller owns every buffer.  The library keeps no pointer to them after the
 *     call returns.  Outputs must not alias inputs.
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream); the
 *     library never synchronises the stream except when it must grow its own
 *     workspace (see awq_gemm).
 *   - Every argument is checked before anything is enqueued; a failed check returns
 *     a negative status and enqueues nothing.  No entry point aborts, prints or
 *     throws.  awq_status_string() names a status.
 *   - Entry points are safe to call from several host threads.
 */
#ifndef AWQ_W4A16_H
#define AWQ_W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* a hipStream_t */

enum awq_status {
  AWQ_OK = 0,
  AWQ_ERR_NULL = -1,        /* a required pointer is NULL */
  AWQ_ERR_SHAPE = -2,       /* tensor shapes disagree with K, N, group_size, or N % 8 != 0 */
  AWQ_ERR_GROUP = -3,       /* group_size is neither -1 nor a positive divisor of K */
  AWQ_ERR_ALIGN = -4,       /* a tensor base pointer is not 16-byte aligned */
  AWQ_ERR_UNSUPPORTED = -5, /* a valid layer outside the kernels' limits (below) */
  AWQ_ERR_HIP = -6          /* the HIP runtime reported an error */
};

/* Human-readable name of a status code; never NULL, static storage. */
const char* awq_status_string(int status);

/*
 * Format rules of the GEMM pack, host-only (touches no device).
 * Source: GPTQModel wiki "AWQ", section "Saved formats and packing" (shapes,
 * INT4 packing needs N % 8 == 0) and section "Group quantization and zero points"
 * (-1 = one group; positive sizes must fit K).  Shapes that do not divide are
 * rejected, never truncated.
 *   K, N          in_features, out_features (both >= 1, N % 8 == 0)
 *   group_size    -1 or a positive divisor of K
 *   *_rows/_cols  the caller's tensor shapes; qweight [K, N/8], qzeros [G, N/8],
 *                 scales [G, N]
 *   bias_len      N, or -1 when there is no bias
 * Returns AWQ_OK, AWQ_ERR_SHAPE or AWQ_ERR_GROUP.
 */
int awq_validate_pack(int64_t K, int64_t N, int64_t group_size,
                      int64_t qweight_rows, int64_t qweight_cols,
                      int64_t qzeros_rows, int64_t qzeros_cols,
                      int64_t scales_rows, int64_t scales_cols,
                      int64_t bias_len);

/*
 * Kernel limits on top of the format rules (AWQ_ERR_UNSUPPORTED otherwise):
 *   K % 32 == 0, N % 32 == 0, group_size == -1 or group_size % 32 == 0,
 *   K, N <= 2^24, M <= 2^24,
 * and every launch of awq_gemm's plan for the shape within the hardware's grid limits
 * (under 2^32 work-items along x, 2^16 workgroups along y) and the kernels' 32-bit
 * offsets (256-row tiles, taken above 128 rows, address a tile's x rows with 32-bit
 * byte offsets: K < 2^23 there).  Plans assume the current device's compute units
 * (256 when no device is visible).
 * Host-only check; returns AWQ_OK, AWQ_ERR_SHAPE, AWQ_ERR_GROUP or AWQ_ERR_UNSUPPORTED.
 */
int awq_check_limits(int64_t M, int64_t K, int64_t N, int64_t group_size);

/*
 * Dequantise the packed weight to float32:  out[k, n] = (float)(q - z) * (float)s.
 * Source: tensref.org "AWQ" format page, Reader (group row k / group_size, no +1 on
 * zeros); orientation [K, N] as multiplied by x (the page's reader returns the
 * transpose, [N, K]).  (q - z) has at most 4 significant bits and s 11, so the
 * product is exact in float32: the result is bit-identical to any correct
 * implementation, including the signed zero of (q - z) == 0 with s < 0.
 *   qweight, qzeros, scales_f16   device, layouts as above
 *   out                           device float32 [K, N], written in full
 * Returns AWQ_OK or an error status (nothing enqueued on error).
 */
int awq_dequant(const int32_t* qweight, const int32_t* qzeros, const void* scales_f16,
                int64_t K, int64_t N, int64_t group_size, float* out,
                struct ihipStream_t* stream);

/*
 * Dequantise the packed weight to fp16:  out[k, n] = fp16((float)(q - z) * (float)s),
 * the exact product of awq_dequant rounded once to nearest even.  This is the weight
 * of the dequantize-then-dense-matmul path the pages use for large batches (vLLM
 * article, section 5.3; GPTQModel wiki "AWQ", section "Native GEMM": above its row
 * limit the native path dequantises and calls a dense matmul), provided so that a
 * caller can run that path, or compare it with awq_gemm, on the same layout.
 *   qweight, qzeros, scales_f16   device, layouts as above
 *   out_f16                       device fp16 [K, N], written in full
 * Returns AWQ_OK or an error status (nothing enqueued on error).
 */
int awq_dequant_f16(const int32_t* qweight, const int32_t* qzeros, const void* scales_f16,
                    int64_t K, int64_t N, int64_t group_size, void* out_f16,
                    struct ihipStream_t* stream);

/*
 * Fused linear y = x . dequant(W) + bias, accumulated in float32 and rounded once
 * to fp16 (round to nearest even) after the bias is added.
 * Source: GPU LLM serving-stack blog, section 1.2 (W4A16: packed weights are
 * unpacked and dequantised on chip inside the matrix multiply, activations stay
 * 16-bit), with the dequant of the format page's Reader; fp32 accumulation as in
 * the GPTQModel wiki "AWQ", sections "Native GEMM" and "Triton GEMM and dispatch
 * policy".
 *   x_f16       device fp16 [M, K]
 *   qweight     device int32 [K, N/8];  qzeros int32 [G, N/8];  scales fp16 [G, N]
 *   bias_f16    device fp16 [N], or NULL for no bias
 *   y_f16       device fp16 [M, N], written in full
 * M == 0 returns AWQ_OK and enqueues nothing (GPTQModel wiki, "Native GEMM": empty
 * input launches no kernel).  Kernel families are chosen by M: bandwidth-bound
 * streaming kernels for small M (the decode family for one to four rows, the skinny
 * family up to 16 rows and where the decode family's limits do not fit) and an MFMA
 * tile family above (awq_gemm_plan reports the choice).  In the tile family a partly filled last 256-row
 * tile that would take one more round of the compute units runs as a second launch
 * of its own (awq_gemm_plan_tail).  The result is deterministic: the same inputs give
 * the same bits on every call.  NaN and infinities in x, scales or bias propagate as
 * float32 accumulation would propagate them.
 * Workspace: the small-M families split K across workgroups and combine the partial
 * sums through a library-owned device buffer, one per (device, stream): integer
 * fixed-point words (order-independent, hence reproducible) or fp32 partials summed
 * in a fixed order.  The first call on a (device, stream) that needs a larger buffer
 * allocates it; later calls allocate nothing, so run one eager call of the largest
 * shape before capturing a stream into a graph.  A call that would have to grow the
 * buffer while its stream is being captured fails with AWQ_ERR_UNSUPPORTED.  A
 * replaced buffer is kept (a graph captured earlier may still replay into it) until
 * awq_release_workspace().  Calls that share a (device, stream) workspace must not run
 * concurrently, e.g. two graphs captured on the same stream replayed at once on two
 * other streams.
 * Returns AWQ_OK or an error status.
 */
int awq_gemm(const void* x_f16, const int32_t* qweight, const int32_t* qzeros,
             const void* scales_f16, const void* bias_f16,
             int64_t M, int64_t K, int64_t N, int64_t group_size,
             void* y_f16, struct ihipStream_t* stream);

/*
 * awq_gemm for callers that cannot allocate device memory (code under HIP graph
 * capture on a fresh stream, serving loops that must not call hipMalloc, harnesses that
 * forbid it).  Same arguments, plans, kernels and results as awq_gemm; the split-K
 * buffers come from one statically sized device array of the library (64 MiB per GPU,
 * held from the first call on that GPU until the process ends: 2 MiB of zero-maintained
 * fixed-point words, 62 MiB of fp32 partials), never from hipMalloc.  The first call on
 * a device clears the word region with a small kernel on `stream`.  A shape whose plan
 * needs more than either region returns AWQ_ERR_UNSUPPORTED before enqueueing anything
 * (awq_gemm_plan's workspace_bytes shows the need).  Every call on one GPU shares that
 * array: calls that overlap in time on one GPU (two streams, or concurrently replayed
 * graphs) race and must not be issued; consecutive calls in any stream order are fine.
 * Returns AWQ_OK or an error status.
 */
int awq_gemm_noalloc(const void* x_f16, const int32_t* qweight, const int32_t* qzeros,
                     const void* scales_f16, const void* bias_f16,
                     int64_t M, int64_t K, int64_t N, int64_t group_size,
                     void* y_f16, struct ihipStream_t* stream);

/*
 * Frees every workspace buffer the library holds, on every device: the current
 * per-(device, stream) buffers and those replaced by larger ones.  It synchronises each
 * device first.  The caller guarantees that no graph captured from a library call will
 * be replayed afterwards (its workspace address would dangle); later calls allocate
 * afresh.  Not safe to call concurrently with other library calls.
 * Returns AWQ_OK, or AWQ_ERR_HIP if the runtime reported an error (the buffers that
 * could be freed are freed either way).
 */
int awq_release_workspace(void);

/*
 * awq_gemm with bfloat16 activations: x, bias and y are bfloat16 (raw 16-bit
 * patterns); qweight, qzeros and the fp16 scales are the same GEMM pack.  The GEMM
 * kernel's declared contract takes FP16 or BF16 inputs (GPTQModel wiki "AWQ",
 * section "Selection and compatibility").  Accumulation is fp32; y is rounded once
 * (to nearest even) to bfloat16 after the bias is added.  Small M multiplies
 * x . (q - z) exactly and scales each group in fp32; large M feeds the MFMA with the
 * weight rounded once to bfloat16, bf16((q - z) s).  Limits, plans, determinism and
 * the workspace rule are those of awq_gemm, except that small-M plans with K splits
 * always combine them through fp32 partials and a second kernel (the fixed-point
 * accumulation of awq_gemm relies on fp16's range).
 *   x_bf16      device bfloat16 [M, K]
 *   bias_bf16   device bfloat16 [N], or NULL
 *   y_bf16      device bfloat16 [M, N], written in full
 * Returns AWQ_OK or an error status.
 */
int awq_gemm_bf16(const void* x_bf16, const int32_t* qweight, const int32_t* qzeros,
                  const void* scales_f16, const void* bias_bf16,
                  int64_t M, int64_t K, int64_t N, int64_t group_size,
                  void* y_bf16, struct ihipStream_t* stream);

/*
 * Routed experts (MoE).  vLLM's AWQ support runs a routed-expert layer on a 4-bit
 * WNA16 MoE kernel over per-expert qweight / qzeros / scales (vLLM article, section
 * 5.4).  Here: T tokens, each routed to topk experts of E; routed slot s = t * topk
 * + j (token t = s / topk) computes
 *   y[s, :] = x[t, :] . dequant(W[expert_ids[s]])      (fp16, fp32 accumulation)
 * The expert's activation function and the weighted sum over a token's topk slots
 * come after this product and are not part of it.
 *
 * awq_moe_tiles: table entries for S = T * topk slots, E experts and tiles of
 * block_rows rows: ceil(S / block_rows) + E (an upper bound of sum over experts of
 * ceil(count / block_rows)); -1 for invalid arguments.  Host-only.
 *
 * awq_moe_align: counting sort of the S slots by expert (device).
 *   expert_ids    device int32 [S]; ids outside [0, E) are not routed
 *   offsets       device int32 [E + 1]: expert e owns sorted rows offsets[e] .. offsets[e+1]-1
 *   sorted_slots  device int32 [S]: slot ids grouped by expert (order within an
 *                 expert unspecified; entries past offsets[E] are not written)
 *   tile_table    device int32 [awq_moe_tiles(S, E, block_rows)][4], 16-byte aligned:
 *                 (expert, first sorted row, rows, 0) per tile of at most block_rows
 *                 rows, then (-1, 0, 0, 0)
 *   1 <= E <= 1024, S < 2^30.  Returns AWQ_OK or an error status.
 *
 * awq_moe_gemm: the grouped product, one call.  Few tokens (up to 16; up to 64 when
 * the experts average at most 8 slots and hold at least 2 MB of packed weight each):
 * one launch of the skinny kernel over (16-token chunk, expert, column tile) blocks,
 * each block's rows being its chunk of the tokens routed to its expert, experts
 * without a slot skipped (plus the split reduce for plans of three or more rows); otherwise:
 * alignment, then the MFMA tile kernel, in which each workgroup gathers the x rows
 * of one expert's tile and scatters its y rows (one launch, or two when the table
 * has 256-row tiles: full tiles first, then each expert's last few rows in 64-row
 * parts).
 *   x_f16        device fp16 [T, K]
 *   qweight      device int32 [E, K, N/8];  qzeros int32 [E, G, N/8];  scales fp16 [E, G, N]
 *   expert_ids   device int32 [T * topk]
 *   y_f16        device fp16 [T * topk, N]; rows of slots with an id outside [0, E)
 *                are left unwritten
 * Limits: those of awq_gemm with M = T * topk, plus 1 <= E <= 1024, topk >= 1 and
 * x below 4 GiB.  T == 0 enqueues nothing.  The alignment and the split-K
 * accumulators or partials live in the same library-owned per-(device, stream)
 * workspace as awq_gemm's, with the same allocation rule.  The result is
 * deterministic (each row depends only on its slot; splits meet in a fixed order).
 * Returns AWQ_OK or an error status.
 */
int64_t awq_moe_tiles(int64_t S, int64_t E, int64_t block_rows);
int awq_moe_align(const int32_t* expert_ids, int64_t S, int64_t E, int64_t block_rows,
                  int32_t* offsets, int32_t* sorted_slots, int32_t* tile_table,
                  struct ihipStream_t* stream);
int awq_moe_gemm(const void* x_f16, const int32_t* qweight, const int32_t* qzeros,
                 const void* scales_f16, const int32_t* expert_ids,
                 int64_t T, int64_t topk, int64_t E, int64_t K, int64_t N, int64_t group_size,
                 void* y_f16, struct ihipStream_t* stream);

/*
 * Round-to-nearest writer of the GEMM pack: quantise an fp16 weight in groups of
 * group_size input rows per output column.  Source: GPTQModel wiki "AWQ", section
 * "Group quantization and zero points" (both quantizers, the clamp of the zero, the
 * 1e-5 floor of the range, -1 = one group) and section "Saved formats and packing"
 * (the nibble order above).  With w the weights of one (group, column):
 *   sym == 0 (asymmetric): s = fp16(max(max w - min w, 1e-5) / 15),
 *                          z = clamp(-round(min w / s), 0, 15),
 *                          q = clamp(round(w / s) + z, 0, 15)
 *   sym == 1 (symmetric):  s = fp16(max(max |w|, 1e-5) / 7), z = 8,
 *                          q = clamp(round(w / s), -8, 7) + 8
 * The scale is computed in float32 and rounded once (to nearest even) to the stored
 * fp16 value; both divisions are float32 divisions, correctly rounded, by that
 * stored value; round() is to nearest with ties to even.  The output is therefore
 * unique: awq_dequant of it gives (q - z) * s for the scale a reader actually uses.
 *   w_f16        device fp16 [K, N], row-major, in the orientation x . W multiplies
 *                (input features by output features; a [N, K] nn.Linear weight must
 *                be transposed first); finite values
 *   K, N, group_size   the format rules of awq_validate_pack (K, N <= 2^24)
 *   sym          0 or 1
 *   qweight      device int32 [K, N/8];  qzeros int32 [G, N/8];  scales_f16 fp16 [G, N];
 *                all written in full
 * Groups of up to 256 rows are quantised in one pass over w.  Longer groups
 * (including group_size == -1 on K > 256) read w twice and keep per-chunk minima
 * and maxima (K/128 x N x 4 bytes) in the same library-owned per-(device, stream)
 * workspace awq_gemm uses, with the same allocation rule: the first call that needs
 * a larger buffer allocates it and synchronises the stream.
 * Returns AWQ_OK or an error status (nothing enqueued on error).
 */
int awq_quantize_rtn(const void* w_f16, int64_t K, int64_t N, int64_t group_size, int sym,
                     int32_t* qweight, int32_t* qzeros, void* scales_f16,
                     struct ihipStream_t* stream);

/*
 * The launch plan awq_gemm would use for this shape (host-only, no device work).
 *   family   0 = skinny split-K family, 1 = MFMA tile family, 2 = decode family
 *   splits   number of K splits across workgroups (1 = none)
 *   grid_x, grid_y, block   launch geometry of the main kernel (tile family: of the
 *                           first launch, over rows 0 .. M - rows of awq_gemm_plan_tail)
 *   workspace_bytes         device workspace the call needs (0 if none)
 * Any output pointer may be NULL.  Returns AWQ_OK or the awq_check_limits status.
 */
int awq_gemm_plan(int64_t M, int64_t K, int64_t N, int64_t group_size,
                  int* family, int* splits, int* grid_x, int* grid_y, int* block,
                  int64_t* workspace_bytes);

/*
 * The second tile launch of awq_gemm for this shape, over the last rows (host-only).
 *   rows     rows of that launch, the last rows of x and y (0: one launch only)
 *   splits, grid_x, grid_y, block   as in awq_gemm_plan, for that launch
 * awq_gemm_plan's workspace_bytes covers both launches (they run in stream order
 * and share it).  Any output pointer may be NULL.  Returns AWQ_OK or the
 * awq_check_limits status.
 */
int awq_gemm_plan_tail(int64_t M, int64_t K, int64_t N, int64_t group_size,
                       int64_t* rows, int* splits, int* grid_x, int* grid_y, int* block);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_W4A16_H */
