/*
 * ggq.h -- C ABI of the MI355X (gfx950) GGUF block-quantized matmul library.
 *
 * Matrix multiplication against GGUF block-quantized weights (Q8_0, Q4_K,
 * Q6_K, and Q4_0, Q5_K: types PR #690 lists in its Summary, with block
 * layouts from the public GGUF format) with activations quantized on the fly
 * to q8_1 blocks; results come
 * out in the activation dtype (or the requested output dtype) with fp32
 * accumulation.  This is the operation FreeToken PR #690 "feat(gguf): serve
 * GGUF checkpoints on vendored ggml-cuda kernels" describes in "What the ggml
 * patch changes" (fp32/bf16 activations quantized directly to q8_1, fp32
 * accumulation, MMVQ for small batches and MMQ above, a routed-MoE grid over
 * only the (expert, column tile) pairs that hold routes with no host sync).
 *
 * Conventions for every entry point:
 *   - All buffers are device memory owned by the caller (the library
 *     allocates nothing on the device and keeps no pointer after returning).
 *     Base pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void * (so that this header needs
 *     no HIP include; NULL = the default stream).  Calls are asynchronous on
 *     it and never synchronize the host.
 *   - Weights are row-major GGUF blocks: row n of an N x K matrix starts at
 *     byte n * ggq_row_bytes(type, K).  Kernels never read outside
 *     [W, W + N * row_bytes) (no tail padding needed); all offsets are 64-bit.
 *   - Element types: GGQ_F32 = IEEE fp32, GGQ_BF16 = bfloat16, GGQ_F16 = IEEE
 *     binary16 (16-bit outputs rounded to nearest even from the fp32 result;
 *     fp16 overflows to inf), GGQ_Q8_1 = q8_1 blocks (input; and the routed
 *     output of ggq_mul_mat_id).  fp16 activations and outputs are among the
 *     variants PR #690 serves ("What the ggml patch changes").
 *   - q8_1 block (40 bytes, 32 values): float d = amax/127 (fp32 division),
 *     float s = d * (sum of the quants), int8 qs[32] = x/d (fp32 division)
 *     rounded half away from zero; an all-zero block has d = s = 0.
 *   - Return value: GGQ_OK or an error code; ggq_last_error() gives a
 *     message for the calling thread's last failure.  All checks are on
 *     the host and nothing is launched when a check fails.  M, N or T equal
 *     to 0 is a valid no-op.
 */
#ifndef GGQ_H
#define GGQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GGUF tensor type ids (public GGUF numbering). */
typedef enum { GGQ_Q4_0 = 2, GGQ_Q8_0 = 8, GGQ_Q4_K = 12, GGQ_Q5_K = 13, GGQ_Q6_K = 14 } ggq_type;
typedef enum { GGQ_F32 = 0, GGQ_BF16 = 1, GGQ_Q8_1 = 2, GGQ_F16 = 3 } ggq_dtype;
/* Kernel choice: AUTO picks MMVQ for few activation rows, MMQ above. */
typedef enum { GGQ_PATH_AUTO = 0, GGQ_PATH_MMVQ = 1, GGQ_PATH_MMQ = 2 } ggq_path;
typedef enum { GGQ_EPI_NONE = 0, GGQ_EPI_SWIGLU = 1 } ggq_epilogue;
typedef enum {
    GGQ_OK = 0,
    GGQ_ERR_INVALID = 1,     /* bad argument: null pointer, bad K, shape, stride, alignment */
    GGQ_ERR_UNSUPPORTED = 2, /* type / dtype / path combination not provided (no fallback) */
    GGQ_ERR_WORKSPACE = 3,   /* workspace smaller than the matching *_ws() size */
    GGQ_ERR_HIP = 4          /* a HIP launch failed */
} ggq_status;

/* Bytes of one row of K weights of `type`; 0 if K is not a multiple of the
 * block length (32 for Q4_0 / Q8_0, 256 for Q4_K / Q5_K / Q6_K) or the type
 * is unknown.  Block bytes: Q4_0 18, Q8_0 34, Q4_K 144, Q5_K 176, Q6_K 210. */
size_t ggq_row_bytes(int type, int64_t K);

/* Bytes of M rows of K activations as q8_1 blocks: M * (K/32) * 40. */
size_t ggq_q8_1_bytes(int64_t M, int64_t K);

/* q8_1 quantization of activations (PR #690, "What the ggml patch changes":
 * activations quantized to q8_1 directly).
 *   x   : [M][ldx] elements of xdt (GGQ_F32, GGQ_BF16 or GGQ_F16); K % 32 == 0, ldx >= K.
 *   q8  : output, [M][K/32] blocks of 40 bytes (ggq_q8_1_bytes(M, K)).
 * Bit-exact: the same blocks as the definition above. */
int ggq_quantize_q8_1(const void *x, int xdt, int64_t M, int64_t K, int64_t ldx,
                      void *q8, void *stream);

/* Dense quantized matmul: y[m][n] = sum_k W[n][k] * x[m][k] for n < N.
 *   W   : N rows of K weights of type wt (Q4_0, Q8_0, Q4_K, Q5_K, Q6_K).
 *   x   : [M][ldx] of xdt (GGQ_F32 / GGQ_BF16 / GGQ_F16), or, with xdt = GGQ_Q8_1,
 *         M rows of K/32 q8_1 blocks (ldx ignored) -- one quantization can
 *         be reused for several weight matrices (PR #690, second item).
 *   y   : [M][ldy] of ydt (GGQ_F32 / GGQ_BF16 / GGQ_F16), ldy >= N; columns >= N are
 *         not written.
 *   ws  : workspace of at least ggq_mul_mat_ws(...) bytes (may be NULL when
 *         that is 0).
 *   path: AUTO, or force MMVQ / MMQ (MMQ: every type; for Q4_0 and Q8_0
 *         only when K % 256 == 0, else AUTO takes MMVQ at every M).  MMVQ
 *         holds one row of K activations in 64 KB of LDS: it takes K up to
 *         43520 for Q6_K and about 52K for the other types; AUTO goes to MMQ
 *         above that, and a call that would need MMVQ for a longer K (forced
 *         MMVQ, or Q4_0 / Q8_0 with K % 256 != 0) returns
 *         GGQ_ERR_UNSUPPORTED before launching anything.
 * fp32 accumulation; per-block integer dots are exact. */
size_t ggq_mul_mat_ws(int wt, int64_t N, int64_t K, int xdt, int64_t M, int path);
int ggq_mul_mat(int wt, const void *W, int64_t N, int64_t K,
                const void *x, int xdt, int64_t M, int64_t ldx,
                void *y, int ydt, int64_t ldy,
                void *ws, size_t ws_bytes, int path, void *stream);

/* Routed-expert matmul (MoE mul_mat_id).  FreeToken PR #690, "What the ggml
 * patch changes": the routed MMQ grid covers only the (expert, column tile)
 * pairs that actually receive routes, and the host never waits for the
 * routing to be known.  Fused GLU and the MoE weighted sum are ops the same
 * PR lists beside mul_mat ("Our own code next to it").
 *   W            : E experts; expert e starts at byte e * expert_stride and
 *                  holds N rows of K weights of type wt.  expert_stride >=
 *                  N * row_bytes and a multiple of 16.
 *   x            : x_per_route == 0: [T][K] (each route of token t uses x[t]);
 *                  x_per_route == 1: [T][top_k][K] (route (t,k) uses x[t][k]).
 *                  Element type xdt (GGQ_F32 / GGQ_BF16 / GGQ_F16), rows contiguous; or
 *                  xdt = GGQ_Q8_1: the same rows as K/32 q8_1 blocks each.
 *   ids          : [T][top_k] int32 expert ids.  id < 0: inactive route
 *                  (contributes nothing).  id >= E: skipped and counted in
 *                  the uint32 at workspace offset 0 (readable after the call).
 *                  Repeated ids within a token are independent routes.
 *   epi          : GGQ_EPI_SWIGLU: o' = silu(o[:N/2]) * o[N/2:] (gate rows
 *                  first, then up rows), N' = N/2 (N even).  Otherwise N' = N.
 *   route_w      : NULL: y is [T][top_k][N'] (inactive routes -> 0);
 *                  else [T][top_k] fp32 weights and y is [T][N'] =
 *                  sum_k route_w[t][k] * o'[t][k] over the active routes,
 *                  in ascending k with fp32 accumulation (deterministic: the
 *                  per-route outputs go to the workspace, then one pass sums
 *                  them per token).  Each route output is held in the output
 *                  dtype first: fp32 for GGQ_F32, else rounded to bf16 / fp16
 *                  (an intermediate in the activation dtype, FreeToken PR #690,
 *                  "Changes").
 *   y            : output of ydt (GGQ_F32 / GGQ_BF16 / GGQ_F16), contiguous.  With
 *                  route_w == NULL, ydt may be GGQ_Q8_1 (N' % 32 == 0): y is
 *                  [T][top_k][N'/32] q8_1 blocks, the blocks ggq_quantize_q8_1
 *                  makes from the plain output (bf16 / fp16 for bf16 / fp16
 *                  x, else fp32),
 *                  bit for bit -- the SwiGLU h in the down projection's own
 *                  input format (PR #690 keeps intermediates in the activation
 *                  dtype and quantizes activations straight to q8_1).  The MMQ
 *                  path quantizes in its epilogue; the MMVQ path stages the
 *                  plain output in the workspace and quantizes after.
 *   ws           : at least ggq_mul_mat_id_ws(...) bytes (includes that
 *                  staging for MMVQ-path calls without route weights).
 *                  ggq_mul_mat_id_ws takes the call's shape and `weighted`
 *                  (nonzero when route_w will be non-NULL: the per-route
 *                  outputs of the weighted sum live in the workspace).
 *   path         : AUTO takes the MMVQ kernel while the routes per expert
 *                  (T * top_k / E) stay at or below 12 and MMQ above (MMVQ
 *                  alone where MMQ has no kernel, as for ggq_mul_mat), or
 *                  force MMVQ / MMQ.
 * Tokens, routes and tiles are grouped on the device; no host sync. */
size_t ggq_mul_mat_id_ws(int wt, int64_t E, int64_t N, int64_t K, int xdt,
                         int64_t T, int x_per_route, int64_t top_k,
                         int epi, int weighted, int path);
int ggq_mul_mat_id(int wt, const void *W, int64_t E, int64_t N, int64_t K,
                   int64_t expert_stride,
                   const void *x, int xdt, int64_t T, int x_per_route,
                   const int32_t *ids, int64_t top_k, const float *route_w, int epi,
                   void *y, int ydt,
                   void *ws, size_t ws_bytes, int path, void *stream);

/* ggq_mul_mat_id without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts that
 * forbid allocation).  The workspace is a fixed device array of
 * GGQ_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; the array of the current device (hipGetDevice) is used, so the
 * stream must belong to that device.  Calls on one GPU share that array: calls
 * that overlap in time on one GPU (on different streams, or from several
 * threads without ordering) race, and must be serialized by the caller.  Each
 * call clears the parts that must start at zero.  Arguments and results as
 * ggq_mul_mat_id; a call whose ggq_mul_mat_id_ws() size exceeds the array
 * returns GGQ_ERR_WORKSPACE and launches nothing.  Calls no allocating
 * routine. */
#define GGQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ggq_mul_mat_id_noalloc(int wt, const void *W, int64_t E, int64_t N, int64_t K,
                           int64_t expert_stride,
                           const void *x, int xdt, int64_t T, int x_per_route,
                           const int32_t *ids, int64_t top_k, const float *route_w, int epi,
                           void *y, int ydt, int path, void *stream);

/* Dequantize (convert) rows of weights: y[r][k] = exact block value in fp32,
 * or its round-to-nearest-even bf16 / fp16 (PR #690 lists dequantize among
 * its ops).  y: [rows][K] of ydt (GGQ_F32 / GGQ_BF16 / GGQ_F16).  Bit-exact. */
int ggq_dequantize(int wt, const void *W, int64_t rows, int64_t K,
                   void *y, int ydt, void *stream);

/* Gather rows of a quantized table (embeddings, or a tied lm_head read as
 * rows), dequantized: y[i][k] = exact value of table row ids[i], weight k, in
 * fp32, or its round-to-nearest-even bf16 / fp16 -- the same values as
 * ggq_dequantize (PR #690 lists get_rows among the ops its backend serves
 * next to the matmuls).
 *   W   : table of `rows` rows of ggq_row_bytes(wt, K) bytes, 16-byte aligned.
 *   ids : [n] int32 row ids, device memory.  An id outside [0, rows) gives a
 *         row of zeros (no fault, no error: ids are not read on the host).
 *   y   : [n][ldy] of ydt (GGQ_F32 / GGQ_BF16 / GGQ_F16); writes K values
 *         per row; ldy >= K and ldy keeps rows 16-byte aligned (multiple of 4
 *         for fp32, 8 for the 16-bit types).
 * n = 0 is a no-op.  Bit-exact.  Returns GGQ_OK or an error code. */
int ggq_get_rows(int wt, const void *W, int64_t rows, int64_t K, const int32_t *ids, int64_t n,
                 void *y, int ydt, int64_t ldy, void *stream);

/* Message describing the calling thread's last failing call ("" if none). */
const char *ggq_last_error(void);

/* Test hook (not part of the product API): per-group int32 dots of raw weight
 * quants with q8_1 quants, out[M][N][K/g] (g = 32 for Q8_0, Q4_0 (nibbles
 * minus 8), Q4_K / Q5_K (values without the min); g = 16 for Q6_K: values
 * minus 32).  They come from separate test kernels that reuse the named
 * path's unpack helpers and dot instructions (GGQ_PATH_MMVQ: the weight
 * decode helpers and v_dot4, reading blocks straight from memory;
 * GGQ_PATH_MMQ: the MMQ staging code with unit sub-scales and the same MFMA
 * fragment layout, Q4_0 / Q8_0 with K % 256 == 0), not from the production
 * kernels' pipelines.  The production kernels' per-block dots are checked
 * bit for bit through their outputs on exact-arithmetic inputs instead.
 * q8 is M rows of K/32 q8_1 blocks; ws needs ggq_test_block_dots_ws() bytes. */
size_t ggq_test_block_dots_ws(int wt, int64_t K, int64_t M, int path);
int ggq_test_block_dots(int wt, const void *W, int64_t N, int64_t K,
                        const void *q8, int64_t M, int32_t *out,
                        void *ws, size_t ws_bytes, int path, void *stream);

/* Bench hooks (not part of the product API): measured ceilings reported next
 * to the published peaks.  Both are asynchronous on `stream`, write nothing
 * to `sink` in practice (a device buffer the caller owns, at least 1 KB for
 * the read and 4 KB for the MFMA loop, else GGQ_ERR_WORKSPACE), and return
 * GGQ_ERR_INVALID for bad arguments.
 *
 * ggq_bench_stream_read: reads the bytes / 16 whole 16-byte pieces of the
 * device buffer buf (16-byte aligned) once, grid-stride, 256 workgroups of
 * 256 threads: the HBM read rate a kernel doing nothing else achieves.
 *
 * ggq_bench_mfma_loop: 1024 workgroups of 4 waves; each wave issues iters x 4
 * independent MFMAs, kind 0 = v_mfma_f32_32x32x16_f16 (32768 flops each),
 * kind 1 = v_mfma_i32_32x32x32_i8 (65536 int8 ops each), with no memory
 * traffic: the matrix-core rate.  iters >= 0. */
int ggq_bench_stream_read(const void *buf, int64_t bytes, void *sink, size_t sink_bytes, void *stream);
int ggq_bench_mfma_loop(int kind, int64_t iters, void *sink, size_t sink_bytes, void *stream);

/* Bench hook (not part of the product API): the MMQ inner loop measured on
 * its own, to compare the two matrix-core choices for the per-block int dot
 * with its exact q8_1 rescale.  256 * blocks_per_cu workgroups (1..8) of 4
 * waves; each wave owns a 64 x 64 output tile and runs `iters` 32-wide q8_1
 * blocks: fragment and scale reads from LDS, then
 *   kind 0: two v_mfma_f32_32x32x16_f16 per 32 x 32 tile (sub-scale folded
 *           into the fp16 weight operand) and one fp32 fma per output;
 *   kind 1: one v_mfma_i32_32x32x32_i8 per 32 x 32 tile, then per output an
 *           integer multiply by the sub-scale, a conversion and an fma;
 *   kind 2: the fragment reads alone (8 x 1 KB of ds_read_b128 per block);
 *   kinds 3 and 4: kinds 0 and 1 software-pipelined, the rescale of one
 *           32 x 32 tile issued under the MFMAs of the next.
 * Work per wave per block: 2 * 64 * 64 * 32 int8 ops (kind 2: 8 KB read).
 * Returns GGQ_ERR_INVALID for a kind outside 0..4 or blocks_per_cu outside 1..8.
 * sink: device buffer of at least 256 * blocks_per_cu * 4 bytes. */
int ggq_bench_inner_loop(int kind, int blocks_per_cu, int64_t iters, void *sink, size_t sink_bytes, void *stream);

/* Bench hook (not part of the product API): the routes per MMVQ-id group
 * (1, 2, 4 or 8; capped by what the type and K allow) for every later routed
 * MMVQ call in this process, or 0 to restore the automatic choice (a little
 * above the mean routes per expert).  Not thread-safe; for tuning sweeps.
 * Returns GGQ_ERR_INVALID for any other value. */
int ggq_bench_set_mmvq_id_cols(int cols);

#ifdef __cplusplus
}
#endif
#endif
