/*
 * ggq_oracle.h -- plain, slow CPU oracle for GGUF block-quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library,
 * its Python binding) may include, link, load or call this code; only the
 * test suite, the package smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no source with the GPU path.
 *
 * What it computes, and where that is defined:
 *  - Weights are GGUF blocks of type Q8_0, Q4_K or Q6_K (and Q4_0, Q5_K),
 *    quantized tensor types listed in FreeToken PR #690 "feat(gguf): serve
 *    GGUF checkpoints on vendored ggml-cuda kernels" (Summary, "Tensor
 *    types") and transformers PR #45977 "GgufLinear" ("What").  The pages
 *    give only block sizes (Q4_K 144 B and Q6_K 210 B per 256 weights, from
 *    the per-expert byte counts in FreeToken PR #196, Windows follow-up) and
 *    the type id of Q4_0 (2); the bit arrangement, and the Q4_0 (18 B per
 *    32) and Q5_K (176 B per 256) sizes, follow the public GGUF layout.
 *  - Activations are quantized on the fly to q8_1 blocks and results come
 *    out in the activation dtype with fp32 accumulation (PR #690, "What the
 *    ggml patch changes", first item).  This project's q8_1 block is
 *    {float d; float s; int8 qs[32]} = 40 bytes, d = amax/127, round half
 *    away from zero, s = d * (sum of the 32 quants).
 *  - mul_mat_id runs each (token, slot) route against its own expert; the
 *    fused GLU and the MoE weighted sum are the ops PR #690 lists beside
 *    mul_mat ("Our own code next to it").
 *
 * Precision: integer block dots are exact (int64, checked to fit int32);
 * every row result is accumulated in fp64 in ascending K and rounded once
 * to fp32.  bf16 outputs are the round-to-nearest-even of that fp32.
 *
 * Return values: 0 on success, -1 on a bad argument (unknown type, K not a
 * multiple of the block length, null pointer).  No function allocates
 * memory that outlives the call.
 */
#ifndef GGQ_ORACLE_H
#define GGQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GGUF tensor type ids (public GGUF numbering). */
enum { GGQO_Q4_0 = 2, GGQO_Q8_0 = 8, GGQO_Q4_K = 12, GGQO_Q5_K = 13, GGQO_Q6_K = 14 };
/* Activation / output element types.  GGQO_Q8_1 = pre-quantized blocks. */
enum { GGQO_F32 = 0, GGQO_BF16 = 1, GGQO_Q8_1 = 2, GGQO_F16 = 3 };
/* Epilogues of mul_mat_id. */
enum { GGQO_EPI_NONE = 0, GGQO_EPI_SWIGLU = 1 };

/* ---- scalar codecs ---- */
float    ggqo_fp16_to_fp32(uint16_t h);
float    ggqo_bf16_to_fp32(uint16_t b);
uint16_t ggqo_fp32_to_bf16(float f);
uint16_t ggqo_fp32_to_fp16(float f);   /* round to nearest even, overflow to inf */

/* ---- geometry ---- */
int64_t ggqo_block_len(int type);    /* weights per block: 32 or 256, 0 if unknown */
int64_t ggqo_block_bytes(int type);  /* 34, 144, 210, 0 if unknown */
int64_t ggqo_group_len(int type);    /* weights per integer scale group: 32, 32, 16 */
int64_t ggqo_row_bytes(int type, int64_t K); /* 0 if K is not a multiple of the block length */

/* ---- q8_1 ---- */
/* One block: 32 fp32 values -> 40 bytes. */
void ggqo_quantize_block_q8_1(const float *x32, uint8_t *blk40);
/* x: [M][ldx] elements of type xdt (F32, BF16 or F16 bits); q8: [M][K/32] blocks. */
int ggqo_quantize_q8_1(const void *x, int xdt, int64_t M, int64_t K, int64_t ldx, void *q8);

/* ---- unpack ---- */
/* One block into integer fields.
 *   q[QK]   : Q8_0 signed quants; Q4_0 and Q4_K nibbles 0..15; Q5_K values
 *             0..31; Q6_K 6-bit values 0..63 (the -8 / -32 offsets of Q4_0 /
 *             Q6_K are NOT applied here).
 *   sc[G]   : per-group integer scale (Q8_0, Q4_0: 1 group, value 1; Q4_K,
 *             Q5_K: 8 groups 0..63; Q6_K: 16 groups, signed int8).
 *   mn[G]   : Q4_K / Q5_K mins 0..63, zero otherwise.
 *   d[2]    : fp32 of the fp16 super-scale d and (Q4_K, Q5_K) dmin. */
int ggqo_unpack_block(int type, const uint8_t *blk, int32_t *q, int32_t *sc, int32_t *mn, float *d);

/* ---- integer block dots ---- */
/* out[M][N][K/g], g = ggqo_group_len(type): the int32 dot of raw weight quants
 * (Q4_K / Q5_K values without the min, Q6_K values minus 32, Q4_0 nibbles
 * minus 8) with the q8_1 quants
 * of the same K positions. */
int ggqo_block_dots(int type, const void *W, int64_t N, int64_t K,
                    const void *q8, int64_t M, int32_t *out);

/* ---- quantized matmul on q8_1 activations ---- */
/* y[m][n] (row stride ldy) for the weight rows listed in rows[0..nrows)
 * (rows == NULL: all N rows, nrows ignored).  With a row list, output column
 * c holds weight row rows[c]. */
int ggqo_mul_mat_q8(int type, const void *W, int64_t N, int64_t K,
                    const void *q8, int64_t M,
                    const int64_t *rows, int64_t nrows,
                    float *y, int64_t ldy);

/* Full path from float activations: quantize each row to q8_1 then
 * ggqo_mul_mat_q8.  xdt: F32, BF16, F16 or Q8_1 (then x is [M][K/32] blocks and
 * ldx is ignored).  Output fp32 [M][ldy]. */
int ggqo_mul_mat(int type, const void *W, int64_t N, int64_t K,
                 const void *x, int xdt, int64_t M, int64_t ldx,
                 const int64_t *rows, int64_t nrows,
                 float *y, int64_t ldy);

/* ---- dequantize ---- */
/* y: [rows][K] of ydt (F32, BF16 or F16 bits). */
int ggqo_dequantize(int type, const void *W, int64_t rows, int64_t K, void *y, int ydt);

/* ---- routed experts ---- */
/* W: E experts, expert e at byte offset e*expert_stride, each N rows x K.
 * x: x_per_route == 0 -> [T][K] (broadcast), == 1 -> [T][top_k][K] (gather),
 *    elements of xdt (F32, BF16 or F16).
 * ids: [T][top_k]; a route with id < 0 or id >= E is inactive.
 * epi SWIGLU: o' = silu(o[:N/2]) * o[N/2:], computed in fp64 from the fp32
 *    route outputs and rounded to fp32; N' = N/2.  Otherwise N' = N.
 * route_w == NULL: y is [ntok][top_k][N'] (inactive routes -> 0).
 * route_w != NULL: y is [ntok][N'] = sum over active k, ascending, of
 *    w[t][k] * o'[t][k], in fp64, rounded to fp32.
 * tokens: the token indices to compute (ntok of them); NULL -> all T. */
int ggqo_mul_mat_id(int type, const void *W, int64_t E, int64_t N, int64_t K, int64_t expert_stride,
                    const void *x, int xdt, int64_t T, int x_per_route,
                    const int32_t *ids, int64_t top_k, const float *route_w, int epi,
                    int route_round, const int64_t *tokens, int64_t ntok, float *y);

#ifdef __cplusplus
}
#endif
#endif
