/*
 * ggq_oracle.c -- plain CPU oracle for GGUF block-quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY (see ggq_oracle.h): used by the tests, the smoke
 * check and the CPU-baseline leg of the benchmark, never by the product path.
 *
 * Written for readability against the definitions, not for speed: one block
 * at a time, integer fields unpacked into plain arrays, fp64 accumulation in
 * ascending K.  OpenMP only splits independent output rows / routes.
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp.
 */
#include "ggq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define QK8_1 32
#define Q8_1_BYTES 40

/* ------------------------------------------------------------------ */
/* scalar codecs                                                        */
/* ------------------------------------------------------------------ */

/* IEEE binary16 -> binary32, decoded field by field (sign, 5-bit exponent
 * biased by 15, 10-bit fraction), subnormals, infinities and NaN included. */
float ggqo_fp16_to_fp32(uint16_t h) {
    unsigned sign = (h >> 15) & 1u;
    unsigned expo = (h >> 10) & 0x1fu;
    unsigned frac = h & 0x3ffu;
    float v;
    if (expo == 0) {
        v = ldexpf((float)frac, -24);             /* 0.frac * 2^-14 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexpf((float)(frac | 0x400u), (int)expo - 25); /* 1.frac * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 is the upper half of a binary32. */
float ggqo_bf16_to_fp32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary32 -> IEEE binary16, round to nearest, ties to even.  The value is
 * written as an integer count of the target's units in the last place and
 * rounded with rint (the default rounding mode is to nearest even); counts
 * are exact in double.  Normal range: a = n * 2^(e - 11) with n in
 * [1024, 2048); subnormal range (a < 2^-14): a = n * 2^-24.  From 65520 (half
 * a unit above the largest finite half, 65504) up the result is infinity;
 * NaN gives a quiet NaN of the same sign. */
uint16_t ggqo_fp32_to_fp16(float f) {
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    float a = fabsf(f);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0f) return (uint16_t)(sign | 0x7c00u);
    if (a < ldexpf(1.0f, -14)) {
        double n = rint((double)a * 16777216.0);   /* units of 2^-24; 1024 is the smallest normal */
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e;
    frexp((double)a, &e);                             /* a = m * 2^e, m in [0.5, 1) */
    double n = rint(ldexp((double)a, 11 - e));       /* in [1024, 2048] */
    if (n == 2048.0) {
        n = 1024.0;
        e += 1;
    }
    unsigned field = (unsigned)(e - 1 + 15);          /* biased exponent, 1..30 here */
    return (uint16_t)(sign | (field << 10) | ((unsigned)n - 1024u));
}

/* binary32 -> bfloat16, round to nearest, ties to even; NaN stays NaN. */
uint16_t ggqo_fp32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;             /* the 16 dropped bits */
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------------ */
/* geometry                                                             */
/* ------------------------------------------------------------------ */

int64_t ggqo_block_len(int type) {
    switch (type) {
    case GGQO_Q4_0: return 32;
    case GGQO_Q8_0: return 32;
    case GGQO_Q4_K: return 256;
    case GGQO_Q5_K: return 256;
    case GGQO_Q6_K: return 256;
    default: return 0;
    }
}

int64_t ggqo_block_bytes(int type) {
    switch (type) {
    case GGQO_Q4_0: return 2 + 16;                 /* fp16 d, 32 nibbles */
    case GGQO_Q8_0: return 2 + 32;                 /* fp16 d, 32 x int8 */
    case GGQO_Q4_K: return 2 + 2 + 12 + 128;       /* d, dmin, packed scales, nibbles */
    case GGQO_Q5_K: return 2 + 2 + 12 + 32 + 128;  /* d, dmin, packed scales, fifth bits, nibbles */
    case GGQO_Q6_K: return 128 + 64 + 16 + 2;      /* ql, qh, int8 scales, d */
    default: return 0;
    }
}

int64_t ggqo_group_len(int type) {
    switch (type) {
    case GGQO_Q4_0: return 32;
    case GGQO_Q8_0: return 32;
    case GGQO_Q4_K: return 32;
    case GGQO_Q5_K: return 32;
    case GGQO_Q6_K: return 16;
    default: return 0;
    }
}

int64_t ggqo_row_bytes(int type, int64_t K) {
    int64_t qk = ggqo_block_len(type);
    if (qk == 0 || K < 0 || K % qk != 0) return 0;
    return (K / qk) * ggqo_block_bytes(type);
}

/* ------------------------------------------------------------------ */
/* q8_1                                                                 */
/* ------------------------------------------------------------------ */

/* Per block of 32: d = amax / 127 (fp32 division); q_i = x_i / d (fp32
 * division) rounded half away from zero; an all-zero block has d = 0 and
 * q = 0; s = d * (float)(sum of q_i). */
void ggqo_quantize_block_q8_1(const float *x, uint8_t *blk) {
    float amax = 0.0f;
    for (int i = 0; i < QK8_1; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    int8_t q[QK8_1];
    int32_t sum = 0;
    for (int i = 0; i < QK8_1; i++) {
        int qi = 0;
        if (amax != 0.0f) {
            float r = roundf(x[i] / d);
            if (r != r) r = 0.0f;                  /* NaN input: outside the contract */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            qi = (int)r;
        }
        q[i] = (int8_t)qi;
        sum += qi;
    }
    if (amax == 0.0f) d = 0.0f;
    float s = d * (float)sum;
    memcpy(blk, &d, 4);
    memcpy(blk + 4, &s, 4);
    memcpy(blk + 8, q, QK8_1);
}

static float load_act(const void *x, int xdt, int64_t idx) {
    if (xdt == GGQO_F32) return ((const float *)x)[idx];
    if (xdt == GGQO_F16) return ggqo_fp16_to_fp32(((const uint16_t *)x)[idx]);
    return ggqo_bf16_to_fp32(((const uint16_t *)x)[idx]);
}

static int act_dt(int xdt) { return xdt == GGQO_F32 || xdt == GGQO_BF16 || xdt == GGQO_F16; }

int ggqo_quantize_q8_1(const void *x, int xdt, int64_t M, int64_t K, int64_t ldx, void *q8) {
    if (!x || !q8 || M < 0 || K < 0 || K % QK8_1 || ldx < K) return -1;
    if (!act_dt(xdt)) return -1;
    int64_t nb = K / QK8_1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float buf[QK8_1];
        for (int64_t b = 0; b < nb; b++) {
            for (int i = 0; i < QK8_1; i++) buf[i] = load_act(x, xdt, m * ldx + b * QK8_1 + i);
            ggqo_quantize_block_q8_1(buf, (uint8_t *)q8 + (m * nb + b) * Q8_1_BYTES);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* unpack (public GGUF block layout)                                    */
/* ------------------------------------------------------------------ */

static void unpack_q8_0(const uint8_t *blk, int32_t *q, int32_t *sc, int32_t *mn, float *d) {
    d[0] = ggqo_fp16_to_fp32(rd16(blk));
    d[1] = 0.0f;
    for (int i = 0; i < 32; i++) q[i] = (int8_t)blk[2 + i];
    sc[0] = 1;
    mn[0] = 0;
}

/* Q4_0: one group of 32: byte b of the 16 quant bytes gives weight b (low
 * nibble) and weight 16 + b (high nibble); the value is d * (nibble - 8). */
static void unpack_q4_0(const uint8_t *blk, int32_t *q, int32_t *sc, int32_t *mn, float *d) {
    d[0] = ggqo_fp16_to_fp32(rd16(blk));
    d[1] = 0.0f;
    for (int i = 0; i < 16; i++) {
        q[i] = blk[2 + i] & 0x0f;
        q[16 + i] = blk[2 + i] >> 4;
    }
    sc[0] = 1;
    mn[0] = 0;
}

/* The 6-bit scales and mins of the 8 groups of a Q4_K / Q5_K block, from
 * the 12 packed bytes s: groups 0..3 use the low 6 bits of bytes 0..3
 * (scales) and 4..7 (mins); groups 4..7 take their low 4 bits from the
 * nibbles of bytes 8..11 and their top 2 bits from the top bits of bytes
 * 0..3 (scales) and 4..7 (mins). */
static void unpack_scales_k(const uint8_t *s, int32_t *sc, int32_t *mn) {
    for (int j = 0; j < 8; j++) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            mn[j] = s[j + 4] & 63;
        } else {
            sc[j] = (s[j + 4] & 0x0f) | ((s[j - 4] >> 6) << 4);
            mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
    }
}

/* Q4_K: 8 groups of 32.  Groups 0..3 take their 6-bit scale and min from the
 * low 6 bits of bytes 0..3 and 4..7 of the packed area; groups 4..7 take the
 * low 4 bits from the nibbles of bytes 8..11 and the top 2 bits from the top
 * bits of bytes 0..3 (scales) and 4..7 (mins).  The 128 quant bytes hold four
 * 64-weight chunks: byte r of a chunk gives weight r (low nibble) and weight
 * 32 + r (high nibble). */
static void unpack_q4_K(const uint8_t *blk, int32_t *q, int32_t *sc, int32_t *mn, float *d) {
    const uint8_t *s = blk + 4;
    const uint8_t *qs = blk + 16;
    d[0] = ggqo_fp16_to_fp32(rd16(blk));
    d[1] = ggqo_fp16_to_fp32(rd16(blk + 2));
    unpack_scales_k(s, sc, mn);
    for (int i = 0; i < 256; i++) {
        int c = i / 64, r = i % 64;
        if (r < 32) q[i] = qs[32 * c + r] & 0x0f;
        else        q[i] = qs[32 * c + r - 32] >> 4;
    }
}

/* Q5_K: the Q4_K arrangement (same scales, mins and nibbles, the nibbles at
 * byte 48) plus a fifth bit per weight: weight i of group j takes bit j of
 * byte (i mod 32) of the 32 bytes at offset 16, as bit 4 of its value 0..31. */
static void unpack_q5_K(const uint8_t *blk, int32_t *q, int32_t *sc, int32_t *mn, float *d) {
    const uint8_t *s = blk + 4;
    const uint8_t *qh = blk + 16;
    const uint8_t *qs = blk + 48;
    d[0] = ggqo_fp16_to_fp32(rd16(blk));
    d[1] = ggqo_fp16_to_fp32(rd16(blk + 2));
    unpack_scales_k(s, sc, mn);
    for (int i = 0; i < 256; i++) {
        int c = i / 64, r = i % 64, j = i / 32, l = i % 32;
        int lo = (r < 32) ? (qs[32 * c + l] & 0x0f) : (qs[32 * c + l] >> 4);
        int hi = (qh[l] >> j) & 1;
        q[i] = lo | (hi << 4);
    }
}

/* Q6_K: 16 groups of 16 with signed int8 scales.  Weight i of the block:
 * half h = i/128, r = i%128, quarter g = r/32, lane l = r%32; low 4 bits from
 * ql[64h + 32(g&1) + l] (low nibble for g < 2, high nibble otherwise), high 2
 * bits from bits 2g..2g+1 of qh[32h + l]. */
static void unpack_q6_K(const uint8_t *blk, int32_t *q, int32_t *sc, int32_t *mn, float *d) {
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    d[0] = ggqo_fp16_to_fp32(rd16(blk + 208));
    d[1] = 0.0f;
    for (int j = 0; j < 16; j++) {
        sc[j] = (int8_t)blk[192 + j];
        mn[j] = 0;
    }
    for (int i = 0; i < 256; i++) {
        int h = i / 128, r = i % 128, g = r / 32, l = r % 32;
        int lo = ql[64 * h + 32 * (g & 1) + l];
        lo = (g < 2) ? (lo & 0x0f) : (lo >> 4);
        int hi = (qh[32 * h + l] >> (2 * g)) & 3;
        q[i] = lo | (hi << 4);
    }
}

int ggqo_unpack_block(int type, const uint8_t *blk, int32_t *q, int32_t *sc, int32_t *mn, float *d) {
    if (!blk || !q || !sc || !mn || !d) return -1;
    switch (type) {
    case GGQO_Q4_0: unpack_q4_0(blk, q, sc, mn, d); return 0;
    case GGQO_Q8_0: unpack_q8_0(blk, q, sc, mn, d); return 0;
    case GGQO_Q4_K: unpack_q4_K(blk, q, sc, mn, d); return 0;
    case GGQO_Q5_K: unpack_q5_K(blk, q, sc, mn, d); return 0;
    case GGQO_Q6_K: unpack_q6_K(blk, q, sc, mn, d); return 0;
    default: return -1;
    }
}

/* Signed weight quant entering the integer dot: Q6_K carries a -32 offset,
 * Q4_0 a -8 offset. */
static int32_t dot_quant(int type, int32_t q) {
    return type == GGQO_Q6_K ? q - 32 : type == GGQO_Q4_0 ? q - 8 : q;
}

/* Types with a per-group min subtracted (d*sc*q - dmin*m). */
static int has_min(int type) { return type == GGQO_Q4_K || type == GGQO_Q5_K; }

/* ------------------------------------------------------------------ */
/* integer block dots                                                   */
/* ------------------------------------------------------------------ */

static int check_w(int type, int64_t N, int64_t K) {
    return ggqo_block_len(type) != 0 && N >= 0 && K >= 0 && K % ggqo_block_len(type) == 0;
}

/* Dot of group j of a block with the q8_1 activation row, int64 then int32. */
static int32_t group_dot(int type, const int32_t *q, int64_t blk_k0, int j,
                         const uint8_t *q8row) {
    int64_t g = ggqo_group_len(type);
    int64_t acc = 0;
    for (int64_t i = 0; i < g; i++) {
        int64_t kpos = blk_k0 + j * g + i;                 /* absolute K index */
        const uint8_t *ab = q8row + (kpos / QK8_1) * Q8_1_BYTES;
        int8_t qa = (int8_t)ab[8 + kpos % QK8_1];
        acc += (int64_t)dot_quant(type, q[j * g + i]) * qa;
    }
    if (acc > INT32_MAX || acc < INT32_MIN) abort();       /* cannot happen for these types */
    return (int32_t)acc;
}

int ggqo_block_dots(int type, const void *W, int64_t N, int64_t K,
                    const void *q8, int64_t M, int32_t *out) {
    if (!W || !q8 || !out || M < 0 || !check_w(type, N, K)) return -1;
    int64_t qk = ggqo_block_len(type), bb = ggqo_block_bytes(type), g = ggqo_group_len(type);
    int64_t nblk = K / qk, ngrp = qk / g, gpr = K / g;
    int64_t q8row_bytes = (K / QK8_1) * Q8_1_BYTES;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        int32_t q[256], sc[16], mn[16];
        float d[2];
        for (int64_t b = 0; b < nblk; b++) {
            const uint8_t *blk = (const uint8_t *)W + (n * nblk + b) * bb;
            ggqo_unpack_block(type, blk, q, sc, mn, d);
            for (int64_t m = 0; m < M; m++) {
                const uint8_t *row = (const uint8_t *)q8 + m * q8row_bytes;
                for (int j = 0; j < ngrp; j++)
                    out[(m * N + n) * gpr + b * ngrp + j] = group_dot(type, q, b * qk, j, row);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* quantized matmul                                                     */
/* ------------------------------------------------------------------ */

static float q8_d(const uint8_t *row, int64_t blk) { float v; memcpy(&v, row + blk * Q8_1_BYTES, 4); return v; }
static float q8_s(const uint8_t *row, int64_t blk) { float v; memcpy(&v, row + blk * Q8_1_BYTES + 4, 4); return v; }

/* Contribution of one weight block to one output, fp64:
 *   Q8_0, Q4_0: d * d8 * D   (Q4_0: D over nibble - 8)
 *   Q4_K, Q5_K: sum_j (d*sc_j) * d8_j * D_j - (dmin*m_j) * s8_j
 *   Q6_K: sum_j (d*sc_j) * d8_(j/2) * D_j                                  */
static double block_contrib(int type, const int32_t *q, const int32_t *sc, const int32_t *mn,
                            const float *d, int64_t blk_k0, const uint8_t *q8row) {
    int64_t g = ggqo_group_len(type), ngrp = ggqo_block_len(type) / g;
    double acc = 0.0;
    for (int j = 0; j < ngrp; j++) {
        int64_t ablk = (blk_k0 + j * g) / QK8_1;          /* q8_1 block holding group j */
        double dot = (double)group_dot(type, q, blk_k0, j, q8row);
        double wscale = (double)d[0] * (double)sc[j];
        acc += wscale * (double)q8_d(q8row, ablk) * dot;
        if (has_min(type))
            acc -= ((double)d[1] * (double)mn[j]) * (double)q8_s(q8row, ablk);
    }
    return acc;
}

int ggqo_mul_mat_q8(int type, const void *W, int64_t N, int64_t K,
                    const void *q8, int64_t M,
                    const int64_t *rows, int64_t nrows,
                    float *y, int64_t ldy) {
    if (!W || !q8 || !y || M < 0 || !check_w(type, N, K)) return -1;
    int64_t ncols = rows ? nrows : N;
    if (ncols < 0 || ldy < ncols) return -1;
    int64_t qk = ggqo_block_len(type), bb = ggqo_block_bytes(type);
    int64_t nblk = K / qk, q8row_bytes = (K / QK8_1) * Q8_1_BYTES;
    if (rows)
        for (int64_t c = 0; c < ncols; c++)
            if (rows[c] < 0 || rows[c] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t c = 0; c < ncols; c++) {
        int64_t n = rows ? rows[c] : c;
        int32_t q[256], sc[16], mn[16];
        float d[2];
        double *acc = (double *)calloc((size_t)(M > 0 ? M : 1), sizeof(double));
        for (int64_t b = 0; b < nblk; b++) {                /* ascending K */
            const uint8_t *blk = (const uint8_t *)W + (n * nblk + b) * bb;
            ggqo_unpack_block(type, blk, q, sc, mn, d);
            for (int64_t m = 0; m < M; m++)
                acc[m] += block_contrib(type, q, sc, mn, d, b * qk,
                                        (const uint8_t *)q8 + m * q8row_bytes);
        }
        for (int64_t m = 0; m < M; m++) y[m * ldy + c] = (float)acc[m];
        free(acc);
    }
    return 0;
}

int ggqo_mul_mat(int type, const void *W, int64_t N, int64_t K,
                 const void *x, int xdt, int64_t M, int64_t ldx,
                 const int64_t *rows, int64_t nrows,
                 float *y, int64_t ldy) {
    if (!x || !check_w(type, N, K) || M < 0) return -1;
    if (xdt == GGQO_Q8_1)
        return ggqo_mul_mat_q8(type, W, N, K, x, M, rows, nrows, y, ldy);
    size_t qbytes = (size_t)(M * (K / QK8_1) * Q8_1_BYTES);
    void *q8 = malloc(qbytes ? qbytes : 1);
    if (!q8) return -1;
    int rc = ggqo_quantize_q8_1(x, xdt, M, K, ldx, q8);
    if (rc == 0) rc = ggqo_mul_mat_q8(type, W, N, K, q8, M, rows, nrows, y, ldy);
    free(q8);
    return rc;
}

/* ------------------------------------------------------------------ */
/* dequantize                                                           */
/* ------------------------------------------------------------------ */

/* Weight values in fp32: Q8_0 d*q; Q4_0 d*(nib-8); Q4_K / Q5_K
 * (d*sc)*q - dmin*m; Q6_K (d*sc)*(q-32).  Every product is exact in fp32
 * (at most 11 + 6 + 5 significant bits), so the only rounding is the
 * subtraction of the min. */
int ggqo_dequantize(int type, const void *W, int64_t rows, int64_t K, void *y, int ydt) {
    if (!W || !y || !check_w(type, rows, K)) return -1;
    if (ydt != GGQO_F32 && ydt != GGQO_BF16 && ydt != GGQO_F16) return -1;
    int64_t qk = ggqo_block_len(type), bb = ggqo_block_bytes(type), g = ggqo_group_len(type);
    int64_t nblk = K / qk;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        int32_t q[256], sc[16], mn[16];
        float d[2];
        for (int64_t b = 0; b < nblk; b++) {
            ggqo_unpack_block(type, (const uint8_t *)W + (r * nblk + b) * bb, q, sc, mn, d);
            for (int64_t i = 0; i < qk; i++) {
                int64_t j = i / g;
                float w;
                if (has_min(type)) {
                    float a = d[0] * (float)sc[j];
                    float m = d[1] * (float)mn[j];
                    float t = a * (float)q[i];
                    w = t - m;
                } else {
                    float a = d[0] * (float)sc[j];
                    w = a * (float)dot_quant(type, q[i]);
                }
                int64_t idx = r * K + b * qk + i;
                if (ydt == GGQO_F32) ((float *)y)[idx] = w;
                else if (ydt == GGQO_F16) ((uint16_t *)y)[idx] = ggqo_fp32_to_fp16(w);
                else ((uint16_t *)y)[idx] = ggqo_fp32_to_bf16(w);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* routed experts                                                       */
/* ------------------------------------------------------------------ */

int ggqo_mul_mat_id(int type, const void *W, int64_t E, int64_t N, int64_t K, int64_t expert_stride,
                    const void *x, int xdt, int64_t T, int x_per_route,
                    const int32_t *ids, int64_t top_k, const float *route_w, int epi,
                    int route_round, const int64_t *tokens, int64_t ntok, float *y) {
    if (!W || !x || !ids || !y || E < 0 || T < 0 || top_k <= 0 || !check_w(type, N, K)) return -1;
    if (!act_dt(xdt)) return -1;
    if (epi != GGQO_EPI_NONE && epi != GGQO_EPI_SWIGLU) return -1;
    if (epi == GGQO_EPI_SWIGLU && N % 2) return -1;
    if (route_round < 0 || route_round > 2) return -1;
    if (expert_stride < ggqo_row_bytes(type, K) * N) return -1;
    int64_t nt = tokens ? ntok : T;
    for (int64_t i = 0; tokens && i < nt; i++)
        if (tokens[i] < 0 || tokens[i] >= T) return -1;
    int64_t Np = epi == GGQO_EPI_SWIGLU ? N / 2 : N;
    int64_t nb = K / QK8_1;
    int64_t out_per_tok = route_w ? Np : top_k * Np;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t it = 0; it < nt; it++) {
        int64_t t = tokens ? tokens[it] : it;
        float *yt = y + it * out_per_tok;
        double *wsum = (double *)calloc((size_t)(Np > 0 ? Np : 1), sizeof(double));
        float *o = (float *)malloc((size_t)(N > 0 ? N : 1) * sizeof(float));
        float *act = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
        uint8_t *q8 = (uint8_t *)malloc((size_t)(nb > 0 ? nb : 1) * Q8_1_BYTES);
        for (int64_t k = 0; k < top_k; k++) {               /* ascending k */
            int32_t e = ids[t * top_k + k];
            int active = e >= 0 && e < E;
            if (!route_w)
                for (int64_t n = 0; n < Np; n++) yt[k * Np + n] = 0.0f;
            if (!active) continue;
            int64_t xrow = x_per_route ? (t * top_k + k) : t;
            for (int64_t i = 0; i < K; i++) act[i] = load_act(x, xdt, xrow * K + i);
            for (int64_t b = 0; b < nb; b++)
                ggqo_quantize_block_q8_1(act + b * QK8_1, q8 + b * Q8_1_BYTES);
            const uint8_t *We = (const uint8_t *)W + (int64_t)e * expert_stride;
            /* o = W_e . act, each output rounded once to fp32 */
            ggqo_mul_mat_q8(type, We, N, K, q8, 1, NULL, 0, o, N);
            for (int64_t n = 0; n < Np; n++) {
                double v;
                if (epi == GGQO_EPI_SWIGLU) {
                    double gte = (double)o[n], up = (double)o[Np + n];
                    v = gte / (1.0 + exp(-gte)) * up;
                } else {
                    v = (double)o[n];
                }
                float vf = (float)v;                          /* route output in fp32 */
                /* weighted: the route output is an intermediate held in the 16-bit
                 * activation dtype when route_round asks for it (1 bf16, 2 fp16) */
                if (route_w && route_round == 1) vf = ggqo_bf16_to_fp32(ggqo_fp32_to_bf16(vf));
                if (route_w && route_round == 2) vf = ggqo_fp16_to_fp32(ggqo_fp32_to_fp16(vf));
                if (route_w) wsum[n] += (double)route_w[t * top_k + k] * (double)vf;
                else yt[k * Np + n] = vf;
            }
        }
        if (route_w)
            for (int64_t n = 0; n < Np; n++) yt[n] = (float)wsum[n];
        free(wsum); free(o); free(act); free(q8);
    }
    return 0;
}
