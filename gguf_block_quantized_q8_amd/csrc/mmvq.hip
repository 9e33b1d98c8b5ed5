// MMVQ: quantized matrix x few-vectors, for small batches (decode).
//
// HBM-bound on the weights, so every weight byte is read exactly once and the
// reads are fully coalesced:
//  - each wave owns a few consecutive rows per work item and copies their
//    bytes into a private LDS buffer with buffer_load_dwordx4 ... lds: 64
//    lanes x 16 B = one contiguous 1 KB span per instruction, straight into
//    LDS without passing through registers; the buffer descriptor's range
//    stops the copy at the last weight byte (no over-read).  Two buffers per
//    wave: item i+1 is in flight while item i is computed;
//  - the activations (a few KB) are quantized to q8_1 (or copied, when given
//    pre-quantized) into LDS once per workgroup, in the kernel prologue, while
//    the first weight copy is in flight.  They are kept planar: int8 quants
//    [col][K], then d [col][K/32], s [col][K/32] and, for Q6_K, -32 x the sum
//    of each half block [col][half][K/32];
//  - lanes decode "units" of the GGUF blocks from LDS (Q4_K: 32 quant bytes =
//    two 32-weight groups + the block header; Q6_K: 48 B of ql/qh = 64
//    weights; Q8_0: one 34 B block) with unaligned LDS reads, take int8 dots
//    with v_dot4 against the q8_1 quants, apply the scales per group in fp32,
//    and reduce each row across its lane segment with DPP.
// The routed form (mul_mat_id for small token counts) runs the same kernel
// per (expert, group of routes), so an expert's weights are read once however
// many of the group's tokens route to it.
#include "kernels.hpp"

namespace ggq {

constexpr int EPI_NONE = 0, EPI_SWIGLU = 1;
constexpr int MMVQ_MAXI = 12;   // DMA instructions (1 KB each) per work item, at most

#define AS3 __attribute__((address_space(3)))
typedef const uint8_t AS3 *lds_bp;
typedef v4i __attribute__((aligned(4))) v4i_u4;                // 16 B at 4-byte alignment

// ---- LDS loads ----
// A ds_read_b128 from a 2-byte (not 4-byte) aligned address is legal here but
// several times slower than an aligned one, so fields of 2-byte aligned blocks
// are read as aligned dwords and shifted into place with v_alignbyte.
__device__ __forceinline__ v4i l128(lds_bp p) { return *(const v4i AS3 *)p; }          // 16-aligned
__device__ __forceinline__ v4i l128w(lds_bp p) { return *(const v4i_u4 AS3 *)p; }      // 4-aligned
__device__ __forceinline__ uint32_t l32(lds_bp p) { return *(const uint32_t AS3 *)p; }  // 4-aligned
__device__ __forceinline__ uint32_t l16(lds_bp p) { return *(const uint16_t AS3 *)p; }
__device__ __forceinline__ float lf(lds_bp p) { return *(const float AS3 *)p; }
__device__ __forceinline__ v2i l64(lds_bp p) { return *(const v2i AS3 *)p; }           // 8-aligned

__device__ __forceinline__ int abyte(uint32_t hi, uint32_t lo, uint32_t s) {
    return (int)__builtin_amdgcn_alignbyte(hi, lo, s);              // bytes s .. s+3 of hi:lo
}
// 16 bytes at a + s (a 4-aligned, s in {0, 2}); reads [a, a + 20).
__device__ __forceinline__ v4i l128s(lds_bp a, uint32_t s) {
    const v4i w = l128w(a);
    const uint32_t w4 = l32(a + 16);
    return v4i{abyte(w.y, w.x, s), abyte(w.z, w.y, s), abyte(w.w, w.z, s), abyte(w4, w.w, s)};
}

// ---- per-type decode helpers (shared by the units and the test hook) ----

// Q4_K: the 6-bit scales (sc) and mins (mn) of groups 2p and 2p+1, from the
// 12 packed bytes s0..s2 (dwords).  Groups 0..3 keep their low 6 bits in bytes
// 0..3 (scales) and 4..7 (mins); groups 4..7 take the low nibble (scale) and
// high nibble (min) of bytes 8..11 plus the top two bits of bytes 0..3 / 4..7.
__device__ __forceinline__ void q4k_scales(int p, uint32_t s0, uint32_t s1, uint32_t s2, int &sc0, int &sc1, int &mn0,
                                           int &mn1) {
    const uint32_t scw = p < 2 ? (s0 & 0x3f3f3f3fu) : ((s2 & 0x0f0f0f0fu) | ((s0 >> 2) & 0x30303030u));
    const uint32_t mnw = p < 2 ? (s1 & 0x3f3f3f3fu) : (((s2 >> 4) & 0x0f0f0f0fu) | ((s1 >> 2) & 0x30303030u));
    const int sh = 16 * (p & 1);
    sc0 = (int)__builtin_amdgcn_ubfe(scw, sh, 8);
    sc1 = (int)__builtin_amdgcn_ubfe(scw, sh + 8, 8);
    mn0 = (int)__builtin_amdgcn_ubfe(mnw, sh, 8);
    mn1 = (int)__builtin_amdgcn_ubfe(mnw, sh + 8, 8);
}
__device__ __forceinline__ int nib_lo(int qs) { return qs & 0x0f0f0f0f; }
__device__ __forceinline__ int nib_hi(int qs) { return (int)(((uint32_t)qs >> 4) & 0x0f0f0f0fu); }

// Q5_K: the fifth bit (bit j of each byte of one qh dword) moved to bit 4 of
// each byte, to be ORed onto the nibbles of group j.
__device__ __forceinline__ int q5k_bit(uint32_t qh, int j) { return (int)(((qh >> j) & 0x01010101u) << 4); }

// Q6_K: 4 packed 6-bit weights (0..63, before the -32 offset) of quarter g
// from one dword of ql (low nibbles for g < 2, high for g >= 2) and one of qh
// (bits 2g, 2g+1 of each byte).
__device__ __forceinline__ int q6k_raw(uint32_t ql, uint32_t qh, int g) {
    const uint32_t lo = g < 2 ? (ql & 0x0f0f0f0fu) : ((ql >> 4) & 0x0f0f0f0fu);
    const uint32_t hb = g == 0 ? (qh << 4) : g == 1 ? (qh << 2) : g == 2 ? qh : (qh >> 2);
    return (int)(lo | (hb & 0x30303030u));
}

// Planar activations of one workgroup in LDS.
struct ActL {
    lds_bp qa;    // int8 [NC][K]
    lds_bp d8;    // float [NC][nb]
    lds_bp s8;    // float [NC][nb]
    lds_bp h16;   // int [NC][2][nb]: -32 * sum of quants 0..15 / 16..31 of each block
    int K, nb;
};

template <int T, int NC>
struct Unit;

// ---- Q4_K: unit = (super-block sb, pair p): the 32 quant bytes of groups 2p
// (low nibbles) and 2p+1 (high nibbles), 64 weights.
// Wide column groups: finish a column's dots before the next column's
// activation loads (else all NC x 16 registers of quants are live at once).
// The empty asm takes the column's sums and orders memory accesses.
template <int NC>
__device__ __forceinline__ void col_fence(float &a0, float &a1) {
    if (NC >= 4) asm volatile("" : "+v"(a0), "+v"(a1) :: "memory");
}

template <int NC>
struct Unit<T_Q4_K, NC> {
    __device__ static void run(int u, lds_bp row0, lds_bp row1, const ActL &A, int ncols, float (&acc)[2][NC]) {
        const int sb = u >> 2, p = u & 3;
        const lds_bp rows[2] = {row0, row1};
        int lo[2][8], hi[2][8];
        float d[2], dm[2], sc0[2], sc1[2], mn0[2], mn1[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const lds_bp blk = rows[i] + sb * 144;
            const v4i hdr = l128(blk);                                // Q4_K blocks stay 16-aligned
            const v4i q0 = l128(blk + 16 + 32 * p), q1 = l128(blk + 32 + 32 * p);
            d[i] = fp16_bits_to_f32((uint32_t)hdr.x & 0xffffu);
            dm[i] = fp16_bits_to_f32((uint32_t)hdr.x >> 16);
            int a, b, c, e;
            q4k_scales(p, (uint32_t)hdr.y, (uint32_t)hdr.z, (uint32_t)hdr.w, a, b, c, e);
            sc0[i] = (float)a; sc1[i] = (float)b; mn0[i] = (float)c; mn1[i] = (float)e;
#pragma unroll
            for (int w = 0; w < 4; w++) {
                lo[i][w] = nib_lo(q0[w]); lo[i][4 + w] = nib_lo(q1[w]);
                hi[i][w] = nib_hi(q0[w]); hi[i][4 + w] = nib_hi(q1[w]);
            }
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
            const int b0 = sb * 8 + 2 * p;                          // q8_1 block of group 2p
            const lds_bp qa = A.qa + col * A.K + b0 * 32;
            const v4i a0 = l128(qa), a1 = l128(qa + 16), a2 = l128(qa + 32), a3 = l128(qa + 48);
            const v2i dd = l64(A.d8 + (col * A.nb + b0) * 4), ss = l64(A.s8 + (col * A.nb + b0) * 4);
            const float d80 = as_float(dd.x), d81 = as_float(dd.y);
            const float s80 = as_float(ss.x), s81 = as_float(ss.y);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                int D0 = 0, D1 = 0;
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    D0 = dot4(lo[i][w], a0[w], D0);
                    D0 = dot4(lo[i][4 + w], a1[w], D0);
                    D1 = dot4(hi[i][w], a2[w], D1);
                    D1 = dot4(hi[i][4 + w], a3[w], D1);
                }
                acc[i][col] += d[i] * (sc0[i] * d80 * (float)D0 + sc1[i] * d81 * (float)D1) -
                               dm[i] * (mn0[i] * s80 + mn1[i] * s81);
            }
            col_fence<NC>(acc[0][col], acc[1][col]);
        }
    }
};

// ---- Q5_K: unit = (super-block sb, pair p), as Q4_K: groups 2p and 2p+1
// from the low / high nibbles of 32 quant bytes (at byte 48 of the block) with
// their fifth bits from bits 2p / 2p+1 of the 32 high-bit bytes (at byte 16).
template <int NC>
struct Unit<T_Q5_K, NC> {
    __device__ static void run(int u, lds_bp row0, lds_bp row1, const ActL &A, int ncols, float (&acc)[2][NC]) {
        const int sb = u >> 2, p = u & 3;
        const lds_bp rows[2] = {row0, row1};
        int lo[2][8], hi[2][8];
        float d[2], dm[2], sc0[2], sc1[2], mn0[2], mn1[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const lds_bp blk = rows[i] + sb * 176;                    // Q5_K blocks stay 16-aligned
            const v4i hdr = l128(blk);
            const v4i h0 = l128(blk + 16), h1 = l128(blk + 32);
            const v4i q0 = l128(blk + 48 + 32 * p), q1 = l128(blk + 64 + 32 * p);
            d[i] = fp16_bits_to_f32((uint32_t)hdr.x & 0xffffu);
            dm[i] = fp16_bits_to_f32((uint32_t)hdr.x >> 16);
            int a, b, c, e;
            q4k_scales(p, (uint32_t)hdr.y, (uint32_t)hdr.z, (uint32_t)hdr.w, a, b, c, e);
            sc0[i] = (float)a; sc1[i] = (float)b; mn0[i] = (float)c; mn1[i] = (float)e;
#pragma unroll
            for (int w = 0; w < 4; w++) {
                lo[i][w] = nib_lo(q0[w]) | q5k_bit((uint32_t)h0[w], 2 * p);
                lo[i][4 + w] = nib_lo(q1[w]) | q5k_bit((uint32_t)h1[w], 2 * p);
                hi[i][w] = nib_hi(q0[w]) | q5k_bit((uint32_t)h0[w], 2 * p + 1);
                hi[i][4 + w] = nib_hi(q1[w]) | q5k_bit((uint32_t)h1[w], 2 * p + 1);
            }
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
            const int b0 = sb * 8 + 2 * p;                          // q8_1 block of group 2p
            const lds_bp qa = A.qa + col * A.K + b0 * 32;
            const v4i a0 = l128(qa), a1 = l128(qa + 16), a2 = l128(qa + 32), a3 = l128(qa + 48);
            const v2i dd = l64(A.d8 + (col * A.nb + b0) * 4), ss = l64(A.s8 + (col * A.nb + b0) * 4);
            const float d80 = as_float(dd.x), d81 = as_float(dd.y);
            const float s80 = as_float(ss.x), s81 = as_float(ss.y);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                int D0 = 0, D1 = 0;
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    D0 = dot4(lo[i][w], a0[w], D0);
                    D0 = dot4(lo[i][4 + w], a1[w], D0);
                    D1 = dot4(hi[i][w], a2[w], D1);
                    D1 = dot4(hi[i][4 + w], a3[w], D1);
                }
                acc[i][col] += d[i] * (sc0[i] * d80 * (float)D0 + sc1[i] * d81 * (float)D1) -
                               dm[i] * (mn0[i] * s80 + mn1[i] * s81);
            }
            col_fence<NC>(acc[0][col], acc[1][col]);
        }
    }
};

// ---- Q6_K: unit = (super-block sb, half hh, lane range t): 64 weights =
// 16 consecutive l of each of the four 32-groups g of the half.  The dots run
// on the raw 0..63 values with the chain started at -32 x (sum of the 16
// activation quants), which is the dot with (q - 32).
template <int NC>
struct Unit<T_Q6_K, NC> {
    __device__ static void run(int u, lds_bp row0, lds_bp row1, const ActL &A, int ncols, float (&acc)[2][NC]) {
        const int sb = u >> 2, hh = (u >> 1) & 1, t = u & 1;
        const lds_bp rows[2] = {row0, row1};
        int q[2][4][4];
        float dsc[2][4];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const lds_bp blk = rows[i] + sb * 210;                    // 2-byte aligned for odd sb
            const uint32_t s = (uint32_t)(uintptr_t)blk & 3;
            const lds_bp ba = blk - s;
            const v4i ql0 = l128s(ba + 64 * hh + 16 * t, s);
            const v4i ql1 = l128s(ba + 64 * hh + 32 + 16 * t, s);
            const v4i qh = l128s(ba + 128 + 32 * hh + 16 * t, s);
            const uint32_t c0 = l32(ba + 192 + 8 * hh), c1 = l32(ba + 196 + 8 * hh), c2 = l32(ba + 200 + 8 * hh);
            const v2i scw = {abyte(c1, c0, s), abyte(c2, c1, s)};       // scales 8hh .. 8hh+7
            const float d = fp16_bits_to_f32(l16(blk + 208));
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int k = 2 * g + t;                               // scale index - 8hh
                const uint32_t sw = (uint32_t)(k < 4 ? scw.x : scw.y);
                dsc[i][g] = d * (float)(int)__builtin_amdgcn_sbfe((int)sw, 8 * (k & 3), 8);   // signed operand: signed extract
#pragma unroll
                for (int w = 0; w < 4; w++) q[i][g][w] = q6k_raw((uint32_t)((g & 1) ? ql1[w] : ql0[w]), (uint32_t)qh[w], g);
            }
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
            const int b0 = sb * 8 + 4 * hh;                            // q8_1 block of g = 0
            const lds_bp qa = A.qa + col * A.K + b0 * 32 + 16 * t;
            const v4i dv = l128(A.d8 + (col * A.nb + b0) * 4);
            const v4i hv = l128(A.h16 + ((col * 2 + t) * A.nb + b0) * 4);
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const v4i a = l128(qa + 32 * g);
                const float d8 = as_float(dv[g]);
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    int D = hv[g];
#pragma unroll
                    for (int w = 0; w < 4; w++) D = dot4(q[i][g][w], a[w], D);
                    acc[i][col] += dsc[i][g] * d8 * (float)D;
                }
            }
            col_fence<NC>(acc[0][col], acc[1][col]);
        }
    }
};

// ---- Q8_0: unit = one 34-byte block (32 weights).
template <int NC>
struct Unit<T_Q8_0, NC> {
    __device__ static void run(int u, lds_bp row0, lds_bp row1, const ActL &A, int ncols, float (&acc)[2][NC]) {
        const lds_bp rows[2] = {row0, row1};
        v4i q[2][2];
        float d[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const lds_bp blk = rows[i] + u * 34;                      // 2-byte aligned
            d[i] = fp16_bits_to_f32(l16(blk));
            const uint32_t s = (uint32_t)(uintptr_t)(blk + 2) & 3;
            const lds_bp qa = blk + 2 - s;
            const v4i w0 = l128w(qa), w1 = l128w(qa + 16);
            const uint32_t w2 = l32(qa + 32);
            q[i][0] = v4i{abyte(w0.y, w0.x, s), abyte(w0.z, w0.y, s), abyte(w0.w, w0.z, s), abyte(w1.x, w0.w, s)};
            q[i][1] = v4i{abyte(w1.y, w1.x, s), abyte(w1.z, w1.y, s), abyte(w1.w, w1.z, s), abyte(w2, w1.w, s)};
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
            const lds_bp qa = A.qa + col * A.K + u * 32;
            const v4i a0 = l128(qa), a1 = l128(qa + 16);
            const float d8 = lf(A.d8 + (col * A.nb + u) * 4);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                int D = 0;
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    D = dot4(q[i][0][w], a0[w], D);
                    D = dot4(q[i][1][w], a1[w], D);
                }
                acc[i][col] += d[i] * d8 * (float)D;
            }
            col_fence<NC>(acc[0][col], acc[1][col]);
        }
    }
};

// ---- Q4_0: unit = one 18-byte block (32 weights): byte b of the 16 quant
// bytes holds weight b (low nibble) and weight 16 + b (high nibble), value
// d * (nibble - 8).  The -8 enters through the block's activation sum:
// d * (d8 * D - 8 * s8), D the dot of the raw nibbles.
template <int NC>
struct Unit<T_Q4_0, NC> {
    __device__ static void run(int u, lds_bp row0, lds_bp row1, const ActL &A, int ncols, float (&acc)[2][NC]) {
        const lds_bp rows[2] = {row0, row1};
        v4i lo[2], hi[2];
        float d[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const lds_bp blk = rows[i] + u * 18;                      // 2-byte aligned
            d[i] = fp16_bits_to_f32(l16(blk));
            const uint32_t s = (uint32_t)(uintptr_t)(blk + 2) & 3;
            const v4i q = l128s(blk + 2 - s, s);
#pragma unroll
            for (int w = 0; w < 4; w++) {
                lo[i][w] = nib_lo(q[w]);
                hi[i][w] = nib_hi(q[w]);
            }
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
            const lds_bp qa = A.qa + col * A.K + u * 32;
            const v4i a0 = l128(qa), a1 = l128(qa + 16);
            const float d8 = lf(A.d8 + (col * A.nb + u) * 4), s8 = lf(A.s8 + (col * A.nb + u) * 4);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                int D = 0;
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    D = dot4(lo[i][w], a0[w], D);
                    D = dot4(hi[i][w], a1[w], D);
                }
                acc[i][col] += d[i] * (d8 * (float)D - 8.0f * s8);
            }
            col_fence<NC>(acc[0][col], acc[1][col]);
        }
    }
};

// YDT: DT_F32, or a 16-bit output (fp16 when h, else bf16).
template <int YDT>
__device__ __forceinline__ void store_out(void *y, int64_t idx, float v, bool h) {
    if (YDT == DT_F32) static_cast<float *>(y)[idx] = v;
    else static_cast<uint16_t *>(y)[idx] = (uint16_t)f32_to_16(v, h);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Stores of a finished row pair (rows r0 and, when v1, r1) for the group's
// columns, by the lane holding the segment totals.  The per-launch choices (fp16
// or bf16 elements, whether a row pair's two outputs share one aligned store)
// are taken once, outside the column loop, so that the loop is straight-line.
// cix: the columns' activation rows (dense) or route indices (routed).
template <int NC, bool MOE, int EPI, int YDT, bool H>
__device__ __forceinline__ void store_cols(const MmvqParams &p, const float (&acc)[2][NC], const int64_t (&cix)[NC],
                                           int ncols, bool v1, int64_t r0, int64_t r1) {
    if (!MOE) {
        if (v1 && (p.ldy & 1) == 0) {                      // r0 even, r1 = r0 + 1: one store per column
#pragma unroll
            for (int c = 0; c < NC; c++) {
                if (c < ncols) {
                    const int64_t idx = cix[c] * p.ldy + r0;
                    if (YDT == DT_F32) {
                        float *yp = static_cast<float *>(p.y) + idx;
                        yp[0] = acc[0][c];
                        yp[1] = acc[1][c];
                    } else
                        *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(p.y) + idx) =
                            f32_to_16(acc[0][c], H) | (f32_to_16(acc[1][c], H) << 16);
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < NC; c++) {
                if (c < ncols) {
                    const int64_t idx = cix[c] * p.ldy + r0;
                    store_out<YDT>(p.y, idx, acc[0][c], H);
                    if (v1) store_out<YDT>(p.y, idx + 1, acc[1][c], H);
                }
            }
        }
    } else {
        // weighted: per-route outputs (output dtype), summed per token afterwards
        void *o = p.oroute ? p.oroute : p.y;
#pragma unroll
        for (int c = 0; c < NC; c++) {
            if (c < ncols) {
                const int64_t r = cix[c];
                if (EPI == EPI_SWIGLU) {
                    store_out<YDT>(o, r * p.Np + r0, silu_mul(acc[0][c], acc[1][c]), H);
                } else {
                    store_out<YDT>(o, r * p.Np + r0, acc[0][c], H);
                    if (v1) store_out<YDT>(o, r * p.Np + r1, acc[1][c], H);
                }
            }
        }
    }
}
template <int NC, bool MOE, int EPI, int YDT>
__device__ __forceinline__ void store_pair(const MmvqParams &p, const float (&acc)[2][NC], const int64_t (&cix)[NC],
                                           int ncols, bool v1, int64_t r0, int64_t r1) {
    if (YDT != DT_F32 && p.y_f16) store_cols<NC, MOE, EPI, YDT, true>(p, acc, cix, ncols, v1, r0, r1);
    else store_cols<NC, MOE, EPI, YDT, false>(p, acc, cix, ncols, v1, r0, r1);
}

// q = round-half-away(x / d) in fp32 with d = amax / 127 and the IEEE
// quotient, as the quantizer defines it, by the compiler's division: the
// fallback of put() for blocks outside the range quant_div() covers, and for
// f32 lanes whose fast rounding is ambiguous.
__device__ __forceinline__ int quant_exact(float x, float d) {
    const float z = x / d;
    const float t = __builtin_truncf(z);
    const float q = fabsf(z - t) >= 0.5f ? t + __builtin_copysignf(1.0f, z) : t;
    return (int)__builtin_amdgcn_fmed3f(q, -127.0f, 127.0f);
}

// The same q without a division instruction per value, for a block scale
// d = amax / 127 with 2^-60 <= amax <= 2^96 and |x| <= amax: z = fl(x / d)
// from q0 = x y (y: v_rcp of d refined by one Newton step) and two
// corrections q + (x - d q) y, each residual exact by the fma (Markstein's
// correction steps); in that range no product, quotient or residual leaves the
// normal range, so no operand scaling is needed.  Then round half away from
// zero.
__device__ __forceinline__ int quant_div(float x, float d, float y) {
    const float q0 = x * y;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-d, q0, x), y, q0);
    const float z = __builtin_fmaf(__builtin_fmaf(-d, q1, x), y, q1);
    // for |z| <= 128, z + copysign(0.5 - 2^-25, z) truncated is z rounded half
    // away from zero (checked for every float in that range)
    return (int)(z + __builtin_copysignf(0x1.fffffep-2f, z));
}

// Activation rows of this block's columns -> planar q8_1 in LDS.  A 32-value
// block is spread over LPB lanes (lane sub of a group holds values VPL sub ..
// VPL sub + VPL - 1): 4 lanes for one column, so that 512 lanes take a
// 4096-value row in one pass; 2 for two columns and 1 for more, so that the
// per-block work (the block maximum and its cross-lane steps, the scale, the
// stores) is shared by fewer lanes when every lane has several blocks to do.
// put() is the arithmetic of the standalone quantizer (amax / 127 with IEEE
// division, round half away from zero, s = d * sum(q)), or takes a given q8_1
// block as is.
// x / 127 correctly rounded, by one multiplication and two fmas: q = x * c
// with c = fl(1/127), then q + (x - 127 q) c.  For 2^-96 <= x <= 2^126 every
// intermediate is a normal number and the result equals IEEE division for all
// such x (checked over every mantissa of a binade; scaling by powers of two
// is exact there).  Other x (tiny, huge, inf) take the division.
__device__ __forceinline__ float div127(float x) {
    if (!(x >= 0x1p-96f && x <= 0x1p126f)) return x / 127.0f;
    constexpr float c = 1.0f / 127.0f;
    const float q = x * c;
    return __builtin_fmaf(__builtin_fmaf(-q, 127.0f, x), c, q);
}

template <int NC>
constexpr int act_lpb() { return NC == 1 ? 4 : NC == 2 ? 2 : 1; }

template <int NC, bool H16>
struct ActStage {
    static constexpr int LPB = act_lpb<NC>(), VPL = QK8_1 / LPB;      // lanes per block, values per lane
    static constexpr int NW = VPL / 4;                                  // 16-byte words of a lane's raw f32 values
    // A lane's raw bytes of a block: f32 values in w[0 .. NW); bf16 / fp16 values
    // in w[0 .. NW / 2); q8_1: d, s in w[0].x, w[0].y, the lane's VPL quants in
    // the ints from w[1] on.
    struct Raw {
        v4i w[NW];
        __device__ int word(int i) const { return w[i >> 2][i & 3]; }
        __device__ void set_word(int i, int v) { w[i >> 2][i & 3] = v; }
    };
    uint32_t nb_magic;            // b / nb == umulhi(b, nb_magic) for every block index b used here

    __device__ void init(uint32_t magic) { nb_magic = magic; }
    __device__ int col_of(int b) const { return (int)__umulhi((uint32_t)b, nb_magic); }
    __device__ static int sub() { return (int)(threadIdx.x & (LPB - 1)); }

    // Raw bytes of block b for this lane from global memory.  XS (the source
    // type) is a template argument so that put() compiles to straight-line code.
    template <int XS>
    __device__ void fetch(const MmvqParams &p, const int64_t *xrow, int nb, int b, Raw &r) const {
        const int c = col_of(b), blk = b - c * nb;
        if (XS == DT_Q8_1) {
            const uint8_t *a0 = p.q8 + xrow[c] * p.q8_row + (int64_t)blk * Q8_1_BYTES;
            const v2i h = *reinterpret_cast<const v2i *>(a0);
            r.w[0] = v4i{h.x, h.y, 0, 0};
#pragma unroll
            for (int i = 0; i < VPL / 8; i++) {
                const v2i q = *reinterpret_cast<const v2i *>(a0 + 8 + VPL * sub() + 8 * i);
                r.set_word(4 + 2 * i, q.x);
                r.set_word(5 + 2 * i, q.y);
            }
        } else {
            constexpr int esz = XS == DT_F32 ? 4 : 2;
            const uint8_t *a0 = static_cast<const uint8_t *>(p.x) + (xrow[c] * p.ldx + blk * QK8_1 + sub() * VPL) * esz;
#pragma unroll
            for (int i = 0; i < VPL * esz / 16; i++) r.w[i] = *reinterpret_cast<const v4i *>(a0 + 16 * i);
        }
    }

    // Same as fetch(), from raw activation rows already copied into LDS at
    // `raw` (column c at c * K * esz, or c * nb * 40 for q8_1 blocks).
    template <int XS>
    __device__ void fetch_lds(const uint8_t *raw, int K, int nb, int b, Raw &r) const {
        const int c = col_of(b), blk = b - c * nb;
        if (XS == DT_Q8_1) {
            const lds_bp a0 = (lds_bp)raw + (c * nb + blk) * Q8_1_BYTES;
            const v2i h = l64(a0);
            r.w[0] = v4i{h.x, h.y, 0, 0};
#pragma unroll
            for (int i = 0; i < VPL / 8; i++) {
                const v2i q = l64(a0 + 8 + VPL * sub() + 8 * i);
                r.set_word(4 + 2 * i, q.x);
                r.set_word(5 + 2 * i, q.y);
            }
        } else {
            constexpr int esz = XS == DT_F32 ? 4 : 2;
            const lds_bp a0 = (lds_bp)raw + (c * K + blk * QK8_1 + sub() * VPL) * esz;
#pragma unroll
            for (int i = 0; i < VPL * esz / 16; i++) r.w[i] = l128(a0 + 16 * i);
        }
    }

    // Quantize (or take) block b and write it to the planar layout.  All LPB
    // lanes of the group take part (cross-lane steps within the group).
    template <int XS>
    __device__ void put(uint8_t *lds, int K, int nb, int b, const Raw &r) const {
        uint8_t *qa = lds;
        float *d8 = reinterpret_cast<float *>(lds + NC * K);
        float *s8 = d8 + NC * nb;
        int *h16 = reinterpret_cast<int *>(s8 + NC * nb);
        int q[VPL / 4];                                   // the lane's quants, 4 per int
        float dq, sq;
        if (XS == DT_Q8_1) {
#pragma unroll
            for (int i = 0; i < VPL / 4; i++) q[i] = r.word(4 + i);
            dq = as_float(r.w[0].x);
            sq = as_float(r.w[0].y);
        } else {
            float v[VPL];
#pragma unroll
            for (int i = 0; i < VPL; i++) {
                if (XS == DT_F32) v[i] = as_float(r.word(i));
                else v[i] = from_16(((uint32_t)r.word(i >> 1) >> (16 * (i & 1))) & 0xffffu, XS == DT_F16);
            }
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < VPL; i++) m = fmaxf(m, fabsf(v[i]));
            if (LPB >= 2) m = fmaxf(m, dpp_f<DPP_XOR1>(m));
            if (LPB >= 4) m = fmaxf(m, dpp_f<DPP_XOR2>(m));
            const float amax = m;
            float d = 0.0f;
#pragma unroll
            for (int i = 0; i < VPL / 4; i++) q[i] = 0;
            if (amax != 0.0f) {
                d = div127(amax);
                const float inv = __builtin_amdgcn_rcpf(d);
                int qb[VPL];
                const bool ranged = amax >= 0x1p-60f && amax <= 0x1p96f;
                if (XS != DT_F32 && ranged) {
                    // 16-bit values: short significands put about 1 value in 200
                    // within 2^-14 of a half-integer quotient (many exactly on one),
                    // so nearly every wave would take a fallback; the exact
                    // quotient for every value costs less.
                    const float y = __builtin_fmaf(__builtin_fmaf(-d, inv, 1.0f), inv, inv);
#pragma unroll
                    for (int i = 0; i < VPL; i++) qb[i] = quant_div(v[i], d, y);
                } else {
                    // fma(v, inv, 1.5 * 2^23) rounds v * inv (|v * inv| <= 128) to
                    // the nearest integer and leaves it, two's complement, in the low
                    // byte of the result's bits.  e is the largest distance of a
                    // product from its integer: below 0.5 - 2^-14 the quotient v / d,
                    // within 128 * 2^-23 of v * inv (v_rcp_f32 is good to 1 ulp),
                    // rounds to the same integer and is no tie; otherwise the lane's
                    // values take the exact division.
                    constexpr float RM = 12582912.0f;
                    float e = 0.0f;
#pragma unroll
                    for (int i = 0; i < VPL; i++) {
                        const float rv = __builtin_fmaf(v[i], inv, RM);
                        e = fmaxf(e, fabsf(__builtin_fmaf(v[i], inv, RM - rv)));
                        qb[i] = __builtin_bit_cast(int, rv);
                    }
                    if (!(e < 0.5f - 0x1p-14f)) {
#pragma unroll
                        for (int i = 0; i < VPL; i++) qb[i] = quant_exact(v[i], d);
                    }
                }
#pragma unroll
                for (int i = 0; i < VPL / 4; i++)
                    q[i] = (int)(__builtin_amdgcn_perm((uint32_t)qb[4 * i + 1], (uint32_t)qb[4 * i], 0x0c0c0400u) |
                                 __builtin_amdgcn_perm((uint32_t)qb[4 * i + 3], (uint32_t)qb[4 * i + 2], 0x04000c0cu));
            }
            dq = d;
        }
        // sums of the lane's quants: by halves of the block when LPB == 1
        int qs0 = 0, qs1 = 0;
#pragma unroll
        for (int i = 0; i < VPL / 4; i++) {
            if (LPB == 1 && i >= VPL / 8) qs1 = dot4(q[i], 0x01010101, qs1);
            else qs0 = dot4(q[i], 0x01010101, qs0);
        }
        if (XS != DT_Q8_1) {
            int qsum = qs0 + qs1;
            if (LPB >= 2) qsum += dpp_i<DPP_XOR1>(qsum);
            if (LPB >= 4) qsum += dpp_i<DPP_XOR2>(qsum);
            sq = dq * (float)qsum;
        }
        const int c = col_of(b), blk = b - c * nb;
        uint8_t *qdst = qa + c * K + blk * QK8_1 + VPL * sub();
        if (VPL == 8) *reinterpret_cast<v2i *>(qdst) = v2i{q[0], q[1]};
#pragma unroll
        for (int i = 0; VPL >= 16 && i < VPL / 16; i++)
            *reinterpret_cast<v4i *>(qdst + 16 * i) = v4i{q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]};
        if (sub() == 0) {
            d8[c * nb + blk] = dq;
            s8[c * nb + blk] = sq;
        }
        if (H16) {
            // sums of the quants 0..15 and 16..31 of the block
            int *hd = h16 + c * 2 * nb + blk;
            if (LPB == 4) {                                  // lanes 0, 1: quants 0..15; lanes 2, 3: 16..31
                const int half = qs0 + dpp_i<DPP_XOR1>(qs0);
                if ((sub() & 1) == 0) hd[(sub() >> 1) * nb] = -32 * half;
            } else if (LPB == 2) {
                hd[sub() * nb] = -32 * qs0;
            } else {
                hd[0] = -32 * qs0;
                hd[nb] = -32 * qs1;
            }
        }
    }
};

// ---- LDS weight staging ----
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(v4i rsrc, AS3 uint32_t *lds, int size, int voffset,
                                                           int soffset, int offset,
                                                           int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }    // vmcnt(0)
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)
// vmcnt(n) for a wave-uniform n in 0..MMVQ_MAXI: everything but the last n
// vector-memory instructions of this wave has completed.
__device__ __forceinline__ void wait_vm_n(int n) {
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    }
}
__device__ __forceinline__ void compiler_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }
// Workgroup barrier for LDS data only: this wave's LDS writes are complete,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global loads (the weight copy in flight); LDS written by DMA must be waited
// for explicitly (vmcnt) before it.
__device__ __forceinline__ void lds_barrier() {
    wait_lgkm();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// One work item of a wave = (group of spw row pairs, K-chunk kc): the 2*spw
// rows ("slots") of the group, blocks [kc*bpc, (kc+1)*bpc) of each.  With A
// the address of the chunk in the group's first row, phi = A & 15 and
// base = A - phi, slot s is the row at byte distance rel_s * row_bytes from
// the first row; its chunk starts phi + rel_s * row_bytes bytes past base and
// is staged from the 16-byte boundary below that on, at LDS offset
// s * cps * 16.  Instruction k moves the 16-byte pieces idx = lane + 64k
// (slot idx / cps, piece idx % cps) from offset (phi + off) & ~15, with
// off = rel_s * row_bytes + 16 * piece fixed per lane for the whole kernel.
// Pieces of unused slots get an offset past the buffer range and land as
// zeros without touching memory; rows past the last weight byte do the same
// through the descriptor's range.
constexpr uint32_t STAGE_UNUSED = 0xffffff00u;
struct Stage {
    uint32_t off[MMVQ_MAXI];     // rel_s * row_bytes + 16 * piece of this lane's piece in instruction k
};

// FIXED: issue all MMVQ_MAXI instructions, the ones past ninst reading
// nothing (offset past the range) into the 1 KB `sink`, so the number of
// vector-memory instructions is known at compile time and the compiler's own
// waits for older loads (the activations in the prologue) count past them.
template <bool FIXED = false>
__device__ __forceinline__ void stage_issue(const uint8_t *A, const uint8_t *wend, uint8_t *buf, const Stage &S,
                                            int ninst, uint8_t *sink = nullptr) {
    const uint32_t phi = (uint32_t)(reinterpret_cast<uintptr_t>(A) & 15);
    const uint8_t *base = A - phi;
    const int64_t avail = wend - base;
    struct { const void *p; uint32_t range; uint32_t cfg; } r = {
        base, (uint32_t)(avail < 0x7fffff00LL ? avail : 0x7fffff00LL), 0x00020000u};
    v4i rsrc = __builtin_bit_cast(v4i, r);
#pragma unroll
    for (int i = 0; i < 4; i++) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);   // wave-uniform descriptor
#pragma unroll
    for (int k = 0; k < MMVQ_MAXI; k++) {
        if (FIXED) {
            const bool use = k < ninst;
            llvm_amdgcn_raw_buffer_load_lds(rsrc, (AS3 uint32_t *)(use ? buf + 1024 * k : sink), 16,
                                            (int)((phi + (use ? S.off[k] : STAGE_UNUSED)) & ~15u), 0, 0, 0);
        } else if (k < ninst) {
            llvm_amdgcn_raw_buffer_load_lds(rsrc, (AS3 uint32_t *)(buf + 1024 * k), 16, (int)((phi + S.off[k]) & ~15u),
                                            0, 0, 0);
        }
    }
}

// The first item of a wave, issued at the top of the kernel before the per-lane
// table exists: the same offsets as stage_issue's, computed per instruction.
template <int EPI>
__device__ __forceinline__ void stage_issue_first(const uint8_t *A, const uint8_t *wend, uint8_t *buf, int ninst,
                                                  int lane, uint32_t cps, uint32_t cps_magic, uint32_t spw,
                                                  uint32_t rb32, uint32_t np_rb);

// wend is 2-byte aligned; when it is not 4-byte aligned the dword holding its
// last two bytes is outside the range and landed as zero: patch those two
// bytes from a 16-bit load (after the copy has landed).
__device__ __forceinline__ void stage_patch(const uint8_t *A, const uint8_t *wend, uint8_t *buf, const Stage &S,
                                            int ninst, int lane) {
    const uint32_t phi = (uint32_t)(reinterpret_cast<uintptr_t>(A) & 15);
    const uint8_t *base = A - phi;
    const uint8_t *last = wend - 2;
    if (last < base) return;
#pragma unroll
    for (int k = 0; k < MMVQ_MAXI; k++) {
        if (k < ninst && S.off[k] != STAGE_UNUSED) {
            const uint8_t *g = base + ((phi + S.off[k]) & ~15u);
            if (g <= last && last < g + 16)
                *reinterpret_cast<uint16_t *>(buf + 1024 * k + 16 * lane + (last - g)) = *reinterpret_cast<const uint16_t *>(last);
        }
    }
}

// Row distance (in rows) of slot s from the first row of its group.
template <int EPI>
__device__ __forceinline__ int64_t slot_rel(int s, int64_t Np) {
    return EPI == EPI_SWIGLU ? (int64_t)(s >> 1) + (s & 1) * Np : (int64_t)s;
}

// Byte offset of row slot s from the first row of its group, in 32 bits (the
// launcher bounds every such offset, row_bytes below 2^24 and np_rb = Np *
// row_bytes below 2^31).
template <int EPI>
__device__ __forceinline__ uint32_t slot_off(uint32_t s, uint32_t rb, uint32_t np_rb) {
    return EPI == EPI_SWIGLU ? __umul24(s >> 1, rb) + ((s & 1) ? np_rb : 0u) : __umul24(s, rb);
}

template <int EPI>
__device__ __forceinline__ void stage_issue_first(const uint8_t *A, const uint8_t *wend, uint8_t *buf, int ninst,
                                                  int lane, uint32_t cps, uint32_t cps_magic, uint32_t spw,
                                                  uint32_t rb32, uint32_t np_rb) {
    const uint32_t phi = (uint32_t)(reinterpret_cast<uintptr_t>(A) & 15);
    const uint8_t *base = A - phi;
    const int64_t avail = wend - base;
    struct { const void *p; uint32_t range; uint32_t cfg; } r = {
        base, (uint32_t)(avail < 0x7fffff00LL ? avail : 0x7fffff00LL), 0x00020000u};
    v4i rsrc = __builtin_bit_cast(v4i, r);
#pragma unroll
    for (int i = 0; i < 4; i++) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
#pragma unroll 1
    for (int k = 0; k < ninst; k++) {
        const uint32_t P = (uint32_t)(lane + 64 * k), slot = __umulhi(P, cps_magic);
        const uint32_t c16 = 16u * P - __umul24(slot, 16u * cps);
        const uint32_t off = slot < 2u * spw ? slot_off<EPI>(slot, rb32, np_rb) + c16 : STAGE_UNUSED;
        llvm_amdgcn_raw_buffer_load_lds(rsrc, (AS3 uint32_t *)(buf + 1024 * k), 16, (int)((phi + off) & ~15u), 0, 0, 0);
    }
}

// Largest workgroup: 16 waves (one workgroup per CU quantizes the activations
// once for all of them); every column count fits 128 registers.
template <int NC>
struct MaxWaves { static constexpr int value = 16; };

// grid: (blocks_x, column groups), blockDim = 64 x waves.  Each block stages
// its columns' q8_1 activations in LDS, then each wave walks its work items
// (spw row pairs x K-chunks), copying item i+1 into its second LDS buffer
// while it computes item i from the first.
// DEEP (one or two columns, many items per wave): two work items in flight per wave.
template <int T, int NC, bool MOE, int EPI, int YDT, bool DEEP = false>
__global__ __launch_bounds__(64 * MaxWaves<NC>::value) void mmvq_kernel(const MmvqParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ int64_t xrow[NC];
    __shared__ uint32_t xoff[NC];     // byte offset of each column's raw activation row (DMA prologue)
    __shared__ int32_t route_s[NC];
    typedef Unit<T, NC> U;
    constexpr int BB = Geom<T>::BYTES;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wpb = blockDim.x >> 6;
    const int seg = p.seg, upl = p.upl, lane_in = lane & (seg - 1), spw = 64 / seg, sid = lane / seg;
    const int64_t grp = blockIdx.y;
    const int ninst = p.stage_ninst, cps = p.stage_cps, bpc = p.stage_bpc;
    const int bufsz = ninst * 1024;
    // item buffers: first buffers of all waves, then their second buffers (which
    // hold the raw activation rows during the prologue), then a 1 KB sink
    uint8_t *wbuf = lds + p.act_lds_bytes + wave * bufsz;
    const int bstride = wpb * bufsz;
    uint8_t *raw = lds + p.act_lds_bytes + bstride;
    uint8_t *sink = raw + p.raw_region;

    // ---- routed, one route per group, no route tables: group grp is route grp,
    // ids[grp] its expert.  Group 0 also counts the ids >= E.  (Block-uniform
    // branches; no copy is in flight yet, so an inactive route can just leave.)
    int32_t de = 0;
    if (MOE && p.ids) {
        if (grp >= p.R) return;
        if (grp == 0 && blockIdx.x == 0) {
            __shared__ uint32_t s_bad;
            if (threadIdx.x == 0) s_bad = 0;
            __syncthreads();
            uint32_t nbad = 0;
            for (int64_t r = threadIdx.x; r < p.R; r += blockDim.x) nbad += p.ids[r] >= p.E;
            if (nbad) atomicAdd(&s_bad, nbad);
            __syncthreads();
            if (threadIdx.x == 0) *p.bad = s_bad;
        }
        de = p.ids[grp];
        if (de < 0 || de >= p.E) {
            // inactive route: an unweighted output row is zeros (a weighted sum skips it)
            if (!p.route_w && blockIdx.x == 0)
                for (int64_t i = threadIdx.x; i < p.Np; i += blockDim.x) store_out<YDT>(p.y, grp * p.Np + i, 0.0f, p.y_f16);
            return;
        }
    }

    // ---- early copies (activation rows through LDS; dense, or routed with one route per
    // group): the activation rows, then the first weight item, go out before any table
    // is built or barrier passed.  A short launch starts with a cold instruction cache,
    // so every instruction ahead of these copies delays the first bytes; the
    // activations stay older than the weights, so waiting for all but the weight
    // instructions still covers them.
    const bool early = p.act_dma && (!MOE || p.ids);
    if (early) {
        // dense: columns grp * NC ..; direct routed: the route's activation row
        const int64_t c0 = !MOE ? grp * NC : (p.x_per_route ? grp : grp / p.top_k);
        const int nce = !MOE ? (int)min<int64_t>(NC, p.M - c0) : 1;
        const int nbe = (int)(p.K / QK8_1);
        const uint32_t rowb = p.xsrc == DT_Q8_1 ? nbe * Q8_1_BYTES : (uint32_t)p.K * (p.xsrc == DT_F32 ? 4 : 2);
        const uint32_t ppc = rowb / 16, pieces = nce * ppc;
        const uint8_t *xb = p.xsrc == DT_Q8_1 ? p.q8 : static_cast<const uint8_t *>(p.x);
        struct { const void *q; uint32_t range; uint32_t cfg; } r = {xb, (uint32_t)p.x_bytes, 0x00020000u};
        v4i rsrc = __builtin_bit_cast(v4i, r);
#pragma unroll
        for (int i = 0; i < 4; i++) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
        for (uint32_t j0 = (uint32_t)wave * 64; j0 < pieces; j0 += (uint32_t)wpb * 64) {
            const uint32_t j = j0 + lane, c = __umulhi(j, p.ppc_magic);
            const uint32_t xo = (uint32_t)((c0 + ((int)c < nce ? (int)c : 0)) * p.x_stride);
            const uint32_t voff = j < pieces ? xo + 16u * (j - __umul24(c, ppc)) : STAGE_UNUSED;
            llvm_amdgcn_raw_buffer_load_lds(rsrc, (AS3 uint32_t *)(raw + j0 * 16), 16, (int)voff, 0, 0, 0);
        }
        const int64_t pwe = ((int64_t)blockIdx.x * wpb + wave) * spw;
        const uint8_t *We = p.W + (int64_t)de * p.expert_stride;
        if (pwe < p.npairs)
            stage_issue_first<EPI>(We + (EPI == EPI_SWIGLU ? pwe : 2 * pwe) * p.row_bytes, p.W + p.w_bytes, wbuf,
                                   ninst, lane, (uint32_t)cps, p.cps_magic, (uint32_t)spw, (uint32_t)p.row_bytes,
                                   (uint32_t)(p.Np * p.row_bytes));
    }

    // ---- columns of this group ----
    const uint8_t *W = p.W;
    int ncols;
    if (!MOE) {
        const int64_t c0 = grp * NC;
        ncols = (int)min<int64_t>(NC, p.M - c0);
        if (threadIdx.x < NC) {
            const int64_t r = c0 + (threadIdx.x < ncols ? threadIdx.x : 0);
            xrow[threadIdx.x] = r;
            xoff[threadIdx.x] = (uint32_t)(r * p.x_stride);
        }
    } else if (p.ids) {
        W += (int64_t)de * p.expert_stride;                     // the route checked above
        ncols = 1;
        if (threadIdx.x < NC) {
            const int32_t r = (int32_t)grp;
            route_s[threadIdx.x] = r;
            const int64_t xr = p.x_per_route ? r : r / p.top_k;
            xrow[threadIdx.x] = xr;
            xoff[threadIdx.x] = (uint32_t)(xr * p.x_stride);
        }
    } else {
        if (grp >= (int64_t)*p.ngroups) return;                 // block-uniform
        const int4 g = p.groups[grp];
        W += (int64_t)g.x * p.expert_stride;
        ncols = g.z;
        if (threadIdx.x < NC) {
            const int c = threadIdx.x < ncols ? threadIdx.x : 0;
            const int32_t r = p.perm[g.y + c];
            route_s[threadIdx.x] = r;
            const int64_t xr = p.x_per_route ? r : r / p.top_k;
            xrow[threadIdx.x] = xr;
            xoff[threadIdx.x] = (uint32_t)(xr * p.x_stride);
        }
    }
    const uint8_t *wend = p.W + p.w_bytes;
    const int64_t rb = p.row_bytes;
    // xrow / route_s visible.  An LDS-only barrier: a full __syncthreads would also wait
    // for the early copies (vmcnt), putting their whole latency ahead of the prologue.
    lds_barrier();

    // ---- per-lane staging tables ----
    Stage S;
    const uint32_t rb32 = (uint32_t)rb, np_rb = (uint32_t)(p.Np * rb);
    {
        // piece P = lane + 64 k of an item: row slot P / cps, bytes 16 (P mod cps) on of that slot's chunk
#pragma unroll
        for (int k = 0; k < MMVQ_MAXI; k++) {
            S.off[k] = STAGE_UNUSED;
            if (k < ninst) {
                const uint32_t P = (uint32_t)(lane + 64 * k), slot = __umulhi(P, p.cps_magic);
                const uint32_t c16 = 16u * P - __umul24(slot, 16u * (uint32_t)cps);
                if (slot < 2u * (uint32_t)spw) S.off[k] = slot_off<EPI>(slot, rb32, np_rb) + c16;
            }
        }
    }
    const uint32_t relrb0 = slot_off<EPI>(2 * sid, rb32, np_rb);
    const uint32_t relrb1 = slot_off<EPI>(2 * sid + 1, rb32, np_rb);
    const int nkc = (p.units + seg * upl - 1) / (seg * upl);    // K-chunks per row
    const int64_t wave_stride = (int64_t)gridDim.x * wpb * spw;
    const int64_t pw0 = ((int64_t)blockIdx.x * wpb + wave) * spw;
    // address of chunk kc in the first row of the group starting at pair pw
    auto chunk_addr = [&](int64_t pw, int kc) {
        return W + (EPI == EPI_SWIGLU ? pw : 2 * pw) * rb + (int64_t)kc * bpc * BB;
    };

    // Prologue: the activation loads of the first batch go out first, then the
    // first weight item, so the quantization below runs while the weights are
    // in flight (waiting only for the activation loads, which are older).
    using ActS = ActStage<NC, T == T_Q6_K>;
    ActS AS;
    const int K = (int)p.K, nb = K / QK8_1, total = ncols * nb;
    AS.init(p.nb_magic);
    const int gstep = (int)(blockDim.x / ActS::LPB);            // lane groups of the block
    const bool first = pw0 < p.npairs;
    if (p.act_dma) {
        // raw activation rows -> LDS by the same DMA path (older than the weight
        // copy, so waiting for all but the weight instructions covers them)
        const uint32_t rowb = p.xsrc == DT_Q8_1 ? nb * Q8_1_BYTES : K * (p.xsrc == DT_F32 ? 4 : 2);
        const uint32_t ppc = rowb / 16, pieces = ncols * ppc;
        const uint8_t *xb = p.xsrc == DT_Q8_1 ? p.q8 : static_cast<const uint8_t *>(p.x);
        struct { const void *q; uint32_t range; uint32_t cfg; } r = {xb, (uint32_t)p.x_bytes, 0x00020000u};
        v4i rsrc = __builtin_bit_cast(v4i, r);
#pragma unroll
        for (int i = 0; i < 4; i++) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
        if (!early) {
            for (uint32_t j0 = (uint32_t)wave * 64; j0 < pieces; j0 += (uint32_t)wpb * 64) {
                const uint32_t j = j0 + lane, c = __umulhi(j, p.ppc_magic);
                const uint32_t voff = j < pieces ? xoff[c] + 16u * (j - __umul24(c, ppc)) : STAGE_UNUSED;
                llvm_amdgcn_raw_buffer_load_lds(rsrc, (AS3 uint32_t *)(raw + j0 * 16), 16, (int)voff, 0, 0, 0);
            }
            if (first) stage_issue(chunk_addr(pw0, 0), wend, wbuf, S, ninst);
        }
        wait_vm_n(first ? ninst : 0);
        lds_barrier();                                          // every wave's share has landed
    }
    // The quantization, compiled once per source type (a branch per element
    // otherwise): from the LDS copies, or from global memory.
    auto quantize = [&](auto xs) {
        constexpr int XS = decltype(xs)::value;
        const int b0 = (int)(threadIdx.x / ActS::LPB);
        if (p.act_dma) {
            if (ActS::LPB > 1 && total > gstep) {
                // several blocks per lane group of 2 or 4 lanes (long rows): two per
                // trip, so that the two blocks' dependency chains overlap (a lane with a
                // whole block has 32 independent values already).  The second index is
                // clamped to the last block: a duplicate writes the same values as its
                // owner.
#pragma unroll 1
                for (int b = b0; b < total; b += 2 * gstep) {
                    const int b2 = min(b + gstep, total - 1);
                    typename ActS::Raw r1, r2;
                    AS.template fetch_lds<XS>(raw, K, nb, b, r1);
                    AS.template fetch_lds<XS>(raw, K, nb, b2, r2);
                    AS.template put<XS>(lds, K, nb, b, r1);
                    AS.template put<XS>(lds, K, nb, b2, r2);
                }
            } else if (total > gstep) {
#pragma unroll 1
                for (int b = b0; b < total; b += gstep) {
                    typename ActS::Raw r1;
                    AS.template fetch_lds<XS>(raw, K, nb, b, r1);
                    AS.template put<XS>(lds, K, nb, b, r1);
                }
            } else if (b0 < total) {
                typename ActS::Raw r1;
                AS.template fetch_lds<XS>(raw, K, nb, b0, r1);
                AS.template put<XS>(lds, K, nb, b0, r1);
            }
        } else {
            // the first block of every lane group is loaded ahead of the weight copy
            typename ActS::Raw r1;
            AS.template fetch<XS>(p, xrow, nb, min(b0, total - 1), r1);
            if (first) stage_issue<true>(chunk_addr(pw0, 0), wend, wbuf, S, ninst, sink);
            else stage_issue<true>(chunk_addr(0, 0), wend, wbuf, S, 0, sink);
            if (b0 < total) AS.template put<XS>(lds, K, nb, b0, r1);
#pragma unroll 1
            for (int b = b0 + gstep; b < total; b += gstep) {      // larger column groups: further blocks
                AS.template fetch<XS>(p, xrow, nb, b, r1);
                AS.template put<XS>(lds, K, nb, b, r1);
            }
        }
    };
    switch (p.xsrc) {
    case DT_F32: quantize(std::integral_constant<int, DT_F32>{}); break;
    case DT_F16: quantize(std::integral_constant<int, DT_F16>{}); break;
    case DT_Q8_1: quantize(std::integral_constant<int, DT_Q8_1>{}); break;
    default: quantize(std::integral_constant<int, DT_BF16>{}); break;
    }
    lds_barrier();                                              // planar activations complete
    ActL A;
    A.K = K;
    A.nb = nb;
    A.qa = (lds_bp)lds;
    A.d8 = A.qa + NC * A.K;
    A.s8 = A.d8 + NC * A.nb * 4;
    A.h16 = A.s8 + NC * A.nb * 4;

    float acc[2][NC];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int c = 0; c < NC; c++) acc[i][c] = 0.0f;

    const bool patch = (reinterpret_cast<uintptr_t>(wend) & 2) != 0;
    if constexpr (DEEP) {
        // row pair complete: reduce across the segment, store, and clear (the
        // one-ahead loop below keeps its own inline copy of these stores:
        // routing it through this lambda changes that loop's code, and the
        // short launches it serves start with a cold instruction cache)
        auto finish_pair = [&](bool pvalid, bool v1, int64_t r0, int64_t r1) {
            seg_sum(acc, seg);
            if (pvalid && lane_in == seg - 1) {          // seg_sum leaves the total in the segment's last lane
                int64_t cix[NC];                              // all column / route indices in one LDS round trip
#pragma unroll
                for (int c = 0; c < NC; c++) cix[c] = MOE ? (int64_t)route_s[c] : xrow[c];
                store_pair<NC, MOE, EPI, YDT>(p, acc, cix, ncols, v1, r0, r1);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int c = 0; c < NC; c++) acc[i][c] = 0.0f;
        };
        // Two items in flight: item i is computed from buffer i & 1 while item
        // i+1 lands in the other; right after item i is consumed, item i+2 goes
        // into its buffer.  Item 1 goes out now that the second buffers no
        // longer hold the raw activation rows; (ipw, ikc) is the next item to copy.
        auto next_item = [&](int64_t &w, int &k) {
            if (++k == nkc) { k = 0; w += wave_stride; }
        };
        int64_t ipw = pw0;
        int ikc = 0;
        next_item(ipw, ikc);
        bool ahead = false;                                     // item i+1 issued
        if (first && ipw < p.npairs) {
            stage_issue(chunk_addr(ipw, ikc), wend, wbuf + bstride, S, ninst);
            next_item(ipw, ikc);
            ahead = true;
        }
        int64_t pw = pw0;
        int kc = 0, cur = 0;
        while (pw < p.npairs) {                                 // wave-uniform
            const int64_t pair = pw + sid;
            const bool pvalid = pair < p.npairs;
            int64_t r0, r1;
            if (EPI == EPI_SWIGLU) { r0 = pair; r1 = pair + p.Np; }
            else { r0 = 2 * pair; r1 = 2 * pair + 1; }
            const bool v1 = pvalid && r1 < p.N;
            const uint8_t *Acur = chunk_addr(pw, kc);
            // item (pw, kc) has landed; the ninst copy instructions of the next one
            // (issued after it, and after any output stores) may still be in flight
            if (ahead) wait_vm_n(ninst);
            else wait_vm();
            if (patch) stage_patch(Acur, wend, wbuf + cur * bstride, S, ninst, lane);
            compiler_fence();
            if (pvalid) {
                const uint32_t phi = (uint32_t)(reinterpret_cast<uintptr_t>(Acur) & 15);
                const uint8_t *b = wbuf + cur * bstride;
                const int back = kc * bpc * BB;
                const lds_bp row0 = (lds_bp)(b + 2 * sid * cps * 16 + ((phi + relrb0) & 15)) - back;
                const lds_bp row1 = (lds_bp)(b + (2 * sid + 1) * cps * 16 + ((phi + relrb1) & 15)) - back;
                const int ubase = kc * seg * upl + lane_in;
                for (int j = 0; j < upl; j++) {
                    const int u = ubase + j * seg;
                    if (u < p.units) U::run(u, row0, row1, A, ncols, acc);
                }
            }
            wait_lgkm();                                        // LDS reads done before this buffer is refilled
            compiler_fence();
            if (kc + 1 == nkc) finish_pair(pvalid, v1, r0, r1);
            compiler_fence();
            ahead = ipw < p.npairs;                             // the item after next into the buffer just consumed
            if (ahead) {
                stage_issue(chunk_addr(ipw, ikc), wend, wbuf + cur * bstride, S, ninst);
                next_item(ipw, ikc);
            }
            cur ^= 1;
            next_item(pw, kc);
        }
        return;
    }
    int64_t pw = pw0;
    int kc = 0, cur = 0;
    while (pw < p.npairs) {                                     // wave-uniform
        const int64_t pair = pw + sid;
        const bool pvalid = pair < p.npairs;
        int64_t r0, r1;
        if (EPI == EPI_SWIGLU) { r0 = pair; r1 = pair + p.Np; }
        else { r0 = 2 * pair; r1 = 2 * pair + 1; }
        const bool v1 = pvalid && r1 < p.N;
        const uint8_t *Acur = chunk_addr(pw, kc);

        wait_vm();                                              // item (pw, kc) has landed
        if (patch) stage_patch(Acur, wend, wbuf + cur * bstride, S, ninst, lane);
        compiler_fence();
        // next item into the other buffer (its previous contents were consumed last iteration)
        int64_t npw = pw;
        int nkc_next = kc + 1;
        if (nkc_next == nkc) { nkc_next = 0; npw = pw + wave_stride; }
        if (npw < p.npairs) stage_issue(chunk_addr(npw, nkc_next), wend, wbuf + (cur ^ 1) * bstride, S, ninst);

        // this lane's units of the chunk, for both rows of its pair
        if (pvalid) {
            const uint32_t phi = (uint32_t)(reinterpret_cast<uintptr_t>(Acur) & 15);
            const uint8_t *b = wbuf + cur * bstride;
            // slot data sits at ((phi + rel*rb) & 15); shift back by the chunk's first
            // block so the unit index addresses whole rows
            const int back = kc * bpc * BB;
            const lds_bp row0 = (lds_bp)(b + 2 * sid * cps * 16 + ((phi + relrb0) & 15)) - back;
            const lds_bp row1 = (lds_bp)(b + (2 * sid + 1) * cps * 16 + ((phi + relrb1) & 15)) - back;
            const int ubase = kc * seg * upl + lane_in;
            for (int j = 0; j < upl; j++) {
                const int u = ubase + j * seg;
                if (u < p.units) U::run(u, row0, row1, A, ncols, acc);
            }
        }
        wait_lgkm();                                            // LDS reads done before this buffer is refilled
        compiler_fence();
        cur ^= 1;

        if (++kc < nkc) continue;
        // ---- row pair complete: reduce across the segment and store ----
        kc = 0;
        pw += wave_stride;
        seg_sum(acc, seg);
        if (pvalid && lane_in == seg - 1) {          // seg_sum leaves the total in the segment's last lane
            int64_t cix[NC];                              // all column / route indices in one LDS round trip
#pragma unroll
            for (int c = 0; c < NC; c++) cix[c] = MOE ? (int64_t)route_s[c] : xrow[c];
            store_pair<NC, MOE, EPI, YDT>(p, acc, cix, ncols, v1, r0, r1);
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int c = 0; c < NC; c++) acc[i][c] = 0.0f;
    }
}

// ---- test hook: per-group int32 dots through the same decode helpers + dot4 ----
// One thread per (m, n, group), reading the blocks straight from global memory.
template <int T>
__global__ __launch_bounds__(256) void mmvq_dots_kernel(const uint8_t *__restrict__ W, int64_t N, int64_t K,
                                                        const uint8_t *__restrict__ q8, int64_t M,
                                                        int32_t *__restrict__ out) {
    constexpr int G = Geom<T>::G;
    const int64_t gpr = K / G;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= M * N * gpr) return;
    const int64_t j = gid % gpr, n = (gid / gpr) % N, m = gid / (gpr * N);
    const uint8_t *row = W + n * (K / Geom<T>::QK) * Geom<T>::BYTES;
    const uint8_t *arow = q8 + m * (K / QK8_1) * Q8_1_BYTES;
    int D = 0;
    if (T == T_Q4_K) {
        const int sb = (int)(j / 8), jj = (int)(j % 8), p = jj >> 1;
        const uint8_t *blk = row + sb * 144;
        const uint8_t *a = arow + (int64_t)(sb * 8 + jj) * Q8_1_BYTES;
        for (int h = 0; h < 2; h++) {
            const v4i qs = ld16_a2(blk + 16 + 32 * p + 16 * h);
            const v4i qa = ld16_a2(a + 8 + 16 * h);
            for (int w = 0; w < 4; w++) D = dot4((jj & 1) ? nib_hi(qs[w]) : nib_lo(qs[w]), qa[w], D);
        }
    } else if (T == T_Q5_K) {
        const int sb = (int)(j / 8), jj = (int)(j % 8), p = jj >> 1;
        const uint8_t *blk = row + sb * 176;
        const uint8_t *a = arow + (int64_t)(sb * 8 + jj) * Q8_1_BYTES;
        for (int h = 0; h < 2; h++) {
            const v4i qs = ld16_a2(blk + 48 + 32 * p + 16 * h);
            const v4i qh = ld16_a2(blk + 16 + 16 * h);
            const v4i qa = ld16_a2(a + 8 + 16 * h);
            for (int w = 0; w < 4; w++)
                D = dot4(((jj & 1) ? nib_hi(qs[w]) : nib_lo(qs[w])) | q5k_bit((uint32_t)qh[w], jj), qa[w], D);
        }
    } else if (T == T_Q4_0) {
        const uint8_t *blk = row + j * 18;
        const uint8_t *a = arow + j * Q8_1_BYTES;
        const v4i q = ld16_a2(blk + 2);
        const v4i a0 = ld16_a2(a + 8), a1 = ld16_a2(a + 24);
        int asum = 0;
        for (int w = 0; w < 4; w++) {
            asum = dot4(a0[w], 0x01010101, dot4(a1[w], 0x01010101, asum));
            D = dot4(nib_lo(q[w]), a0[w], D);
            D = dot4(nib_hi(q[w]), a1[w], D);
        }
        D -= 8 * asum;
    } else if (T == T_Q6_K) {
        const int sb = (int)(j / 16), jj = (int)(j % 16);          // 16-weight group
        const int hh = jj / 8, g = (jj % 8) / 2, t = jj & 1;
        const uint8_t *blk = row + sb * 210;
        const v4i ql = ld16_a2(blk + 64 * hh + 32 * (g & 1) + 16 * t);
        const v4i qh = ld16_a2(blk + 128 + 32 * hh + 16 * t);
        const v4i qa = ld16_a2(arow + (int64_t)(sb * 8 + 4 * hh + g) * Q8_1_BYTES + 8 + 16 * t);
        int asum = 0;
        for (int w = 0; w < 4; w++) asum = dot4(qa[w], 0x01010101, asum);
        D = -32 * asum;
        for (int w = 0; w < 4; w++) D = dot4(q6k_raw((uint32_t)ql[w], (uint32_t)qh[w], g), qa[w], D);
    } else {
        const uint8_t *blk = row + j * 34;
        const uint8_t *a = arow + j * Q8_1_BYTES;
        const v4i q0 = ld16_a2(blk + 2), q1 = ld16_a2(blk + 18);
        const v4i a0 = ld16_a2(a + 8), a1 = ld16_a2(a + 24);
        for (int w = 0; w < 4; w++) {
            D = dot4(q0[w], a0[w], D);
            D = dot4(q1[w], a1[w], D);
        }
    }
    out[gid] = D;
}

// ---------------------------------------------------------------------------
template <class K>
static void raise_lds_limit(K kernel, size_t lds) {
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
}

template <int T, int NC, bool MOE, int EPI, int YDT, bool DEEP = false>
static void launch_one(const MmvqParams &p, dim3 g, int waves, size_t lds, hipStream_t s) {
    auto k = mmvq_kernel<T, NC, MOE, EPI, YDT, DEEP>;
    raise_lds_limit(k, lds);
    hipLaunchKernelGGL(k, g, dim3(64 * waves), lds, s, p);
}

template <int T, int NC>
static void launch_deep(bool moe, int epi, int ydt, const MmvqParams &p, dim3 g, int waves, size_t lds, hipStream_t s) {
    if (!moe) {
        if (ydt == DT_F32) launch_one<T, NC, false, EPI_NONE, DT_F32, true>(p, g, waves, lds, s);
        else launch_one<T, NC, false, EPI_NONE, DT_BF16, true>(p, g, waves, lds, s);
    } else if (epi == EPI_SWIGLU) {
        if (ydt == DT_F32) launch_one<T, NC, true, EPI_SWIGLU, DT_F32, true>(p, g, waves, lds, s);
        else launch_one<T, NC, true, EPI_SWIGLU, DT_BF16, true>(p, g, waves, lds, s);
    } else {
        if (ydt == DT_F32) launch_one<T, NC, true, EPI_NONE, DT_F32, true>(p, g, waves, lds, s);
        else launch_one<T, NC, true, EPI_NONE, DT_BF16, true>(p, g, waves, lds, s);
    }
}

template <int T, int NC>
static void launch_nc(bool moe, int epi, int ydt, const MmvqParams &p, dim3 g, int waves, size_t lds, hipStream_t s) {
    if constexpr (NC <= 2) {
        if (p.deep) {
            launch_deep<T, NC>(moe, epi, ydt, p, g, waves, lds, s);
            return;
        }
    }
    if (!moe) {
        if (ydt == DT_F32) launch_one<T, NC, false, EPI_NONE, DT_F32>(p, g, waves, lds, s);
        else launch_one<T, NC, false, EPI_NONE, DT_BF16>(p, g, waves, lds, s);
    } else if (epi == EPI_SWIGLU) {
        if (ydt == DT_F32) launch_one<T, NC, true, EPI_SWIGLU, DT_F32>(p, g, waves, lds, s);
        else launch_one<T, NC, true, EPI_SWIGLU, DT_BF16>(p, g, waves, lds, s);
    } else {
        if (ydt == DT_F32) launch_one<T, NC, true, EPI_NONE, DT_F32>(p, g, waves, lds, s);
        else launch_one<T, NC, true, EPI_NONE, DT_BF16>(p, g, waves, lds, s);
    }
}

template <int T>
static void launch_t(int nc, bool moe, int epi, int ydt, const MmvqParams &p, dim3 g, int waves, size_t lds,
                     hipStream_t s) {
    switch (nc) {
    case 1: launch_nc<T, 1>(moe, epi, ydt, p, g, waves, lds, s); break;
    case 2: launch_nc<T, 2>(moe, epi, ydt, p, g, waves, lds, s); break;
    case 4: launch_nc<T, 4>(moe, epi, ydt, p, g, waves, lds, s); break;
    default: launch_nc<T, 8>(moe, epi, ydt, p, g, waves, lds, s); break;
    }
}

// LDS bytes of nc planar activation rows of length K.
static size_t act_lds(int t, int nc, int64_t K) {
    const size_t per = (size_t)K + (size_t)(K / QK8_1) * (t == T_Q6_K ? 16 : 8);
    return ((size_t)nc * per + 15) & ~size_t(15);
}

int mmvq_max_cols(int t, int64_t K) {
    for (int nc = 8; nc > 1; nc >>= 1)
        if (act_lds(t, nc, K) <= MMVQ_LDS_MAX) return nc;
    return 1;
}

// Work item geometry: units per row, lanes per row segment, units per lane,
// blocks per chunk, 16-byte pieces per staged row chunk, DMA instructions.
struct ItemGeo {
    int units, seg, upl, bpc, cps, ninst;
};

static ItemGeo item_geo(int t, int64_t K) {
    const int upb = (t == T_Q8_0 || t == T_Q4_0) ? 1 : 4;        // units per block
    const double ub = (double)block_bytes(t) / upb;                // bytes per unit
    ItemGeo G{};
    G.units = (int)(K / block_len(t)) * upb;
    auto bytes = [&](int seg, int upl) { return (128.0 / seg) * std::min<double>(G.units, (double)seg * upl) * ub; };
    int seg = 1;
    while (seg < G.units && seg < 64) seg <<= 1;
    int upl = 1;
    // more units per lane while a row does not fit one chunk and the item stays small
    while ((int64_t)seg * upl < G.units && upl < 4 && bytes(seg, upl + 1) <= 9216) upl++;
    // small items: fewer lanes per row, more rows per item
    while (seg > 4 && upl * 2 <= 4 && bytes(seg, upl) < 4096 && bytes(seg / 2, upl * 2) <= 9216) {
        seg >>= 1;
        upl <<= 1;
    }
    G.seg = seg;
    G.upl = upl;
    G.bpc = std::min(G.units, seg * upl) / upb;
    G.cps = (int)((G.bpc * block_bytes(t) + 15 + 15) / 16);       // pieces covering a chunk at any phase
    G.ninst = (2 * (64 / seg) * G.cps + 63) / 64;
    return G;
}

bool mmvq_supported(int t, int64_t K) {
    return K > 0 && K <= INT32_MAX / 16 && act_lds(t, 1, K) <= MMVQ_LDS_MAX && item_geo(t, K).ninst <= MMVQ_MAXI;
}

hipError_t launch_mmvq(int t, int nc, bool moe, int epi, int ydt, const MmvqParams &p0, int64_t ngroups_bound,
                       hipStream_t s) {
    MmvqParams p = p0;
    if (p.npairs == 0 || ngroups_bound == 0) return hipSuccess;
    const size_t act = act_lds(t, nc, p.K);
    if (act > MMVQ_LDS_MAX || p.K > INT32_MAX / 16) return hipErrorInvalidValue;
    const ItemGeo G = item_geo(t, p.K);
    if (G.ninst > MMVQ_MAXI) return hipErrorInvalidValue;
    p.units = G.units;
    p.seg = G.seg;
    p.upl = G.upl;
    p.stage_bpc = G.bpc;
    p.stage_cps = G.cps;
    p.stage_ninst = G.ninst;
    p.cps_magic = (uint32_t)((((uint64_t)1 << 32) + G.cps - 1) / G.cps);
    p.nb_magic = (uint32_t)((((uint64_t)1 << 32) + p.K / QK8_1 - 1) / (p.K / QK8_1));
    if (p.row_bytes >= (int64_t(1) << 24)) return hipErrorInvalidValue;
    p.act_lds_bytes = (int64_t)act;
    const int spw = 64 / G.seg;
    // staging offsets are 32-bit from the first row of an item
    if ((epi == EPI_SWIGLU ? p.Np + spw : 2 * spw) * p.row_bytes + G.cps * 16 >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    // Waves per block: as many as LDS (two item buffers per wave) and registers
    // allow, so that one resident block per CU quantizes the activations once
    // for all its waves; fewer when the row groups would not fill them.
    const size_t per_wave = 2 * (size_t)G.ninst * 1024;
    const size_t lds_cap = 160 * 1024 - 256;                    // room for the static LDS of the kernel
    const int max_waves = nc <= 2 ? MaxWaves<1>::value : nc == 4 ? MaxWaves<4>::value : MaxWaves<8>::value;
    if (act + per_wave + 1024 > lds_cap) return hipErrorInvalidValue;
    int waves = (int)std::min<size_t>((size_t)max_waves, (lds_cap - act - 1024) / per_wave);
    const int64_t groups = (p.npairs + spw - 1) / spw;          // row groups (one wave's worth per K-chunk)
    const int64_t fill = (groups + 255) / 256;                   // waves per block to give every CU one block
    if (fill < waves) waves = (int)std::max<int64_t>(fill, std::min<int64_t>(waves, 4));
    // Raw activation rows through LDS when every row starts 16-byte aligned at a
    // 32-bit offset and they fit the region after the first item buffers: the
    // waves' second buffers, extended when the rows need more and LDS allows.
    const size_t bufs = (size_t)waves * G.ninst * 1024;          // one buffer per wave
    size_t region = bufs;
    {
        const int64_t nb = p.K / QK8_1;
        const int64_t rowb = p.xsrc == DT_Q8_1 ? nb * Q8_1_BYTES : p.K * (p.xsrc == DT_F32 ? 4 : 2);
        const int64_t stride = p.xsrc == DT_Q8_1 ? p.q8_row : p.ldx * (p.xsrc == DT_F32 ? 4 : 2);
        const size_t raw_need = ((size_t)nc * (size_t)rowb + 1023) & ~size_t(1023);
        p.act_dma = rowb % 16 == 0 && stride % 16 == 0 && act + bufs + std::max(bufs, raw_need) + 1024 <= lds_cap &&
                    p.x_bytes > 0 && p.x_bytes < 0x7fffff00LL;
        if (p.act_dma) region = std::max(bufs, raw_need);
        p.x_stride = stride;
        p.ppc_magic = p.act_dma ? (uint32_t)((((uint64_t)1 << 32) + rowb / 16 - 1) / (rowb / 16)) : 0u;
    }
    p.raw_region = (uint32_t)region;
    const size_t lds = act + bufs + region + 1024;              // + the prologue's 1 KB sink
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(8, (int64_t)lds_cap / (int64_t)lds));
    const int64_t need = (groups + waves - 1) / waves;
    // routed: about min(E, routes) groups are active, whatever the host-side bound;
    // spread one wave of workgroups over them (more only adds prologues: measured)
    const int64_t active = moe ? std::max<int64_t>(1, std::min<int64_t>(ngroups_bound, p.groups_expected)) : ngroups_bound;
    const int64_t cap = std::max<int64_t>(1, 256 * per_cu / active);
    const dim3 g((unsigned)std::min<int64_t>(need, cap), (unsigned)ngroups_bound);
    // One- and two-column calls where a wave walks several items (lm_head-sized
    // matrices; routed decode, per expert) keep two items in flight per wave
    // (a separate instantiation: the extra code would slow the short launches,
    // whose instruction cache starts cold).
    const int64_t nkc = (G.units + G.seg * G.upl - 1) / (G.seg * G.upl);
    p.deep = nc <= 2 && groups * nkc >= 4 * (int64_t)g.x * waves;
    if (t == T_Q4_K) launch_t<T_Q4_K>(nc, moe, epi, ydt, p, g, waves, lds, s);
    else if (t == T_Q6_K) launch_t<T_Q6_K>(nc, moe, epi, ydt, p, g, waves, lds, s);
    else if (t == T_Q5_K) launch_t<T_Q5_K>(nc, moe, epi, ydt, p, g, waves, lds, s);
    else if (t == T_Q4_0) launch_t<T_Q4_0>(nc, moe, epi, ydt, p, g, waves, lds, s);
    else launch_t<T_Q8_0>(nc, moe, epi, ydt, p, g, waves, lds, s);
    return hipGetLastError();
}

hipError_t launch_mmvq_dots(int t, const uint8_t *W, int64_t N, int64_t K, const uint8_t *q8, int64_t M,
                            int32_t *out, hipStream_t s) {
    const int64_t n = M * N * (K / group_len(t));
    if (n == 0) return hipSuccess;
    dim3 g((unsigned)((n + 255) / 256));
    if (t == T_Q4_K) hipLaunchKernelGGL(mmvq_dots_kernel<T_Q4_K>, g, dim3(256), 0, s, W, N, K, q8, M, out);
    else if (t == T_Q6_K) hipLaunchKernelGGL(mmvq_dots_kernel<T_Q6_K>, g, dim3(256), 0, s, W, N, K, q8, M, out);
    else if (t == T_Q5_K) hipLaunchKernelGGL(mmvq_dots_kernel<T_Q5_K>, g, dim3(256), 0, s, W, N, K, q8, M, out);
    else if (t == T_Q4_0) hipLaunchKernelGGL(mmvq_dots_kernel<T_Q4_0>, g, dim3(256), 0, s, W, N, K, q8, M, out);
    else hipLaunchKernelGGL(mmvq_dots_kernel<T_Q8_0>, g, dim3(256), 0, s, W, N, K, q8, M, out);
    return hipGetLastError();
}

}  // namespace ggq
