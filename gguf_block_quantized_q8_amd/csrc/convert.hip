// q8_1 quantization of activations, dequantization of weight blocks, and the
// small fill / finalize kernels used around the matmuls.
#include "kernels.hpp"

namespace ggq {

// ---------------------------------------------------------------------------
// q8_1: 8 lanes per 32-value block, 4 values per lane.
//   d = amax / 127 (IEEE fp32 division), q = roundf(x / d) (half away from
//   zero), all-zero block -> d = s = 0, s = d * (float)sum(q).
// Output either 40-byte blocks (q8 != nullptr) and/or the MMQ operand
// (xq != nullptr; K % 256 == 0): fp16 quants xq, d xd, and the min-term operand
// xm (each block's s split exactly into three parts, planar_write_min), row-major
// or tiled (xq_index).
// ---------------------------------------------------------------------------
template <int XDT, bool VEC>
__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const void *__restrict__ x, int64_t M, int64_t K,
                                                            int64_t ldx, uint8_t *__restrict__ q8,
                                                            _Float16 *__restrict__ xq, float *__restrict__ xd,
                                                            uint16_t *__restrict__ xm, bool tiled) {
    const int64_t nb = K / QK8_1;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = gid >> 3;            // block index over M * nb
    const int sub = threadIdx.x & 7;
    const bool valid = b < M * nb;
    const int64_t m = valid ? b / nb : 0;
    const int64_t blk = valid ? b - m * nb : 0;
    const int64_t e0 = m * ldx + blk * QK8_1 + sub * 4;

    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
        if (XDT == DT_F32) {
            const float *xf = static_cast<const float *>(x) + e0;
            if (VEC) {
                v4f t = *reinterpret_cast<const v4f *>(xf);
                v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
            } else {
                for (int i = 0; i < 4; i++) v[i] = xf[i];
            }
        } else {                           // bf16 or fp16
            const bool h = XDT == DT_F16;
            const uint16_t *xb = static_cast<const uint16_t *>(x) + e0;
            if (VEC) {
                v2i t = *reinterpret_cast<const v2i *>(xb);
                v[0] = from_16((uint32_t)t.x & 0xffffu, h);
                v[1] = from_16((uint32_t)t.x >> 16, h);
                v[2] = from_16((uint32_t)t.y & 0xffffu, h);
                v[3] = from_16((uint32_t)t.y >> 16, h);
            } else {
                for (int i = 0; i < 4; i++) v[i] = from_16(xb[i], h);
            }
        }
    }
    const float amax = max8(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    float d = amax / 127.0f;
    int q[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        q[i] = q8_1_quant(v[i], d, amax);
        sum += q[i];
    }
    sum = sum8(sum);
    if (amax == 0.0f) d = 0.0f;
    const float s = d * (float)sum;
    if (!valid) return;
    if (q8) {
        uint8_t *out = q8 + b * Q8_1_BYTES;
        uint32_t packed = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                          ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
        reinterpret_cast<uint32_t *>(out + 8)[sub] = packed;
        if (sub == 0) *reinterpret_cast<float2 *>(out) = make_float2(d, s);
    }
    if (xq) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        h4 hv = {(_Float16)q[0], (_Float16)q[1], (_Float16)q[2], (_Float16)q[3]};
        *reinterpret_cast<h4 *>(xq + xq_index(tiled, m, K, blk * QK8_1 + sub * 4)) = hv;
        if (sub == 0) {
            xd[xd_index(tiled, m, nb, blk)] = d;
            planar_write_min(xm, tiled, m, K, blk, s);
        }
    }
}

// Wide variants for rows that allow 16-byte loads (ldx a multiple of VPL, a
// 16-byte aligned base): LPB = 4 or 2 lanes per 32-value block, VPL = 32 / LPB
// values per lane.  The same arithmetic, value by value, as
// quantize_q8_1_kernel (block amax by DPP over the block's lanes, IEEE
// division, half-away rounding, exact integer sum): identical bits, more bytes
// per lane, fewer lanes.
template <int XDT, int LPB>
__global__ __launch_bounds__(256) void quantize_q8_1_wide_kernel(const void *__restrict__ x, int64_t M, int64_t K,
                                                                 int64_t ldx, uint8_t *__restrict__ q8,
                                                                 _Float16 *__restrict__ xq, float *__restrict__ xd,
                                                                 uint16_t *__restrict__ xm, bool tiled) {
    constexpr int VPL = QK8_1 / LPB;
    const int64_t nb = K / QK8_1;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = gid / LPB;           // block index over M * nb; LPB aligned lanes are one block
    const int sub = threadIdx.x & (LPB - 1);
    const bool valid = b < M * nb;
    const int64_t m = valid ? b / nb : 0;
    const int64_t blk = valid ? b - m * nb : 0;
    const int64_t e0 = m * ldx + blk * QK8_1 + sub * VPL;

    float v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; i++) v[i] = 0.0f;
    if (valid) {
        if (XDT == DT_F32) {
            const float *xf = static_cast<const float *>(x) + e0;
#pragma unroll
            for (int c = 0; c < VPL / 4; c++) {
                const v4f t = *reinterpret_cast<const v4f *>(xf + 4 * c);
                v[4 * c] = t.x; v[4 * c + 1] = t.y; v[4 * c + 2] = t.z; v[4 * c + 3] = t.w;
            }
        } else {                           // bf16 or fp16
            const bool h = XDT == DT_F16;
            const uint16_t *xb = static_cast<const uint16_t *>(x) + e0;
#pragma unroll
            for (int c = 0; c < VPL / 8; c++) {
                const v4i t = *reinterpret_cast<const v4i *>(xb + 8 * c);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    v[8 * c + 2 * i] = from_16((uint32_t)t[i] & 0xffffu, h);
                    v[8 * c + 2 * i + 1] = from_16((uint32_t)t[i] >> 16, h);
                }
            }
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; i++) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, dpp_f<DPP_XOR1>(amax));
    if (LPB == 4) amax = fmaxf(amax, dpp_f<DPP_XOR2>(amax));
    float d = amax / 127.0f;
    int q[VPL];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        q[i] = q8_1_quant(v[i], d, amax);
        sum += q[i];
    }
    sum += dpp_i<DPP_XOR1>(sum);
    if (LPB == 4) sum += dpp_i<DPP_XOR2>(sum);
    if (amax == 0.0f) d = 0.0f;
    const float s = d * (float)sum;
    if (!valid) return;
    if (q8) {
        uint8_t *out = q8 + b * Q8_1_BYTES + 8 + VPL * sub;
#pragma unroll
        for (int c = 0; c < VPL / 8; c++) {
            uint32_t w[2];
#pragma unroll
            for (int k = 0; k < 2; k++)
                w[k] = (uint32_t)(q[8 * c + 4 * k] & 0xff) | ((uint32_t)(q[8 * c + 4 * k + 1] & 0xff) << 8) |
                       ((uint32_t)(q[8 * c + 4 * k + 2] & 0xff) << 16) | ((uint32_t)(q[8 * c + 4 * k + 3] & 0xff) << 24);
            *reinterpret_cast<v2i *>(out + 8 * c) = v2i{(int)w[0], (int)w[1]};
        }
        if (sub == 0) *reinterpret_cast<float2 *>(q8 + b * Q8_1_BYTES) = make_float2(d, s);
    }
    if (xq) {
#pragma unroll
        for (int c = 0; c < VPL / 8; c++) {
            v8h hv;
#pragma unroll
            for (int i = 0; i < 8; i++) hv[i] = (_Float16)q[8 * c + i];
            *reinterpret_cast<v8h *>(xq + xq_index(tiled, m, K, blk * QK8_1 + sub * VPL + 8 * c)) = hv;
        }
        if (sub == 0) {
            xd[xd_index(tiled, m, nb, blk)] = d;
            planar_write_min(xm, tiled, m, K, blk, s);
        }
    }
}

// q8_1 blocks -> MMQ operand (for pre-quantized input).
__global__ __launch_bounds__(256) void q8_1_to_planar_kernel(const uint8_t *__restrict__ q8, int64_t M, int64_t K,
                                                             _Float16 *__restrict__ xq, float *__restrict__ xd,
                                                             uint16_t *__restrict__ xm, bool tiled) {
    const int64_t nb = K / QK8_1;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = gid >> 3;
    const int sub = threadIdx.x & 7;
    if (b >= M * nb) return;
    const uint8_t *in = q8 + b * Q8_1_BYTES;
    uint32_t w = reinterpret_cast<const uint32_t *>(in + 8)[sub];
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 hv = {(_Float16)(int8_t)(w & 0xff), (_Float16)(int8_t)((w >> 8) & 0xff),
             (_Float16)(int8_t)((w >> 16) & 0xff), (_Float16)(int8_t)(w >> 24)};
    const int64_t m = b / nb, blk = b - m * nb;
    *reinterpret_cast<h4 *>(xq + xq_index(tiled, m, K, blk * QK8_1 + sub * 4)) = hv;
    if (sub == 0) {
        float2 ds = *reinterpret_cast<const float2 *>(in);
        xd[xd_index(tiled, m, nb, blk)] = ds.x;
        planar_write_min(xm, tiled, m, K, blk, ds.y);
    }
}

// ---------------------------------------------------------------------------
// Dequantize: 16 consecutive weights of an output row at a time.
//   Q8_0: d*q; Q4_0: d*(nib-8); Q4_K / Q5_K: (d*sc)*q - dmin*m; Q6_K: (d*sc)*(q-32).
// Every product is exact in fp32; the subtraction of the min rounds once.
// Output row r (of n) holds table row ids[r] (r itself without ids); a row id
// outside [0, rows) gives a row of zeros.  y rows are ldy elements apart.
// ---------------------------------------------------------------------------

#define AS3 __attribute__((address_space(3)))
typedef const uint8_t AS3 *lds_bp;
extern "C" __device__ v4i llvm_amdgcn_raw_buffer_load_v4i32(v4i rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");

// Bytes of one block, from global memory or from a row staged in LDS.  Block
// sizes and field offsets are even, so every 16-bit field and 16-byte run
// starts 2-byte aligned in both.
struct GlobalBytes {
    const uint8_t *p;
    __device__ uint32_t u8(int o) const { return p[o]; }
    __device__ uint32_t u16(int o) const { return ld_u16(p + o); }
    template <int N> __device__ v4i v(int o) const {
        static_assert(N == 16, "global reads take 16-byte runs");
        return ld16_a2(p + o);
    }
};
struct LdsBytes {
    lds_bp p;
    __device__ uint32_t u8(int o) const { return p[o]; }
    __device__ uint32_t u16(int o) const { return *(const uint16_t AS3 *)(p + o); }   // 2-byte aligned
    // N bytes (4, 8 or 16) at a 2-byte aligned offset: N/4 + 1 aligned dwords
    // shifted into place; words past N/4 are zero.
    template <int N> __device__ v4i v(int o) const {
        const lds_bp q = p + o;
        const uint32_t sh = (uint32_t)(uintptr_t)q & 3u;
        const uint32_t AS3 *w = (const uint32_t AS3 *)(q - sh);
        uint32_t x[N / 4 + 1];
#pragma unroll
        for (int i = 0; i <= N / 4; i++) x[i] = w[i];
        v4i r = v4i{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < N / 4; i++) r[i] = (int)__builtin_amdgcn_alignbyte(x[i + 1], x[i], sh);
        return r;
    }
};

// Weights ib .. ib + N - 1 of the block at B (N = 4, 8 or 16; ib a multiple of
// N below the block length): byte i of a run read at offset o is field byte
// o + i.  Each group of four codes is gathered into the four bytes of a dword,
// then turned into floats byte by byte: Q4_K / Q5_K codes as unsigned values u
// with w = fma(d*sc, u, -dmin*m) (the product is exact, the one rounding is
// that of the min subtraction, as in the block formula); Q4_0 / Q6_K codes
// with their offset (8, 32) taken off in two's complement (flipping the top
// bit of the field) and Q8_0's int8 as they are, sign-extended, then
// w = scale * code, the block formula itself (signed zeros included).
template <int T, int N, class Bytes>
__device__ __forceinline__ void decode(const Bytes &B, int ib, float (&w)[N]) {
    uint32_t x[N / 4];
    float a, b = 0.0f;
    if (T == T_Q4_0) {
        // weights 0..15: low nibbles of the 16 quant bytes, 16..31: high nibbles
        const v4i q = B.template v<N>(2 + ib % 16);
#pragma unroll
        for (int k = 0; k < N / 4; k++)
            x[k] = ((ib >= 16 ? (uint32_t)q[k] >> 4 : (uint32_t)q[k]) & 0x0f0f0f0fu) ^ 0x08080808u;
        a = fp16_bits_to_f32(B.u16(0));
    } else if (T == T_Q4_K || T == T_Q5_K) {
        // Q5_K: the nibble | bit j of the fifth-bit byte << 4
        const float d = fp16_bits_to_f32(B.u16(0)), dmin = fp16_bits_to_f32(B.u16(2));
        const int j = ib / 32;
        int sc, mn;
        if (j < 4) { sc = B.u8(4 + j) & 63; mn = B.u8(8 + j) & 63; }
        else {
            sc = (B.u8(8 + j) & 0x0f) | ((B.u8(j) >> 6) << 4);
            mn = (B.u8(8 + j) >> 4) | ((B.u8(4 + j) >> 6) << 4);
        }
        const int c = ib / 64, l0 = ib % 32;
        const bool hi = (ib % 64) >= 32;
        const v4i q = B.template v<N>((T == T_Q4_K ? 16 : 48) + 32 * c + l0);
        v4i h = v4i{0, 0, 0, 0};
        if (T == T_Q5_K) h = B.template v<N>(16 + l0);
#pragma unroll
        for (int k = 0; k < N / 4; k++) {
            x[k] = (hi ? (uint32_t)q[k] >> 4 : (uint32_t)q[k]) & 0x0f0f0f0fu;
            if (T == T_Q5_K) x[k] |= (((uint32_t)h[k] >> j) & 0x01010101u) << 4;
        }
        a = d * (float)sc; b = -(dmin * (float)mn);
    } else if (T == T_Q8_0) {
        const v4i q = B.template v<N>(2 + ib);
#pragma unroll
        for (int k = 0; k < N / 4; k++) x[k] = (uint32_t)q[k];
        a = fp16_bits_to_f32(B.u16(0));
    } else {
        // 6-bit code = 4 bits of ql | 2 bits of qh << 4, scale d * sc
        const int h = ib / 128, rr = ib % 128, g = rr / 32, l = rr % 32;
        const v4i ql = B.template v<N>(64 * h + 32 * (g & 1) + l);
        const v4i qh = B.template v<N>(128 + 32 * h + l);
#pragma unroll
        for (int k = 0; k < N / 4; k++)
            x[k] = (((g < 2 ? (uint32_t)ql[k] : (uint32_t)ql[k] >> 4) & 0x0f0f0f0fu) |
                    ((((uint32_t)qh[k] >> (2 * g)) & 0x03030303u) << 4)) ^ 0x20202020u;
        a = fp16_bits_to_f32(B.u16(208)) * (float)(int8_t)B.u8(192 + ib / 16);
    }
    constexpr int BITS = T == T_Q8_0 ? 8 : T == T_Q4_0 ? 4 : 6;   // signed field width
#pragma unroll
    for (int i = 0; i < N; i++) {
        if (T == T_Q4_K || T == T_Q5_K)
            w[i] = fmaf(a, (float)((x[i / 4] >> (8 * (i % 4))) & 0xffu), b);
        else
            w[i] = a * (float)((int32_t)(x[i / 4] << (32 - BITS - 8 * (i % 4))) >> (32 - BITS));
    }
}

// Two values as bf16 (v_cvt_pk_bf16_f32, round to nearest even) or fp16 bits.
template <int YDT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if (YDT == DT_BF16) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
    }
    return f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
}

// N converted values (N * size = 16 bytes) as one 16-byte store.
template <int YDT, int N>
__device__ __forceinline__ void store_run(void *y, int64_t o, const float *w) {
    static_assert(N * (YDT == DT_F32 ? 4 : 2) == 16, "one 16-byte store");
    if (YDT == DT_F32) {
        *reinterpret_cast<v4f *>(static_cast<float *>(y) + o) = v4f{w[0], w[1], w[2], w[3]};
    } else {
        v4i t;
#pragma unroll
        for (int k = 0; k < 4; k++) t[k] = (int)pack2<YDT>(w[2 * k], w[2 * k + 1]);
        *reinterpret_cast<v4i *>(static_cast<uint16_t *>(y) + o) = t;
    }
}

template <int YDT>
__device__ __forceinline__ void store16(void *y, int64_t o, const float (&w)[16]) {
    constexpr int S = YDT == DT_F32 ? 4 : 8;
#pragma unroll
    for (int i = 0; i < 16; i += S) store_run<YDT, S>(y, o + i, w + i);
}

// One thread per 16 weights, read from global memory: rows longer than the
// staged kernel's limit.
template <int T, int YDT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ W, int64_t rows, int64_t K,
                                                      const int32_t *__restrict__ ids, int64_t n,
                                                      void *__restrict__ y, int64_t ldy) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_row = K / 16;
    if (gid >= n * per_row) return;
    const int64_t r = gid / per_row;
    const int64_t i0 = (gid - r * per_row) * 16;         // first weight index in the row
    const int64_t src = ids ? (int64_t)ids[r] : r;
    constexpr int QK = Geom<T>::QK, BB = Geom<T>::BYTES;
    float w[16];
    if (src < 0 || src >= rows) {
        for (int i = 0; i < 16; i++) w[i] = 0.0f;
    } else {
        decode<T, 16>(GlobalBytes{W + src * (K / QK) * BB + (i0 / QK) * BB}, (int)(i0 % QK), w);
    }
    store16<YDT>(y, r * ldy + i0, w);
}

// Rows of up to DQ_ROW_MAX bytes: each wave walks output rows r, r + waves, ...
// A row's bytes go to LDS by 16-byte loads from the 16-byte boundary at or
// below its start, NL a lane (a buffer resource over the matrix, so nothing
// past its end is read); the next row's loads are issued before the current
// row is decoded, so they land while the wave decodes and stores.  Each lane
// then decodes 8 bf16 / fp16 or 4 fp32 outputs (16 bytes) a step from LDS:
// every store instruction writes 1 KB of the row.  A wave's LDS slot is `slot`
// bytes (the row rounded up to 16, plus 32 for the phase and the last dword
// read).
constexpr int DQ_ROW_MAX = 8192;
constexpr int DQ_MAX_WG = 2048;          // workgroups (4 waves each) at most

template <int NL> struct RowFetch {
    v4i v[NL];
    int ph;
    bool valid;
};

// Table row src (wave-uniform) into f.
template <int T, int NL>
__device__ __forceinline__ void row_fetch(RowFetch<NL> &f, const uint8_t *W, int64_t wbytes, int64_t rows,
                                          int64_t rb, int64_t src, int lane) {
    f.valid = src >= 0 && src < rows;
    f.ph = 0;
    if (!f.valid) return;
    const int64_t start = src * rb, a0 = start & ~(int64_t)15;
    f.ph = (int)(start - a0);
    const int npc = (int)((f.ph + rb + 15) / 16);
    struct { const void *q; uint32_t range; uint32_t cfg; } rd = {W + a0, (uint32_t)(wbytes - a0), 0x00020000u};
    v4i rsrc = __builtin_bit_cast(v4i, rd);
#pragma unroll
    for (int i = 0; i < 4; i++) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
    const int64_t lim = wbytes - a0;                      // readable bytes from W + a0 (even)
#pragma unroll
    for (int i = 0; i < NL; i++) {
        const int pc = lane + 64 * i;
        if (pc < npc) {                                   // (words past npc are never stored to LDS)
            f.v[i] = llvm_amdgcn_raw_buffer_load_v4i32(rsrc, 16 * pc, 0, 0);
            // The range check zeroes each dword not wholly inside the range: a
            // table whose end is 2 bytes into a dword gets those 2 bytes here.
            const int64_t rem = lim - 16 * pc;
            if (rem < 16 && (rem & 2)) f.v[i][rem >> 2] = (int)ld_u16(W + a0 + 16 * pc + (rem & ~3));
        }
    }
}

template <int T, int YDT, int NL>
__global__ __launch_bounds__(256) void dequant_rows_kernel(const uint8_t *__restrict__ W, int64_t wbytes,
                                                           int64_t rows, int64_t K, const int32_t *__restrict__ ids,
                                                           int64_t n, void *__restrict__ y, int64_t ldy, int slot) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dq_stage[];
    // wave index made uniform so row ids come in by scalar loads
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = (int)(threadIdx.x & 63);
    const int64_t waves = (int64_t)gridDim.x * 4;
    int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= n) return;                                   // wave-uniform; no workgroup barrier below
    constexpr int QK = Geom<T>::QK, BB = Geom<T>::BYTES;
    constexpr int N = YDT == DT_F32 ? 4 : 8;
    const int64_t rb = K / QK * BB;
    uint8_t AS3 *const srow = (uint8_t AS3 *)&dq_stage[wave * slot];
    auto src_of = [&](int64_t rr) -> int64_t { return rr < n ? (ids ? (int64_t)ids[rr] : rr) : -1; };
    RowFetch<NL> f;
    row_fetch<T>(f, W, wbytes, rows, rb, src_of(r), lane);
    int64_t src_next = src_of(r + waves);                 // one row ahead of the fetch
    for (; r < n; r += waves) {
        // Lanes read bytes other lanes wrote and the slot is reused row after
        // row: keep the compiler from moving LDS accesses across these points
        // (a wave's LDS operations complete in order).
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const bool valid = f.valid;
        const lds_bp row = srow + f.ph;
        if (valid) {
#pragma unroll
            for (int i = 0; i < NL; i++)
                if (lane + 64 * i < (f.ph + rb + 15) / 16) *(v4i AS3 *)(srow + 16 * (lane + 64 * i)) = f.v[i];
        }
        if (r + waves < n) {
            row_fetch<T>(f, W, wbytes, rows, rb, src_next, lane);
            src_next = src_of(r + 2 * waves);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // a step covers N * 64 weights, whole blocks: the lane's place in its
        // block is the same every step
        if (valid) {
            int bo = (N * lane) / QK * BB;
            for (int64_t i0 = N * (int64_t)lane; i0 < K; i0 += N * 64, bo += N * 64 / QK * BB) {
                float w[N];
                decode<T, N>(LdsBytes{row + bo}, (N * lane) % QK, w);
                store_run<YDT, N>(y, r * ldy + i0, w);
            }
        } else {
            const float w[N] = {};
            for (int64_t i0 = N * (int64_t)lane; i0 < K; i0 += N * 64) store_run<YDT, N>(y, r * ldy + i0, w);
        }
    }
}

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *__restrict__ p, int64_t n, uint32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t st = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += st) p[i] = v;
}

// Route-weighted sum of per-route outputs o (stored in the output dtype: fp32,
// or the 16-bit type of y, as the activation-dtype intermediates of the pages):
//   y[t][n] = sum over k in ascending order of w[t][k] * o[t*top_k + k][n]
// for the active routes of token t (0 <= id < E), accumulated in fp32, then
// stored in the output dtype.  One thread per V consecutive n (16 bytes of o
// when Np allows it: V = 4 fp32 or 8 16-bit values, else V = 1).  The routes go
// in chunks of 8 whose row loads are all issued before the first fma (one
// memory latency per chunk, not per route); an inactive route's row (never
// written) is skipped, so it cannot feed a NaN into the sum.
template <int YDT, int V>
__device__ __forceinline__ void load_route(const void *o, int64_t idx, float (&v)[V]) {
    if (YDT == DT_F32) {
        const float *of = static_cast<const float *>(o) + idx;
        if (V == 4) {
            const v4f t = *reinterpret_cast<const v4f *>(of);
#pragma unroll
            for (int c = 0; c < V; c++) v[c] = t[c & 3];
        } else {
#pragma unroll
            for (int c = 0; c < V; c++) v[c] = of[c];
        }
    } else {
        const uint16_t *oh = static_cast<const uint16_t *>(o) + idx;
        if (V == 8) {
            const v4i t = *reinterpret_cast<const v4i *>(oh);
#pragma unroll
            for (int c = 0; c < V; c++) v[c] = from_16(((uint32_t)t[(c >> 1) & 3] >> (16 * (c & 1))) & 0xffffu, YDT == DT_F16);
        } else {
#pragma unroll
            for (int c = 0; c < V; c++) v[c] = from_16(oh[c], YDT == DT_F16);
        }
    }
}

template <int YDT, int V>
__global__ __launch_bounds__(256) void route_sum_kernel(const void *__restrict__ o, const int32_t *__restrict__ ids,
                                                        const float *__restrict__ w, int64_t T, int top_k, int64_t E,
                                                        int64_t Np, void *__restrict__ y) {
    constexpr int KC = 8;
    const int64_t q = Np / V;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t st = (int64_t)gridDim.x * blockDim.x;
    for (; i < T * q; i += st) {
        const int64_t t = i / q, n = V * (i - t * q);
        float acc[V];
#pragma unroll
        for (int c = 0; c < V; c++) acc[c] = 0.0f;
        for (int k0 = 0; k0 < top_k; k0 += KC) {
            bool on[KC];
            float wk[KC];
            float v[KC][V];
#pragma unroll
            for (int k = 0; k < KC; k++) {
                const int64_t r = t * top_k + k0 + k;
                on[k] = false;
                wk[k] = 0.0f;
                if (k0 + k < top_k) {
                    const int32_t e = ids[r];
                    on[k] = e >= 0 && e < E;
                    wk[k] = w[r];
                    load_route<YDT, V>(o, r * Np + n, v[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < KC; k++) {
                if (!on[k]) continue;
#pragma unroll
                for (int c = 0; c < V; c++) acc[c] = __builtin_fmaf(wk[k], v[k][c], acc[c]);
            }
        }
        const int64_t idx = t * Np + n;
        if (YDT == DT_F32) {
            if (V == 4) *reinterpret_cast<v4f *>(static_cast<float *>(y) + idx) = v4f{acc[0], acc[V > 1 ? 1 : 0], acc[V > 2 ? 2 : 0], acc[V > 3 ? 3 : 0]};
            else for (int c = 0; c < V; c++) static_cast<float *>(y)[idx + c] = acc[c];
        } else {
            const bool h = YDT == DT_F16;
            if (V == 8) {
                v4i b;
#pragma unroll
                for (int c = 0; c < 4; c++)
                    b[c] = (int)(f32_to_16(acc[(2 * c) % V], h) | (f32_to_16(acc[(2 * c + 1) % V], h) << 16));
                *reinterpret_cast<v4i *>(static_cast<uint16_t *>(y) + idx) = b;
            } else {
                for (int c = 0; c < V; c++) static_cast<uint16_t *>(y)[idx + c] = (uint16_t)f32_to_16(acc[c], h);
            }
        }
    }
}

// Split-K finish: y[m][n] = sum over slices k in order of part[k][m][n]
// (fp32), stored in the output dtype.  One thread per output.
template <int YDT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int ks, int64_t M,
                                                            int64_t N, void *__restrict__ y, int y_f16, int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * N) return;
    const int64_t m = i / N, n = i - m * N;
    float acc = part[i];
    for (int k = 1; k < ks; k++) acc += part[(int64_t)k * M * N + i];
    if (YDT == DT_F32) static_cast<float *>(y)[m * ldy + n] = acc;
    else static_cast<uint16_t *>(y)[m * ldy + n] = (uint16_t)f32_to_16(acc, y_f16 != 0);
}

// Zero the output rows of inactive routes (id < 0 or id >= E) in the
// unweighted mul_mat_id output y[T*top_k][Np]: one lane per route.
template <int YDT>
__global__ __launch_bounds__(256) void zero_inactive_kernel(const int32_t *__restrict__ ids, int64_t R, int64_t E,
                                                            int64_t Np, void *__restrict__ y) {
    const int64_t r0 = (int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~63u);   // this wave's first route
    zero_dead_routes<YDT>(ids, R, E, Np, y, r0, threadIdx.x & 63);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

hipError_t launch_quantize(const void *x, int xdt, int64_t M, int64_t K, int64_t ldx, uint8_t *q8, _Float16 *xq,
                           float *xd, uint16_t *xm, bool tiled, hipStream_t s) {
    const int64_t threads = M * (K / QK8_1) * 8;
    if (threads == 0) return hipSuccess;
    const uintptr_t a = reinterpret_cast<uintptr_t>(x);
    // 16 values per lane (2 lanes per block) where the rows allow it, else 8 (4 lanes):
    // measured 14.5 / 16.0 / 20.1 us for 8192 bf16 rows of 2048 (this kernel, 16 and 8
    // values per lane, 4 per lane in the 8-lane kernel)
    if ((ldx % 8) == 0 && (a % 16) == 0) {
#define GGQ_QW(LPB)                                                                                                   \
    {                                                                                                                 \
        dim3 g(grid_for(threads / 8 * LPB)), b(256);                                                                  \
        if (xdt == DT_F32) hipLaunchKernelGGL((quantize_q8_1_wide_kernel<DT_F32, LPB>), g, b, 0, s, x, M, K, ldx, q8, xq, xd, xm, tiled); \
        else if (xdt == DT_F16) hipLaunchKernelGGL((quantize_q8_1_wide_kernel<DT_F16, LPB>), g, b, 0, s, x, M, K, ldx, q8, xq, xd, xm, tiled); \
        else hipLaunchKernelGGL((quantize_q8_1_wide_kernel<DT_BF16, LPB>), g, b, 0, s, x, M, K, ldx, q8, xq, xd, xm, tiled); \
    }
        if ((ldx % 16) == 0) GGQ_QW(2) else GGQ_QW(4)
#undef GGQ_QW
        return hipGetLastError();
    }
    const bool vec = xdt == DT_F32 ? ((ldx % 4) == 0 && (a % 16) == 0) : ((ldx % 4) == 0 && (a % 8) == 0);
    dim3 g(grid_for(threads)), b(256);
    if (xdt == DT_F32) {
        if (vec) hipLaunchKernelGGL((quantize_q8_1_kernel<DT_F32, true>), g, b, 0, s, x, M, K, ldx, q8, xq, xd, xm, tiled);
        else hipLaunchKernelGGL((quantize_q8_1_kernel<DT_F32, false>), g, b, 0, s, x, M, K, ldx, q8, xq, xd, xm, tiled);
    } else if (xdt == DT_F16) {
        if (vec) hipLaunchKernelGGL((quantize_q8_1_kernel<DT_F16, true>), g, b, 0, s, x, M, K, ldx, q8, xq, xd, xm, tiled);
        else hipLaunchKernelGGL((quantize_q8_1_kernel<DT_F16, false>), g, b, 0, s, x, M, K, ldx, q8, xq, xd, xm, tiled);
    } else {
        if (vec) hipLaunchKernelGGL((quantize_q8_1_kernel<DT_BF16, true>), g, b, 0, s, x, M, K, ldx, q8, xq, xd, xm, tiled);
        else hipLaunchKernelGGL((quantize_q8_1_kernel<DT_BF16, false>), g, b, 0, s, x, M, K, ldx, q8, xq, xd, xm, tiled);
    }
    return hipGetLastError();
}

hipError_t launch_q8_1_to_planar(const uint8_t *q8, int64_t M, int64_t K, _Float16 *xq, float *xd, uint16_t *xm,
                                 bool tiled, hipStream_t s) {
    const int64_t threads = M * (K / QK8_1) * 8;
    if (threads == 0) return hipSuccess;
    hipLaunchKernelGGL(q8_1_to_planar_kernel, dim3(grid_for(threads)), dim3(256), 0, s, q8, M, K, xq, xd, xm, tiled);
    return hipGetLastError();
}

hipError_t launch_dequant(int t, const uint8_t *W, int64_t rows, int64_t K, const int32_t *ids, int64_t n, void *y,
                          int ydt, int64_t ldy, hipStream_t s) {
    const int64_t threads = n * (K / 16);
    if (threads == 0) return hipSuccess;
    const int64_t rb = K / (t == T_Q4_0 || t == T_Q8_0 ? 32 : 256) *
                       (t == T_Q4_0 ? 18 : t == T_Q8_0 ? 34 : t == T_Q4_K ? 144 : t == T_Q5_K ? 176 : 210);
    const int64_t wbytes = rows * rb;
    // staged rows: up to DQ_ROW_MAX bytes, buffer offsets within 32 bits
    const bool staged = rb <= DQ_ROW_MAX && wbytes < (int64_t(1) << 31);
    const int slot = (int)((rb + 15) / 16 * 16 + 32);
    const int64_t chunks = (rb + 30) / 16;                // 16-byte loads a row needs at most
    const int nl = chunks <= 128 ? 2 : chunks <= 256 ? 4 : 9;
    dim3 g(grid_for(threads)), b(256), gr((unsigned)std::min<int64_t>((n + 3) / 4, DQ_MAX_WG));
#define GGQ_DQ2(TT, D, NLV)                                                                                            \
    hipLaunchKernelGGL((dequant_rows_kernel<TT, D, NLV>), gr, b, 4 * slot, s, W, wbytes, rows, K, ids, n, y, ldy, slot);
#define GGQ_DQ1(TT, D)                                                                                                 \
    if (!staged) hipLaunchKernelGGL((dequant_kernel<TT, D>), g, b, 0, s, W, rows, K, ids, n, y, ldy);                 \
    else if (nl == 2) { GGQ_DQ2(TT, D, 2) }                                                                           \
    else if (nl == 4) { GGQ_DQ2(TT, D, 4) }                                                                           \
    else { GGQ_DQ2(TT, D, 9) }
#define GGQ_DQ(TT)                                                                                                    \
    if (t == TT) {                                                                                                    \
        if (ydt == DT_F32) { GGQ_DQ1(TT, DT_F32) }                                                                    \
        else if (ydt == DT_F16) { GGQ_DQ1(TT, DT_F16) }                                                               \
        else { GGQ_DQ1(TT, DT_BF16) }                                                                                 \
    }
    GGQ_DQ(T_Q4_0) GGQ_DQ(T_Q8_0) GGQ_DQ(T_Q4_K) GGQ_DQ(T_Q5_K) GGQ_DQ(T_Q6_K)
#undef GGQ_DQ
#undef GGQ_DQ1
#undef GGQ_DQ2
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const unsigned g = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(g), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_route_sum(const void *o, const int32_t *ids, const float *w, int64_t T, int top_k, int64_t E,
                            int64_t Np, void *y, int ydt, hipStream_t s) {
    // 16-byte rows pieces when Np allows (o, y and the workspace are 16-byte aligned)
    const int V = ydt == DT_F32 ? (Np % 4 == 0 ? 4 : 1) : (Np % 8 == 0 ? 8 : 1);
    const int64_t n = T * (Np / V);
    if (n == 0) return hipSuccess;
    const dim3 g((unsigned)std::min<int64_t>((n + 255) / 256, 16384)), b(256);
#define GGQ_RS(D, VV) hipLaunchKernelGGL((route_sum_kernel<D, VV>), g, b, 0, s, o, ids, w, T, top_k, E, Np, y)
    if (ydt == DT_F32) {
        if (V == 4) GGQ_RS(DT_F32, 4);
        else GGQ_RS(DT_F32, 1);
    } else if (ydt == DT_F16) {
        if (V == 8) GGQ_RS(DT_F16, 8);
        else GGQ_RS(DT_F16, 1);
    } else {
        if (V == 8) GGQ_RS(DT_BF16, 8);
        else GGQ_RS(DT_BF16, 1);
    }
#undef GGQ_RS
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *part, int ks, int64_t M, int64_t N, void *y, int ydt, int y_f16,
                                int64_t ldy, hipStream_t s) {
    if (M * N == 0) return hipSuccess;
    const dim3 g(grid_for(M * N)), b(256);
    if (ydt == DT_F32) hipLaunchKernelGGL(splitk_reduce_kernel<DT_F32>, g, b, 0, s, part, ks, M, N, y, y_f16, ldy);
    else hipLaunchKernelGGL(splitk_reduce_kernel<DT_BF16>, g, b, 0, s, part, ks, M, N, y, y_f16, ldy);
    return hipGetLastError();
}

hipError_t launch_zero_inactive(const int32_t *ids, int64_t R, int64_t E, int64_t Np, void *y, int ydt,
                                hipStream_t s) {
    if (R == 0) return hipSuccess;
    const dim3 g(grid_for(R)), b(256);
    if (ydt == DT_F32) hipLaunchKernelGGL(zero_inactive_kernel<DT_F32>, g, b, 0, s, ids, R, E, Np, y);
    else if (ydt == DT_BF16 || ydt == DT_F16)                                     // 16-bit zeros
        hipLaunchKernelGGL(zero_inactive_kernel<DT_BF16>, g, b, 0, s, ids, R, E, Np, y);
    else hipLaunchKernelGGL(zero_inactive_kernel<DT_Q8_1>, g, b, 0, s, ids, R, E, Np, y);
    return hipGetLastError();
}

}  // namespace ggq
