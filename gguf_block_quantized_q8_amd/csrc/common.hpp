// Shared device helpers for the gfx950 kernels: scalar codecs, block
// geometry, byte loads from 2-byte aligned block fields, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ggq {

enum : int { T_Q4_0 = 2, T_Q8_0 = 8, T_Q4_K = 12, T_Q5_K = 13, T_Q6_K = 14 };
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_Q8_1 = 2, DT_F16 = 3 };

constexpr int QK8_1 = 32;
constexpr int Q8_1_BYTES = 40;   // float d, float s, int8 qs[32]

template <int T> struct Geom;
template <> struct Geom<T_Q4_0> { static constexpr int QK = 32,  BYTES = 18,  G = 32; };
template <> struct Geom<T_Q8_0> { static constexpr int QK = 32,  BYTES = 34,  G = 32; };
template <> struct Geom<T_Q4_K> { static constexpr int QK = 256, BYTES = 144, G = 32; };
template <> struct Geom<T_Q5_K> { static constexpr int QK = 256, BYTES = 176, G = 32; };
template <> struct Geom<T_Q6_K> { static constexpr int QK = 256, BYTES = 210, G = 16; };

__host__ __device__ inline int64_t block_len(int t) {
    return (t == T_Q4_0 || t == T_Q8_0) ? 32 : (t == T_Q4_K || t == T_Q5_K || t == T_Q6_K) ? 256 : 0;
}
__host__ __device__ inline int64_t block_bytes(int t) {
    return t == T_Q4_0 ? 18 : t == T_Q8_0 ? 34 : t == T_Q4_K ? 144 : t == T_Q5_K ? 176 : t == T_Q6_K ? 210 : 0;
}
__host__ __device__ inline int64_t group_len(int t) { return t == T_Q6_K ? 16 : 32; }

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v4i_a4 __attribute__((ext_vector_type(4), aligned(4)));  // 16 B, dword alignment
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---- scalar codecs ----
// int bits -> float.  Takes its argument by value: clang's __builtin_bit_cast
// applied directly to an ext_vector element (v.y, v[i]) reads element 0.
__device__ __forceinline__ float as_float(int bits) { return __builtin_bit_cast(float, bits); }
__device__ __forceinline__ float fp16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);   // v_cvt_f32_f16: exact, subnormals kept
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, b << 16);
}
// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16, nan = (u >> 16) | 0x40u;
    return (u & 0x7fffffffu) > 0x7f800000u ? nan : r;                  // a select, not a branch
}
// fp32 -> IEEE binary16 bits, round to nearest even (v_cvt_f16_f32 in the
// default rounding mode, subnormal halves kept); past the largest finite half
// the result is inf.  f is a final fp32 value: the empty asm keeps the
// compiler from folding the product that made it into a mixed fma that rounds
// once, straight to fp16.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    __asm__("" : "+v"(f));
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// 16-bit elements: fp16 when h, else bf16.
__device__ __forceinline__ uint32_t f32_to_16(float f, bool h) { return h ? f32_to_f16_bits(f) : f32_to_bf16_bits(f); }
__device__ __forceinline__ float from_16(uint32_t b, bool h) { return h ? fp16_bits_to_f32(b) : bf16_bits_to_f32(b & 0xffffu); }

// q8_1 quant of one value of a block whose largest magnitude is amax, with
// d = amax / 127: x / d (IEEE fp32 division) rounded half away from zero; an
// all-zero block gives 0.  |x / d| <= 127 (1 + 2^-23), so the clamp only
// guards the rounding of that bound.
__device__ __forceinline__ int q8_1_quant(float x, float d, float amax) {
    if (amax == 0.0f) return 0;
    return (int)fminf(fmaxf(roundf(x / d), -127.0f), 127.0f);
}

// ---- MMQ planar activation operand ----
// The Q4_K / Q5_K min term of MMQ multiplies each weight row's integer mins
// by the activations' q8_1 sums s through a bf16 MFMA: per row and
// super-block (256 values, 8 q8_1 blocks) the operand is 32 bf16 entries,
// entries 3g, 3g + 1, 3g + 2 the three parts of s_g (their exact sum is s_g)
// and entries 24..31 zero.  Written by whoever writes the quantized row.
__device__ __forceinline__ uint16_t bf16_trunc_bits(float v) { return (uint16_t)(__builtin_bit_cast(uint32_t, v) >> 16); }
__device__ __forceinline__ void split3_bf16_bits(float v, uint16_t &p0, uint16_t &p1, uint16_t &p2) {
    const float h0 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & 0xffff0000u);
    const float r1 = v - h0;                                   // exact
    const float h1 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, r1) & 0xffff0000u);
    const float r2 = r1 - h1;                                  // exact, at most 8 significant bits
    p0 = bf16_trunc_bits(h0);
    p1 = bf16_trunc_bits(h1);
    p2 = bf16_trunc_bits(r2);
}
// Operand layouts.  Row-major (routed MMQ gathers arbitrary rows): xq [rows][K],
// xd [rows][K/32], xm [rows][K/256][32].  Tiled (dense MMQ, rows padded to a multiple
// of 64): every 32-row group and 32-value stage of xq is one contiguous 2 KB piece
// holding the two 1 KB MFMA fragment images the kernel stages (half kk of 16 K values;
// lane r + 32 h of a half holds row r, K values 16 kk + 8 h .. + 8); xd is
// [rows / 64][K/32][64]; xm is [rows / 32][K/256][2][64][8] with the same fragment
// order over its 32 entries.  So each copy the kernel issues reads whole cache lines.
__device__ __forceinline__ int64_t xq_index(bool tiled, int64_t m, int64_t K, int64_t k) {
    if (!tiled) return m * K + k;
    const int kin = (int)(k & 31);
    return ((((m >> 5) * (K >> 5) + (k >> 5)) * 2 + (kin >> 4)) * 64 + (m & 31) + 32 * ((kin >> 3) & 1)) * 8 + (kin & 7);
}
__device__ __forceinline__ int64_t xd_index(bool tiled, int64_t m, int64_t nb, int64_t blk) {
    return tiled ? ((m >> 6) * nb + blk) * 64 + (m & 63) : m * nb + blk;
}
__device__ __forceinline__ int64_t xm_index(bool tiled, int64_t m, int64_t nsb, int64_t sb, int ent) {
    if (!tiled) return (m * nsb + sb) * 32 + ent;
    return ((((m >> 5) * nsb + sb) * 2 + (ent >> 4)) * 64 + (m & 31) + 32 * ((ent >> 3) & 1)) * 8 + (ent & 7);
}
// row m, q8_1 block blk (K % 256 == 0)
__device__ __forceinline__ void planar_write_min(uint16_t *xm, bool tiled, int64_t m, int64_t K, int64_t blk, float s) {
    const int64_t nsb = K / 256, sb = blk >> 3;
    const int g = (int)(blk & 7);
    uint16_t p0, p1, p2;
    split3_bf16_bits(s, p0, p1, p2);
    xm[xm_index(tiled, m, nsb, sb, 3 * g)] = p0;
    xm[xm_index(tiled, m, nsb, sb, 3 * g + 1)] = p1;
    xm[xm_index(tiled, m, nsb, sb, 3 * g + 2)] = p2;
    if (g == 7) *reinterpret_cast<v4i *>(xm + xm_index(tiled, m, nsb, sb, 24)) = v4i{0, 0, 0, 0};   // entries 24..31
}

// ---- loads ----
__device__ __forceinline__ uint32_t ld_u16(const uint8_t *p) {
    return *reinterpret_cast<const uint16_t *>(p);
}

// Read 16 bytes starting at a 2-byte aligned address p as 4 little-endian
// dwords.  Touches only [p, p + 16) when p is 4-byte aligned, and
// [p - 2, p + 16) otherwise (the last two bytes come from a 16-bit load), so a
// field never pulls in bytes past its own end.
__device__ __forceinline__ v4i ld16_a2(const uint8_t *p) {
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (a & 2) {
        const uint32_t *q = reinterpret_cast<const uint32_t *>(a - 2);
        uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3];
        uint32_t w4 = *reinterpret_cast<const uint16_t *>(p + 14);
        return v4i{(int)__builtin_amdgcn_alignbyte(w1, w0, 2), (int)__builtin_amdgcn_alignbyte(w2, w1, 2),
                   (int)__builtin_amdgcn_alignbyte(w3, w2, 2), (int)__builtin_amdgcn_alignbyte(w4, w3, 2)};
    }
    return *reinterpret_cast<const v4i_a4 *>(p);
}

// 4 bytes at a 2-byte aligned address; touches [p, p + 4) or [p - 2, p + 4).
__device__ __forceinline__ uint32_t ld4_a2(const uint8_t *p) {
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (a & 2) {
        uint32_t w0 = *reinterpret_cast<const uint32_t *>(a - 2);
        uint32_t w1 = *reinterpret_cast<const uint16_t *>(p + 2);
        return __builtin_amdgcn_alignbyte(w1, w0, 2);
    }
    return *reinterpret_cast<const uint32_t *>(p);
}

// ---- packed int8 dot ----
__device__ __forceinline__ int dot4(int a, int b, int c) {
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// ---- cross-lane reductions ----
// DPP / permlane based: no LDS traffic.  dpp(v, ctrl) reads lane-permuted v.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <- 7 - i within 8 lanes
constexpr int DPP_MIRROR = 0x140;       // lane i <- 15 - i within 16 lanes
constexpr int DPP_ROW_BCAST15 = 0x142;  // lane 15 of each row -> next row
constexpr int DPP_ROW_BCAST31 = 0x143;  // lane 31 -> rows 2 and 3

// Max / sum over aligned groups of 8 lanes, result in every lane of the group.
__device__ __forceinline__ float max8(float v) {
    v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    return fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
}
__device__ __forceinline__ int sum8(int v) {
    v += dpp_i<DPP_XOR1>(v);
    v += dpp_i<DPP_XOR2>(v);
    return v + dpp_i<DPP_HALF_MIRROR>(v);
}

// Sum over aligned segments of `width` lanes (a power of two <= 64), with the
// segment total in the LAST lane of each segment (width <= 16: in every lane),
// for every value of a [2][N] array.  Within a 16-lane row: DPP butterflies;
// across rows: DPP row broadcasts (lane 15 of a row into the next row, lane 31
// into rows 2 and 3).  One step at a time for all values: `width` is a runtime
// value, so a branch per step rather than per value and step, and the values'
// independent DPP moves overlap.
template <int N>
__device__ __forceinline__ void seg_sum(float (&a)[2][N], int width) {
    auto step = [&](auto f) {
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int c = 0; c < N; c++) a[i][c] += f(a[i][c]);
    };
    if (width >= 2) step([](float v) { return dpp_f<DPP_XOR1>(v); });
    if (width >= 4) step([](float v) { return dpp_f<DPP_XOR2>(v); });
    if (width >= 8) step([](float v) { return dpp_f<DPP_HALF_MIRROR>(v); });
    if (width >= 16) step([](float v) { return dpp_f<DPP_MIRROR>(v); });
    if (width >= 32)                        // rows 1, 3 += lane 15 of rows 0, 2
        step([](float v) {
            return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), DPP_ROW_BCAST15, 0xA, 0xF, false));
        });
    if (width >= 64)                        // rows 2, 3 += lane 31
        step([](float v) {
            return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), DPP_ROW_BCAST31, 0xC, 0xF, false));
        });
}

}  // namespace ggq
