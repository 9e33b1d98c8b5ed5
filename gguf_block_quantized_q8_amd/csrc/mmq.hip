// MMQ: tiled quantized matmul for prefill, on fp16 MFMA with exact integer
// operands.
//
// Why fp16 MFMA and not int8 MFMA: each output needs one fp32 rescale per
// 32-wide q8_1 block (weight sub-scale x activation scale), and the VALU does
// one wave64 operation per 4 cycles per SIMD, about the time a 32x32 MFMA
// needs for its 1024 outputs.  With int8 MFMA the rescale costs cvt + int
// multiply by the sub-scale + fma per output per block; here the integer
// sub-scale is folded into the fp16 weight operand instead (Q4_K: sc * nibble
// <= 945, Q5_K: sc * value <= 1953, Q6_K: sc * (q - 32) split into two exact
// fp16 parts), the MFMA sums
// the block's dot in fp32 exactly, and one fma per output per block remains
// (times the activation scale d8).  Every product and partial sum is an
// integer below 2^24, so the per-block dot is exact, as with int8.  Q8_0 and
// Q4_0 carry their fp16 scale per 32-weight block: their staged operand is the
// plain quant (q, or nibble - 8), and each stage applies d * d8 per output.
//
// Tiles: 128 weight rows x 128 activation rows per workgroup, 4 waves of
// 64 x 64 (2 x 2 MFMA 32x32x16 tiles).  K advances one q8_1 block (32) per
// stage, software-pipelined: each thread holds the next stage's raw weight
// bytes and activation quants in registers while the current stage computes
// from one of two LDS buffers, and a stage ends with an LDS-only barrier (no
// wait on the global loads in flight).  Per 256-wide super-block the weight
// d / dmin and the activation d8 / s8 are staged once.  The Q4_K / Q5_K min term
// -dmin * sum_j m_j * s8_j runs as a bf16 MFMA with s8 split exactly into
// three bf16 parts.
#include "kernels.hpp"

namespace ggq {

constexpr int NT = MMQ_NT, MT = MMQ_MT, KS = 32, LDA = KS + 8, LDM = 40;
constexpr int EPI_NONE_ = 0, EPI_SWIGLU_ = 1;

// Q8_0 / Q4_0: one fp16 weight scale per 32-weight block, i.e. per stage.
template <int T> constexpr bool kBlk32 = T == T_Q8_0 || T == T_Q4_0;

template <int T>
struct __attribute__((aligned(16))) MmqSmem {
    static constexpr int NA = T == T_Q6_K ? 2 : 1;       // Q6_K: high and low parts of sc*(q-32)
    static constexpr int NMIN = (T == T_Q4_K || T == T_Q5_K) ? 1 : 0;
    _Float16 A[2][NA][NT][LDA];   // two stage buffers
    _Float16 B[2][MT][LDA];
    float d8[2][8][MT];           // by super-block parity; [block][column]: conflict-free column reads
    float wd[kBlk32<T> ? 2 : 1][NT];   // K-quants: d of the super-block; Q8_0 / Q4_0: d of the stage's block
    float wdmin[NT];
    __bf16 Amin[NMIN ? NT : 1][LDM];
    __bf16 Bmin[NMIN ? MT : 1][LDM];
    int32_t xrow[MT];     // activation row of each tile column (-1: none)
    int32_t route[MT];    // routed: route id of each tile column
    const uint8_t *wrow[NT];
};

// Split an fp32 value into three bf16 parts whose exact sum is the value.
__device__ __forceinline__ void split3_bf16(float v, __bf16 &p0, __bf16 &p1, __bf16 &p2) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const float h0 = __builtin_bit_cast(float, u & 0xffff0000u);
    const float r1 = v - h0;                                   // exact
    const float h1 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, r1) & 0xffff0000u);
    const float r2 = r1 - h1;                                  // exact, <= 8 significant bits
    p0 = __builtin_bit_cast(__bf16, (uint16_t)(__builtin_bit_cast(uint32_t, h0) >> 16));
    p1 = __builtin_bit_cast(__bf16, (uint16_t)(__builtin_bit_cast(uint32_t, h1) >> 16));
    p2 = __builtin_bit_cast(__bf16, (uint16_t)(__builtin_bit_cast(uint32_t, r2) >> 16));
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2v as_h2(uint32_t u) { return __builtin_bit_cast(h2v, u); }
__device__ __forceinline__ uint32_t h2_bits(h2v h) { return __builtin_bit_cast(uint32_t, h); }

// Bytes 0,1 (sel = 0x00050004) or 2,3 (sel = 0x00070006) of x, each as the low
// byte of a 16-bit half whose high byte is 0x64: read through `mask`, the half
// is the fp16 number 1024 + (byte & low bits of mask).
__device__ __forceinline__ uint32_t spread2(uint32_t x, uint32_t sel, uint32_t mask) {
    return __builtin_amdgcn_perm(x, 0x64646464u, sel) & mask;
}

// Q4_K: 8 packed 6-bit values (scales or mins) of the 12 header bytes
// s0..s2, one per byte: groups 0..3 in `lo`, 4..7 in `hi`.
__device__ __forceinline__ void q4k_pack(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t &sc_lo, uint32_t &sc_hi,
                                         uint32_t &mn_lo, uint32_t &mn_hi) {
    sc_lo = s0 & 0x3f3f3f3fu;
    mn_lo = s1 & 0x3f3f3f3fu;
    sc_hi = (s2 & 0x0f0f0f0fu) | ((s0 >> 2) & 0x30303030u);
    mn_hi = ((s2 >> 4) & 0x0f0f0f0fu) | ((s1 >> 2) & 0x30303030u);
}

// 16-byte global load (the pointer may have come through LDS, so name the
// address space: a flat load would also count against the LDS counter).
__device__ __forceinline__ v4i gld16(const uint8_t *p) {
    return *(const v4i __attribute__((address_space(1))) *)p;
}

// One stage's raw operands in registers: thread t stages weight row t/2 (16
// of the stage's 32 K values, half t&1) and tile column t/2 (same split).
// Rows and columns past the matrix read a valid row instead (their results
// are never stored), so staging has no branches.
// UNIT: all sub-scales 1 and no activation scales (test hook: raw dots).
template <int T, bool UNIT>
struct Stager {
    static constexpr bool HAS_MIN = T == T_Q4_K || T == T_Q5_K;   // d*sc*q - dmin*m types
    const uint8_t *wrow;      // this thread's weight row
    const _Float16 *xrow;     // this thread's activation row + 16 * half
    const float *xd, *xs;     // d, s of this thread's activation row + 4 * half
    v4i hdr;        // Q4_K / Q5_K: block header (d, dmin, 12 scale bytes); Q6_K: the 16 int8 scales
    v4i q0, q1;     // Q4_K: 16 quant bytes (q0); Q5_K: also 16 fifth-bit bytes (q1);
    v4i q0o;        // Q6_K: the 16 ql bytes of the odd groups (q0: even groups)
                    // Q6_K: 16 ql bytes (q0), 16 qh bytes (q1); Q8_0: this half's 16 int8 quants;
                    // Q4_0: the block's 16 nibble bytes (both halves)
    uint32_t d6;    // Q6_K, Q8_0, Q4_0: fp16 d
    v4i b0, b1;     // 16 fp16 activation quants
    v4f m;          // stage 0 of a super-block: 4 d8; stage 1 (Q4_K, Q5_K): 4 s8

    __device__ void init(const uint8_t *row, const _Float16 *xq, const float *d, const float *sx, int64_t K,
                         int64_t xr) {
        const int hf = threadIdx.x & 1;
        wrow = row;
        xrow = xq + xr * K + 16 * hf;
        const int64_t nb = K / QK8_1;
        xd = UNIT ? nullptr : d + xr * nb + 4 * hf;
        xs = (UNIT || !HAS_MIN) ? nullptr : sx + xr * nb + 4 * hf;
    }

    // Stages are loaded once each, in order (load(s + 1) after store(s)), so
    // registers that the next stage would load again keep their bytes: a
    // K-quant super-block's header (Q5_K: also its fifth bits; Q6_K: its
    // scales and d) is loaded at its first stage only, Q4_K / Q5_K quant bytes
    // once per pair of stages (low nibbles, then high), Q6_K low bits once per
    // pair (groups g and g + 2) and high bits once per four.
    __device__ void load(int s) {
        const int hf = threadIdx.x & 1;
        const int sb = s >> 3, j = s & 7;
        if (T == T_Q4_K) {
            const uint8_t *blk = wrow + (int64_t)sb * 144;
            if (j == 0) hdr = gld16(blk);
            if ((j & 1) == 0) q0 = gld16(blk + 16 + 32 * (j >> 1) + 16 * hf);
        } else if (T == T_Q5_K) {
            const uint8_t *blk = wrow + (int64_t)sb * 176;
            if (j == 0) {
                hdr = gld16(blk);
                q1 = gld16(blk + 16 + 16 * hf);                     // fifth bits of positions 16 hf ..
            }
            if ((j & 1) == 0) q0 = gld16(blk + 48 + 32 * (j >> 1) + 16 * hf);
        } else if (T == T_Q8_0) {
            const uint8_t *blk = wrow + (int64_t)s * 34;           // one block per stage
            q0 = ld16_a2(blk + 2 + 16 * hf);
            d6 = ld_u16(blk);
        } else if (T == T_Q4_0) {
            const uint8_t *blk = wrow + (int64_t)s * 18;
            q0 = ld16_a2(blk + 2);                                  // weights l (low nibble) and l + 16 (high)
            d6 = ld_u16(blk);
        } else {
            const uint8_t *blk = wrow + (int64_t)sb * 210;
            const int hh = j >> 2, g = j & 3;
            // groups g and g + 2 share their ql bytes (low, then high nibbles)
            if (g == 0) q0 = ld16_a2(blk + 64 * hh + 16 * hf);
            if (g == 1) q0o = ld16_a2(blk + 64 * hh + 32 + 16 * hf);
            if (g == 0) q1 = ld16_a2(blk + 128 + 32 * hh + 16 * hf);
            if (j == 0) {
                hdr = ld16_a2(blk + 192);
                d6 = ld_u16(blk + 208);
            }
        }
        const _Float16 *src = xrow + (int64_t)s * KS;
        b0 = *reinterpret_cast<const v4i *>(src);
        b1 = *reinterpret_cast<const v4i *>(src + 8);
        if (!UNIT && j == 0) m = *reinterpret_cast<const v4f *>(xd + sb * 8);
        if (!UNIT && HAS_MIN && j == 1) m = *reinterpret_cast<const v4f *>(xs + sb * 8);
    }

    __device__ void store(MmqSmem<T> &sm, int s) {
        const int tid = threadIdx.x, tr = tid >> 1, hf = tid & 1;
        const int sb = s >> 3, j = s & 7, buf = s & 1;
        // ---- weights: fp16 of sub-scale x quant, built in packed halves ----
        if (kBlk32<T>) {
            // Q8_0: q + 128 as a byte, read as fp16 1024 + byte, minus 1152; Q4_0: nibble - 8 likewise
            const _Float16 off = (_Float16)(T == T_Q8_0 ? -1152.0f : -1032.0f);
            const h2v off2 = {off, off};
            uint32_t o[8];
#pragma unroll
            for (int w = 0; w < 4; w++) {
                const uint32_t x = T == T_Q8_0 ? (uint32_t)q0[w] ^ 0x80808080u
                                               : (hf ? ((uint32_t)q0[w] >> 4) : (uint32_t)q0[w]) & 0x0f0f0f0fu;
                o[2 * w] = h2_bits(as_h2(__builtin_amdgcn_perm(x, 0x64646464u, 0x00050004u)) + off2);
                o[2 * w + 1] = h2_bits(as_h2(__builtin_amdgcn_perm(x, 0x64646464u, 0x00070006u)) + off2);
            }
            v4i *dst = reinterpret_cast<v4i *>(&sm.A[buf][0][tr][16 * hf]);
            dst[0] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
            dst[1] = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
            if (!UNIT && hf == 0) sm.wd[buf][tr] = fp16_bits_to_f32(d6);
        } else if (HAS_MIN) {
            uint32_t sc_lo, sc_hi, mn_lo, mn_hi;
            q4k_pack((uint32_t)hdr.y, (uint32_t)hdr.z, (uint32_t)hdr.w, sc_lo, sc_hi, mn_lo, mn_hi);
            const int sc = UNIT ? 1 : (int)__builtin_amdgcn_ubfe(j < 4 ? sc_lo : sc_hi, 8 * (j & 3), 8);
            // (1024 + nib) * sc - 1024 * sc = sc * nib, exact in one fused rounding
            const _Float16 scf = (_Float16)(float)sc, off = (_Float16)(float)(-1024 * sc);
            const h2v sc2 = {scf, scf}, off2 = {off, off};
            uint32_t o[8];
#pragma unroll
            for (int w = 0; w < 4; w++) {
                uint32_t x = (j & 1) ? ((uint32_t)q0[w] >> 4) : (uint32_t)q0[w];   // odd groups: high nibbles
                // Q5_K: value = nibble | fifth bit (bit j of the byte) << 4, at most 31, so sc * value
                // stays below 2048 and exact in fp16 as well
                uint32_t mask = 0x640f640fu;
                if (T == T_Q5_K) {
                    x = (x & 0x0f0f0f0fu) | ((((uint32_t)q1[w] >> j) & 0x01010101u) << 4);
                    mask = 0x641f641fu;
                }
                o[2 * w] = h2_bits(__builtin_elementwise_fma(as_h2(spread2(x, 0x00050004u, mask)), sc2, off2));
                o[2 * w + 1] = h2_bits(__builtin_elementwise_fma(as_h2(spread2(x, 0x00070006u, mask)), sc2, off2));
            }
            v4i *dst = reinterpret_cast<v4i *>(&sm.A[buf][0][tr][16 * hf]);
            dst[0] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
            dst[1] = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
        } else {
            const int hh = (j >> 2), g = j & 3;
            const int sc = UNIT ? 1 : (int)(int8_t)__builtin_amdgcn_ubfe((uint32_t)hdr[(8 * hh + 2 * g + hf) >> 2],
                                                                          8 * ((2 * g + hf) & 3), 8);
            const int sl = sc & 15, shi = sc - sl;
            const _Float16 shf = (_Float16)(float)shi, slf = (_Float16)(float)sl, moff = (_Float16)-1056.0f;
            const h2v sh2 = {shf, shf}, sl2 = {slf, slf}, off2 = {moff, moff};
            uint32_t oh[8], ol[8];
#pragma unroll
            for (int w = 0; w < 4; w++) {
                const uint32_t ql = (uint32_t)((g & 1) ? q0o[w] : q0[w]);
                const uint32_t lo = g < 2 ? (ql & 0x0f0f0f0fu) : ((ql >> 4) & 0x0f0f0f0fu);
                const uint32_t q6 = lo | ((((uint32_t)q1[w] >> (2 * g)) & 0x03030303u) << 4);   // 0..63 per byte
#pragma unroll
                for (int hlf = 0; hlf < 2; hlf++) {
                    const h2v v = as_h2(spread2(q6, hlf ? 0x00070006u : 0x00050004u, 0x643f643fu)) + off2;   // q - 32, exact
                    oh[2 * w + hlf] = h2_bits(v * sh2);                                                        // exact
                    ol[2 * w + hlf] = h2_bits(v * sl2);
                }
            }
            v4i *dh = reinterpret_cast<v4i *>(&sm.A[buf][0][tr][16 * hf]);
            v4i *dl = reinterpret_cast<v4i *>(&sm.A[buf][1][tr][16 * hf]);
            dh[0] = v4i{(int)oh[0], (int)oh[1], (int)oh[2], (int)oh[3]};
            dh[1] = v4i{(int)oh[4], (int)oh[5], (int)oh[6], (int)oh[7]};
            dl[0] = v4i{(int)ol[0], (int)ol[1], (int)ol[2], (int)ol[3]};
            dl[1] = v4i{(int)ol[4], (int)ol[5], (int)ol[6], (int)ol[7]};
        }
        // ---- activations ----
        {
            v4i *dst = reinterpret_cast<v4i *>(&sm.B[buf][tr][16 * hf]);
            dst[0] = b0;
            dst[1] = b1;
        }
        if (UNIT) return;
        // ---- per super-block scales ----
        if (j == 0)
            for (int i = 0; i < 4; i++) sm.d8[sb & 1][4 * hf + i][tr] = m[i];
        if (j == 1 && !kBlk32<T>) {
            if (hf == 0) {
                if (HAS_MIN) {
                    sm.wd[0][tr] = fp16_bits_to_f32((uint32_t)hdr.x & 0xffffu);
                    sm.wdmin[tr] = fp16_bits_to_f32((uint32_t)hdr.x >> 16);
                } else {
                    sm.wd[0][tr] = fp16_bits_to_f32(d6);
                }
            }
            if (HAS_MIN) {
                uint32_t sc_lo, sc_hi, mn_lo, mn_hi;
                q4k_pack((uint32_t)hdr.y, (uint32_t)hdr.z, (uint32_t)hdr.w, sc_lo, sc_hi, mn_lo, mn_hi);
                const uint32_t mw = hf ? mn_hi : mn_lo;
#pragma unroll
                for (int jj = 0; jj < 4; jj++) {
                    const int g = 4 * hf + jj;
                    const __bf16 mb = (__bf16)(float)(int)__builtin_amdgcn_ubfe(mw, 8 * jj, 8);
                    sm.Amin[tr][3 * g] = mb;
                    sm.Amin[tr][3 * g + 1] = mb;
                    sm.Amin[tr][3 * g + 2] = mb;
                    split3_bf16(m[jj], sm.Bmin[tr][3 * g], sm.Bmin[tr][3 * g + 1], sm.Bmin[tr][3 * g + 2]);
                }
                if (hf == 1)
                    for (int k = 24; k < 32; k++) { sm.Amin[tr][k] = (__bf16)0.0f; sm.Bmin[tr][k] = (__bf16)0.0f; }
            }
        }
    }
};

// LDS-only workgroup barrier: this wave's LDS accesses are complete, then
// s_barrier.  Global loads in flight (the next stage's operands) are not
// waited for, unlike __syncthreads().
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// YDT: DT_F32, or a 16-bit output (fp16 when h, else bf16).
template <int YDT>
__device__ __forceinline__ void store4(void *y, int64_t idx, const float *v, int n_valid, bool h = false) {
    if (YDT == DT_F32) {
        float *o = static_cast<float *>(y) + idx;
        if (n_valid == 4 && (idx & 3) == 0) *reinterpret_cast<v4f *>(o) = v4f{v[0], v[1], v[2], v[3]};
        else for (int i = 0; i < n_valid; i++) o[i] = v[i];
    } else {
        uint16_t *o = static_cast<uint16_t *>(y) + idx;
        if (n_valid == 4 && (idx & 3) == 0) {
            v2i t = {(int)(f32_to_16(v[0], h) | (f32_to_16(v[1], h) << 16)),
                     (int)(f32_to_16(v[2], h) | (f32_to_16(v[3], h) << 16))};
            *reinterpret_cast<v2i *>(o) = t;
        } else {
            for (int i = 0; i < n_valid; i++) o[i] = (uint16_t)f32_to_16(v[i], h);
        }
    }
}

// Tile order: workgroup b runs on XCD b % 8; the tiles of one XCD are a
// contiguous range of the grouped order below, so the workgroups resident on
// an XCD at one time share a few weight tiles and a few activation tiles in
// that XCD's L2.  Grouped order: 8 weight tiles (bn) side by side, then the
// activation tiles (bm), then the next 8 weight tiles.
__device__ __forceinline__ void tile_of(int64_t b, int64_t m_tiles, int64_t n_tiles, int64_t &bm, int64_t &bn) {
    const int64_t total = m_tiles * n_tiles;
    const int64_t per = total / 8;                            // tiles per XCD in the balanced part
    const int64_t t = b < 8 * per ? (b % 8) * per + b / 8 : b;
    const int64_t G = 8;
    const int64_t gsize = G * m_tiles;                        // tiles per group of G weight tiles
    const int64_t grp = t / gsize, in = t % gsize;
    const int64_t gw = min<int64_t>(G, n_tiles - grp * G);   // weight tiles in this group
    bm = in / gw;
    bn = grp * G + in % gw;
}

// Routed output as q8_1 blocks, y[route][Np / 32] (Np % 32 == 0).  A block is
// 32 consecutive outputs of one route: one 32-row MFMA tile row group of one
// column, held 16 + 16 by lanes l and l + 32 (rows 8g + 4h + i, h = lane / 32),
// so its amax and quant sum take one lane exchange.  The values are those the
// plain epilogue would store (SwiGLU applied, rounded first to bf16 or fp16
// per p.q8_round), quantized as the q8_1 kernel does.
template <int EPI, int T>
__device__ __forceinline__ void store_q8_1(const MmqParams &p, const MmqSmem<T> &sm, const v16f (&acc)[2][2],
                                           int64_t bn, int tile_count, int wn, int wm, int lane) {
    const int lr = lane & 31, h = lane >> 5;
    const int64_t bpr = p.Np / QK8_1;                       // blocks per route
#pragma unroll
    for (int mi = 0; mi < 2; mi++) {
        const int col = 64 * wm + 32 * mi + lr;
        const bool live = col < tile_count && sm.xrow[col] >= 0;   // the same in lanes l and l + 32
        const int64_t r = live ? sm.route[col] : 0;
#pragma unroll
        for (int bi = 0; bi < (EPI == EPI_SWIGLU_ ? 1 : 2); bi++) {
            const int64_t n0 = EPI == EPI_SWIGLU_ ? bn * 64 + 32 * wn : bn * NT + 64 * wn + 32 * bi;
            float v[16];
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; e++) {
                float o;
                if (EPI == EPI_SWIGLU_) {
                    const float gt = acc[0][mi][e], up = acc[1][mi][e];
                    o = gt / (1.0f + expf(-gt)) * up;
                } else {
                    o = acc[bi][mi][e];
                }
                if (p.q8_round) o = from_16(f32_to_16(o, p.q8_round == 2), p.q8_round == 2);
                v[e] = o;
                amax = fmaxf(amax, fabsf(o));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            float d = amax / 127.0f;
            uint32_t qw[4];
            int sum = 0;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                uint32_t w = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int q = q8_1_quant(v[4 * g + i], d, amax);
                    sum += q;
                    w |= (uint32_t)(q & 0xff) << (8 * i);
                }
                qw[g] = w;
            }
            sum += __shfl_xor(sum, 32);
            if (amax == 0.0f) d = 0.0f;
            if (!live || n0 >= p.Np) continue;
            uint8_t *blk = static_cast<uint8_t *>(p.y) + (r * bpr + n0 / QK8_1) * Q8_1_BYTES;
#pragma unroll
            for (int g = 0; g < 4; g++) *reinterpret_cast<uint32_t *>(blk + 8 + 8 * g + 4 * h) = qw[g];
            if (h == 0) *reinterpret_cast<float2 *>(blk) = make_float2(d, d * (float)sum);
        }
    }
}

// grid: 1-D, m_tiles * n_tiles workgroups of 256 threads (routed: m_tiles rounded up to 8).
template <int T, bool MOE, int EPI, int YDT>
__global__ __launch_bounds__(256, 2) void mmq_kernel(const MmqParams p) {
    __shared__ MmqSmem<T> sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wn = wave & 1, wm = wave >> 1;
    int64_t bm, bn;
    int slice = 0;
    if (MOE) {
        // Workgroup b runs on XCD b mod 8.  That XCD takes the route tiles
        // t = b mod 8 (mod 8), each with all its weight tiles back to back, so a
        // route tile's activations are read into one L2 once, and the tiles of
        // one expert (neighbours in the list) spread evenly over the XCDs.
        const int64_t b = blockIdx.x, x = b & 7, i = b >> 3;
        bm = 8 * (i / p.n_tiles) + x;
        bn = i % p.n_tiles;
    } else {
        // split K: workgroups [k * tiles, (k + 1) * tiles) take the k-th of p.ksplit equal K ranges
        const int64_t tiles = p.m_tiles * p.n_tiles;
        slice = p.ksplit > 1 ? (int)(blockIdx.x / tiles) : 0;
        tile_of(blockIdx.x - (int64_t)slice * tiles, p.m_tiles, p.n_tiles, bm, bn);
    }

    // ---- tile columns (activation rows / routes) ----
    int tile_count = MT;
    const uint8_t *W = p.W;
    if (MOE) {
        if (bm >= (int64_t)*p.ntiles) return;                 // block-uniform
        const int4 tl = p.tiles[bm];
        W += (int64_t)tl.x * p.expert_stride;
        tile_count = tl.z;
        if (tid < MT) {
            int32_t xr = -1, r = -1;
            if (tid < tl.z) {
                r = p.perm[tl.y + tid];
                xr = p.x_per_route ? r : r / p.top_k;
            }
            sm.xrow[tid] = xr;
            sm.route[tid] = r;
        }
    } else {
        tile_count = (int)min<int64_t>(MT, p.M - bm * MT);     // activation rows present in this tile
        if (tid < MT) {
            const int64_t m = bm * MT + tid;
            sm.xrow[tid] = m < p.M ? (int32_t)m : -1;
        }
    }
    // ---- tile rows (weight rows) ----
    if (tid >= MT) {
        const int tr = tid - MT;
        int64_t n;
        bool ok;
        if (EPI == EPI_SWIGLU_) {
            const int w2 = tr >> 6, ni = (tr >> 5) & 1, rr = tr & 31;
            const int64_t gate = bn * 64 + 32 * w2 + rr;
            ok = gate < p.Np;
            n = (ni ? p.Np : 0) + gate;
        } else {
            n = bn * NT + tr;
            ok = n < p.N;
        }
        sm.wrow[tr] = ok ? W + n * p.row_bytes : nullptr;
    }
    __syncthreads();

    v16f acc[2][2], P[2][2];                                  // P: this super-block, set at its first block
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) acc[a][b] = v16f{};

    // stages [s0, nst) of this workgroup: whole super-blocks (the slice length is a multiple of 8)
    const int nst_all = (int)(p.K / KS), per = nst_all / (!MOE && p.ksplit > 1 ? p.ksplit : 1);
    const int s0 = slice * per, nst = s0 + per;
    const int lr = lane & 31, kh = 8 * (lane >> 5);
    const bool live = 64 * wm < tile_count;                   // this wave's columns are not all empty
    Stager<T, false> S;
    {
        // rows / columns past the matrix stage row 0 / activation row 0 (never stored)
        const uint8_t *wr = sm.wrow[tid >> 1];
        const int32_t xr = sm.xrow[tid >> 1];
        S.init(wr ? wr : W, p.xq, p.xd, p.xs, p.K, xr >= 0 ? xr : 0);
    }
    S.load(s0);
    S.store(sm, s0);
    if (s0 + 1 < nst) S.load(s0 + 1);
    lds_sync();
#pragma unroll 1
    for (int s = s0; s < nst; s++) {
        const int buf = s & 1, j = s & 7;
        if (s + 1 < nst) S.store(sm, s + 1);                 // into the other buffer
        if (s + 2 < nst) S.load(s + 2);
        // ---- this stage: one q8_1 block of every column ----
        // (a wave whose 64 columns are all empty, in a routed tile's remainder or
        // past the last activation row, skips the compute; it still stages and
        // meets the barriers)
#pragma unroll
        for (int ni = 0; ni < (live ? 2 : 0); ni++) {
            v16f C[2] = {v16f{}, v16f{}};
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                const int ko = 16 * kk + kh;
                v8h bf[2];
#pragma unroll
                for (int mi = 0; mi < 2; mi++) bf[mi] = *reinterpret_cast<const v8h *>(&sm.B[buf][64 * wm + 32 * mi + lr][ko]);
#pragma unroll
                for (int x = 0; x < MmqSmem<T>::NA; x++) {
                    const v8h af = *reinterpret_cast<const v8h *>(&sm.A[buf][x][64 * wn + 32 * ni + lr][ko]);
#pragma unroll
                    for (int mi = 0; mi < 2; mi++) C[mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[mi], C[mi], 0, 0, 0);
                }
            }
            if (kBlk32<T>) {
                // the block's weight scale per row, straight into acc: rows 8 q + 4 h + i of the half-tile
                const float *dwr = &sm.wd[buf][64 * wn + 32 * ni + 4 * (lane >> 5)];
#pragma unroll
                for (int mi = 0; mi < 2; mi++) {
                    const float d8 = sm.d8[(s >> 3) & 1][j][64 * wm + 32 * mi + lr];
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const v4f dw = *reinterpret_cast<const v4f *>(dwr + 8 * q);
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[ni][mi][4 * q + i] = __builtin_fmaf(C[mi][4 * q + i], d8 * dw[i], acc[ni][mi][4 * q + i]);
                    }
                }
                continue;
            }
#pragma unroll
            for (int mi = 0; mi < 2; mi++) {
                const float d8 = sm.d8[(s >> 3) & 1][j][64 * wm + 32 * mi + lr];
                if (j == 0) {                                 // first block of a super-block starts P
#pragma unroll
                    for (int e = 0; e < 16; e++) P[ni][mi][e] = C[mi][e] * d8;
                } else {
#pragma unroll
                    for (int e = 0; e < 16; e++) P[ni][mi][e] = __builtin_fmaf(C[mi][e], d8, P[ni][mi][e]);
                }
            }
        }
        if (j == 7 && !kBlk32<T> && live) {
            // ---- end of super-block: P * d (- dmin * min term) into acc ----
            if (MmqSmem<T>::NMIN) {
                // one weight half-tile (ni) at a time: 32 registers of min-term sums live, not 64
#pragma unroll
                for (int ni = 0; ni < 2; ni++) {
                    v16f Q[2] = {v16f{}, v16f{}};
#pragma unroll
                    for (int kk = 0; kk < 2; kk++) {
                        const int ko = 16 * kk + kh;
                        const v8bf am = *reinterpret_cast<const v8bf *>(&sm.Amin[64 * wn + 32 * ni + lr][ko]);
#pragma unroll
                        for (int mi = 0; mi < 2; mi++) {
                            const v8bf bmv = *reinterpret_cast<const v8bf *>(&sm.Bmin[64 * wm + 32 * mi + lr][ko]);
                            Q[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bmv, Q[mi], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int tr = 64 * wn + 32 * ni + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        const float d = sm.wd[0][tr], dm = sm.wdmin[tr];
#pragma unroll
                        for (int mi = 0; mi < 2; mi++) {
                            acc[ni][mi][e] = __builtin_fmaf(P[ni][mi][e], d, acc[ni][mi][e]);
                            acc[ni][mi][e] = __builtin_fmaf(Q[mi][e], -dm, acc[ni][mi][e]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int ni = 0; ni < 2; ni++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int tr = 64 * wn + 32 * ni + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        const float d = sm.wd[0][tr];
#pragma unroll
                        for (int mi = 0; mi < 2; mi++) {
                            acc[ni][mi][e] = __builtin_fmaf(P[ni][mi][e], d, acc[ni][mi][e]);
                        }
                    }
            }
        }
        lds_sync();
    }

    // ---- epilogue ----
    if (YDT == DT_Q8_1) {
        store_q8_1<EPI>(p, sm, acc, bn, tile_count, wn, wm, lane);
        return;
    }
#pragma unroll
    for (int mi = 0; mi < 2; mi++) {
        const int col = 64 * wm + 32 * mi + lr;
        if (col >= tile_count) continue;
        const int32_t xr = sm.xrow[col];
        if (xr < 0) continue;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            if (!MOE) {
#pragma unroll
                for (int ni = 0; ni < 2; ni++) {
                    const int64_t n0 = bn * NT + 64 * wn + 32 * ni + 8 * g + 4 * (lane >> 5);
                    if (n0 >= p.N) continue;
                    const int nv = (int)min<int64_t>(4, p.N - n0);
                    float v[4] = {acc[ni][mi][4 * g], acc[ni][mi][4 * g + 1], acc[ni][mi][4 * g + 2], acc[ni][mi][4 * g + 3]};
                    if (p.ksplit > 1) store4<DT_F32>(p.part, ((int64_t)slice * p.M + xr) * p.N + n0, v, nv);
                    else store4<YDT>(p.y, (int64_t)xr * p.ldy + n0, v, nv, p.y_f16);
                }
            } else {
                // weighted: per-route fp32 outputs, summed per token afterwards
                const int64_t r = sm.route[col];
                if (EPI == EPI_SWIGLU_) {
                    const int64_t n0 = bn * 64 + 32 * wn + 8 * g + 4 * (lane >> 5);
                    if (n0 >= p.Np) continue;
                    const int nv = (int)min<int64_t>(4, p.Np - n0);
                    float h[4];
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const float gt = acc[0][mi][4 * g + i], up = acc[1][mi][4 * g + i];
                        h[i] = gt / (1.0f + expf(-gt)) * up;
                    }
                    if (p.o32) store4<DT_F32>(p.o32, r * p.Np + n0, h, nv);
                    else store4<YDT>(p.y, r * p.Np + n0, h, nv, p.y_f16);
                } else {
#pragma unroll
                    for (int ni = 0; ni < 2; ni++) {
                        const int64_t n0 = bn * NT + 64 * wn + 32 * ni + 8 * g + 4 * (lane >> 5);
                        if (n0 >= p.N) continue;
                        const int nv = (int)min<int64_t>(4, p.N - n0);
                        float v[4] = {acc[ni][mi][4 * g], acc[ni][mi][4 * g + 1], acc[ni][mi][4 * g + 2], acc[ni][mi][4 * g + 3]};
                        if (p.o32) store4<DT_F32>(p.o32, r * p.Np + n0, v, nv);
                        else store4<YDT>(p.y, r * p.Np + n0, v, nv, p.y_f16);
                    }
                }
            }
        }
    }
}

// ---- test hook: per-group int32 dots from the staged tiles and the MFMA ----
// Same staging (sub-scales forced to 1) and fragment layout as mmq_kernel;
// one stage per q8_1 block, the 16-wide MFMA K steps give Q6_K's 16-groups.
template <int T>
__global__ __launch_bounds__(256) void mmq_dots_kernel(const uint8_t *__restrict__ W, int64_t N, int64_t K,
                                                       const _Float16 *__restrict__ xq, int64_t M, int64_t m_tiles,
                                                       int32_t *__restrict__ out) {
    __shared__ MmqSmem<T> sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t bm = (int64_t)blockIdx.x % m_tiles, bn = (int64_t)blockIdx.x / m_tiles;
    const int64_t row_bytes = K / Geom<T>::QK * Geom<T>::BYTES;
    if (tid < MT) {
        const int64_t m = bm * MT + tid;
        sm.xrow[tid] = m < M ? (int32_t)m : -1;
    } else {
        const int64_t n = bn * NT + tid - MT;
        sm.wrow[tid - MT] = n < N ? W + n * row_bytes : nullptr;
    }
    __syncthreads();
    constexpr int G = Geom<T>::G;
    const int64_t gpr = K / G;
    const int lr = lane & 31, kh = 8 * (lane >> 5);
    Stager<T, true> S;
    {
        const uint8_t *wr = sm.wrow[tid >> 1];
        const int32_t xr = sm.xrow[tid >> 1];
        S.init(wr ? wr : W, xq, nullptr, nullptr, K, xr >= 0 ? xr : 0);
    }
    for (int s = 0; s < (int)(K / KS); s++) {
        __syncthreads();
        S.load(s);
        S.store(sm, s);
        __syncthreads();
        const int buf = s & 1;
        v16f C[2][2];
        for (int a = 0; a < 2; a++) for (int b = 0; b < 2; b++) C[a][b] = v16f{};
        for (int kk = 0; kk < 2; kk++) {
            const int ko = 16 * kk + kh;
            if (G == 16) for (int a = 0; a < 2; a++) for (int b = 0; b < 2; b++) C[a][b] = v16f{};
            v8h bf[2];
            for (int mi = 0; mi < 2; mi++) bf[mi] = *reinterpret_cast<const v8h *>(&sm.B[buf][64 * wm + 32 * mi + lr][ko]);
            for (int x = 0; x < MmqSmem<T>::NA; x++) {
                v8h af[2];
                for (int ni = 0; ni < 2; ni++) af[ni] = *reinterpret_cast<const v8h *>(&sm.A[buf][x][64 * wn + 32 * ni + lr][ko]);
                for (int ni = 0; ni < 2; ni++)
                    for (int mi = 0; mi < 2; mi++)
                        C[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ni], bf[mi], C[ni][mi], 0, 0, 0);
            }
            if (G == 32 && kk == 0) continue;
            const int64_t grp = G == 16 ? ((int64_t)s * KS + 16 * kk) / 16 : (int64_t)s;
            for (int ni = 0; ni < 2; ni++)
                for (int mi = 0; mi < 2; mi++)
                    for (int e = 0; e < 16; e++) {
                        const int64_t n = bn * NT + 64 * wn + 32 * ni + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        const int64_t m = bm * MT + 64 * wm + 32 * mi + lr;
                        if (n >= N || m >= M) continue;
                        out[(m * N + n) * gpr + grp] = (int32_t)C[ni][mi][e];
                    }
        }
    }
}

// ---------------------------------------------------------------------------
template <int T>
static void launch_t(bool moe, int epi, int ydt, const MmqParams &p, hipStream_t s) {
    // routed: route tiles rounded up to a multiple of 8 (the XCD interleave); the
    // extra workgroups, like those past the device's tile count, exit at once
    const int64_t mt = moe ? (p.m_tiles + 7) / 8 * 8 : p.m_tiles;
    const int64_t ks = !moe && p.ksplit > 1 ? p.ksplit : 1;
    const dim3 g((unsigned)(mt * p.n_tiles * ks)), b(256);
#define GGQ_L(MOE, EPI, YDT) hipLaunchKernelGGL((mmq_kernel<T, MOE, EPI, YDT>), g, b, 0, s, p)
    if (!moe) {
        if (ydt == DT_F32) GGQ_L(false, EPI_NONE_, DT_F32); else GGQ_L(false, EPI_NONE_, DT_BF16);
    } else if (epi == EPI_SWIGLU_) {
        if (ydt == DT_F32) GGQ_L(true, EPI_SWIGLU_, DT_F32);
        else if (ydt == DT_BF16) GGQ_L(true, EPI_SWIGLU_, DT_BF16);
        else GGQ_L(true, EPI_SWIGLU_, DT_Q8_1);
    } else {
        if (ydt == DT_F32) GGQ_L(true, EPI_NONE_, DT_F32);
        else if (ydt == DT_BF16) GGQ_L(true, EPI_NONE_, DT_BF16);
        else GGQ_L(true, EPI_NONE_, DT_Q8_1);
    }
#undef GGQ_L
}

hipError_t launch_mmq(int t, bool moe, int epi, int ydt, const MmqParams &p, hipStream_t s) {
    if (p.m_tiles == 0 || p.n_tiles == 0) return hipSuccess;
    if (t == T_Q4_K) launch_t<T_Q4_K>(moe, epi, ydt, p, s);
    else if (t == T_Q6_K) launch_t<T_Q6_K>(moe, epi, ydt, p, s);
    else if (t == T_Q5_K) launch_t<T_Q5_K>(moe, epi, ydt, p, s);
    else if (t == T_Q8_0) launch_t<T_Q8_0>(moe, epi, ydt, p, s);
    else if (t == T_Q4_0) launch_t<T_Q4_0>(moe, epi, ydt, p, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mmq_dots(int t, const uint8_t *W, int64_t N, int64_t K, const _Float16 *xq, int64_t M,
                           int32_t *out, hipStream_t s) {
    const int64_t mt = (M + MT - 1) / MT, nt = (N + NT - 1) / NT;
    if (mt == 0 || nt == 0) return hipSuccess;
    const dim3 g((unsigned)(mt * nt)), b(256);
    if (t == T_Q4_K) hipLaunchKernelGGL(mmq_dots_kernel<T_Q4_K>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else if (t == T_Q6_K) hipLaunchKernelGGL(mmq_dots_kernel<T_Q6_K>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else if (t == T_Q5_K) hipLaunchKernelGGL(mmq_dots_kernel<T_Q5_K>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else if (t == T_Q8_0) hipLaunchKernelGGL(mmq_dots_kernel<T_Q8_0>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else if (t == T_Q4_0) hipLaunchKernelGGL(mmq_dots_kernel<T_Q4_0>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ggq
