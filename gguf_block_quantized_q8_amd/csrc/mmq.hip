// MMQ: tiled quantized matmul for prefill and routed experts, on fp16 MFMA
// with exact integer operands, every operand brought into LDS by DMA.
//
// Arithmetic.  Per 32-wide q8_1 block the weights' integer sub-scale times
// quant is an exact fp16 operand (Q4_K sc * nibble <= 945, Q5_K sc * value
// <= 1953, Q6_K sc * (q - 32) <= 2048 in magnitude when |sc| <= 64, else two
// exact parts; Q8_0 / Q4_0 the plain quant), the activation quants are exact
// fp16, and two v_mfma_f32_32x32x16_f16 sum the block's integer dot exactly
// in fp32 (every partial sum is an integer below 2^24).  One fma per output
// per block applies the activation scale d8 (P += C * d8); per 256-wide
// super-block the weight scale d is applied once (acc += P * d), and the
// Q4_K / Q5_K min term -dmin * sum_j m_j s8_j runs as a bf16 MFMA of the
// integer mins against the three exact bf16 parts of each s8.  Q8_0 / Q4_0
// carry their fp16 scale per 32-weight block: acc += C * (d8 * d) per block.
//
// Why fp16 and not int8 MFMA: measured on the inner loop alone
// (ggq_bench_inner_loop), int8 MFMA plus its exact per-block rescale
// (multiply by the sub-scale, convert, fma: three VALU per output per block)
// runs at about 0.8 POP/s, the fp16 form (one fma) at about 1.25 POP/s.
//
// Tiles: 128 weight rows x 256 activation rows per workgroup, one workgroup
// per CU, 8 waves of 64 x 64 (2 x 2 tiles of 32 x 32).  K advances one q8_1
// block (32) per stage.  Per stage s a workgroup
//   1. issues the LDS-DMA copies (buffer_load ... lds) of stage s + 2: the
//      activation quants in MFMA-fragment order; at a super-block start also
//      the whole super-block of every weight row (raw GGUF bytes) and the
//      block scales d8; mid super-block the min-term operand;
//   2. waits for its own copies of stage s + 1;
//   3. decodes stage s + 1's weights from the raw bytes its own wave copied
//      into the fp16 fragment layout (no wait on other waves' copies);
//   4. runs stage s's MFMAs and rescales from LDS;
//   5. meets one LDS-only barrier.
// Three activation slots, two decoded-weight slots and two raw super-block
// slots rotate; no global load is held in registers across a barrier.
#include <type_traits>
#include <utility>

#include "kernels.hpp"

namespace ggq {

namespace {

constexpr int NT = MMQ_NT;          // weight rows per tile
constexpr int MT = MMQ_MT;          // activation rows (routes) per tile
constexpr int NTHR = 512;           // 8 waves
constexpr int KS = 32;              // K per stage
constexpr int EPI_NONE_ = 0, EPI_SWIGLU_ = 1;

template <int T> constexpr bool kBlk32 = T == T_Q8_0 || T == T_Q4_0;   // fp16 scale per 32-weight block
template <int T> constexpr bool kMin = T == T_Q4_K || T == T_Q5_K;     // d * sc * q - dmin * m

// One row's super-block (256 weights, 8 stages): its bytes and the 16-byte
// pieces copied to cover it from the 16-byte boundary at or below its start
// (Q6_K super-blocks start at any even phase; the others at phase 0 when K %
// 256 == 0).
// PP: the row pitch of the LDS copy in pieces, P or more: 16 rows at a pitch of 4 PP
// dwords fall in 16 distinct LDS banks when 4 PP mod 64 is 4 times an odd number
// (Q6_K's 14 pieces give 56 dwords, 8 distinct banks and two-way conflicts in the
// decode's reads; 15 give 60: conflicts 35 % -> 15 % of LDS-active cycles).
template <int T> struct SbGeo;
template <> struct SbGeo<T_Q4_K> { static constexpr int B = 144, P = 9, PP = 9; };
template <> struct SbGeo<T_Q5_K> { static constexpr int B = 176, P = 11, PP = 11; };
template <> struct SbGeo<T_Q6_K> { static constexpr int B = 210, P = 14, PP = 15; };
template <> struct SbGeo<T_Q8_0> { static constexpr int B = 272, P = 17, PP = 17; };   // 8 blocks of 34
template <> struct SbGeo<T_Q4_0> { static constexpr int B = 144, P = 9, PP = 9; };     // 8 blocks of 18

// LDS-DMA instructions per wave for a super-block of its 16 rows.
template <int T> constexpr int NIRAW = (16 * SbGeo<T>::PP + 63) / 64;

// Dynamic LDS layout (bytes).  Fragment-ordered buffers hold 1 KB per MFMA
// operand fragment: lane l's 16 bytes at 16 * l (row or column l & 31, K
// values 8 * (l >> 5) .. + 8 of a 16-wide half).
template <int T> struct Lds {
    static constexpr int NA = T == T_Q6_K ? 2 : 1;                 // weight operand parts
    static constexpr int ACT = 0;                                  // [3][8 col groups][2 halves][1 KB]
    static constexpr int DEC = ACT + 3 * 16 * 1024;                // [2][NA][4 row groups][2 halves][1 KB]
    static constexpr int RAWSLOT = NT * SbGeo<T>::PP * 16;
    static constexpr int RAW = DEC + 2 * NA * 8 * 1024;            // [2][NT rows][PP pieces][16]
    static constexpr int D8 = RAW + 2 * RAWSLOT;                   // float [2 sb][8 blocks][MT]
    static constexpr int BMIN = D8 + 2 * 8 * MT * 4;               // [8][2][1 KB] bf16 min operand (min types)
    static constexpr int AMIN = BMIN + (kMin<T> ? 16 * 1024 : 0);  // [4][2][1 KB]
    static constexpr int WD = AMIN + (kMin<T> ? 8 * 1024 : 0);     // float [2][NT]: d by super-block (by stage for Q8_0 / Q4_0)
    static constexpr int WDM = WD + 2 * NT * 4;                    // float [2][NT]: dmin (min types)
    static constexpr int WOFF = WDM + (kMin<T> ? 2 * NT * 4 : 0);  // uint32 [NT]: row byte offset from the raw base
    static constexpr int XROW = WOFF + NT * 4;                     // int32 [MT]: activation row of each column (-1: none)
    static constexpr int ROUTE = XROW + MT * 4;                    // int32 [MT]: routed: route of each column
    static constexpr int FLAG = ROUTE + MT * 4;                    // int32 [2][8]: Q6_K rows of decode wave w need two parts
    static constexpr int TOTAL = FLAG + 64;
    static_assert(TOTAL <= 160 * 1024, "LDS");
};

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2v as_h2(uint32_t u) { return __builtin_bit_cast(h2v, u); }
__device__ __forceinline__ uint32_t h2_bits(h2v h) { return __builtin_bit_cast(uint32_t, h); }
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint8_t lds_u8;      // LDS bytes: ds_read / ds_write, never flat
template <class V> __device__ __forceinline__ V ld_lds(const lds_u8 *p) {
    return *(const __attribute__((address_space(3))) V *)p;
}
template <class V> __device__ __forceinline__ void st_lds(lds_u8 *p, V v) { *(__attribute__((address_space(3))) V *)p = v; }

extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(v4i rsrc, lds_u32 *lds, int size, int voffset, int soffset,
                                                           int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Buffer descriptor over [base, base + bytes) (bytes capped below 2^31):
// loads past the range return zeros without touching memory.
__device__ __forceinline__ v4i make_rsrc(const void *base, int64_t bytes) {
    struct { const void *p; uint32_t range; uint32_t cfg; } r = {
        base, (uint32_t)(bytes < 0 ? 0 : bytes < 0x7fffff00LL ? bytes : 0x7fffff00LL), 0x00020000u};
    v4i d = __builtin_bit_cast(v4i, r);
#pragma unroll
    for (int i = 0; i < 4; i++) d[i] = __builtin_amdgcn_readfirstlane(d[i]);
    return d;
}

// vmcnt(N) with N an immediate below 16.
template <int N> __device__ __forceinline__ void wait_vm_c() {
    static_assert(N >= 0 && N < 16, "vmcnt");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

template <class F, int... I>
__device__ __forceinline__ void static_for_(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in order
template <int N, class F> __device__ __forceinline__ void static_for(F &&f) {
    static_for_(f, std::make_integer_sequence<int, N>{});
}

// LDS-only workgroup barrier: this wave's LDS accesses are complete, then
// s_barrier; DMA copies in flight are not waited for (vmcnt is explicit).
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// 8 bytes at a 2-byte aligned LDS address, from aligned dword reads.
__device__ __forceinline__ v2i lds8(const lds_u8 *p) {
    const uint32_t a = (uint32_t)(uintptr_t)p;
    const lds_u8 *q = p - (a & 3);
    const uint32_t sh = a & 3;
    const uint32_t w0 = ld_lds<uint32_t>(q), w1 = ld_lds<uint32_t>(q + 4), w2 = ld_lds<uint32_t>(q + 8);
    return v2i{(int)__builtin_amdgcn_alignbyte(w1, w0, sh), (int)__builtin_amdgcn_alignbyte(w2, w1, sh)};
}
__device__ __forceinline__ uint32_t lds_u16(const lds_u8 *p) { return ld_lds<uint16_t>(p); }

// Q4_K / Q5_K: the 8 six-bit scales and mins of the 12 header bytes, one per byte.
__device__ __forceinline__ void q4k_pack(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t &sc_lo, uint32_t &sc_hi,
                                         uint32_t &mn_lo, uint32_t &mn_hi) {
    sc_lo = s0 & 0x3f3f3f3fu;
    mn_lo = s1 & 0x3f3f3f3fu;
    sc_hi = (s2 & 0x0f0f0f0fu) | ((s0 >> 2) & 0x30303030u);
    mn_hi = ((s2 >> 4) & 0x0f0f0f0fu) | ((s1 >> 2) & 0x30303030u);
}

// Four values (bytes of x, each < 2^11 - 1024) as fp16 pairs 1024 + byte, times sc, minus 1024 sc:
// sc * byte exactly (one rounding of an exact result).
__device__ __forceinline__ void bytes_to_h2(uint32_t x, h2v sc2, h2v off2, uint32_t &o0, uint32_t &o1) {
    o0 = h2_bits(__builtin_elementwise_fma(as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x07010600u)), sc2, off2));
    o1 = h2_bits(__builtin_elementwise_fma(as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x07030602u)), sc2, off2));
}

// Per-thread state of the weight decode: the thread decodes 8 weights (K
// values 8p .. 8p + 7 of each 32-wide block) of one tile row.
struct DecodeState {
    uint32_t s0, s1, s2, s3;   // Q4_K / Q5_K: packed scales lo, hi, mins lo, hi; Q6_K: the 16 int8 scales
    int need2;                 // Q6_K: this row has a sub-scale with |sc| > 64
    // select among loaded values (a select between member addresses would keep the state in scratch)
    __device__ __forceinline__ uint32_t w(int i) const {
        const uint32_t a = s0, b = s1, c = s2, d = s3;
        return i == 0 ? a : i == 1 ? b : i == 2 ? c : d;
    }
};

// Decode stage j (block j of the super-block) of one row into fp16 operand
// dwords o[0..3] (part 0) and, for Q6_K, o2[0..3] (part 1; zero unless the
// row needs two parts).  raw: this row's super-block bytes in LDS.  UNIT:
// every sub-scale 1 (test hook: raw integer dots).
template <int T, bool UNIT>
__device__ __forceinline__ void decode8(const lds_u8 *raw, int j, int p, const DecodeState st, uint32_t (&o)[4],
                                        uint32_t (&o2)[4]) {
    // branch-free in j: offsets, shifts and sub-scale fields are computed, not selected by branches
    if (T == T_Q4_K || T == T_Q5_K) {
        // phase-0 rows: the nibble bytes (and fifth bits) are 8-byte aligned
        const int c = j >> 1, sh = 4 * (j & 1);
        const v2i q = ld_lds<v2i>(raw + (T == T_Q4_K ? 16 : 48) + 32 * c + 8 * p);
        uint32_t x0 = ((uint32_t)q.x >> sh) & 0x0f0f0f0fu, x1 = ((uint32_t)q.y >> sh) & 0x0f0f0f0fu;
        if (T == T_Q5_K) {
            const v2i h = ld_lds<v2i>(raw + 16 + 8 * p);         // fifth bits: bit j of byte l
            x0 |= (((uint32_t)h.x >> j) & 0x01010101u) << 4;
            x1 |= (((uint32_t)h.y >> j) & 0x01010101u) << 4;
        }
        const int sc = UNIT ? 1 : (int)__builtin_amdgcn_ubfe(st.w(j >> 2), 8 * (j & 3), 8);
        const _Float16 scf = (_Float16)(float)sc, off = (_Float16)(float)(-1024 * sc);
        const h2v sc2 = {scf, scf}, off2 = {off, off};
        bytes_to_h2(x0, sc2, off2, o[0], o[1]);
        bytes_to_h2(x1, sc2, off2, o[2], o[3]);
    } else if (T == T_Q6_K) {
        const int hh = j >> 2, g = j & 3;
        const v2i ql = lds8(raw + 64 * hh + 32 * (g & 1) + 8 * p);
        const v2i qh = lds8(raw + 128 + 32 * hh + 8 * p);
        const int lsh = 4 * (g >> 1), hsh = 2 * g;
        uint32_t x[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const uint32_t l = (uint32_t)(i ? ql.y : ql.x), h = (uint32_t)(i ? qh.y : qh.x);
            x[i] = ((l >> lsh) & 0x0f0f0f0fu) | (((h >> hsh) & 0x03030303u) << 4);
        }
        // sub-scale of weights 16 * (2 * g + (p >> 1)) .. + 16 of this half
        const int si = 8 * hh + 2 * g + (p >> 1);
        const int sc = UNIT ? 1 : (int)(int8_t)__builtin_amdgcn_ubfe(st.w(si >> 2), 8 * (si & 3), 8);
        // q - 32 exactly: (1024 + q) - 1056; then times the sub-scale, in one or two exact parts
        const int shi = st.need2 ? (sc & ~15) : sc, slo = st.need2 ? (sc & 15) : 0;
        const _Float16 hf = (_Float16)(float)shi, lf = (_Float16)(float)slo, moff = (_Float16)-1056.0f;
        const h2v one = {(_Float16)1.0f, (_Float16)1.0f}, off2 = {moff, moff}, sh2 = {hf, hf}, sl2 = {lf, lf};
#pragma unroll
        for (int i = 0; i < 2; i++) {
            uint32_t v0, v1;
            bytes_to_h2(x[i], one, off2, v0, v1);              // q - 32 as fp16 pairs
            o[2 * i] = h2_bits(as_h2(v0) * sh2);
            o[2 * i + 1] = h2_bits(as_h2(v1) * sh2);
            o2[2 * i] = h2_bits(as_h2(v0) * sl2);
            o2[2 * i + 1] = h2_bits(as_h2(v1) * sl2);
        }
    } else if (T == T_Q8_0) {
        // q + 128 as a byte, read as fp16 1024 + byte, minus 1152
        const v2i q = lds8(raw + 34 * j + 2 + 8 * p);
        const h2v one = {(_Float16)1.0f, (_Float16)1.0f}, off2 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
        bytes_to_h2((uint32_t)q.x ^ 0x80808080u, one, off2, o[0], o[1]);
        bytes_to_h2((uint32_t)q.y ^ 0x80808080u, one, off2, o[2], o[3]);
    } else {                                                     // Q4_0: nibble - 8
        const v2i q = lds8(raw + 18 * j + 2 + 8 * (p & 1));
        const int sh = 4 * (p >> 1);
        const h2v one = {(_Float16)1.0f, (_Float16)1.0f}, off2 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
        bytes_to_h2(((uint32_t)q.x >> sh) & 0x0f0f0f0fu, one, off2, o[0], o[1]);
        bytes_to_h2(((uint32_t)q.y >> sh) & 0x0f0f0f0fu, one, off2, o[2], o[3]);
    }
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
    const int64_t per = total / 8;
    const int64_t t = b < 8 * per ? (b % 8) * per + b / 8 : b;
    const int64_t G = 8;
    const int64_t gsize = G * m_tiles;
    const int64_t grp = t / gsize, in = t % gsize;
    const int64_t gw = min<int64_t>(G, n_tiles - grp * G);
    bm = in / gw;
    bn = grp * G + in % gw;
}

// Routed output as q8_1 blocks, y[route][Np / 32] (Np % 32 == 0).  A block is
// 32 consecutive outputs of one route: two 16-row MFMA tiles of one column,
// rows 16 hh + 4 g + i held by lane c + 16 g (c: the column's lane, g = 0..3),
// so its amax and quant sum take two lane exchanges.  The values are those the
// plain epilogue would store (SwiGLU applied, rounded first to bf16 or fp16
// per p.q8_round), quantized as the q8_1 kernel does.
typedef __attribute__((address_space(3))) int32_t lds_i32;
template <int EPI>
__device__ __forceinline__ void store_q8_1(const MmqParams &p, const lds_i32 *xrow, const lds_i32 *route,
                                           const v4f (&acc)[4][4], int64_t bn, int tile_count, int wn, int wm,
                                           int lane) {
    const int g = lane >> 4;
    const int64_t bpr = p.Np / QK8_1;
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        const int col = 64 * wm + 16 * mt + (lane & 15);
        const bool live = col < tile_count && xrow[col] >= 0;
        const int64_t r = live ? route[col] : 0;
#pragma unroll
        for (int bi = 0; bi < (EPI == EPI_SWIGLU_ ? 1 : 2); bi++) {
            const int64_t n0 = EPI == EPI_SWIGLU_ ? bn * 64 + 32 * wn : bn * NT + 64 * wn + 32 * bi;
            float v[8];
            float amax = 0.0f;
#pragma unroll
            for (int hh = 0; hh < 2; hh++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    float o;
                    if (EPI == EPI_SWIGLU_) {
                        const float gt = acc[hh][mt][i], up = acc[hh + 2][mt][i];
                        o = gt / (1.0f + expf(-gt)) * up;
                    } else {
                        o = acc[2 * bi + hh][mt][i];
                    }
                    if (p.q8_round) o = from_16(f32_to_16(o, p.q8_round == 2), p.q8_round == 2);
                    v[4 * hh + i] = o;
                    amax = fmaxf(amax, fabsf(o));
                }
            amax = fmaxf(amax, __shfl_xor(amax, 16));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            float d = amax / 127.0f;
            uint32_t qw[2];
            int sum = 0;
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                uint32_t w = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int q = q8_1_quant(v[4 * hh + i], d, amax);
                    sum += q;
                    w |= (uint32_t)(q & 0xff) << (8 * i);
                }
                qw[hh] = w;
            }
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            if (amax == 0.0f) d = 0.0f;
            if (!live || n0 >= p.Np) continue;
            uint8_t *blk = static_cast<uint8_t *>(p.y) + (r * bpr + n0 / QK8_1) * Q8_1_BYTES;
#pragma unroll
            for (int hh = 0; hh < 2; hh++) *reinterpret_cast<uint32_t *>(blk + 8 + 16 * hh + 4 * g) = qw[hh];
            if (g == 0) *reinterpret_cast<float2 *>(blk) = make_float2(d, d * (float)sum);
        }
    }
}

}  // namespace

// grid: 1-D, m_tiles * n_tiles (* ksplit) workgroups of 512 threads (routed:
// m_tiles rounded up to 8); dynamic LDS Lds<T>::TOTAL bytes.
template <int T, bool MOE, int EPI, int YDT>
__global__ __launch_bounds__(NTHR, 1) void mmq_kernel(const MmqParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    lds_u8 *lds = (lds_u8 *)lds_raw;
    using L = Lds<T>;
    using G = SbGeo<T>;
    constexpr int NA = L::NA;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wn = wave & 1, wm = wave >> 1;                  // compute role: rows 64 wn.., columns 64 wm..
    __attribute__((address_space(3))) int32_t *xrow = (__attribute__((address_space(3))) int32_t *)(lds + L::XROW);
    __attribute__((address_space(3))) int32_t *route = (__attribute__((address_space(3))) int32_t *)(lds + L::ROUTE);
    __attribute__((address_space(3))) uint32_t *woff = (__attribute__((address_space(3))) uint32_t *)(lds + L::WOFF);

    int64_t bm, bn;
    int slice = 0;
    if (MOE) {
        // Workgroup b runs on XCD b mod 8.  That XCD takes the route tiles
        // t = b mod 8 (mod 8), each with all its weight tiles back to back, so a
        // route tile's activations are read into one L2 once.
        const int64_t b = blockIdx.x, x = b & 7, i = b >> 3;
        bm = 8 * (i / p.n_tiles) + x;
        bn = i % p.n_tiles;
    } else {
        const int64_t tiles = p.m_tiles * p.n_tiles;
        slice = p.ksplit > 1 ? (int)(blockIdx.x / tiles) : 0;
        tile_of(blockIdx.x - (int64_t)slice * tiles, p.m_tiles, p.n_tiles, bm, bn);
    }

    // ---- tile columns: activation rows (routed: of the tile's routes) ----
    int tile_count = MT;
    const uint8_t *W = p.W;
    int64_t xbase_row = 0, xrows = 0;                         // activation rows the descriptors cover
    if (MOE) {
        if (bm >= (int64_t)*p.ntiles) return;                 // workgroup-uniform
        const int4 tl = p.tiles[bm];
        W += (int64_t)tl.x * p.expert_stride;
        tile_count = tl.z;
        if (tid < MT) {
            int32_t xr = -1, r = -1;
            if (tid < tl.z) {
                r = p.perm[tl.y + tid];
                xr = p.x_per_route ? r : r / p.top_k;
            }
            xrow[tid] = xr;
            route[tid] = r;
        }
        xrows = p.x_rows;
    } else {
        tile_count = (int)min<int64_t>(MT, p.M - bm * MT);
        if (tid < MT) xrow[tid] = tid < tile_count ? tid : -1;
        xbase_row = bm * MT;
        xrows = min<int64_t>(MT, p.x_rows - xbase_row);      // tiled operand: whole 64-row groups
    }
    // ---- tile rows: weight rows, as byte offsets from the raw descriptor base ----
    // SwiGLU: tile row 64 w2 + 32 ni + rr is gate (ni = 0) or up (ni = 1) row
    // of output bn * 64 + 32 w2 + rr.  Rows past the matrix repeat the last row
    // (their results are never stored).
    const int64_t rb = p.row_bytes;
    const int64_t row0 = EPI == EPI_SWIGLU_ ? bn * 64 : bn * NT;
    const int64_t wbase_off = (row0 * rb) & ~(int64_t)15;
    const uint8_t *wbase = W + wbase_off;
    const int64_t wend_off = p.N * rb;                         // this matrix's (expert's) last byte + 1
    if (tid >= 256 && tid < 256 + NT) {
        const int tr = tid - 256;
        int64_t n;
        if (EPI == EPI_SWIGLU_) {
            const int w2 = tr >> 6, ni = (tr >> 5) & 1, rr = tr & 31;
            const int64_t gate = min<int64_t>(bn * 64 + 32 * w2 + rr, p.Np - 1);
            n = (ni ? p.Np : 0) + gate;
        } else {
            n = min<int64_t>(bn * NT + tr, p.N - 1);
        }
        woff[tr] = (uint32_t)(n * rb - wbase_off);
    }
    __syncthreads();

    const v4i act_rsrc = make_rsrc(p.xq + xbase_row * p.K, xrows * p.K * 2);
    const v4i d8_rsrc = make_rsrc(p.xd + xbase_row * (p.K / QK8_1), xrows * (p.K / QK8_1) * 4);
    const v4i min_rsrc = kMin<T> ? make_rsrc(p.xm + xbase_row * (p.K / 8), xrows * (p.K / 256) * 64) : act_rsrc;
    const v4i raw_rsrc = make_rsrc(wbase, wend_off - wbase_off);

    // this lane's activation fragments (2 per wave of the 16 per stage).  Dense (tiled
    // operand): fragment 2 gcol + kk of stage s is the 1 KB at ((gcol K/32 + s) 2 + kk) KB
    // of the tile; routed (row-major): 16 bytes of the lane's gathered row
    uint32_t aoff[2];
    const int64_t nblk = p.K / QK8_1;
#pragma unroll
    for (int f = 0; f < 2; f++) {
        const int fr = 2 * wave + f, gcol = fr >> 1, kk = fr & 1;
        if (MOE) {
            const int32_t xr = xrow[32 * gcol + (lane & 31)];
            aoff[f] = (uint32_t)((int64_t)(xr < 0 ? 0 : xr) * p.K * 2) + (uint32_t)((16 * kk + 8 * (lane >> 5)) * 2);
        } else {
            aoff[f] = (uint32_t)((gcol * nblk * 2 + kk) * 1024 + 16 * lane);
        }
    }
    constexpr uint32_t ASTEP = MOE ? KS * 2 : 2048;           // bytes from one stage to the next

    v4f acc[4][4], P[4][4];                                    // [16-row tile][16-column tile]
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) { acc[a][b] = v4f{}; P[a][b] = v4f{}; }
    // 16 x 16 tiles: lane l holds column l & 15 and rows 4 fg .. + 4; its operand
    // fragments start at foff in a 32-row fragment group (plus 256 for the upper 16 rows)
    const int fg = lane >> 4;
    const uint32_t foff = (fg >> 1) * 1024 + 16 * ((fg & 1) * 32 + (lane & 15));

    const int nst_all = (int)(p.K / KS), per = nst_all / (!MOE && p.ksplit > 1 ? p.ksplit : 1);
    const int s0 = slice * per, nst = s0 + per;
    const bool live = 64 * wm < tile_count;                   // this wave's columns are not all empty
    const int lr = lane & 31;
    // decode role: rows 16 wave + (lane & 15), K values 8 pd .. + 8 of each block
    const int drow = 16 * wave + (lane & 15), pd = lane >> 4;
    DecodeState st{};
    // Q6_K: a matrix that ends 2 bytes past a 4-byte boundary has its last dword (the
    // last row's last d) outside the copies' range, where it lands as zero; the thread
    // decoding that row reads those two bytes here, before any copy is in flight, so
    // no wait on loads is needed inside the pipeline
    uint32_t dlast = 0;
    bool dpatch = false;
    if (T == T_Q6_K && (wend_off & 3) == 2) {
        const int64_t rend = (int64_t)woff[drow] + wbase_off + (p.K / 256) * G::B;
        if (rend == wend_off) {
            dpatch = true;
            dlast = *reinterpret_cast<const uint16_t *>(W + wend_off - 2);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt(0)
    }

    // ---- per stage: the copies two stages ahead, the weight decode one stage ahead, the
    // MFMAs of the current stage.  A stage issues two LDS-DMA instructions per wave (its
    // activations); the first stage of a super-block also issues that super-block's min
    // operand and the next one's raw bytes and d8.  Wait counts are immediates. ----
    const uint32_t my_woff = woff[drow];
    const lds_u8 *my_raw = lds + L::RAW + (16 * wave + (lane & 15)) * G::PP * 16;

    auto issue_act = [&](int s, int slot) {
#pragma unroll
        for (int f = 0; f < 2; f++) {
            const int fr = 2 * wave + f;
            llvm_amdgcn_raw_buffer_load_lds(act_rsrc, (lds_u32 *)(lds + L::ACT + (slot * 16 + fr) * 1024), 16,
                                            (int)(aoff[f] + (uint32_t)s * ASTEP), 0, 0, 0);
        }
    };
    // raw super-block sb of this wave's 16 rows, instruction i: slots P = 64 i + lane
    // (row P / G::PP, piece P % G::PP); lanes past the wave's pieces, and the pitch's
    // spare pieces, copy nothing (an exec-masked lane writes no LDS: the rest of that
    // kilobyte belongs to the next wave's rows); lane 0 is always active
    auto issue_raw = [&](int sb, int i) {
        lds_u8 *slot = lds + L::RAW + (sb & 1) * L::RAWSLOT + 16 * wave * G::PP * 16;
        const int P_ = 64 * i + lane;
        const int rl = P_ / G::PP, q = P_ - rl * G::PP;
        if (P_ < 16 * G::PP && q < G::P) {
            const uint32_t start = woff[16 * wave + rl] + (uint32_t)sb * G::B;
            const uint32_t off = (start & ~15u) + 16u * (uint32_t)q;
            llvm_amdgcn_raw_buffer_load_lds(raw_rsrc, (lds_u32 *)(slot + 1024 * i), 16, (int)off, 0, 0, 0);
        }
    };
    // block scales d8 of super-block sb: wave w copies block w of columns 64 i .. + 64
    auto issue_d8 = [&](int sb, int i) {
        uint32_t off;
        if (MOE) {
            const int32_t xr = xrow[64 * i + lane];
            off = (uint32_t)(((int64_t)(xr < 0 ? 0 : xr) * nblk + 8 * sb + wave) * 4);
        } else {
            off = (uint32_t)(((i * nblk + 8 * sb + wave) * 64 + lane) * 4);
        }
        llvm_amdgcn_raw_buffer_load_lds(d8_rsrc, (lds_u32 *)(lds + L::D8 + (((sb & 1) * 8 + wave) * MT + 64 * i) * 4),
                                        4, (int)off, 0, 0, 0);
    };
    // min-term operand of super-block sb, fragment 2 wave + f
    auto issue_min = [&](int sb, int f) {
        const int fr = 2 * wave + f, gcol = fr >> 1, kk = fr & 1;
        uint32_t off;
        if (MOE) {
            const int32_t xr = xrow[32 * gcol + lr];
            off = (uint32_t)(((int64_t)(xr < 0 ? 0 : xr) * (p.K / 256) + sb) * 64) + (uint32_t)((16 * kk + 8 * (lane >> 5)) * 2);
        } else {
            off = (uint32_t)(((gcol * (p.K / 256) + sb) * 2 + kk) * 1024 + 16 * lane);
        }
        llvm_amdgcn_raw_buffer_load_lds(min_rsrc, (lds_u32 *)(lds + L::BMIN + fr * 1024), 16, (int)off, 0, 0, 0);
    };
    // everything a super-block needs besides the activations, for the stages of super-block
    // sb: its min-term operand (read at its end) and the next super-block's raw bytes and d8
    // (landed long before the decode of that super-block's first stage)
    constexpr int NSB = NIRAW<T> + MT / 64 + (kMin<T> ? 2 : 0);   // copies per wave per super-block
    auto issue_sb = [&](int sb) {
        if (kMin<T>) {
            issue_min(sb, 0);
            issue_min(sb, 1);
        }
#pragma unroll
        for (int i = 0; i < NIRAW<T>; i++) issue_raw(sb + 1, i);
#pragma unroll
        for (int i = 0; i < MT / 64; i++) issue_d8(sb + 1, i);
    };

    // decode stage s (position j) of this thread's row into the fp16 fragment slot s & 1
    auto decode = [&](int s) {
        const int j = s & 7, sb = s >> 3;
        const lds_u8 *raw = my_raw + (sb & 1) * L::RAWSLOT + (T == T_Q6_K ? ((my_woff + (uint32_t)sb * G::B) & 15u) : 0u);
        if (j == 0 && !kBlk32<T>) {
            // super-block header: scales, mins, d (Q6_K: whether two operand parts are needed)
            float d, dmin = 0.0f;
            if (kMin<T>) {
                const v4i hd = ld_lds<v4i>(raw);
                const uint32_t h0 = (uint32_t)hd.x;
                q4k_pack((uint32_t)hd.y, (uint32_t)hd.z, (uint32_t)hd.w, st.s0, st.s1, st.s2, st.s3);
                d = fp16_bits_to_f32(h0 & 0xffffu);
                dmin = fp16_bits_to_f32(h0 >> 16);
            } else {
                const v2i a = lds8(raw + 192), b = lds8(raw + 200);
                st.s0 = (uint32_t)a.x; st.s1 = (uint32_t)a.y; st.s2 = (uint32_t)b.x; st.s3 = (uint32_t)b.y;
                int need = 0;
#pragma unroll
                for (int k = 0; k < 16; k++) {
                    const int v = (int)(int8_t)__builtin_amdgcn_ubfe(st.w(k >> 2), 8 * (k & 3), 8);
                    need |= v > 64 || v < -64;
                }
                st.need2 = need;
                uint32_t dbits = lds_u16(raw + 208);
                if (dpatch && sb == (int)(p.K / 256) - 1) dbits = dlast;
                d = fp16_bits_to_f32(dbits);
                const uint64_t any = __ballot(need);
                if (lane == 0) st_lds<int32_t>(lds + L::FLAG + ((sb & 1) * 8 + wave) * 4, any != 0);
            }
            if (pd == 0) {
                st_lds<float>(lds + L::WD + ((sb & 1) * NT + drow) * 4, d);
                if (kMin<T>) st_lds<float>(lds + L::WDM + ((sb & 1) * NT + drow) * 4, dmin);
            }
        }
        uint32_t o[4], o2[4];
        decode8<T, false>(raw, j, pd, st, o, o2);
        const int ni = drow >> 5, kk = pd >> 1, lp = (drow & 31) + 32 * (pd & 1);
        lds_u8 *dst = lds + L::DEC + ((s & 1) * NA * 8 + ni * 2 + kk) * 1024 + 16 * lp;
        st_lds<v4i>(dst, v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]});
        if (NA == 2) st_lds<v4i>(dst + 8 * 1024, v4i{(int)o2[0], (int)o2[1], (int)o2[2], (int)o2[3]});
        if (kBlk32<T> && pd == 0)
            st_lds<float>(lds + L::WD + ((s & 1) * NT + drow) * 4, fp16_bits_to_f32(lds_u16(raw + (T == T_Q8_0 ? 34 : 18) * j)));
        if (kMin<T> && j == 1) {
            // the min operand of this row (bf16 integer mins, each 3 times, entries 24..31 zero),
            // written one stage into the super-block: the previous one's was read at its end
            uint32_t w[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; e2++) {
                uint32_t pair = 0;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int e = 8 * pd + 2 * e2 + h, g = e / 3;
                    const uint32_t m = e < 24 ? __builtin_amdgcn_ubfe(st.w(2 + (g >> 2)), 8 * (g & 3), 8) : 0u;
                    pair |= (uint32_t)bf16_trunc_bits((float)m) << (16 * h);
                }
                w[e2] = pair;
            }
            st_lds<v4i>(lds + L::AMIN + (ni * 2 + kk) * 1024 + 16 * lp, v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]});
        }
    };

    // stage s (activation slot aslot): MFMAs and rescale of this wave's 64 x 64
    // Stage compute on 16 x 16 x 32 MFMAs: one instruction covers a whole q8_1 block of
    // a 16 x 16 tile, so each tile's rescale is independent of the next tile's MFMA.  The
    // staging buffers keep the 32-row fragment layout (a 32-row group of one stage is two
    // 1 KB halves kk of 16 K values; lane l of half kk holds row l & 31, K values
    // 16 kk + 8 (l >> 5) .. + 8); a 16 x 16 x 32 operand needs in lane l row 16 hh + (l & 15)
    // and 8 consecutive K values, group l >> 4: found at foff + 256 hh.  Weight and
    // activation operands use the same K order, so the dot is the block's.
    auto compute = [&](int s, int aslot) {
        const int j = s & 7, sb = s >> 3;
        const lds_u8 *act = lds + L::ACT + aslot * 16 * 1024 + 2 * wm * 2048 + foff;
        const lds_u8 *dec = lds + L::DEC + (s & 1) * NA * 8 * 1024 + 2 * wn * 2048 + foff;
        const lds_u8 *d8t = lds + L::D8 + (((sb & 1) * 8 + j) * MT + 64 * wm + (lane & 15)) * 4;
        float d8[4];
        v8h bf[4];
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            d8[mt] = ld_lds<float>(d8t + 64 * mt);
            bf[mt] = ld_lds<v8h>(act + (mt >> 1) * 2048 + (mt & 1) * 256);
        }
        bool two[2] = {false, false};
        if (NA == 2) {
            const lds_u8 *fl = lds + L::FLAG + (sb & 1) * 32;
#pragma unroll
            for (int ni = 0; ni < 2; ni++) {
                const int g4 = 2 * (2 * wn + ni);                   // decode waves of this 32-row group
                two[ni] = (ld_lds<int32_t>(fl + 4 * g4) | ld_lds<int32_t>(fl + 4 * g4 + 4)) != 0;
            }
        }
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
            const lds_u8 *a = dec + (nt >> 1) * 2048 + (nt & 1) * 256;
            const v8h af = ld_lds<v8h>(a);
            v4f C[4];
#pragma unroll
            for (int mt = 0; mt < 4; mt++) C[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[mt], v4f{}, 0, 0, 0);
            if (NA == 2 && two[nt >> 1]) {
                const v8h af2 = ld_lds<v8h>(a + 8 * 1024);
#pragma unroll
                for (int mt = 0; mt < 4; mt++) C[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af2, bf[mt], C[mt], 0, 0, 0);
            }
            if (kBlk32<T>) {
                // the block's weight scale per row: rows 16 nt + 4 (l >> 4) + i of the wave's 64
                const v4f w4 = ld_lds<v4f>(lds + L::WD + ((s & 1) * NT + 64 * wn + 16 * nt + 4 * fg) * 4);
#pragma unroll
                for (int mt = 0; mt < 4; mt++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[nt][mt][i] = __builtin_fmaf(C[mt][i], d8[mt] * w4[i], acc[nt][mt][i]);
            } else {
                // P holds zeros at a super-block's first block
#pragma unroll
                for (int mt = 0; mt < 4; mt++)
#pragma unroll
                    for (int i = 0; i < 4; i++) P[nt][mt][i] = __builtin_fmaf(C[mt][i], d8[mt], P[nt][mt][i]);
            }
        }
        if (j == 7 && !kBlk32<T>) {
            // end of the super-block: acc += P * d (- dmin * min term), and P restarts at zero
            const lds_u8 *wd = lds + L::WD + ((sb & 1) * NT + 64 * wn + 4 * fg) * 4;
            const lds_u8 *wdm = lds + L::WDM + ((sb & 1) * NT + 64 * wn + 4 * fg) * 4;
            v8bf bmv[4];
            if (kMin<T>)
#pragma unroll
                for (int mt = 0; mt < 4; mt++)
                    bmv[mt] = ld_lds<v8bf>(lds + L::BMIN + 2 * wm * 2048 + foff + (mt >> 1) * 2048 + (mt & 1) * 256);
#pragma unroll
            for (int nt = 0; nt < 4; nt++) {
                v4f Q[4] = {v4f{}, v4f{}, v4f{}, v4f{}};
                if (kMin<T>) {
                    const v8bf am = ld_lds<v8bf>(lds + L::AMIN + 2 * wn * 2048 + foff + (nt >> 1) * 2048 + (nt & 1) * 256);
#pragma unroll
                    for (int mt = 0; mt < 4; mt++) Q[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bmv[mt], v4f{}, 0, 0, 0);
                }
                const v4f d4 = ld_lds<v4f>(wd + 64 * nt);
                v4f m4 = {0.f, 0.f, 0.f, 0.f};
                if (kMin<T>) m4 = ld_lds<v4f>(wdm + 64 * nt);
#pragma unroll
                for (int mt = 0; mt < 4; mt++) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        acc[nt][mt][i] = __builtin_fmaf(P[nt][mt][i], d4[i], acc[nt][mt][i]);
                        if (kMin<T>) acc[nt][mt][i] = __builtin_fmaf(Q[mt][i], -m4[i], acc[nt][mt][i]);
                    }
                    P[nt][mt] = v4f{};
                }
            }
        }
    };

    // ---- pipeline ----
    // prologue: the first super-block and the first two stages' activations, then the
    // first stage's decode
    {
        const int sb0 = s0 >> 3;
#pragma unroll
        for (int i = 0; i < NIRAW<T>; i++) issue_raw(sb0, i);
#pragma unroll
        for (int i = 0; i < MT / 64; i++) issue_d8(sb0, i);
        issue_act(s0, s0 % 3);
        issue_act(s0 + 1, (s0 + 1) % 3);
        wait_vm_c<2>();                                        // all but stage s0 + 1's activations
        decode(s0);
        lds_sync();
    }
    int aslot = s0 % 3;                                        // activation slot of stage s
    // Iteration s: copies of stage s + 2 (and at a super-block start that super-block's
    // burst), decode of stage s + 1, MFMAs of stage s, then the wait for this wave's copies
    // issued before this iteration (stage s + 1's activations, everything older) and one
    // barrier.  So a copy has the rest of its iteration and the whole next one to land; a
    // decode reads raw bytes issued at least seven iterations earlier; a compute reads
    // activations that every wave waited for before the previous barrier.
#pragma unroll 1
    for (int s = s0; s < nst; s++) {
        const int j = s & 7, sb = s >> 3;
        // stage s + 2 (its slot is stage s - 1's, read before the last barrier); near the end
        // these copies (and the last super-block's burst) run past the slice and are never read
        issue_act(s + 2, aslot == 0 ? 2 : aslot - 1);
        if (j == 0) issue_sb(sb);
        // the two waves of a SIMD (w and w + 4) take the stage's two phases in opposite
        // orders, so one's MFMAs and rescales overlap the other's decode (the phases touch
        // different LDS slots: decode writes slot s + 1, compute reads slot s)
        if (wave < 4) {
            if (live) compute(s, aslot);
            if (s + 1 < nst) decode(s + 1);
        } else {
            if (s + 1 < nst) decode(s + 1);
            if (live) compute(s, aslot);
        }
        if (j == 0) wait_vm_c<2 + NSB>();                      // this wave's copies before this iteration have landed
        else wait_vm_c<2>();
        lds_sync();
        aslot = aslot == 2 ? 0 : aslot + 1;
    }
    wait_vm_c<0>();                                            // no copy outlives the workgroup

    // ---- epilogue ----
    // 16-bit outputs go through LDS: each column's rows of this tile (128, or 64 SwiGLU
    // outputs) are staged contiguously, then written as whole 16-byte pieces, 256 (128)
    // contiguous bytes per column, rather than 8-byte pieces from the MFMA layout
    if (YDT == DT_BF16 && (MOE || p.ksplit == 1)) {
        constexpr int RW = EPI == EPI_SWIGLU_ ? 64 : NT;        // output rows of one column here
        constexpr int PITCH = RW * 2 + 16;                      // staged bytes per column (16-byte aligned)
        static_assert(MT * PITCH <= L::WOFF, "staging overlaps the tile tables");
        const bool hf = p.y_f16;
        __syncthreads();                                        // every wave is past its last LDS read
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
            lds_u8 *cst = lds + (64 * wm + 16 * mt + (lane & 15)) * PITCH;
#pragma unroll
            for (int nt = 0; nt < (EPI == EPI_SWIGLU_ ? 2 : 4); nt++) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    if (EPI == EPI_SWIGLU_) {
                        const float gt = acc[nt][mt][i], up = acc[nt + 2][mt][i];
                        v[i] = gt / (1.0f + expf(-gt)) * up;
                    } else {
                        v[i] = acc[nt][mt][i];
                    }
                }
                const int row = (EPI == EPI_SWIGLU_ ? 32 : 64) * wn + 16 * nt + 4 * fg;
                st_lds<v2i>(cst + 2 * row, v2i{(int)(f32_to_16(v[0], hf) | (f32_to_16(v[1], hf) << 16)),
                                                (int)(f32_to_16(v[2], hf) | (f32_to_16(v[3], hf) << 16))});
            }
        }
        __syncthreads();
        constexpr int LPC = RW / 8;                             // lanes per column, 8 values each
        const int64_t row0 = EPI == EPI_SWIGLU_ ? bn * 64 : bn * NT;
        const int64_t nrows = MOE ? p.Np : p.N;
        const int nvalid = (int)min<int64_t>(RW, nrows - row0);
        uint16_t *dst0 = static_cast<uint16_t *>(MOE && p.oroute ? p.oroute : p.y);
        const int64_t ld = MOE ? p.Np : p.ldy;
        const bool vec = (ld % 8) == 0;
#pragma unroll 1
        for (int c = tid / LPC; c < MT; c += NTHR / LPC) {
            if (c >= tile_count) break;
            const int32_t xr = xrow[c];
            const int e0 = 8 * (tid % LPC);
            if (xr < 0 || e0 >= nvalid) continue;
            const int64_t orow = MOE ? (int64_t)route[c] : xbase_row + xr;
            uint16_t *d = dst0 + orow * ld + row0 + e0;
            const v4i v = ld_lds<v4i>(lds + c * PITCH + 2 * e0);
            if (vec && e0 + 8 <= nvalid) {
                *reinterpret_cast<v4i *>(d) = v;
            } else {
                const int n = min(8, nvalid - e0);
                for (int i = 0; i < n; i++) d[i] = (uint16_t)((uint32_t)v[i >> 1] >> (16 * (i & 1)));
            }
        }
        return;
    }
    if (YDT == DT_Q8_1) {
        store_q8_1<EPI>(p, xrow, route, acc, bn, tile_count, wn, wm, lane);
        return;
    }
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        const int col = 64 * wm + 16 * mt + (lane & 15);
        if (col >= tile_count) continue;
        const int32_t xr = xrow[col];
        if (xr < 0) continue;
        if (!MOE) {
            const int64_t m = xbase_row + xr;
#pragma unroll
            for (int nt = 0; nt < 4; nt++) {
                const int64_t n0 = bn * NT + 64 * wn + 16 * nt + 4 * fg;
                if (n0 >= p.N) continue;
                const int nv = (int)min<int64_t>(4, p.N - n0);
                float v[4] = {acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]};
                if (p.ksplit > 1) store4<DT_F32>(p.part, ((int64_t)slice * p.M + m) * p.N + n0, v, nv);
                else store4<YDT>(p.y, m * p.ldy + n0, v, nv, p.y_f16);
            }
        } else {
            const int64_t r = route[col];
            if (EPI == EPI_SWIGLU_) {
                // tiles 0, 1 hold gate rows, tiles 2, 3 the up rows of the same outputs
#pragma unroll
                for (int nt = 0; nt < 2; nt++) {
                    const int64_t n0 = bn * 64 + 32 * wn + 16 * nt + 4 * fg;
                    if (n0 >= p.Np) continue;
                    const int nv = (int)min<int64_t>(4, p.Np - n0);
                    float h[4];
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const float gt = acc[nt][mt][i], up = acc[nt + 2][mt][i];
                        h[i] = gt / (1.0f + expf(-gt)) * up;
                    }
                    if (p.oroute) store4<YDT>(p.oroute, r * p.Np + n0, h, nv, p.y_f16);
                    else store4<YDT>(p.y, r * p.Np + n0, h, nv, p.y_f16);
                }
            } else {
#pragma unroll
                for (int nt = 0; nt < 4; nt++) {
                    const int64_t n0 = bn * NT + 64 * wn + 16 * nt + 4 * fg;
                    if (n0 >= p.N) continue;
                    const int nv = (int)min<int64_t>(4, p.N - n0);
                    float v[4] = {acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]};
                    if (p.oroute) store4<YDT>(p.oroute, r * p.Np + n0, v, nv, p.y_f16);
                    else store4<YDT>(p.y, r * p.Np + n0, v, nv, p.y_f16);
                }
            }
        }
    }
}

// ---- test hook: per-group int32 dots from the same weight decode and MFMA ----
// One workgroup of 64 threads per (32 weight rows, 32 activation rows).  Each
// thread copies its row's super-block into LDS, decodes its 8 weights per
// block with decode8 (sub-scales 1) straight into an MFMA A fragment, reads
// the planar activation quants as the B fragment, and the two
// v_mfma_f32_32x32x16_f16 of a block give the raw integer dot (Q6_K: one per
// 16-wide half, its 16-weight group).
template <int T>
__global__ __launch_bounds__(64) void mmq_dots_kernel(const uint8_t *__restrict__ W, int64_t N, int64_t K,
                                                      const _Float16 *__restrict__ xq, int64_t M, int64_t m_tiles,
                                                      int32_t *__restrict__ out) {
    using G = SbGeo<T>;
    // rows 16-byte aligned at phase 0, as in the production kernel's Q4_K / Q5_K rows; one
    // spare row: the decode's aligned dword reads run up to 3 bytes past a row's last byte
    constexpr int RS = G::P * 16;
    __shared__ __attribute__((aligned(16))) uint8_t raw_s[33 * RS];
    lds_u8 *raw = (lds_u8 *)&raw_s[0];
    const int lane = threadIdx.x;
    const int64_t bm = (int64_t)blockIdx.x % m_tiles, bn = (int64_t)blockIdx.x / m_tiles;
    const int64_t rb = K / Geom<T>::QK * Geom<T>::BYTES;
    constexpr int GL = Geom<T>::G;
    const int64_t gpr = K / GL;
    const int r = lane & 31, h = lane >> 5;
    const int64_t n = min<int64_t>(bn * 32 + r, N - 1), m = min<int64_t>(bm * 32 + r, M - 1);
    DecodeState st{};
    for (int64_t sb = 0; sb < K / 256; sb++) {
        __syncthreads();
        const uint8_t *src = W + n * rb + sb * G::B;
        for (int b = h; b < G::B; b += 2) raw[r * RS + b] = src[b];
        __syncthreads();
        for (int j = 0; j < 8; j++) {
            v8h af[2], bf[2];
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                uint32_t o[4], o2[4];
                decode8<T, true>(raw + r * RS, j, 2 * kk + h, st, o, o2);
                af[kk] = __builtin_bit_cast(v8h, v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]});
                bf[kk] = *reinterpret_cast<const v8h *>(xq + m * K + sb * 256 + 32 * j + 16 * kk + 8 * h);
            }
            v16f C[2];
            C[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[0], bf[0], v16f{}, 0, 0, 0);
            if (GL == 16) C[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[1], bf[1], v16f{}, 0, 0, 0);
            else C[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[1], bf[1], C[0], 0, 0, 0);
            const int64_t col = bm * 32 + r;
#pragma unroll
            for (int half = 0; half < (GL == 16 ? 2 : 1); half++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int64_t row = bn * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                    if (row >= N || col >= M) continue;
                    const int64_t grp = GL == 16 ? (sb * 256 + 32 * j + 16 * half) / 16 : sb * 8 + j;
                    out[(col * N + row) * gpr + grp] = (int32_t)C[half][e];
                }
        }
    }
}

// ---------------------------------------------------------------------------
template <int T>
static hipError_t launch_t(bool moe, int epi, int ydt, const MmqParams &p, hipStream_t s) {
    // routed: route tiles rounded up to a multiple of 8 (the XCD interleave); the
    // extra workgroups, like those past the device's tile count, exit at once
    const int64_t mt = moe ? (p.m_tiles + 7) / 8 * 8 : p.m_tiles;
    const int64_t ks = !moe && p.ksplit > 1 ? p.ksplit : 1;
    const dim3 g((unsigned)(mt * p.n_tiles * ks)), b(NTHR);
    const size_t lds = Lds<T>::TOTAL;
#define GGQ_L(MOE, EPI, YDT)                                                                                \
    {                                                                                                       \
        auto k = mmq_kernel<T, MOE, EPI, YDT>;                                                              \
        static bool lds_set = false;                  /* once per instantiation (per process) */            \
        if (!lds_set) {                                                                                     \
            hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
            if (e != hipSuccess) return e;                                                                  \
            lds_set = true;                                                                                 \
        }                                                                                                   \
        hipLaunchKernelGGL(k, g, b, lds, s, p);                                                             \
    }
    if (!moe) {
        if (ydt == DT_F32) GGQ_L(false, EPI_NONE_, DT_F32) else GGQ_L(false, EPI_NONE_, DT_BF16)
    } else if (epi == EPI_SWIGLU_) {
        if (ydt == DT_F32) GGQ_L(true, EPI_SWIGLU_, DT_F32)
        else if (ydt == DT_BF16) GGQ_L(true, EPI_SWIGLU_, DT_BF16)
        else GGQ_L(true, EPI_SWIGLU_, DT_Q8_1)
    } else {
        if (ydt == DT_F32) GGQ_L(true, EPI_NONE_, DT_F32)
        else if (ydt == DT_BF16) GGQ_L(true, EPI_NONE_, DT_BF16)
        else GGQ_L(true, EPI_NONE_, DT_Q8_1)
    }
#undef GGQ_L
    return hipGetLastError();
}

hipError_t launch_mmq(int t, bool moe, int epi, int ydt, const MmqParams &p, hipStream_t s) {
    if (p.m_tiles == 0 || p.n_tiles == 0) return hipSuccess;
    if (t == T_Q4_K) return launch_t<T_Q4_K>(moe, epi, ydt, p, s);
    if (t == T_Q6_K) return launch_t<T_Q6_K>(moe, epi, ydt, p, s);
    if (t == T_Q5_K) return launch_t<T_Q5_K>(moe, epi, ydt, p, s);
    if (t == T_Q8_0) return launch_t<T_Q8_0>(moe, epi, ydt, p, s);
    if (t == T_Q4_0) return launch_t<T_Q4_0>(moe, epi, ydt, p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_mmq_dots(int t, const uint8_t *W, int64_t N, int64_t K, const _Float16 *xq, int64_t M,
                           int32_t *out, hipStream_t s) {
    const int64_t mt = (M + 31) / 32, nt = (N + 31) / 32;
    if (mt == 0 || nt == 0) return hipSuccess;
    const dim3 g((unsigned)(mt * nt)), b(64);
    if (t == T_Q4_K) hipLaunchKernelGGL(mmq_dots_kernel<T_Q4_K>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else if (t == T_Q6_K) hipLaunchKernelGGL(mmq_dots_kernel<T_Q6_K>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else if (t == T_Q5_K) hipLaunchKernelGGL(mmq_dots_kernel<T_Q5_K>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else if (t == T_Q8_0) hipLaunchKernelGGL(mmq_dots_kernel<T_Q8_0>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else if (t == T_Q4_0) hipLaunchKernelGGL(mmq_dots_kernel<T_Q4_0>, g, b, 0, s, W, N, K, xq, M, mt, out);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ggq
