// MMVQ: quantized matrix x few-vectors, for small batches (decode).
//
// HBM-bound on the weights, so every weight byte is read exactly once and the
// reads are fully coalesced:
//  - each wave owns a few consecutive rows per iteration and copies their
//    bytes into a private LDS region with buffer_load_dwordx4 ... lds: 64
//    lanes x 16 B = one contiguous 1 KB span per instruction, straight into
//    LDS without passing through registers; the buffer descriptor's range
//    stops the copy at the last weight byte (no over-read);
//  - the activations (a few KB) are quantized to q8_1 (or copied, when given
//    pre-quantized) into LDS once per workgroup, in the kernel prologue, while
//    the first weight copy is in flight;
//  - lanes then decode 16-byte "units" of the GGUF blocks from LDS (Q4_K: one
//    16 B quant chunk + the block header; Q6_K: 48 B of ql/qh for 64 weights;
//    Q8_0: one 34 B block), take int8 dots with v_dot4 against the q8_1
//    quants, apply the scales per group in fp32, and reduce each row across
//    its lane segment with cross-lane shuffles.
// Rows too long to stage are read straight from global memory by the same
// unit code.  The routed form (mul_mat_id for small token counts) runs the same
// kernel per (expert, group of routes), so an expert's weights are read once
// however many of the group's tokens route to it.
#include "kernels.hpp"

namespace ggq {

constexpr int EPI_NONE = 0, EPI_SWIGLU = 1;

// ---- byte access in a given address space (1 = global, 3 = LDS) ----
template <int AS>
struct Mem {
    typedef const uint8_t __attribute__((address_space(AS))) *bp;
    typedef const uint16_t __attribute__((address_space(AS))) *hp;
    typedef const uint32_t __attribute__((address_space(AS))) *wp;
    __device__ static uint32_t u16(bp p) { return *(hp)p; }
    __device__ static uint32_t u32(bp p) { return *(wp)p; }                       // 4-byte aligned
    __device__ static v4i v16(bp p) {                                               // 4-byte aligned
        wp w = (wp)p;
        return v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
    // 16 bytes at a 2-byte aligned address: touches [p, p+16) or [p-2, p+16).
    __device__ static v4i a2_16(bp p) {
        if (reinterpret_cast<uintptr_t>(p) & 2) {
            wp w = (wp)(p - 2);
            const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3], w4 = u16(p + 14);
            return v4i{(int)__builtin_amdgcn_alignbyte(w1, w0, 2), (int)__builtin_amdgcn_alignbyte(w2, w1, 2),
                       (int)__builtin_amdgcn_alignbyte(w3, w2, 2), (int)__builtin_amdgcn_alignbyte(w4, w3, 2)};
        }
        return v16(p);
    }
    // 4 bytes at a 2-byte aligned address.
    __device__ static uint32_t a2_4(bp p) {
        if (reinterpret_cast<uintptr_t>(p) & 2) return __builtin_amdgcn_alignbyte(u16(p + 2), u32(p - 2), 2);
        return u32(p);
    }
};
typedef Mem<3>::bp lds_bp;

// ---- per-type decode helpers (shared by the units and the test hook) ----

// Q4_K scale / min of group j from the 12 packed bytes (as 3 dwords s0..s2).
__device__ __forceinline__ void q4k_scale_min(int j, uint32_t s0, uint32_t s1, uint32_t s2, int &sc, int &mn) {
    auto byte = [&](int k) -> int {
        const uint32_t w = k < 4 ? s0 : (k < 8 ? s1 : s2);
        return (int)((w >> (8 * (k & 3))) & 0xffu);
    };
    if (j < 4) {
        sc = byte(j) & 63;
        mn = byte(j + 4) & 63;
    } else {
        sc = (byte(j + 4) & 0x0f) | ((byte(j - 4) >> 6) << 4);
        mn = (byte(j + 4) >> 4) | ((byte(j) >> 6) << 4);
    }
}

__device__ __forceinline__ int q4k_lo(int qs) { return qs & 0x0f0f0f0f; }
__device__ __forceinline__ int q4k_hi(int qs) { return (int)(((uint32_t)qs >> 4) & 0x0f0f0f0fu); }

// Q6_K: 4 packed weights (value - 32, as signed bytes) of quarter g from one
// dword of ql (low nibbles for g < 2, high for g >= 2) and one of qh.
__device__ __forceinline__ int q6k_quants(uint32_t ql, uint32_t qh, int g) {
    const uint32_t lo = g < 2 ? (ql & 0x0f0f0f0fu) : ((ql >> 4) & 0x0f0f0f0fu);
    const uint32_t hb = ((qh >> (2 * g)) & 0x03030303u) << 4;
    return (int)((((lo | hb) | 0x80808080u) - 0x20202020u) ^ 0x80808080u);   // bytewise v - 32
}

// 16 activation quants at byte offset `off` (a multiple of 16) of a q8_1 block in LDS.
__device__ __forceinline__ v4i act16(lds_bp blk, int off) {
    typedef const v2i __attribute__((address_space(3))) *v2p;
    const v2p p = (v2p)(blk + 8 + off);
    const v2i a = p[0], b = p[1];
    return v4i{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ float2 act_ds(lds_bp blk) {
    typedef const float __attribute__((address_space(3))) *fp;
    const fp f = (fp)blk;
    return make_float2(f[0], f[1]);
}

template <int T, int NC, int AS>
struct Unit;

// ---- Q4_K: unit = (super-block sb, chunk c): 16 quant bytes = 16 weights of
// group 2p (low nibbles) and 16 of group 2p+1 (high nibbles), p = c/2.
template <int NC, int AS>
struct Unit<T_Q4_K, NC, AS> {
    typedef typename Mem<AS>::bp bp;
    __device__ static void run(int u, bp row0, bp row1, lds_bp act, int act_stride, int ncols, float (&acc)[2][NC]) {
        const int sb = u >> 3, c = u & 7, p = c >> 1, h = c & 1;
        const bp rows[2] = {row0, row1};
        int lo[2][4], hi[2][4];
        float d[2], dmin[2], sc0[2], sc1[2], mn0[2], mn1[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const bp blk = rows[i] + sb * 144;
            const v4i hdr = Mem<AS>::v16(blk);
            const v4i qs = Mem<AS>::v16(blk + 16 + 32 * p + 16 * h);
            d[i] = fp16_bits_to_f32((uint32_t)hdr.x & 0xffffu);
            dmin[i] = fp16_bits_to_f32((uint32_t)hdr.x >> 16);
            int a, b;
            q4k_scale_min(2 * p, hdr.y, hdr.z, hdr.w, a, b);
            sc0[i] = (float)a; mn0[i] = (float)b;
            q4k_scale_min(2 * p + 1, hdr.y, hdr.z, hdr.w, a, b);
            sc1[i] = (float)a; mn1[i] = (float)b;
#pragma unroll
            for (int w = 0; w < 4; w++) { lo[i][w] = q4k_lo(qs[w]); hi[i][w] = q4k_hi(qs[w]); }
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
            const lds_bp a0 = act + col * act_stride + (sb * 8 + 2 * p) * Q8_1_BYTES;
            const lds_bp a1 = a0 + Q8_1_BYTES;
            const float2 ds0 = act_ds(a0), ds1 = act_ds(a1);
            const v4i q0 = act16(a0, 16 * h), q1 = act16(a1, 16 * h);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                int D0 = 0, D1 = 0;
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    D0 = dot4(lo[i][w], q0[w], D0);
                    D1 = dot4(hi[i][w], q1[w], D1);
                }
                float v = d[i] * (sc0[i] * ds0.x * (float)D0 + sc1[i] * ds1.x * (float)D1);
                if (h == 0) v -= dmin[i] * (mn0[i] * ds0.y + mn1[i] * ds1.y);
                acc[i][col] += v;
            }
        }
    }
};

// ---- Q6_K: unit = (super-block sb, half hh, lane range t): 64 weights =
// 16 consecutive l of each of the four 32-groups g of the half.
template <int NC, int AS>
struct Unit<T_Q6_K, NC, AS> {
    typedef typename Mem<AS>::bp bp;
    __device__ static void run(int u, bp row0, bp row1, lds_bp act, int act_stride, int ncols, float (&acc)[2][NC]) {
        const int sb = u >> 2, hh = (u >> 1) & 1, t = u & 1;
        const bp rows[2] = {row0, row1};
        int q[2][4][4];
        float dsc[2][4];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const bp blk = rows[i] + sb * 210;
            const v4i ql0 = Mem<AS>::a2_16(blk + 64 * hh + 16 * t);
            const v4i ql1 = Mem<AS>::a2_16(blk + 64 * hh + 32 + 16 * t);
            const v4i qh = Mem<AS>::a2_16(blk + 128 + 32 * hh + 16 * t);
            const uint32_t s01 = Mem<AS>::a2_4(blk + 192 + 8 * hh);       // scales 8hh .. 8hh+3
            const uint32_t s23 = Mem<AS>::a2_4(blk + 192 + 8 * hh + 4);   // scales 8hh+4 .. 8hh+7
            const float d = fp16_bits_to_f32(Mem<AS>::u16(blk + 208));
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int k = 2 * g + t;                                   // scale index - 8hh
                const uint32_t sw = k < 4 ? s01 : s23;
                dsc[i][g] = d * (float)(int8_t)((sw >> (8 * (k & 3))) & 0xffu);
#pragma unroll
                for (int w = 0; w < 4; w++) q[i][g][w] = q6k_quants((uint32_t)((g & 1) ? ql1[w] : ql0[w]), (uint32_t)qh[w], g);
            }
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const lds_bp a = act + col * act_stride + (sb * 8 + 4 * hh + g) * Q8_1_BYTES;
                const float d8 = act_ds(a).x;
                const v4i qa = act16(a, 16 * t);
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    int D = 0;
#pragma unroll
                    for (int w = 0; w < 4; w++) D = dot4(q[i][g][w], qa[w], D);
                    acc[i][col] += dsc[i][g] * d8 * (float)D;
                }
            }
        }
    }
};

// ---- Q8_0: unit = one 34-byte block (32 weights).
template <int NC, int AS>
struct Unit<T_Q8_0, NC, AS> {
    typedef typename Mem<AS>::bp bp;
    __device__ static void run(int u, bp row0, bp row1, lds_bp act, int act_stride, int ncols, float (&acc)[2][NC]) {
        const bp rows[2] = {row0, row1};
        v4i q[2][2];
        float d[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const bp blk = rows[i] + u * 34;
            d[i] = fp16_bits_to_f32(Mem<AS>::u16(blk));
            q[i][0] = Mem<AS>::a2_16(blk + 2);
            q[i][1] = Mem<AS>::a2_16(blk + 18);
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
            const lds_bp a = act + col * act_stride + u * Q8_1_BYTES;
            const float d8 = act_ds(a).x;
            const v4i qa0 = act16(a, 0), qa1 = act16(a, 16);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                int D = 0;
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    D = dot4(q[i][0][w], qa0[w], D);
                    D = dot4(q[i][1][w], qa1[w], D);
                }
                acc[i][col] += d[i] * d8 * (float)D;
            }
        }
    }
};

template <int YDT>
__device__ __forceinline__ void store_out(void *y, int64_t idx, float v) {
    if (YDT == DT_F32) static_cast<float *>(y)[idx] = v;
    else static_cast<uint16_t *>(y)[idx] = (uint16_t)f32_to_bf16_bits(v);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Quantize (or copy) the activation rows of this block's columns into LDS as
// q8_1 blocks: the same arithmetic as the standalone quantizer (IEEE division,
// round half away from zero), 8 lanes per 32-value block; the loads of four
// passes are issued together.
__device__ __forceinline__ void stage_acts(uint8_t *lds, const MmvqParams &p, const int64_t *xrow, int ncols,
                                           int64_t nb) {
    const int64_t total = (int64_t)ncols * nb;
    if (p.xsrc == DT_Q8_1) {
        const int64_t words = total * (Q8_1_BYTES / 4);
        for (int64_t w = threadIdx.x; w < words; w += blockDim.x) {
            const int64_t b = w / (Q8_1_BYTES / 4), o = w % (Q8_1_BYTES / 4);
            const int64_t c = b / nb, blk = b % nb;
            reinterpret_cast<uint32_t *>(lds)[w] =
                reinterpret_cast<const uint32_t *>(p.q8 + xrow[c] * p.q8_row + blk * Q8_1_BYTES)[o];
        }
        return;
    }
    constexpr int PASSES = 4;
    const int sub = threadIdx.x & 7;
    const int64_t per_pass = blockDim.x / 8;
    for (int64_t base = 0; base < total; base += PASSES * per_pass) {   // block-uniform trip count
        // all loads of the four passes first (clamped in-bounds), then the math
        float v[PASSES][4];
#pragma unroll
        for (int ps = 0; ps < PASSES; ps++) {
            const int64_t b = min<int64_t>(base + ps * per_pass + (threadIdx.x >> 3), total - 1);
            const int64_t c = b / nb, blk = b - c * nb;
            const int64_t e0 = xrow[c] * p.ldx + blk * QK8_1 + sub * 4;
            if (p.xsrc == DT_F32) {
                const float *xf = static_cast<const float *>(p.x) + e0;
#pragma unroll
                for (int i = 0; i < 4; i++) v[ps][i] = xf[i];
            } else {
                const uint16_t *xb = static_cast<const uint16_t *>(p.x) + e0;
#pragma unroll
                for (int i = 0; i < 4; i++) v[ps][i] = bf16_bits_to_f32(xb[i]);
            }
        }
#pragma unroll
        for (int ps = 0; ps < PASSES; ps++) {
            const int64_t b = base + ps * per_pass + (threadIdx.x >> 3);
            const float amax = max8(fmaxf(fmaxf(fabsf(v[ps][0]), fabsf(v[ps][1])), fmaxf(fabsf(v[ps][2]), fabsf(v[ps][3]))));
            float d = amax / 127.0f;
            int q[4], sum = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                int qi = 0;
                if (amax != 0.0f) qi = (int)fminf(fmaxf(roundf(v[ps][i] / d), -127.0f), 127.0f);
                q[i] = qi;
                sum += qi;
            }
            sum = sum8(sum);
            if (amax == 0.0f) d = 0.0f;
            if (b < total) {
                uint8_t *out = lds + b * Q8_1_BYTES;
                reinterpret_cast<uint32_t *>(out + 8)[sub] = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                                                             ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
                if (sub == 0) {
                    reinterpret_cast<float *>(out)[0] = d;
                    reinterpret_cast<float *>(out)[1] = d * (float)sum;
                }
            }
        }
    }
}

// ---- LDS weight staging ----
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(v4i rsrc, __attribute__((address_space(3))) uint32_t *lds,
                                                           int size, int voffset, int soffset, int offset,
                                                           int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }    // vmcnt(0)
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// One work item of a wave = (group of spw row pairs, K-chunk kc).  The chunk
// holds the blocks [sb0, sb0 + bpc) of each of the 2*spw rows ("slots"), one
// unit per lane.  Slot s is staged at LDS offset s*cps*16 + (address & 15),
// copied by buffer_load_dwordx4 ... lds: instruction k moves the 16-byte
// pieces idx = lane + 64k (slot idx / cps, piece idx % cps), each lane with
// its own source address, into 1 KB of consecutive LDS.  Pieces of invalid
// slots (rows past the matrix) get an offset past the buffer range and land
// as zeros without touching memory.
struct Stage {
    const uint8_t *W;         // weight matrix of this group
    int64_t row_bytes, N, Np, npairs;
    int bpc, bb, cps, ninst;  // blocks per chunk, bytes per block, pieces per slot, DMA instructions
    int nslots;               // rows staged per item (2 per lane segment)
    const uint8_t *wend;      // end of the readable weight bytes
};

template <int EPI>
__device__ __forceinline__ int64_t slot_row(const Stage &S, int64_t pw, int slot) {
    const int64_t pair = pw + (slot >> 1);
    if (pair >= S.npairs) return -1;
    const int64_t r = EPI == EPI_SWIGLU ? ((slot & 1) ? pair + S.Np : pair) : 2 * pair + (slot & 1);
    return r < S.N ? r : -1;
}

template <int EPI>
__device__ __forceinline__ void stage_issue(const Stage &S, uint8_t *buf, int64_t pw, int kc, int lane) {
    const int sb0 = kc * S.bpc;
    const uint8_t *base = S.W + (EPI == EPI_SWIGLU ? pw : 2 * pw) * S.row_bytes + sb0 * S.bb;
    base = reinterpret_cast<const uint8_t *>(reinterpret_cast<uintptr_t>(base) & ~uintptr_t(15));
    struct { const void *p; uint32_t range; uint32_t cfg; } r = {
        base, (uint32_t)min<int64_t>(S.wend - base, 0x7fffff00LL), 0x00020000u};
    v4i rsrc = __builtin_bit_cast(v4i, r);
#pragma unroll
    for (int i = 0; i < 4; i++) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);   // wave-uniform descriptor
    for (int k = 0; k < S.ninst; k++) {
        const int idx = lane + 64 * k, slot = idx / S.cps, c = idx - slot * S.cps;
        uint32_t voff = 0xfffffff0u;                          // out of range: zeros, no memory access
        const int64_t row = slot < S.nslots ? slot_row<EPI>(S, pw, slot) : -1;
        if (row >= 0) {
            const uintptr_t g = (reinterpret_cast<uintptr_t>(S.W + row * S.row_bytes + sb0 * S.bb) & ~uintptr_t(15)) + 16 * c;
            voff = (uint32_t)(g - reinterpret_cast<uintptr_t>(base));
        }
        llvm_amdgcn_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) uint32_t *)(buf + 1024 * k), 16,
                                        (int)voff, 0, 0, 0);
    }
}

// wend is 2-byte aligned; when it is not 4-byte aligned the dword holding its
// last two bytes is outside the range and landed as zero: patch those two
// bytes from a 16-bit load (after the copy has landed).
template <int EPI>
__device__ __forceinline__ void stage_patch(const Stage &S, uint8_t *buf, int64_t pw, int kc, int lane, int nslots) {
    if (!(reinterpret_cast<uintptr_t>(S.wend) & 2)) return;
    const int sb0 = kc * S.bpc;
    for (int k = 0; k < S.ninst; k++) {
        const int idx = lane + 64 * k, slot = idx / S.cps, c = idx - slot * S.cps;
        if (slot >= nslots) break;
        const int64_t row = slot_row<EPI>(S, pw, slot);
        if (row < 0) continue;
        const uint8_t *g = reinterpret_cast<const uint8_t *>(
            (reinterpret_cast<uintptr_t>(S.W + row * S.row_bytes + sb0 * S.bb) & ~uintptr_t(15)) + 16 * c);
        if (g <= S.wend - 2 && S.wend - 2 < g + 16)
            *reinterpret_cast<uint16_t *>(buf + 16 * idx + (S.wend - 2 - g)) = *reinterpret_cast<const uint16_t *>(S.wend - 2);
    }
}

// grid: (blocks_x, column groups).  Each block stages its columns' q8_1
// activations in LDS, then each wave walks its work items (spw row pairs x
// K-chunks), copying item i+1 into its second LDS buffer while it computes
// item i from the first.
template <int T, int NC, bool MOE, int EPI, int YDT>
__global__ __launch_bounds__(256) void mmvq_kernel(const MmvqParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ int64_t xrow[NC];
    __shared__ int32_t route_s[NC];
    constexpr int UPB = T == T_Q4_K ? 8 : T == T_Q6_K ? 4 : 1;       // units per block
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int seg = p.seg, lane_in = lane & (seg - 1), spw = 64 / seg, sid = lane / seg;
    const int64_t grp = blockIdx.y;
    const int64_t nb = p.K / QK8_1;
    const int act_stride = (int)(nb * Q8_1_BYTES);
    uint8_t *act_lds = lds;
    const int bufsz = p.stage_ninst * 1024;
    uint8_t *wbuf = lds + p.act_lds_bytes + wave * 2 * bufsz;

    // ---- columns of this group ----
    const uint8_t *W = p.W;
    int ncols;
    if (!MOE) {
        const int64_t c0 = grp * NC;
        ncols = (int)min<int64_t>(NC, p.M - c0);
        if (threadIdx.x < NC) xrow[threadIdx.x] = c0 + (threadIdx.x < ncols ? threadIdx.x : 0);
    } else {
        if (grp >= (int64_t)*p.ngroups) return;                 // block-uniform
        const int4 g = p.groups[grp];
        W += (int64_t)g.x * p.expert_stride;
        ncols = g.z;
        if (threadIdx.x < NC) {
            const int c = threadIdx.x < ncols ? threadIdx.x : 0;
            const int32_t r = p.perm[g.y + c];
            route_s[threadIdx.x] = r;
            xrow[threadIdx.x] = p.x_per_route ? r : r / p.top_k;
        }
    }
    Stage S;
    S.W = W;
    S.row_bytes = p.row_bytes;
    S.N = p.N;
    S.Np = p.Np;
    S.npairs = p.npairs;
    S.bpc = seg / UPB;
    S.bb = Geom<T>::BYTES;
    S.cps = p.stage_cps;
    S.ninst = p.stage_ninst;
    S.nslots = 2 * spw;
    S.wend = p.W + p.w_bytes;
    const int nkc = (p.units + seg - 1) / seg;                  // K-chunks per row
    const int nslots = 2 * spw;

    const int64_t wave_stride = (int64_t)gridDim.x * 4 * spw;
    const int64_t pw0 = ((int64_t)blockIdx.x * 4 + wave) * spw;
    if (pw0 < p.npairs) stage_issue<EPI>(S, wbuf, pw0, 0, lane);   // first weights in flight during the prologue
    __syncthreads();
    stage_acts(act_lds, p, xrow, ncols, nb);
    __syncthreads();

    float acc[2][NC];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int c = 0; c < NC; c++) acc[i][c] = 0.0f;

    int64_t pw = pw0;
    int kc = 0, cur = 0;
    while (pw < p.npairs) {                                     // wave-uniform
        const int64_t pair = pw + sid;
        const bool pvalid = pair < p.npairs;
        int64_t r0, r1;
        if (EPI == EPI_SWIGLU) { r0 = pair; r1 = pair + p.Np; }
        else { r0 = 2 * pair; r1 = 2 * pair + 1; }
        const bool v1 = pvalid && r1 < p.N;

        wait_vm();                                              // item (pw, kc) has landed
        stage_patch<EPI>(S, wbuf + cur * bufsz, pw, kc, lane, nslots);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // next item into the other buffer (its previous contents were consumed last iteration)
        int64_t npw = pw;
        int nkc_next = kc + 1;
        if (nkc_next == nkc) { nkc_next = 0; npw = pw + wave_stride; }
        if (npw < p.npairs) stage_issue<EPI>(S, wbuf + (cur ^ 1) * bufsz, npw, nkc_next, lane);

        // compute this lane's unit of this chunk for both rows of its pair
        const int u = kc * seg + lane_in;
        if (pvalid && u < p.units) {
            uint8_t *b = wbuf + cur * bufsz;
            const int sb0 = kc * S.bpc;
            const uint8_t *g0 = W + r0 * p.row_bytes + sb0 * S.bb;
            const uint8_t *g1 = W + (v1 ? r1 : r0) * p.row_bytes + sb0 * S.bb;
            const int s1 = v1 ? 2 * sid + 1 : 2 * sid;
            // slot data sits at (address & 15); shift back by sb0 blocks so the unit indexes whole rows
            const lds_bp row0 = (lds_bp)(b + 2 * sid * S.cps * 16 + (reinterpret_cast<uintptr_t>(g0) & 15)) - sb0 * S.bb;
            const lds_bp row1 = (lds_bp)(b + s1 * S.cps * 16 + (reinterpret_cast<uintptr_t>(g1) & 15)) - sb0 * S.bb;
            Unit<T, NC, 3>::run(u, row0, row1, (lds_bp)act_lds, act_stride, ncols, acc);
        }
        wait_lgkm();                                            // LDS reads done before this buffer is refilled
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        cur ^= 1;

        if (++kc < nkc) continue;
        // ---- row pair complete: reduce across the segment and store ----
        kc = 0;
        pw += wave_stride;
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int c = 0; c < NC; c++) acc[i][c] = seg_sum(acc[i][c], seg);
        if (pvalid && lane_in == seg - 1) {          // seg_sum leaves the total in the segment's last lane
#pragma unroll
            for (int c = 0; c < NC; c++) {
                if (c >= ncols) break;
                if (!MOE) {
                    const int64_t col = xrow[c];
                    store_out<YDT>(p.y, col * p.ldy + r0, acc[0][c]);
                    if (v1) store_out<YDT>(p.y, col * p.ldy + r1, acc[1][c]);
                } else {
                    const int64_t r = route_s[c];
                    const int64_t t = r / p.top_k;
                    if (EPI == EPI_SWIGLU) {
                        const float h = silu_mul(acc[0][c], acc[1][c]);
                        if (p.route_w) atomicAdd(&p.acc32[t * p.Np + r0], p.route_w[r] * h);
                        else store_out<YDT>(p.y, r * p.Np + r0, h);
                    } else if (p.route_w) {
                        const float w = p.route_w[r];
                        atomicAdd(&p.acc32[t * p.Np + r0], w * acc[0][c]);
                        if (v1) atomicAdd(&p.acc32[t * p.Np + r1], w * acc[1][c]);
                    } else {
                        store_out<YDT>(p.y, r * p.Np + r0, acc[0][c]);
                        if (v1) store_out<YDT>(p.y, r * p.Np + r1, acc[1][c]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int c = 0; c < NC; c++) acc[i][c] = 0.0f;
    }
}

// ---- test hook: per-group int32 dots through the same decode helpers + dot4 ----
// One thread per (m, n, group).
template <int T>
__global__ __launch_bounds__(256) void mmvq_dots_kernel(const uint8_t *__restrict__ W, int64_t N, int64_t K,
                                                        const uint8_t *__restrict__ q8, int64_t M,
                                                        int32_t *__restrict__ out) {
    constexpr int G = Geom<T>::G;
    typedef Mem<1> gm;
    const int64_t gpr = K / G;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= M * N * gpr) return;
    const int64_t j = gid % gpr, n = (gid / gpr) % N, m = gid / (gpr * N);
    const gm::bp row = (gm::bp)(W + n * (K / Geom<T>::QK) * Geom<T>::BYTES);
    const gm::bp arow = (gm::bp)(q8 + m * (K / QK8_1) * Q8_1_BYTES);
    int D = 0;
    if (T == T_Q4_K) {
        const int sb = (int)(j / 8), jj = (int)(j % 8), p = jj >> 1;
        const gm::bp blk = row + sb * 144;
        const gm::bp a = arow + (sb * 8 + jj) * Q8_1_BYTES;
        for (int h = 0; h < 2; h++) {
            const v4i qs = gm::v16(blk + 16 + 32 * p + 16 * h);
            const v4i qa = gm::v16(a + 8 + 16 * h);
            for (int w = 0; w < 4; w++) D = dot4((jj & 1) ? q4k_hi(qs[w]) : q4k_lo(qs[w]), qa[w], D);
        }
    } else if (T == T_Q6_K) {
        const int sb = (int)(j / 16), jj = (int)(j % 16);          // 16-weight group
        const int hh = jj / 8, g = (jj % 8) / 2, t = jj & 1;
        const gm::bp blk = row + sb * 210;
        const v4i ql = gm::a2_16(blk + 64 * hh + 32 * (g & 1) + 16 * t);
        const v4i qh = gm::a2_16(blk + 128 + 32 * hh + 16 * t);
        const v4i qa = gm::v16(arow + (sb * 8 + 4 * hh + g) * Q8_1_BYTES + 8 + 16 * t);
        for (int w = 0; w < 4; w++) D = dot4(q6k_quants((uint32_t)ql[w], (uint32_t)qh[w], g), qa[w], D);
    } else {
        const gm::bp blk = row + j * 34;
        const gm::bp a = arow + j * Q8_1_BYTES;
        const v4i q0 = gm::a2_16(blk + 2), q1 = gm::a2_16(blk + 18);
        const v4i a0 = gm::v16(a + 8), a1 = gm::v16(a + 24);
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

template <int T, int NC, bool MOE, int EPI, int YDT>
static void launch_one(const MmvqParams &p, dim3 g, size_t lds, hipStream_t s) {
    auto k = mmvq_kernel<T, NC, MOE, EPI, YDT>;
    raise_lds_limit(k, lds);
    hipLaunchKernelGGL(k, g, dim3(256), lds, s, p);
}

template <int T, int NC>
static void launch_nc(bool moe, int epi, int ydt, const MmvqParams &p, dim3 g, size_t lds, hipStream_t s) {
    if (!moe) {
        if (ydt == DT_F32) launch_one<T, NC, false, EPI_NONE, DT_F32>(p, g, lds, s);
        else launch_one<T, NC, false, EPI_NONE, DT_BF16>(p, g, lds, s);
    } else if (epi == EPI_SWIGLU) {
        if (ydt == DT_F32) launch_one<T, NC, true, EPI_SWIGLU, DT_F32>(p, g, lds, s);
        else launch_one<T, NC, true, EPI_SWIGLU, DT_BF16>(p, g, lds, s);
    } else {
        if (ydt == DT_F32) launch_one<T, NC, true, EPI_NONE, DT_F32>(p, g, lds, s);
        else launch_one<T, NC, true, EPI_NONE, DT_BF16>(p, g, lds, s);
    }
}

template <int T>
static void launch_t(int nc, bool moe, int epi, int ydt, const MmvqParams &p, dim3 g, size_t lds, hipStream_t s) {
    switch (nc) {
    case 1: launch_nc<T, 1>(moe, epi, ydt, p, g, lds, s); break;
    case 2: launch_nc<T, 2>(moe, epi, ydt, p, g, lds, s); break;
    case 4: launch_nc<T, 4>(moe, epi, ydt, p, g, lds, s); break;
    default: launch_nc<T, 8>(moe, epi, ydt, p, g, lds, s); break;
    }
}

int mmvq_max_cols(int64_t K) {
    for (int nc = 8; nc > 1; nc >>= 1)
        if ((size_t)nc * (size_t)(K / QK8_1) * Q8_1_BYTES <= MMVQ_LDS_MAX) return nc;
    return 1;
}

hipError_t launch_mmvq(int t, int nc, bool moe, int epi, int ydt, const MmvqParams &p0, int64_t ngroups_bound,
                       hipStream_t s) {
    MmvqParams p = p0;
    if (p.npairs == 0 || ngroups_bound == 0) return hipSuccess;
    const size_t act = ((size_t)nc * (size_t)(p.K / QK8_1) * Q8_1_BYTES + 15) & ~size_t(15);
    if (act > MMVQ_LDS_MAX) return hipErrorInvalidValue;
    const int upb = t == T_Q4_K ? 8 : t == T_Q6_K ? 4 : 1;
    int seg = 1;
    while (seg < p.units && seg < 64) seg <<= 1;
    p.seg = seg;
    const int spw = 64 / seg;
    const int64_t bb = block_bytes(t);
    p.stage_cps = (int)((seg / upb * bb + 15 + 15) / 16);       // pieces covering a chunk of a row at any phase
    p.stage_ninst = (2 * spw * p.stage_cps + 63) / 64;
    p.act_lds_bytes = (int64_t)act;
    // staging offsets are 32-bit from the first row of an item
    if ((epi == EPI_SWIGLU ? p.Np + spw : 2 * spw) * p.row_bytes >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const size_t lds = act + 4 * 2 * (size_t)p.stage_ninst * 1024;
    // one round of resident blocks (each quantizes its activations once)
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(8, (int64_t)(160 * 1024) / (int64_t)lds));
    const int64_t pairs_per_block = 4 * spw;
    const int64_t need = (p.npairs + pairs_per_block - 1) / pairs_per_block;
    const int64_t cap = std::max<int64_t>(1, 256 * per_cu / ngroups_bound);
    const dim3 g((unsigned)std::min<int64_t>(need, cap), (unsigned)ngroups_bound);
    if (t == T_Q4_K) launch_t<T_Q4_K>(nc, moe, epi, ydt, p, g, lds, s);
    else if (t == T_Q6_K) launch_t<T_Q6_K>(nc, moe, epi, ydt, p, g, lds, s);
    else launch_t<T_Q8_0>(nc, moe, epi, ydt, p, g, lds, s);
    return hipGetLastError();
}

hipError_t launch_mmvq_dots(int t, const uint8_t *W, int64_t N, int64_t K, const uint8_t *q8, int64_t M,
                            int32_t *out, hipStream_t s) {
    const int64_t n = M * N * (K / group_len(t));
    if (n == 0) return hipSuccess;
    dim3 g((unsigned)((n + 255) / 256));
    if (t == T_Q4_K) hipLaunchKernelGGL(mmvq_dots_kernel<T_Q4_K>, g, dim3(256), 0, s, W, N, K, q8, M, out);
    else if (t == T_Q6_K) hipLaunchKernelGGL(mmvq_dots_kernel<T_Q6_K>, g, dim3(256), 0, s, W, N, K, q8, M, out);
    else hipLaunchKernelGGL(mmvq_dots_kernel<T_Q8_0>, g, dim3(256), 0, s, W, N, K, q8, M, out);
    return hipGetLastError();
}

}  // namespace ggq
