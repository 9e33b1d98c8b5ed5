// MMVQ: quantized matrix x few-vectors, for small batches (decode).
//
// HBM-bound on the weights, so every weight byte is read exactly once:
//  - a wave owns row pairs; within a row, lanes take consecutive 16-byte
//    "units" of the GGUF blocks (Q4_K: one 16 B quant chunk + the block
//    header; Q6_K: 48 B of ql/qh for 64 weights; Q8_0: one 34 B block), so a
//    segment of lanes streams a contiguous span of the row;
//  - the q8_1 activations (a few KB, L2-resident) are loaded once per unit
//    and reused for both rows of the pair and for every column;
//  - integer dots use v_dot4 (4 int8 products + int32 accumulate), the scale
//    product is applied in fp32 per scale group, and the partial sums of a
//    row are reduced across the lane segment with cross-lane shuffles.
// The routed form (mul_mat_id for small token counts) runs the same code per
// (expert, group of routes) so each expert's weights are read once however
// many tokens route to it.
#include "kernels.hpp"

namespace ggq {

constexpr int EPI_NONE = 0, EPI_SWIGLU = 1;

// Q4_K scale / min of group j from the 12 packed bytes (as 3 dwords s0..s2).
__device__ __forceinline__ void q4k_scale_min(int j, uint32_t s0, uint32_t s1, uint32_t s2, int &sc, int &mn) {
    auto byte = [&](int k) -> int {
        uint32_t w = k < 4 ? s0 : (k < 8 ? s1 : s2);
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

// 16 activation quants at byte offset `off` (a multiple of 16) inside a q8_1 block.
__device__ __forceinline__ v4i act16(const uint8_t *blk, int off) {
    const v2i *p = reinterpret_cast<const v2i *>(blk + 8 + off);
    v2i a = p[0], b = p[1];
    return v4i{a.x, a.y, b.x, b.y};
}

// Unsigned 6-bit values packed in bytes -> signed (value - 32) bytes.
__device__ __forceinline__ int minus32(uint32_t q) {
    return (int)(((q | 0x80808080u) - 0x20202020u) ^ 0x80808080u);
}

template <int T, int NC>
struct Unit;

// ---- Q4_K: unit = (super-block sb, chunk c): 16 quant bytes = 16 weights of
// group 2p (low nibbles) and 16 of group 2p+1 (high nibbles), p = c/2.
template <int NC>
struct Unit<T_Q4_K, NC> {
    static constexpr int PER_BLOCK = 8;
    __device__ static void run(int u, const uint8_t *row0, const uint8_t *row1, const uint8_t *const *act,
                               int ncols, float (&acc)[2][NC]) {
        const int sb = u >> 3, c = u & 7, p = c >> 1, h = c & 1;
        const uint8_t *rows[2] = {row0, row1};
        v4i lo[2], hi[2];
        float d[2], dmin[2], sc0[2], sc1[2], mn0[2], mn1[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const uint8_t *blk = rows[i] + (int64_t)sb * 144;
            const v4i hdr = *reinterpret_cast<const v4i *>(blk);
            const v4i qs = *reinterpret_cast<const v4i *>(blk + 16 + 32 * p + 16 * h);
            d[i] = fp16_bits_to_f32((uint32_t)hdr.x & 0xffffu);
            dmin[i] = fp16_bits_to_f32((uint32_t)hdr.x >> 16);
            int a, b;
            q4k_scale_min(2 * p, hdr.y, hdr.z, hdr.w, a, b);
            sc0[i] = (float)a; mn0[i] = (float)b;
            q4k_scale_min(2 * p + 1, hdr.y, hdr.z, hdr.w, a, b);
            sc1[i] = (float)a; mn1[i] = (float)b;
#pragma unroll
            for (int w = 0; w < 4; w++) {
                lo[i][w] = qs[w] & 0x0f0f0f0f;
                hi[i][w] = (int)(((uint32_t)qs[w] >> 4) & 0x0f0f0f0fu);
            }
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
            const uint8_t *a0 = act[col] + (int64_t)(sb * 8 + 2 * p) * Q8_1_BYTES;
            const uint8_t *a1 = a0 + Q8_1_BYTES;
            const float2 ds0 = *reinterpret_cast<const float2 *>(a0);
            const float2 ds1 = *reinterpret_cast<const float2 *>(a1);
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
template <int NC>
struct Unit<T_Q6_K, NC> {
    static constexpr int PER_BLOCK = 4;
    __device__ static void run(int u, const uint8_t *row0, const uint8_t *row1, const uint8_t *const *act,
                               int ncols, float (&acc)[2][NC]) {
        const int sb = u >> 2, hh = (u >> 1) & 1, t = u & 1;
        const uint8_t *rows[2] = {row0, row1};
        int q[2][4][4];
        float dsc[2][4];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const uint8_t *blk = rows[i] + (int64_t)sb * 210;
            const v4i ql0 = ld16_a2(blk + 64 * hh + 16 * t);
            const v4i ql1 = ld16_a2(blk + 64 * hh + 32 + 16 * t);
            const v4i qh = ld16_a2(blk + 128 + 32 * hh + 16 * t);
            const uint32_t s01 = ld4_a2(blk + 192 + 8 * hh);       // scales 8hh .. 8hh+3
            const uint32_t s23 = ld4_a2(blk + 192 + 8 * hh + 4);   // scales 8hh+4 .. 8hh+7
            const float d = fp16_bits_to_f32(ld_u16(blk + 208));
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int k = 2 * g + t;                            // scale index - 8hh
                const uint32_t sw = k < 4 ? s01 : s23;
                dsc[i][g] = d * (float)(int8_t)((sw >> (8 * (k & 3))) & 0xffu);
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    const uint32_t l4 = (uint32_t)((g & 1) ? ql1[w] : ql0[w]);
                    const uint32_t lo = g < 2 ? (l4 & 0x0f0f0f0fu) : ((l4 >> 4) & 0x0f0f0f0fu);
                    const uint32_t hb = (((uint32_t)qh[w] >> (2 * g)) & 0x03030303u) << 4;
                    q[i][g][w] = minus32(lo | hb);
                }
            }
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const uint8_t *a = act[col] + (int64_t)(sb * 8 + 4 * hh + g) * Q8_1_BYTES;
                const float d8 = *reinterpret_cast<const float *>(a);
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
template <int NC>
struct Unit<T_Q8_0, NC> {
    static constexpr int PER_BLOCK = 1;
    __device__ static void run(int u, const uint8_t *row0, const uint8_t *row1, const uint8_t *const *act,
                               int ncols, float (&acc)[2][NC]) {
        const uint8_t *rows[2] = {row0, row1};
        v4i q[2][2];
        float d[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const uint8_t *blk = rows[i] + (int64_t)u * 34;
            d[i] = fp16_bits_to_f32(ld_u16(blk));
            q[i][0] = ld16_a2(blk + 2);
            q[i][1] = ld16_a2(blk + 18);
        }
#pragma unroll
        for (int col = 0; col < NC; col++) {
            if (col >= ncols) break;
            const uint8_t *a = act[col] + (int64_t)u * Q8_1_BYTES;
            const float d8 = *reinterpret_cast<const float *>(a);
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

// grid: 1-D, row_blocks * groups blocks of 256 threads (4 waves).
template <int T, int NC, bool MOE, int EPI, int YDT>
__global__ __launch_bounds__(256) void mmvq_kernel(const MmvqParams p) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int seg = p.seg, lane_in = lane & (seg - 1), spw = 64 / seg;
    const int64_t rb = (int64_t)blockIdx.x % p.row_blocks;
    const int64_t grp = (int64_t)blockIdx.x / p.row_blocks;
    const int64_t pair0 = (rb * 4 + wave) * spw;
    if (pair0 >= p.npairs) return;                          // wave-uniform
    const int64_t pair = pair0 + lane / seg;
    const bool pvalid = pair < p.npairs;

    // columns of this group
    const uint8_t *W = p.W;
    int ncols;
    int32_t route[NC];
    const uint8_t *act[NC];
    if (!MOE) {
        const int64_t c0 = grp * NC;
        ncols = (int)min<int64_t>(NC, p.M - c0);
#pragma unroll
        for (int c = 0; c < NC; c++) act[c] = p.q8 + (c0 + (c < ncols ? c : 0)) * p.q8_row;
    } else {
        if (grp >= (int64_t)*p.ngroups) return;               // block-uniform
        const int4 g = p.groups[grp];
        W += (int64_t)g.x * p.expert_stride;
        ncols = g.z;
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const int32_t r = p.perm[g.y + (c < ncols ? c : 0)];
            route[c] = r;
            const int64_t xrow = p.x_per_route ? r : r / p.top_k;
            act[c] = p.q8 + xrow * p.q8_row;
        }
    }

    // the two weight rows of this pair
    int64_t r0, r1;
    if (EPI == EPI_SWIGLU) { r0 = pair; r1 = pair + p.Np; }
    else { r0 = 2 * pair; r1 = 2 * pair + 1; }
    const bool v1 = r1 < p.N;
    if (!pvalid) { r0 = 0; r1 = 0; }
    const uint8_t *row0 = W + r0 * p.row_bytes;
    const uint8_t *row1 = W + (v1 && pvalid ? r1 : r0) * p.row_bytes;

    float acc[2][NC];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int c = 0; c < NC; c++) acc[i][c] = 0.0f;

    if (pvalid)
        for (int u = lane_in; u < p.units; u += seg) Unit<T, NC>::run(u, row0, row1, act, ncols, acc);

#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int c = 0; c < NC; c++) acc[i][c] = seg_sum(acc[i][c], seg);

    if (!pvalid || lane_in != 0) return;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        if (c >= ncols) break;
        if (!MOE) {
            const int64_t col = grp * NC + c;
            store_out<YDT>(p.y, col * p.ldy + r0, acc[0][c]);
            if (v1) store_out<YDT>(p.y, col * p.ldy + r1, acc[1][c]);
        } else {
            const int64_t r = route[c];
            const int64_t t = r / p.top_k;
            if (EPI == EPI_SWIGLU) {
                const float h = silu_mul(acc[0][c], acc[1][c]);
                if (p.route_w) atomicAdd(&p.acc32[t * p.Np + r0], p.route_w[r] * h);
                else store_out<YDT>(p.y, r * p.Np + r0, h);
            } else {
                if (p.route_w) {
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
}

// ---- test hook: per-group int32 dots through the same unit decode + dot4 ----
// One thread per (m, n, group); decodes the group's weight quants with the
// same helpers as the units above.
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
        const uint8_t *blk = row + (int64_t)sb * 144;
        const uint8_t *a = arow + (int64_t)(sb * 8 + jj) * Q8_1_BYTES;
        for (int h = 0; h < 2; h++) {
            const v4i qs = *reinterpret_cast<const v4i *>(blk + 16 + 32 * p + 16 * h);
            const v4i qa = act16(a, 16 * h);
            for (int w = 0; w < 4; w++) {
                const int nib = (jj & 1) ? (int)(((uint32_t)qs[w] >> 4) & 0x0f0f0f0fu) : (qs[w] & 0x0f0f0f0f);
                D = dot4(nib, qa[w], D);
            }
        }
    } else if (T == T_Q6_K) {
        const int sb = (int)(j / 16), jj = (int)(j % 16);          // 16-weight group
        const int hh = jj / 8, g = (jj % 8) / 2, t = jj & 1;
        const uint8_t *blk = row + (int64_t)sb * 210;
        const v4i ql = ld16_a2(blk + 64 * hh + 32 * (g & 1) + 16 * t);
        const v4i qh = ld16_a2(blk + 128 + 32 * hh + 16 * t);
        const uint8_t *a = arow + (int64_t)(sb * 8 + 4 * hh + g) * Q8_1_BYTES;
        const v4i qa = act16(a, 16 * t);
        for (int w = 0; w < 4; w++) {
            const uint32_t lo = g < 2 ? ((uint32_t)ql[w] & 0x0f0f0f0fu) : (((uint32_t)ql[w] >> 4) & 0x0f0f0f0fu);
            const uint32_t hb = (((uint32_t)qh[w] >> (2 * g)) & 0x03030303u) << 4;
            D = dot4(minus32(lo | hb), qa[w], D);
        }
    } else {
        const uint8_t *blk = row + j * 34;
        const uint8_t *a = arow + j * Q8_1_BYTES;
        const v4i q0 = ld16_a2(blk + 2), q1 = ld16_a2(blk + 18);
        const v4i a0 = act16(a, 0), a1 = act16(a, 16);
        for (int w = 0; w < 4; w++) {
            D = dot4(q0[w], a0[w], D);
            D = dot4(q1[w], a1[w], D);
        }
    }
    out[gid] = D;
}

// ---------------------------------------------------------------------------
template <int T, int NC>
static void launch_nc(bool moe, int epi, int ydt, const MmvqParams &p, dim3 g, hipStream_t s) {
#define GGQ_L(MOE, EPI, YDT) hipLaunchKernelGGL((mmvq_kernel<T, NC, MOE, EPI, YDT>), g, dim3(256), 0, s, p)
    if (!moe) {
        if (ydt == DT_F32) GGQ_L(false, EPI_NONE, DT_F32); else GGQ_L(false, EPI_NONE, DT_BF16);
    } else if (epi == EPI_SWIGLU) {
        if (ydt == DT_F32) GGQ_L(true, EPI_SWIGLU, DT_F32); else GGQ_L(true, EPI_SWIGLU, DT_BF16);
    } else {
        if (ydt == DT_F32) GGQ_L(true, EPI_NONE, DT_F32); else GGQ_L(true, EPI_NONE, DT_BF16);
    }
#undef GGQ_L
}

template <int T>
static void launch_t(int nc, bool moe, int epi, int ydt, const MmvqParams &p, dim3 g, hipStream_t s) {
    switch (nc) {
    case 1: launch_nc<T, 1>(moe, epi, ydt, p, g, s); break;
    case 2: launch_nc<T, 2>(moe, epi, ydt, p, g, s); break;
    case 4: launch_nc<T, 4>(moe, epi, ydt, p, g, s); break;
    default: launch_nc<T, 8>(moe, epi, ydt, p, g, s); break;
    }
}

hipError_t launch_mmvq(int t, int nc, bool moe, int epi, int ydt, const MmvqParams &p0, int64_t ngroups_bound,
                       hipStream_t s) {
    MmvqParams p = p0;
    if (p.npairs == 0 || ngroups_bound == 0) return hipSuccess;
    int seg = 1;
    while (seg < p.units && seg < 64) seg <<= 1;
    p.seg = seg;
    const int64_t pairs_per_block = 4 * (64 / seg);
    p.row_blocks = (p.npairs + pairs_per_block - 1) / pairs_per_block;
    dim3 g((unsigned)(p.row_blocks * ngroups_bound));
    if (t == T_Q4_K) launch_t<T_Q4_K>(nc, moe, epi, ydt, p, g, s);
    else if (t == T_Q6_K) launch_t<T_Q6_K>(nc, moe, epi, ydt, p, g, s);
    else launch_t<T_Q8_0>(nc, moe, epi, ydt, p, g, s);
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
