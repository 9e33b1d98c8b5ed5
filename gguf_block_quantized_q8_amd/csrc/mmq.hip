// MMQ: tiled quantized matmul for prefill, on fp16 MFMA with exact integer
// operands.
//
// Why fp16 MFMA and not int8 MFMA: each output needs one fp32 rescale per
// 32-wide q8_1 block (weight sub-scale x activation scale), and on gfx950 the
// int8 MFMA and the VALU barely overlap.  With int8 MFMA the rescale costs
// cvt + int multiply by the sub-scale + fma per output per block; here the
// integer sub-scale is folded into the fp16 weight operand instead
// (Q4_K: sc * nibble <= 945, Q6_K: sc * (q - 32) split into two exact fp16
// parts), the MFMA accumulates the block's dot in fp32 exactly, and only one
// fma per output per block remains (times the activation scale d8).  Every
// product and partial sum is an integer below 2^24, so the per-block dot is
// exact, as with int8.
//
// Tiles: 128 weight rows x 128 activation rows per workgroup, 4 waves of
// 64 x 64 (2 x 2 MFMA 32x32x16 tiles).  K is staged 64 at a time through LDS
// (fp16, row stride 72 halves: conflict-free 16-byte fragment reads); per
// 256-wide super-block the weight scales and the activation d8 are staged once.
// Q4_K's min term  -dmin * sum_j m_j * s8_j  runs as a bf16 MFMA with s8
// split exactly into three bf16 parts.
#include "kernels.hpp"

namespace ggq {

constexpr int NT = MMQ_NT, MT = MMQ_MT, KS = 64, LDA = KS + 8, LDM = 40;
constexpr int EPI_NONE_ = 0, EPI_SWIGLU_ = 1;

template <int T>
struct __attribute__((aligned(16))) MmqSmem {
    static constexpr int NA = T == T_Q6_K ? 2 : 1;       // Q6_K: high and low parts of sc*(q-32)
    static constexpr int NMIN = T == T_Q4_K ? 1 : 0;
    _Float16 A[NA][NT][LDA];
    _Float16 B[MT][LDA];
    float wd[NT];
    float wdmin[NT];
    int8_t sc[NT][16];
    float d8[MT][8];
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

__device__ __forceinline__ void q4k_scale_min_b(int j, const uint8_t *s, int &sc, int &mn) {
    if (j < 4) {
        sc = s[j] & 63;
        mn = s[j + 4] & 63;
    } else {
        sc = (s[j + 4] & 0x0f) | ((s[j - 4] >> 6) << 4);
        mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

// Per super-block metadata: weight scales (threads 0..127 = weight rows) and
// activation d8 / s8 (threads 128..255 = tile columns).  UNIT: all integer
// sub-scales forced to 1 (test hook: raw per-group dots).
template <int T, bool UNIT>
__device__ __forceinline__ void stage_meta(MmqSmem<T> &sm, int sb, int64_t K, const float *__restrict__ xd,
                                           const float *__restrict__ xs) {
    const int tid = threadIdx.x;
    if (tid < NT) {
        const uint8_t *row = sm.wrow[tid];
        if (T == T_Q4_K) {
            float d = 0.f, dmin = 0.f;
            uint8_t s[12] = {};
            if (row) {
                const uint8_t *blk = row + (int64_t)sb * 144;
                const v4i hdr = *reinterpret_cast<const v4i *>(blk);
                d = fp16_bits_to_f32((uint32_t)hdr.x & 0xffffu);
                dmin = fp16_bits_to_f32((uint32_t)hdr.x >> 16);
                for (int k = 0; k < 12; k++) s[k] = (uint8_t)(((uint32_t)hdr[1 + k / 4] >> (8 * (k & 3))) & 0xffu);
            }
            sm.wd[tid] = d;
            sm.wdmin[tid] = dmin;
            for (int j = 0; j < 8; j++) {
                int sc = 0, mn = 0;
                if (row) q4k_scale_min_b(j, s, sc, mn);
                sm.sc[tid][j] = (int8_t)(UNIT ? 1 : sc);
                const __bf16 mb = (__bf16)(float)mn;
                sm.Amin[tid][3 * j] = mb;
                sm.Amin[tid][3 * j + 1] = mb;
                sm.Amin[tid][3 * j + 2] = mb;
            }
            for (int k = 24; k < 32; k++) sm.Amin[tid][k] = (__bf16)0.0f;
        } else if (T == T_Q6_K) {
            float d = 0.f;
            v4i scw = {0, 0, 0, 0};
            if (row) {
                const uint8_t *blk = row + (int64_t)sb * 210;
                d = fp16_bits_to_f32(ld_u16(blk + 208));
                scw = ld16_a2(blk + 192);
            }
            sm.wd[tid] = d;
            for (int j = 0; j < 16; j++)
                sm.sc[tid][j] = UNIT ? (int8_t)1 : (int8_t)(((uint32_t)scw[j / 4] >> (8 * (j & 3))) & 0xffu);
        }
    } else {
        const int i = tid - NT;
        const int32_t xr = sm.xrow[i];
        const int64_t nb = K / QK8_1;
        for (int j = 0; j < 8; j++) {
            float d8 = 0.f, s8 = 0.f;
            if (xr >= 0 && !UNIT) {
                d8 = xd[(int64_t)xr * nb + sb * 8 + j];
                if (T == T_Q4_K) s8 = xs[(int64_t)xr * nb + sb * 8 + j];
            }
            sm.d8[i][j] = d8;
            if (T == T_Q4_K) split3_bf16(s8, sm.Bmin[i][3 * j], sm.Bmin[i][3 * j + 1], sm.Bmin[i][3 * j + 2]);
        }
        if (T == T_Q4_K)
            for (int k = 24; k < 32; k++) sm.Bmin[i][k] = (__bf16)0.0f;
    }
}

// Stage weights [NT][KS] for K offset 64*st of super-block sb: fp16 of the
// integer sub-scale times the raw quant (Q4_K) or the two exact parts of
// sc*(q-32) (Q6_K).  Thread: row = tid/2, 16 weights of each of two groups.
template <int T>
__device__ __forceinline__ void stage_A(MmqSmem<T> &sm, int sb, int st) {
    const int tid = threadIdx.x, tr = tid >> 1, hf = tid & 1;
    const uint8_t *row = sm.wrow[tr];
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    if (T == T_Q4_K) {
        h8 lo[2], hi[2];
        if (row) {
            const v4i qs = *reinterpret_cast<const v4i *>(row + (int64_t)sb * 144 + 16 + 32 * st + 16 * hf);
            const int sc0 = sm.sc[tr][2 * st], sc1 = sm.sc[tr][2 * st + 1];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int byte = (qs[i / 4] >> (8 * (i % 4))) & 0xff;
                lo[i / 8][i % 8] = (_Float16)(float)(sc0 * (byte & 15));
                hi[i / 8][i % 8] = (_Float16)(float)(sc1 * (byte >> 4));
            }
        } else {
            lo[0] = lo[1] = hi[0] = hi[1] = h8{};
        }
        h8 *dlo = reinterpret_cast<h8 *>(&sm.A[0][tr][16 * hf]);
        h8 *dhi = reinterpret_cast<h8 *>(&sm.A[0][tr][32 + 16 * hf]);
        dlo[0] = lo[0]; dlo[1] = lo[1];
        dhi[0] = hi[0]; dhi[1] = hi[1];
    } else {
        const int hh = st >> 1, g0 = 2 * (st & 1);
        h8 ah[2][2], al[2][2];
        if (row) {
            const uint8_t *blk = row + (int64_t)sb * 210;
            const v4i qla = ld16_a2(blk + 64 * hh + 16 * hf);
            const v4i qlb = ld16_a2(blk + 64 * hh + 32 + 16 * hf);
            const v4i qh = ld16_a2(blk + 128 + 32 * hh + 16 * hf);
#pragma unroll
            for (int gg = 0; gg < 2; gg++) {
                const int g = g0 + gg;
                const int sc = sm.sc[tr][8 * hh + 2 * g + hf];
                const int sl = sc & 15, sh = sc - sl;
                const v4i ql = gg == 0 ? qla : qlb;
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int lb = (ql[i / 4] >> (8 * (i % 4))) & 0xff;
                    const int lo = g < 2 ? (lb & 15) : (lb >> 4);
                    const int hb = ((qh[i / 4] >> (8 * (i % 4))) >> (2 * g)) & 3;
                    const int q = (lo | (hb << 4)) - 32;
                    ah[gg][i / 8][i % 8] = (_Float16)(float)(sh * q);
                    al[gg][i / 8][i % 8] = (_Float16)(float)(sl * q);
                }
            }
        } else {
            ah[0][0] = ah[0][1] = ah[1][0] = ah[1][1] = h8{};
            al[0][0] = al[0][1] = al[1][0] = al[1][1] = h8{};
        }
#pragma unroll
        for (int gg = 0; gg < 2; gg++) {
            h8 *dh = reinterpret_cast<h8 *>(&sm.A[0][tr][32 * gg + 16 * hf]);
            h8 *dl = reinterpret_cast<h8 *>(&sm.A[MmqSmem<T>::NA - 1][tr][32 * gg + 16 * hf]);
            dh[0] = ah[gg][0]; dh[1] = ah[gg][1];
            dl[0] = al[gg][0]; dl[1] = al[gg][1];
        }
    }
}

// Stage activations [MT][KS] (fp16 quants) from the planar layout.
template <int T>
__device__ __forceinline__ void stage_B(MmqSmem<T> &sm, const _Float16 *__restrict__ xq, int64_t K, int64_t k0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const int q = tid + 256 * c, i = q >> 3, part = q & 7;
        const int32_t xr = sm.xrow[i];
        v4i v = {0, 0, 0, 0};
        if (xr >= 0) v = *reinterpret_cast<const v4i *>(xq + (int64_t)xr * K + k0 + 8 * part);
        *reinterpret_cast<v4i *>(&sm.B[i][8 * part]) = v;
    }
}

template <int YDT>
__device__ __forceinline__ void store4(void *y, int64_t idx, const float *v, int n_valid) {
    if (YDT == DT_F32) {
        float *o = static_cast<float *>(y) + idx;
        if (n_valid == 4 && (idx & 3) == 0) *reinterpret_cast<v4f *>(o) = v4f{v[0], v[1], v[2], v[3]};
        else for (int i = 0; i < n_valid; i++) o[i] = v[i];
    } else {
        uint16_t *o = static_cast<uint16_t *>(y) + idx;
        if (n_valid == 4 && (idx & 3) == 0) {
            v2i t = {(int)(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16)),
                     (int)(f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16))};
            *reinterpret_cast<v2i *>(o) = t;
        } else {
            for (int i = 0; i < n_valid; i++) o[i] = (uint16_t)f32_to_bf16_bits(v[i]);
        }
    }
}

// grid: 1-D, m_tiles * n_tiles workgroups of 256 threads.
template <int T, bool MOE, int EPI, int YDT>
__global__ __launch_bounds__(256, 2) void mmq_kernel(const MmqParams p) {
    __shared__ MmqSmem<T> sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t bm = (int64_t)blockIdx.x % p.m_tiles;
    const int64_t bn = (int64_t)blockIdx.x / p.m_tiles;

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
    } else if (tid < MT) {
        const int64_t m = bm * MT + tid;
        sm.xrow[tid] = m < p.M ? (int32_t)m : -1;
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

    v16f acc[2][2], P[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) { acc[a][b] = v16f{}; P[a][b] = v16f{}; }

    const int nsb = (int)(p.K / 256);
    const int lr = lane & 31, kh = 8 * (lane >> 5);
#pragma unroll 1
    for (int sb = 0; sb < nsb; sb++) {
        __syncthreads();                                      // previous super-block's meta no longer read
        stage_meta<T, false>(sm, sb, p.K, p.xd, p.xs);
#pragma unroll 1
        for (int st = 0; st < 4; st++) {
            __syncthreads();                                  // meta visible / previous stage consumed
            stage_A<T>(sm, sb, st);
            stage_B<T>(sm, p.xq, p.K, (int64_t)sb * 256 + 64 * st);
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 2; j++) {
                v16f C[2][2];
#pragma unroll
                for (int a = 0; a < 2; a++)
#pragma unroll
                    for (int b = 0; b < 2; b++) C[a][b] = v16f{};
#pragma unroll
                for (int kk = 0; kk < 2; kk++) {
                    const int ko = 32 * j + 16 * kk + kh;
                    v8h bf[2];
#pragma unroll
                    for (int mi = 0; mi < 2; mi++) bf[mi] = *reinterpret_cast<const v8h *>(&sm.B[64 * wm + 32 * mi + lr][ko]);
#pragma unroll
                    for (int x = 0; x < MmqSmem<T>::NA; x++) {
                        v8h af[2];
#pragma unroll
                        for (int ni = 0; ni < 2; ni++) af[ni] = *reinterpret_cast<const v8h *>(&sm.A[x][64 * wn + 32 * ni + lr][ko]);
#pragma unroll
                        for (int ni = 0; ni < 2; ni++)
#pragma unroll
                            for (int mi = 0; mi < 2; mi++)
                                C[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ni], bf[mi], C[ni][mi], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int mi = 0; mi < 2; mi++) {
                    const float d8 = sm.d8[64 * wm + 32 * mi + lr][2 * st + j];
#pragma unroll
                    for (int ni = 0; ni < 2; ni++)
#pragma unroll
                        for (int e = 0; e < 16; e++) P[ni][mi][e] = __builtin_fmaf(C[ni][mi][e], d8, P[ni][mi][e]);
                }
            }
        }
        // ---- end of super-block: P * d (- dmin * min term) into acc ----
        if (T == T_Q4_K) {
            v16f Q[2][2];
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int b = 0; b < 2; b++) Q[a][b] = v16f{};
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                const int ko = 16 * kk + kh;
                v8bf am[2], bmv[2];
#pragma unroll
                for (int ni = 0; ni < 2; ni++) am[ni] = *reinterpret_cast<const v8bf *>(&sm.Amin[64 * wn + 32 * ni + lr][ko]);
#pragma unroll
                for (int mi = 0; mi < 2; mi++) bmv[mi] = *reinterpret_cast<const v8bf *>(&sm.Bmin[64 * wm + 32 * mi + lr][ko]);
#pragma unroll
                for (int ni = 0; ni < 2; ni++)
#pragma unroll
                    for (int mi = 0; mi < 2; mi++)
                        Q[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[ni], bmv[mi], Q[ni][mi], 0, 0, 0);
            }
#pragma unroll
            for (int ni = 0; ni < 2; ni++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int tr = 64 * wn + 32 * ni + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    const float d = sm.wd[tr], dm = sm.wdmin[tr];
#pragma unroll
                    for (int mi = 0; mi < 2; mi++) {
                        acc[ni][mi][e] = __builtin_fmaf(P[ni][mi][e], d, acc[ni][mi][e]);
                        acc[ni][mi][e] = __builtin_fmaf(Q[ni][mi][e], -dm, acc[ni][mi][e]);
                        P[ni][mi][e] = 0.0f;
                    }
                }
        } else {
#pragma unroll
            for (int ni = 0; ni < 2; ni++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int tr = 64 * wn + 32 * ni + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    const float d = sm.wd[tr];
#pragma unroll
                    for (int mi = 0; mi < 2; mi++) {
                        acc[ni][mi][e] = __builtin_fmaf(P[ni][mi][e], d, acc[ni][mi][e]);
                        P[ni][mi][e] = 0.0f;
                    }
                }
        }
    }

    // ---- epilogue ----
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
                    store4<YDT>(p.y, (int64_t)xr * p.ldy + n0, v, nv);
                }
            } else {
                const int64_t r = sm.route[col];
                const int64_t t = r / p.top_k;
                const float w = p.route_w ? p.route_w[r] : 0.0f;
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
                    if (p.route_w) { for (int i = 0; i < nv; i++) atomicAdd(&p.acc32[t * p.Np + n0 + i], w * h[i]); }
                    else store4<YDT>(p.y, r * p.Np + n0, h, nv);
                } else {
#pragma unroll
                    for (int ni = 0; ni < 2; ni++) {
                        const int64_t n0 = bn * NT + 64 * wn + 32 * ni + 8 * g + 4 * (lane >> 5);
                        if (n0 >= p.N) continue;
                        const int nv = (int)min<int64_t>(4, p.N - n0);
                        float v[4] = {acc[ni][mi][4 * g], acc[ni][mi][4 * g + 1], acc[ni][mi][4 * g + 2], acc[ni][mi][4 * g + 3]};
                        if (p.route_w) { for (int i = 0; i < nv; i++) atomicAdd(&p.acc32[t * p.Np + n0 + i], w * v[i]); }
                        else store4<YDT>(p.y, r * p.Np + n0, v, nv);
                    }
                }
            }
        }
    }
}

// ---- test hook: per-group int32 dots from the staged tiles and the MFMA ----
// Same staging (sub-scales forced to 1) and fragment layout as mmq_kernel.
template <int T>
__global__ __launch_bounds__(256) void mmq_dots_kernel(const uint8_t *__restrict__ W, int64_t N, int64_t K,
                                                       const _Float16 *__restrict__ xq, int64_t M, int64_t m_tiles,
                                                       int32_t *__restrict__ out) {
    __shared__ MmqSmem<T> sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t bm = (int64_t)blockIdx.x % m_tiles, bn = (int64_t)blockIdx.x / m_tiles;
    const int64_t row_bytes = K / 256 * Geom<T>::BYTES;
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
    for (int sb = 0; sb < (int)(K / 256); sb++) {
        __syncthreads();
        stage_meta<T, true>(sm, sb, K, nullptr, nullptr);
        for (int st = 0; st < 4; st++) {
            __syncthreads();
            stage_A<T>(sm, sb, st);
            stage_B<T>(sm, xq, K, (int64_t)sb * 256 + 64 * st);
            __syncthreads();
            for (int q16 = 0; q16 < 4; q16++) {                // 16-wide K steps of this stage
                v16f C[2][2];
                for (int a = 0; a < 2; a++) for (int b = 0; b < 2; b++) C[a][b] = v16f{};
                const int ko = 16 * q16 + kh;
                v8h bf[2];
                for (int mi = 0; mi < 2; mi++) bf[mi] = *reinterpret_cast<const v8h *>(&sm.B[64 * wm + 32 * mi + lr][ko]);
                for (int x = 0; x < MmqSmem<T>::NA; x++) {
                    v8h af[2];
                    for (int ni = 0; ni < 2; ni++) af[ni] = *reinterpret_cast<const v8h *>(&sm.A[x][64 * wn + 32 * ni + lr][ko]);
                    for (int ni = 0; ni < 2; ni++)
                        for (int mi = 0; mi < 2; mi++)
                            C[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ni], bf[mi], C[ni][mi], 0, 0, 0);
                }
                const int64_t kabs = (int64_t)sb * 256 + 64 * st + 16 * q16;
                for (int ni = 0; ni < 2; ni++)
                    for (int mi = 0; mi < 2; mi++)
                        for (int e = 0; e < 16; e++) {
                            const int64_t n = bn * NT + 64 * wn + 32 * ni + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                            const int64_t m = bm * MT + 64 * wm + 32 * mi + lr;
                            if (n >= N || m >= M) continue;
                            int32_t *o = out + (m * N + n) * gpr + kabs / G;
                            const int32_t v = (int32_t)C[ni][mi][e];
                            if (G == 16) *o = v;
                            else if ((q16 & 1) == 0) *o = v;
                            else *o += v;                         // same thread wrote the first half
                        }
            }
        }
    }
}

// ---------------------------------------------------------------------------
template <int T>
static void launch_t(bool moe, int epi, int ydt, const MmqParams &p, hipStream_t s) {
    const dim3 g((unsigned)(p.m_tiles * p.n_tiles)), b(256);
#define GGQ_L(MOE, EPI, YDT) hipLaunchKernelGGL((mmq_kernel<T, MOE, EPI, YDT>), g, b, 0, s, p)
    if (!moe) {
        if (ydt == DT_F32) GGQ_L(false, EPI_NONE_, DT_F32); else GGQ_L(false, EPI_NONE_, DT_BF16);
    } else if (epi == EPI_SWIGLU_) {
        if (ydt == DT_F32) GGQ_L(true, EPI_SWIGLU_, DT_F32); else GGQ_L(true, EPI_SWIGLU_, DT_BF16);
    } else {
        if (ydt == DT_F32) GGQ_L(true, EPI_NONE_, DT_F32); else GGQ_L(true, EPI_NONE_, DT_BF16);
    }
#undef GGQ_L
}

hipError_t launch_mmq(int t, bool moe, int epi, int ydt, const MmqParams &p, hipStream_t s) {
    if (p.m_tiles == 0 || p.n_tiles == 0) return hipSuccess;
    if (t == T_Q4_K) launch_t<T_Q4_K>(moe, epi, ydt, p, s);
    else if (t == T_Q6_K) launch_t<T_Q6_K>(moe, epi, ydt, p, s);
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
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ggq
