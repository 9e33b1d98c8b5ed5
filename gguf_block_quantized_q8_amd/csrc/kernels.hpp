// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <algorithm>
#include "common.hpp"

namespace ggq {

// Zero the output rows of the inactive routes (id < 0 or id >= E) among
// routes [r0, r0 + 64) of the unweighted mul_mat_id output y[R][Np]: each lane
// reads one id, and the wave zeroes each inactive route's row with all 64
// lanes (inactive routes are rare, so most waves only read ids).  YDT: DT_F32,
// DT_BF16 (any 16-bit output) or DT_Q8_1 (Np / 32 all-zero blocks, what an
// all-zero row quantizes to).  Called by whole waves.
template <int YDT>
__device__ __forceinline__ void zero_dead_routes(const int32_t *__restrict__ ids, int64_t R, int64_t E, int64_t Np,
                                                 void *__restrict__ y, int64_t r0, int lane) {
    bool dead = false;
    if (r0 + lane < R) {
        const int32_t e = ids[r0 + lane];
        dead = e < 0 || e >= E;
    }
    for (uint64_t m = __ballot(dead); m; m &= m - 1) {
        const int64_t r = r0 + __builtin_ctzll(m);
        if (YDT == DT_Q8_1) {
            const int64_t words = Np / QK8_1 * (Q8_1_BYTES / 4);
            uint32_t *o = reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(y) + r * (Np / QK8_1) * Q8_1_BYTES);
            for (int64_t i = lane; i < words; i += 64) o[i] = 0u;
        } else {
            for (int64_t n = lane; n < Np; n += 64) {
                if (YDT == DT_F32) static_cast<float *>(y)[r * Np + n] = 0.0f;
                else static_cast<uint16_t *>(y)[r * Np + n] = 0;
            }
        }
    }
}

// ---- convert.hip ----
// q8 != nullptr: 40-byte q8_1 blocks; xq != nullptr (K % 256 == 0): the MMQ operand
// (fp16 quants xq, d xd, min-term operand xm), row-major or tiled (dense MMQ; rows a
// multiple of 64 allocated, xq_index)
hipError_t launch_quantize(const void *x, int xdt, int64_t M, int64_t K, int64_t ldx, uint8_t *q8, _Float16 *xq,
                           float *xd, uint16_t *xm, bool tiled, hipStream_t s);
hipError_t launch_q8_1_to_planar(const uint8_t *q8, int64_t M, int64_t K, _Float16 *xq, float *xd, uint16_t *xm,
                                 bool tiled, hipStream_t s);
// y row r (of n) = table row ids[r] (r without ids), zeros for ids outside [0, rows); rows ldy apart
hipError_t launch_dequant(int t, const uint8_t *W, int64_t rows, int64_t K, const int32_t *ids, int64_t n, void *y,
                          int ydt, int64_t ldy, hipStream_t s);
hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t s);
hipError_t launch_route_sum(const void *o, const int32_t *ids, const float *w, int64_t T, int top_k, int64_t E,
                            int64_t Np, void *y, int ydt, hipStream_t s);
// y[m][n] = sum over k < ks, in order, of part[k][m][n] (fp32), stored as ydt (fp16 when y_f16)
hipError_t launch_splitk_reduce(const float *part, int ks, int64_t M, int64_t N, void *y, int ydt, int y_f16,
                                int64_t ldy, hipStream_t s);
hipError_t launch_zero_inactive(const int32_t *ids, int64_t R, int64_t E, int64_t Np, void *y, int ydt,
                                hipStream_t s);

// ---- route.hip ----
// Work list of (expert, first sorted route, route count) triples, one per
// tile of at most J routes of one expert; built on the device from ids.
struct RouteTables {
    uint32_t *bad;        // count of ids >= E (workspace offset 0)
    uint32_t *counts;     // [E]
    uint32_t *offsets;    // [E + 1] exclusive scan of counts
    uint32_t *tile_off;   // [E + 1] exclusive scan of ceil(count / J)
    uint32_t *ntiles;     // [1] total tiles
    int32_t *rank;        // [R] position of a route inside its expert list (-1: inactive)
    int32_t *perm;        // [R] routes sorted by expert
    int4 *tiles;          // [max_tiles] {expert, start, count, 0}
};
int64_t route_max_tiles(int64_t R, int64_t E, int J);
// zy != nullptr: also zero the rows of the inactive routes in zy[R][Np] (dtype zdt) when the
// build runs as one workgroup (returns whether it did; else the caller zeroes them)
hipError_t launch_route_build(const int32_t *ids, int64_t R, int64_t E, int J, const RouteTables &rt,
                              hipStream_t s, void *zy = nullptr, int64_t Np = 0, int zdt = 0, bool *zeroed = nullptr);

// ---- mmvq.hip ----
struct MmvqParams {
    const uint8_t *W;
    int64_t row_bytes;
    int64_t expert_stride;
    int64_t N;            // weight rows of one matrix
    int64_t Np;           // output rows (N, or N/2 with SwiGLU)
    int64_t npairs;       // row pairs handled (ceil(N/2), or Np with SwiGLU)
    int64_t K;
    // work geometry (set by the launcher)
    int units;            // decode units per row
    int seg;              // lanes per row segment (power of two, <= 64)
    int upl;              // units per lane per work item
    // activations: float rows quantized in the kernel prologue (xsrc = DT_F32 /
    // DT_BF16, x with row stride ldx elements) or q8_1 rows copied (xsrc =
    // DT_Q8_1, q8 with q8_row bytes per row)
    int xsrc;
    const void *x;
    int64_t ldx;
    const uint8_t *q8;
    int64_t q8_row;
    int64_t x_bytes;      // readable bytes from x (or q8): the activation buffer's extent
    int64_t M;            // dense: activation rows (columns of y^T)
    void *y;
    int64_t ldy;
    // routed experts
    const int32_t *perm;
    const int4 *groups;
    const uint32_t *ngroups;
    int top_k;
    int x_per_route;
    const float *route_w;
    void *oroute;         // weighted: per-route outputs [R][Np] in the output dtype (fp32, or the
                          // 16-bit type of y), summed per token afterwards
    int y_f16;            // 16-bit output is fp16 (else bf16)
    int64_t groups_expected;   // routed: expected active groups (min(E, routes))
    // routed, one route per group without route tables: group g is route g (ids[g]
    // its expert); perm / groups / ngroups unused.  Null otherwise.
    const int32_t *ids;
    int64_t R, E;         // direct: routes and experts
    uint32_t *bad;        // direct: receives the count of ids >= E (group 0 writes it)
    // set by the launcher
    int64_t w_bytes;        // readable weight bytes from W (N*row_bytes, or up to the last expert's last row)
    int64_t act_lds_bytes;  // LDS bytes of the activation region (set by the launcher)
    int stage_bpc;          // blocks per staged row chunk (set by the launcher)
    int stage_cps;          // 16-byte pieces per staged row chunk (set by the launcher)
    int stage_ninst;        // 1 KB copy instructions per work item (set by the launcher)
    int deep;               // two work items in flight per wave (set by the launcher)
    int act_dma;            // activation rows copied to LDS by DMA in the prologue (set by the launcher)
    uint32_t nb_magic;      // ceil(2^32 / (K / 32)): block index -> column by one high multiply (set by the launcher)
    uint32_t cps_magic;     // ceil(2^32 / stage_cps): piece index -> row slot (set by the launcher)
    uint32_t ppc_magic;     // ceil(2^32 / (raw activation row bytes / 16)) when act_dma (set by the launcher)
    int64_t x_stride;       // bytes between activation rows (x or q8) (set by the launcher)
    uint32_t raw_region;    // LDS bytes after the first item buffers: second buffers, or the raw rows if larger (set by the launcher)
};
constexpr size_t MMVQ_LDS_MAX = 64 * 1024;     // activation bytes staged per block
int mmvq_max_cols(int t, int64_t K);          // largest column group (8, 4, 2, 1) whose activations fit in LDS
// whether MMVQ takes this K: one activation row fits its LDS region (K up to about 52K for
// Q4_K / Q5_K / Q8_0 / Q4_0, 43K for Q6_K) and a row chunk fits one work item
bool mmvq_supported(int t, int64_t K);
hipError_t launch_mmvq(int t, int nc, bool moe, int epi, int ydt, const MmvqParams &p, int64_t ngroups_bound,
                       hipStream_t s);
hipError_t launch_mmvq_dots(int t, const uint8_t *W, int64_t N, int64_t K, const uint8_t *q8, int64_t M,
                            int32_t *out, hipStream_t s);

// ---- mmq.hip ----
struct MmqParams {
    const uint8_t *W;
    int64_t row_bytes;
    int64_t expert_stride;
    int64_t N;            // weight rows of one matrix
    int64_t Np;           // output rows (N, or N/2 with SwiGLU)
    int64_t K;
    const _Float16 *xq;   // activations: fp16 quants (dense: tiled layout, routed: row-major; xq_index)
    const float *xd;      // q8_1 d (xd_index)
    const uint16_t *xm;   // bf16 min-term operand (xm_index, planar_write_min)
    int64_t x_rows;       // rows of the operand (dense: M padded to 64; routed: T, or T * top_k)
    int64_t M;            // dense: activation rows
    int64_t m_tiles;      // dense: tiles along M; routed: tile-list bound
    int64_t n_tiles;      // tiles along the output rows
    void *y;
    int64_t ldy;
    // routed experts
    const int32_t *perm;
    const int4 *tiles;
    const uint32_t *ntiles;
    int top_k;
    int x_per_route;
    const float *route_w;
    void *oroute;         // weighted: per-route outputs [R][Np] in the output dtype (fp32, or the
                          // 16-bit type of y), summed per token afterwards
    int q8_round;         // q8_1 output: round the values to bf16 (1) or fp16 (2) before quantizing
    int y_f16;            // 16-bit output is fp16 (else bf16)
    // dense split K: ksplit workgroups per tile, each over K / ksplit (whole super-blocks),
    // writing fp32 partial sums part[ksplit][M][N] that splitk_reduce adds in slice order
    int ksplit;
    float *part;
};
constexpr int MMQ_NT = 128;   // weight rows per workgroup tile
constexpr int MMQ_MT = 256;   // activation rows (routes) per workgroup tile
hipError_t launch_mmq(int t, bool moe, int epi, int ydt, const MmqParams &p, hipStream_t s);
hipError_t launch_mmq_dots(int t, const uint8_t *W, int64_t N, int64_t K, const _Float16 *xq, int64_t M,
                           int32_t *out, hipStream_t s);

// ---- ceiling.hip (bench-only measured ceilings) ----
constexpr int CEIL_READ_BLOCKS = 256;    // workgroups of the streaming read (256 threads each)
constexpr int CEIL_MFMA_BLOCKS = 1024;   // workgroups of the MFMA loops (4 waves each)
// reads bytes / 16 whole 16-byte pieces of buf (16-byte aligned); sink: CEIL_READ_BLOCKS ints
hipError_t launch_stream_read(const void *buf, int64_t bytes, int *sink, hipStream_t s);
// kind 0: fp16 32x32x16, 1: int8 32x32x32; each wave runs iters x 4 MFMAs; sink: CEIL_MFMA_BLOCKS ints
hipError_t launch_mfma_loop(int kind, int64_t iters, int *sink, hipStream_t s);
// the MMQ inner loop on a 64 x 64 wave tile: kind 0 fp16 MFMA + one fma per output per block,
// kind 1 int8 MFMA + multiply, convert and fma per output per block, kind 2 LDS reads only;
// 256 * blocks_per_cu workgroups of 4 waves; sink: 256 * blocks_per_cu ints
hipError_t launch_inner_loop(int kind, int blocks_per_cu, int64_t iters, int *sink, hipStream_t s);

}  // namespace ggq
