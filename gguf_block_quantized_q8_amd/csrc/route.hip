// Routed-expert work list built on the device, with no host synchronization:
// histogram of expert ids -> exclusive scans -> scatter of routes by expert ->
// flat list of (expert, route tile) pairs of width J.  Only the tiles that hold
// routes are listed; the kernels that consume the list are launched with the
// host-side bound route_max_tiles() and blocks past the device count exit.
#include "kernels.hpp"

namespace ggq {

int64_t route_max_tiles(int64_t R, int64_t E, int J) {
    // sum_e ceil(c_e / J) <= sum_e (c_e / J + 1 for c_e > 0) <= R / J + min(E, R)
    return R / J + std::min<int64_t>(E, R) + 1;
}

__global__ __launch_bounds__(256) void route_count_kernel(const int32_t *__restrict__ ids, int64_t R, int64_t E,
                                                          uint32_t *__restrict__ counts, int32_t *__restrict__ rank,
                                                          uint32_t *__restrict__ bad) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= R) return;
    const int32_t e = ids[r];
    if (e >= 0 && e < E) {
        rank[r] = (int32_t)atomicAdd(&counts[e], 1u);
    } else {
        rank[r] = -1;
        if (e >= E) atomicAdd(bad, 1u);
    }
}

// Larger problems with E <= 4096: 4096 routes per workgroup, ranks from LDS
// atomics on a per-workgroup histogram, then one global atomic per expert
// present in the workgroup (instead of one per route on the few hot counters).
constexpr int ROUTE_CHUNK = 4096;
constexpr int64_t ROUTE_LDS_E = 4096;

__global__ __launch_bounds__(1024) void route_count_lds_kernel(const int32_t *__restrict__ ids, int64_t R, int64_t E,
                                                              uint32_t *__restrict__ counts, int32_t *__restrict__ rank,
                                                              uint32_t *__restrict__ bad) {
    __shared__ uint32_t s_cnt[ROUTE_LDS_E];
    const int tid = threadIdx.x;
    for (int64_t e = tid; e < E; e += 1024) s_cnt[e] = 0;
    __syncthreads();
    const int64_t r0 = (int64_t)blockIdx.x * ROUTE_CHUNK;
    int32_t ex[ROUTE_CHUNK / 1024], k[ROUTE_CHUNK / 1024];
#pragma unroll
    for (int i = 0; i < ROUTE_CHUNK / 1024; i++) {
        const int64_t r = r0 + i * 1024 + tid;
        ex[i] = r < R ? ids[r] : -1;
        k[i] = -1;
        if (ex[i] >= 0 && ex[i] < E) k[i] = (int32_t)atomicAdd(&s_cnt[ex[i]], 1u);
        else if (ex[i] >= E) atomicAdd(bad, 1u);
    }
    __syncthreads();
    for (int64_t e = tid; e < E; e += 1024) {
        const uint32_t c = s_cnt[e];
        if (c) s_cnt[e] = atomicAdd(&counts[e], c);                // this workgroup's first rank in expert e
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ROUTE_CHUNK / 1024; i++) {
        const int64_t r = r0 + i * 1024 + tid;
        if (r < R) rank[r] = k[i] >= 0 ? (int32_t)s_cnt[ex[i]] + k[i] : -1;
    }
}

// Single workgroup: exclusive scans of the counts and of the tile counts,
// then the tile list.
__global__ __launch_bounds__(1024) void route_scan_kernel(const uint32_t *__restrict__ counts, int64_t E, int J,
                                                          uint32_t *__restrict__ offsets, uint32_t *__restrict__ tile_off,
                                                          uint32_t *__restrict__ ntiles, int4 *__restrict__ tiles) {
    __shared__ uint32_t s_c[1024], s_t[1024];
    __shared__ uint32_t carry_c, carry_t;
    const int tid = threadIdx.x;
    if (tid == 0) { carry_c = 0; carry_t = 0; }
    __syncthreads();
    for (int64_t base = 0; base < E; base += 1024) {
        const int64_t e = base + tid;
        const uint32_t c = e < E ? counts[e] : 0u;
        const uint32_t nt = (c + (uint32_t)J - 1) / (uint32_t)J;
        s_c[tid] = c;
        s_t[tid] = nt;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {      // inclusive Hillis-Steele scan
            uint32_t vc = tid >= off ? s_c[tid - off] : 0u;
            uint32_t vt = tid >= off ? s_t[tid - off] : 0u;
            __syncthreads();
            s_c[tid] += vc;
            s_t[tid] += vt;
            __syncthreads();
        }
        const uint32_t oc = carry_c + s_c[tid] - c;     // exclusive
        const uint32_t ot = carry_t + s_t[tid] - nt;
        if (e < E) {
            offsets[e] = oc;
            tile_off[e] = ot;
            for (uint32_t i = 0; i < nt; i++)
                tiles[ot + i] = int4{(int)e, (int)(oc + i * (uint32_t)J), (int)min((uint32_t)J, c - i * (uint32_t)J), 0};
        }
        __syncthreads();
        if (tid == 1023) { carry_c += s_c[1023]; carry_t += s_t[1023]; }
        __syncthreads();
    }
    if (tid == 0) {
        offsets[E] = carry_c;
        tile_off[E] = carry_t;
        *ntiles = carry_t;
    }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(const int32_t *__restrict__ ids, int64_t R,
                                                            const uint32_t *__restrict__ offsets,
                                                            const int32_t *__restrict__ rank,
                                                            int32_t *__restrict__ perm) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= R) return;
    const int32_t k = rank[r];
    if (k < 0) return;
    perm[offsets[ids[r]] + k] = (int32_t)r;
}

// Small problems: the whole build in one workgroup (counts in LDS), one launch.
constexpr int64_t ROUTE_SMALL_R = 16384;
constexpr int64_t ROUTE_SMALL_E = 4096;

// ZDT >= 0: also zero the inactive routes' rows of the unweighted output zy
// (what zero_inactive_kernel does), saving that launch.
template <int ZDT>
__global__ __launch_bounds__(1024) void route_build_small_kernel(const int32_t *__restrict__ ids, int64_t R, int64_t E,
                                                                 int J, uint32_t *__restrict__ counts,
                                                                 uint32_t *__restrict__ offsets,
                                                                 uint32_t *__restrict__ tile_off,
                                                                 uint32_t *__restrict__ ntiles, int4 *__restrict__ tiles,
                                                                 int32_t *__restrict__ rank, int32_t *__restrict__ perm,
                                                                 uint32_t *__restrict__ bad, void *__restrict__ zy,
                                                                 int64_t Np) {
    __shared__ uint32_t s_cnt[ROUTE_SMALL_E], s_off[ROUTE_SMALL_E];
    __shared__ uint32_t s_c[1024], s_t[1024];
    __shared__ uint32_t s_bad, carry_c, carry_t;
    const int tid = threadIdx.x;
    for (int64_t e = tid; e < E; e += 1024) s_cnt[e] = 0;
    if (tid == 0) { s_bad = 0; carry_c = 0; carry_t = 0; }
    __syncthreads();
    // ranks within each expert (LDS atomics)
    for (int64_t r = tid; r < R; r += 1024) {
        const int32_t e = ids[r];
        int32_t k = -1;
        if (e >= 0 && e < E) k = (int32_t)atomicAdd(&s_cnt[e], 1u);
        else if (e >= E) atomicAdd(&s_bad, 1u);
        rank[r] = k;
    }
    __syncthreads();
    // exclusive scans of the counts and of the tile counts, tile list
    for (int64_t base = 0; base < E; base += 1024) {
        const int64_t e = base + tid;
        const uint32_t c = e < E ? s_cnt[e] : 0u;
        const uint32_t nt = (c + (uint32_t)J - 1) / (uint32_t)J;
        s_c[tid] = c;
        s_t[tid] = nt;
        __syncthreads();
        for (int o = 1; o < 1024; o <<= 1) {
            const uint32_t vc = tid >= o ? s_c[tid - o] : 0u;
            const uint32_t vt = tid >= o ? s_t[tid - o] : 0u;
            __syncthreads();
            s_c[tid] += vc;
            s_t[tid] += vt;
            __syncthreads();
        }
        const uint32_t oc = carry_c + s_c[tid] - c, ot = carry_t + s_t[tid] - nt;
        if (e < E) {
            s_off[e] = oc;
            counts[e] = c;
            offsets[e] = oc;
            tile_off[e] = ot;
            for (uint32_t i = 0; i < nt; i++)
                tiles[ot + i] = int4{(int)e, (int)(oc + i * (uint32_t)J), (int)min((uint32_t)J, c - i * (uint32_t)J), 0};
        }
        __syncthreads();
        if (tid == 1023) { carry_c += s_c[1023]; carry_t += s_t[1023]; }
        __syncthreads();
    }
    // scatter (each thread reads back the ranks it wrote)
    for (int64_t r = tid; r < R; r += 1024) {
        const int32_t k = rank[r];
        if (k >= 0) perm[s_off[ids[r]] + k] = (int32_t)r;
    }
    if (tid == 0) {
        offsets[E] = carry_c;
        tile_off[E] = carry_t;
        *ntiles = carry_t;
        *bad = s_bad;
    }
    if (ZDT >= 0)
        for (int64_t r0 = (int64_t)(tid & ~63); r0 < R; r0 += 1024) zero_dead_routes<ZDT>(ids, R, E, Np, zy, r0, tid & 63);
}

hipError_t launch_route_build(const int32_t *ids, int64_t R, int64_t E, int J, const RouteTables &rt,
                              hipStream_t s, void *zy, int64_t Np, int zdt, bool *zeroed) {
    if (zeroed) *zeroed = false;
    if (R <= ROUTE_SMALL_R && E <= ROUTE_SMALL_E) {
#define GGQ_RB(Z) hipLaunchKernelGGL(route_build_small_kernel<Z>, dim3(1), dim3(1024), 0, s, ids, R, E, J, rt.counts, \
                                     rt.offsets, rt.tile_off, rt.ntiles, rt.tiles, rt.rank, rt.perm, rt.bad, zy, Np)
        if (!zy) GGQ_RB(-1);
        else if (zdt == DT_F32) GGQ_RB(DT_F32);
        else if (zdt == DT_Q8_1) GGQ_RB(DT_Q8_1);
        else GGQ_RB(DT_BF16);                                   // any 16-bit output: 16-bit zeros
#undef GGQ_RB
        if (zeroed) *zeroed = zy != nullptr;
        return hipGetLastError();
    }
    hipError_t err = launch_fill_u32(rt.counts, E, 0u, s);
    if (err != hipSuccess) return err;
    err = launch_fill_u32(rt.bad, 1, 0u, s);
    if (err != hipSuccess) return err;
    const unsigned g = (unsigned)((R + 255) / 256);
    if (R > 0 && E <= ROUTE_LDS_E)
        hipLaunchKernelGGL(route_count_lds_kernel, dim3((unsigned)((R + ROUTE_CHUNK - 1) / ROUTE_CHUNK)), dim3(1024), 0, s,
                           ids, R, E, rt.counts, rt.rank, rt.bad);
    else if (R > 0)
        hipLaunchKernelGGL(route_count_kernel, dim3(g), dim3(256), 0, s, ids, R, E, rt.counts, rt.rank, rt.bad);
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, rt.counts, E, J, rt.offsets, rt.tile_off,
                       rt.ntiles, rt.tiles);
    if (R > 0) hipLaunchKernelGGL(route_scatter_kernel, dim3(g), dim3(256), 0, s, ids, R, rt.offsets, rt.rank, rt.perm);
    return hipGetLastError();
}

}  // namespace ggq
