// Measured ceilings for the benchmark report, next to the published peaks: a
// plain streaming read of a device buffer (what HBM delivers to a kernel that
// does nothing else) and MFMA-only loops (what the matrix cores deliver with
// no memory traffic).  Not part of the method; bench-only exports.
#include "kernels.hpp"

namespace ggq {

// Grid-stride read, 8 independent 16-byte loads per lane per trip.  The XOR of
// the data is stored only if it equals a value the caller never plants, so
// the loads cannot be dropped and nothing is written in practice.
__global__ __launch_bounds__(256) void stream_read_kernel(const v4i *__restrict__ p, int64_t n16,
                                                          int *__restrict__ sink) {
    constexpr int U = 8;
    int acc = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        v4i v[U];
#pragma unroll
        for (int u = 0; u < U; u++) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const v4i v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x5a17c0de) sink[blockIdx.x] = acc;
}

typedef int v16i __attribute__((ext_vector_type(16)));

// KIND 0: v_mfma_f32_32x32x16_f16; KIND 1: v_mfma_i32_32x32x32_i8.  Four
// independent accumulators per wave, iters trips.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int64_t iters, int *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    int r = 0;
    if (KIND == 0) {
        v8h a, b;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            a[i] = (_Float16)(float)((lane + i) & 7);
            b[i] = (_Float16)(float)((lane * 3 + i) & 7);
        }
        v16f c[4] = {v16f{}, v16f{}, v16f{}, v16f{}};
        for (int64_t t = 0; t < iters; t++)
#pragma unroll
            for (int j = 0; j < 4; j++) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; j++) r += (int)c[j][0] + (int)c[j][15];
    } else {
        const v4i a = {lane, lane + 1, lane + 2, lane + 3}, b = {3 * lane, lane, 7, lane ^ 5};
        v16i c[4] = {v16i{}, v16i{}, v16i{}, v16i{}};
        for (int64_t t = 0; t < iters; t++)
#pragma unroll
            for (int j = 0; j < 4; j++) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; j++) r += c[j][0] + c[j][15];
    }
    if (r == 0x5a17c0de) sink[blockIdx.x] = r;
}

hipError_t launch_stream_read(const void *buf, int64_t bytes, int *sink, hipStream_t s) {
    if (bytes < 16) return hipSuccess;
    hipLaunchKernelGGL(stream_read_kernel, dim3(CEIL_READ_BLOCKS), dim3(256), 0, s, static_cast<const v4i *>(buf),
                       bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_mfma_loop(int kind, int64_t iters, int *sink, hipStream_t s) {
    if (kind == 0) hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(CEIL_MFMA_BLOCKS), dim3(256), 0, s, iters, sink);
    else hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(CEIL_MFMA_BLOCKS), dim3(256), 0, s, iters, sink);
    return hipGetLastError();
}

}  // namespace ggq
