// C ABI: argument validation, workspace carving, path dispatch.  All checks
// run on the host before anything is launched; nothing here synchronizes.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kernels.hpp"
#include "../../include/ggq.h"

using namespace ggq;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(GGQ_ERR_HIP, "%s: HIP error %s", what, hipGetErrorString(e));
    return GGQ_OK;
}

const char *tname(int t) {
    return t == GGQ_Q4_0 ? "Q4_0" : t == GGQ_Q8_0 ? "Q8_0" : t == GGQ_Q4_K ? "Q4_K" : t == GGQ_Q5_K ? "Q5_K"
         : t == GGQ_Q6_K ? "Q6_K" : "?";
}

bool known_type(int t) { return t == GGQ_Q4_0 || t == GGQ_Q8_0 || t == GGQ_Q4_K || t == GGQ_Q5_K || t == GGQ_Q6_K; }
// MMQ kernels: every type; Q8_0 / Q4_0 (32-weight blocks) when K is a multiple of
// 256 (the kernel stages activation scales 8 blocks at a time).
bool has_mmq(int t, int64_t K) {
    return t == GGQ_Q4_K || t == GGQ_Q5_K || t == GGQ_Q6_K || ((t == GGQ_Q8_0 || t == GGQ_Q4_0) && K % 256 == 0);
}
// Float element types of activations and outputs: fp32, bf16, fp16.
bool float_dt(int dt) { return dt == GGQ_F32 || dt == GGQ_BF16 || dt == GGQ_F16; }
// Kernel instantiation for an output dtype: the 16-bit ones share one (fp16 by flag).
int kernel_dt(int dt) { return dt == GGQ_F16 ? GGQ_BF16 : dt; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// activation rows quantized on the fly (MMVQ: none, it stages them in LDS; MMQ: planar fp16
// quants, d, and the bf16 min-term operand)
size_t act_bytes(bool mmq, int64_t rows, int64_t K) {
    if (mmq) return align256((size_t)rows * K * 2) + align256((size_t)rows * (K / 32) * 4) + align256((size_t)rows * (K / 4));
    return 0;
}

// rows of the dense MMQ operand: a multiple of 64 (the tiled layout's d groups)
int64_t mmq_rows(int64_t M) { return (M + 63) & ~(int64_t)63; }

struct Carve {
    uint8_t *base;
    size_t off = 0;
    explicit Carve(void *b) : base(static_cast<uint8_t *>(b)) {}
    template <class T> T *take(size_t bytes) {
        T *p = reinterpret_cast<T *>(base ? base + off : nullptr);
        off += align256(bytes);
        return p;
    }
};

struct Planar {
    _Float16 *xq;
    float *xd;
    uint16_t *xm;
};

Planar carve_planar(Carve &c, int64_t rows, int64_t K) {
    Planar p;
    p.xq = c.take<_Float16>((size_t)rows * K * 2);
    p.xd = c.take<float>((size_t)rows * (K / 32) * 4);
    p.xm = c.take<uint16_t>((size_t)rows * (K / 4));
    return p;
}

// Dense dispatch: MMVQ for up to 16 activation rows, MMQ above (when it has a kernel for the type and K).
// Measured on Q4_K 4096 x 4096 (caches evicted) and 8192 x 2048: MMVQ is ahead through
// M = 16 (two 8-column groups), MMQ from M = 24.
constexpr int64_t MMVQ_MAX_ROWS = 16;
// Routed dispatch: MMVQ-id while the routes per expert stay at or below this mean,
// MMQ-id above.  Measured on the E=256 top-8 H=2048 I=512 projections (caches
// evicted): gate_up crosses over between 256 and 384 tokens (8 and 12 routes per
// expert), the down projection between 384 and 512 (12 and 16).
constexpr int64_t MMVQ_ID_MAX_ROUTES_PER_EXPERT = 12;

// AUTO also takes MMQ when MMVQ cannot hold a row of K activations in LDS.
bool use_mmq(int wt, int64_t K, int64_t M, int path) {
    if (path == GGQ_PATH_MMQ) return true;
    if (path == GGQ_PATH_MMVQ) return false;
    return has_mmq(wt, K) && (M > MMVQ_MAX_ROWS || !mmvq_supported(wt, K));
}

bool use_mmq_id(int wt, int64_t K, int64_t R, int64_t E, int path) {
    if (path == GGQ_PATH_MMQ) return true;
    if (path == GGQ_PATH_MMVQ) return false;
    return has_mmq(wt, K) && (R > MMVQ_ID_MAX_ROUTES_PER_EXPERT * E || !mmvq_supported(wt, K));
}

int mmvq_too_long(const char *what, int wt, int64_t K) {
    int64_t kmax = 65536 / block_len(wt) * block_len(wt);
    while (kmax > 0 && !mmvq_supported(wt, kmax)) kmax -= block_len(wt);
    return fail(GGQ_ERR_UNSUPPORTED, "%s: K=%lld is too long for the MMVQ path of %s (a row of K activations must fit "
                "its 64 KB of LDS: K <= %lld)%s", what, (long long)K, tname(wt), (long long)kmax,
                has_mmq(wt, K) ? "; use MMQ" : "");
}

// Dense MMQ split K: with fewer tiles than one workgroup per CU (256), split
// K (in whole super-blocks, at most 8 ways) until the grid fills the chip.
int mmq_ksplit(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + MMQ_MT - 1) / MMQ_MT) * ((N + MMQ_NT - 1) / MMQ_NT), nsb = K / 256;
    int ks = 1;
    while (ks < 8 && nsb % (2 * ks) == 0 && tiles * 2 * ks <= 256) ks *= 2;
    return ks;
}

size_t splitk_bytes(int64_t M, int64_t N, int64_t K) {
    const int ks = mmq_ksplit(M, N, K);
    return ks > 1 ? align256((size_t)ks * M * N * 4) : 0;
}

int check_weights(int wt, int64_t N, int64_t K) {
    if (!known_type(wt))
        return fail(GGQ_ERR_UNSUPPORTED, "ggml type %d is not supported (Q4_0=2, Q8_0=8, Q4_K=12, Q5_K=13, Q6_K=14)", wt);
    if (N < 0 || K <= 0) return fail(GGQ_ERR_INVALID, "ggml type %s: bad shape N=%lld K=%lld", tname(wt), (long long)N, (long long)K);
    if (K % block_len(wt) != 0)
        return fail(GGQ_ERR_INVALID, "ggml type %s K=%lld is not a multiple of the block length %lld", tname(wt),
                    (long long)K, (long long)block_len(wt));
    return GGQ_OK;
}

int nc_for(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

// Routes per MMVQ-id group, from the mean routes per expert m = R / E.  Measured
// on the E=256 top-8 projections (uniform and skewed routing alike): one route
// per group is fastest up to m = 1 (T <= 32: the single-column kernel streams the
// weights best and experts with a second route are few), four from m = 2 to
// m = 4 (T = 64, 128), eight above.
int g_id_cols_override = 0;                                // bench hook: 0 = the rule below
int mmvq_id_cols(int wt, int64_t R, int64_t E, int64_t K) {
    if (g_id_cols_override) return std::min(g_id_cols_override, mmvq_max_cols(wt, K));
    const int j = R <= E ? 1 : R <= 4 * E ? 4 : 8;
    return std::min(j, mmvq_max_cols(wt, K));
}

}  // namespace

extern "C" {

const char *ggq_last_error(void) { return g_err; }

size_t ggq_row_bytes(int type, int64_t K) {
    if (!known_type(type) || K < 0 || K % block_len(type)) return 0;
    return (size_t)(K / block_len(type) * block_bytes(type));
}

size_t ggq_q8_1_bytes(int64_t M, int64_t K) {
    if (M < 0 || K < 0) return 0;
    return (size_t)M * (size_t)(K / 32) * Q8_1_BYTES;
}

int ggq_quantize_q8_1(const void *x, int xdt, int64_t M, int64_t K, int64_t ldx, void *q8, void *stream) {
    g_err[0] = 0;
    if (!float_dt(xdt)) return fail(GGQ_ERR_UNSUPPORTED, "quantize_q8_1: input dtype %d must be F32, BF16 or F16", xdt);
    if (M < 0 || K < 0 || K % 32) return fail(GGQ_ERR_INVALID, "quantize_q8_1: K=%lld must be a non-negative multiple of 32", (long long)K);
    if (ldx < K) return fail(GGQ_ERR_INVALID, "quantize_q8_1: ldx=%lld < K=%lld", (long long)ldx, (long long)K);
    if (M == 0 || K == 0) return GGQ_OK;
    if (!x || !q8) return fail(GGQ_ERR_INVALID, "quantize_q8_1: null pointer");
    if (!aligned16(x) || !aligned16(q8)) return fail(GGQ_ERR_INVALID, "quantize_q8_1: pointers must be 16-byte aligned");
    return hip_status(launch_quantize(x, xdt, M, K, ldx, static_cast<uint8_t *>(q8), nullptr, nullptr, nullptr, false,
                                      static_cast<hipStream_t>(stream)), "quantize_q8_1");
}

int ggq_dequantize(int wt, const void *W, int64_t rows, int64_t K, void *y, int ydt, void *stream) {
    g_err[0] = 0;
    int rc = check_weights(wt, rows, K);
    if (rc) return rc;
    if (!float_dt(ydt)) return fail(GGQ_ERR_UNSUPPORTED, "dequantize: output dtype %d must be F32, BF16 or F16", ydt);
    if (rows == 0) return GGQ_OK;
    if (!W || !y) return fail(GGQ_ERR_INVALID, "dequantize: null pointer");
    if (!aligned16(W) || !aligned16(y)) return fail(GGQ_ERR_INVALID, "dequantize: pointers must be 16-byte aligned");
    return hip_status(launch_dequant(wt, static_cast<const uint8_t *>(W), rows, K, nullptr, rows, y, ydt, K,
                                     static_cast<hipStream_t>(stream)),
                      "dequantize");
}

int ggq_get_rows(int wt, const void *W, int64_t rows, int64_t K, const int32_t *ids, int64_t n, void *y, int ydt,
                 int64_t ldy, void *stream) {
    g_err[0] = 0;
    int rc = check_weights(wt, rows, K);
    if (rc) return rc;
    if (!float_dt(ydt)) return fail(GGQ_ERR_UNSUPPORTED, "get_rows: output dtype %d must be F32, BF16 or F16", ydt);
    if (n < 0) return fail(GGQ_ERR_INVALID, "get_rows: n=%lld < 0", (long long)n);
    if (ldy < K) return fail(GGQ_ERR_INVALID, "get_rows: ldy=%lld < K=%lld", (long long)ldy, (long long)K);
    if (ldy % (ydt == GGQ_F32 ? 4 : 8))
        return fail(GGQ_ERR_INVALID, "get_rows: ldy=%lld must keep output rows 16-byte aligned", (long long)ldy);
    if (n == 0) return GGQ_OK;
    if (!W || !ids || !y) return fail(GGQ_ERR_INVALID, "get_rows: null pointer");
    if (!aligned16(W) || !aligned16(y)) return fail(GGQ_ERR_INVALID, "get_rows: W and y must be 16-byte aligned");
    return hip_status(launch_dequant(wt, static_cast<const uint8_t *>(W), rows, K, ids, n, y, ydt, ldy,
                                     static_cast<hipStream_t>(stream)),
                      "get_rows");
}

size_t ggq_mul_mat_ws(int wt, int64_t N, int64_t K, int xdt, int64_t M, int path) {
    if (!known_type(wt) || M <= 0 || N <= 0 || K <= 0 || K % block_len(wt)) return 0;
    const bool mmq = use_mmq(wt, K, M, path);
    return act_bytes(mmq, mmq ? mmq_rows(M) : M, K) + (mmq ? splitk_bytes(M, N, K) : 0);
}

int ggq_mul_mat(int wt, const void *W, int64_t N, int64_t K, const void *x, int xdt, int64_t M, int64_t ldx, void *y,
                int ydt, int64_t ldy, void *ws, size_t ws_bytes, int path, void *stream) {
    g_err[0] = 0;
    int rc = check_weights(wt, N, K);
    if (rc) return rc;
    if (!float_dt(xdt) && xdt != GGQ_Q8_1) return fail(GGQ_ERR_UNSUPPORTED, "mul_mat: input dtype %d", xdt);
    if (!float_dt(ydt)) return fail(GGQ_ERR_UNSUPPORTED, "mul_mat: output dtype %d must be F32, BF16 or F16", ydt);
    if (path != GGQ_PATH_AUTO && path != GGQ_PATH_MMVQ && path != GGQ_PATH_MMQ) return fail(GGQ_ERR_INVALID, "mul_mat: bad path %d", path);
    if (path == GGQ_PATH_MMQ && !has_mmq(wt, K))
        return fail(GGQ_ERR_UNSUPPORTED, "mul_mat: MMQ path has no %s kernel for K=%lld (Q8_0 / Q4_0 need K %% 256 == 0); use MMVQ", tname(wt), (long long)K);
    if (M < 0) return fail(GGQ_ERR_INVALID, "mul_mat: M=%lld < 0", (long long)M);
    if (xdt != GGQ_Q8_1 && ldx < K) return fail(GGQ_ERR_INVALID, "mul_mat: ldx=%lld < K=%lld", (long long)ldx, (long long)K);
    if (ldy < N) return fail(GGQ_ERR_INVALID, "mul_mat: ldy=%lld < N=%lld", (long long)ldy, (long long)N);
    if (M == 0 || N == 0) return GGQ_OK;
    if (!W || !x || !y) return fail(GGQ_ERR_INVALID, "mul_mat: null pointer");
    if (!aligned16(W) || !aligned16(x) || !aligned16(y)) return fail(GGQ_ERR_INVALID, "mul_mat: pointers must be 16-byte aligned");
    const size_t need = ggq_mul_mat_ws(wt, N, K, xdt, M, path);
    if (ws_bytes < need || (need && !ws)) return fail(GGQ_ERR_WORKSPACE, "mul_mat: workspace %zu bytes < %zu required", ws_bytes, need);
    if (need && !aligned16(ws)) return fail(GGQ_ERR_INVALID, "mul_mat: workspace must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool mmq = use_mmq(wt, K, M, path);
    if (!mmq && !mmvq_supported(wt, K)) return mmvq_too_long("mul_mat", wt, K);
    const int64_t rb = (int64_t)ggq_row_bytes(wt, K);
    Carve c(ws);
    if (!mmq) {
        // MMVQ quantizes (or copies) the activations into LDS in its prologue: no workspace.
        MmvqParams p{};
        p.W = static_cast<const uint8_t *>(W);
        p.row_bytes = rb;
        p.N = N;
        p.Np = N;
        p.npairs = (N + 1) / 2;
        p.K = K;
        p.xsrc = xdt;
        p.x = x;
        p.ldx = ldx;
        p.q8 = static_cast<const uint8_t *>(x);
        p.q8_row = (K / 32) * Q8_1_BYTES;
        p.x_bytes = xdt == GGQ_Q8_1 ? M * p.q8_row : ((M - 1) * ldx + K) * (xdt == GGQ_F32 ? 4 : 2);
        p.M = M;
        p.y = y;
        p.ldy = ldy;
        p.y_f16 = ydt == GGQ_F16;
        p.w_bytes = N * rb;
        const int nc = std::min(nc_for(M), mmvq_max_cols(wt, K));
        return hip_status(launch_mmvq(wt, nc, false, GGQ_EPI_NONE, kernel_dt(ydt), p, (M + nc - 1) / nc, s), "mul_mat mmvq");
    }
    // tiled operand, rows padded to a multiple of 64 (the padding rows are never written;
    // they only feed output columns that are not stored)
    Planar pl = carve_planar(c, mmq_rows(M), K);
    if (xdt == GGQ_Q8_1) rc = hip_status(launch_q8_1_to_planar(static_cast<const uint8_t *>(x), M, K, pl.xq, pl.xd, pl.xm, true, s), "mul_mat expand");
    else rc = hip_status(launch_quantize(x, xdt, M, K, ldx, nullptr, pl.xq, pl.xd, pl.xm, true, s), "mul_mat quantize");
    if (rc) return rc;
    MmqParams p{};
    p.W = static_cast<const uint8_t *>(W);
    p.row_bytes = rb;
    p.N = N;
    p.Np = N;
    p.K = K;
    p.xq = pl.xq;
    p.xd = pl.xd;
    p.xm = pl.xm;
    p.M = M;
    p.x_rows = mmq_rows(M);
    p.m_tiles = (M + MMQ_MT - 1) / MMQ_MT;
    p.n_tiles = (N + MMQ_NT - 1) / MMQ_NT;
    p.y = y;
    p.ldy = ldy;
    p.y_f16 = ydt == GGQ_F16;
    p.ksplit = mmq_ksplit(M, N, K);
    p.part = p.ksplit > 1 ? c.take<float>((size_t)p.ksplit * M * N * 4) : nullptr;
    rc = hip_status(launch_mmq(wt, false, GGQ_EPI_NONE, kernel_dt(ydt), p, s), "mul_mat mmq");
    if (!rc && p.ksplit > 1)
        rc = hip_status(launch_splitk_reduce(p.part, p.ksplit, M, N, y, kernel_dt(ydt), p.y_f16, ldy, s), "mul_mat split-K sum");
    return rc;
}

// ---------------------------------------------------------------------------
// routed experts
// ---------------------------------------------------------------------------
namespace {

struct IdLayout {
    RouteTables rt;
    int64_t max_tiles;
    Planar pl;
    void *oroute;         // weighted: per-route outputs [R][Np] (fp32 room; 16-bit when y is)
    void *hstage;         // MMVQ, unweighted: outputs [R][Np] (fp32 room) before a q8_1 output's quantization
    size_t total;
};

IdLayout id_layout(void *ws, int wt, int64_t E, int64_t N, int64_t K, int64_t T, int x_per_route, int64_t top_k,
                   int epi, bool weighted, bool mmq) {
    IdLayout L{};
    const int64_t R = T * top_k;
    const int J = mmq ? MMQ_MT : mmvq_id_cols(wt, R, E, K);
    L.max_tiles = route_max_tiles(R, E, J);
    const int64_t Np = epi == GGQ_EPI_SWIGLU ? N / 2 : N;
    const int64_t rows = x_per_route ? R : T;
    Carve c(ws);
    L.rt.bad = c.take<uint32_t>(4);                       // offset 0
    L.rt.counts = c.take<uint32_t>((size_t)E * 4);
    L.rt.offsets = c.take<uint32_t>((size_t)(E + 1) * 4);
    L.rt.tile_off = c.take<uint32_t>((size_t)(E + 1) * 4);
    L.rt.ntiles = c.take<uint32_t>(4);
    L.rt.rank = c.take<int32_t>((size_t)R * 4);
    L.rt.perm = c.take<int32_t>((size_t)R * 4);
    L.rt.tiles = c.take<int4>((size_t)L.max_tiles * 16);
    if (mmq) L.pl = carve_planar(c, rows, K);
    L.oroute = weighted ? c.take<float>((size_t)R * Np * 4) : nullptr;
    L.hstage = !mmq && !weighted ? c.take<float>((size_t)R * Np * 4) : nullptr;
    L.total = c.off;
    (void)wt;
    return L;
}

}  // namespace

size_t ggq_mul_mat_id_ws(int wt, int64_t E, int64_t N, int64_t K, int xdt, int64_t T, int x_per_route, int64_t top_k,
                         int epi, int weighted, int path) {
    (void)xdt;
    if (!known_type(wt) || E <= 0 || N <= 0 || K <= 0 || K % block_len(wt) || T < 0 || top_k <= 0) return 0;
    return id_layout(nullptr, wt, E, N, K, T, x_per_route, top_k, epi, weighted != 0, use_mmq_id(wt, K, T * top_k, E, path)).total;
}

int ggq_mul_mat_id(int wt, const void *W, int64_t E, int64_t N, int64_t K, int64_t expert_stride, const void *x, int xdt,
                   int64_t T, int x_per_route, const int32_t *ids, int64_t top_k, const float *route_w, int epi, void *y,
                   int ydt, void *ws, size_t ws_bytes, int path, void *stream) {
    g_err[0] = 0;
    int rc = check_weights(wt, N, K);
    if (rc) return rc;
    if (!float_dt(xdt) && xdt != GGQ_Q8_1) return fail(GGQ_ERR_UNSUPPORTED, "mul_mat_id: input dtype %d", xdt);
    if (!float_dt(ydt) && ydt != GGQ_Q8_1) return fail(GGQ_ERR_UNSUPPORTED, "mul_mat_id: output dtype %d", ydt);
    if (epi != GGQ_EPI_NONE && epi != GGQ_EPI_SWIGLU) return fail(GGQ_ERR_INVALID, "mul_mat_id: bad epilogue %d", epi);
    if (epi == GGQ_EPI_SWIGLU && N % 2) return fail(GGQ_ERR_INVALID, "mul_mat_id: SwiGLU needs an even N (gate rows then up rows), N=%lld", (long long)N);
    if (ydt == GGQ_Q8_1 && route_w) return fail(GGQ_ERR_UNSUPPORTED, "mul_mat_id: q8_1 output is per route (route_w must be NULL)");
    if (ydt == GGQ_Q8_1 && (epi == GGQ_EPI_SWIGLU ? N / 2 : N) % QK8_1)
        return fail(GGQ_ERR_INVALID, "mul_mat_id: q8_1 output needs output rows N'=%lld divisible by 32", (long long)(epi == GGQ_EPI_SWIGLU ? N / 2 : N));
    if (path != GGQ_PATH_AUTO && path != GGQ_PATH_MMVQ && path != GGQ_PATH_MMQ) return fail(GGQ_ERR_INVALID, "mul_mat_id: bad path %d", path);
    if (path == GGQ_PATH_MMQ && !has_mmq(wt, K))
        return fail(GGQ_ERR_UNSUPPORTED, "mul_mat_id: MMQ path has no %s kernel for K=%lld (Q8_0 / Q4_0 need K %% 256 == 0); use MMVQ", tname(wt), (long long)K);
    if (E <= 0 || T < 0 || top_k <= 0) return fail(GGQ_ERR_INVALID, "mul_mat_id: bad E=%lld T=%lld top_k=%lld", (long long)E, (long long)T, (long long)top_k);
    if (x_per_route != 0 && x_per_route != 1) return fail(GGQ_ERR_INVALID, "mul_mat_id: x_per_route must be 0 or 1");
    const int64_t rb = (int64_t)ggq_row_bytes(wt, K);
    if (expert_stride < rb * N || expert_stride % 16) return fail(GGQ_ERR_INVALID, "mul_mat_id: expert_stride=%lld must be >= N*row_bytes=%lld and a multiple of 16", (long long)expert_stride, (long long)(rb * N));
    if (T * top_k > INT32_MAX || E > INT32_MAX) return fail(GGQ_ERR_INVALID, "mul_mat_id: too many routes");
    if (T == 0 || N == 0) return GGQ_OK;
    if (!W || !x || !ids || !y) return fail(GGQ_ERR_INVALID, "mul_mat_id: null pointer");
    if (!aligned16(W) || !aligned16(x) || !aligned16(y) || !aligned16(ids)) return fail(GGQ_ERR_INVALID, "mul_mat_id: pointers must be 16-byte aligned");
    const bool mmq = use_mmq_id(wt, K, T * top_k, E, path);
    if (!mmq && !mmvq_supported(wt, K)) return mmvq_too_long("mul_mat_id", wt, K);
    // routed MMQ gathers activation rows and SwiGLU up rows with 32-bit offsets
    if (mmq && (x_per_route ? T * top_k : T) * K * 2 >= (int64_t)0x7fffff00)
        return fail(GGQ_ERR_UNSUPPORTED, "mul_mat_id: MMQ path takes at most 2 GiB of fp16 activation rows (%lld rows of K=%lld); split the tokens",
                    (long long)(x_per_route ? T * top_k : T), (long long)K);
    if (mmq && epi == GGQ_EPI_SWIGLU && N * rb >= (int64_t)0x7fffff00)
        return fail(GGQ_ERR_UNSUPPORTED, "mul_mat_id: SwiGLU on the MMQ path needs an expert matrix below 2 GiB");
    const bool weighted = route_w != nullptr;
    IdLayout L = id_layout(ws, wt, E, N, K, T, x_per_route, top_k, epi, weighted, mmq);
    if (!ws || ws_bytes < L.total) return fail(GGQ_ERR_WORKSPACE, "mul_mat_id: workspace %zu bytes < %zu required", ws_bytes, L.total);
    if (!aligned16(ws)) return fail(GGQ_ERR_INVALID, "mul_mat_id: workspace must be 16-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t R = T * top_k;
    const int64_t Np = epi == GGQ_EPI_SWIGLU ? N / 2 : N;
    const int64_t rows = x_per_route ? R : T;
    const int J = mmq ? MMQ_MT : mmvq_id_cols(wt, R, E, K);
    // q8_1 output: MMQ quantizes in its epilogue; MMVQ writes the values (in the
    // 16-bit input's dtype, else fp32) to the workspace and the q8_1 kernel follows
    const bool q8_out = ydt == GGQ_Q8_1;
    const int hdt = xdt == GGQ_BF16 || xdt == GGQ_F16 ? xdt : GGQ_F32;
    void *yk = q8_out && !mmq ? L.hstage : y;               // what the matmul kernel writes
    const int ydt_k = q8_out && !mmq ? hdt : ydt;
    // One route per MMVQ group: the kernel takes group g as route g straight from
    // ids, zeroes an inactive route's unweighted row and counts the ids >= E; no
    // route tables (one launch fewer).  Otherwise the route build groups routes by
    // expert, and the rows of inactive routes of an unweighted output are zeros (by
    // the one-workgroup route build when it runs, else by their own kernel).
    const bool direct = !mmq && J == 1 && R > 0 && Np > 0;
    if (!direct) {
        bool zeroed = false;
        rc = hip_status(launch_route_build(ids, R, E, J, L.rt, s, weighted ? nullptr : yk, Np, ydt_k, &zeroed),
                        "mul_mat_id routes");
        if (rc) return rc;
        if (!weighted && !zeroed) {
            rc = hip_status(launch_zero_inactive(ids, R, E, Np, yk, ydt_k, s), "mul_mat_id zero");
            if (rc) return rc;
        }
    }

    if (!mmq) {
        MmvqParams p{};
        p.W = static_cast<const uint8_t *>(W);
        p.row_bytes = rb;
        p.expert_stride = expert_stride;
        p.N = N;
        p.Np = Np;
        p.npairs = epi == GGQ_EPI_SWIGLU ? Np : (N + 1) / 2;
        p.K = K;
        p.xsrc = xdt;
        p.x = x;
        p.ldx = K;
        p.q8 = static_cast<const uint8_t *>(x);
        p.q8_row = (K / 32) * Q8_1_BYTES;
        p.x_bytes = xdt == GGQ_Q8_1 ? rows * p.q8_row : rows * K * (xdt == GGQ_F32 ? 4 : 2);
        p.y = yk;
        p.y_f16 = ydt_k == GGQ_F16;
        p.perm = L.rt.perm;
        p.groups = L.rt.tiles;
        p.ngroups = L.rt.ntiles;
        p.top_k = (int)top_k;
        p.x_per_route = x_per_route;
        p.route_w = route_w;
        p.oroute = L.oroute;
        p.groups_expected = std::min<int64_t>(E, R);
        p.w_bytes = (E - 1) * expert_stride + N * rb;
        if (direct) {
            p.ids = ids;
            p.R = R;
            p.E = E;
            p.bad = L.rt.bad;
        }
        rc = hip_status(launch_mmvq(wt, J, true, epi, kernel_dt(ydt_k), p, direct ? R : L.max_tiles, s), "mul_mat_id mmvq");
        if (!rc && q8_out)
            rc = hip_status(launch_quantize(L.hstage, hdt, R, Np, Np, static_cast<uint8_t *>(y), nullptr, nullptr, nullptr, false, s),
                            "mul_mat_id q8_1 output");
    } else {
        if (xdt == GGQ_Q8_1)
            rc = hip_status(launch_q8_1_to_planar(static_cast<const uint8_t *>(x), rows, K, L.pl.xq, L.pl.xd, L.pl.xm, false, s),
                            "mul_mat_id expand");
        else
            rc = hip_status(launch_quantize(x, xdt, rows, K, K, nullptr, L.pl.xq, L.pl.xd, L.pl.xm, false, s), "mul_mat_id quantize");
        if (rc) return rc;
        MmqParams p{};
        p.W = static_cast<const uint8_t *>(W);
        p.row_bytes = rb;
        p.expert_stride = expert_stride;
        p.N = N;
        p.Np = Np;
        p.K = K;
        p.xq = L.pl.xq;
        p.xd = L.pl.xd;
        p.xm = L.pl.xm;
        p.x_rows = rows;
        p.m_tiles = L.max_tiles;
        p.n_tiles = epi == GGQ_EPI_SWIGLU ? (Np + 63) / 64 : (N + MMQ_NT - 1) / MMQ_NT;
        p.y = y;
        p.perm = L.rt.perm;
        p.tiles = L.rt.tiles;
        p.ntiles = L.rt.ntiles;
        p.top_k = (int)top_k;
        p.x_per_route = x_per_route;
        p.route_w = route_w;
        p.oroute = L.oroute;
        p.q8_round = !q8_out ? 0 : hdt == GGQ_BF16 ? 1 : hdt == GGQ_F16 ? 2 : 0;
        p.y_f16 = ydt == GGQ_F16;
        rc = hip_status(launch_mmq(wt, true, epi, kernel_dt(ydt), p, s), "mul_mat_id mmq");
    }
    if (rc) return rc;
    if (weighted) rc = hip_status(launch_route_sum(L.oroute, ids, route_w, T, (int)top_k, E, Np, y, ydt, s), "mul_mat_id route sum");
    return rc;
}

size_t ggq_test_block_dots_ws(int wt, int64_t K, int64_t M, int path) {
    if (path != GGQ_PATH_MMQ || !known_type(wt) || M <= 0 || K <= 0) return 0;
    return act_bytes(true, M, K);
}

int ggq_test_block_dots(int wt, const void *W, int64_t N, int64_t K, const void *q8, int64_t M, int32_t *out,
                        void *ws, size_t ws_bytes, int path, void *stream) {
    g_err[0] = 0;
    int rc = check_weights(wt, N, K);
    if (rc) return rc;
    if (path != GGQ_PATH_MMVQ && path != GGQ_PATH_MMQ) return fail(GGQ_ERR_INVALID, "test_block_dots: path must be MMVQ or MMQ");
    if (path == GGQ_PATH_MMQ && !has_mmq(wt, K))
        return fail(GGQ_ERR_UNSUPPORTED, "test_block_dots: MMQ path has no %s kernel for K=%lld", tname(wt), (long long)K);
    if (M < 0) return fail(GGQ_ERR_INVALID, "test_block_dots: M < 0");
    if (M == 0 || N == 0) return GGQ_OK;
    if (!W || !q8 || !out) return fail(GGQ_ERR_INVALID, "test_block_dots: null pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (path == GGQ_PATH_MMVQ)
        return hip_status(launch_mmvq_dots(wt, static_cast<const uint8_t *>(W), N, K, static_cast<const uint8_t *>(q8), M, out, s),
                          "test_block_dots mmvq");
    const size_t need = ggq_test_block_dots_ws(wt, K, M, path);
    if (!ws || ws_bytes < need) return fail(GGQ_ERR_WORKSPACE, "test_block_dots: workspace %zu bytes < %zu required", ws_bytes, need);
    Carve c(ws);
    Planar pl = carve_planar(c, M, K);
    rc = hip_status(launch_q8_1_to_planar(static_cast<const uint8_t *>(q8), M, K, pl.xq, pl.xd, pl.xm, false, s), "test_block_dots expand");
    if (rc) return rc;
    return hip_status(launch_mmq_dots(wt, static_cast<const uint8_t *>(W), N, K, pl.xq, M, out, s), "test_block_dots mmq");
}

int ggq_bench_stream_read(const void *buf, int64_t bytes, void *sink, size_t sink_bytes, void *stream) {
    g_err[0] = 0;
    if (bytes < 0) return fail(GGQ_ERR_INVALID, "bench_stream_read: bytes < 0");
    if (bytes == 0) return GGQ_OK;
    if (!buf || !sink) return fail(GGQ_ERR_INVALID, "bench_stream_read: null pointer");
    if (!aligned16(buf)) return fail(GGQ_ERR_INVALID, "bench_stream_read: buffer not 16-byte aligned");
    if (sink_bytes < (size_t)CEIL_READ_BLOCKS * 4)
        return fail(GGQ_ERR_WORKSPACE, "bench_stream_read: sink %zu bytes < %d required", sink_bytes, CEIL_READ_BLOCKS * 4);
    return hip_status(launch_stream_read(buf, bytes, static_cast<int *>(sink), static_cast<hipStream_t>(stream)),
                      "bench_stream_read");
}

int ggq_bench_mfma_loop(int kind, int64_t iters, void *sink, size_t sink_bytes, void *stream) {
    g_err[0] = 0;
    if (kind != 0 && kind != 1) return fail(GGQ_ERR_INVALID, "bench_mfma_loop: kind must be 0 (fp16) or 1 (int8)");
    if (iters < 0) return fail(GGQ_ERR_INVALID, "bench_mfma_loop: iters < 0");
    if (!sink) return fail(GGQ_ERR_INVALID, "bench_mfma_loop: null sink");
    if (sink_bytes < (size_t)CEIL_MFMA_BLOCKS * 4)
        return fail(GGQ_ERR_WORKSPACE, "bench_mfma_loop: sink %zu bytes < %d required", sink_bytes, CEIL_MFMA_BLOCKS * 4);
    return hip_status(launch_mfma_loop(kind, iters, static_cast<int *>(sink), static_cast<hipStream_t>(stream)),
                      "bench_mfma_loop");
}

int ggq_bench_set_mmvq_id_cols(int cols) {
    g_err[0] = 0;
    if (cols != 0 && cols != 1 && cols != 2 && cols != 4 && cols != 8)
        return fail(GGQ_ERR_INVALID, "bench_set_mmvq_id_cols: cols must be 0 (automatic), 1, 2, 4 or 8");
    g_id_cols_override = cols;
    return GGQ_OK;
}

int ggq_bench_inner_loop(int kind, int blocks_per_cu, int64_t iters, void *sink, size_t sink_bytes, void *stream) {
    g_err[0] = 0;
    if (kind < 0 || kind > 4) return fail(GGQ_ERR_INVALID, "bench_inner_loop: kind must be 0..4");
    if (blocks_per_cu < 1 || blocks_per_cu > 8) return fail(GGQ_ERR_INVALID, "bench_inner_loop: blocks_per_cu must be 1..8");
    if (iters < 0) return fail(GGQ_ERR_INVALID, "bench_inner_loop: iters < 0");
    if (!sink) return fail(GGQ_ERR_INVALID, "bench_inner_loop: null sink");
    if (sink_bytes < (size_t)256 * blocks_per_cu * 4)
        return fail(GGQ_ERR_WORKSPACE, "bench_inner_loop: sink %zu bytes < %d required", sink_bytes, 256 * blocks_per_cu * 4);
    return hip_status(launch_inner_loop(kind, blocks_per_cu, iters, static_cast<int *>(sink), static_cast<hipStream_t>(stream)),
                      "bench_inner_loop");
}

// ---------------------------------------------------------------------------
// routed experts without an allocation: the workspace is a fixed device array
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// One copy per GPU, for the life of the process.  Host code never names it in a launch
// or copy: its address on a device comes from hipGetSymbolAddress, taken once per device
// with that device current.
static __device__ __align__(256) uint8_t scratch[GGQ_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

int scratch_of_current_device(void **out) {
    int dev = -1;
    int rc = hip_status(hipGetDevice(&dev), "mul_mat_id_noalloc: current device");
    if (rc) return rc;
    if (dev < 0 || dev >= MAX_DEVICES) return fail(GGQ_ERR_INVALID, "mul_mat_id_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        rc = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "mul_mat_id_noalloc: scratch address");
        if (rc) return rc;
        if (!ptr) return fail(GGQ_ERR_HIP, "mul_mat_id_noalloc: no scratch address on device %d", dev);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GGQ_OK;
}

}  // namespace

extern "C" {

int ggq_mul_mat_id_noalloc(int wt, const void *W, int64_t E, int64_t N, int64_t K, int64_t expert_stride,
                           const void *x, int xdt, int64_t T, int x_per_route, const int32_t *ids, int64_t top_k,
                           const float *route_w, int epi, void *y, int ydt, int path, void *stream) {
    g_err[0] = 0;
    const size_t need = ggq_mul_mat_id_ws(wt, E, N, K, xdt, T, x_per_route, top_k, epi, route_w != nullptr, path);
    if (need > GGQ_NOALLOC_SCRATCH_BYTES)
        return fail(GGQ_ERR_WORKSPACE,
                    "mul_mat_id_noalloc: this call needs %zu bytes of workspace, the fixed scratch holds %zu; "
                    "call ggq_mul_mat_id with a workspace of ggq_mul_mat_id_ws() bytes",
                    need, (size_t)GGQ_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    const int rc = scratch_of_current_device(&ws);
    if (rc) return rc;
    return ggq_mul_mat_id(wt, W, E, N, K, expert_stride, x, xdt, T, x_per_route, ids, top_k, route_w, epi, y, ydt, ws,
                          GGQ_NOALLOC_SCRATCH_BYTES, path, stream);
}

}  // extern "C"
