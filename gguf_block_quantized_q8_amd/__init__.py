"""GGUF block-quantized matmul (Q4_0 / Q8_0 / Q4_K / Q5_K / Q6_K x q8_1) on MI355X.

Thin Python binding over the C ABI in include/ggq.h (libggq.so, hand-written
HIP for gfx950).  This module only marshals arguments: it takes torch tensors
on the GPU, allocates the output and the workspace with torch, and passes
pointers, sizes and the current stream.  Every step of the computation runs
in the library's kernels; there is no CPU or PyTorch fallback -- if the
library is missing, the calls raise.
"""
import ctypes
import os

import torch

Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 2, 8, 12, 13, 14
F32, BF16, Q8_1, F16 = 0, 1, 2, 3
PATH_AUTO, PATH_MMVQ, PATH_MMQ = 0, 1, 2
EPI_NONE, EPI_SWIGLU = 0, 1
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
Q8_1_BYTES = 40

_HERE = os.path.dirname(os.path.abspath(__file__))
# GGQ_LIB: another build of the same library (the tests load a host-sanitized build this way)
LIB_PATH = os.environ.get("GGQ_LIB") or os.path.join(_HERE, "libggq.so")
_PATHS = {"auto": PATH_AUTO, "mmvq": PATH_MMVQ, "mmq": PATH_MMQ}
_lib = None

EXPORTS = ["ggq_row_bytes", "ggq_q8_1_bytes", "ggq_quantize_q8_1", "ggq_mul_mat_ws", "ggq_mul_mat",
           "ggq_mul_mat_id_ws", "ggq_mul_mat_id", "ggq_mul_mat_id_noalloc", "ggq_dequantize", "ggq_get_rows", "ggq_last_error",
           "ggq_test_block_dots_ws", "ggq_test_block_dots", "ggq_bench_stream_read", "ggq_bench_mfma_loop",
           "ggq_bench_inner_loop", "ggq_bench_set_mmvq_id_cols"]


def lib():
    """Load libggq.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.ggq_row_bytes.restype = sz
    L.ggq_row_bytes.argtypes = [i32, i64]
    L.ggq_q8_1_bytes.restype = sz
    L.ggq_q8_1_bytes.argtypes = [i64, i64]
    L.ggq_quantize_q8_1.restype = i32
    L.ggq_quantize_q8_1.argtypes = [vp, i32, i64, i64, i64, vp, vp]
    L.ggq_mul_mat_ws.restype = sz
    L.ggq_mul_mat_ws.argtypes = [i32, i64, i64, i32, i64, i32]
    L.ggq_mul_mat.restype = i32
    L.ggq_mul_mat.argtypes = [i32, vp, i64, i64, vp, i32, i64, i64, vp, i32, i64, vp, sz, i32, vp]
    L.ggq_mul_mat_id_ws.restype = sz
    L.ggq_mul_mat_id_ws.argtypes = [i32, i64, i64, i64, i32, i64, i32, i64, i32, i32, i32]
    L.ggq_mul_mat_id.restype = i32
    L.ggq_mul_mat_id.argtypes = [i32, vp, i64, i64, i64, i64, vp, i32, i64, i32, vp, i64, vp, i32,
                                 vp, i32, vp, sz, i32, vp]
    L.ggq_mul_mat_id_noalloc.restype = i32
    L.ggq_mul_mat_id_noalloc.argtypes = [i32, vp, i64, i64, i64, i64, vp, i32, i64, i32, vp, i64, vp, i32,
                                         vp, i32, i32, vp]
    L.ggq_dequantize.restype = i32
    L.ggq_dequantize.argtypes = [i32, vp, i64, i64, vp, i32, vp]
    L.ggq_get_rows.restype = i32
    L.ggq_get_rows.argtypes = [i32, vp, i64, i64, vp, i64, vp, i32, i64, vp]
    L.ggq_last_error.restype = ctypes.c_char_p
    L.ggq_last_error.argtypes = []
    L.ggq_test_block_dots_ws.restype = sz
    L.ggq_test_block_dots_ws.argtypes = [i32, i64, i64, i32]
    L.ggq_test_block_dots.restype = i32
    L.ggq_test_block_dots.argtypes = [i32, vp, i64, i64, vp, i64, vp, vp, sz, i32, vp]
    L.ggq_bench_stream_read.restype = i32
    L.ggq_bench_stream_read.argtypes = [vp, i64, vp, sz, vp]
    L.ggq_bench_mfma_loop.restype = i32
    L.ggq_bench_mfma_loop.argtypes = [i32, i64, vp, sz, vp]
    L.ggq_bench_inner_loop.restype = i32
    L.ggq_bench_inner_loop.argtypes = [i32, i32, i64, vp, sz, vp]
    L.ggq_bench_set_mmvq_id_cols.restype = i32
    L.ggq_bench_set_mmvq_id_cols.argtypes = [i32]
    _lib = L
    return L


class GgqError(RuntimeError):
    pass


def _raise(rc, what):
    if rc == OK:
        return
    msg = f"{what}: {lib().ggq_last_error().decode()}"
    if rc == ERR_INVALID:
        raise ValueError(msg)
    if rc == ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise GgqError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _xdt(x):
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    if x.dtype == torch.float16:
        return F16
    if x.dtype == torch.uint8:
        return Q8_1
    raise TypeError(f"activations must be float32, bfloat16, float16 or uint8 q8_1 blocks, got {x.dtype}")


def _ydt(dtype):
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float16:
        return F16
    raise TypeError(f"output dtype must be float32, bfloat16 or float16, got {dtype}")


def _check_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def row_bytes(wt, K):
    return lib().ggq_row_bytes(wt, K)


def quantize_q8_1(x, out=None):
    """x [M, K] float32/bfloat16 (row stride may exceed K) -> uint8 [M, K/32*40] q8_1 blocks."""
    _check_gpu(x)
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along K")
    if out is None:
        out = torch.empty((M, (K // 32) * Q8_1_BYTES), dtype=torch.uint8, device=x.device)
    rc = lib().ggq_quantize_q8_1(_ptr(x), _xdt(x), M, K, x.stride(0), _ptr(out), _stream(x.device))
    _raise(rc, "quantize_q8_1")
    return out


def mul_mat(W, wt, x, K=None, out_dtype=None, path="auto", out=None):
    """y[m, n] = sum_k W[n, k] x[m, k].

    W: uint8 [N, row_bytes] GGUF blocks of type wt.  x: [M, K] float32/bfloat16,
    or uint8 [M, K/32*40] q8_1 blocks (then K must be given).  Output dtype
    defaults to the activation dtype (float32 for q8_1 input)."""
    _check_gpu(W, x)
    N = W.shape[0]
    xdt = _xdt(x)
    M = x.shape[0]
    if xdt == Q8_1:
        if K is None:
            raise ValueError("K is required with q8_1 input")
        ldx = K
    else:
        K = x.shape[1]
        ldx = x.stride(0)
        if x.stride(1) != 1:
            raise ValueError("x must have unit stride along K")
    if out_dtype is None:
        out_dtype = x.dtype if xdt != Q8_1 else torch.float32
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    p = _PATHS[path]
    L = lib()
    wsb = L.ggq_mul_mat_ws(wt, N, K, xdt, M, p)
    ws = _workspace(wsb, x.device)
    rc = L.ggq_mul_mat(wt, _ptr(W), N, K, _ptr(x), xdt, M, ldx, _ptr(out), _ydt(out.dtype), out.stride(0),
                       _ptr(ws), wsb, p, _stream(x.device))
    _raise(rc, "mul_mat")
    return out


def mul_mat_id(W, wt, x, ids, K, route_w=None, epi=EPI_NONE, x_per_route=False, out_dtype=None,
               path="auto", return_workspace=False):
    """Routed experts.  W: uint8 [E, N, row_bytes] (or [E, stride] with stride >= N*row_bytes);
    x: [T, K] (broadcast) or [T, top_k, K] (x_per_route), float32 / bfloat16, or uint8 rows of
    K/32 q8_1 blocks; ids: int32 [T, top_k].
    Returns y [T, top_k, N'] (route_w None) or [T, N'] (route_w [T, top_k] float32).
    out_dtype "q8_1" (route_w None): y is uint8 [T, top_k, N'/32*40], each route's outputs as
    q8_1 blocks (rounded to bf16 first for bfloat16 x)."""
    _check_gpu(W, x, ids, route_w)
    E = W.shape[0]
    rb = row_bytes(wt, K)
    stride = W.stride(0)
    N = W.shape[1] if W.dim() == 3 else stride // rb
    T, top_k = ids.shape
    Np = N // 2 if epi == EPI_SWIGLU else N
    if out_dtype is None:
        out_dtype = x.dtype if _xdt(x) != Q8_1 else torch.float32
    if out_dtype == "q8_1":
        y = torch.empty((T, top_k, Np // 32 * Q8_1_BYTES), dtype=torch.uint8, device=x.device)
        ydt = Q8_1
    else:
        shape = (T, Np) if route_w is not None else (T, top_k, Np)
        y = torch.empty(shape, dtype=out_dtype, device=x.device)
        ydt = _ydt(out_dtype)
    p = _PATHS[path]
    L = lib()
    wsb = L.ggq_mul_mat_id_ws(wt, E, N, K, _xdt(x), T, int(x_per_route), top_k, epi, int(route_w is not None), p)
    ws = _workspace(max(wsb, 256), x.device)
    rc = L.ggq_mul_mat_id(wt, _ptr(W), E, N, K, stride, _ptr(x), _xdt(x), T, int(x_per_route),
                          _ptr(ids), top_k, _ptr(route_w), epi, _ptr(y), ydt,
                          _ptr(ws), ws.numel(), p, _stream(x.device))
    _raise(rc, "mul_mat_id")
    return (y, ws) if return_workspace else y


def mul_mat_id_noalloc(W, wt, x, ids, K, route_w=None, epi=EPI_NONE, x_per_route=False, out_dtype=None,
                       path="auto"):
    """mul_mat_id through ggq_mul_mat_id_noalloc: the library's fixed per-GPU scratch
    (NOALLOC_SCRATCH_BYTES) replaces the workspace; the output is allocated here."""
    _check_gpu(W, x, ids, route_w)
    E = W.shape[0]
    rb = row_bytes(wt, K)
    stride = W.stride(0)
    N = W.shape[1] if W.dim() == 3 else stride // rb
    T, top_k = ids.shape
    Np = N // 2 if epi == EPI_SWIGLU else N
    if out_dtype is None:
        out_dtype = x.dtype if _xdt(x) != Q8_1 else torch.float32
    if out_dtype == "q8_1":
        y = torch.empty((T, top_k, Np // 32 * Q8_1_BYTES), dtype=torch.uint8, device=x.device)
        ydt = Q8_1
    else:
        shape = (T, Np) if route_w is not None else (T, top_k, Np)
        y = torch.empty(shape, dtype=out_dtype, device=x.device)
        ydt = _ydt(out_dtype)
    rc = lib().ggq_mul_mat_id_noalloc(wt, _ptr(W), E, N, K, stride, _ptr(x), _xdt(x), T, int(x_per_route),
                                      _ptr(ids), top_k, _ptr(route_w), epi, _ptr(y), ydt, _PATHS[path],
                                      _stream(x.device))
    _raise(rc, "mul_mat_id_noalloc")
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20


def dequantize(W, wt, K, out_dtype=torch.float32):
    _check_gpu(W)
    rows = W.shape[0] if W.dim() == 2 else W.numel() // row_bytes(wt, K)
    y = torch.empty((rows, K), dtype=out_dtype, device=W.device)
    rc = lib().ggq_dequantize(wt, _ptr(W), rows, K, _ptr(y), _ydt(out_dtype), _stream(W.device))
    _raise(rc, "dequantize")
    return y


def get_rows(W, wt, K, ids, out_dtype=torch.float32):
    """Rows ids of the quantized table W, dequantized: [len(ids), K] (ids outside the table give zeros)."""
    _check_gpu(W, ids)
    if ids.dtype != torch.int32:
        raise ValueError("get_rows: ids must be int32")
    rows = W.shape[0] if W.dim() == 2 else W.numel() // row_bytes(wt, K)
    n = ids.numel()
    y = torch.empty((n, K), dtype=out_dtype, device=W.device)
    rc = lib().ggq_get_rows(wt, _ptr(W), rows, K, _ptr(ids), n, _ptr(y), _ydt(out_dtype), K, _stream(W.device))
    _raise(rc, "get_rows")
    return y


def test_block_dots(W, wt, q8, K, path="mmvq"):
    """Per-group int32 dots [M, N, K/g] from the named path's device code (test hook)."""
    _check_gpu(W, q8)
    N, M = W.shape[0], q8.shape[0]
    g = 16 if wt == Q6_K else 32
    out = torch.empty((M, N, K // g), dtype=torch.int32, device=W.device)
    p = _PATHS[path]
    L = lib()
    wsb = L.ggq_test_block_dots_ws(wt, K, M, p)
    ws = _workspace(wsb, W.device)
    rc = L.ggq_test_block_dots(wt, _ptr(W), N, K, _ptr(q8), M, _ptr(out), _ptr(ws), wsb, p, _stream(W.device))
    _raise(rc, "test_block_dots")
    return out
