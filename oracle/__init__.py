"""CPU oracle for GGUF block-quantized matmul -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``libggq_oracle.so`` (plain C, see ggq_oracle.h).
Only the tests, the smoke check of ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package; the product path (the HIP
library and its binding) never does.

All arrays are numpy arrays on the host.  Weights are raw GGUF bytes
(uint8), activations float32 or bfloat16 bit patterns (uint16), q8_1
activations uint8 blocks of 40 bytes.
"""
import ctypes
import os

import numpy as np

from . import build as _build

Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 2, 8, 12, 13, 14
F32, BF16, Q8_1, F16 = 0, 1, 2, 3
EPI_NONE, EPI_SWIGLU = 0, 1
Q8_1_BYTES = 40

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("GGQO_LIB")                   # another build (the sanitized one)
        if not path:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.ggqo_fp16_to_fp32.restype = ctypes.c_float
        L.ggqo_fp16_to_fp32.argtypes = [ctypes.c_uint16]
        L.ggqo_bf16_to_fp32.restype = ctypes.c_float
        L.ggqo_bf16_to_fp32.argtypes = [ctypes.c_uint16]
        L.ggqo_fp32_to_bf16.restype = ctypes.c_uint16
        L.ggqo_fp32_to_bf16.argtypes = [ctypes.c_float]
        L.ggqo_fp32_to_fp16.restype = ctypes.c_uint16
        L.ggqo_fp32_to_fp16.argtypes = [ctypes.c_float]
        for f in ("ggqo_block_len", "ggqo_block_bytes", "ggqo_group_len"):
            getattr(L, f).restype = i64
            getattr(L, f).argtypes = [i32]
        L.ggqo_row_bytes.restype = i64
        L.ggqo_row_bytes.argtypes = [i32, i64]
        L.ggqo_quantize_block_q8_1.restype = None
        L.ggqo_quantize_block_q8_1.argtypes = [vp, vp]
        L.ggqo_quantize_q8_1.restype = i32
        L.ggqo_quantize_q8_1.argtypes = [vp, i32, i64, i64, i64, vp]
        L.ggqo_unpack_block.restype = i32
        L.ggqo_unpack_block.argtypes = [i32, vp, vp, vp, vp, vp]
        L.ggqo_block_dots.restype = i32
        L.ggqo_block_dots.argtypes = [i32, vp, i64, i64, vp, i64, vp]
        L.ggqo_mul_mat_q8.restype = i32
        L.ggqo_mul_mat_q8.argtypes = [i32, vp, i64, i64, vp, i64, vp, i64, vp, i64]
        L.ggqo_mul_mat.restype = i32
        L.ggqo_mul_mat.argtypes = [i32, vp, i64, i64, vp, i32, i64, i64, vp, i64, vp, i64]
        L.ggqo_dequantize.restype = i32
        L.ggqo_dequantize.argtypes = [i32, vp, i64, i64, vp, i32]
        L.ggqo_mul_mat_id.restype = i32
        L.ggqo_mul_mat_id.argtypes = [i32, vp, i64, i64, i64, i64, vp, i32, i64, i32,
                                      vp, i64, vp, i32, i32, vp, i64, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments")


def _dt(x):
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float16:
        return F16
    raise TypeError("activations must be float32, bf16 bits (uint16) or float16")


def block_len(t):
    return lib().ggqo_block_len(t)


def block_bytes(t):
    return lib().ggqo_block_bytes(t)


def group_len(t):
    return lib().ggqo_group_len(t)


def row_bytes(t, K):
    return lib().ggqo_row_bytes(t, K)


def fp16_to_fp32(h):
    return lib().ggqo_fp16_to_fp32(int(h))


def bf16_to_fp32(b):
    return lib().ggqo_bf16_to_fp32(int(b))


def fp32_to_bf16(f):
    return lib().ggqo_fp32_to_bf16(float(f))


def fp32_to_fp16(f):
    """IEEE binary16 bits (uint16) of float32 f, round to nearest even."""
    return lib().ggqo_fp32_to_fp16(float(f))


def fp32_to_fp16_array(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    f = lib().ggqo_fp32_to_fp16
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def fp32_to_bf16_array(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    f = lib().ggqo_fp32_to_bf16
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def quantize_block_q8_1(x32):
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    assert x32.shape == (32,)
    out = np.zeros(Q8_1_BYTES, dtype=np.uint8)
    lib().ggqo_quantize_block_q8_1(_p(x32), _p(out))
    return out


def quantize_q8_1(x, K=None):
    """x: [M][ldx] float32 or bf16 bits; returns uint8 [M][K/32*40]."""
    x = np.ascontiguousarray(x)
    M, ldx = x.shape
    K = ldx if K is None else K
    out = np.zeros((M, (K // 32) * Q8_1_BYTES), dtype=np.uint8)
    _check(lib().ggqo_quantize_q8_1(_p(x), _dt(x), M, K, ldx, _p(out)), "quantize_q8_1")
    return out


def unpack_block(t, blk):
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    q = np.zeros(256, dtype=np.int32)
    sc = np.zeros(16, dtype=np.int32)
    mn = np.zeros(16, dtype=np.int32)
    d = np.zeros(2, dtype=np.float32)
    _check(lib().ggqo_unpack_block(t, _p(blk), _p(q), _p(sc), _p(mn), _p(d)), "unpack_block")
    qk, g = block_len(t), group_len(t)
    return q[:qk], sc[:qk // g], mn[:qk // g], d


def block_dots(t, W, N, K, q8, M):
    W = np.ascontiguousarray(W, dtype=np.uint8)
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    g = group_len(t)
    out = np.zeros((M, N, K // g), dtype=np.int32)
    _check(lib().ggqo_block_dots(t, _p(W), N, K, _p(q8), M, _p(out)), "block_dots")
    return out


def mul_mat_q8(t, W, N, K, q8, M, rows=None):
    W = np.ascontiguousarray(W, dtype=np.uint8)
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nc = N if r is None else len(r)
    y = np.zeros((M, nc), dtype=np.float32)
    _check(lib().ggqo_mul_mat_q8(t, _p(W), N, K, _p(q8), M, _p(r), 0 if r is None else len(r),
                                 _p(y), nc), "mul_mat_q8")
    return y


def mul_mat(t, W, N, K, x, rows=None, xdt=None):
    """Full path: x float32 [M][K] / bf16 bits [M][K] / q8_1 blocks (xdt=Q8_1)."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    x = np.ascontiguousarray(x)
    if xdt is None:
        xdt = _dt(x)
    M = x.shape[0]
    ldx = x.shape[1] if xdt != Q8_1 else K
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nc = N if r is None else len(r)
    y = np.zeros((M, nc), dtype=np.float32)
    _check(lib().ggqo_mul_mat(t, _p(W), N, K, _p(x), xdt, M, ldx, _p(r),
                              0 if r is None else len(r), _p(y), nc), "mul_mat")
    return y


def dequantize(t, W, rows, K, ydt=F32):
    W = np.ascontiguousarray(W, dtype=np.uint8)
    y = np.zeros((rows, K), dtype=np.float32 if ydt == F32 else np.uint16)   # 16-bit: bf16 / fp16 bits
    _check(lib().ggqo_dequantize(t, _p(W), rows, K, _p(y), ydt), "dequantize")
    return y


def mul_mat_id(t, W, E, N, K, expert_stride, x, T, x_per_route, ids, top_k,
               route_w=None, epi=EPI_NONE, tokens=None, route_round=None):
    """route_round (weighted only): None keeps each route's output in fp32 before the
    weighted sum; "bf16" / "f16" rounds it to that 16-bit type first (the intermediate
    held in a 16-bit activation dtype)."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = None if route_w is None else np.ascontiguousarray(route_w, dtype=np.float32)
    tk = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    nt = T if tk is None else len(tk)
    Np = N // 2 if epi == EPI_SWIGLU else N
    shape = (nt, Np) if w is not None else (nt, top_k, Np)
    y = np.zeros(shape, dtype=np.float32)
    _check(lib().ggqo_mul_mat_id(t, _p(W), E, N, K, expert_stride, _p(x), _dt(x), T, int(x_per_route),
                                 _p(ids), top_k, _p(w), epi, {None: 0, "bf16": 1, "f16": 2}[route_round],
                                 _p(tk), nt, _p(y)), "mul_mat_id")
    return y
