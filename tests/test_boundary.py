"""CPU-only checks of the C-ABI library: it loads, exports every symbol the
header declares, and its host-side validation returns the documented error
codes without touching a GPU (every call here fails a check before any launch)."""
import ctypes
import os
import re

import pytest

import gguf_block_quantized_q8_amd as g
from gguf_block_quantized_q8_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ggq.h")
FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: every call below fails a check first


@pytest.fixture(scope="module")
def L():
    newest_src = max(os.path.getmtime(s) for s in _build.sources())
    if not os.path.exists(g.LIB_PATH) or os.path.getmtime(g.LIB_PATH) < newest_src:
        _build.build()
    return g.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ggq_\w+)\s*\(", text)))


def test_exports_every_header_symbol(L):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(g.EXPORTS)


def test_geometry(L):
    assert L.ggq_row_bytes(g.Q8_0, 512) == 16 * 34
    assert L.ggq_row_bytes(g.Q4_K, 2048) == 8 * 144
    assert L.ggq_row_bytes(g.Q6_K, 2048) == 8 * 210
    assert L.ggq_row_bytes(g.Q4_0, 256) == 8 * 18
    assert L.ggq_row_bytes(g.Q5_K, 2048) == 8 * 176
    assert L.ggq_row_bytes(g.Q4_K, 300) == 0
    assert L.ggq_row_bytes(g.Q4_0, 48) == 0
    assert L.ggq_row_bytes(3, 256) == 0                                 # Q4_1: not provided
    assert L.ggq_q8_1_bytes(3, 64) == 3 * 2 * 40


def err(L):
    return L.ggq_last_error().decode()


def test_unsupported_type(L):
    rc = L.ggq_mul_mat(3, FAKE, 16, 2816, FAKE, g.F32, 1, 2816, FAKE, g.F32, 16, None, 0, 0, None)
    assert rc == g.ERR_UNSUPPORTED and "type 3" in err(L)
    assert L.ggq_dequantize(42, FAKE, 1, 256, FAKE, g.F32, None) == g.ERR_UNSUPPORTED


def test_bad_K(L):
    rc = L.ggq_mul_mat(g.Q4_K, FAKE, 16, 300, FAKE, g.F32, 1, 300, FAKE, g.F32, 16, None, 0, 0, None)
    assert rc == g.ERR_INVALID and "K=300" in err(L)
    assert L.ggq_quantize_q8_1(FAKE, g.F32, 1, 33, 33, FAKE, None) == g.ERR_INVALID


def test_bad_strides_and_pointers(L):
    assert L.ggq_mul_mat(g.Q4_K, FAKE, 16, 256, FAKE, g.F32, 1, 128, FAKE, g.F32, 16, None, 0, 0, None) == g.ERR_INVALID
    assert L.ggq_mul_mat(g.Q4_K, FAKE, 16, 256, FAKE, g.F32, 1, 256, FAKE, g.F32, 8, None, 0, 0, None) == g.ERR_INVALID
    assert L.ggq_mul_mat(g.Q4_K, None, 16, 256, FAKE, g.F32, 1, 256, FAKE, g.F32, 16, None, 0, 0, None) == g.ERR_INVALID
    mis = ctypes.c_void_p(0x10002)
    assert L.ggq_mul_mat(g.Q4_K, mis, 16, 256, FAKE, g.F32, 1, 256, FAKE, g.F32, 16, None, 0, 0, None) == g.ERR_INVALID
    assert L.ggq_quantize_q8_1(FAKE, g.F32, 4, 64, 32, FAKE, None) == g.ERR_INVALID


def test_bad_dtypes_and_paths(L):
    assert L.ggq_mul_mat(g.Q4_K, FAKE, 16, 256, FAKE, 7, 1, 256, FAKE, g.F32, 16, None, 0, 0, None) == g.ERR_UNSUPPORTED
    assert L.ggq_mul_mat(g.Q4_K, FAKE, 16, 256, FAKE, g.F32, 1, 256, FAKE, g.Q8_1, 16, None, 0, 0, None) == g.ERR_UNSUPPORTED
    # MMQ for the 32-weight-block types needs K % 256 == 0
    assert L.ggq_mul_mat(g.Q8_0, FAKE, 16, 288, FAKE, g.F32, 64, 288, FAKE, g.F32, 16, None, 0, g.PATH_MMQ, None) == g.ERR_UNSUPPORTED
    assert L.ggq_mul_mat(g.Q4_0, FAKE, 16, 288, FAKE, g.F32, 64, 288, FAKE, g.F32, 16, None, 0, g.PATH_MMQ, None) == g.ERR_UNSUPPORTED
    assert L.ggq_mul_mat_ws(g.Q8_0, 16, 256, g.F32, 64, g.PATH_AUTO) > 0          # MMQ (planar operand)
    assert L.ggq_mul_mat_ws(g.Q8_0, 16, 288, g.F32, 64, g.PATH_AUTO) == 0         # MMVQ
    assert L.ggq_mul_mat_ws(g.Q4_0, 16, 288, g.F32, 4096, g.PATH_AUTO) == 0   # K % 256 != 0: MMVQ at any M
    assert L.ggq_mul_mat(g.Q4_K, FAKE, 16, 256, FAKE, g.F32, 1, 256, FAKE, g.F32, 16, None, 0, 9, None) == g.ERR_INVALID


def test_workspace_too_small(L):
    need = L.ggq_mul_mat_ws(g.Q4_K, 64, 256, g.BF16, 100, g.PATH_AUTO)
    assert need > 0
    rc = L.ggq_mul_mat(g.Q4_K, FAKE, 64, 256, FAKE, g.BF16, 100, 256, FAKE, g.BF16, 64, FAKE, need - 1, 0, None)
    assert rc == g.ERR_WORKSPACE
    assert L.ggq_mul_mat_ws(g.Q4_K, 64, 256, g.Q8_1, 1, g.PATH_AUTO) == 0   # pre-quantized MMVQ needs none


def test_noops(L):
    assert L.ggq_mul_mat(g.Q4_K, None, 0, 256, None, g.F32, 0, 256, None, g.F32, 0, None, 0, 0, None) == g.OK
    assert L.ggq_quantize_q8_1(None, g.F32, 0, 64, 64, None, None) == g.OK
    assert L.ggq_dequantize(g.Q6_K, None, 0, 256, None, g.F32, None) == g.OK


def test_mul_mat_id_validation(L):
    i64 = ctypes.c_int64
    def call(wt=g.Q4_K, E=4, N=32, K=256, stride=None, T=2, xpr=0, top_k=2, epi=0, ws_bytes=1 << 20, path=0, ws=FAKE,
             xdt=g.F32, ydt=g.F32, route_w=None):
        stride = stride if stride is not None else N * L.ggq_row_bytes(wt, K)
        return L.ggq_mul_mat_id(wt, FAKE, E, N, K, stride, FAKE, xdt, T, xpr, FAKE, top_k, route_w, epi,
                                FAKE, ydt, ws, ws_bytes, path, None)
    assert call(stride=32 * 144 - 16) == g.ERR_INVALID          # stride < N * row_bytes
    assert call(stride=32 * 144 + 8) == g.ERR_INVALID           # stride % 16
    assert call(N=33, epi=g.EPI_SWIGLU) == g.ERR_INVALID        # SwiGLU needs even N
    assert call(xpr=2) == g.ERR_INVALID
    assert call(ws_bytes=64) == g.ERR_WORKSPACE
    assert call(wt=g.Q8_0, K=64, path=g.PATH_MMQ) == g.ERR_UNSUPPORTED
    assert call(T=0) == g.OK
    assert call(xdt=4) == g.ERR_UNSUPPORTED
    assert call(ydt=4) == g.ERR_UNSUPPORTED
    assert call(ydt=g.Q8_1, route_w=FAKE) == g.ERR_UNSUPPORTED    # q8_1 output is per route
    assert call(ydt=g.Q8_1, N=48) == g.ERR_INVALID                  # N' % 32
    assert call(ydt=g.Q8_1, N=64, epi=g.EPI_SWIGLU, ws_bytes=64) == g.ERR_WORKSPACE   # N' = 32 passes
    ws_small = L.ggq_mul_mat_id_ws(g.Q4_K, 256, 1024, 2048, g.BF16, 16, 0, 8, 1, 0, 0)
    ws_big = L.ggq_mul_mat_id_ws(g.Q4_K, 256, 1024, 2048, g.BF16, 8192, 0, 8, 1, 0, 0)
    assert 0 < ws_small < ws_big


def test_get_rows_validation(L):
    def call(wt=g.Q4_K, rows=8, K=256, ids=FAKE, n=3, y=FAKE, ydt=g.F32, ldy=256):
        return L.ggq_get_rows(wt, FAKE, rows, K, ids, n, y, ydt, ldy, None)
    assert call(wt=3) == g.ERR_UNSUPPORTED
    assert call(K=300) == g.ERR_INVALID and "K=300" in err(L)
    assert call(ydt=g.Q8_1) == g.ERR_UNSUPPORTED
    assert call(n=-1) == g.ERR_INVALID
    assert call(ldy=128) == g.ERR_INVALID                      # ldy < K
    assert call(ldy=258) == g.ERR_INVALID                      # rows not 16-byte aligned (fp32)
    assert call(ydt=g.BF16, ldy=260) == g.ERR_INVALID          # rows not 16-byte aligned (bf16)
    assert call(ids=None) == g.ERR_INVALID
    assert call(y=ctypes.c_void_p(0x10008)) == g.ERR_INVALID   # y not 16-byte aligned
    assert call(n=0, ids=None, y=None) == g.OK


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(g, "_lib", None)
    monkeypatch.setattr(g, "LIB_PATH", "/nonexistent/libggq.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        g.lib()


def test_bench_hooks_validate_before_launch(L):
    # streaming read: negative size, null buffer, misaligned buffer, small sink
    assert L.ggq_bench_stream_read(FAKE, -16, FAKE, 4096, None) == g.ERR_INVALID
    assert L.ggq_bench_stream_read(None, 1024, FAKE, 4096, None) == g.ERR_INVALID
    assert L.ggq_bench_stream_read(ctypes.c_void_p(0x10004), 1024, FAKE, 4096, None) == g.ERR_INVALID
    assert "aligned" in err(L)
    assert L.ggq_bench_stream_read(FAKE, 1024, FAKE, 1023, None) == g.ERR_WORKSPACE
    assert L.ggq_bench_stream_read(FAKE, 0, None, 0, None) == g.OK              # empty: no launch
    # MFMA loop: unknown kind, negative trips, null or small sink
    assert L.ggq_bench_mfma_loop(2, 10, FAKE, 4096, None) == g.ERR_INVALID
    assert L.ggq_bench_mfma_loop(0, -1, FAKE, 4096, None) == g.ERR_INVALID
    assert L.ggq_bench_mfma_loop(1, 10, None, 4096, None) == g.ERR_INVALID
    assert L.ggq_bench_mfma_loop(1, 10, FAKE, 4095, None) == g.ERR_WORKSPACE


def test_mmvq_k_limit(L):
    """MMVQ keeps one row of K activations in 64 KB of LDS: longer rows are
    refused on the host before any launch (forced MMVQ, or AUTO for types
    without an MMQ kernel at that K), and AUTO takes MMQ when it has one."""
    rc = L.ggq_mul_mat(g.Q4_K, FAKE, 16, 65536, FAKE, g.F32, 1, 65536, FAKE, g.F32, 16, None, 0, g.PATH_MMVQ, None)
    assert rc == g.ERR_UNSUPPORTED and "too long" in err(L) and "use MMQ" in err(L)
    # AUTO at M = 1 now needs MMQ's workspace (the planar activations)
    assert L.ggq_mul_mat_ws(g.Q4_K, 16, 65536, g.F32, 1, g.PATH_AUTO) > 0
    assert L.ggq_mul_mat_ws(g.Q4_K, 16, 4096, g.F32, 1, g.PATH_AUTO) == 0
    rc = L.ggq_mul_mat(g.Q4_K, FAKE, 16, 65536, FAKE, g.F32, 1, 65536, FAKE, g.F32, 16, None, 0, g.PATH_AUTO, None)
    assert rc == g.ERR_WORKSPACE
    # Q8_0 with K % 256 != 0 has no MMQ kernel: refused under AUTO too
    rc = L.ggq_mul_mat(g.Q8_0, FAKE, 16, 65568, FAKE, g.F32, 1, 65568, FAKE, g.F32, 16, None, 0, g.PATH_AUTO, None)
    assert rc == g.ERR_UNSUPPORTED and "too long" in err(L) and "K <= 52416" in err(L)
    # the largest K MMVQ takes (43520 for Q6_K) keeps AUTO on MMVQ at M = 1 (no workspace); one block more goes to MMQ
    assert L.ggq_mul_mat_ws(g.Q6_K, 16, 43520, g.F32, 1, g.PATH_AUTO) == 0
    assert L.ggq_mul_mat_ws(g.Q6_K, 16, 43776, g.F32, 1, g.PATH_AUTO) > 0
    rc = L.ggq_mul_mat_id(g.Q6_K, FAKE, 4, 16, 43776, 16 * 171 * 210, FAKE, g.F32, 2, 0, FAKE, 2, None, 0,
                          FAKE, g.F32, FAKE, 1 << 20, g.PATH_MMVQ, None)
    assert rc == g.ERR_UNSUPPORTED and "too long" in err(L)
