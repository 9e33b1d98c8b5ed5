"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on
the same seeded inputs.

Bars: q8_1 blocks, per-group int32 dots and dequantized weights bit-exact;
fp32 outputs max|gpu - ref| / max|ref| <= 1e-5; bf16 outputs <= 8e-3, where
ref is the oracle's fp64-accumulated result (rounded to fp32, then to bf16 for
bf16 outputs).  Full-size workloads are checked on seeded samples of output
rows / tokens, computed one by one by the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import gguf_block_quantized_q8_amd as g
from gguf_block_quantized_q8_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 8e-3, "f16": 1e-3}     # f16: two units of its 2^-10 relative spacing
TYPES = [g.Q8_0, g.Q4_K, g.Q6_K, g.Q4_0, g.Q5_K]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def T(a, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


def ref_out(y32, kind):
    """Oracle fp32 result as the output dtype would hold it."""
    if kind == "f32":
        return y32
    if kind == "f16":
        return oracle.fp32_to_fp16_array(y32).view(np.float16).astype(np.float32)
    return torch.from_numpy(y32).to(torch.bfloat16).float().numpy()


def log(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ q8_1

@pytest.mark.parametrize("xdt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,K,ldx", [(1, 32, 32), (7, 512, 512), (33, 2048, 2080), (300, 4096, 4096),
                                     (4, 96, 104),                  # ldx % 16 == 8: 8 values per lane
                                     (5, 32, 36), (9, 64, 66)])     # ldx % 8 != 0: the 8-lane kernel
def test_quantize_bit_exact(dev, xdt, M, K, ldx):
    log("quantize", xdt, M, K, ldx)
    x = inputs.gen_act(M, ldx, 1000 + M, xdt)
    if M > 3:
        x[3, :64] = 0                       # all-zero blocks
    xt = T(x, dev)[:, :K] if ldx != K else T(x, dev)
    q = host(g.quantize_q8_1(xt))
    ref = oracle.quantize_q8_1(np.ascontiguousarray(x[:, :K]))
    assert np.array_equal(q, ref)


def test_quantize_ties_and_scales(dev):
    x = np.zeros((4, 64), np.float32)
    x[0, :7] = [127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5]
    x[1] = np.float32(2.5) * np.arange(-32, 32)
    x[2] = np.float32(1e-30) * np.arange(64)                 # tiny values
    x[3] = np.float32(3e37) * np.sin(np.arange(64))          # huge values
    assert np.array_equal(host(g.quantize_q8_1(T(x, dev))), oracle.quantize_q8_1(x))


# ------------------------------------------------------------------ dequantize

@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16, torch.float16])
def test_dequantize_bit_exact(dev, wt, ydt):
    log("dequant", wt, ydt)
    K = 512 if wt == g.Q8_0 else 1024
    W = inputs.gen_weights(wt, 37, K, 7 + wt)
    y = g.dequantize(T(W, dev), wt, K, ydt)
    if ydt == torch.float32:
        assert np.array_equal(host(y).view(np.uint32), oracle.dequantize(wt, W, 37, K).view(np.uint32))
    else:
        ref = oracle.dequantize(wt, W, 37, K, oracle.BF16 if ydt == torch.bfloat16 else oracle.F16)
        assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref)


def test_dequantize_q6_K_large_scales(dev):
    """Q6_K with full-range int8 scales (-128..127), beyond the [-64, 63] draw."""
    W = inputs.gen_q6_K(16, 512, 9)
    r = inputs.rng(10)
    W.reshape(-1, 210)[:, 192:208] = r.integers(-128, 128, (W.size // 210, 16), dtype=np.int8).view(np.uint8)
    y = g.dequantize(T(W, dev), g.Q6_K, 512)
    assert np.array_equal(host(y).view(np.uint32), oracle.dequantize(g.Q6_K, W, 16, 512).view(np.uint32))


@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16, torch.float16])
def test_get_rows_bit_exact(dev, wt, ydt):
    """Gathered rows equal the oracle's dequantized table rows bit for bit; ids
    outside the table give zeros; repeated ids repeat the row."""
    log("get_rows", wt, ydt)
    rows, K = 300, 512
    W = inputs.gen_weights(wt, rows, K, 40 + wt)
    ids = inputs.rng(41).integers(-3, rows + 3, 97).astype(np.int32)
    ids[:4] = [0, rows - 1, 5, 5]
    y = g.get_rows(T(W, dev), wt, K, T(ids, dev), ydt)
    kind = {torch.bfloat16: oracle.BF16, torch.float16: oracle.F16, torch.float32: oracle.F32}[ydt]
    table = oracle.dequantize(wt, W, rows, K, kind)
    ok = (ids >= 0) & (ids < rows)
    ref = np.zeros((ids.size, K), table.dtype)
    ref[ok] = table[ids[ok]]
    got = host(y) if ydt == torch.float32 else y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got.view(np.uint32) if ydt == torch.float32 else got,
                          ref.view(np.uint32) if ydt == torch.float32 else ref)


# Row lengths around the staged kernel's 8192-byte limit, short rows whose
# start phase within a 16-byte line takes every even value (18- and 34-byte
# blocks, an odd number of them), and rows of 2..4 KB: K for each type.
RAGGED_K = {g.Q4_0: [96, 14560, 14592, 4096], g.Q8_0: [96, 7680, 7744, 2048], g.Q4_K: [256, 14336, 14592, 4096],
            g.Q5_K: [768, 11776, 12032, 4096], g.Q6_K: [768, 9984, 10240, 4096]}


@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("ki", [0, 1, 2, 3])
def test_dequant_row_lengths(dev, wt, ki):
    """dequantize and get_rows bit-exact for row lengths at and past the LDS
    staging limit (8064..8400 bytes), rows of 2..4 KB (four loads a lane), and
    short rows at every 16-byte phase, including the last row of a table whose
    end is not 16-byte aligned."""
    K = RAGGED_K[wt][ki]
    rows = 11
    log("dequant rows", wt, K)
    W = inputs.gen_weights(wt, rows, K, 60 + wt + ki)
    y = g.dequantize(T(W, dev), wt, K)
    table = oracle.dequantize(wt, W, rows, K)
    assert np.array_equal(host(y).view(np.uint32), table.view(np.uint32))
    ids = np.array([rows - 1, 0, -1, rows, 3, 3, rows - 2, 7, 2**31 - 1, 1], np.int32)
    yb = g.get_rows(T(W, dev), wt, K, T(ids, dev), torch.bfloat16)
    tb = oracle.dequantize(wt, W, rows, K, oracle.BF16)
    ok = (ids >= 0) & (ids < rows)
    ref = np.zeros((ids.size, K), tb.dtype)
    ref[ok] = tb[ids[ok]]
    assert np.array_equal(yb.view(torch.int16).cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("wt", [g.Q4_K, g.Q6_K, g.Q8_0])
def test_dequant_many_rows_per_wave(dev, wt):
    """More output rows than the staged kernel's 8192 waves, so each wave walks
    several rows with the next row's loads in flight: dequantize of a
    20,000-row table and get_rows of 30,000 ids (a run of invalid ids in the
    middle, so waves go from valid to invalid rows and back), bit-exact."""
    rows, K = 20000, 256
    log("dequant many rows", wt)
    W = inputs.gen_weights(wt, rows, K, 80 + wt)
    table = oracle.dequantize(wt, W, rows, K, oracle.BF16)
    y = g.dequantize(T(W, dev), wt, K, torch.bfloat16)
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), table)
    ids = inputs.rng(81).integers(0, rows, 30000).astype(np.int32)
    ids[12000:12500] = -1
    ids[20000:20003] = [rows, rows + 7, -5]
    yb = g.get_rows(T(W, dev), wt, K, T(ids, dev), torch.bfloat16)
    ok = (ids >= 0) & (ids < rows)
    ref = np.zeros((ids.size, K), np.uint16)
    ref[ok] = table[ids[ok]]
    assert np.array_equal(yb.view(torch.int16).cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32])
def test_get_rows_strided_output(dev, ydt):
    """Output rows ldy > K apart (through the C ABI): each row's K values equal
    the oracle's table row; the gap after each row keeps its canary; a row
    table over 8 KB takes the unstaged kernel with the same result."""
    import ctypes
    L = g.lib()
    for wt, K in [(g.Q6_K, 512), (g.Q8_0, 7744)]:
        log("get_rows strided", wt, K, ydt)
        rows, n = 9, 6
        W = inputs.gen_weights(wt, rows, K, 70 + wt)
        ids = np.array([8, 0, 3, -2, 3, 7], np.int32)
        ldy = K + (8 if ydt == torch.bfloat16 else 4) * 3
        canary = torch.full((n, ldy), -7.0, dtype=ydt, device=dev)
        Wd, idd = T(W, dev), T(ids, dev)
        ydt_c = g.BF16 if ydt == torch.bfloat16 else g.F32
        rc = L.ggq_get_rows(wt, ctypes.c_void_p(Wd.data_ptr()), rows, K, ctypes.c_void_p(idd.data_ptr()), n,
                            ctypes.c_void_p(canary.data_ptr()), ydt_c, ldy, None)
        assert rc == 0
        torch.cuda.synchronize()
        got = canary.float().cpu().numpy()
        table = oracle.dequantize(wt, W, rows, K)
        if ydt == torch.bfloat16:
            table = torch.from_numpy(table).to(torch.bfloat16).float().numpy()
        ok = (ids >= 0) & (ids < rows)
        ref = np.zeros((n, K), np.float32)
        ref[ok] = table[ids[ok]]
        assert np.array_equal(got[:, :K].view(np.uint32), ref.view(np.uint32))
        assert (got[:, K:] == -7.0).all()


def test_get_rows_empty_and_errors(dev):
    W = T(inputs.gen_q4_K(8, 256, 42), dev)
    assert g.get_rows(W, g.Q4_K, 256, torch.empty(0, dtype=torch.int32, device=dev)).shape == (0, 256)
    with pytest.raises(ValueError):
        g.get_rows(W, g.Q4_K, 200, torch.zeros(3, dtype=torch.int32, device=dev))   # K not a multiple of 256


# ------------------------------------------------------------------ per-group int dots

@pytest.mark.parametrize("wt,path", [(g.Q8_0, "mmvq"), (g.Q4_K, "mmvq"), (g.Q6_K, "mmvq"), (g.Q4_K, "mmq"), (g.Q6_K, "mmq"),
                                     (g.Q4_0, "mmvq"), (g.Q5_K, "mmvq"), (g.Q5_K, "mmq"), (g.Q8_0, "mmq"),
                                     (g.Q4_0, "mmq")])
def test_block_dots_bit_exact(dev, wt, path):
    log("dots", wt, path)
    N, K, M = 131, (512 if wt == g.Q8_0 else 768), 133      # ragged against the 128 x 128 MMQ tiles
    W = inputs.gen_weights(wt, N, K, 20 + wt)
    x = inputs.gen_act(M, K, 21, "f32")
    x[5] *= 1e3
    q8 = oracle.quantize_q8_1(x)
    d = host(g.test_block_dots(T(W, dev), wt, T(q8, dev), K, path))
    assert np.array_equal(d, oracle.block_dots(wt, W, N, K, q8, M))


def test_block_dots_q6_K_large_scales_mmq(dev):
    W = inputs.gen_q6_K(64, 512, 30)
    W.reshape(-1, 210)[:, 192:208] = inputs.rng(31).integers(-128, 128, (W.size // 210, 16), dtype=np.int8).view(np.uint8)
    x = inputs.gen_act(40, 512, 32, "f32")
    q8 = oracle.quantize_q8_1(x)
    d = host(g.test_block_dots(T(W, dev), g.Q6_K, T(q8, dev), 512, "mmq"))
    assert np.array_equal(d, oracle.block_dots(g.Q6_K, W, 64, 512, q8, 40))


# ------------------------------------------------------------------ dense mul_mat, small / ragged

def _check_mul_mat(dev, wt, N, K, M, xdt, ydt, path, seed, rows=None, W=None):
    W = inputs.gen_weights(wt, N, K, seed) if W is None else W
    x = inputs.gen_act(M, K, seed + 1, xdt)
    y = g.mul_mat(T(W, dev), wt, T(x, dev), out_dtype=torch.float32 if ydt == "f32" else torch.bfloat16, path=path)
    yh = host(y)
    if rows is not None:
        yh = yh[:, rows]
    ref = ref_out(oracle.mul_mat(wt, W, N, K, x, rows=rows), ydt)
    r = rel(yh, ref)
    log(f"mul_mat type={wt} N={N} K={K} M={M} {xdt}->{ydt} path={path} rel={r:.3g}")
    assert r <= TOL[ydt], r
    return r


@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_mmvq_small(dev, wt, M):
    K = 512 if wt in (g.Q8_0, g.Q4_0) else 768
    _check_mul_mat(dev, wt, 97, K, M, "f32", "f32", "mmvq", 40 + wt)


@pytest.mark.parametrize("wt", [g.Q4_K, g.Q6_K, g.Q5_K])
@pytest.mark.parametrize("K", [256, 512])
def test_mmvq_short_rows(dev, wt, K):
    _check_mul_mat(dev, wt, 300, K, 4, "bf16", "bf16", "mmvq", 50 + K)


def test_mmvq_many_columns(dev):
    """M above the 8 columns of one MMVQ group; Q8_0 / Q4_0 with K not a multiple of
    256 take MMVQ at any M under AUTO."""
    _check_mul_mat(dev, g.Q8_0, 64, 256, 21, "f32", "f32", "mmvq", 60)
    _check_mul_mat(dev, g.Q4_0, 64, 256, 21, "f32", "f32", "mmvq", 61)
    _check_mul_mat(dev, g.Q8_0, 64, 288, 21, "f32", "f32", "auto", 62)
    _check_mul_mat(dev, g.Q4_0, 64, 288, 21, "f32", "f32", "auto", 63)


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
def test_q8_0_full_int8_range(dev, path):
    """Q8_0 quants of -128 (a valid int8 that the [-127, 127] draw never makes)."""
    W = inputs.gen_q8_0(100, 512, 64)
    blocks = W.reshape(-1, 34)
    rng = inputs.rng(65)
    hit = rng.random((blocks.shape[0], 32)) < 0.2
    q = blocks[:, 2:].view(np.int8)
    q[hit] = -128
    _check_mul_mat(dev, g.Q8_0, 100, 512, 40, "f32", "f32", path, 66, W=W)


@pytest.mark.parametrize("wt", [g.Q4_0, g.Q5_K, g.Q8_0])
def test_new_types_decode_shape(dev, wt):
    """The 4096 x 4096 decode shape (bf16 in and out) at M = 1 and 8, and a prefill-sized
    MMQ call, sampled rows against the oracle."""
    W = inputs.gen_weights(wt, 4096, 4096, 90 + wt)
    for M in (1, 8):
        _check_mul_mat(dev, wt, 4096, 4096, M, "bf16", "bf16", "auto", 91 + wt + M, W=W)
    rows = inputs.sample_rows(4096, 128, 95)
    _check_mul_mat(dev, wt, 4096, 4096, 512, "bf16", "bf16", "auto", 96, rows=rows, W=W)


@pytest.mark.parametrize("wt", [g.Q4_K, g.Q6_K, g.Q5_K, g.Q8_0, g.Q4_0])
@pytest.mark.parametrize("M,N,K", [(1, 5, 256), (40, 100, 512), (129, 257, 768), (300, 128, 1024)])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_mmq_small_ragged(dev, wt, M, N, K, ydt):
    _check_mul_mat(dev, wt, N, K, M, "bf16", ydt, "mmq", 70 + M + wt)


def test_mmq_q6_K_large_scales(dev):
    W = inputs.gen_q6_K(200, 512, 80)
    W.reshape(-1, 210)[:, 192:208] = inputs.rng(81).integers(-128, 128, (W.size // 210, 16), dtype=np.int8).view(np.uint8)
    _check_mul_mat(dev, g.Q6_K, 200, 512, 150, "f32", "f32", "mmq", 82, W=W)
    _check_mul_mat(dev, g.Q6_K, 200, 512, 3, "f32", "f32", "mmvq", 83, W=W)


@pytest.mark.parametrize("wt", [g.Q4_K, g.Q6_K, g.Q8_0])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16, torch.float16])
def test_mmq_split_k(dev, wt, ydt):
    """Few tiles, long K: the K range is split over up to 8 workgroups per tile and the
    fp32 partial sums are added in slice order; strided output rows (ldy > N)."""
    N, K, M = 200, 2048, 70
    W = inputs.gen_weights(wt, N, K, 620 + wt)
    x = inputs.gen_act(M, K, 621, "bf16")
    out = torch.full((M, 256), 3.0, dtype=ydt, device=dev)
    g.mul_mat(T(W, dev), wt, T(x, dev), path="mmq", out=out[:, :N])
    kind = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[ydt]
    r = rel(host(out[:, :N]), ref_out(oracle.mul_mat(wt, W, N, K, x), kind))
    log("split-K", wt, kind, r)
    assert r <= TOL[kind]
    assert (out[:, N:] == 3.0).all()


@pytest.mark.parametrize("wt", [g.Q4_K, g.Q6_K, g.Q8_0])
@pytest.mark.parametrize("path,M", [("mmvq", 1), ("mmvq", 5), ("mmq", 40)])
@pytest.mark.parametrize("xdt,pad", [("bf16", 8), ("bf16", 3), ("f32", 1)])
def test_input_row_stride(dev, wt, path, M, xdt, pad):
    """Activation rows ldx = K + pad apart: 16-byte multiples (MMVQ copies the rows
    by DMA, the wide quantizer runs) and odd strides (MMVQ's direct loads at 2-byte
    alignment, the 8-lane quantizer)."""
    N, K = 96, 512
    W = inputs.gen_weights(wt, N, K, 900 + wt)
    xf = inputs.gen_act(M, K + pad, 901 + pad, xdt)
    y = g.mul_mat(T(W, dev), wt, T(xf, dev)[:, :K], out_dtype=torch.float32, path=path)
    r = rel(host(y), oracle.mul_mat(wt, W, N, K, np.ascontiguousarray(xf[:, :K])))
    log("input stride", wt, path, M, xdt, pad, r)
    assert r <= TOL["f32"]


def test_q8_1_input_reuse(dev):
    """Pre-quantized q8_1 input gives the same result as float input, on both paths."""
    W = inputs.gen_q4_K(96, 512, 90)
    x = inputs.gen_act(20, 512, 91, "bf16")
    xt = T(x, dev)
    q8 = g.quantize_q8_1(xt)
    for path in ("mmvq", "mmq"):
        a = g.mul_mat(T(W, dev), g.Q4_K, xt, out_dtype=torch.float32, path=path)
        b = g.mul_mat(T(W, dev), g.Q4_K, q8, K=512, path=path)
        assert torch.equal(a, b), path


def test_output_row_stride(dev):
    W = inputs.gen_q6_K(64, 256, 92)
    x = inputs.gen_act(12, 256, 93, "f32")
    out = torch.full((12, 80), 7.0, device=dev)
    for path in ("mmvq", "mmq"):
        g.mul_mat(T(W, dev), g.Q6_K, T(x, dev), path=path, out=out[:, :64])
        assert (out[:, 64:] == 7.0).all()
        assert rel(host(out[:, :64]), oracle.mul_mat(g.Q6_K, W, 64, 256, x)) <= 1e-5


# ------------------------------------------------------------------ full-size workloads (sampled)

def test_c1_q8_0_matvec(dev):
    for M in (1, 4):
        _check_mul_mat(dev, g.Q8_0, 256, 512, M, "f32", "f32", "auto", 101)


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_c2_q4_K_decode(dev, M):
    W = inputs.gen_q4_K(4096, 4096, 201)
    x = inputs.gen_act(M, 4096, 202, "bf16")
    y = host(g.mul_mat(T(W, dev), g.Q4_K, T(x, dev)))
    r = rel(y, ref_out(oracle.mul_mat(g.Q4_K, W, 4096, 4096, x), "bf16"))
    log("C2 M", M, "rel", r)
    assert r <= TOL["bf16"]


def test_c3_q4_K_prefill_sampled(dev):
    W = inputs.gen_q4_K(8192, 2048, 301)
    x = inputs.gen_act(8192, 2048, 302, "bf16")
    y = host(g.mul_mat(T(W, dev), g.Q4_K, T(x, dev)))
    rows = inputs.sample_rows(8192, 256, 303)
    r = rel(y[:, rows], ref_out(oracle.mul_mat(g.Q4_K, W, 8192, 2048, x, rows=rows), "bf16"))
    log("C3 sampled rel", r)
    assert r <= TOL["bf16"]


@pytest.mark.parametrize("M", [16, 24, 32, 64])
def test_c3_crossover_sweep_both_paths(dev, M):
    W = inputs.gen_q4_K(8192, 2048, 301)
    x = inputs.gen_act(M, 2048, 302, "bf16")
    ref = ref_out(oracle.mul_mat(g.Q4_K, W, 8192, 2048, x), "bf16")
    for path in ("mmvq", "mmq"):
        r = rel(host(g.mul_mat(T(W, dev), g.Q4_K, T(x, dev), path=path)), ref)
        log("C3 sweep M", M, path, r)
        assert r <= TOL["bf16"]


# Long single-column matrices: a wave walks many work items, so the kernel keeps
# two of them in flight (the lm_head-sized case); odd N (last row pair half
# empty), K split over two items per row, and a weight end that is 2-byte but
# not 4-byte aligned (the tail patch) are all covered here.
@pytest.mark.parametrize("wt,N,K,xdt,ydt,M", [
    (g.Q4_K, 262147, 512, "bf16", "bf16", 1),
    (g.Q4_K, 262147, 512, "f32", "f32", 2),
    (g.Q4_K, 12289, 16384, "f32", "f32", 1),
    (g.Q8_0, 2000001, 32, "bf16", "f32", 1),
    (g.Q6_K, 400001, 256, "f32", "bf16", 1),
    (g.Q5_K, 200001, 1024, "bf16", "bf16", 1),
])
def test_mmvq_long_matrix(dev, wt, N, K, xdt, ydt, M):
    log("long matrix", wt, N, K, xdt, ydt, "M", M)
    W = inputs.gen_weights(wt, N, K, 700 + wt)
    x = inputs.gen_act(M, K, 701, xdt)
    out = torch.float32 if ydt == "f32" else torch.bfloat16
    y = host(g.mul_mat(T(W, dev), wt, T(x, dev), out_dtype=out, path="mmvq"))
    r = rel(y, ref_out(oracle.mul_mat(wt, W, N, K, x), ydt))
    log("  rel", r)
    assert r <= TOL[ydt]


def test_c4_q6_K_lm_head_m1_all_rows(dev):
    W = inputs.gen_q6_K(248320, 2048, 401)
    x = inputs.gen_act(1, 2048, 402, "bf16")
    y = host(g.mul_mat(T(W, dev), g.Q6_K, T(x, dev), out_dtype=torch.float32))
    r = rel(y, oracle.mul_mat(g.Q6_K, W, 248320, 2048, x))
    log("C4 M=1 rel", r)
    assert r <= TOL["f32"]


def test_get_rows_full_table_sampled(dev):
    """The get_rows workload as timed: 8192 ids over the whole 248320 x 2048
    Q6_K table, bf16 out; 96 sampled output rows bit-exact against the
    oracle's dequantization of their table rows, plus every row's first and
    last 16 values."""
    rows, K, n = 248320, 2048, 8192
    W = inputs.gen_q6_K(rows, K, 401)
    ids = inputs.rng(404).integers(0, rows, n).astype(np.int32)
    y = g.get_rows(T(W, dev), g.Q6_K, K, T(ids, dev), torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    rb = W.size // rows
    Wr = W.reshape(rows, rb)
    pick = inputs.rng(405).choice(n, 96, replace=False)
    ref = oracle.dequantize(g.Q6_K, np.ascontiguousarray(Wr[ids[pick]]).reshape(-1), 96, K, oracle.BF16)
    assert np.array_equal(y[pick], ref)
    # ends of every row: the first and the last block of each id
    first = oracle.dequantize(g.Q6_K, np.ascontiguousarray(Wr[ids, :210]).reshape(-1), n, 256, oracle.BF16)
    last = oracle.dequantize(g.Q6_K, np.ascontiguousarray(Wr[ids, rb - 210:]).reshape(-1), n, 256, oracle.BF16)
    assert np.array_equal(y[:, :16], first[:, :16])
    assert np.array_equal(y[:, -16:], last[:, -16:])


def test_c4_q6_K_lm_head_m2048_sampled(dev):
    W = inputs.gen_q6_K(248320, 2048, 401)
    x = inputs.gen_act(2048, 2048, 402, "bf16")
    y = g.mul_mat(T(W, dev), g.Q6_K, T(x, dev), out_dtype=torch.float32)
    rows = inputs.sample_rows(248320, 4096, 403)
    yh = y[:, torch.from_numpy(rows).to(dev)].cpu().numpy()
    del y
    r = rel(yh, oracle.mul_mat(g.Q6_K, W, 248320, 2048, x, rows=rows))
    log("C4 M=2048 sampled rel", r)
    assert r <= TOL["f32"]


# ------------------------------------------------------------------ routed experts

def _moe_ref(wt, W, K, x, ids, top_k, route_w=None, epi=oracle.EPI_NONE, x_per_route=False, tokens=None,
             route_round=None):
    E, N = W.shape[0], W.shape[1]
    Tn = ids.shape[0]
    return oracle.mul_mat_id(wt, W, E, N, K, W.shape[1] * W.shape[2], x, Tn, int(x_per_route), ids, top_k,
                             route_w=route_w, epi=epi, tokens=tokens, route_round=route_round)


@pytest.mark.parametrize("path,wt", [("mmvq", g.Q4_K), ("mmq", g.Q4_K), ("mmvq", g.Q6_K), ("mmq", g.Q6_K),
                                     ("mmvq", g.Q5_K), ("mmq", g.Q5_K), ("mmvq", g.Q4_0), ("mmq", g.Q4_0),
                                     ("mmvq", g.Q8_0), ("mmq", g.Q8_0)])
def test_moe_edge_routes(dev, path, wt):
    """Duplicate ids in a token, inactive (-1) and out-of-range ids, experts with no routes."""
    E, N, K, Tn, top_k = 9, 96, 512, 37, 4
    W = inputs.gen_experts(wt, E, N, K, 500 + wt)
    x = inputs.gen_act(Tn, K, 501, "f32")
    ids = inputs.rng(502).integers(0, 5, (Tn, top_k)).astype(np.int32)   # experts 5..8 get nothing
    ids[0] = [1, 1, 1, 1]
    ids[1, 2] = -1
    ids[2, 0] = 12                                                      # >= E: skipped and counted
    ids[3] = [-1, -1, -1, -1]
    y, ws = g.mul_mat_id(T(W, dev), wt, T(x, dev), T(ids, dev), K, out_dtype=torch.float32, path=path,
                         return_workspace=True)
    ref = _moe_ref(wt, W, K, x, ids, top_k)
    r = rel(host(y), ref)
    log("moe edges", wt, path, r)
    assert r <= TOL["f32"]
    assert (host(y)[1, 2] == 0).all() and (host(y)[3] == 0).all() and (host(y)[2, 0] == 0).all()
    assert int(ws[:4].view(torch.int32).item()) == 1


@pytest.mark.parametrize("epi", [0, 1])
def test_moe_decode_many_experts_edges(dev, epi):
    """Routed decode with many active experts and long expert matrices, the
    shape where each wave walks several items and keeps two in flight:
    duplicate, inactive and out-of-range ids, plain and SwiGLU outputs."""
    E, N, K, Tn, top_k = 128, 4096, 512, 16, 8                           # one route per expert on average: one-route groups
    W = inputs.gen_experts(g.Q4_K, E, N, K, 530)
    x = inputs.gen_act(Tn, K, 531, "bf16")
    ids = inputs.rng(532).integers(0, E, (Tn, top_k)).astype(np.int32)
    ids[0] = 5                                                           # one token, one expert, 8 times
    ids[1, :3] = -1
    ids[2, 7] = E + 3                                                    # skipped and counted
    y, ws = g.mul_mat_id(T(W, dev), g.Q4_K, T(x, dev), T(ids, dev), K, epi=epi, out_dtype=torch.float32,
                         path="mmvq", return_workspace=True)
    ref = _moe_ref(g.Q4_K, W, K, x, ids, top_k, epi=oracle.EPI_SWIGLU if epi else oracle.EPI_NONE)
    r = rel(host(y), ref)
    log("moe decode, many experts", epi, r)
    assert r <= TOL["f32"]
    assert (host(y)[1, :3] == 0).all() and (host(y)[2, 7] == 0).all()
    assert int(ws[:4].view(torch.int32).item()) == 1


@pytest.mark.parametrize("case", ["weighted_bf16", "plain_f32", "swiglu_bf16", "swiglu_q8_1"])
def test_moe_direct_routes(dev, case):
    """Routes <= experts: every MMVQ group is one route, taken straight from ids
    (no route tables).  Duplicate, inactive and out-of-range ids; the out-of-range
    count at workspace offset 0; zero rows for inactive routes of a plain output;
    a q8_1 output equal to ggq_quantize_q8_1 of the bf16 output."""
    E, H, I, Tn, top_k = 64, 512, 256, 6, 8
    swiglu = case.startswith("swiglu")
    N, K = (2 * I, H) if swiglu else (H, I)
    W = inputs.gen_experts(g.Q4_K if swiglu else g.Q6_K, E, N, K, 540)
    wt = g.Q4_K if swiglu else g.Q6_K
    x = inputs.gen_act(Tn, K, 541, "bf16" if case != "plain_f32" else "f32")
    ids, w = inputs.gen_routing(Tn, E, top_k, 542)
    ids[0, :3] = 7                                                       # one expert, three routes of a token
    ids[1, 1] = -1
    ids[4] = -1                                                          # a token with no active route
    ids[2, 5] = E + 1                                                    # skipped and counted
    ids[5, 0] = E + 40
    epi = g.EPI_SWIGLU if swiglu else g.EPI_NONE
    oepi = oracle.EPI_SWIGLU if swiglu else oracle.EPI_NONE
    xt, idt = T(x, dev), T(ids, dev)
    weighted = case == "weighted_bf16"
    odt = torch.float32 if case == "plain_f32" else torch.bfloat16
    rw = T(w, dev) if weighted else None
    y, ws = g.mul_mat_id(T(W, dev), wt, xt, idt, K, route_w=rw, epi=epi, out_dtype=odt, path="mmvq",
                         return_workspace=True)
    ref = _moe_ref(wt, W, K, x, ids, top_k, route_w=w if weighted else None, epi=oepi,
                   route_round="bf16" if weighted else None)
    r = rel(host(y), ref)
    log("moe direct routes", case, r)
    assert r <= TOL["f32" if odt == torch.float32 else "bf16"]
    assert int(ws[:4].view(torch.int32).item()) == 2
    if not weighted:
        yh = host(y)
        assert (yh[ids < 0] == 0).all() and (yh[ids >= E] == 0).all()
    if case == "swiglu_q8_1":
        yq = g.mul_mat_id(T(W, dev), wt, xt, idt, K, epi=epi, out_dtype="q8_1", path="mmvq")
        Np = N // 2
        want = g.quantize_q8_1(y.reshape(Tn * top_k, Np)).reshape(yq.shape)
        assert torch.equal(yq, want)


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
def test_moe_edge_routes_many(dev, path):
    """Over 16K routes (the multi-workgroup route build): hot and empty experts,
    inactive and out-of-range ids, all counted and skipped as in the small case."""
    E, N, K, Tn, top_k = 9, 96, 512, 5000, 4
    W = inputs.gen_experts(g.Q4_K, E, N, K, 520)
    x = inputs.gen_act(Tn, K, 521, "f32")
    rng = inputs.rng(522)
    ids = rng.integers(0, 6, (Tn, top_k)).astype(np.int32)             # experts 6..8 get nothing
    ids[rng.random((Tn, top_k)) < 0.3] = 2                              # one hot expert
    ids[rng.random((Tn, top_k)) < 0.02] = -1
    bad = rng.random((Tn, top_k)) < 0.01
    ids[bad] = 9 + rng.integers(0, 100, int(bad.sum())).astype(np.int32)
    y, ws = g.mul_mat_id(T(W, dev), g.Q4_K, T(x, dev), T(ids, dev), K, out_dtype=torch.float32, path=path,
                         return_workspace=True)
    ref = _moe_ref(g.Q4_K, W, K, x, ids, top_k)
    r = rel(host(y), ref)
    log("moe edges, many routes", path, r, "bad", int(bad.sum()))
    assert r <= TOL["f32"]
    assert (host(y)[ids < 0] == 0).all() and (host(y)[ids >= E] == 0).all()
    assert int(ws[:4].view(torch.int32).item()) == int(bad.sum())


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
def test_moe_all_routes_one_expert(dev, path):
    E, N, K, Tn, top_k = 4, 64, 256, 300, 2
    W = inputs.gen_experts(g.Q4_K, E, N, K, 510)
    x = inputs.gen_act(Tn, K, 511, "bf16")
    ids = np.full((Tn, top_k), 2, np.int32)
    y = g.mul_mat_id(T(W, dev), g.Q4_K, T(x, dev), T(ids, dev), K, out_dtype=torch.float32, path=path)
    assert rel(host(y), _moe_ref(g.Q4_K, W, K, x, ids, top_k)) <= TOL["f32"]


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
def test_moe_swiglu_and_weighted_gather(dev, path):
    E, H, I, Tn, top_k = 16, 512, 256, 45, 4
    Wgu = inputs.gen_experts(g.Q4_K, E, 2 * I, H, 520)
    Wd = inputs.gen_experts(g.Q6_K, E, H, I, 521)
    x = inputs.gen_act(Tn, H, 522, "bf16")
    ids, w = inputs.gen_routing(Tn, E, top_k, 523)
    h = g.mul_mat_id(T(Wgu, dev), g.Q4_K, T(x, dev), T(ids, dev), H, epi=g.EPI_SWIGLU, path=path)
    h_ref32 = _moe_ref(g.Q4_K, Wgu, H, x, ids, top_k, epi=oracle.EPI_SWIGLU)
    r = rel(host(h), ref_out(h_ref32, "bf16"))
    log("swiglu", path, r)
    assert r <= TOL["bf16"]
    # down projection on identical inputs (the oracle's bf16 h) -> same q8_1 decisions
    h_in = oracle.fp32_to_bf16_array(h_ref32)
    y = g.mul_mat_id(T(Wd, dev), g.Q6_K, T(h_in, dev), T(ids, dev), I, route_w=T(w, dev), x_per_route=True,
                     out_dtype=torch.float32, path=path)
    r = rel(host(y), _moe_ref(g.Q6_K, Wd, I, h_in, ids, top_k, route_w=w, x_per_route=True))
    log("weighted down", path, r)
    assert r <= TOL["f32"]


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
@pytest.mark.parametrize("wt", [g.Q4_K, g.Q6_K, g.Q8_0])
def test_fp16_activations_and_outputs(dev, path, wt):
    """fp16 in, fp16 out (and fp16 in, fp32 out) on both paths."""
    N, K, M = 200, 512, (5 if path == "mmvq" else 70)
    W = inputs.gen_weights(wt, N, K, 600 + wt)
    x = inputs.gen_act(M, K, 601, "f16")
    ref = oracle.mul_mat(wt, W, N, K, x)
    yh = g.mul_mat(T(W, dev), wt, T(x, dev), path=path)
    assert yh.dtype == torch.float16
    r16 = rel(host(yh), ref_out(ref, "f16"))
    y32 = g.mul_mat(T(W, dev), wt, T(x, dev), out_dtype=torch.float32, path=path)
    r32 = rel(host(y32), ref)
    log("fp16", wt, path, r16, r32)
    assert r16 <= TOL["f16"] and r32 <= TOL["f32"]


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
def test_fp16_moe_layer(dev, path):
    """The routed layer in fp16: SwiGLU gate_up with fp16 h (and its q8_1 form,
    rounded to fp16 before quantizing), weighted down with fp16 output.  The
    activations are scaled by 1/16 so that h (a product of two projections)
    stays inside fp16's range (65504)."""
    E, H, I, Tn, top_k = 16, 512, 256, 45, 4
    Wgu = inputs.gen_experts(g.Q4_K, E, 2 * I, H, 610)
    Wd = inputs.gen_experts(g.Q6_K, E, H, I, 611)
    x = (inputs.gen_act(Tn, H, 612, "f32") * np.float32(1 / 16)).astype(np.float16)
    ids, w = inputs.gen_routing(Tn, E, top_k, 613)
    ids[2, 1] = -1
    Wgu_t, Wd_t, ids_t, w_t = T(Wgu, dev), T(Wd, dev), T(ids, dev), T(w, dev)
    h = g.mul_mat_id(Wgu_t, g.Q4_K, T(x, dev), ids_t, H, epi=g.EPI_SWIGLU, path=path)
    assert h.dtype == torch.float16
    h_ref = _moe_ref(g.Q4_K, Wgu, H, x, ids, top_k, epi=oracle.EPI_SWIGLU)
    assert rel(host(h), ref_out(h_ref, "f16")) <= TOL["f16"]
    hq = g.mul_mat_id(Wgu_t, g.Q4_K, T(x, dev), ids_t, H, epi=g.EPI_SWIGLU, out_dtype="q8_1", path=path)
    h_gpu = h.cpu().numpy()
    assert np.array_equal(hq.cpu().numpy().reshape(Tn * top_k, -1), oracle.quantize_q8_1(h_gpu.reshape(Tn * top_k, I)))
    y = g.mul_mat_id(Wd_t, g.Q6_K, h, ids_t, I, route_w=w_t, x_per_route=True, path=path)
    assert y.dtype == torch.float16
    y_ref = _moe_ref(g.Q6_K, Wd, I, h_gpu, ids, top_k, route_w=w, x_per_route=True, route_round="f16")
    r = rel(host(y), ref_out(y_ref, "f16"))
    log("fp16 moe", path, r)
    assert r <= TOL["f16"]


def _bits(y):
    """Output tensor as the oracle's input array: bf16 bits (uint16) or float32."""
    if y.dtype == torch.bfloat16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy()


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
@pytest.mark.parametrize("epi", [g.EPI_NONE, g.EPI_SWIGLU])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_moe_q8_1_output(dev, path, epi, xdt):
    """q8_1 output: each route's outputs as q8_1 blocks, equal bit for bit to the
    oracle's q8_1 of the same call's plain output (bf16 for bf16 input, else
    fp32).  Tiles cover partial weight tiles (N' = 160 and 192); inactive and
    out-of-range routes give all-zero blocks."""
    E, K, Tn, top_k = 9, 512, 41, 4
    N = 320 if epi == g.EPI_SWIGLU else 192
    Np = N // 2 if epi == g.EPI_SWIGLU else N
    W = inputs.gen_experts(g.Q4_K, E, N, K, 530)
    x = inputs.gen_act(Tn, K, 531, xdt)
    ids = inputs.rng(532).integers(0, 6, (Tn, top_k)).astype(np.int32)
    ids[0] = [2, 2, 2, 2]
    ids[1, 1] = -1
    ids[2, 3] = 40                                                      # >= E
    kind = torch.bfloat16 if xdt == "bf16" else torch.float32
    args = (T(W, dev), g.Q4_K, T(x, dev), T(ids, dev), K)
    y = g.mul_mat_id(*args, epi=epi, out_dtype=kind, path=path)
    q = g.mul_mat_id(*args, epi=epi, out_dtype="q8_1", path=path)
    R = Tn * top_k
    want = oracle.quantize_q8_1(_bits(y).reshape(R, Np))
    got = q.cpu().numpy().reshape(R, -1)
    log("q8_1 out", path, epi, xdt, "blocks equal:", np.array_equal(got, want))
    assert np.array_equal(got, want)
    dead = ((ids < 0) | (ids >= E)).reshape(R)
    assert (got[dead] == 0).all()
    ref = _moe_ref(g.Q4_K, W, K, x, ids, top_k, epi=epi)
    assert rel(host(y), ref_out(ref, "bf16" if xdt == "bf16" else "f32")) <= TOL["bf16" if xdt == "bf16" else "f32"]


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
@pytest.mark.parametrize("x_per_route", [False, True])
def test_moe_q8_1_input(dev, path, x_per_route):
    """q8_1 activations in: the same result as the oracle on the float rows
    those blocks are the quantization of (identical q8_1 decisions)."""
    E, N, K, Tn, top_k = 16, 256, 512, 45, 4
    W = inputs.gen_experts(g.Q6_K, E, N, K, 540)
    ids, w = inputs.gen_routing(Tn, E, top_k, 541)
    ids[3, 0] = -1
    rows = Tn * top_k if x_per_route else Tn
    x = inputs.gen_act(rows, K, 542, "bf16")
    q8 = oracle.quantize_q8_1(x)
    xq = T(q8, dev).view(Tn, top_k, -1) if x_per_route else T(q8, dev)
    xf = x.reshape(Tn, top_k, K) if x_per_route else x
    y = g.mul_mat_id(T(W, dev), g.Q6_K, xq, T(ids, dev), K, x_per_route=x_per_route, out_dtype=torch.float32,
                     path=path)
    r = rel(host(y), _moe_ref(g.Q6_K, W, K, xf, ids, top_k, x_per_route=x_per_route))
    yw = g.mul_mat_id(T(W, dev), g.Q6_K, xq, T(ids, dev), K, route_w=T(w, dev), x_per_route=x_per_route,
                      out_dtype=torch.float32, path=path)
    rw = rel(host(yw), _moe_ref(g.Q6_K, W, K, xf, ids, top_k, route_w=w, x_per_route=x_per_route))
    log("q8_1 in", path, x_per_route, r, rw)
    assert r <= TOL["f32"] and rw <= TOL["f32"]


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
def test_moe_layer_q8_1_chain(dev, path):
    """gate_up with SwiGLU straight to q8_1, then the weighted down projection
    from those blocks: the same bits as the chain through a bf16 h."""
    E, H, I, Tn, top_k = 16, 512, 256, 45, 4
    Wgu = T(inputs.gen_experts(g.Q4_K, E, 2 * I, H, 550), dev)
    Wd = T(inputs.gen_experts(g.Q6_K, E, H, I, 551), dev)
    x = T(inputs.gen_act(Tn, H, 552, "bf16"), dev)
    ids, w = inputs.gen_routing(Tn, E, top_k, 553)
    ids, w = T(ids, dev), T(w, dev)
    h = g.mul_mat_id(Wgu, g.Q4_K, x, ids, H, epi=g.EPI_SWIGLU, path=path)
    y0 = g.mul_mat_id(Wd, g.Q6_K, h, ids, I, route_w=w, x_per_route=True, path=path)
    hq = g.mul_mat_id(Wgu, g.Q4_K, x, ids, H, epi=g.EPI_SWIGLU, out_dtype="q8_1", path=path)
    y1 = g.mul_mat_id(Wd, g.Q6_K, hq, ids, I, route_w=w, x_per_route=True, out_dtype=torch.bfloat16, path=path)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


def _c5(dev, Tn, path, tokens=None):
    E, H, I, top_k = 256, 2048, 512, 8
    Wgu = inputs.gen_experts(g.Q4_K, E, 2 * I, H, 501)
    Wd = inputs.gen_experts(g.Q6_K, E, H, I, 502)
    x = inputs.gen_act(Tn, H, 503, "bf16")
    ids, w = inputs.gen_routing(Tn, E, top_k, 504)
    Wgu_t, Wd_t, x_t, ids_t, w_t = T(Wgu, dev), T(Wd, dev), T(x, dev), T(ids, dev), T(w, dev)
    h = g.mul_mat_id(Wgu_t, g.Q4_K, x_t, ids_t, H, epi=g.EPI_SWIGLU, path=path)
    y = g.mul_mat_id(Wd_t, g.Q6_K, h, ids_t, I, route_w=w_t, x_per_route=True, path=path)
    hh = host(h)
    yh = host(y)
    sel = slice(None) if tokens is None else tokens
    h_ref32 = _moe_ref(g.Q4_K, Wgu, H, x, ids, top_k, epi=oracle.EPI_SWIGLU, tokens=tokens)
    r_h = rel(hh[sel], ref_out(h_ref32, "bf16"))
    # down on the GPU's own h (identical inputs for the oracle)
    h_gpu = h.view(torch.int16).cpu().numpy().view(np.uint16)
    y_ref32 = _moe_ref(g.Q6_K, Wd, I, h_gpu, ids, top_k, route_w=w, x_per_route=True, tokens=tokens,
                       route_round="bf16")
    r_y = rel(yh[sel], ref_out(y_ref32, "bf16"))
    log(f"C5 T={Tn} path={path} gate_up rel={r_h:.3g} down rel={r_y:.3g}")
    assert r_h <= TOL["bf16"] and r_y <= TOL["bf16"]
    # the layer through q8_1 h (fused quantization in the gate_up epilogue): the same bits
    hq = g.mul_mat_id(Wgu_t, g.Q4_K, x_t, ids_t, H, epi=g.EPI_SWIGLU, out_dtype="q8_1", path=path)
    assert np.array_equal(hq.cpu().numpy().reshape(Tn * top_k, -1), oracle.quantize_q8_1(h_gpu.reshape(Tn * top_k, I)))
    yq = g.mul_mat_id(Wd_t, g.Q6_K, hq, ids_t, I, route_w=w_t, x_per_route=True, out_dtype=torch.bfloat16, path=path)
    assert torch.equal(yq.view(torch.int16), y.view(torch.int16))


def test_c5_moe_t16(dev):
    _c5(dev, 16, "auto")


def test_c5_moe_t16_mmq(dev):
    _c5(dev, 16, "mmq")


def test_c5_moe_t8192_sampled(dev):
    toks = inputs.sample_rows(8192, 512, 505)
    _c5(dev, 8192, "auto", tokens=toks)


# ------------------------------------------------------------------ streams and graphs

def _graph_case(dev):
    """Static inputs and a step that runs every kind of call once: quantize,
    MMVQ and MMQ (split K) dense calls, and a routed layer twice (16 tokens:
    the one-workgroup route build; 2100 tokens x 8: the multi-kernel build with
    its counter fills), unweighted SwiGLU gate_up and a weighted down."""
    E, H, I, top_k = 8, 1024, 256, 8
    W = T(inputs.gen_q4_K(512, H, 810), dev)
    Wgu = T(inputs.gen_experts(g.Q4_K, E, 2 * I, H, 811), dev)
    Wd = T(inputs.gen_experts(g.Q6_K, E, H, I, 812), dev)
    st = {"x1": torch.empty((1, H), dtype=torch.bfloat16, device=dev),
          "x2": torch.empty((64, H), dtype=torch.bfloat16, device=dev)}
    for Tn in (16, 2100):
        st[f"xt{Tn}"] = torch.empty((Tn, H), dtype=torch.bfloat16, device=dev)
        st[f"ids{Tn}"] = torch.empty((Tn, top_k), dtype=torch.int32, device=dev)
        st[f"w{Tn}"] = torch.empty((Tn, top_k), dtype=torch.float32, device=dev)

    def fill(seed):
        st["x1"].copy_(T(inputs.gen_act(1, H, seed, "bf16"), dev))
        st["x2"].copy_(T(inputs.gen_act(64, H, seed + 1, "bf16"), dev))
        for Tn in (16, 2100):
            st[f"xt{Tn}"].copy_(T(inputs.gen_act(Tn, H, seed + 2, "bf16"), dev))
            ids, w = inputs.gen_routing(Tn, E, top_k, seed + 3)
            ids[0, 1] = -1                                  # an inactive route
            st[f"ids{Tn}"].copy_(T(ids, dev))
            st[f"w{Tn}"].copy_(T(w, dev))

    def step():
        out = [g.quantize_q8_1(st["x2"]),
               g.mul_mat(W, g.Q4_K, st["x1"], path="mmvq"),
               g.mul_mat(W, g.Q4_K, st["x2"], path="mmq")]
        for Tn in (16, 2100):
            h = g.mul_mat_id(Wgu, g.Q4_K, st[f"xt{Tn}"], st[f"ids{Tn}"], H, epi=g.EPI_SWIGLU)
            out += [h, g.mul_mat_id(Wd, g.Q6_K, h, st[f"ids{Tn}"], I, route_w=st[f"w{Tn}"], x_per_route=True)]
        return out

    return fill, step


def test_side_stream_matches_default(dev):
    fill, step = _graph_case(dev)
    fill(820)
    ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_graph_replay_matches_eager(dev):
    """Captured once, replayed three times on new inputs with eager work and
    synchronizations between replays: every replay equals the eager call bit
    for bit (all kernels are deterministic)."""
    fill, step = _graph_case(dev)
    fill(830)
    step()                                                  # warm call before capture
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        outs = step()
    for rep in range(3):
        fill(840 + 10 * rep)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        ref = step()                                        # eager, same inputs
        torch.cuda.synchronize()
        log("graph replay", rep)
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
