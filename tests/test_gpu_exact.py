"""Bit-exact parity of the production kernels on exact-arithmetic inputs.

Every weight scale (d, dmin) is 1 or 2, every sub-scale a small integer, every
activation an integer times a q8_1 scale of 1 or 2 (one value of each 32-block
is +-127 times that scale, so the block's d = amax / 127 is exactly 1 or 2
and each quant equals the integer it was built from).  Then every product
and partial sum the kernels form -- per-block int dots, sub-scale and scale
multiplies, super-block sums, the Q4_K / Q5_K min term, split-K partials,
route weights of 1 or 2 -- is an integer below 2^24 (checked per case from
the construction's bounds), which fp32 holds exactly in any order.  So the
fp32 output must equal the oracle's bit for bit, and a one-unit error in
any block's int32 dot of the MMVQ, MMQ, split-K or routed kernels shows up
as a different output.  This checks the production kernels themselves, not
the separate block-dot test hook.

The second half feeds exact and near ties of the q8_1 rounding rule (round
half away from zero: FreeToken PR #690 quantizes activations to q8_1 as the
ggml q8_1 format defines it) through every quantizer: the standalone kernels
(2-, 4- and 8-lane), the MMVQ prologue, the MMQ operand writer, and the
routed q8_1 output of both paths.
"""
import numpy as np
import pytest
import torch

import oracle
import gguf_block_quantized_q8_amd as g
from gguf_block_quantized_q8_amd import inputs
from tests import gguf_pack as gp

pytestmark = pytest.mark.gpu

TYPES = [g.Q8_0, g.Q4_K, g.Q6_K, g.Q4_0, g.Q5_K]
EXACT = 1 << 24          # integers below this are exact in fp32
F16_ONE, F16_TWO = 0x3C00, 0x4000


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def T(a, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def log(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ exact inputs

def exact_weights(t, N, K, seed, smax=6):
    """Random quants (the workload generator's bytes) with every scale field
    replaced: d, dmin in {1, 2}; Q4_K / Q5_K sub-scales and mins in [0, smax];
    Q6_K int8 sub-scales in [-smax, smax].  Returns (bytes [N, row_bytes],
    the largest magnitude per weight of any partial term the kernels form)."""
    W = inputs.gen_weights(t, N, K, seed)
    r = inputs.rng(seed + 7919)
    qk, bb = inputs.BLOCK[t]
    blk = W.reshape(-1, bb)
    nb = blk.shape[0]
    dbits = r.choice(np.array([F16_ONE, F16_TWO], np.uint16), nb)
    if t in (g.Q8_0, g.Q4_0):
        blk[:, 0:2] = dbits.view(np.uint8).reshape(nb, 2)
        # Q8_0: |q| <= 128; Q4_0: nibble (<= 15) and the -8 offset as separate partial terms
        return W, 2 * (128 if t == g.Q8_0 else 23)
    if t in (g.Q4_K, g.Q5_K):
        # a table of 64 headers (d, dmin, 8 sub-scales, 8 mins) packed by the test packer
        hdr = np.zeros((64, 16), np.uint8)
        for i in range(64):
            sc = r.integers(0, smax + 1, 8)
            mn = r.integers(0, smax + 1, 8)
            d = int(r.choice([F16_ONE, F16_TWO]))
            dm = int(r.choice([F16_ONE, F16_TWO]))
            if t == g.Q4_K:
                hdr[i] = gp.pack_q4_K(d, dm, sc, mn, np.zeros(256, int))[:16]
            else:
                hdr[i] = gp.pack_q5_K(d, dm, sc, mn, np.zeros(256, int))[:16]
        blk[:, 0:16] = hdr[r.integers(0, 64, nb)]
        qmax = 15 if t == g.Q4_K else 31
        return W, 2 * smax * qmax + 2 * smax
    # Q6_K: sub-scales in [-smax, smax]; partial terms up to d |sc| (q6 + 32) with q6 <= 63
    # (inside one 32-block, MMQ's two exact operand parts of |sc| <= 16 stay below
    # 31 * 32 * 220 < 2^24 whatever the construction)
    assert smax <= 16
    blk[:, 192:208] = r.integers(-smax, smax + 1, (nb, 16)).astype(np.int8).view(np.uint8)
    blk[:, 208:210] = dbits.view(np.uint8).reshape(nb, 2)
    return W, 2 * smax * 95


def exact_acts(M, K, seed, dtype="f32", amp=3):
    """x = s * q per 32-block: s in {1, 2}, q integers in [-amp, amp] with one
    +-127 at a random position, so q8_1 gives d = s and quants q exactly."""
    r = inputs.rng(seed)
    nb = K // 32
    q = r.integers(-amp, amp + 1, (M, nb, 32)).astype(np.float32)
    pos = r.integers(0, 32, (M, nb))
    sgn = r.choice(np.array([-127.0, 127.0], np.float32), (M, nb))
    np.put_along_axis(q, pos[..., None], sgn[..., None], axis=2)
    s = r.choice(np.array([1.0, 2.0], np.float32), (M, nb, 1))
    x = (q * s).reshape(M, K).astype(np.float32)
    if dtype == "bf16":
        return inputs.to_bf16_bits(x)           # integers up to 254: exact in bf16
    if dtype == "f16":
        return x.astype(np.float16)
    return x


def act_abs_sum(x):
    """sum_k |x[m, k]| per row, from float values (bf16 bits decoded by shifting)."""
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return np.abs(x.astype(np.float64)).sum(axis=1)


def assert_exact_range(wmax, x, extra=1.0):
    """Every partial sum is bounded by wmax * sum|x| (times route weights): below 2^24."""
    b = float(act_abs_sum(x).max()) * wmax * extra
    assert b < EXACT, f"construction not exact in fp32: bound {b:.3g}"


def same_bits(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.astype(np.float32).view(np.uint32)
    bad = np.flatnonzero(a.ravel() != b.ravel())
    assert bad.size == 0, f"{bad.size} of {a.size} outputs differ, first at {np.unravel_index(bad[0], a.shape)}"


def gpu_bits(y):
    """Output tensor as fp32 values or bf16 bit patterns (uint16)."""
    if y.dtype == torch.bfloat16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy()


def oracle_bits(y32, kind):
    return y32 if kind == "f32" else oracle.fp32_to_bf16_array(y32)


def _dense(dev, wt, N, K, M, path, seed, ydt="f32", xdt="f32", rows=None, smax=6, W=None, wmax=None, ldx=None):
    if W is None:
        W, wmax = exact_weights(wt, N, K, seed, smax)
    x = exact_acts(M, K, seed + 1, xdt)
    assert_exact_range(wmax, x)
    xt = T(x, dev)
    if ldx is not None:                      # activation rows ldx elements apart
        buf = torch.zeros((M, ldx), dtype=xt.dtype, device=dev)
        buf[:, :K] = xt
        xt = buf[:, :K]
    y = g.mul_mat(T(W, dev), wt, xt, out_dtype=torch.float32 if ydt == "f32" else torch.bfloat16, path=path)
    got = gpu_bits(y)
    if rows is not None:
        got = got[:, rows]
    want = oracle_bits(oracle.mul_mat(wt, W, N, K, x, rows=rows), ydt)
    same_bits(got, want)
    log(f"exact dense type={wt} N={N} K={K} M={M} path={path} {xdt}->{ydt}: bit-exact")


# ------------------------------------------------------------------ MMVQ

@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 13, 16])
def test_exact_mmvq(dev, wt, M):
    """Every column-group width (1, 2, 4, 8 and ragged groups), ragged row count;
    13 and 16 rows: two column groups, as AUTO runs them up to 16 rows."""
    K = 512 if wt in (g.Q8_0, g.Q4_0, g.Q6_K) else 1024
    _dense(dev, wt, 301, K, M, "mmvq", 1100 + 10 * wt + M)


@pytest.mark.parametrize("wt,N,K,M", [
    (g.Q4_K, 262147, 512, 1), (g.Q4_K, 262147, 512, 2), (g.Q6_K, 400001, 256, 1),
    (g.Q8_0, 2000001, 32, 1), (g.Q5_K, 200001, 1024, 1), (g.Q4_0, 300001, 512, 2),
])
def test_exact_mmvq_deep(dev, wt, N, K, M):
    """Long matrices: the instantiation with two work items in flight per wave."""
    _dense(dev, wt, N, K, M, "mmvq", 1200 + wt + M)


@pytest.mark.parametrize("wt", [g.Q4_K, g.Q6_K, g.Q8_0])
@pytest.mark.parametrize("xdt,pad", [("bf16", 8), ("bf16", 3), ("f32", 1), ("f16", 0)])
def test_exact_mmvq_activation_forms(dev, wt, xdt, pad):
    """Activation rows copied by DMA (16-byte strides) and read directly (odd
    strides), from fp32, bf16 and fp16; bf16 output too."""
    K = 512
    _dense(dev, wt, 200, K, 4, "mmvq", 1300 + wt, xdt=xdt, ldx=K + pad)
    _dense(dev, wt, 200, K, 1, "mmvq", 1310 + wt, xdt=xdt, ydt="bf16", ldx=K + pad)


def test_exact_c2_decode_full_size(dev):
    """The 4096 x 4096 Q4_K decode shape at M = 1..8 (the benchmark's launch
    configuration), fp32 and bf16 outputs."""
    W, wmax = exact_weights(g.Q4_K, 4096, 4096, 1400, smax=4)
    for M in (1, 2, 4, 8):
        _dense(dev, g.Q4_K, 4096, 4096, M, "auto", 1401 + M, W=W, wmax=wmax)
    _dense(dev, g.Q4_K, 4096, 4096, 1, "auto", 1410, ydt="bf16", xdt="bf16", W=W, wmax=wmax)


def test_exact_c4_lm_head_m1_full_size(dev):
    """The 248320 x 2048 Q6_K lm_head at M = 1, all rows, fp32 logits."""
    W, wmax = exact_weights(g.Q6_K, 248320, 2048, 1420, smax=3)
    _dense(dev, g.Q6_K, 248320, 2048, 1, "auto", 1421, xdt="bf16", W=W, wmax=wmax)


# ------------------------------------------------------------------ MMQ

@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("M,N,K", [(40, 100, 512), (129, 257, 768), (300, 130, 1024)])
def test_exact_mmq(dev, wt, M, N, K):
    """Ragged tiles in both dimensions, several super-blocks."""
    smax = 4 if wt in (g.Q6_K, g.Q5_K) else 6
    _dense(dev, wt, N, K, M, "mmq", 1500 + wt + M, smax=smax)
    _dense(dev, wt, N, K, M, "mmq", 1550 + wt + M, smax=smax, ydt="bf16", xdt="bf16")


@pytest.mark.parametrize("wt", TYPES)
def test_exact_mmq_split_k(dev, wt):
    """Few tiles and a long K: K split over workgroups, partials summed in order."""
    _dense(dev, wt, 200, 2048, 70, "mmq", 1600 + wt, smax=2)


def test_exact_c3_prefill_sampled(dev):
    """The 8192 x 2048 Q4_K prefill at M = 8192 (the benchmark's launch
    configuration) on 128 sampled weight rows, and the M = 16..64 sweep on
    both paths on every row."""
    W, wmax = exact_weights(g.Q4_K, 8192, 2048, 1700, smax=6)
    rows = inputs.sample_rows(8192, 128, 1701)
    _dense(dev, g.Q4_K, 8192, 2048, 8192, "auto", 1702, ydt="bf16", xdt="bf16", rows=rows, W=W, wmax=wmax)
    for M in (16, 24, 32, 64):
        for path in ("mmvq", "mmq"):
            _dense(dev, g.Q4_K, 8192, 2048, M, path, 1710 + M, W=W, wmax=wmax)


def test_exact_c4_lm_head_m2048_sampled(dev):
    """The 248320 x 2048 Q6_K lm_head at M = 2048 on 256 sampled rows."""
    W, wmax = exact_weights(g.Q6_K, 248320, 2048, 1720, smax=2)
    rows = inputs.sample_rows(248320, 256, 1721)
    _dense(dev, g.Q6_K, 248320, 2048, 2048, "auto", 1722, xdt="bf16", rows=rows, W=W, wmax=wmax)


# ------------------------------------------------------------------ routed

def _moe(dev, wt, E, N, K, Tn, top_k, path, seed, weighted=False, x_per_route=False, hot=False, smax=4):
    W, wmax = exact_weights(wt, E * N, K, seed, smax)
    W = W.reshape(E, N, -1)
    rows = Tn * top_k if x_per_route else Tn
    x = exact_acts(rows, K, seed + 1)
    r = inputs.rng(seed + 2)
    ids = r.integers(0, E, (Tn, top_k)).astype(np.int32)
    if hot:
        ids[r.random((Tn, top_k)) < 0.4] = 1
    ids[0] = 2                                              # one expert four times in a token
    ids[1, 0] = -1
    ids[min(2, Tn - 1), top_k - 1] = E + 5                  # >= E: skipped
    w = r.choice(np.array([1.0, 2.0], np.float32), (Tn, top_k)) if weighted else None
    assert_exact_range(wmax, x, extra=(2.0 * top_k if weighted else 1.0))
    xin = x.reshape(Tn, top_k, K) if x_per_route else x
    y = g.mul_mat_id(T(W, dev), wt, T(xin, dev), T(ids, dev), K, route_w=None if w is None else T(w, dev),
                     x_per_route=x_per_route, out_dtype=torch.float32, path=path)
    want = oracle.mul_mat_id(wt, W, E, N, K, W.shape[1] * W.shape[2], xin, Tn, int(x_per_route), ids, top_k,
                             route_w=w)
    same_bits(y.cpu().numpy(), want)
    log(f"exact routed type={wt} E={E} N={N} K={K} T={Tn} top_k={top_k} path={path} weighted={weighted}: bit-exact")


@pytest.mark.parametrize("wt", TYPES)
@pytest.mark.parametrize("path", ["mmvq", "mmq"])
def test_exact_routed(dev, wt, path):
    K = 512
    _moe(dev, wt, 9, 96, K, 37, 4, path, 1800 + wt)
    _moe(dev, wt, 9, 160, 256, 29, 4, path, 1850 + wt, weighted=True, x_per_route=True, smax=2)


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
def test_exact_routed_many_routes(dev, path):
    """Over 16K routes (the multi-workgroup route build) with a hot expert."""
    _moe(dev, g.Q4_K, 9, 64, 256, 5000, 4, path, 1900, hot=True)


def test_exact_routed_decode_deep(dev):
    """Routed decode over many experts with long expert matrices: each wave
    walks several items and keeps two in flight."""
    _moe(dev, g.Q4_K, 128, 4096, 512, 16, 8, "mmvq", 1910)
    _moe(dev, g.Q6_K, 64, 2048, 512, 16, 8, "mmvq", 1920, weighted=True, x_per_route=True, smax=1)


# ------------------------------------------------------------------ ties of the q8_1 rounding

def tie_matrix(M, K, seed):
    """fp32 rows whose 32-blocks hold exact ties (x / d = k + 1/2 exactly) and
    near ties (x / d one or two units from k + 1/2), with d = 1, 2^j, 3 and
    inexact d = amax / 127, plus zero, tiny and huge blocks."""
    r = inputs.rng(seed)
    x = np.zeros((M, K), np.float32)
    for m in range(M):
        for b in range(K // 32):
            kind = (m * (K // 32) + b) % 8
            k = r.integers(0, 127, 31).astype(np.float32)
            sg = r.choice(np.array([-1.0, 1.0], np.float32), 31)
            blk = np.zeros(32, np.float32)
            if kind == 0:                                   # d = 1: half-integers
                blk[1:] = sg * (k + np.float32(0.5))
                blk[0] = 127
            elif kind == 1:                                 # d = 2^j
                j = np.float32(2.0) ** r.integers(-6, 7)
                blk[1:] = sg * (k + np.float32(0.5)) * j
                blk[0] = -127 * j
            elif kind == 2:                                 # d = 3: ties after an inexact reciprocal
                kk = r.integers(0, 126, 31).astype(np.float32)
                blk[1:] = sg * np.float32(3) * (kk + np.float32(0.5))
                blk[0] = 381
            elif kind == 3:                                 # inexact d: values at, just above and just below k + 1/2
                amax = np.float32(r.uniform(0.5, 200.0))
                d = np.float32(amax / np.float32(127))
                v = ((k + np.float32(0.5)) * d).astype(np.float32)
                for i, st in enumerate(r.integers(-2, 3, 31)):
                    for _ in range(abs(int(st))):
                        v[i] = np.nextafter(v[i], np.float32(np.inf if st > 0 else -np.inf))
                blk[1:] = sg * v                            # |v| < amax: k <= 126
                blk[0] = amax
            elif kind == 4:                                 # all zero
                pass
            elif kind == 5:                                 # tiny values
                blk[:] = np.float32(1e-30) * (np.arange(32, dtype=np.float32) - 15.5)
            elif kind == 6:                                 # huge values (their dots stay finite in fp32)
                blk[:] = np.float32(1e30) * np.sin(np.arange(32, dtype=np.float32) + m)
            else:                                           # d = 1 with 127 at the end, ties near +-0.5
                blk[:31] = sg * (np.float32(0.5) + (k % 3))
                blk[31] = -127
            x[m, 32 * b:32 * b + 32] = r.permutation(blk)
    return x


def _as(x, kind):
    if kind == "bf16":
        return inputs.to_bf16_bits(x)
    if kind == "f16":
        return np.clip(x, -60000, 60000).astype(np.float16)
    return x


@pytest.mark.parametrize("kind", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("K,pad", [(256, 0), (256, 8), (96, 1), (128, 4), (64, 2)])
def test_ties_standalone_quantizers(dev, kind, K, pad):
    """The standalone kernels on tie blocks: 2 lanes per block (16-element
    aligned rows), 4 lanes (8-element), the 8-lane kernel with vector and
    scalar loads (other strides)."""
    M = 12
    x = _as(tie_matrix(M, K + pad, 2000 + K + pad), kind)
    xt = T(x, dev)[:, :K]
    got = g.quantize_q8_1(xt).cpu().numpy()
    want = oracle.quantize_q8_1(np.ascontiguousarray(x[:, :K]))
    same_bits(got, want)


@pytest.mark.parametrize("kind", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,pad", [(1, 0), (2, 0), (4, 8), (8, 0), (3, 1)])
def test_ties_mmvq_prologue(dev, kind, M, pad):
    """The quantizer inside the MMVQ prologue: float tie rows in give the same
    output bits as the oracle's q8_1 blocks of those rows in (the dots after
    the prologue are the same code, so any differing quant shows)."""
    K, N = 512, 160
    W = inputs.gen_q8_0(N, K, 2100)
    W.reshape(-1, 34)[:, 0:2] = np.array([F16_ONE], np.uint16).view(np.uint8)
    xf = _as(tie_matrix(M, K + pad, 2101 + M), kind)
    xt = T(xf, dev)[:, :K]
    x = np.ascontiguousarray(xf[:, :K])
    q8 = oracle.quantize_q8_1(x)
    a = g.mul_mat(T(W, dev), g.Q8_0, xt, out_dtype=torch.float32, path="mmvq").cpu().numpy()
    b = g.mul_mat(T(W, dev), g.Q8_0, T(q8, dev), K=K, path="mmvq").cpu().numpy()
    same_bits(a, b)


@pytest.mark.parametrize("kind", ["f32", "bf16", "f16"])
def test_ties_mmq_operand(dev, kind):
    """The quantizer that writes MMQ's operand: float tie rows in equal the
    oracle's q8_1 blocks of those rows in, bit for bit."""
    K, N, M = 512, 96, 40
    W = inputs.gen_q8_0(N, K, 2200)
    xf = _as(tie_matrix(M, K, 2201), kind)
    q8 = oracle.quantize_q8_1(xf)
    a = g.mul_mat(T(W, dev), g.Q8_0, T(xf, dev), out_dtype=torch.float32, path="mmq").cpu().numpy()
    b = g.mul_mat(T(W, dev), g.Q8_0, T(q8, dev), K=K, path="mmq").cpu().numpy()
    same_bits(a, b)


def tie_output_case(N, K, E, seed):
    """Q8_0 experts (d = 1) and activations whose products are exact integers
    arranged so that each route's 32-output q8_1 blocks hold exact ties: one
    output of 254 (so the block's d = 2) and odd integers elsewhere (so each
    x / d is k + 1/2), or 127 and a mix (d = 1, no ties)."""
    r = inputs.rng(seed)
    W = inputs.gen_q8_0(E * N, K, seed + 1).reshape(-1, 34)
    W[:, 0:2] = np.array([F16_ONE], np.uint16).view(np.uint8)
    q = W[:, 2:].view(np.int8).reshape(E, N, K // 32, 32)
    q[:, :, 0, 0] = 0
    q[:, :, 0, 1] = (2 * r.integers(-63, 63, (E, N)) + 1).astype(np.int8)   # odd
    lead = np.arange(N) % 32 == 0
    q[:, lead, 0, 0] = 2
    q[:, lead, 0, 1] = 0
    q[1, lead, 0, 0] = 1                                                   # expert 1: d = 1 blocks
    q[1, lead, 0, 1] = 0
    x = np.zeros(K, np.float32)
    x[0], x[1] = 127, 1
    return W.reshape(E, N, -1), x


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_ties_routed_q8_1_output(dev, path, kind):
    """Routed q8_1 output (quantized in the MMQ epilogue, or staged and
    quantized after MMVQ) on outputs built to be exact ties: the blocks equal
    the oracle's q8_1 of the oracle's (exact) plain output."""
    E, N, K, Tn, top_k = 3, 96, 256, 40, 2
    W, x1 = tie_output_case(N, K, E, 2300)
    xs = np.tile(x1, (Tn, 1))
    xs[::3] *= -1                                                           # negative ties too
    ids = inputs.rng(2301).integers(0, E, (Tn, top_k)).astype(np.int32)
    ids[0, 1] = -1
    xin = _as(xs, kind)
    q = g.mul_mat_id(T(W, dev), g.Q8_0, T(xin, dev), T(ids, dev), K, out_dtype="q8_1", path=path)
    plain = oracle.mul_mat_id(g.Q8_0, W, E, N, K, W.shape[1] * W.shape[2], xin, Tn, 0, ids, top_k)
    R = Tn * top_k
    src = plain.reshape(R, N) if kind == "f32" else oracle.fp32_to_bf16_array(plain.reshape(R, N))
    same_bits(q.cpu().numpy().reshape(R, -1), oracle.quantize_q8_1(src))
