"""The boundary's safety claims under test (ggq.h: kernels never read past the
last weight row of a matrix or expert, offsets are 64-bit, nothing is written
past y or the workspace).

- Weight bytes right after the last row, and between experts when
  expert_stride > N * row_bytes, are garbage blocks whose scales are NaN: a
  kernel that reads one leaks NaN into its outputs (NaN * 0 is NaN), the
  failure the pages report for MMQ without tail padding (FreeToken PR #690,
  the offload slot-cache tail-padding comment and "64ef88f - NaN after
  prefill with offload").
- A dense matrix and a routed bank larger than 4 GiB, checked on sampled rows
  against the oracle: a 32-bit byte offset would wrap onto other rows
  (FreeToken issue #671, "Known issues").
- Canary bytes after y and after the workspace must be unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
import gguf_block_quantized_q8_amd as g
from gguf_block_quantized_q8_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 8e-3}
# bytes of one block and the byte offsets of its fp16 scale fields
BLOCK = {g.Q4_0: (18, (0,)), g.Q8_0: (34, (0,)), g.Q4_K: (144, (0, 2)), g.Q5_K: (176, (0, 2)), g.Q6_K: (210, (208,))}
CANARY = 0xA5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def log(*a):
    print(*a, flush=True)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


def nan_blocks(wt, nbytes, seed):
    """nbytes of garbage laid out as whole blocks of type wt (the tail of the last
    one cut), random bytes with every scale field set to fp16 NaN (0x7e00)."""
    bb, fields = BLOCK[wt]
    n = (nbytes + bb - 1) // bb
    a = inputs.rng(seed).integers(0, 256, (n, bb), dtype=np.uint8)
    for f in fields:
        a[:, f] = 0x00
        a[:, f + 1] = 0x7e
    return a.reshape(-1)[:nbytes]


def bf16_host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dev_bf16(a, dev):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)


def vp(t, offset=0):
    import ctypes
    return ctypes.c_void_p(t.data_ptr() + offset)


def stream():
    import ctypes
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def check_rc(rc, what):
    assert rc == g.OK, f"{what}: {g.lib().ggq_last_error().decode()}"


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
@pytest.mark.parametrize("wt", [g.Q4_K, g.Q6_K, g.Q8_0, g.Q4_0, g.Q5_K])
def test_dense_nan_blocks_after_last_row_and_canaries(dev, wt, path):
    N, K = 1000, 512                                     # N not a multiple of the 128-row tile
    M = 5 if path == "mmvq" else 300                     # MMQ: a ragged second 256-column tile
    W = inputs.gen_weights(wt, N, K, 700 + wt)
    rb = g.row_bytes(wt, K)
    tail = 64 * 1024
    buf = torch.from_numpy(np.concatenate([W.reshape(-1), nan_blocks(wt, tail, 701 + wt)])).to(dev)
    x = inputs.gen_act(M, K, 702, "bf16")
    xd = dev_bf16(x, dev)
    L = g.lib()
    p = g._PATHS[path]
    wsb = L.ggq_mul_mat_ws(wt, N, K, g.BF16, M, p)
    ws = torch.full((wsb + 4096,), CANARY, dtype=torch.uint8, device=dev)
    ybuf = torch.full((M * N * 2 + 4096,), CANARY, dtype=torch.uint8, device=dev)
    rc = L.ggq_mul_mat(wt, vp(buf), N, K, vp(xd), g.BF16, M, K, vp(ybuf), g.BF16, N, vp(ws), wsb, p, stream())
    check_rc(rc, "mul_mat")
    torch.cuda.synchronize()
    y = ybuf[:M * N * 2].view(torch.bfloat16).view(M, N)
    assert torch.isfinite(y.float()).all(), "NaN or inf in the output: garbage past the last row was read"
    r = rel(y.float().cpu().numpy(), oracle.mul_mat(wt, W, N, K, x))
    assert (ybuf[M * N * 2:] == CANARY).all(), "bytes written after y"
    assert (ws[wsb:] == CANARY).all(), "bytes written after the workspace"
    log(f"dense NaN tail type={wt} path={path} ws={wsb}: rel {r:.3g}, canaries intact")
    assert r <= TOL["bf16"]


@pytest.mark.parametrize("path", ["mmvq", "mmq"])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("wt", [g.Q4_K, g.Q6_K])
def test_routed_nan_padding_between_experts_and_canaries(dev, wt, path, weighted):
    E, N, K, Tn, top_k = 5, 192, 512, (6 if path == "mmvq" else 200), 3
    rb = g.row_bytes(wt, K)
    stride = N * rb + 16 * 211                           # padding between experts, a multiple of 16
    Wc = inputs.gen_experts(wt, E, N, K, 710 + wt)       # compact [E, N, rb]
    host = nan_blocks(wt, E * stride + 64 * 1024, 711 + wt).copy()
    for e in range(E):
        host[e * stride:e * stride + N * rb] = Wc[e].reshape(-1)
    buf = torch.from_numpy(host).to(dev)
    x = inputs.gen_act(Tn, K, 712, "bf16")
    ids, w = inputs.gen_routing(Tn, E, top_k, 713)
    ids[0, 0] = -1
    ids[1, 1] = E + 3                                    # >= E: skipped
    L = g.lib()
    p = g._PATHS[path]
    wsb = L.ggq_mul_mat_id_ws(wt, E, N, K, g.BF16, Tn, 0, top_k, g.EPI_NONE, int(weighted), p)
    ws = torch.full((wsb + 4096,), CANARY, dtype=torch.uint8, device=dev)
    ny = (Tn * N if weighted else Tn * top_k * N) * 2
    ybuf = torch.full((ny + 4096,), CANARY, dtype=torch.uint8, device=dev)
    xd = dev_bf16(x, dev)
    ids_d = torch.from_numpy(ids).to(dev)
    w_d = torch.from_numpy(w).to(dev) if weighted else None
    rc = L.ggq_mul_mat_id(wt, vp(buf), E, N, K, stride, vp(xd), g.BF16, Tn, 0, vp(ids_d), top_k,
                          vp(w_d) if weighted else None, g.EPI_NONE, vp(ybuf), g.BF16, vp(ws), wsb, p, stream())
    check_rc(rc, "mul_mat_id")
    torch.cuda.synchronize()
    y = ybuf[:ny].view(torch.bfloat16).float().cpu().numpy()
    assert np.isfinite(y).all(), "NaN or inf in the output: padding between experts was read"
    want = oracle.mul_mat_id(wt, Wc, E, N, K, N * rb, x, Tn, 0, ids, top_k, route_w=w if weighted else None,
                             route_round="bf16" if weighted else None)
    r = rel(y.reshape(want.shape), want)
    assert (ybuf[ny:] == CANARY).all(), "bytes written after y"
    assert (ws[wsb:] == CANARY).all(), "bytes written after the workspace"
    log(f"routed NaN padding type={wt} path={path} weighted={weighted}: rel {r:.3g}, canaries intact")
    assert r <= TOL["bf16"]


def _fill_repeating(Wd, base):
    """Fill device rows Wd [N, rb] with the rows of base [B, rb] repeated."""
    N, B = Wd.shape[0], base.shape[0]
    full = N // B
    Wd[:full * B].view(full, B, -1).copy_(base.unsqueeze(0).expand(full, B, base.shape[1]))
    Wd[full * B:].copy_(base[:N - full * B])


@pytest.mark.parametrize("path,M", [("mmvq", 1), ("mmq", 64)])
def test_dense_weight_over_4_gib(dev, path, M):
    wt, K = g.Q4_K, 4096
    rb = g.row_bytes(wt, K)                              # 2304
    N = (4 << 30) // rb + 4096                           # 4.3 GB of weights
    B = 4099                                             # base rows, repeated (not a divisor of the wrap)
    base = torch.from_numpy(inputs.gen_q4_K(B, K, 720)).to(dev)
    Wd = torch.empty((N, rb), dtype=torch.uint8, device=dev)
    _fill_repeating(Wd, base)
    # distinct rows around the 4 GiB byte boundary and at the end: a wrapped 32-bit
    # offset would read a repeated base row instead
    edge = (4 << 30) // rb
    special = np.unique(np.concatenate([np.arange(edge - 3, edge + 4), np.arange(N - 64, N)]))
    uniq = inputs.gen_q4_K(len(special), K, 721)
    Wd[torch.from_numpy(special).to(dev)] = torch.from_numpy(uniq).to(dev)
    sample = np.unique(np.concatenate([np.arange(4), special, inputs.sample_rows(N, 32, 722)]))
    Ws = Wd[torch.from_numpy(sample).to(dev)].cpu().numpy()
    x = inputs.gen_act(M, K, 723, "f32")
    log(f"dense > 4 GiB: N={N} ({N * rb / 2**30:.2f} GiB), path={path}, M={M}, {len(sample)} sampled rows")
    y = g.mul_mat(Wd, wt, torch.from_numpy(x).to(dev), out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    got = y[:, torch.from_numpy(sample).to(dev)].cpu().numpy()
    want = oracle.mul_mat(wt, Ws, len(sample), K, x)
    r = rel(got, want)
    log(f"dense > 4 GiB path={path}: rel {r:.3g}")
    del Wd, y, base
    torch.cuda.empty_cache()
    assert r <= TOL["f32"]


@pytest.mark.parametrize("path,Tn", [("mmvq", 8), ("mmq", 300)])
def test_routed_bank_over_4_gib(dev, path, Tn):
    wt, E, N, K, top_k = g.Q4_K, 3, 256, 1024, 2
    rb = g.row_bytes(wt, K)
    stride = (2 << 30) + 4096                            # E * stride = 6.4 GB; expert 2 starts past 4 GiB
    Wc = inputs.gen_experts(wt, E, N, K, 730)
    buf = torch.empty(E * stride, dtype=torch.uint8, device=dev)
    pad = torch.from_numpy(nan_blocks(wt, 1 << 20, 731)).to(dev)
    for e in range(E):                                   # rows, then NaN garbage in the first MB of padding
        o = e * stride
        buf[o:o + N * rb] = torch.from_numpy(Wc[e].reshape(-1)).to(dev)
        buf[o + N * rb:o + N * rb + pad.numel()] = pad
    W = torch.as_strided(buf, (E, N, rb), (stride, rb, 1))
    x = inputs.gen_act(Tn, K, 732, "f32")
    ids = inputs.rng(733).integers(0, E, (Tn, top_k)).astype(np.int32)
    ids[:, 0] = 2                                        # every token uses the expert past 4 GiB
    w = inputs.rng(734).uniform(0.1, 1.0, (Tn, top_k)).astype(np.float32)
    xd, ids_d, w_d = torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
    log(f"routed bank > 4 GiB: E*stride={E * stride / 2**30:.2f} GiB, path={path}, T={Tn}")
    y = g.mul_mat_id(W, wt, xd, ids_d, K, out_dtype=torch.float32, path=path)
    yw = g.mul_mat_id(W, wt, xd, ids_d, K, route_w=w_d, out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    want = oracle.mul_mat_id(wt, Wc, E, N, K, N * rb, x, Tn, 0, ids, top_k)
    want_w = oracle.mul_mat_id(wt, Wc, E, N, K, N * rb, x, Tn, 0, ids, top_k, route_w=w)
    r, rw = rel(y.cpu().numpy(), want), rel(yw.cpu().numpy(), want_w)
    log(f"routed bank > 4 GiB path={path}: rel {r:.3g}, weighted {rw:.3g}")
    del buf, W
    torch.cuda.empty_cache()
    assert r <= TOL["f32"] and rw <= TOL["f32"]
