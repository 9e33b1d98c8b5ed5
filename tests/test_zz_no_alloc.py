"""ggq_mul_mat_id_noalloc against ggq_mul_mat_id: the same kernels, so the same bits.

Two calls in a row on each path, the second on a smaller input, so stale scratch
contents from the first call would show; then a call too large for the fixed scratch,
which must fail with a workspace error before launching anything."""
import numpy as np
import pytest
import torch

import gguf_block_quantized_q8_amd as g
from gguf_block_quantized_q8_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _t(a, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _bits(t):
    return t.contiguous().view(torch.uint8).cpu()


def _case(dev, wt, E, N, K, Tn, top_k, seed, weighted, epi, out_dtype, path, xdt="bf16"):
    W = _t(inputs.gen_experts(wt, E, N, K, seed), dev)
    x = _t(inputs.gen_act(Tn, K, seed + 1, xdt), dev)
    ids, w = inputs.gen_routing(Tn, E, top_k, seed + 2)
    ids_t, w_t = _t(ids, dev), (_t(w, dev) if weighted else None)
    ref = g.mul_mat_id(W, wt, x, ids_t, K, route_w=w_t, epi=epi, out_dtype=out_dtype, path=path)
    got = g.mul_mat_id_noalloc(W, wt, x, ids_t, K, route_w=w_t, epi=epi, out_dtype=out_dtype, path=path)
    torch.cuda.synchronize()
    print(f"noalloc wt={wt} E={E} N={N} K={K} T={Tn} top_k={top_k} path={path} weighted={weighted} "
          f"epi={epi} out={out_dtype}", flush=True)
    assert got.shape == ref.shape
    assert torch.equal(_bits(got), _bits(ref))


@pytest.mark.parametrize("path", ["mmq", "mmvq"])
def test_noalloc_matches_workspace_call_twice(dev, path):
    # weighted fp32 output, then a smaller unweighted bf16 output on the same scratch
    big_T = 300 if path == "mmq" else 12
    _case(dev, g.Q4_K, 8, 256, 512, big_T, 2, 11, True, g.EPI_NONE, torch.float32, path)
    _case(dev, g.Q4_K, 8, 256, 512, big_T // 4, 2, 21, False, g.EPI_NONE, torch.bfloat16, path)


def test_noalloc_swiglu_q8_1_then_smaller(dev):
    # gate/up with SwiGLU into q8_1 routes (MMQ), then a smaller routed call on MMVQ
    _case(dev, g.Q6_K, 4, 128, 256, 200, 2, 31, False, g.EPI_SWIGLU, "q8_1", "mmq")
    _case(dev, g.Q8_0, 4, 64, 256, 5, 2, 41, False, g.EPI_SWIGLU, "q8_1", "mmvq")


def test_noalloc_rejects_oversized_request(dev):
    # 8192 activation rows of K = 4096 on the MMQ path need about 80 MB of workspace
    E, N, K, Tn, top_k = 2, 32, 4096, 8192, 1
    need = g.lib().ggq_mul_mat_id_ws(g.Q4_K, E, N, K, g.BF16, Tn, 0, top_k, g.EPI_NONE, 0, g.PATH_MMQ)
    assert need > g.NOALLOC_SCRATCH_BYTES
    W = torch.zeros((E, N, g.row_bytes(g.Q4_K, K)), dtype=torch.uint8, device=dev)
    x = torch.zeros((Tn, K), dtype=torch.bfloat16, device=dev)
    ids = torch.zeros((Tn, top_k), dtype=torch.int32, device=dev)
    with pytest.raises(g.GgqError, match="fixed scratch"):
        g.mul_mat_id_noalloc(W, g.Q4_K, x, ids, K, out_dtype=torch.float32, path="mmq")
