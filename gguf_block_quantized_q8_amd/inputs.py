"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random data and lays it out in the GGUF byte formats;
it holds none of the method's arithmetic (no quantization, no dot products,
no dequantization).  Both the GPU path and the CPU oracle consume what it
produces.

Distributions (one numpy PCG64 stream per seed):
  * Q8_0 blocks: fp16 d ~ U(1e-3, 2e-2) (drawn in fp32, rounded to fp16),
    32 int8 quants uniform in [-127, 127].
  * Q4_K super-blocks: fp16 d, dmin ~ U(1e-3, 2e-2); the 12 packed scale
    bytes and the 128 quant bytes are uniform random bytes, which makes
    every 6-bit scale/min and every nibble uniform.
  * Q6_K super-blocks: ql and qh uniform random bytes, the 16 int8 scales
    uniform in [-64, 63], fp16 d ~ U(1e-4, 5e-3).
  * Q4_0 blocks: fp16 d ~ U(1e-3, 2e-2), 16 uniform random quant bytes.
  * Q5_K super-blocks: as Q4_K, plus 32 uniform random bytes of fifth bits.
  * Activations: fp32 N(0, 1); bf16 activations are those fp32 values
    rounded to bf16 by torch (returned as uint16 bit patterns); fp16
    activations are them rounded to float16 by numpy.
  * Routing: router logits fp32 N(0, 1) [T, E] -> softmax in fp64 -> fp32
    probabilities; top-k by probability, ties to the lower expert id; the
    route weights are the top-k probabilities, not renormalized.

Block byte layouts follow the public GGUF format:
  Q8_0 (34 B / 32): fp16 d | 32 x int8
  Q4_K (144 B / 256): fp16 d | fp16 dmin | 12 B scales | 128 B quants
  Q6_K (210 B / 256): 128 B ql | 64 B qh | 16 x int8 scales | fp16 d
  Q4_0 (18 B / 32): fp16 d | 16 B quants
  Q5_K (176 B / 256): fp16 d | fp16 dmin | 12 B scales | 32 B fifth bits | 128 B quants
"""
import numpy as np

Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 2, 8, 12, 13, 14
BLOCK = {Q4_0: (32, 18), Q8_0: (32, 34), Q4_K: (256, 144), Q5_K: (256, 176), Q6_K: (256, 210)}
NAMES = {Q4_0: "Q4_0", Q8_0: "Q8_0", Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K"}


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def row_bytes(t, K):
    qk, bb = BLOCK[t]
    assert K % qk == 0
    return K // qk * bb


def _fp16_bits(r, lo, hi, n):
    return r.uniform(lo, hi, n).astype(np.float32).astype(np.float16).view(np.uint16)


def gen_q8_0(N, K, seed, dlo=1e-3, dhi=2e-2):
    r = rng(seed)
    nb = N * K // 32
    blk = np.zeros((nb, 34), dtype=np.uint8)
    blk[:, 0:2] = _fp16_bits(r, dlo, dhi, nb).view(np.uint8).reshape(nb, 2)
    blk[:, 2:34] = r.integers(-127, 128, size=(nb, 32), dtype=np.int8).view(np.uint8)
    return blk.reshape(N, row_bytes(Q8_0, K))


def gen_q4_K(N, K, seed, dlo=1e-3, dhi=2e-2):
    r = rng(seed)
    nb = N * K // 256
    blk = np.zeros((nb, 144), dtype=np.uint8)
    blk[:, 0:2] = _fp16_bits(r, dlo, dhi, nb).view(np.uint8).reshape(nb, 2)
    blk[:, 2:4] = _fp16_bits(r, dlo, dhi, nb).view(np.uint8).reshape(nb, 2)
    blk[:, 4:144] = r.integers(0, 256, size=(nb, 140), dtype=np.uint8)
    return blk.reshape(N, row_bytes(Q4_K, K))


def gen_q6_K(N, K, seed, dlo=1e-4, dhi=5e-3):
    r = rng(seed)
    nb = N * K // 256
    blk = np.zeros((nb, 210), dtype=np.uint8)
    blk[:, 0:192] = r.integers(0, 256, size=(nb, 192), dtype=np.uint8)
    blk[:, 192:208] = r.integers(-64, 64, size=(nb, 16), dtype=np.int8).view(np.uint8)
    blk[:, 208:210] = _fp16_bits(r, dlo, dhi, nb).view(np.uint8).reshape(nb, 2)
    return blk.reshape(N, row_bytes(Q6_K, K))


def gen_q4_0(N, K, seed, dlo=1e-3, dhi=2e-2):
    r = rng(seed)
    nb = N * K // 32
    blk = np.zeros((nb, 18), dtype=np.uint8)
    blk[:, 0:2] = _fp16_bits(r, dlo, dhi, nb).view(np.uint8).reshape(nb, 2)
    blk[:, 2:18] = r.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    return blk.reshape(N, row_bytes(Q4_0, K))


def gen_q5_K(N, K, seed, dlo=1e-3, dhi=2e-2):
    r = rng(seed)
    nb = N * K // 256
    blk = np.zeros((nb, 176), dtype=np.uint8)
    blk[:, 0:2] = _fp16_bits(r, dlo, dhi, nb).view(np.uint8).reshape(nb, 2)
    blk[:, 2:4] = _fp16_bits(r, dlo, dhi, nb).view(np.uint8).reshape(nb, 2)
    blk[:, 4:176] = r.integers(0, 256, size=(nb, 172), dtype=np.uint8)
    return blk.reshape(N, row_bytes(Q5_K, K))


def gen_weights(t, N, K, seed):
    return {Q4_0: gen_q4_0, Q8_0: gen_q8_0, Q4_K: gen_q4_K, Q5_K: gen_q5_K, Q6_K: gen_q6_K}[t](N, K, seed)


def gen_experts(t, E, N, K, seed):
    """Expert bank [E, N, row_bytes] as one contiguous uint8 array."""
    return gen_weights(t, E * N, K, seed).reshape(E, N, row_bytes(t, K))


def to_bf16_bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gen_act(M, K, seed, dtype="f32"):
    """Activations N(0,1): float32 [M, K], bf16 bit patterns uint16 [M, K], or float16 [M, K]
    (numpy's round-to-nearest-even conversion)."""
    x = rng(seed).standard_normal((M, K), dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    return x if dtype == "f32" else to_bf16_bits(x)


def gen_routing(T, E, top_k, seed):
    """ids int32 [T, top_k], weights float32 [T, top_k] from softmax(N(0,1) logits)."""
    logits = rng(seed).standard_normal((T, E), dtype=np.float32).astype(np.float64)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    p32 = p.astype(np.float32)
    order = np.argsort(-p32, axis=1, kind="stable")[:, :top_k]   # ties -> lower id
    ids = order.astype(np.int32)
    w = np.take_along_axis(p32, order, axis=1).astype(np.float32)
    return ids, w


def gen_routing_skewed(T, E, top_k, seed, hot=8, boost=2.5):
    """As gen_routing, with `boost` added to the logits of experts 0..hot-1 (a few
    experts draw most routes: about 60 % of them for hot=8, boost=2.5, E=256,
    top_k=8)."""
    logits = rng(seed).standard_normal((T, E), dtype=np.float32).astype(np.float64)
    logits[:, :hot] += boost
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    p32 = p.astype(np.float32)
    order = np.argsort(-p32, axis=1, kind="stable")[:, :top_k]
    return order.astype(np.int32), np.take_along_axis(p32, order, axis=1).astype(np.float32)


def sample_rows(N, count, seed):
    """Sorted distinct row indices: `count` seeded picks plus the first and last row."""
    picks = rng(seed).choice(N, size=min(count, N), replace=False)
    return np.unique(np.concatenate([picks, [0, N - 1]])).astype(np.int64)


# The five workloads (weights, activations and routing drawn as above).
CONFIGS = {
    "q8_0_256x512": dict(type=Q8_0, N=256, K=512, M=(1, 4), xdtype="f32", ydtype="f32", seeds=(101, 102)),
    "q4_K_4096x4096_decode": dict(type=Q4_K, N=4096, K=4096, M=(1, 2, 4, 8), xdtype="bf16", ydtype="bf16", seeds=(201, 202)),
    "q4_K_8192x2048_prefill": dict(type=Q4_K, N=8192, K=2048, M=(8192,), sweep=(16, 24, 32, 64), xdtype="bf16", ydtype="bf16", seeds=(301, 302)),
    "q6_K_248320x2048_lm_head": dict(type=Q6_K, N=248320, K=2048, M=(1, 2048), xdtype="bf16", ydtype="f32", seeds=(401, 402, 403)),
    "moe_e256_top8_h2048_i512": dict(E=256, top_k=8, H=2048, I=512, T=(16, 8192), gate_up=Q4_K, down=Q6_K,
                                     xdtype="bf16", ydtype="bf16", seeds=(501, 502, 503, 504)),
}
