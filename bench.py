"""Benchmark of the GGUF block-quantized matmul hot path on one MI355X.

Default (the headline): Q4_K 4096 x 4096 decode at M = 1 (bf16 activations
quantized to q8_1 on the fly, MMVQ, bf16 out).  One step = one full call
(q8_1 quantization + MMVQ) against the next of about 114 weight copies
(1 GiB), captured in one HIP graph so launch overhead on the host is not
timed.  Before each timed graph replay 1 GiB of an unrelated buffer is
streamed through the caches, so the timed steps read their weights from HBM
rather than the 256 MB last-level cache, whatever the step count.
value = algorithmic bytes per step x K / time (GB/s) of the first timed
region; step_us_median / p10 / p90 come from that region and the repeats.

The same JSON line carries, under "also", the other workloads of the
benchmark set, each timed the same way: Q4_K 4096x4096 at M = 2, 4, 8; the
Q4_K 8192 x 2048 prefill at M = 8192 (MMQ, TOPS) and its M = 16..64 sweep on
both paths; the Q6_K 248320 x 2048 lm_head at M = 1 (GB/s) and M = 2048
(TOPS); the E = 256, top-8 MoE layer (gate_up Q4_K + SwiGLU, down Q6_K +
route-weighted sum) at T = 16 and T = 8192.

roofline: the dominant kernel's algorithmic bytes (or int8 ops) per launch over
its launch duration from HIP events recorded on the launch stream (the source
is named in each object), against MI355X peaks (HBM 8 TB/s; dense int8 MFMA
5.0 POP/s).  cpu_baseline: the CPU oracle on the whole headline workload, on
all of this host's cores and on one thread.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gguf_block_quantized_q8_amd as g  # noqa: E402
from gguf_block_quantized_q8_amd import inputs  # noqa: E402

TNAME = {2: "Q4_0", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K"}
METRIC = "MMVQ GB/s @M=1 and MMQ/mul_mat_id TOPS @M=8192 (Q4_K,Q6_K), % of roofline"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
ROTATE_BYTES = 1 << 30
# HBM bytes per launch from rocprofv3 counter runs (2.0 x FETCH_SIZE + 1.0 x WRITE_SIZE,
# calibrated on a plain copy; profiles/hbm_counter_calibration_copy256MiB.md), keyed
# by kernel, with the hash of the kernel sources they were measured on: reported
# as null once those sources change.
PROFILE_TRAFFIC = {
    "mmvq_kernel<Q4_K,NC=1>": (9799948, "91c2d6acffd71e4b"),
    "mmvq_kernel<Q6_K,NC=1>": (419662083, "91c2d6acffd71e4b"),
    "mmq_kernel<Q4_K> 8192x2048 M=8192": (539850193, "c853d2e2da691aaf"),
    "dequant_rows_kernel<Q6_K> (get_rows)": (48517864, "00bc638143aba435"),
}
KERNEL_SOURCES = {"mmvq": ("mmvq.hip", "common.hpp", "kernels.hpp"),
                  "mmq": ("mmq.hip", "common.hpp", "kernels.hpp"),
                  "dequant": ("convert.hip", "common.hpp", "kernels.hpp")}


def source_hash(kind):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "gguf_block_quantized_q8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(kernel):
    rec = PROFILE_TRAFFIC.get(kernel)
    if rec is None:
        return None
    kind = kernel.split("_")[0]
    return rec[0] if kind in KERNEL_SOURCES and source_hash(kind) == rec[1] else None


def vp(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def bf16(a, dev):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)


def check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: {g.lib().ggq_last_error().decode()}")


class Ctx:
    def __init__(self, dev):
        self.dev = dev
        self.L = g.lib()
        self.stream = torch.cuda.current_stream(dev)
        self._flush = None
        self._sink = torch.zeros(4096, dtype=torch.uint8, device=dev)

    def evict(self):
        """Stream 1 GiB of an unrelated buffer through the caches (4x the
        256 MB last-level cache), so the next timed region reads its inputs from HBM."""
        if self._flush is None:
            self._flush = torch.ones(ROTATE_BYTES, dtype=torch.uint8, device=self.dev)
        check(self.L.ggq_bench_stream_read(vp(self._flush), ROTATE_BYTES, vp(self._sink), 4096, self.s), "evict")

    @property
    def s(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.dev).cuda_stream)


def time_steps(step, K, W, graph, evict=None, reps=5):
    """W untimed warmup steps, then exactly K timed steps (optionally as one HIP graph).

    Before every timed region `evict` (if given) streams 1 GiB through the
    caches, so the steps' inputs come from HBM, whatever K is: the untimed
    replay just before has read the same buffers.  The first timed region is
    the measurement; `reps` - 1 more (each after an eviction) give the spread.

    Returns (wall seconds from perf_counter between two synchronizations, GPU
    seconds between HIP events recorded on the launch stream around the timed
    region, list of per-step GPU seconds of every timed region)."""
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    gr = None
    if graph:
        gr = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(0)                        # side-stream warm call before capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            for i in range(K):
                step(i)
        gr.replay()                        # untimed first replay (uploads the graph)
        torch.cuda.synchronize()

    def run():
        if gr is not None:
            gr.replay()
        else:
            for i in range(K):
                step(i)

    per_step, first = [], None
    for rep in range(max(1, reps)):
        if evict is not None:
            evict()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        gpu = e0.elapsed_time(e1) * 1e-3
        per_step.append(gpu / K)
        if first is None:
            first = (dt, gpu)
    del gr
    return first[0], first[1], per_step


def spread(per_step_s):
    """Median and 10th / 90th percentiles of per-step times, in microseconds."""
    a = np.asarray(per_step_s) * 1e6
    return {"step_us_median": round(float(np.median(a)), 3), "step_us_p10": round(float(np.percentile(a, 10)), 3),
            "step_us_p90": round(float(np.percentile(a, 90)), 3), "timed_regions": int(a.size)}


def time_launches(launch, n, evict=None, stats=False):
    """Duration of one launch: HIP events recorded on the launch stream around
    each launch (after an eviction of the caches when `evict` is given).
    Returns the mean, or (mean, median, p10, p90) with stats."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    launch(0)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        if evict is not None:
            evict()
        a.record()
        launch(i)
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs]) * 1e-3
    if stats:
        return float(ms.mean()), float(np.median(ms)), float(np.percentile(ms, 10)), float(np.percentile(ms, 90))
    return float(ms.mean())


def roofline_bytes(nbytes, sec, kernel):
    a = nbytes / sec / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic(kernel), "kernel": kernel,
            "kernel_us": round(sec * 1e6, 3)}


def roofline_ops(ops, sec, kernel):
    a = ops / sec / 1e12
    return {"bound": "mfma", "achieved": round(a, 2), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
            "frac": round(a / INT8_PEAK_TOPS, 4), "traffic": traffic(kernel), "kernel": kernel,
            "kernel_us": round(sec * 1e6, 3), "ops_note": "int8 ops = 2*M*N*K, peak = dense int8 MFMA"}


# ------------------------------------------------------------------ measured ceilings

def bench_ceilings(ctx, steps, warmup):
    """Measured ceilings next to the published peaks: a plain streaming read at
    the headline's size (rotating through 1 GiB so every launch reads from HBM,
    graph-timed like the headline) and at the lm_head's weight size,
    MFMA-only loops (fp16 32x32x16, int8 32x32x32) and the MMQ inner loop with
    its per-block rescale in both operand types."""
    dev, L = ctx.dev, ctx.L
    sink = torch.zeros(4096, dtype=torch.uint8, device=dev)
    out = {}
    small = 9453568                                     # the headline step's bytes, a multiple of 16
    buf = torch.empty(ROTATE_BYTES, dtype=torch.uint8, device=dev)
    R = ROTATE_BYTES // small

    def step(i):
        check(L.ggq_bench_stream_read(ctypes.c_void_p(buf.data_ptr() + (i % R) * small), small, vp(sink), 4096,
                                      ctx.s), "bench_stream_read")
    dt, gpu, _ = time_steps(step, steps, warmup, graph=True, evict=ctx.evict, reps=1)
    out["read_gbs_9MB"] = round(small * steps / gpu / 1e9, 1)
    big = 417177600                                     # the lm_head's weight bytes
    sec = time_launches(lambda i: check(L.ggq_bench_stream_read(vp(buf), big, vp(sink), 4096, ctx.s),
                                        "bench_stream_read"), 10, evict=ctx.evict)
    out["read_gbs_417MB"] = round(big / sec / 1e9, 1)
    del buf
    iters = 20000
    waves = 1024 * 4
    for kind, name, ops in ((0, "mfma_f16_tflops", 32 * 32 * 16 * 2), (1, "mfma_i8_tops", 32 * 32 * 32 * 2)):
        sec = time_launches(lambda i: check(L.ggq_bench_mfma_loop(kind, iters, vp(sink), 4096, ctx.s),
                                            "bench_mfma_loop"), 5)
        out[name] = round(waves * iters * 4 * ops / sec / 1e12, 1)
    # the MMQ inner loop alone (fragments and d8 from LDS, exact rescale per
    # q8_1 block), fp16 against int8 MFMA, plain and software-pipelined, at 1
    # and 2 workgroups of 4 waves per CU; kind 2 is the LDS read rate alone
    iters = 20000
    inner = {}
    for kind, name in ((0, "f16"), (1, "i8"), (3, "f16_pipelined"), (4, "i8_pipelined"), (2, "lds_read")):
        for bpc in (1, 2):
            sec = time_launches(lambda i: check(L.ggq_bench_inner_loop(kind, bpc, iters, vp(sink), 4096, ctx.s),
                                                "bench_inner_loop"), 3)
            nw = 256 * bpc * 4
            if kind == 2:
                inner[f"{name}_B_per_clk_cu_{bpc}wg"] = round(nw * iters * 8192 / sec / 256 / 2.4e9, 1)
            else:
                inner[f"{name}_tops_{bpc}wg"] = round(nw * iters * 2 * 64 * 64 * 32 / sec / 1e12, 1)
    out["mmq_inner_loop"] = inner
    return out


def with_ceiling(roof, ceiling):
    """Add the fraction of a measured ceiling to a roofline object."""
    if roof and ceiling:
        roof = dict(roof)
        roof["measured_ceiling"] = ceiling
        roof["frac_of_measured"] = round(roof["achieved"] / ceiling, 4)
    return roof


# ------------------------------------------------------------------ dense decode (MMVQ)

def bench_decode(ctx, wt, N, K, M, seed_w, seed_x, ydt, steps, warmup, rotate=True):
    dev = ctx.dev
    rb = g.row_bytes(wt, K)
    wbytes = N * rb
    R = max(1, -(-ROTATE_BYTES // wbytes)) if rotate else 1
    W0 = torch.from_numpy(inputs.gen_weights(wt, N, K, seed_w)).to(dev)
    Wr = W0.unsqueeze(0).repeat(R, 1, 1).contiguous() if R > 1 else W0.unsqueeze(0)
    del W0
    x = bf16(inputs.gen_act(M, K, seed_x, "bf16"), dev)
    y = torch.empty((M, N), dtype=ydt, device=dev)
    ydt_c = g.F32 if ydt == torch.float32 else g.BF16
    wsb = ctx.L.ggq_mul_mat_ws(wt, N, K, g.BF16, M, g.PATH_MMVQ)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

    def step(i):
        check(ctx.L.ggq_mul_mat(wt, vp(Wr[i % R]), N, K, vp(x), g.BF16, M, K, vp(y), ydt_c, N, vp(ws), wsb,
                                g.PATH_MMVQ, ctx.s), "mul_mat")

    # one step is one launch of the MMVQ kernel (it quantizes the activations itself)
    dt, gpu, per = time_steps(step, steps, warmup, graph=True, evict=ctx.evict)
    ysz = 4 if ydt == torch.float32 else 2
    step_bytes = wbytes + M * K * 2 + M * N * ysz     # weights + bf16 activations + output
    del Wr
    roof = roofline_bytes(step_bytes, gpu / steps, f"mmvq_kernel<{TNAME[wt]},NC={min(8, M)}>")
    roof["kernel_us_source"] = "HIP events around the timed graph replay of K launches, divided by K"
    return {"value": step_bytes * steps / dt / 1e9, "unit": "GB/s", "ms_per_step": dt / steps * 1e3,
            "step_bytes": step_bytes, "rotating_copies": R, "rotating_bytes": R * wbytes, **spread(per),
            "roofline": roof}


def bench_get_rows(ctx, wt, rows, K, n, seed_w, seed_ids, ydt, steps, warmup):
    """n random rows of a quantized table (the lm_head-shaped Q6_K table read as embeddings)."""
    dev = ctx.dev
    W = torch.from_numpy(inputs.gen_weights(wt, rows, K, seed_w)).to(dev)
    ids = torch.from_numpy(inputs.rng(seed_ids).integers(0, rows, n).astype(np.int32)).to(dev)
    y = torch.empty((n, K), dtype=ydt, device=dev)
    ydt_c = g.F32 if ydt == torch.float32 else g.BF16

    def step(i):
        check(ctx.L.ggq_get_rows(wt, vp(W), rows, K, vp(ids), n, vp(y), ydt_c, K, ctx.s), "get_rows")

    dt, gpu, per = time_steps(step, steps, warmup, graph=True, evict=ctx.evict)
    step_bytes = n * (g.row_bytes(wt, K) + 4 + K * (4 if ydt == torch.float32 else 2))
    return {"value": step_bytes * steps / dt / 1e9, "unit": "GB/s", "ms_per_step": dt / steps * 1e3,
            "step_bytes": step_bytes, **spread(per),
            "roofline": roofline_bytes(step_bytes, gpu / steps, f"dequant_rows_kernel<{TNAME[wt]}> (get_rows)")}


# ------------------------------------------------------------------ dense prefill (MMQ)

def bench_prefill(ctx, wt, N, K, M, seed_w, seed_x, ydt, steps, warmup, path=g.PATH_AUTO):
    dev = ctx.dev
    W = torch.from_numpy(inputs.gen_weights(wt, N, K, seed_w)).to(dev)
    x = bf16(inputs.gen_act(M, K, seed_x, "bf16"), dev)
    y = torch.empty((M, N), dtype=ydt, device=dev)
    ydt_c = g.F32 if ydt == torch.float32 else g.BF16
    wsb = ctx.L.ggq_mul_mat_ws(wt, N, K, g.BF16, M, path)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

    def step(i):
        check(ctx.L.ggq_mul_mat(wt, vp(W), N, K, vp(x), g.BF16, M, K, vp(y), ydt_c, N, vp(ws), wsb, path, ctx.s),
              "mul_mat")

    graph = M * N * K < 2e11
    dt, _, per = time_steps(step, steps, warmup, graph=graph, evict=ctx.evict, reps=3)
    ops = 2.0 * M * N * K
    res = {"value": ops * steps / dt / 1e12, "unit": "TOPS", "ms_per_step": dt / steps * 1e3, **spread(per)}
    if path != g.PATH_MMVQ and M > 8:
        # kernel alone: pre-quantized planar operands are produced inside the call, so time the
        # whole call and subtract the quantize kernel measured on its own
        q8 = torch.empty(M * (K // 32) * 40, dtype=torch.uint8, device=dev)
        tq = time_launches(lambda i: check(ctx.L.ggq_quantize_q8_1(vp(x), g.BF16, M, K, K, vp(q8), ctx.s), "q"), 20)
        tc, tc_med, tc10, tc90 = time_launches(step, 20, stats=True)
        res["roofline"] = roofline_ops(ops, max(tc - tq, 1e-9), f"mmq_kernel<{TNAME[wt]}> {N}x{K} M={M}")
        res["roofline"]["kernel_us_source"] = "HIP events around each of 20 calls (mean) minus the quantize kernel's"
        res["call_us_median"], res["call_us_p10"], res["call_us_p90"] = (round(tc_med * 1e6, 2), round(tc10 * 1e6, 2),
                                                                         round(tc90 * 1e6, 2))
        res["quantize_us"] = round(tq * 1e6, 2)
    return res


# ------------------------------------------------------------------ crossover with dequantize + GEMM

def bench_crossover(ctx, Ms=(1, 8, 64, 512, 8192)):
    """Three ways to multiply the Q4_K 8192x2048 weight by M bf16 rows: MMVQ, MMQ,
    and the baseline the pages compare against -- dequantize the weight to bf16
    (this library's kernel) and multiply with the vendor GEMM (torch.mm,
    hipBLASLt).  The baseline skips the q8_1 activation quantization, so
    its result is not the method's; it is timed, not tested.  Mean call times
    from HIP events; the weights stay in cache (same buffers every call)."""
    dev, L = ctx.dev, ctx.L
    N, K, wt = 8192, 2048, g.Q4_K
    W = torch.from_numpy(inputs.gen_weights(wt, N, K, 301)).to(dev)
    Wd = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    out = []
    for M in Ms:
        x = bf16(inputs.gen_act(M, K, 302, "bf16"), dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        row = {"workload": "q4_K_8192x2048_crossover", "M": M}
        for path, pn in ((g.PATH_MMVQ, "mmvq"), (g.PATH_MMQ, "mmq")):
            if pn == "mmvq" and M > 512:
                continue
            wsb = L.ggq_mul_mat_ws(wt, N, K, g.BF16, M, path)
            ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
            t = time_launches(lambda i: check(L.ggq_mul_mat(wt, vp(W), N, K, vp(x), g.BF16, M, K, vp(y), g.BF16, N,
                                                            vp(ws), wsb, path, ctx.s), pn), 20)
            row[pn + "_us"] = round(t * 1e6, 2)
        dq = lambda i: check(L.ggq_dequantize(wt, vp(W), N, K, vp(Wd), g.BF16, ctx.s), "dequantize")
        gemm = lambda i: torch.mm(x, Wd.t(), out=y)          # 2-D GEMM, weight as the transposed operand
        row["dequant_us"] = round(time_launches(dq, 20) * 1e6, 2)
        row["gemm_us"] = round(time_launches(gemm, 20) * 1e6, 2)
        row["dequant_gemm_us"] = round(row["dequant_us"] + row["gemm_us"], 2)
        out.append(row)
    return out


# ------------------------------------------------------------------ dispatch thresholds

def bench_thresholds(ctx):
    """Call times that set the dispatch rules, caches evicted before every launch
    (decode-sized calls read their weights from HBM in a real model):
    dense Q4_K 4096x4096 at M = 1..16, 24 .. 192 on both paths; the MoE projections of
    E=256 top-8 H=2048 I=512 at T = 8..1024 on both paths; the routes per MMVQ-id
    group (1, 2, 4, 8) at T = 16..128 for uniform and skewed routing; and
    MMQ-id at T = 8192 for both routings."""
    dev, L = ctx.dev, ctx.L
    out = []
    N, K, wt = 4096, 4096, g.Q4_K
    W = torch.from_numpy(inputs.gen_weights(wt, N, K, 201)).to(dev)
    for M in list(range(1, 17)) + [24, 32, 48, 64, 96, 128, 192]:
        x = bf16(inputs.gen_act(M, K, 202, "bf16"), dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        row = {"workload": "thresholds_dense_q4_K_4096x4096", "M": M}
        for path, pn in ((g.PATH_MMVQ, "mmvq"), (g.PATH_MMQ, "mmq")):
            wsb = L.ggq_mul_mat_ws(wt, N, K, g.BF16, M, path)
            ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
            t = time_launches(lambda i: check(L.ggq_mul_mat(wt, vp(W), N, K, vp(x), g.BF16, M, K, vp(y), g.BF16, N,
                                                            vp(ws), wsb, path, ctx.s), pn), 10, evict=ctx.evict)
            row[pn + "_us"] = round(t * 1e6, 2)
        out.append(row)
    del W
    E, H, I, top_k = 256, 2048, 512, 8
    Wgu = torch.from_numpy(inputs.gen_experts(g.Q4_K, E, 2 * I, H, 501)).to(dev)
    Wd = torch.from_numpy(inputs.gen_experts(g.Q6_K, E, H, I, 502)).to(dev)

    def moe_calls(Tn, routing, paths, reps):
        ids_np, w_np = routing
        x = bf16(inputs.gen_act(Tn, H, 503, "bf16"), dev)
        h = bf16(inputs.gen_act(Tn * top_k, I, 505, "bf16"), dev)
        ids, w = torch.from_numpy(ids_np).to(dev), torch.from_numpy(w_np).to(dev)
        yg = torch.empty((Tn, top_k, I), dtype=torch.bfloat16, device=dev)
        yd = torch.empty((Tn, H), dtype=torch.bfloat16, device=dev)
        res = {}
        for path, pn in paths:
            w1 = L.ggq_mul_mat_id_ws(g.Q4_K, E, 2 * I, H, g.BF16, Tn, 0, top_k, g.EPI_SWIGLU, 0, path)
            w2 = L.ggq_mul_mat_id_ws(g.Q6_K, E, H, I, g.BF16, Tn, 1, top_k, g.EPI_NONE, 1, path)
            ws = torch.empty(max(w1, w2, 256), dtype=torch.uint8, device=dev)
            gu = lambda i: check(L.ggq_mul_mat_id(g.Q4_K, vp(Wgu), E, 2 * I, H, Wgu.stride(0), vp(x), g.BF16, Tn, 0,
                                                  vp(ids), top_k, None, g.EPI_SWIGLU, vp(yg), g.BF16, vp(ws), w1,
                                                  path, ctx.s), "gate_up")
            dn = lambda i: check(L.ggq_mul_mat_id(g.Q6_K, vp(Wd), E, H, I, Wd.stride(0), vp(h), g.BF16, Tn, 1,
                                                  vp(ids), top_k, vp(w), g.EPI_NONE, vp(yd), g.BF16, vp(ws), w2,
                                                  path, ctx.s), "down")
            res[pn + "_gate_up_us"] = round(time_launches(gu, reps, evict=ctx.evict) * 1e6, 2)
            res[pn + "_down_us"] = round(time_launches(dn, reps, evict=ctx.evict) * 1e6, 2)
        return res

    both = ((g.PATH_MMVQ, "mmvq"), (g.PATH_MMQ, "mmq"))
    for Tn in (8, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512, 1024):
        r = moe_calls(Tn, inputs.gen_routing(Tn, E, top_k, 504), both, 8 if Tn <= 256 else 4)
        out.append({"workload": "thresholds_moe_e256_top8_h2048_i512", "T": Tn, **r})
    for kind, gen in (("uniform", inputs.gen_routing), ("skewed", inputs.gen_routing_skewed)):
        for Tn in (16, 32, 64, 128):
            routing = gen(Tn, E, top_k, 504)
            row = {"workload": "thresholds_mmvq_id_cols", "T": Tn, "routing": kind}
            for J in (1, 2, 4, 8):
                check(L.ggq_bench_set_mmvq_id_cols(J), "set cols")
                r = moe_calls(Tn, routing, ((g.PATH_MMVQ, "mmvq"),), 8)
                row[f"J{J}_gate_up_us"], row[f"J{J}_down_us"] = r["mmvq_gate_up_us"], r["mmvq_down_us"]
            check(L.ggq_bench_set_mmvq_id_cols(0), "set cols")
            r = moe_calls(Tn, routing, ((g.PATH_MMVQ, "mmvq"),), 8)
            row["auto_gate_up_us"], row["auto_down_us"] = r["mmvq_gate_up_us"], r["mmvq_down_us"]
            out.append(row)
        r = moe_calls(8192, gen(8192, E, top_k, 504), ((g.PATH_MMQ, "mmq"),), 3)
        out.append({"workload": "thresholds_mmq_id_t8192", "T": 8192, "routing": kind, **r})
    return out


# ------------------------------------------------------------------ MoE layer

def bench_moe(ctx, Tn, steps, warmup):
    dev = ctx.dev
    E, H, I, top_k = 256, 2048, 512, 8
    Wgu0 = torch.from_numpy(inputs.gen_experts(g.Q4_K, E, 2 * I, H, 501)).to(dev)
    Wd0 = torch.from_numpy(inputs.gen_experts(g.Q6_K, E, H, I, 502)).to(dev)
    # decode-sized batches stream the experts' weights: rotate copies (0.5 GB each)
    # so that no step finds them in the 256 MB last-level cache
    ncopy = 4 if Tn <= 64 else 1
    Wgus = [Wgu0] + [Wgu0.clone() for _ in range(ncopy - 1)]
    Wds = [Wd0] + [Wd0.clone() for _ in range(ncopy - 1)]
    Wgu, Wd = Wgu0, Wd0
    x = bf16(inputs.gen_act(Tn, H, 503, "bf16"), dev)
    ids_np, w_np = inputs.gen_routing(Tn, E, top_k, 504)
    ids = torch.from_numpy(ids_np).to(dev)
    w = torch.from_numpy(w_np).to(dev)
    # h between the projections: q8_1 blocks straight from the gate_up epilogue
    # (the down projection's own input format), or bf16 (then quantized again)
    h = torch.empty((Tn, top_k, I), dtype=torch.bfloat16, device=dev)
    hq = torch.empty((Tn, top_k, I // 32 * 40), dtype=torch.uint8, device=dev)
    y = torch.empty((Tn, H), dtype=torch.bfloat16, device=dev)
    L = ctx.L
    ws1b = L.ggq_mul_mat_id_ws(g.Q4_K, E, 2 * I, H, g.BF16, Tn, 0, top_k, g.EPI_SWIGLU, 0, g.PATH_AUTO)
    ws2b = L.ggq_mul_mat_id_ws(g.Q6_K, E, H, I, g.BF16, Tn, 1, top_k, g.EPI_NONE, 1, g.PATH_AUTO)
    ws1 = torch.empty(ws1b, dtype=torch.uint8, device=dev)
    ws2 = torch.empty(ws2b, dtype=torch.uint8, device=dev)
    s_gu = Wgu.stride(0)
    s_d = Wd.stride(0)

    def gate_up(i, q8=True):
        check(L.ggq_mul_mat_id(g.Q4_K, vp(Wgus[i % ncopy]), E, 2 * I, H, s_gu, vp(x), g.BF16, Tn, 0, vp(ids), top_k, None,
                               g.EPI_SWIGLU, vp(hq if q8 else h), g.Q8_1 if q8 else g.BF16, vp(ws1), ws1b,
                               g.PATH_AUTO, ctx.s), "gate_up")

    def down(i, q8=True):
        check(L.ggq_mul_mat_id(g.Q6_K, vp(Wds[i % ncopy]), E, H, I, s_d, vp(hq if q8 else h), g.Q8_1 if q8 else g.BF16,
                               Tn, 1, vp(ids), top_k, vp(w), g.EPI_NONE, vp(y), g.BF16, vp(ws2), ws2b, g.PATH_AUTO,
                               ctx.s), "down")

    def step(i):
        gate_up(i, False)
        down(i, False)

    def step_q8_h(i):
        gate_up(i)
        down(i)

    dt, _, per = time_steps(step, steps, warmup, graph=Tn <= 64, evict=ctx.evict, reps=3)
    sq = max(steps // 2, 1)
    dt_q, _, _ = time_steps(step_q8_h, sq, max(warmup // 2, 1), graph=Tn <= 64, evict=ctx.evict, reps=1)
    R = Tn * top_k
    res = {"ms_per_step": dt / steps * 1e3, "h_between": "bf16", **spread(per),
           "ms_per_step_q8_1_h": round(dt_q / sq * 1e3, 4)}
    tg = time_launches(lambda i: gate_up(i, False), 20)
    td = time_launches(lambda i: down(i, False), 20)
    if Tn <= 64:
        distinct = len(np.unique(ids_np))
        moved = distinct * (Wgu.stride(0) + Wd.stride(0)) + Tn * H * 2 * 2 + R * I * 2 * 2
        res.update({"value": moved * steps / dt / 1e9, "unit": "GB/s", "distinct_experts": int(distinct),
                    "rotating_weight_copies": ncopy,
                    "roofline": roofline_bytes(distinct * Wgu.stride(0), tg, "mmvq_id gate_up (call)"),
                    "down_call_us": round(td * 1e6, 2)})
    else:
        ops_gu = 2.0 * R * 2 * I * H
        ops_d = 2.0 * R * H * I
        res.update({"value": (ops_gu + ops_d) * steps / dt / 1e12, "unit": "TOPS",
                    "roofline": roofline_ops(ops_gu, tg, "mmq_id gate_up (call)"),
                    "down": roofline_ops(ops_d, td, "mmq_id down (call)")})
    return res


# ------------------------------------------------------------------ CPU baseline

def cpu_oracle_c2(seconds):
    """Child-process body of the CPU baseline: the oracle on the whole headline
    workload (Q4_K 4096 x 4096, one bf16 row: q8_1 quantization + fp64
    quantized dot of every weight row), repeated for about `seconds`, with
    the OpenMP thread count the environment sets."""
    import oracle
    N, K = 4096, 4096
    W = inputs.gen_q4_K(N, K, 201)
    x = inputs.gen_act(1, K, 202, "bf16")
    oracle.mul_mat(oracle.Q4_K, W, N, K, x)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        oracle.mul_mat(oracle.Q4_K, W, N, K, x)
        n += 1
    dt = time.perf_counter() - t0
    moved = N * g.row_bytes(g.Q4_K, K) + K * 2 + 2 * (K // 32) * 40 + N * 2
    return {"value": round(moved * n / dt / 1e9, 3), "unit": "GB/s", "calls": n, "seconds": round(dt, 2),
            "ms_per_call": round(dt / n * 1e3, 3)}


def cpu_baseline(seconds=10.0):
    """The CPU oracle on the headline workload, on this host's cores (all of
    them, then one thread), each run in a child process with OMP_NUM_THREADS
    set (the oracle parallelizes over output rows with OpenMP)."""
    import subprocess
    allc = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    runs = {}
    for name, threads, sec in (("all", allc, seconds), ("one", 1, max(2.0, seconds / 2))):
        env = dict(os.environ, OMP_NUM_THREADS=str(threads))
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-oracle-child", str(sec)], env=env,
                           capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError(f"cpu baseline child failed: {r.stderr[-2000:]}")
        runs[name] = json.loads(r.stdout.strip().splitlines()[-1])
    a = runs["all"]
    quota = None
    try:                                               # cgroup v2 CPU quota, if the host sets one
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        quota = None if q == "max" else round(int(q) / int(per), 2)
    except (OSError, ValueError):
        pass
    return {"value": a["value"], "unit": "GB/s", "cores": allc, "kind": "oracle",
            "cpus_allowed": len(os.sched_getaffinity(0)), "cgroup_cpu_quota": quota,
            "speedup_all_vs_one": round(a["value"] / max(runs["one"]["value"], 1e-12), 2),
            "sample": f"the whole q4_K 4096x4096 M=1 workload per call (bf16 row -> q8_1, fp64 quantized dot of all "
                      f"4096 rows): {a['calls']} calls in {a['seconds']} s, {a['ms_per_call']} ms per call",
            "host_cpus": os.cpu_count(),
            "single_thread": {"value": runs["one"]["value"], "unit": "GB/s", "cores": 1,
                              "ms_per_call": runs["one"]["ms_per_call"], "calls": runs["one"]["calls"]}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--workloads", default="all",
                    help="comma list of: decode, prefill, sweep, lmhead1, lmhead2048, getrows, types, crossover, "
                         "moe16, moe8192 (default all), and thresholds (only when named)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-oracle-child", type=float, default=None, help=argparse.SUPPRESS)
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 256 MiB device copy 10 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.cpu_oracle_child is not None:              # CPU baseline child: no GPU use
        print(json.dumps(cpu_oracle_c2(args.cpu_oracle_child)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ctx = Ctx(dev)
    K, W = args.steps, args.warmup
    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": a.numel(), "calib_copy_bytes_written": b.numel(), "launches": 10}))
        return

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    log("measured ceilings: streaming read, MFMA loops")
    ceil = bench_ceilings(ctx, K, W)
    log("headline: q4_K 4096x4096 decode M=1")
    head = bench_decode(ctx, g.Q4_K, 4096, 4096, 1, 201, 202, torch.bfloat16, K, W)
    also = []
    sel = set(args.workloads.split(",")) if args.workloads != "all" else {
        "decode", "prefill", "sweep", "lmhead1", "lmhead2048", "getrows", "types", "crossover", "moe16", "moe8192"}
    if args.only_headline:
        sel = set()
    if "decode" in sel:
        for M in (2, 4, 8):
            log(f"q4_K 4096x4096 decode M={M}")
            r = bench_decode(ctx, g.Q4_K, 4096, 4096, M, 201, 202, torch.bfloat16, K, W)
            also.append({"workload": "q4_K_4096x4096_decode", "M": M, **r})
    if "prefill" in sel:
        log("q4_K 8192x2048 prefill M=8192")
        r = bench_prefill(ctx, g.Q4_K, 8192, 2048, 8192, 301, 302, torch.bfloat16, max(5, K // 20), max(2, W // 10))
        also.append({"workload": "q4_K_8192x2048_prefill", "M": 8192, **r})
    if "sweep" in sel:
        for M in (16, 24, 32, 64):
            for path, pn in ((g.PATH_MMVQ, "mmvq"), (g.PATH_MMQ, "mmq")):
                log(f"q4_K 8192x2048 sweep M={M} {pn}")
                r = bench_prefill(ctx, g.Q4_K, 8192, 2048, M, 301, 302, torch.bfloat16, max(20, K // 4), W, path)
                also.append({"workload": "q4_K_8192x2048_prefill_sweep", "M": M, "path": pn, **r})
    if "lmhead1" in sel:
        log("q6_K 248320x2048 lm_head M=1")
        r = bench_decode(ctx, g.Q6_K, 248320, 2048, 1, 401, 402, torch.float32, max(20, K // 4), W)
        also.append({"workload": "q6_K_248320x2048_lm_head", "M": 1, **r})
    if "types" in sel:
        for wt, name in ((g.Q4_0, "q4_0"), (g.Q5_K, "q5_K")):
            log(f"{name} 4096x4096 decode M=1")
            r = bench_decode(ctx, wt, 4096, 4096, 1, 201, 202, torch.bfloat16, K, W)
            also.append({"workload": f"{name}_4096x4096_decode", "M": 1, **r})
        for wt, name in ((g.Q5_K, "q5_K"), (g.Q8_0, "q8_0"), (g.Q4_0, "q4_0")):
            log(f"{name} 8192x2048 prefill M=8192")
            r = bench_prefill(ctx, wt, 8192, 2048, 8192, 301, 302, torch.bfloat16, max(5, K // 20), max(2, W // 10))
            also.append({"workload": f"{name}_8192x2048_prefill", "M": 8192, **r})
    if "thresholds" in sel:
        log("dispatch thresholds: dense M=1..16, routed T=8..128, MMVQ-id group widths, MMQ-id routings")
        also.extend(bench_thresholds(ctx))
    if "crossover" in sel:
        log("q4_K 8192x2048 crossover: MMVQ / MMQ / dequantize + GEMM")
        also.extend(bench_crossover(ctx))
    if "getrows" in sel:
        log("q6_K 248320x2048 get_rows n=8192")
        r = bench_get_rows(ctx, g.Q6_K, 248320, 2048, 8192, 401, 404, torch.bfloat16, max(20, K // 4), W)
        also.append({"workload": "q6_K_248320x2048_get_rows", "n": 8192, **r})
    if "lmhead2048" in sel:
        log("q6_K 248320x2048 lm_head M=2048")
        r = bench_prefill(ctx, g.Q6_K, 248320, 2048, 2048, 401, 402, torch.float32, max(3, K // 40), 1)
        also.append({"workload": "q6_K_248320x2048_lm_head", "M": 2048, **r})
    torch.cuda.empty_cache()
    for Tn in (16, 8192):
        if f"moe{Tn}" in sel:
            log(f"moe T={Tn}")
            r = bench_moe(ctx, Tn, max(5, K // (1 if Tn <= 64 else 20)), max(2, W // 4))
            also.append({"workload": "moe_e256_top8_h2048_i512", "T": Tn, **r})
    # secondary column: each kernel against the measured ceiling of its bound
    for a in also:
        r = a.get("roofline")
        if not r:
            continue
        if r["bound"] == "hbm":
            big = a.get("step_bytes", 0) > 32e6 or a["workload"].startswith("moe")
            a["roofline"] = with_ceiling(r, ceil["read_gbs_417MB"] if big else ceil["read_gbs_9MB"])
        else:
            a["roofline"] = with_ceiling(r, ceil["mfma_i8_tops"])
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)
    line = {
        "metric": METRIC, "value": round(head["value"], 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(head["ms_per_step"], 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "q4_K_4096x4096_decode", "M": 1, "N": 4096, "K": 4096, "weights": "Q4_K",
                   "activations": "bf16 -> q8_1", "output": "bf16", "rotating_weight_copies": head["rotating_copies"],
                   "step_bytes": head["step_bytes"]},
        "roofline": with_ceiling(head["roofline"], ceil["read_gbs_9MB"]), "cpu_baseline": cpu,
        "ceilings": ceil, "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
