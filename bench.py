"""Benchmark of the block-scaled FP4 hot path on one MI355X.

Headline (one JSON line on stdout): quantize throughput in GB/s of
algorithmic bytes over the scale-format sweep workload -- a 4096x4096 bf16
tensor (N(0, 0.02), 0.1% of entries x100) quantized with E4M3, UE5M3, E3M4
and E1M6 block-16 scales (current amax) and E8M0 block-32 scales (MXFP4),
round-to-nearest.  One step = those five quantize calls.  Inputs rotate
over 24 resident copies (768 MiB, three times the 256 MB last-level cache)
so the rate is an HBM rate; each rotation slot is a captured HIP graph so
the host launch rate does not limit the GPU.

Algorithmic bytes per call: input read once (2 B/elem), codes (0.5 B/elem),
scales (1/B B/elem) and the tensor scale (8 B).  A current-amax call needs
the tensor maximum before any code, but the minimum traffic is still one
read: the single-pass kernel holds the tensor in registers while the grid
agrees on the maximum.

Further legs reported in "legs": stochastic rounding with delayed amax over
200 successive 8192x8192 gradients, the same gradients quantized column-wise
(the backward-pass operands), dequantize, quantize with the blockwise
randomized Hadamard transform, the INT4 element grid (quantize and GEMM), the 8-bit MX grids (quantize), the block-scaled GEMM on the
Llama-2 7B linear shapes, and the weight-only GEMM at Qwen-2.5 decode
shapes.  "roofline" is the dominant kernel of the step (the single-pass
E4M3 block-16 current-amax quantize kernel: four of the five calls) timed
alone with HIP events on its stream over the rotating inputs;
"cpu_baseline" is the CPU oracle on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the roofline kernel, from rocprofv3 counters
# (TCC_EA0_RDREQ_128B / _64B / _32B and TCC_EA0_WRREQ / _64B, per dispatch,
# times the request size), recorded with the SHA-256 of the kernel sources it
# was measured on; reported only while those sources are unchanged.
MEASURED_TRAFFIC = {
    "sources": ["fp4_block_scaled_quantize_amd/csrc/quant.hip", "fp4_block_scaled_quantize_amd/csrc/fp4_device.hpp",
                "fp4_block_scaled_quantize_amd/csrc/fp4_internal.h"],
    "sha256": "5b9276969ebeac3214d9d7dcb1300c735b2e8947247a76ef0f677e336c4bb3a5",
    "read_bytes": 33861632,
    "write_bytes": 9453696,
    "profile": "profiles/quantize_fused_4096_hbm_traffic.md",
}


def measured_traffic():
    import hashlib
    h = hashlib.sha256()
    for f in MEASURED_TRAFFIC["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != MEASURED_TRAFFIC["sha256"]:
        return None
    return MEASURED_TRAFFIC["read_bytes"] + MEASURED_TRAFFIC["write_bytes"]
MFMA_PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "bf16": 2500.0}
# the one kernel each GEMM call launches, by the operands' scale encoding
GEMM_KERNEL = {("e8m0", 32): "k_gemm_mx (scaled FP4 MFMA)",
               ("e4m3", 16): "k_gemm_nv (FP4->f16 in registers, f16 MFMA)",
               ("ue5m3", 16): "k_gemm_nv (FP4->fp32 x scale->bf16 in registers, bf16 MFMA)",
               ("e8m0", 16): "k_gemm_mx16 (scaled FP4 MFMA, two instructions per K-half)"}

SWEEP = [("e4m3", 16, "current"), ("ue5m3", 16, "current"), ("e3m4", 16, "current"), ("e1m6", 16, "current"),
         ("e8m0", 32, "none")]


def quant_bytes(rows, cols, block, in_bytes=2):
    n = rows * cols
    return n * in_bytes + n // 2 + n // block + 8


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--rot", type=int, default=24, help="resident input copies rotated through")
    p.add_argument("--legs", default="small,sr,srt,dequant,rht,int4,w8,gemm,gemmsmall,wo,wowide",
                   help="extra legs (comma list, or 'none')")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 64 MiB device copy three times (calibrates HBM byte counters)")
    return p.parse_args()


class GraphSet:
    """One captured HIP graph per rotation slot; replay(i) runs slot i."""

    def __init__(self, torch, n, record):
        self.graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(n):          # eager warm-up of every slot (allocations, module load)
                record(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                record(i)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def replay(self, i):
        self.graphs[i % len(self.graphs)].replay()


def time_graphs(torch, gs, n_iter, n_warm, per_iter_slots=1):
    """Replay the graphs n_iter times after n_warm; return ms per replay."""
    for i in range(n_warm):
        gs.replay(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_iter):
        gs.replay(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n_iter


def leg_roofline(torch, fq, xs):
    """The dominant kernel of the step: E4M3 block-16 round-to-nearest with
    the current amax (single-pass kernel), one launch per input over the
    rotating copies, timed with HIP events around graph replays on the
    stream the kernels run on.  The same kernel with no tensor scale (no
    grid exchange) is timed beside it for reference."""
    rows, cols = xs[0].shape
    algo = quant_bytes(rows, cols, 16)
    res = {}
    for pol in ("current", "none"):
        outs = [fq.QTensor.empty(rows, cols, 16, "e4m3", amax=pol) for _ in xs]
        st = fq.AmaxState(1) if pol == "current" else None

        def rec(i):
            for j in range(len(xs)):
                fq.fp4_quantize(xs[j], 16, "e4m3", amax=pol, state=st, out=outs[j])
        gs = GraphSet(torch, 1, rec)
        ms = time_graphs(torch, gs, 40, 5) / len(xs)
        res[pol] = ms
        if st is not None:
            st.get()                     # raises if a grid exchange timed out
    achieved = algo / (res["current"] * 1e-3) / 1e9
    none_gbs = algo / (res["none"] * 1e-3) / 1e9
    traffic = measured_traffic()
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "traffic_over_algorithmic": round(traffic / algo, 4) if traffic else None,
            "kernel": "k_quantize<bf16,16,RTN,ExMy,single-pass current amax>",
            "us_per_launch": round(res["current"] * 1e3, 3), "algo_bytes_per_launch": algo,
            "no_tensor_scale_kernel": {"us_per_launch": round(res["none"] * 1e3, 3), "GB/s": round(none_gbs, 1),
                                       "frac": round(none_gbs / HBM_PEAK_GBS, 4)}}


def leg_sr(torch, fq, inputs, steps):
    """200 successive 8192x8192 bf16 Laplace(1e-4) gradients, E4M3 block 16,
    stochastic rounding (seed 0x5EED, offset = t), delayed amax every 50."""
    rows = cols = 8192
    ntens = 200
    xs = [inputs.device_laplace((rows, cols), 1e-4, inputs.GRADS_SEED0 + t, torch.bfloat16) for t in range(ntens)]
    outs = [fq.QTensor.empty(rows, cols, 16, "e4m3", rounding="stochastic", amax="delayed") for _ in range(2)]
    st = fq.AmaxState(50)

    def rec(_):
        for t in range(ntens):
            fq.fp4_quantize(xs[t], 16, "e4m3", rounding="stochastic", amax="delayed", state=st, seed=0x5EED,
                            offset=t, out=outs[t % 2])
    gs = GraphSet(torch, 1, rec)
    reps = max(1, min(3, steps // 10))
    ms = time_graphs(torch, gs, reps, 1)
    total = ntens * quant_bytes(rows, cols, 16)
    gbs = total / (ms * 1e-3) / 1e9
    del gs
    # the same sequence with round-to-nearest: the row-wise kernel's rate at
    # 8192^2 (4 of the 200 calls also read the tensor for the refresh)
    outs_n = [fq.QTensor.empty(rows, cols, 16, "e4m3", rounding="nearest", amax="delayed") for _ in range(2)]
    st_n = fq.AmaxState(50)

    def rec_n(_):
        for t in range(ntens):
            fq.fp4_quantize(xs[t], 16, "e4m3", rounding="nearest", amax="delayed", state=st_n, out=outs_n[t % 2])
    gs = GraphSet(torch, 1, rec_n)
    ms_n = time_graphs(torch, gs, reps, 1)
    gbs_n = total / (ms_n * 1e-3) / 1e9
    del xs, gs
    return {"workload": "200 x 8192x8192 bf16 Laplace(1e-4) grads, E4M3 B16, SR Philox, delayed amax N=50",
            "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "ms_per_sequence": round(ms, 3),
            "rtn": {"GB/s": round(gbs_n, 1), "frac_hbm": round(gbs_n / HBM_PEAK_GBS, 4),
                    "ms_per_sequence": round(ms_n, 3), "us_per_call": round(ms_n * 1e3 / ntens, 2)}}


def leg_sr_transposed(torch, fq, inputs, steps):
    """Backward-pass operands: the same 200 gradients quantized column-wise
    (blocks of 16 down the columns, i.e. the quantized transpose), E4M3,
    stochastic rounding (seed 0x5EED, offset = t), delayed amax every 50;
    and the round-to-nearest column-wise kernel on the same tensors."""
    rows = cols = 8192
    ntens = 200
    xs = [inputs.device_laplace((rows, cols), 1e-4, inputs.GRADS_SEED0 + t, torch.bfloat16) for t in range(ntens)]
    res = {}
    for rnd in ("stochastic", "nearest"):
        outs = [fq.QTensor.empty(cols, rows, 16, "e4m3", rounding=rnd, amax="delayed") for _ in range(2)]
        st = fq.AmaxState(50)

        def rec(_):
            for t in range(ntens):
                fq.fp4_quantize_transposed(xs[t], 16, "e4m3", rounding=rnd, amax="delayed", state=st, seed=0x5EED,
                                           offset=t, out=outs[t % 2])
        gs = GraphSet(torch, 1, rec)
        reps = max(1, min(3, steps // 10))
        ms = time_graphs(torch, gs, reps, 1)
        gbs = ntens * quant_bytes(rows, cols, 16) / (ms * 1e-3) / 1e9
        res["sr" if rnd == "stochastic" else "rtn"] = {"GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                                     "ms_per_sequence": round(ms, 3)}
        del gs, outs
    # both orientations of every gradient: one two-orientation call against
    # a row-wise plus a column-wise call (each reads the tensor)
    for rnd, mode in (("stochastic", "both"), ("stochastic", "separate"), ("nearest", "both"),
                      ("nearest", "separate")):
        outs = [(fq.QTensor.empty(rows, cols, 16, "e4m3", rounding=rnd, amax="delayed"),
                 fq.QTensor.empty(cols, rows, 16, "e4m3", rounding=rnd, amax="delayed")) for _ in range(2)]
        st, st2 = fq.AmaxState(50), fq.AmaxState(50)

        def rec(_):
            for t in range(ntens):
                o = outs[t % 2]
                if mode == "both":
                    fq.fp4_quantize_both(xs[t], 16, "e4m3", rounding=rnd, amax="delayed", state=st,
                                         seed=0x5EED, offset=t, out=o)
                else:
                    fq.fp4_quantize(xs[t], 16, "e4m3", rounding=rnd, amax="delayed", state=st, seed=0x5EED,
                                    offset=t, out=o[0])
                    fq.fp4_quantize_transposed(xs[t], 16, "e4m3", rounding=rnd, amax="delayed", state=st2,
                                               seed=0x5EED, offset=t, out=o[1])
        gs = GraphSet(torch, 1, rec)
        reps = max(1, min(3, steps // 10))
        ms = time_graphs(torch, gs, reps, 1)
        n = rows * cols
        algo = ntens * (n * 2 + 2 * (n // 2 + n // 16 + 8))        # the input read once, both outputs
        res[f"{'sr' if rnd == 'stochastic' else 'rtn'}_{mode}"] = {
            "ms_per_sequence": round(ms, 3), "GB/s": round(algo / (ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del gs, outs
    del xs
    res["workload"] = ("200 x 8192x8192 bf16 Laplace(1e-4) grads quantized column-wise (x^T), E4M3 B16, "
                       "delayed amax N=50; SR Philox and RTN; both orientations from one read (*_both) "
                       "against a row-wise plus a column-wise call (*_separate), GB/s of one input read "
                       "plus both outputs")
    return res


def leg_rht(torch, fq, xs):
    """Cost of the blockwise randomized Hadamard transform fused into the
    quantize kernel: the sweep tensor quantized E4M3 block 16 (current
    amax, single-pass kernel) and E8M0 block 32, with and without the
    transform, over the rotating inputs."""
    rows, cols = xs[0].shape
    res = {}
    for fmt, block, pol in (("e4m3", 16, "current"), ("e8m0", 32, "none")):
        for signs in (None, 0x9E3779B9):
            outs = [fq.QTensor.empty(rows, cols, block, fmt, amax=pol) for _ in xs]
            st = fq.AmaxState(1) if pol == "current" else None

            def rec(_):
                for j in range(len(xs)):
                    fq.fp4_quantize(xs[j], block, fmt, amax=pol, state=st, out=outs[j], rht_signs=signs)
            gs = GraphSet(torch, 1, rec)
            ms = time_graphs(torch, gs, 20, 3) / len(xs)
            algo = quant_bytes(rows, cols, block)
            res[f"{fmt}_b{block}_{'rht' if signs is not None else 'plain'}"] = {
                "us_per_call": round(ms * 1e3, 3), "GB/s": round(algo / (ms * 1e-3) / 1e9, 1)}
            del gs, outs
    res["workload"] = "4096x4096 bf16 sweep tensor, RTN, with / without the block-16/32 randomized Hadamard transform"
    return res


def leg_small_nvfp4(torch, fq, inputs):
    """The small correctness configuration, timed: B 256x256 fp32 (1% of
    entries x50) quantized NVFP4 (E4M3 block 16, current amax, RTN) and
    dequantized to fp32, A 64x256 fp32 quantized the same way, then
    C = A B^T; per-call latency between graph replays (launch-bound at this
    size)."""
    b = torch.from_numpy(inputs.small_b()).cuda()
    a = torch.from_numpy(inputs.small_a()).cuda()
    st_b, st_a = fq.AmaxState(1), fq.AmaxState(1)
    qb = fq.QTensor.empty(256, 256, 16, "e4m3")
    qa = fq.QTensor.empty(64, 256, 16, "e4m3")
    c = torch.empty((64, 256), dtype=torch.bfloat16, device="cuda")
    yb = torch.empty((256, 256), dtype=torch.float32, device="cuda")
    res = {}
    for name, fn in {"quantize_b_us": lambda: fq.fp4_quantize(b, 16, "e4m3", state=st_b, out=qb),
                     "dequantize_b_us": lambda: fq.fp4_dequantize(qb, torch.float32, out=yb),
                     "quantize_a_us": lambda: fq.fp4_quantize(a, 16, "e4m3", state=st_a, out=qa),
                     "gemm_us": lambda: fq.fp4_gemm(qa, qb, out=c)}.items():
        def rec(_, fn=fn):
            for _ in range(10):
                fn()
        gs = GraphSet(torch, 1, rec)
        res[name] = round(time_graphs(torch, gs, 20, 3) / 10 * 1e3, 3)
        del gs
    res["workload"] = ("256x256 fp32 B (quantized and dequantized to fp32) and 64x256 fp32 A, NVFP4 (E4M3 B16, "
                       "current amax, RTN); C = A B^T (8.39 MFLOP); microseconds per call, ten calls per graph replay")
    return res


def leg_dequant(torch, fq, xs):
    rows, cols = xs[0].shape
    qts = [fq.fp4_quantize(x, 16, "e4m3", amax="current") for x in xs]
    ys = [torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda") for _ in xs]

    def rec(_):
        for j in range(len(xs)):
            fq.fp4_dequantize(qts[j], out=ys[j])
    gs = GraphSet(torch, 1, rec)
    ms = time_graphs(torch, gs, 20, 3) / len(xs)
    n = rows * cols
    algo = n // 2 + n // 16 + 8 + n * 2
    return {"workload": "4096x4096 E4M3 B16 -> bf16", "GB/s": round(algo / (ms * 1e-3) / 1e9, 1),
            "us_per_call": round(ms * 1e3, 3)}


def leg_gemm_small(torch, fq, inputs):
    """Small products on both GEMM paths: the one-wave-per-32x32-tile path
    (bound raised above every shape) against the tiled kernels (bound 0),
    NVFP4 (E4M3 block 16), UE5M3 block 16 and MXFP4 (E8M0 block 32) at M = 64 / 256 / 512
    against Llama-2 7B-shaped weights; per-call time between graph replays
    (ten calls per replay), and the path the default bound picks."""
    shapes = [(64, 256, 256), (64, 11008, 4096), (256, 11008, 4096), (512, 4096, 4096)]
    res = {}
    default = fq.set_gemm_small_outputs(0)
    fq.set_gemm_small_outputs(default)
    try:
        for fmt, block, pol in (("e4m3", 16, "current"), ("ue5m3", 16, "current"), ("e8m0", 32, "none")):
            for m, n, k in shapes:
                a = inputs.device_normal((m, k), 1.0, inputs.SEEDS["llama_a"], torch.bfloat16)
                w = inputs.device_normal((n, k), 0.02, inputs.SEEDS["llama_up"], torch.bfloat16)
                qa = fq.fp4_quantize(a, block, fmt, amax=pol)
                qw = fq.fp4_quantize(w, block, fmt, amax=pol)
                c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
                row = {}
                for path, bound in (("tiled", 0), ("small", 1 << 40)):
                    fq.set_gemm_small_outputs(bound)

                    def rec(_):
                        for _ in range(10):
                            fq.fp4_gemm(qa, qw, out=c)
                    gs = GraphSet(torch, 1, rec)
                    us = time_graphs(torch, gs, 10, 2) / 10 * 1e3
                    del gs
                    row[path + "_us"] = round(us, 2)
                    row[path + "_TFLOP/s"] = round(2.0 * m * n * k / us / 1e6, 1)
                mn = m * n
                limit = {"e8m0": default / 8, "ue5m3": 1.5 * default}.get(fmt, default)
                row["default_path"] = "small" if mn <= limit else "tiled"
                res[f"{fmt}_b{block}_{m}x{n}x{k}"] = row
    finally:
        fq.set_gemm_small_outputs(default)
    res["workload"] = ("small products, A M x K N(0,1) bf16 and W N x K N(0,0.02) bf16 quantized NVFP4 (E4M3 B16, "
                       "current amax), UE5M3 B16 or MXFP4 (E8M0 B32); the small path against the tiled kernels")
    return res


def leg_gemm(torch, fq, inputs):
    """Llama-2 7B linears at M = 8192: both operands quantized NVFP4 (E4M3
    block 16, exact in-register FP4->f16 path on f16 matrix cores), MXFP4
    (E8M0 block 32, native scaled FP4 matrix cores) and UE5M3 block 16
    (ue5m3-fp4-pretraining "Что сделали": every linear in FP4 with UE5M3
    scales; exact in-register bf16 path, since the products leave f16's
    range)."""
    shapes = {"up": (11008, 4096), "down": (4096, 11008), "sq": (4096, 4096)}
    res = {}
    for fmt, block, pol, peak in [("e8m0", 32, "none", "fp4"), ("e4m3", 16, "current", "bf16"),
                                  ("ue5m3", 16, "current", "bf16"), ("e8m0", 16, "none", "fp4")]:
        for name, (n, k) in shapes.items():
            m = 8192
            a = inputs.device_normal((m, k), 0.02, inputs.SEEDS["llama_a"], torch.bfloat16)
            w = inputs.device_normal((n, k), 0.02, inputs.SEEDS["llama_" + name], torch.bfloat16)
            qa = fq.fp4_quantize(a, block, fmt, amax=pol)
            qw = fq.fp4_quantize(w, block, fmt, amax=pol)
            c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
            key = f"{fmt}_{name}" if block == (32 if fmt == "e8m0" else 16) else f"{fmt}_b{block}_{name}"
            try:
                fq.fp4_gemm(qa, qw, out=c)
            except fq.Fp4Error as e:
                res[key] = {"error": str(e)}
                continue

            def rec(_):
                fq.fp4_gemm(qa, qw, out=c)
            gs = GraphSet(torch, 1, rec)
            ms = time_graphs(torch, gs, 10, 2)
            tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            res[key] = {"M": m, "N": n, "K": k, "TFLOP/s": round(tf, 1), "ms": round(ms, 4),
                                    "frac_fp4_peak": round(tf / MFMA_PEAK_TFLOPS["fp4"], 4),
                                    "frac_fp8_peak": round(tf / MFMA_PEAK_TFLOPS["fp8"], 4),
                                    "frac_path_peak": round(tf / MFMA_PEAK_TFLOPS[peak], 4),
                                    "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                                 "peak": MFMA_PEAK_TFLOPS[peak], "unit": "TFLOP/s",
                                                 "frac": round(tf / MFMA_PEAK_TFLOPS[peak], 4),
                                                 "kernel": GEMM_KERNEL[(fmt, block)], "us_per_launch": round(ms * 1e3, 2),
                                                 "algo_flops_per_launch": 2 * m * n * k, "traffic": None}}
            del a, w, qa, qw, c, gs
    return res


def leg_int4(torch, fq, inputs, xs):
    """The INT4 element grid: quantize throughput on the sweep tensor
    (NVINT4 = E4M3 block 16 with current amax, MXINT4 = E8M0 block 32) and
    the GEMM at the Llama-2 7B up-projection shape on the exact dequantize
    path (bf16 matrix cores)."""
    rows, cols = xs[0].shape
    res = {}
    for name, (fmt, block, pol) in {"nvint4": ("e4m3", 16, "current"), "mxint4": ("e8m0", 32, "none")}.items():
        outs = [fq.QTensor.empty(rows, cols, block, fmt, amax=pol, element="int4") for _ in xs]
        st = fq.AmaxState(1) if pol == "current" else None

        def rec(_):
            for j in range(len(xs)):
                fq.fp4_quantize(xs[j], block, fmt, amax=pol, state=st, out=outs[j], element="int4")
        gs = GraphSet(torch, 1, rec)
        ms = time_graphs(torch, gs, 20, 3) / len(xs)
        algo = quant_bytes(rows, cols, block)
        res[f"{name}_quantize"] = {"us_per_call": round(ms * 1e3, 3), "GB/s": round(algo / (ms * 1e-3) / 1e9, 1),
                                   "frac_hbm": round(algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del gs, outs
        m, n, k = 8192, 11008, 4096
        a = inputs.device_normal((m, k), 0.02, inputs.SEEDS["llama_a"], torch.bfloat16)
        w = inputs.device_normal((n, k), 0.02, inputs.SEEDS["llama_up"], torch.bfloat16)
        qa = fq.fp4_quantize(a, block, fmt, amax=pol, element="int4")
        qw = fq.fp4_quantize(w, block, fmt, amax=pol, element="int4")
        c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

        def rec_g(_):
            fq.fp4_gemm(qa, qw, out=c)
        gs = GraphSet(torch, 1, rec_g)
        ms = time_graphs(torch, gs, 10, 2)
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        res[f"{name}_gemm_up"] = {"M": m, "N": n, "K": k, "TFLOP/s": round(tf, 1), "ms": round(ms, 4),
                                  "frac_bf16_peak": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4)}
        del a, w, qa, qw, c, gs
    res["workload"] = ("INT4 grid: 4096x4096 bf16 sweep tensor quantized NVINT4 (E4M3 B16, current amax) and MXINT4 "
                       "(E8M0 B32); Llama-2 7B up projection 8192x4096 @ 11008x4096 on the exact dequantize path")
    return res


def leg_8bit(torch, fq, inputs, xs):
    """The 8- and 6-bit MX grids: the sweep tensor quantized MXFP8-style (E4M3
    elements), MXINT8-style (E8M0 block 32), one byte per element, and
    MXFP6 / MXINT6-style (six bits per element), and
    the GEMM at the Llama-2 7B up-projection shape: MXFP8 (bf16) and INT8
    elements with E4M3 block-16 scales (f16) on the in-register conversion
    kernel, MXFP6 and MXINT6 (bf16) on the exact dequantize path."""
    rows, cols = xs[0].shape
    res = {}
    n = rows * cols
    names = {"fp8_e4m3": "mxfp8", "int8": "mxint8", "fp6_e2m3": "mxfp6_e2m3", "fp6_e3m2": "mxfp6_e3m2",
             "int6": "mxint6"}
    for elem, name in names.items():
        outs = [fq.QTensor.empty(rows, cols, 32, "e8m0", amax="none", element=elem) for _ in xs]

        def rec(_):
            for j in range(len(xs)):
                fq.fp4_quantize(xs[j], 32, "e8m0", amax="none", out=outs[j], element=elem)
        gs = GraphSet(torch, 1, rec)
        ms = time_graphs(torch, gs, 20, 3) / len(xs)
        nb = n * 2 + n * fq.ELEMENT_BITS[elem] // 8 + n // 32 + 8
        res[f"{name}_quantize"] = {
            "us_per_call": round(ms * 1e3, 3), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del gs, outs
    for elem, name in (("fp8_e4m3", "mxfp8"), ("int8", "mxint8"), ("fp6_e2m3", "mxfp6_e2m3"), ("int6", "mxint6")):
        outs = [fq.QTensor.empty(cols, rows, 32, "e8m0", amax="none", element=elem) for _ in xs]

        def rec_t(_):
            for j in range(len(xs)):
                fq.fp4_quantize_transposed(xs[j], 32, "e8m0", amax="none", out=outs[j], element=elem)
        gs = GraphSet(torch, 1, rec_t)
        ms = time_graphs(torch, gs, 20, 3) / len(xs)
        nb = n * 2 + n * fq.ELEMENT_BITS[elem] // 8 + n // 32 + 8
        res[f"{name}_quantize_colwise"] = {
            "us_per_call": round(ms * 1e3, 3), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del gs, outs
    for elem, name in (("fp8_e4m3", "mxfp8"), ("int6", "mxint6")):
        outs = [(fq.QTensor.empty(rows, cols, 32, "e8m0", amax="none", element=elem),
                 fq.QTensor.empty(cols, rows, 32, "e8m0", amax="none", element=elem)) for _ in xs]

        def rec_b(_):
            for j in range(len(xs)):
                fq.fp4_quantize_both(xs[j], 32, "e8m0", amax="none", out=outs[j], element=elem)
        gs = GraphSet(torch, 1, rec_b)
        ms = time_graphs(torch, gs, 20, 3) / len(xs)
        nb = n * 2 + 2 * (n * fq.ELEMENT_BITS[elem] // 8 + n // 32 + 8)
        res[f"{name}_quantize_both"] = {
            "us_per_call": round(ms * 1e3, 3), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del gs, outs
    m, n, k = 8192, 11008, 4096
    for name, (elem, fmt, block, pol) in {"mxfp8": ("fp8_e4m3", "e8m0", 32, "none"),
                                          "nvint8": ("int8", "e4m3", 16, "current"),
                                          "mxfp6_e2m3": ("fp6_e2m3", "e8m0", 32, "none"),
                                          "mxint6": ("int6", "e8m0", 32, "none")}.items():
        a = inputs.device_normal((m, k), 0.02, inputs.SEEDS["llama_a"], torch.bfloat16)
        w = inputs.device_normal((n, k), 0.02, inputs.SEEDS["llama_up"], torch.bfloat16)
        qa = fq.fp4_quantize(a, block, fmt, amax=pol, element=elem)
        qw = fq.fp4_quantize(w, block, fmt, amax=pol, element=elem)
        c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

        def rec_g(_):
            fq.fp4_gemm(qa, qw, out=c)
        gs = GraphSet(torch, 1, rec_g)
        ms = time_graphs(torch, gs, 10, 2)
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        res[f"{name}_gemm_up"] = {"M": m, "N": n, "K": k, "TFLOP/s": round(tf, 1), "ms": round(ms, 4),
                                  "frac_bf16_peak": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4),
                                  "frac_fp8_peak": round(tf / MFMA_PEAK_TFLOPS["fp8"], 4)}
        del a, w, qa, qw, c, gs
    res["workload"] = ("4096x4096 bf16 sweep tensor, E8M0 block 32, FP8 E4M3 / INT8 elements (1 byte each) and "
                       "FP6 E2M3 / FP6 E3M2 / INT6 elements (6 bits each), RTN, row-wise, column-wise and "
                       "both orientations (MXFP8, MXINT6); "
                       "Llama-2 7B up projection 8192x4096 @ 11008x4096, MXFP8 (in-register FP8 -> bf16), INT8 with "
                       "E4M3 block-16 scales (in-register INT8 -> f16), MXFP6 (E2M3) and MXINT6 (exact dequantize "
                       "path)")
    return res


def leg_wo(torch, fq, inputs):
    """Weight-only NVFP4 GEMM, W [N, K] = [18944, 3584] and [3584, 18944],
    M in {1, 8, 16}; 12 weight copies rotate (>= 450 MB) so weights stream
    from HBM."""
    res = {}
    for name, (n, k) in {"up": (18944, 3584), "down": (3584, 18944)}.items():
        w = inputs.device_normal((n, k), 0.02, inputs.SEEDS["decode_" + name], torch.bfloat16)
        qws = [fq.fp4_quantize(w, 16, "e4m3", amax="current") for _ in range(12)]
        del w
        for m in (1, 8, 16):
            x = inputs.device_normal((m, k), 1.0, 10 + m, torch.bfloat16)
            y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
            try:
                fq.fp4_wo_gemm(x, qws[0], out=y)
            except fq.Fp4Error as e:
                res[f"{name}_m{m}"] = {"error": str(e)}
                continue

            def rec(_):
                for q in qws:
                    fq.fp4_wo_gemm(x, q, out=y)
            gs = GraphSet(torch, 1, rec)
            ms = time_graphs(torch, gs, 20, 3) / len(qws)
            algo = n * k // 2 + n * k // 16 + 8 + m * k * 2 + m * n * 2
            gbs = algo / (ms * 1e-3) / 1e9
            res[f"{name}_m{m}"] = {"M": m, "N": n, "K": k, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                                   "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                                "kernel": "k_wo_gemm", "us_per_launch": round(ms * 1e3, 2),
                                                "algo_bytes_per_launch": algo, "traffic": None}}
        del qws
    return res


def leg_wo_wide(torch, fq, inputs):
    """Weight-only GEMM on the 8- and 6-bit grids with E8M0 block-32 scales
    (MXFP8, MXINT8, MXFP6 E2M3, MXINT6), W [18944, 3584] and [3584, 18944],
    M in {1, 16}; 6 weight copies rotate (>= 200 MB)."""
    res = {}
    for elem, name in (("fp8_e4m3", "mxfp8"), ("int8", "mxint8"), ("fp6_e2m3", "mxfp6_e2m3"), ("int6", "mxint6")):
        for proj, (n, k) in {"up": (18944, 3584), "down": (3584, 18944)}.items():
            w = inputs.device_normal((n, k), 0.02, inputs.SEEDS["decode_" + proj], torch.bfloat16)
            qws = [fq.fp4_quantize(w, 32, "e8m0", amax="none", element=elem) for _ in range(6)]
            del w
            for m in (1, 16):
                x = inputs.device_normal((m, k), 1.0, 10 + m, torch.bfloat16)
                y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

                def rec(_):
                    for q in qws:
                        fq.fp4_wo_gemm(x, q, out=y)
                gs = GraphSet(torch, 1, rec)
                ms = time_graphs(torch, gs, 20, 3) / len(qws)
                algo = n * k * fq.ELEMENT_BITS[elem] // 8 + n * k // 32 + 8 + m * k * 2 + m * n * 2
                gbs = algo / (ms * 1e-3) / 1e9
                res[f"{name}_{proj}_m{m}"] = {"us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                                              "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
                del gs
            del qws
    res["workload"] = ("Qwen-2.5 7B MLP decode shapes, weights quantized on the 8- and 6-bit grids with E8M0 "
                       "block-32 scales, bf16 X with M = 1 and 16")
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(min_seconds=10.0, one_thread_seconds=4.0):
    """The CPU oracle (as written, not tuned) on the whole sweep workload:
    full steps (the 4096x4096 tensor through all five formats) repeated
    until at least min_seconds have passed on min(16, usable cores) threads;
    then one thread on single E4M3 calls for about one_thread_seconds.  Same
    bytes accounting as the GPU step."""
    import numpy as np
    import oracle
    import fp4_inputs as inputs
    x = inputs.sweep()
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = min(16, usable)
    rows, cols = x.shape
    step_bytes = sum(quant_bytes(rows, cols, b) for _, b, _ in SWEEP)
    steps = 0
    t0 = time.perf_counter()
    while True:
        for fmt, block, pol in SWEEP:
            oracle.quantize_tensor(x, block, fmt, pol, nthreads=threads)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    calls = 0
    t1 = time.perf_counter()
    while True:
        oracle.quantize_tensor(x, 16, "e4m3", "current", nthreads=1)
        calls += 1
        dt1 = time.perf_counter() - t1
        if dt1 >= one_thread_seconds:
            break
    # the GEMM reference: both operands dequantized exactly in binary64, the
    # product and the tolerance matrix |A||W|^T (numpy's BLAS threads)
    ga = inputs.normal((1024, 4096), 0.02, inputs.SEEDS["llama_a"]).astype(np.float32)
    gw = inputs.normal((1024, 4096), 0.02, inputs.SEEDS["llama_up"]).astype(np.float32)
    t2 = time.perf_counter()
    qa_, sa_, g_a, _ = oracle.quantize_tensor(ga, 16, "e4m3", "current", nthreads=threads)
    qw_, sw_, g_w, _ = oracle.quantize_tensor(gw, 16, "e4m3", "current", nthreads=threads)
    a_hat = oracle.dequantize_f64(qa_, sa_, g_a, 16, "e4m3")
    w_hat = oracle.dequantize_f64(qw_, sw_, g_w, 16, "e4m3")
    oracle.gemm_ref(a_hat, w_hat)
    dt2 = time.perf_counter() - t2
    gflop = 2.0 * 1024 * 1024 * 4096 / 1e9
    return {"value": round(steps * step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full sweep steps (4096x4096 bf16, 5 formats) in {dt:.1f} s",
            "host_cores_usable": usable, "host_cores_total": os.cpu_count(), "cpu_model": _cpu_model(),
            "one_thread": {"value": round(calls * quant_bytes(rows, cols, 16) / dt1 / 1e9, 4), "unit": "GB/s",
                           "sample": f"{calls} E4M3 block-16 calls on the sweep tensor in {dt1:.1f} s"},
            "gemm_oracle": {"value": round(gflop / dt2, 3), "unit": "GFLOP/s",
                            "sample": f"NVFP4 1024x4096 @ (1024x4096)^T: quantize, binary64 dequantize, product "
                                      f"and |A||W|^T tolerance in {dt2:.2f} s ({gflop:.1f} GFLOP of the product)"}}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import fp4_block_scaled_quantize_amd as fq
    import fp4_inputs as inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    rows = cols = 4096
    base = inputs.device_outliers(inputs.device_normal((rows, cols), 0.02, inputs.SEEDS["sweep"], torch.bfloat16),
                                  0.001, 100.0, inputs.SEEDS["sweep"])
    xs = [base.clone() for _ in range(args.rot)]
    states = [fq.AmaxState(1) for _ in SWEEP]
    outs = {f: [fq.QTensor.empty(rows, cols, b, f, amax=p) for _ in range(args.rot)] for f, b, p in SWEEP}

    def step(i):
        for (f, b, p), st in zip(SWEEP, states):
            fq.fp4_quantize(xs[i], b, f, amax=p, state=st if p != "none" else None, out=outs[f][i])
    gs = GraphSet(torch, args.rot, step)
    for i in range(args.warmup):
        gs.replay(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        gs.replay(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    step_bytes = sum(quant_bytes(rows, cols, b) for _, b, _ in SWEEP)
    value = step_bytes / (ms * 1e-3) / 1e9

    # quantization error per format on the sweep tensor (fp64 mean squared
    # error of the dequantized tensor; gonzo_ML/3986 "Форматы FP4" compares
    # the scale encodings by the loss they reach)
    mse = {}
    ref = xs[0].double()
    for f, b, p in SWEEP:
        y = fq.fp4_dequantize(outs[f][0], torch.float32)
        mse[f"{f}_b{b}"] = float(((y.double() - ref) ** 2).mean())
    del ref, y

    roof = leg_roofline(torch, fq, xs)
    if args.copy_probe:
        # torch's elementwise copy kernel: 64 MiB read, 64 MiB written
        src = torch.ones(32 * 2**20, dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            dst = src.clone()
        torch.cuda.synchronize()
        del src, dst
    legs = {}
    want = [] if args.legs == "none" else args.legs.split(",")
    if "small" in want:
        legs["small_nvfp4_256x256"] = leg_small_nvfp4(torch, fq, inputs)
    if "gemmsmall" in want:
        legs["gemm_small_products"] = leg_gemm_small(torch, fq, inputs)
    if "dequant" in want:
        legs["dequant"] = leg_dequant(torch, fq, xs[:8])
    if "rht" in want:
        legs["rht"] = leg_rht(torch, fq, xs[:8])
    if "int4" in want:
        legs["int4"] = leg_int4(torch, fq, inputs, xs[:8])
        torch.cuda.empty_cache()
    if "w8" in want:
        legs["mx8"] = leg_8bit(torch, fq, inputs, xs[:8])
        torch.cuda.empty_cache()
    del outs
    if "sr" in want:
        legs["sr_delayed"] = leg_sr(torch, fq, inputs, args.steps)
        torch.cuda.empty_cache()
    if "srt" in want:
        legs["transposed_delayed"] = leg_sr_transposed(torch, fq, inputs, args.steps)
        torch.cuda.empty_cache()
    if "gemm" in want:
        legs["gemm_llama2_7b"] = leg_gemm(torch, fq, inputs)
        torch.cuda.empty_cache()
    if "wo" in want:
        legs["wo_gemm_qwen25"] = leg_wo(torch, fq, inputs)
        torch.cuda.empty_cache()
    if "wowide" in want:
        legs["wo_gemm_qwen25_wide_grids"] = leg_wo_wide(torch, fq, inputs)
    cpu = None if args.no_cpu_baseline else cpu_baseline()

    line = {"metric": "FP4 quantize GB/s (% HBM peak); block-scaled FP4 GEMM TFLOP/s (% MFMA peak)",
            "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "wall_s": round(wall, 3), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16->e2m1 (fp32 decisions)", "data": "synthetic",
            "frac_hbm": round(value / HBM_PEAK_GBS, 4),
            "config": {"workload": "scale-format sweep: 4096x4096 bf16 N(0,0.02)+0.1% x100 outliers; "
                                   "E4M3/UE5M3/E3M4/E1M6 block 16 (current amax) + E8M0 block 32, RTN",
                       "rows": rows, "cols": cols, "formats": [f for f, _, _ in SWEEP],
                       "rotating_inputs": args.rot, "bytes_per_step": step_bytes},
            "quantization_mse": mse, "roofline": roof, "cpu_baseline": cpu, "legs": legs}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
