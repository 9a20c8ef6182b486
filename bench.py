"""Benchmark of the sparse FP8 row-wise linear layer on one MI355X.

A step is one forward pass of the layer over one batch: dynamic row-wise FP8
quantization of the bf16 activation, then the 2:4 sparse FP8 GEMM with its
fused scale/bias/bf16 epilogue.  The weight is prepared (row-wise FP8
quantization + 2:4 compression) once, before timing, as a linear layer's
weight is; its cost is timed separately and reported as ``weight_prep_ms``.

Workload (headline): Llama-3.1-8B MLP up-projection at prefill,
M=8192 tokens, K=4096, N=14336, e4m3 x e4m3, bf16 output, synthetic seeded
inputs.  ``value`` is dense-equivalent TFLOP/s (2*M*N*K per step).  The
decode-shaped secondary metric (GB/s at M in {1,4,16}, and batched decode at M in {32,64}; K=N=4096, bf16 bias)
is reported under ``decode``; those calls rotate over enough distinct weight
buffers (> 2x the 256 MB last-level cache) that every call reads HBM.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
SETTLE_S = 0.5                    # untimed sustained load before the warmup steps
PEAK_FP8_TFLOPS = 5000.0          # dense FP8 MFMA, MI355X
PEAK_FP8_SPARSE_TFLOPS = 10000.0  # 2:4 sparse FP8 MFMA (dense-equivalent), MI355X


def gemm_bytes(m, n, k, bias, out_bytes=2):
    """Algorithmic bytes of one linear call: compressed weight + metadata +
    activation codes + scales (+ bias) + output."""
    return n * k // 2 + n * k // 8 + m * k + 4 * m + 4 * n + (2 * n if bias else 0) + out_bytes * m * n


def quant_bytes(m, k):
    return 3 * m * k + 4 * m


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--no-decode", action="store_true", help="skip the decode-shaped GB/s measurement")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-algo-search", action="store_true", help="skip the per-shape kernel configuration search")
    p.add_argument("--no-bsr", action="store_true", help="skip the block-sparse (BSR) decode measurement")
    p.add_argument("--cpu-rows", type=int, default=160, help="activation rows in the CPU oracle sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain device copy of known size (for scaling HBM byte counters) and exit")
    return p.parse_args()


# Kernel sources whose hash tags the stored HBM-traffic measurement: once any of
# them changes, the stored figure no longer describes the kernel and is not reported.
TRAFFIC_SOURCES = ("sparse_fp8_row_amd/csrc/gemm.hip", "sparse_fp8_row_amd/csrc/sfr_device.hpp",
                   "sparse_fp8_row_amd/csrc/sfr_launch.hpp")
TRAFFIC_FILE = "profiles/traffic_linear_prefill_up.txt"
# the kernel behind each configuration the prefill workload can take
ALGO_KERNELS = {2: "linear_tiled_kernel (64x64 tile, 4 wavefronts)", 3: "linear_tiled_kernel (128x128 tile, 4 wavefronts)",
                4: "linear_persistent_kernel (256x256 tile, 8 wavefronts, one workgroup per CU)",
                5: "linear_wide_kernel (256x256 tile, 4 wavefronts)"}
COPY_BYTES = 1 << 30


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the prefill GEMM from the stored counter summary,
    or None if it is absent or was taken on different kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0].strip() in ("kernel_source_sha256", "traffic_bytes_per_launch"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def calibrate_copy():
    """A plain device-to-device copy of COPY_BYTES, five times: the reference
    against which the FETCH_SIZE / WRITE_SIZE counters are scaled."""
    import torch
    src = torch.randint(0, 255, (COPY_BYTES,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus}: multi-GPU runs are not implemented "
              "(the layer would shard along N, with no communication)", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch
    import sfr_inputs
    import sparse_fp8_row_amd as sfr

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sfr.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    case = sfr_inputs.prefill_up_case()
    M, N, K = case.m, case.n, case.k
    x = to_dev(sfr_inputs.draw_x(case))
    w = to_dev(sfr_inputs.draw_w(case))
    print(f"[bench] {case.name}: inputs resident", file=sys.stderr, flush=True)

    # weight preparation (once per weight), timed on its own
    for _ in range(2):
        pw = sfr.prepare_weight(w, torch.float8_e4m3fn)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    reps = 5
    for _ in range(reps):
        pw = sfr.prepare_weight(w, torch.float8_e4m3fn)
    e1.record(stream)
    torch.cuda.synchronize()
    prep_ms = e0.elapsed_time(e1) / reps

    xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    xs = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    lib = sfr.load()
    h = int(stream.cuda_stream)

    def quant():
        st = lib.quantize_rowwise_fp8(x.data_ptr(), M, K, sfr.SFR_E4M3, xq.data_ptr(), xs.data_ptr(), h)
        assert st == 0, st

    def gemm():
        st = lib.sparse_fp8_rowwise_linear(xq.data_ptr(), sfr.SFR_E4M3, xs.data_ptr(), M, K, pw.values.data_ptr(),
                                           pw.meta.data_ptr(), sfr.SFR_E4M3, pw.scale.data_ptr(), N, None,
                                           out.data_ptr(), sfr.SFR_OUT_BF16, h)
        assert st == 0, st

    # The GPU's clocks take a few hundred milliseconds of sustained load to
    # settle (the GEMM's duration falls by about a quarter over its first ~80
    # calls), so the step runs untimed for SETTLE_S before the warmup steps.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(20):
            quant()
            gemm()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        quant()
        gemm()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        quant()
        evs[i][1].record(stream)
        gemm()
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    g_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    step_ms = evs[0][0].elapsed_time(evs[-1][2]) / args.steps
    print(f"[bench] timed {args.steps} steps: step {step_ms:.4f} ms (quantize {q_ms:.4f}, gemm {g_ms:.4f}), "
          f"host wall {wall * 1e3 / args.steps:.4f} ms/step", file=sys.stderr, flush=True)

    flops = 2.0 * M * N * K
    value = flops / (step_ms * 1e-3) / 1e12
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    result = {
        "metric": "sparse FP8 linear TFLOP/s (dense-equiv) @M=8192 K=4096 N=14336; GB/s @M=1..16",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic (seeded; Llama-3.1-8B up-proj shape)",
        "config": {"workload": "prefill_up: quantize bf16 X[8192,4096] + 2:4 sparse FP8 linear N=14336, "
                               "e4m3 x e4m3, bf16 out, no bias",
                   "m": M, "n": N, "k": K, "x_dtype": "e4m3", "w_dtype": "e4m3", "out_dtype": "bf16",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": ALGO_KERNELS.get(sfr.default_algo(M, N, K), "?"),
                     "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "frac_of_sparse_peak": round(gemm_tflops / PEAK_FP8_SPARSE_TFLOPS, 4),
                     "traffic": stored_traffic()},
        "kernels_ms": {"quantize": round(q_ms, 5), "gemm": round(g_ms, 5)},
        "quantize_gbs": round(quant_bytes(M, K) / (q_ms * 1e-3) / 1e9, 1),
        "weight_prep_ms": round(prep_ms, 4),
        "clock_settle_s": SETTLE_S,
    }
    result["tensorwise"] = bench_tensorwise(torch, sfr, lib, w, x, M, N, K, h, stream)
    del xq, xs, out

    if not args.no_decode:
        result["decode"] = bench_decode(torch, sfr, sfr_inputs, lib, dev, stream)

    if not args.no_bsr:
        result["bsr_decode"] = bench_bsr(torch, sfr, sfr_inputs, dev)

    if not args.no_algo_search:
        result["algo_search"] = bench_algo_search()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_rows)
    print(json.dumps(result), flush=True)


def bench_tensorwise(torch, sfr, lib, w, x, M, N, K, h, stream, steps=20, warmup=10):
    """The same prefill step with tensor-wise scales: quantize_tensorwise_fp8
    (two launches) + the linear layer with one activation and one weight scale."""
    pw = sfr.prepare_weight(w, torch.float8_e4m3fn, scaling="tensor")
    xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=x.device)
    xs = torch.empty((1,), dtype=torch.float32, device=x.device)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    nbytes = int(lib.sfr_quantize_tensorwise_workspace_bytes(M, K))
    work = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=x.device)

    def quant():
        st = lib.quantize_tensorwise_fp8(x.data_ptr(), M, K, sfr.SFR_E4M3, xq.data_ptr(), xs.data_ptr(),
                                         work.data_ptr(), nbytes, h)
        assert st == 0, st

    def gemm():
        st = lib.sparse_fp8_scaled_linear(xq.data_ptr(), sfr.SFR_E4M3, xs.data_ptr(), sfr.SFR_SCALE_TENSOR, M, K,
                                          pw.values.data_ptr(), pw.meta.data_ptr(), sfr.SFR_E4M3, pw.scale.data_ptr(),
                                          sfr.SFR_SCALE_TENSOR, N, None, out.data_ptr(), sfr.SFR_OUT_BF16, h)
        assert st == 0, st

    for _ in range(warmup):
        quant()
        gemm()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        quant()
        evs[i][1].record(stream)
        gemm()
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    q_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    g_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    step_ms = evs[0][0].elapsed_time(evs[-1][2]) / steps
    print(f"[bench] tensorwise: step {step_ms:.4f} ms (quantize {q_ms:.4f}, gemm {g_ms:.4f})", file=sys.stderr,
          flush=True)
    return {"steps": steps, "warmup": warmup, "ms_per_step": round(step_ms, 5),
            "TFLOP/s": round(2.0 * M * N * K / (step_ms * 1e-3) / 1e12, 2),
            "kernels_ms": {"quantize_tensorwise": round(q_ms, 5), "gemm": round(g_ms, 5)},
            "quantize_gbs": round(quant_bytes(M, K) / (q_ms * 1e-3) / 1e9, 1)}


def bsr_bytes(m, n, k, nnz, bias):
    """Algorithmic bytes of one BSR linear call: kept blocks, their column
    indices, the block-row pointers, bf16 activation and output (and bias)."""
    return nnz * 64 * 64 * 2 + 4 * nnz + 4 * (n // 64 + 1) + 2 * m * k + 2 * m * n + (2 * n if bias else 0)


def bench_bsr(torch, sfr, sfr_inputs, dev):
    """Block-sparse (64 x 64 blocks, sparsity 0.9) bf16 decode at M in {1, 4, 16}
    on the Llama-3.1-8B o-projection (N = K = 4096) and up-projection
    (N = 14336, K = 4096) shapes, bf16 bias: per call from a HIP graph,
    rotating over >= 600 MB of weight copies; beside it the dense bf16 layer
    (torch.matmul, same rotation and graph timing) as the reference the pages
    compare against."""
    from sparse_fp8_row_amd import tune
    res = {}
    for shape in ("o", "up"):
        n, k = sfr_inputs.LLAMA_SHAPES[shape]
        case = sfr_inputs.Case("bsr_bench", 30, 16, n, k, bias=True)
        wb = sfr_inputs.draw_bsr_w(case)
        w = torch.from_numpy(wb.view(np.int16)).to(dev).view(torch.bfloat16)
        base = sfr.bsr_from_dense(w)
        bias = torch.from_numpy(sfr_inputs.draw_bias(case).view(np.int16)).to(dev).view(torch.bfloat16)
        per = base.values.numel() * 2
        copies = max(2, int(np.ceil(600e6 / max(per, 1))))
        weights = [base] + [sfr.BsrWeight(base.crow, base.col, base.values.clone(), n, k) for _ in range(copies - 1)]
        dcopies = max(2, int(np.ceil(600e6 / (2 * n * k))))
        wt = w.t().contiguous()  # [K, N]: the dense product takes a contiguous right operand
        dense = [wt] + [wt.clone() for _ in range(dcopies - 1)]
        for m in (1, 4, 16):
            x = torch.from_numpy(sfr_inputs.draw_x(sfr_inputs.Case("bsr_bench", 30, m, n, k)).view(np.int16)) \
                .to(dev).view(torch.bfloat16)
            out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            lib = sfr.load()

            def call(i, hs):
                bw = weights[i]
                st = lib.bsr_linear_bf16(x.data_ptr(), m, k, bw.crow.data_ptr(), bw.col.data_ptr(),
                                         bw.values.data_ptr(), n, bias.data_ptr(), out.data_ptr(), sfr.SFR_OUT_BF16, hs)
                assert st == 0, st

            dout = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

            def dcall(i, hs):
                torch.addmm(bias, x, dense[i], out=dout)

            us = tune.graph_us(call, copies, calls=2 * copies)
            dus = tune.graph_us(dcall, dcopies, calls=2 * dcopies)
            b = bsr_bytes(m, n, k, base.nnz, True)
            gbs = b / (us * 1e-6) / 1e9
            res[f"{shape}_M{m}"] = {"us_per_call": round(us, 3), "bytes": b, "GB/s": round(gbs, 1),
                                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "nnz_blocks": base.nnz,
                                    "dense_bf16_torch_us": round(dus, 3), "speedup_vs_dense": round(dus / us, 2)}
            print(f"[bench] bsr {shape} M={m}: {us:.3f} us/call ({gbs:.1f} GB/s), dense bf16 (torch) {dus:.3f} us, "
                  f"x{dus / us:.2f}", file=sys.stderr, flush=True)
        del weights, dense, wt
    return res


def bench_algo_search():
    """Per-shape kernel configuration search (sparse_fp8_row_amd.tune) over the
    Llama-3.1-8B layer shapes at M in {16, 512, 8192}, e4m3 x e4m3: the
    built-in choice against the fastest configuration."""
    from sparse_fp8_row_amd import tune
    import sfr_inputs
    shapes = [(m, n, k) for (n, k) in sfr_inputs.LLAMA_SHAPES.values() for m in (16, 512, 8192)]
    res = tune.search(shapes, reps=10, warmup=2)
    out = {}
    for r in res["timings"]:
        key = f"M{r['m']}N{r['n']}K{r['k']}"
        out[key] = {"default": r["default"], "default_us": r["default_us"], "best": r["best"], "best_us": r["best_us"],
                    "us": r["us"]}
        print(f"[bench] algo {key}: default {r['default']} {r['default_us']} us, best {r['best']} {r['best_us']} us",
              file=sys.stderr, flush=True)
    return out


def bench_decode(torch, sfr, sfr_inputs, lib, dev, stream):
    """GEMM GB/s at M in {1,4,16} (and 32, 64: batched decode), K=N=4096, bf16 bias, rotating weights (> 512 MB);
    per-call times from a HIP graph of the calls (the eager loop's rate too)."""
    from sparse_fp8_row_amd import tune
    res = {}
    n, k = 4096, 4096
    case0 = sfr_inputs.decode_cases()[0]
    wb = sfr_inputs.draw_w(case0)
    bb = sfr_inputs.draw_bias(case0)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    w = to_dev(wb)
    bias = to_dev(bb)
    base = sfr.prepare_weight(w, torch.float8_e4m3fn)
    per = n * k // 2 + n * k // 8
    copies = int(np.ceil(600e6 / per))
    vals = [base.values.clone() for _ in range(copies)]
    metas = [base.meta.clone() for _ in range(copies)]
    h = int(stream.cuda_stream)
    for case in sfr_inputs.decode_cases():
        m = case.m
        x = to_dev(sfr_inputs.draw_x(case))
        xq, xs = sfr.quantize_rowwise_fp8(x, torch.float8_e4m3fn)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

        def call(i, hs=h):
            st = lib.sparse_fp8_rowwise_linear(xq.data_ptr(), sfr.SFR_E4M3, xs.data_ptr(), m, k,
                                               vals[i].data_ptr(), metas[i].data_ptr(), sfr.SFR_E4M3,
                                               base.scale.data_ptr(), n, bias.data_ptr(), out.data_ptr(),
                                               sfr.SFR_OUT_BF16, hs)
            assert st == 0, st

        for i in range(copies):
            call(i)
        torch.cuda.synchronize()
        reps = 4 * copies
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            call(i % copies)
        e1.record(stream)
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / reps
        # the same calls replayed from a HIP graph: the GPU's own rate (an
        # eager loop of few-microsecond launches is paced by the host)
        us = tune.graph_us(call, copies, calls=2 * copies)
        b = gemm_bytes(m, n, k, True)
        gbs = b / (us * 1e-6) / 1e9
        res[f"M{m}"] = {"us_per_call": round(us, 3), "bytes": b, "GB/s": round(gbs, 1),
                        "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "eager_us_per_call": round(eager_us, 3)}
        print(f"[bench] decode M={m}: {us:.3f} us/call in a graph ({eager_us:.3f} eager), {gbs:.1f} GB/s",
              file=sys.stderr, flush=True)

        # the layer from the bf16 activation: quantization + GEMM as two
        # launches, and fused into one (sparse_fp8_rowwise_linear_dynamic)
        xq2 = torch.empty_like(xq)
        xs2 = torch.empty_like(xs)

        def two(i, hs=h):
            st = lib.quantize_rowwise_fp8(x.data_ptr(), m, k, sfr.SFR_E4M3, xq2.data_ptr(), xs2.data_ptr(), hs)
            assert st == 0, st
            st = lib.sparse_fp8_rowwise_linear(xq2.data_ptr(), sfr.SFR_E4M3, xs2.data_ptr(), m, k,
                                               vals[i].data_ptr(), metas[i].data_ptr(), sfr.SFR_E4M3,
                                               base.scale.data_ptr(), n, bias.data_ptr(), out.data_ptr(),
                                               sfr.SFR_OUT_BF16, hs)
            assert st == 0, st

        def fused(i, hs=h):
            st = lib.sparse_fp8_rowwise_linear_dynamic(x.data_ptr(), sfr.SFR_E4M3, m, k, vals[i].data_ptr(),
                                                       metas[i].data_ptr(), sfr.SFR_E4M3, base.scale.data_ptr(),
                                                       sfr.SFR_SCALE_ROW, n, bias.data_ptr(), out.data_ptr(),
                                                       sfr.SFR_OUT_BF16, xq2.data_ptr(), xs2.data_ptr(), hs)
            assert st == 0, st

        for name, fn in (("quantize_plus_gemm", two), ("fused", fused)):
            t = tune.graph_us(fn, copies, calls=2 * copies)
            res[f"M{m}"][f"{name}_us_per_call"] = round(t, 3)
            print(f"[bench] decode M={m} from bf16, {name}: {t:.3f} us/call in a graph", file=sys.stderr, flush=True)
    return res


def cpu_baseline(case, rows):
    """The CPU oracle on a bounded sample of the same workload: quantize `rows`
    activation rows, and evaluate the linear layer for those rows and all N
    outputs (the weight's quantization and compression are not timed)."""
    import oracle
    import sfr_inputs
    t_prep = time.perf_counter()
    xb = sfr_inputs.draw_x(case)[:rows]
    wb = sfr_inputs.draw_w(case)
    v, m, ws, _ = oracle.prepare_weight(wb, oracle.E4M3)
    t_prep = time.perf_counter() - t_prep
    t0 = time.perf_counter()
    xq, xs = oracle.quantize_rows(xb, oracle.E4M3)
    oracle.linear(xq, oracle.E4M3, xs, v, m, oracle.E4M3, ws)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * case.n * case.k
    print(f"[bench] cpu oracle: {rows} rows in {dt:.2f} s", file=sys.stderr, flush=True)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{rows} of {case.m} activation rows x all N={case.n} outputs, K={case.k} "
                      f"(activation quantization + linear; {dt:.1f} s)"}


if __name__ == "__main__":
    main()
