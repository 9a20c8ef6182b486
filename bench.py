"""Benchmark of the sparse FP8 row-wise linear layer on one MI355X.

A step is one forward pass of the layer over one batch: dynamic row-wise FP8
quantization of the bf16 activation, then the 2:4 sparse FP8 GEMM with its
fused scale/bias/bf16 epilogue.  The weight is prepared (2:4 pruning of the
bf16 weight, row-wise FP8 quantization, compression) once, before timing, as a
linear layer's weight is; its cost is timed separately (``weight_prep_ms``).

Workload (headline): Llama-3.1-8B MLP up-projection at prefill, M=8192
tokens, K=4096, N=14336, e4m3 x e4m3, bf16 output, synthetic seeded inputs,
with the library's built-in algorithm (binary32-grade accumulation).
``value`` is dense-equivalent TFLOP/s (2*M*N*K per step).  The same step with
FP8 matrix-instruction accumulation is reported under ``fast_accumulation``.

``decode`` holds the decode-shaped metric: GB/s of the GEMM at M in {1, 4, 16}
on the four Llama-3.1-8B layer shapes (and batched decode M in {32, 64} on the
4096 x 4096 one), both accumulations, and the layer from the bf16 activation
(``sparse_fp8_rowwise_linear_dynamic``).  Those calls are replayed from a HIP
graph and rotate over enough distinct weight buffers (> 2x the 256 MB
last-level cache) that every call reads HBM.

Prints one JSON line.  ``--profile prefill|decode`` only runs a few calls of
the kernels for a counter run (no JSON line).
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
PEAK_FP8_TFLOPS = 5000.0          # dense FP8 matrix instructions, MI355X
PEAK_BF16_TFLOPS = 2500.0         # dense bf16 matrix instructions, MI355X


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
    p.add_argument("--no-tensorwise", action="store_true", help="skip the tensor-wise scaled prefill step")
    p.add_argument("--profile", choices=("prefill", "decode"),
                   help="only run a few calls of the prefill or decode kernels (for counter runs) and exit")
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
    """HBM bytes per launch of the prefill GEMM ({"default": .., "f8acc": ..})
    from the stored counter summary; empty if it is absent or was taken on
    different kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return {}
    keys = {"traffic_bytes_per_launch": "default", "traffic_bytes_per_launch_f8acc": "f8acc"}
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return {}
    out = {}
    for k, name in keys.items():
        try:
            out[name] = int(float(fields[k]))
        except (KeyError, ValueError):
            pass
    return out


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


def prefill_inputs(torch, sfr, sfr_inputs, dev):
    case = sfr_inputs.prefill_up_case()
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    x = to_dev(sfr_inputs.draw_x(case))
    w = to_dev(sfr_inputs.draw_w(case))
    return case, x, w


class PrefillStep:
    """One step of the prefill workload: row-wise quantization of X, then the
    linear layer with the given algorithm id, both on `stream`."""

    def __init__(self, torch, sfr, lib, x, pw, m, n, k, stream):
        self.torch, self.sfr, self.lib = torch, sfr, lib
        self.x, self.pw, self.m, self.n, self.k = x, pw, m, n, k
        self.stream, self.h = stream, int(stream.cuda_stream)
        self.xq = torch.empty((m, k), dtype=torch.float8_e4m3fn, device=x.device)
        self.xs = torch.empty((m,), dtype=torch.float32, device=x.device)
        self.out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)

    def quant(self):
        st = self.lib.quantize_rowwise_fp8(self.x.data_ptr(), self.m, self.k, self.sfr.SFR_E4M3, self.xq.data_ptr(),
                                           self.xs.data_ptr(), self.h)
        assert st == 0, st

    def gemm(self, algo):
        sfr, pw = self.sfr, self.pw
        st = self.lib.sparse_fp8_scaled_linear_algo(self.xq.data_ptr(), sfr.SFR_E4M3, self.xs.data_ptr(),
                                                    sfr.SFR_SCALE_ROW, self.m, self.k, pw.values.data_ptr(),
                                                    pw.meta.data_ptr(), sfr.SFR_E4M3, pw.scale.data_ptr(),
                                                    sfr.SFR_SCALE_ROW, self.n, None, self.out.data_ptr(),
                                                    sfr.SFR_OUT_BF16, algo, self.h)
        assert st == 0, st

    def settle(self, algo, seconds=SETTLE_S):
        # The GPU's clocks take a few hundred milliseconds of sustained load
        # to settle (the GEMM's duration falls by about a quarter over its
        # first ~80 calls), so the step runs untimed first.
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                self.quant()
                self.gemm(algo)
            self.torch.cuda.synchronize()

    def timed(self, algo, steps, warmup):
        """Mean ms of the step, of the quantization and of the GEMM, from HIP
        events recorded on the launch stream around each kernel."""
        torch = self.torch
        for _ in range(warmup):
            self.quant()
            self.gemm(algo)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            evs[i][0].record(self.stream)
            self.quant()
            evs[i][1].record(self.stream)
            self.gemm(algo)
            evs[i][2].record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        q_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        g_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
        step_ms = evs[0][0].elapsed_time(evs[-1][2]) / steps
        return step_ms, q_ms, g_ms, wall * 1e3 / steps


def mfma_roofline(m, n, k, g_ms, peak, kernel, traffic):
    """Roofline of the GEMM: the method's own work is M*N*K/2 multiply-adds
    (the kept half of the products), i.e. M*N*K flops, against the dense peak
    of the matrix instructions that run (a 2:4 sparse instruction retires its
    kept products at the dense instruction's rate)."""
    own = float(m) * n * k / (g_ms * 1e-3) / 1e12
    dense_eq = 2.0 * own
    return {"bound": "mfma", "kernel": kernel, "achieved": round(own, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(own / peak, 4), "traffic": traffic,
            "achieved_dense_equiv": round(dense_eq, 2),
            "frac_dense_equiv_of_fp8_dense_peak": round(dense_eq / PEAK_FP8_TFLOPS, 4)}


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
    lib = sfr.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    if args.profile == "decode":
        profile_decode(torch, sfr, sfr_inputs, lib, dev, stream)
        return

    case, x, w = prefill_inputs(torch, sfr, sfr_inputs, dev)
    M, N, K = case.m, case.n, case.k
    print(f"[bench] {case.name}: inputs resident", file=sys.stderr, flush=True)

    # weight preparation (once per weight: prune, row quantization, compression), timed on its own
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

    step = PrefillStep(torch, sfr, lib, x, pw, M, N, K, stream)
    dflt = sfr.default_algo(M, N, K)
    fast = dflt | sfr.SFR_ALGO_ACC_F8
    names = dict(sfr.linear_algos())

    if args.profile == "prefill":
        # a few steps of each accumulation, for counter runs
        step.settle(dflt)
        for algo in (dflt, fast):
            print(f"[profile] prefill {names[algo]}: 3 steps", file=sys.stderr, flush=True)
            for _ in range(3):
                step.quant()
                step.gemm(algo)
            torch.cuda.synchronize()
        return

    step.settle(dflt)
    step_ms, q_ms, g_ms, wall_ms = step.timed(dflt, args.steps, args.warmup)
    print(f"[bench] {names[dflt]}: timed {args.steps} steps: step {step_ms:.4f} ms (quantize {q_ms:.4f}, "
          f"gemm {g_ms:.4f}), host wall {wall_ms:.4f} ms/step", file=sys.stderr, flush=True)
    step.settle(fast)
    f_step, f_q, f_g, _ = step.timed(fast, args.steps, args.warmup)
    print(f"[bench] {names[fast]}: step {f_step:.4f} ms (quantize {f_q:.4f}, gemm {f_g:.4f})", file=sys.stderr,
          flush=True)

    flops = 2.0 * M * N * K
    value = flops / (step_ms * 1e-3) / 1e12
    traffic = stored_traffic()
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
        "dtype": "e4m3 operands, bf16 matrix instructions (exact widening), binary32 accumulation",
        "data": "synthetic (seeded; Llama-3.1-8B up-proj shape)",
        "config": {"workload": "prefill_up: quantize bf16 X[8192,4096] + 2:4 sparse FP8 linear N=14336, "
                               "e4m3 x e4m3, bf16 out, no bias",
                   "m": M, "n": N, "k": K, "x_dtype": "e4m3", "w_dtype": "e4m3", "out_dtype": "bf16",
                   "algo": names[dflt], "parallelism": "single GPU"},
        "roofline": mfma_roofline(M, N, K, g_ms, PEAK_BF16_TFLOPS, ALGO_KERNELS.get(dflt & 0xFF, "?"),
                                  traffic.get("default")),
        "kernels_ms": {"quantize": round(q_ms, 5), "gemm": round(g_ms, 5)},
        "quantize_gbs": round(quant_bytes(M, K) / (q_ms * 1e-3) / 1e9, 1),
        "weight_prep_ms": round(prep_ms, 4),
        "clock_settle_s": SETTLE_S,
        "fast_accumulation": {
            "algo": names[fast],
            "accuracy": "FP8 matrix-instruction accumulation (products of one instruction summed in fixed point "
                        "13 bits below the largest): outside the binary32 bound on cancelling inputs",
            "ms_per_step": round(f_step, 5), "TFLOP/s": round(flops / (f_step * 1e-3) / 1e12, 2),
            "kernels_ms": {"quantize": round(f_q, 5), "gemm": round(f_g, 5)},
            "roofline": mfma_roofline(M, N, K, f_g, PEAK_FP8_TFLOPS, ALGO_KERNELS.get(fast & 0xFF, "?"),
                                      traffic.get("f8acc")),
        },
    }
    if not args.no_tensorwise:
        result["tensorwise"] = bench_tensorwise(torch, sfr, lib, w, x, M, N, K, int(stream.cuda_stream), stream)
    del step

    if not args.no_decode:
        result["decode"] = bench_decode(torch, sfr, sfr_inputs, lib, dev)

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


# Decode-shaped workloads: the 4096 x 4096 o-projection as the decode
# configuration (M in {1, 4, 16}, bf16 bias; batched decode M in {32, 64}),
# and the qkv, up and down projections of the layer sweep (seed 0, no bias).
DECODE_SHAPES = (("o", (1, 2, 4, 16, 32, 64)), ("qkv", (1, 2, 4, 16)), ("up", (1, 2, 4, 16)), ("down", (1, 2, 4, 16)))


def decode_case(sfr_inputs, shape, m):
    n, k = sfr_inputs.LLAMA_SHAPES[shape]
    if shape == "o":
        return sfr_inputs.Case("decode", 2, m, n, k, bias=True)
    return sfr_inputs.Case("sweep", 5, m, n, k)


class DecodeLayer:
    """One decode-shaped layer: the prepared weight in `copies` copies (the
    calls rotate over them), its bias, and per-M activations."""

    def __init__(self, torch, sfr, sfr_inputs, lib, dev, shape, rotate_bytes, min_copies=2):
        self.torch, self.sfr, self.sfr_inputs, self.lib, self.dev = torch, sfr, sfr_inputs, lib, dev
        self.shape = shape
        self.n, self.k = sfr_inputs.LLAMA_SHAPES[shape]
        case = decode_case(sfr_inputs, shape, 1)
        to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        self.to_dev = to_dev
        self.has_bias = case.bias
        self.bias = to_dev(sfr_inputs.draw_bias(case)) if case.bias else None
        self.base = sfr.prepare_weight(to_dev(sfr_inputs.draw_w(case)), torch.float8_e4m3fn)
        per = self.n * self.k // 2 + self.n * self.k // 8
        self.copies = max(min_copies, int(np.ceil(rotate_bytes / per)))
        self.vals = [self.base.values] + [self.base.values.clone() for _ in range(self.copies - 1)]
        self.metas = [self.base.meta] + [self.base.meta.clone() for _ in range(self.copies - 1)]

    def activation(self, m):
        torch, sfr = self.torch, self.sfr
        x = self.to_dev(self.sfr_inputs.draw_x(decode_case(self.sfr_inputs, self.shape, m)))
        xq, xs = sfr.quantize_rowwise_fp8(x, torch.float8_e4m3fn)
        out = torch.empty((m, self.n), dtype=torch.bfloat16, device=self.dev)
        return x, xq, xs, out, torch.empty_like(xq), torch.empty_like(xs)

    def gemm(self, i, hs, m, xq, xs, out, algo):
        sfr = self.sfr
        st = self.lib.sparse_fp8_scaled_linear_algo(
            xq.data_ptr(), sfr.SFR_E4M3, xs.data_ptr(), sfr.SFR_SCALE_ROW, m, self.k, self.vals[i].data_ptr(),
            self.metas[i].data_ptr(), sfr.SFR_E4M3, self.base.scale.data_ptr(), sfr.SFR_SCALE_ROW, self.n,
            self.bias.data_ptr() if self.has_bias else None, out.data_ptr(), sfr.SFR_OUT_BF16, algo, hs)
        assert st == 0, st

    def dynamic(self, i, hs, m, x, xq, xs, out):
        sfr = self.sfr
        st = self.lib.sparse_fp8_rowwise_linear_dynamic(
            x.data_ptr(), sfr.SFR_E4M3, m, self.k, self.vals[i].data_ptr(), self.metas[i].data_ptr(), sfr.SFR_E4M3,
            self.base.scale.data_ptr(), sfr.SFR_SCALE_ROW, self.n, self.bias.data_ptr() if self.has_bias else None,
            out.data_ptr(), sfr.SFR_OUT_BF16, xq.data_ptr(), xs.data_ptr(), hs)
        assert st == 0, st

    def quantize(self, hs, m, x, xq, xs):
        st = self.lib.quantize_rowwise_fp8(x.data_ptr(), m, self.k, self.sfr.SFR_E4M3, xq.data_ptr(), xs.data_ptr(),
                                           hs)
        assert st == 0, st


def bench_decode(torch, sfr, sfr_inputs, lib, dev):
    """GEMM GB/s on the decode shapes, both accumulations, and the layer from
    the bf16 activation (one fused launch where the library has one, else
    quantization + GEMM), each per call from a HIP graph of calls that rotate
    over >= 600 MB of weight copies."""
    from sparse_fp8_row_amd import tune
    names = dict(sfr.linear_algos())
    res = {}
    for shape, ms in DECODE_SHAPES:
        layer = DecodeLayer(torch, sfr, sfr_inputs, lib, dev, shape, 600e6)
        n, k, copies = layer.n, layer.k, layer.copies
        for m in ms:
            x, xq, xs, out, xq2, xs2 = layer.activation(m)
            b = gemm_bytes(m, n, k, layer.has_bias)
            rec = {"n": n, "k": k, "bias": layer.has_bias, "bytes": b}
            dflt = sfr.default_algo(m, n, k)
            for key, algo in (("default", dflt), ("f8acc", dflt | sfr.SFR_ALGO_ACC_F8)):
                us = tune.graph_us(lambda i, hs: layer.gemm(i, hs, m, xq, xs, out, algo), copies, calls=2 * copies)
                gbs = b / (us * 1e-6) / 1e9
                rec[key] = {"algo": names[algo], "us_per_call": round(us, 3), "GB/s": round(gbs, 1),
                            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
            if m <= 16:
                def two(i, hs):
                    layer.quantize(hs, m, x, xq2, xs2)
                    layer.gemm(i, hs, m, xq2, xs2, out, -1)
                rec["quantize_plus_gemm_us_per_call"] = round(tune.graph_us(two, copies, calls=2 * copies), 3)
                rec["dynamic_us_per_call"] = round(
                    tune.graph_us(lambda i, hs: layer.dynamic(i, hs, m, x, xq2, xs2, out), copies, calls=2 * copies), 3)
            res[f"{shape}_M{m}"] = rec
            extra = (f", from bf16: dynamic {rec['dynamic_us_per_call']:.3f} us, two launches "
                     f"{rec['quantize_plus_gemm_us_per_call']:.3f} us" if m <= 16 else "")
            print(f"[bench] decode {shape} {n}x{k} M={m}: {rec['default']['us_per_call']:.3f} us "
                  f"({rec['default']['GB/s']:.0f} GB/s), f8acc {rec['f8acc']['us_per_call']:.3f} us{extra}",
                  file=sys.stderr, flush=True)
        del layer
        torch.cuda.empty_cache()
    return res


def profile_decode(torch, sfr, sfr_inputs, lib, dev, stream, calls=4):
    """Counter runs: `calls` eager calls of the GEMM per (shape, M in {1, 16},
    accumulation), each on a different weight copy (none of them in L2), in
    this order; the FP8-input GEMM, then the dynamic entry point."""
    h = int(stream.cuda_stream)
    j = 0
    for shape, _ in DECODE_SHAPES:
        layer = DecodeLayer(torch, sfr, sfr_inputs, lib, dev, shape, 0, min_copies=8)
        for m in (1, 16):
            x, xq, xs, out, xq2, xs2 = layer.activation(m)
            dflt = sfr.default_algo(m, layer.n, layer.k)
            for tag, algo in (("default", dflt), ("f8acc", dflt | sfr.SFR_ALGO_ACC_F8)):
                torch.cuda.synchronize()
                print(f"[profile] decode {shape} M={m} {tag}: {calls} calls, "
                      f"{gemm_bytes(m, layer.n, layer.k, layer.has_bias)} algorithmic bytes each",
                      file=sys.stderr, flush=True)
                for _ in range(calls):
                    layer.gemm(j % layer.copies, h, m, xq, xs, out, algo)
                    j += 1
            torch.cuda.synchronize()
            print(f"[profile] decode {shape} M={m} dynamic: {calls} calls", file=sys.stderr, flush=True)
            for _ in range(calls):
                layer.dynamic(j % layer.copies, h, m, x, xq2, xs2, out)
                j += 1
            torch.cuda.synchronize()
        del layer
        torch.cuda.empty_cache()


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
