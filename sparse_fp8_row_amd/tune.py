"""Per-shape kernel configuration search for the sparse FP8 linear layer.

The best configuration depends on the shape (pytorch/ao PR #4432, "Add
algorithm search to FP8 sparse linear benchmark"; PR #1671's remaining task of
a meaningful config selection).  ``search`` times every algorithm that can run
each shape on the current GPU and returns a table for
``sparse_fp8_row_amd.set_algo_table``:

    import sparse_fp8_row_amd as sfr
    from sparse_fp8_row_amd import tune
    result = tune.search([(16, 4096, 4096), (8192, 14336, 4096)])
    sfr.set_algo_table(result["table"])
    tune.save(result, "algos.json")        # later: sfr.set_algo_table(tune.load_table("algos.json"))

Inputs are random FP8 codes (the kernels' speed does not depend on the
values); timing is with HIP events on the current stream, after warm-up
calls, with the weight rotated over enough copies that small shapes read HBM,
and small shapes' calls replayed from a HIP graph so that the host's launch
rate does not set the time.
"""
from __future__ import annotations

import json
import time
from typing import Iterable, Optional, Sequence, Tuple

import torch

from . import (SFR_ALGO_ACC_F8, SFR_E4M3, SFR_E5M2, SFR_OUT_BF16, SFR_SCALE_ROW, _check, _stream, algo_supported,
               default_algo, linear_algos, load, m_bucket)

_FMT = {torch.float8_e4m3fn: SFR_E4M3, torch.float8_e5m2: SFR_E5M2}


class _Inputs:
    """Random operands of one (m, n, k) layer, the weight in enough copies that
    small shapes read it from HBM on every call."""

    def __init__(self, m, n, k, x_dtype, w_dtype, rotate_bytes):
        dev = torch.device("cuda")
        g = torch.Generator(device=dev).manual_seed(m * 131 + n * 7 + k)
        self.m, self.n, self.k, self.x_dtype, self.w_dtype = m, n, k, x_dtype, w_dtype
        self.xq = torch.randint(0, 0x78, (m, k), dtype=torch.uint8, device=dev, generator=g).view(x_dtype)
        self.xs = torch.full((m,), 1e-3, dtype=torch.float32, device=dev)
        self.ws = torch.full((n,), 1e-3, dtype=torch.float32, device=dev)
        self.out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        wbytes = n * k // 2 + n * k // 8
        self.copies = max(1, min(64, rotate_bytes // max(wbytes, 1))) if m <= 64 else 1
        self.vals = [torch.randint(0, 0x78, (n, k // 2), dtype=torch.uint8, device=dev, generator=g).view(w_dtype)
                     for _ in range(self.copies)]
        # metadata: every nibble a valid (i0 < i1) pair
        pairs = torch.tensor([0x4, 0x8, 0xC, 0x9, 0xD, 0xE], dtype=torch.uint8, device=dev)
        self.metas = [(pairs[torch.randint(0, 6, (n, k // 8), device=dev, generator=g)] |
                       (pairs[torch.randint(0, 6, (n, k // 8), device=dev, generator=g)] << 4))
                      for _ in range(self.copies)]


def graph_us(call, copies: int, calls: int = 0, replays: int = 0, min_ms: float = 2.0) -> float:
    """Mean GPU microseconds per call of `call(i, stream_handle)` (i cycles over
    `copies` weight copies), with the calls captured in one HIP graph and the
    graph replayed, so that the host's launch rate does not set the time.

    Every copy is used once eagerly (on a side stream) before the capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(copies):
            call(i, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    calls = calls or max(copies, 64)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        for i in range(calls):
            call(i % copies, h)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def batch(r):
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(r):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    batch(1)
    r = replays or 3
    ms = batch(r)
    if not replays and ms < min_ms:
        r = int(r * min_ms / max(ms, 1e-3)) + 1
        ms = batch(r)
    del g
    return ms * 1e3 / (r * calls)


def time_algo(m: int, n: int, k: int, algo: int, x_dtype=torch.float8_e4m3fn, w_dtype=torch.float8_e4m3fn,
              reps: int = 20, warmup: int = 3, rotate_bytes: int = 600 << 20, stream=None,
              inputs: Optional[_Inputs] = None, min_ms: float = 2.0) -> float:
    """Mean microseconds per call of algorithm `algo` on an (m, n, k) layer.

    Every weight copy is used once before timing; the timed batch holds at
    least `reps` calls, every copy twice, and `min_ms` of GPU time.  That
    does not bring an idle GPU's clocks up: run the kernel for about half a
    second first (search does) when comparing times taken in a fresh
    process.  Up to 64 rows (kernels of a few microseconds) the calls are
    timed inside a HIP graph, so that the host's launch rate does not set
    the time."""
    inp = inputs if inputs is not None else _Inputs(m, n, k, x_dtype, w_dtype, rotate_bytes)
    lib = load()
    h = _stream(stream)
    xf, wf = _FMT[inp.x_dtype], _FMT[inp.w_dtype]

    def call(i):
        _check(lib.sparse_fp8_scaled_linear_algo(
            inp.xq.data_ptr(), xf, inp.xs.data_ptr(), SFR_SCALE_ROW, m, k, inp.vals[i].data_ptr(),
            inp.metas[i].data_ptr(), wf, inp.ws.data_ptr(), SFR_SCALE_ROW, n, None, inp.out.data_ptr(),
            SFR_OUT_BF16, algo, h), "sparse_fp8_scaled_linear_algo")

    if stream is None and m <= 64:
        # short kernels: time inside a graph (the host's launch rate would set
        # an eager loop's pace)
        def gcall(i, hs):
            _check(lib.sparse_fp8_scaled_linear_algo(
                inp.xq.data_ptr(), xf, inp.xs.data_ptr(), SFR_SCALE_ROW, m, k, inp.vals[i].data_ptr(),
                inp.metas[i].data_ptr(), wf, inp.ws.data_ptr(), SFR_SCALE_ROW, n, None, inp.out.data_ptr(),
                SFR_OUT_BF16, algo, hs), "sparse_fp8_scaled_linear_algo")
        return graph_us(gcall, inp.copies, calls=max(reps, 2 * inp.copies), min_ms=min_ms)

    s = torch.cuda.current_stream() if stream is None else stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def batch(count):
        torch.cuda.synchronize()
        e0.record(s)
        for i in range(count):
            call(i % inp.copies)
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    batch(max(warmup, inp.copies))
    count = max(reps, 2 * inp.copies)
    ms = batch(count)
    if ms < min_ms:
        count = int(count * min_ms / max(ms, 1e-3)) + 1
        ms = batch(count)
    return ms * 1e3 / count


def search(shapes: Iterable[Tuple[int, int, int]], x_dtype=torch.float8_e4m3fn, w_dtype=torch.float8_e4m3fn,
           reps: int = 20, warmup: int = 3, algos: Optional[Sequence[int]] = None, settle_s: float = 0.5) -> dict:
    """Time every supported algorithm on each (m, n, k).

    Before the first timing the first shape's first candidate runs for
    `settle_s` seconds, so that a search in an idle process does not time its
    first candidates while the clocks are still rising (which would favour
    the later ones).

    Returns {"table": {(m_bucket, n, k): best algo}, "timings": [per-shape
    records with the default and best algorithm and every time in us]}."""
    names = dict(linear_algos())
    table, records = {}, []
    settled = settle_s <= 0
    for m, n, k in shapes:
        # by default the candidates share the built-in choice's accumulation
        # (a faster but less accurate choice is never made silently)
        acc = default_algo(m, n, k) & SFR_ALGO_ACC_F8
        pool = algos if algos is not None else [a for a in names if a & SFR_ALGO_ACC_F8 == acc]
        cand = [a for a in pool if algo_supported(a, m, n, k)]
        inp = _Inputs(m, n, k, x_dtype, w_dtype, 600 << 20)
        if not settled and cand:
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < settle_s:
                time_algo(m, n, k, cand[0], reps=reps, warmup=0, inputs=inp)
            settled = True
        times = {a: time_algo(m, n, k, a, reps=reps, warmup=warmup, inputs=inp) for a in cand}
        del inp
        best = min(times, key=times.get)
        dflt = default_algo(m, n, k)
        table[(m_bucket(m), n, k)] = best
        records.append({"m": m, "n": n, "k": k, "default": names[dflt], "best": names[best],
                        "default_us": round(times.get(dflt, float("nan")), 3), "best_us": round(times[best], 3),
                        "us": {names[a]: round(t, 3) for a, t in times.items()}})
    return {"table": table, "timings": records}


def save(result: dict, path: str):
    rows = [{"m_bucket": b, "n": n, "k": k, "algo": a} for (b, n, k), a in result["table"].items()]
    with open(path, "w") as f:
        json.dump({"table": rows, "timings": result.get("timings", [])}, f, indent=1)


def load_table(path: str) -> dict:
    with open(path) as f:
        rows = json.load(f)["table"]
    return {(r["m_bucket"], r["n"], r["k"]): r["algo"] for r in rows}
