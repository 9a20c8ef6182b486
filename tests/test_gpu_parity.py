"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Quantization, scales and compression are compared bit for bit; the linear
layer's binary32 output within 1e-5 * sum|xq*wq| * xs * ws of the oracle's
exact value, and its bf16 output within 1 bf16 ulp (rules in parity.py).
Shapes span several tiles of every kernel configuration and ragged tails in
M and N; the full-size workloads are checked on sampled output rows.
"""
import itertools
import sys

import numpy as np
import pytest
import torch

import oracle
import sfr_inputs
from parity import (check_bf16, check_f32, dev_bf16, dev_fp8, host_bf16_bits, host_bytes, host_f32, rows_bits,
                    FP8_TORCH)

pytestmark = pytest.mark.gpu

E4, E5 = oracle.E4M3, oracle.E5M2
PAIRS = list(itertools.product([E4, E5], [E4, E5]))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_fp8_row_amd as sfr
    sfr.load()
    return sfr


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# quantize_rowwise_fp8
# ---------------------------------------------------------------------------
# rows <= 64 take the one-row-per-workgroup kernel; (80, 4096) and (66, 14336)
# take the one-row-per-wavefront kernel with whole rows of 8 and 28 chunks per
# lane (its unconditional load and store path), (70, 1000) its ragged path
QSHAPES = [(1, 8), (3, 256), (17, 4096), (64, 4104), (5, 16384), (4, 16392), (130, 512), (9, 14336),
           (80, 4096), (66, 14336), (70, 1000)]


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("kind", ["normal", "student", "wide", "tiny", "edge"])
@pytest.mark.parametrize("shape", QSHAPES)
def test_quantize_bit_exact(gpu, fmt, kind, shape):
    rows, cols = shape
    say(f"quantize {kind} {shape} fmt={fmt}")
    x = rows_bits(kind, rows, cols, rows * 7 + cols)
    q, s = gpu.quantize_rowwise_fp8(dev_bf16(x), FP8_TORCH[fmt])
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_rows(x, fmt)
    assert np.array_equal(host_f32(s).view(np.uint32), os_.view(np.uint32))
    got = host_bytes(q)
    bad = np.argwhere(got != oq)
    assert bad.size == 0, (bad[:5].tolist(), got[tuple(bad[0])], oq[tuple(bad[0])])


# ---------------------------------------------------------------------------
# compress_2to4_fp8
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 128), (16, 4096), (33, 384), (7, 14336)])
@pytest.mark.parametrize("alphabet", ["uniform", "ties"])
def test_compress_bit_exact(gpu, shape, alphabet):
    n, k = shape
    say(f"compress {alphabet} {shape}")
    rng = np.random.default_rng(n + k)
    if alphabet == "uniform":
        w = rng.integers(0, 256, (n, k), dtype=np.uint8)
    else:
        w = rng.choice(np.array([0x00, 0x80, 0x38, 0xB8, 0x01, 0x81, 0x7E], np.uint8), (n, k))
    for fmt in (E4, E5):
        v, m = gpu.compress_2to4_fp8(dev_fp8(w, fmt))
        torch.cuda.synchronize()
        ov, om = oracle.compress_2to4(w)
        assert np.array_equal(host_bytes(v), ov)
        assert np.array_equal(host_bytes(m), om)


# ---------------------------------------------------------------------------
# prune_2to4_bf16
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 8), (16, 4096), (33, 392), (7, 14336), (6144, 4096)])
@pytest.mark.parametrize("alphabet", ["normal", "ties"])
def test_prune_bit_exact(gpu, shape, alphabet):
    n, k = shape
    say(f"prune {alphabet} {shape}")
    rng = np.random.default_rng(n * 3 + k)
    if alphabet == "normal":
        w = sfr_inputs.to_bf16_bits(rng.normal(0.0, 0.02, (n, k)))
        w[rng.random((n, k)) < 0.1] = 0x8000
    else:
        w = rng.choice(np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x3C00, 0xBC00, 0x0001, 0x8001, 0x7F7F, 0xFF7F],
                                np.uint16), (n, k))
    want = oracle.prune_2to4_bf16(w)
    t = dev_bf16(w)
    got = gpu.prune_2to4_bf16(t)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(got), want)
    gpu.prune_2to4_bf16(t, out=t)          # in place
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(t), want)


# ---------------------------------------------------------------------------
# sparse_fp8_rowwise_linear
# ---------------------------------------------------------------------------
def prepare(case):
    """Draw the case's inputs (bf16 bits)."""
    xb = sfr_inputs.draw_x(case)
    wb = sfr_inputs.draw_w(case)
    bb = sfr_inputs.draw_bias(case)
    return xb, wb, bb


def gpu_path(gpu, xb, wb, bb, xf, wf, out_dtype=torch.bfloat16):
    xq, xs = gpu.quantize_rowwise_fp8(dev_bf16(xb), FP8_TORCH[xf])
    pw = gpu.prepare_weight(dev_bf16(wb), FP8_TORCH[wf])
    b = None if bb is None else dev_bf16(bb)
    y = gpu.sparse_fp8_rowwise_linear(xq, xs, pw.values, pw.meta, pw.scale, b, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return xq, xs, pw, y


def oracle_path(xb, wb, bb, xf, wf, rows=None, cols=None):
    oxq, oxs = oracle.quantize_rows(xb, xf)
    ov, om, ows, _ = oracle.prepare_weight(wb, wf)
    ref = oracle.linear(oxq, xf, oxs, ov, om, wf, ows, bias=bb, rows=rows, cols=cols)
    return oxq, oxs, ov, om, ows, ref


def assert_linear(gpu, case, rows=None, out_dtypes=(torch.bfloat16, torch.float32)):
    """The whole path on the default algorithm: bytes bit-exact, every output
    element within the stated bound (no miss budget)."""
    xb, wb, bb = prepare(case)
    oxq, oxs, ov, om, ows, ref = oracle_path(xb, wb, bb, case.x_fmt, case.w_fmt, rows=rows)
    sel = slice(None) if rows is None else rows
    for od in out_dtypes:
        say(f"linear {case.name} out={od} rows={'all' if rows is None else len(rows)}")
        xq, xs, pw, y = gpu_path(gpu, xb, wb, bb, case.x_fmt, case.w_fmt, od)
        assert np.array_equal(host_bytes(xq), oxq)
        assert np.array_equal(host_f32(xs).view(np.uint32), oxs.view(np.uint32))
        assert np.array_equal(host_bytes(pw.values), ov)
        assert np.array_equal(host_bytes(pw.meta), om)
        assert np.array_equal(host_f32(pw.scale).view(np.uint32), ows.view(np.uint32))
        if od == torch.float32:
            r = check_f32(host_f32(y)[sel], ref, bb is not None)
        else:
            r = check_bf16(host_bf16_bits(y)[sel], ref)
        say(f"  {r}")
        assert r["bad"] == 0, r


@pytest.mark.parametrize("xf,wf", PAIRS)
@pytest.mark.parametrize("bias", [False, True])
def test_linear_smoke_all_pairs(gpu, xf, wf, bias):
    assert_linear(gpu, sfr_inputs.Case("smoke", 1, 32, 128, 256, x_fmt=xf, w_fmt=wf, bias=bias))


@pytest.mark.parametrize("case", sfr_inputs.decode_cases(), ids=lambda c: c.name)
def test_linear_decode(gpu, case):
    assert_linear(gpu, case)


# ragged shapes that land on each tile configuration (64x64, 128x128, 256x256)
# and on each decode variant
RAGGED = [
    sfr_inputs.Case("ragged", 6, 100, 1040, 384, x_fmt=E4, w_fmt=E5, bias=True),
    sfr_inputs.Case("ragged", 6, 17, 4096, 256, x_fmt=E5, w_fmt=E4),
    sfr_inputs.Case("ragged", 6, 1000, 4112, 256, x_fmt=E4, w_fmt=E4, bias=True),
    sfr_inputs.Case("ragged", 6, 4100, 8208, 256, x_fmt=E5, w_fmt=E5),
    sfr_inputs.Case("ragged", 6, 2, 144, 128, x_fmt=E4, w_fmt=E4, bias=True),
    # decode kernels: one 1024-k unit per wavefront (one and several units per
    # wavefront, the single-row activation path), K beyond one unit per wavefront
    sfr_inputs.Case("ragged", 6, 3, 64, 1024, x_fmt=E5, w_fmt=E4, bias=True),
    sfr_inputs.Case("ragged", 6, 16, 32, 16384, x_fmt=E4, w_fmt=E5),
    sfr_inputs.Case("ragged", 6, 1, 48, 16384, x_fmt=E5, w_fmt=E5, bias=True),
    sfr_inputs.Case("ragged", 6, 7, 96, 2048, x_fmt=E4, w_fmt=E4),
    # 256 x 256 pipelined kernel (>= 512 tiles, K >= 512): the smallest K, odd
    # and even step counts with and without the paired main loop, ragged M, N
    sfr_inputs.Case("ragged", 6, 4100, 8208, 512, x_fmt=E4, w_fmt=E5, bias=True),
    sfr_inputs.Case("ragged", 6, 4352, 8192, 640, x_fmt=E5, w_fmt=E4),
    sfr_inputs.Case("ragged", 6, 4096, 8448, 896, x_fmt=E4, w_fmt=E4, bias=True),
    sfr_inputs.Case("ragged", 6, 4097, 8192, 1280, x_fmt=E5, w_fmt=E5, bias=True),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: c.name)
def test_linear_ragged(gpu, case):
    rows = None
    if case.m * case.n * case.k > 2e9:
        rng = np.random.default_rng(0)
        rows = np.unique(np.concatenate([rng.choice(case.m, 120, replace=False), [0, case.m - 1]]))
    assert_linear(gpu, case, rows=rows)


def sampled_rows(m, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.choice(m, min(count, m), replace=False), [0, m - 1]]))


@pytest.mark.parametrize("case", [sfr_inputs.prefill_up_case(), sfr_inputs.prefill_down_hard_case()],
                         ids=lambda c: c.name)
def test_linear_full_size_sampled(gpu, case):
    """Full-size prefill workloads, in the launch configuration the benchmark
    times: quantize/compress bit-exact on every byte, the linear layer's bf16
    and binary32 outputs on 128 sampled rows (all N)."""
    assert_linear(gpu, case, rows=sampled_rows(case.m, 128, 1))


SWEEP_ROWS = 24   # sampled activation rows for M > 16 (plus the first and last)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("shape", list(sfr_inputs.LLAMA_SHAPES))
def test_linear_llama_sweep(gpu, shape, seed):
    """Llama-3.1-8B layer sweep: every M and dtype pair, bf16 and binary32
    outputs, each seed; every row for M <= 16, sampled rows above."""
    n, k = sfr_inputs.LLAMA_SHAPES[shape]
    base = sfr_inputs.Case("sweep", 5, 1, n, k, seed=seed)
    wb = sfr_inputs.draw_w(base)
    weights = {}
    for wf in (E4, E5):
        say(f"sweep {shape} weight fmt={wf}")
        ov, om, ows, _ = oracle.prepare_weight(wb, wf)
        pw = gpu.prepare_weight(dev_bf16(wb), FP8_TORCH[wf])
        torch.cuda.synchronize()
        assert np.array_equal(host_bytes(pw.values), ov) and np.array_equal(host_bytes(pw.meta), om)
        assert np.array_equal(host_f32(pw.scale).view(np.uint32), ows.view(np.uint32))
        weights[wf] = (pw, ov, om, ows)
    for m in (1, 16, 512, 8192):
        case = sfr_inputs.Case("sweep", 5, m, n, k, seed=seed)
        xb = sfr_inputs.draw_x(case)
        rows = np.arange(m) if m <= 16 else sampled_rows(m, SWEEP_ROWS, m + seed)
        for xf in (E4, E5):
            xq, xs = gpu.quantize_rowwise_fp8(dev_bf16(xb), FP8_TORCH[xf])
            oxq, oxs = oracle.quantize_rows(xb[rows], xf)
            torch.cuda.synchronize()
            assert np.array_equal(host_bytes(xq)[rows], oxq)
            assert np.array_equal(host_f32(xs)[rows].view(np.uint32), oxs.view(np.uint32))
            # oracle operands restricted to the sampled rows (row i of oxq is row rows[i])
            for wf in (E4, E5):
                pw, ov, om, ows = weights[wf]
                ref = oracle.linear(oxq, xf, oxs, ov, om, wf, ows)
                for od in (torch.bfloat16, torch.float32):
                    say(f"sweep {shape} s{seed} M={m} {xf}x{wf} out={od}")
                    y = gpu.sparse_fp8_rowwise_linear(xq, xs, pw.values, pw.meta, pw.scale, out_dtype=od)
                    torch.cuda.synchronize()
                    if od == torch.float32:
                        r = check_f32(host_f32(y)[rows], ref, False)
                    else:
                        r = check_bf16(host_bf16_bits(y)[rows], ref)
                    say(f"  {r}")
                    assert r["bad"] == 0, r


def test_linear_deterministic(gpu):
    case = sfr_inputs.Case("det", 7, 333, 4096, 1024, bias=True)
    xb, wb, bb = prepare(case)
    say("determinism", case.name)
    outs = [host_bf16_bits(gpu_path(gpu, xb, wb, bb, E4, E4)[3]) for _ in range(2)]
    assert np.array_equal(outs[0], outs[1])
    dec = sfr_inputs.Case("det", 7, 7, 4096, 4096, bias=True)
    xb, wb, bb = prepare(dec)
    outs = [host_bf16_bits(gpu_path(gpu, xb, wb, bb, E4, E5)[3]) for _ in range(2)]
    assert np.array_equal(outs[0], outs[1])
    wide = sfr_inputs.Case("det", 7, 4096, 8192, 640, bias=True)
    xb, wb, bb = prepare(wide)
    say("determinism", wide.name)
    outs = [host_bf16_bits(gpu_path(gpu, xb, wb, bb, E5, E4)[3]) for _ in range(2)]
    assert np.array_equal(outs[0], outs[1])


def test_zero_rows_give_bias(gpu):
    case = sfr_inputs.Case("zero", 8, 40, 256, 512, bias=True)
    xb, wb, bb = prepare(case)
    xb[[0, 7, 39]] = 0x8000
    say("zero rows", case.name)
    _, xs, _, y = gpu_path(gpu, xb, wb, bb, E4, E4)
    assert np.all(host_f32(xs)[[0, 7, 39]] == 0)
    out = host_bf16_bits(y)
    for r in (0, 7, 39):
        assert np.array_equal(out[r], bb)


def test_empty_calls_are_noops(gpu):
    say("empty calls")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = gpu.quantize_rowwise_fp8(x)
    assert q.shape == (0, 256)
    w = torch.empty((0, 256), dtype=torch.float8_e4m3fn, device="cuda")
    v, m = gpu.compress_2to4_fp8(w)
    assert v.shape == (0, 128)
    xq = torch.zeros((0, 256), dtype=torch.float8_e4m3fn, device="cuda")
    xs = torch.zeros((0,), dtype=torch.float32, device="cuda")
    vals = torch.zeros((32, 128), dtype=torch.float8_e4m3fn, device="cuda")
    meta = torch.full((32, 32), 0x44, dtype=torch.uint8, device="cuda")
    ws = torch.ones(32, dtype=torch.float32, device="cuda")
    y = gpu.sparse_fp8_rowwise_linear(xq, xs, vals, meta, ws)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)
