"""GPU parity on seeded random shapes, through the built-in choice of kernel.

M from 1 to 2100, N a multiple of 16 up to 6144, K a multiple of 128 up to
4096 (half of the decode cases a multiple of 1024, which the unit kernels
need), every dtype pair, with and without bias.  Each case runs the whole
path (row quantization, weight preparation, the linear layer with bf16 and
binary32 output) against the oracle on every row, or on sampled rows for the
larger cases, with the bounds of the fixed-shape tests; cases of at most 16
rows also run the bf16-activation entry point, whose codes and scales must
equal the oracle's and whose output must equal the FP8-input path's bit for
bit.  The shapes reach every branch of the built-in choice (unit, register
and 32-row decode, single-launch decode from bf16, 64x64 and 128x128 tiles,
the persistent kernel with 256x128 and 256x256 tiles) at sizes nobody picked
by hand.  A second set runs every algorithm id that supports its shape
(each accumulation, both outputs), FP8-accumulation ids held to the bound
plus the FP8 instruction's truncation bound, as test_gpu_algos does.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sfr_inputs
from parity import check_bf16, check_f32, dev_bf16, host_bf16_bits, host_bytes, host_f32, hw_bound, is_f8_acc, FP8_TORCH

pytestmark = pytest.mark.gpu

E4, E5 = oracle.E4M3, oracle.E5M2
SAMPLED_ROWS = 40


def _cases(count=60, seed=20261203):
    rng = np.random.default_rng(seed)
    # the smallest shapes, then single-launch decode from bf16 with 1, 3 and 4 rows
    out = [(1, 16, 128, E4, E4, False), (2, 32, 1024, E5, E4, True), (1, 2000, 2048, E5, E5, True),
           (3, 1040, 3072, E4, E5, False), (4, 4000, 4096, E5, E4, True)]
    while len(out) < count:
        regime = len(out) % 3
        if regime == 0:       # decode
            m = int(rng.integers(1, 65))
            k = 1024 * int(rng.integers(1, 5)) if rng.random() < 0.5 else 128 * int(rng.integers(1, 33))
        elif regime == 1:     # mid sizes
            m = int(rng.integers(65, 701))
            k = 128 * int(rng.integers(1, 33))
        else:                 # large
            m = int(rng.integers(701, 2101))
            k = 128 * int(rng.integers(2, 33))
        n = 16 * int(rng.integers(1, 385))
        xf, wf = [(E4, E4), (E4, E5), (E5, E4), (E5, E5)][int(rng.integers(0, 4))]
        out.append((m, n, k, xf, wf, bool(rng.random() < 0.5)))
    return out


CASES = _cases()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_fp8_row_amd as sfr
    sfr.load()
    return sfr


@pytest.mark.parametrize("shape", CASES, ids=lambda c: f"M{c[0]}N{c[1]}K{c[2]}")
def test_random_shape(gpu, shape):
    m, n, k, xf, wf, bias = shape
    case = sfr_inputs.Case("random", 17, m, n, k, x_fmt=xf, w_fmt=wf, bias=bias)
    say(f"random {case.name} algo={gpu.default_algo(m, n, k)}")
    xb = sfr_inputs.draw_x(case)
    wb = sfr_inputs.draw_w(case)
    bb = sfr_inputs.draw_bias(case)
    rows = None
    if m > SAMPLED_ROWS:
        rng = np.random.default_rng(m * 31 + n + k)
        rows = np.unique(np.concatenate([rng.choice(m, SAMPLED_ROWS, replace=False), [0, m - 1]]))
    sel = slice(None) if rows is None else rows
    oxq, oxs = oracle.quantize_rows(xb, xf)
    ov, om, ows, _ = oracle.prepare_weight(wb, wf)
    ref = oracle.linear(oxq, xf, oxs, ov, om, wf, ows, bias=bb, rows=rows)
    x = dev_bf16(xb)
    xq, xs = gpu.quantize_rowwise_fp8(x, FP8_TORCH[xf])
    pw = gpu.prepare_weight(dev_bf16(wb), FP8_TORCH[wf])
    b = None if bb is None else dev_bf16(bb)
    torch.cuda.synchronize()
    assert np.array_equal(host_bytes(xq), oxq)
    assert np.array_equal(host_f32(xs).view(np.uint32), oxs.view(np.uint32))
    assert np.array_equal(host_bytes(pw.values), ov) and np.array_equal(host_bytes(pw.meta), om)
    assert np.array_equal(host_f32(pw.scale).view(np.uint32), ows.view(np.uint32))
    ys = {}
    for od in (torch.bfloat16, torch.float32):
        y = gpu.sparse_fp8_rowwise_linear(xq, xs, pw.values, pw.meta, pw.scale, b, out_dtype=od)
        torch.cuda.synchronize()
        ys[od] = y
        if od == torch.float32:
            r = check_f32(host_f32(y)[sel], ref, bb is not None)
        else:
            r = check_bf16(host_bf16_bits(y)[sel], ref)
        say(f"  out={od} {r}")
        assert r["bad"] == 0, r
    if m <= 16:
        yd, xqd, xsd = gpu.sparse_fp8_rowwise_linear_dynamic(x, pw.values, pw.meta, pw.scale, b,
                                                             act_dtype=FP8_TORCH[xf])
        torch.cuda.synchronize()
        assert np.array_equal(host_bytes(xqd), oxq)
        assert np.array_equal(host_f32(xsd).view(np.uint32), oxs.view(np.uint32))
        assert np.array_equal(host_bf16_bits(yd), host_bf16_bits(ys[torch.bfloat16]))


def _algo_cases(count=16, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m = int(rng.integers(1, 65)) if i % 2 == 0 else int(rng.integers(65, 1201))
        k = 1024 * int(rng.integers(1, 4)) if i % 4 < 2 else 128 * int(rng.integers(1, 25))
        n = 32 * int(rng.integers(1, 129))   # a multiple of 32: the 32-row decode can run
        xf, wf = [(E4, E4), (E4, E5), (E5, E4), (E5, E5)][int(rng.integers(0, 4))]
        out.append((m, n, k, xf, wf, bool(rng.random() < 0.5)))
    return out


ALGO_CASES = _algo_cases()


@pytest.mark.parametrize("shape", ALGO_CASES, ids=lambda c: f"M{c[0]}N{c[1]}K{c[2]}")
def test_random_shape_every_algo(gpu, shape):
    m, n, k, xf, wf, bias = shape
    case = sfr_inputs.Case("random_algo", 18, m, n, k, x_fmt=xf, w_fmt=wf, bias=bias)
    xb, wb, bb = sfr_inputs.draw_x(case), sfr_inputs.draw_w(case), sfr_inputs.draw_bias(case)
    rows = np.arange(m)
    if m > SAMPLED_ROWS:
        rng = np.random.default_rng(m * 37 + n + k)
        rows = np.unique(np.concatenate([rng.choice(m, SAMPLED_ROWS, replace=False), [0, m - 1]]))
    oxq, oxs = oracle.quantize_rows(xb, xf)
    ov, om, ows, _ = oracle.prepare_weight(wb, wf)
    ref = oracle.linear(oxq, xf, oxs, ov, om, wf, ows, bias=bb, rows=rows)
    hwb = hw_bound(oxq, xf, oxs, oracle.decompress_2to4(ov, om), wf, ows, rows, np.arange(n))
    xq, xs = gpu.quantize_rowwise_fp8(dev_bf16(xb), FP8_TORCH[xf])
    pw = gpu.prepare_weight(dev_bf16(wb), FP8_TORCH[wf])
    b = None if bb is None else dev_bf16(bb)
    ran = 0
    for algo, aname in gpu.linear_algos():
        if not gpu.algo_supported(algo, m, n, k):
            continue
        for od in (torch.bfloat16, torch.float32):
            say(f"random algo {aname} {case.name} out={od}")
            y = gpu.sparse_fp8_scaled_linear(xq, xs, pw.values, pw.meta, pw.scale, b, out_dtype=od, algo=algo)
            torch.cuda.synchronize()
            allow = hwb if is_f8_acc(algo) else None
            if od == torch.float32:
                r = check_f32(host_f32(y)[rows], ref, bb is not None, allow)
            else:
                r = check_bf16(host_bf16_bits(y)[rows], ref, allow)
            say(f"  {r}")
            assert r["bad"] == 0, r
        ran += 1
    assert ran >= 6   # the tiled configurations (three sizes, 256x128) with both accumulations at least
