"""GPU parity of the tensor-wise scaling variant (one scale per operand).

quantize_tensorwise_fp8 against the oracle's tensor-wise quantization, bit for
bit (codes and the single scale), on shapes whose chunk count is below one
block, ragged, and large enough to need the full 512 partial maxima; and
sparse_fp8_scaled_linear with every mix of row and tensor scales on the
decode, tiled and pipelined kernels, against the oracle's linear layer given
the broadcast scales (same rules as the row-wise tests).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sfr_inputs
from parity import (check_bf16, check_f32, dev_bf16, host_bf16_bits, host_bytes, host_f32, rows_bits,
                    FP8_TORCH)

pytestmark = pytest.mark.gpu

E4, E5 = oracle.E4M3, oracle.E5M2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_fp8_row_amd as sfr
    sfr.load()
    return sfr


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


TSHAPES = [(1, 8), (3, 256), (17, 4096), (64, 4104), (130, 512), (9, 14336), (2048, 4096)]


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("kind", ["normal", "student", "wide", "tiny", "edge", "zero"])
@pytest.mark.parametrize("shape", TSHAPES)
def test_tensorwise_quantize_bit_exact(gpu, fmt, kind, shape):
    rows, cols = shape
    if kind == "zero":
        x = np.zeros((rows, cols), np.uint16)
        x[:, ::5] = 0x8000
    else:
        x = rows_bits(kind, rows, cols, rows * 5 + cols)
    say(f"quantize_tensorwise {kind} {shape} fmt={fmt}")
    q, s = gpu.quantize_tensorwise_fp8(dev_bf16(x), FP8_TORCH[fmt])
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_tensor(x, fmt)
    assert host_f32(s).shape == (1,)
    assert host_f32(s).view(np.uint32)[0] == os_.view(np.uint32)[0]
    got = host_bytes(q)
    bad = np.argwhere(got != oq)
    assert bad.size == 0, (bad[:5].tolist(), got[tuple(bad[0])], oq[tuple(bad[0])])


def test_tensorwise_quantize_deterministic(gpu):
    x = rows_bits("student", 4096, 4096, 99)
    outs = [gpu.quantize_tensorwise_fp8(dev_bf16(x), torch.float8_e4m3fn) for _ in range(2)]
    torch.cuda.synchronize()
    assert np.array_equal(host_bytes(outs[0][0]), host_bytes(outs[1][0]))
    assert host_f32(outs[0][1])[0] == host_f32(outs[1][1])[0]


def _random_tensors(count=10, seed=20261206):
    rng = np.random.default_rng(seed)
    kinds = ["normal", "student", "wide", "tiny", "edge"]
    return [(int(rng.integers(1, 301)), 8 * int(rng.integers(1, 3001)), kinds[int(rng.integers(0, 5))],
             [E4, E5][int(rng.integers(0, 2))]) for _ in range(count)]


@pytest.mark.parametrize("rows,cols,kind,fmt", _random_tensors(), ids=lambda v: str(v))
def test_tensorwise_quantize_random_shapes(gpu, rows, cols, kind, fmt):
    # seeded random tensors (rows 1 .. 300, cols a multiple of 8 up to 24000)
    x = rows_bits(kind, rows, cols, rows * 11 + cols)
    say(f"quantize_tensorwise random {kind} ({rows}, {cols}) fmt={fmt}")
    q, s = gpu.quantize_tensorwise_fp8(dev_bf16(x), FP8_TORCH[fmt])
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_tensor(x, fmt)
    assert host_f32(s).view(np.uint32)[0] == os_.view(np.uint32)[0]
    assert np.array_equal(host_bytes(q), oq)


# (name, m, n, k): decode, tiled, persistent 256x256 and 256x128 (ragged in m
# and n; the last takes tiled_256x128 on a 256-CU device)
LINEAR_SHAPES = [("decode1", 1, 4096, 4096), ("decode16", 16, 4096, 4096), ("decode_blocks", 40, 4096, 2048),
                 ("tiled", 100, 1040, 384),
                 ("persistent", 4100, 8208, 512), ("persistent_256x128", 1000, 7120, 512)]
KINDS = [("tensor", "row"), ("row", "tensor"), ("tensor", "tensor")]


@pytest.mark.parametrize("xk,wk", KINDS)
@pytest.mark.parametrize("shape", LINEAR_SHAPES, ids=lambda s: s[0])
def test_scaled_linear(gpu, shape, xk, wk):
    name, m, n, k = shape
    case = sfr_inputs.Case(f"tensorwise_{name}", 9, m, n, k, x_fmt=E4 if xk == "tensor" else E5,
                           w_fmt=E5 if wk == "tensor" else E4, bias=(name != "tiled"))
    xb = sfr_inputs.draw_x(case)
    wb = sfr_inputs.draw_w(case)
    bb = sfr_inputs.draw_bias(case)
    xf, wf = case.x_fmt, case.w_fmt
    rows = None
    if m * n * k > 2e9:
        rng = np.random.default_rng(1)
        rows = np.unique(np.concatenate([rng.choice(m, 120, replace=False), [0, m - 1]]))
    # oracle: the chosen quantization of each operand, scales broadcast to rows
    oxq, oxs = (oracle.quantize_tensor if xk == "tensor" else oracle.quantize_rows)(xb, xf)
    ov, om, ows, _ = oracle.prepare_weight(wb, wf, scaling=wk)
    xs_full = np.full(m, oxs[0], np.float32) if xk == "tensor" else oxs
    ws_full = np.full(n, ows[0], np.float32) if wk == "tensor" else ows
    ref = oracle.linear(oxq, xf, xs_full, ov, om, wf, ws_full, bias=bb, rows=rows)
    sel = slice(None) if rows is None else rows
    # GPU
    qx = gpu.quantize_tensorwise_fp8 if xk == "tensor" else gpu.quantize_rowwise_fp8
    xq, xs = qx(dev_bf16(xb), FP8_TORCH[xf])
    pw = gpu.prepare_weight(dev_bf16(wb), FP8_TORCH[wf], scaling=wk)
    b = None if bb is None else dev_bf16(bb)
    for od in (torch.bfloat16, torch.float32):
        say(f"scaled_linear {case.name} x={xk} w={wk} out={od}")
        y = gpu.sparse_fp8_scaled_linear(xq, xs, pw.values, pw.meta, pw.scale, b, out_dtype=od)
        torch.cuda.synchronize()
        assert np.array_equal(host_bytes(xq), oxq)
        assert np.array_equal(host_f32(xs).view(np.uint32), oxs.view(np.uint32))
        assert np.array_equal(host_bytes(pw.values), ov) and np.array_equal(host_bytes(pw.meta), om)
        assert np.array_equal(host_f32(pw.scale).view(np.uint32), ows.view(np.uint32))
        if od == torch.float32:
            r = check_f32(host_f32(y)[sel], ref, bb is not None)
        else:
            r = check_bf16(host_bf16_bits(y)[sel], ref)
        say(f"  {r}")
        assert r["bad"] == 0, r


def test_rowwise_entry_equals_scaled_entry(gpu):
    # sparse_fp8_rowwise_linear is sparse_fp8_scaled_linear with row scales
    case = sfr_inputs.Case("rowwise_eq", 9, 33, 256, 512, bias=True)
    xq, xs = gpu.quantize_rowwise_fp8(dev_bf16(sfr_inputs.draw_x(case)))
    pw = gpu.prepare_weight(dev_bf16(sfr_inputs.draw_w(case)))
    b = dev_bf16(sfr_inputs.draw_bias(case))
    y1 = gpu.sparse_fp8_rowwise_linear(xq, xs, pw.values, pw.meta, pw.scale, b)
    y2 = gpu.sparse_fp8_scaled_linear(xq, xs, pw.values, pw.meta, pw.scale, b)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(y1), host_bf16_bits(y2))
