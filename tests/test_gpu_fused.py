"""GPU parity of sparse_fp8_rowwise_linear_dynamic (activation quantization
fused into the decode GEMM launch for one activation row).

The codes and scales it writes are compared bit for bit with the oracle's
row-wise quantization, the output with the oracle's linear layer (same rules
as the row-wise tests), on every fused shape class (K from one 1024-k unit
to 16384, one and two units per wavefront, uneven unit counts, grids smaller
and larger than the chip holds at once, row and tensor weight scales, an
all-zero row) and on shapes that take the two-launch path.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sfr_inputs
from parity import check_bf16, check_f32, dev_bf16, host_bf16_bits, host_bytes, host_f32, hw_bound, FP8_TORCH

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


def run_case(gpu, case, wscale="row", seed_shift=0):
    xb = sfr_inputs.draw_x(case)
    wb = sfr_inputs.draw_w(case)
    bb = sfr_inputs.draw_bias(case)
    xf, wf = case.x_fmt, case.w_fmt
    oxq, oxs = oracle.quantize_rows(xb, xf)
    owq, ows = (oracle.quantize_tensor if wscale == "tensor" else oracle.quantize_rows)(wb, wf)
    ov, om = oracle.compress_2to4(owq)
    ws_full = np.full(case.n, ows[0], np.float32) if wscale == "tensor" else ows
    ref = oracle.linear(oxq, xf, oxs, ov, om, wf, ws_full, bias=bb)
    hwb = hw_bound(oxq, xf, oxs, oracle.decompress_2to4(ov, om), wf, ws_full, np.arange(case.m), np.arange(case.n))
    pw = gpu.prepare_weight(dev_bf16(wb), FP8_TORCH[wf], scaling=wscale)
    b = None if bb is None else dev_bf16(bb)
    for od in (torch.bfloat16, torch.float32):
        say(f"dynamic {case.name} w={wscale} out={od}")
        y, xq, xs = gpu.sparse_fp8_rowwise_linear_dynamic(dev_bf16(xb), pw.values, pw.meta, pw.scale, b,
                                                          act_dtype=FP8_TORCH[xf], out_dtype=od)
        torch.cuda.synchronize()
        assert np.array_equal(host_bytes(xq), oxq)
        assert np.array_equal(host_f32(xs).view(np.uint32), oxs.view(np.uint32))
        if od == torch.float32:
            r = check_f32(host_f32(y), ref, bb is not None, hwb)
        else:
            r = check_bf16(host_bf16_bits(y), ref, hwb)
        say(f"  {r}")
        assert r["bad"] == 0, r
        assert r["strict_rate_ok"], r


# (m, n, k): fused shapes (n/16 workgroups: 16 .. 896, more than the chip's 256 CUs;
# K/1024 units over up to 8 wavefronts: 1, 2, 4, 5 x (2,2,2,2,1), 7 x 2, 8 x 2)
FUSED = [(1, 4096, 4096), (1, 1040, 1024), (1, 14336, 4096), (1, 256, 2048), (1, 2048, 9216), (1, 512, 14336),
         (1, 4096, 16384)]


@pytest.mark.parametrize("shape", FUSED, ids=lambda s: f"M{s[0]}N{s[1]}K{s[2]}")
def test_dynamic_fused(gpu, shape):
    m, n, k = shape
    xf, wf = [(E4, E4), (E5, E4), (E4, E5), (E5, E5)][(m + n // 16) % 4]
    run_case(gpu, sfr_inputs.Case(f"dyn_M{m}N{n}K{k}", 10, m, n, k, x_fmt=xf, w_fmt=wf, bias=((n // 16) % 2 == 0)))


def test_dynamic_fused_tensor_weight_scale(gpu):
    run_case(gpu, sfr_inputs.Case("dyn_tensor", 10, 1, 4096, 2048, x_fmt=E4, w_fmt=E5, bias=True), wscale="tensor")
    run_case(gpu, sfr_inputs.Case("dyn_tensor", 10, 2, 4096, 2048, x_fmt=E5, w_fmt=E5, bias=True), wscale="tensor")


def test_dynamic_fused_zero_row(gpu):
    # an all-zero activation row (both zero signs): codes keep each sign, scale 0, out = bias
    n, k = 1024, 2048
    case = sfr_inputs.Case("dyn_zero", 13, 1, n, k, bias=True)
    xb = np.zeros((1, k), np.uint16)
    xb[0, 1::3] = 0x8000
    pw = gpu.prepare_weight(dev_bf16(sfr_inputs.draw_w(case)), torch.float8_e4m3fn)
    bb = sfr_inputs.draw_bias(case)
    y, xq, xs = gpu.sparse_fp8_rowwise_linear_dynamic(dev_bf16(xb), pw.values, pw.meta, pw.scale, dev_bf16(bb))
    torch.cuda.synchronize()
    oxq, oxs = oracle.quantize_rows(xb, E4)
    assert np.array_equal(host_bytes(xq), oxq)
    assert host_f32(xs)[0] == 0.0 and oxs[0] == 0.0
    assert np.array_equal(host_bf16_bits(y)[0], bb)


# shapes that take the two-launch path: m > 1, k not a multiple of 1024, k > 16384
@pytest.mark.parametrize("shape", [(17, 1024, 1024), (5, 512, 640), (16, 4096, 14336), (16, 4096, 4096),
                                   (2, 1024, 1024), (4, 4096, 4096), (1, 4096, 640), (1, 256, 17408)],
                         ids=lambda s: f"M{s[0]}N{s[1]}K{s[2]}")
def test_dynamic_two_launch(gpu, shape):
    m, n, k = shape
    run_case(gpu, sfr_inputs.Case(f"dyn2_M{m}N{n}K{k}", 10, m, n, k, x_fmt=E5, w_fmt=E4, bias=True))


def test_dynamic_back_to_back(gpu):
    # several calls in a row on one stream (fused and two-launch), each checked
    n, k = 4096, 4096
    case_w = sfr_inputs.Case("dyn_seq", 11, 16, n, k, bias=True)
    wb = sfr_inputs.draw_w(case_w)
    pw = gpu.prepare_weight(dev_bf16(wb), torch.float8_e4m3fn)
    owq, ows = oracle.quantize_rows(wb, E4)
    ov, om = oracle.compress_2to4(owq)
    outs, refs = [], []
    for i, m in enumerate((1, 4, 1, 9)):
        case = sfr_inputs.Case("dyn_seq", 20 + i, m, n, k)
        xb = sfr_inputs.draw_x(case)
        y, xq, xs = gpu.sparse_fp8_rowwise_linear_dynamic(dev_bf16(xb), pw.values, pw.meta, pw.scale)
        outs.append((y, xq, xs, xb))
    torch.cuda.synchronize()
    for y, xq, xs, xb in outs:
        oxq, oxs = oracle.quantize_rows(xb, E4)
        assert np.array_equal(host_bytes(xq), oxq)
        ref = oracle.linear(oxq, E4, oxs, ov, om, E4, ows)
        hwb = hw_bound(oxq, E4, oxs, oracle.decompress_2to4(ov, om), E4, ows, np.arange(len(xb)), np.arange(n))
        r = check_bf16(host_bf16_bits(y), ref, hwb)
        say(f"  seq m={len(xb)} {r}")
        assert r["bad"] == 0, r


def test_dynamic_matches_two_step_path(gpu):
    # the fused call gives the same bytes as quantize_rowwise_fp8 + sparse_fp8_rowwise_linear
    case = sfr_inputs.Case("dyn_eq", 12, 1, 2048, 4096, x_fmt=E5, w_fmt=E5, bias=True)
    xb = dev_bf16(sfr_inputs.draw_x(case))
    pw = gpu.prepare_weight(dev_bf16(sfr_inputs.draw_w(case)), torch.float8_e5m2)
    b = dev_bf16(sfr_inputs.draw_bias(case))
    y, xq, xs = gpu.sparse_fp8_rowwise_linear_dynamic(xb, pw.values, pw.meta, pw.scale, b,
                                                      act_dtype=torch.float8_e5m2)
    xq2, xs2 = gpu.quantize_rowwise_fp8(xb, torch.float8_e5m2)
    y2 = gpu.sparse_fp8_rowwise_linear(xq2, xs2, pw.values, pw.meta, pw.scale, b)
    torch.cuda.synchronize()
    assert np.array_equal(host_bytes(xq), host_bytes(xq2))
    assert np.array_equal(host_f32(xs).view(np.uint32), host_f32(xs2).view(np.uint32))
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y2))
