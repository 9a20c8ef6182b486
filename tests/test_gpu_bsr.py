"""GPU parity of the block-sparse (BSR, 64 x 64 blocks) bf16 path
("promote blocksparse from prototype, make it faster", pytorch/ao PR #1734)
against the oracle.

Conversion (bsr_count_bf16 + bsr_fill_bf16): crow, col and values bit-exact,
on shapes with -0.0-only and subnormal-only blocks, more than 256 block
columns (the fill kernel's chunk loop), empty block rows, an all-zero matrix
and the Llama-3.1-8B shapes at sparsity 0.9.  Linear (bsr_linear_bf16):
binary32 output within 1e-5 * sum |x * w| (+ the bias add's half ulp) of the
binary64 oracle, bf16 output within one bf16 ulp of the oracle's rounding of
it (or inside that tolerance window), for M = 1 .. 40 (ragged 16-row tiles),
with and without bias, many kept blocks per row and empty block rows, and on
12 seeded random shapes (M up to 80, N and K up to 8192, sparsity 0 .. 0.97)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import sfr_inputs
from parity import check_bf16, check_f32, dev_bf16, host_bf16_bits, host_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_fp8_row_amd as sfr
    sfr.load()
    return sfr


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_i32(t):
    return t.cpu().numpy().astype(np.int32)


FORMAT = [(128, 192, 0.5, True), (256, 19200, 0.9, True), (512, 1024, 1.0, False), (192, 256, 1.0 - 1e-9, False),
          (4096, 4096, 0.9, False), (14336, 4096, 0.9, True)]


@pytest.mark.parametrize("shape", FORMAT, ids=lambda s: f"N{s[0]}K{s[1]}s{s[2]:.2f}")
def test_bsr_format(gpu, shape):
    n, k, sparsity, special = shape
    case = sfr_inputs.Case("bsr_fmt", 20, 1, n, k)
    w = sfr_inputs.draw_bsr_w(case, sparsity=sparsity, special=special)
    crow, col, values = oracle.bsr_from_dense(w)
    say(f"bsr format N{n} K{k} sparsity {sparsity}: nnz {len(col)}")
    bw = gpu.bsr_from_dense(dev_bf16(w))
    torch.cuda.synchronize()
    assert np.array_equal(host_i32(bw.crow), crow)
    assert np.array_equal(host_i32(bw.col), col)
    assert np.array_equal(host_bf16_bits(bw.values), values)


def test_bsr_format_all_zero(gpu):
    w = np.zeros((128, 256), np.uint16)
    w[5, 7] = 0x8000
    bw = gpu.bsr_from_dense(dev_bf16(w))
    torch.cuda.synchronize()
    assert host_i32(bw.crow).tolist() == [0, 0, 0] and bw.nnz == 0


def run_linear(gpu, case, sparsity, bias):
    w = sfr_inputs.draw_bsr_w(case, sparsity=sparsity)
    x = sfr_inputs.draw_x(case)
    bb = sfr_inputs.draw_bias(case) if bias else None
    crow, col, values = oracle.bsr_from_dense(w)
    ref = oracle.bsr_linear(x, crow, col, values, case.n, bias=bb)
    bw = gpu.bsr_from_dense(dev_bf16(w))
    xb = dev_bf16(x)
    b = None if bb is None else dev_bf16(bb)
    for od in (torch.bfloat16, torch.float32):
        say(f"bsr linear {case.name} sparsity {sparsity} out={od}")
        y = gpu.bsr_linear(xb, bw, b, out_dtype=od)
        torch.cuda.synchronize()
        if od == torch.float32:
            r = check_f32(host_f32(y), ref, bb is not None)
        else:
            r = check_bf16(host_bf16_bits(y), ref)
        say(f"  {r}")
        assert r["bad"] == 0, r


LINEAR = [(1, 4096, 4096, 0.9, True), (3, 128, 192, 0.5, False), (16, 1024, 1024, 0.0, True),
          (17, 256, 640, 0.7, False), (40, 512, 2048, 0.9, True), (5, 4096, 14336, 0.9, False),
          (2, 192, 128, 0.999, True)]


@pytest.mark.parametrize("shape", LINEAR, ids=lambda s: f"M{s[0]}N{s[1]}K{s[2]}s{s[3]}")
def test_bsr_linear(gpu, shape):
    m, n, k, sparsity, bias = shape
    run_linear(gpu, sfr_inputs.Case("bsr_lin", 21, m, n, k, bias=bias), sparsity, bias)


def test_bsr_linear_deterministic(gpu):
    case = sfr_inputs.Case("bsr_det", 22, 16, 1024, 4096, bias=True)
    w = sfr_inputs.draw_bsr_w(case)
    bw = gpu.bsr_from_dense(dev_bf16(w))
    x = dev_bf16(sfr_inputs.draw_x(case))
    b = dev_bf16(sfr_inputs.draw_bias(case))
    y0 = gpu.bsr_linear(x, bw, b, out_dtype=torch.float32)
    for _ in range(3):
        y1 = gpu.bsr_linear(x, bw, b, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))


def _random_linear(count=12, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        m = int(rng.integers(1, 81))
        n, k = 64 * int(rng.integers(1, 129)), 64 * int(rng.integers(1, 129))
        sparsity = float(rng.choice([0.0, 0.5, 0.9, 0.97, float(rng.random())]))
        out.append((m, n, k, sparsity, bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("shape", _random_linear(), ids=lambda s: f"M{s[0]}N{s[1]}K{s[2]}s{s[3]:.2f}")
def test_bsr_linear_random_shapes(gpu, shape):
    # seeded random shapes: M 1 .. 80 (up to five 16-row tiles, ragged),
    # N and K multiples of 64 up to 8192, sparsity from dense to 0.97
    m, n, k, sparsity, bias = shape
    run_linear(gpu, sfr_inputs.Case("bsr_rand", 23, m, n, k, bias=bias), sparsity, bias)
