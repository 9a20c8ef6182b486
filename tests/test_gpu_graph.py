"""The library's calls captured in a HIP graph (decode as a serving loop runs
it): quantization + linear, the fused one-row path, and the BSR layer are
captured once and replayed several times, with eager work and
synchronizations between the replays, and every replay must equal the eager
result bit for bit (the kernels are deterministic and allocate nothing)."""
import numpy as np
import pytest
import torch

import sfr_inputs
from parity import dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_fp8_row_amd as sfr
    sfr.load()
    return sfr


def replay_matches(fn, outs_eager, replays=4):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                    # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        outs = fn()
    for r in range(replays):
        for o in outs:
            o.view(torch.uint8).fill_(0)        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, outs_eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"replay {r}"


@pytest.mark.parametrize("m", [1, 4, 16])
def test_graph_quantize_and_linear(gpu, m):
    case = sfr_inputs.Case("graph", 40, m, 4096, 4096, bias=True)
    x = dev_bf16(sfr_inputs.draw_x(case))
    pw = gpu.prepare_weight(dev_bf16(sfr_inputs.draw_w(case)))
    b = dev_bf16(sfr_inputs.draw_bias(case))

    def step():
        xq, xs = gpu.quantize_rowwise_fp8(x)
        y = gpu.sparse_fp8_rowwise_linear(xq, xs, pw.values, pw.meta, pw.scale, b)
        return xq, xs, y

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    replay_matches(step, eager)


def test_graph_fused_one_row(gpu):
    case = sfr_inputs.Case("graph", 41, 1, 4096, 4096, bias=True)
    x = dev_bf16(sfr_inputs.draw_x(case))
    pw = gpu.prepare_weight(dev_bf16(sfr_inputs.draw_w(case)))
    b = dev_bf16(sfr_inputs.draw_bias(case))

    def step():
        return gpu.sparse_fp8_rowwise_linear_dynamic(x, pw.values, pw.meta, pw.scale, b)

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    replay_matches(step, eager)


@pytest.mark.parametrize("m,n,k", [(2, 14336, 4096), (4, 4096, 4096), (16, 14336, 4096), (16, 4096, 14336)])
def test_graph_dynamic_rows(gpu, m, n, k):
    # 2 and 4 rows: one launch; 16: quantization and linear layer (32 weight
    # rows per workgroup at n = 14336, 14 wavefronts of one unit at k = 14336)
    case = sfr_inputs.Case("graph", 43, m, n, k, bias=True)
    x = dev_bf16(sfr_inputs.draw_x(case))
    pw = gpu.prepare_weight(dev_bf16(sfr_inputs.draw_w(case)))
    b = dev_bf16(sfr_inputs.draw_bias(case))

    def step():
        return gpu.sparse_fp8_rowwise_linear_dynamic(x, pw.values, pw.meta, pw.scale, b)

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    replay_matches(step, eager)


def test_graph_bsr(gpu):
    case = sfr_inputs.Case("graph", 42, 4, 4096, 4096, bias=True)
    x = dev_bf16(sfr_inputs.draw_x(case))
    bw = gpu.bsr_from_dense(dev_bf16(sfr_inputs.draw_bsr_w(case)))
    b = dev_bf16(sfr_inputs.draw_bias(case))

    def step():
        return (gpu.bsr_linear(x, bw, b),)

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    replay_matches(step, eager)
