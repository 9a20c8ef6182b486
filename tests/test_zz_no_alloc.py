"""GPU: quantize_tensorwise_fp8_noalloc (the library's own device workspace)
against quantize_tensorwise_fp8 (caller workspace), through the C ABI: the
same bytes and scale on two calls in a row, the second on a smaller tensor
(so it reads only slots it wrote itself after the first call filled more)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import dev_bf16, host_bytes, host_f32, rows_bits, FP8_TORCH

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_fp8_row_amd as sfr
    sfr.load()
    return sfr


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_noalloc_matches_workspace_entry(gpu, fmt):
    lib = gpu.load()
    h = int(torch.cuda.current_stream().cuda_stream)
    # large then small: the second call uses fewer workspace slots than the first
    for (rows, cols, kind) in [(2048, 4096, "student"), (3, 256, "normal")]:
        print(f"noalloc {rows}x{cols} {kind} fmt={fmt}", flush=True)
        sys.stdout.flush()
        x = dev_bf16(rows_bits(kind, rows, cols, rows + cols))
        q1 = torch.empty((rows, cols), dtype=FP8_TORCH[fmt], device="cuda")
        s1 = torch.empty((1,), dtype=torch.float32, device="cuda")
        st = lib.quantize_tensorwise_fp8_noalloc(x.data_ptr(), rows, cols, fmt, q1.data_ptr(), s1.data_ptr(), h)
        assert st == 0, st
        q2, s2 = gpu.quantize_tensorwise_fp8(x, FP8_TORCH[fmt])
        torch.cuda.synchronize()
        assert np.array_equal(host_bytes(q1), host_bytes(q2))
        assert np.array_equal(host_f32(s1).view(np.uint32), host_f32(s2).view(np.uint32))
        # and the oracle's tensor-wise quantization
        oq, os_ = oracle.quantize_tensor(rows_bits(kind, rows, cols, rows + cols), fmt)
        assert np.array_equal(host_bytes(q1), oq)
        assert np.array_equal(host_f32(s1).view(np.uint32), os_.view(np.uint32))


def test_noalloc_validation(gpu):
    lib = gpu.load()
    x = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((4, 16), dtype=torch.float8_e4m3fn, device="cuda")
    s = torch.empty((1,), dtype=torch.float32, device="cuda")
    assert lib.quantize_tensorwise_fp8_noalloc(x.data_ptr(), 4, 12, 0, q.data_ptr(), s.data_ptr(), None) == 2
    assert lib.quantize_tensorwise_fp8_noalloc(x.data_ptr(), 4, 16, 7, q.data_ptr(), s.data_ptr(), None) == 4
    assert lib.quantize_tensorwise_fp8_noalloc(None, 4, 16, 0, q.data_ptr(), s.data_ptr(), None) == 1
