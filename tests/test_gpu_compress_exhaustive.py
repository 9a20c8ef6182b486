"""GPU 2:4 compressor over every 4-byte group.

The compressor's decision for one group of four FP8 codes depends on those
four bytes only (PR "Add CUTLASS-based row-wise scaled sparse FP8 kernel",
ready-for-review comment, items 1 and 3: keep the two largest magnitudes of
each group of four along K, -0.0 counted as zero).  So the whole input space
is the 2^32 groups, and the GPU kernel is compared with the oracle on all of
them, bit for bit: the group u (little-endian bytes of the 32-bit integer u)
sits at position u of a matrix of 2^32 groups, cut into 16 chunks of 2^28
groups (65536 rows of K = 16384), each compressed on the GPU and by the
oracle.  Both FP8 formats share the byte-level rule; the first chunk is run
under both format tags.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from parity import host_bytes

pytestmark = pytest.mark.gpu

K = 16384                     # 4096 groups per row
ROWS = 1 << 16                # 2^28 groups per chunk
CHUNKS = 16                   # 2^32 groups in all


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_fp8_row_amd as sfr
    sfr.load()
    return sfr


def test_compress_every_group(gpu):
    dev = torch.device("cuda:0")
    n_groups = ROWS * K // 4
    mism_v = mism_m = 0
    t0 = time.time()
    for c in range(CHUNKS):
        base = c * n_groups
        # group u = base + i at position i: its four bytes are u's little-endian bytes
        host = np.arange(base, base + n_groups, dtype=np.uint32).view(np.uint8).reshape(ROWS, K)
        ov, om = oracle.compress_2to4(host)
        d = torch.from_numpy(host).to(dev)
        fmts = (torch.float8_e4m3fn, torch.float8_e5m2) if c == 0 else (torch.float8_e4m3fn,)
        for f in fmts:
            v, m = gpu.compress_2to4_fp8(d.view(f))
            torch.cuda.synchronize()
            gv, gm = host_bytes(v), host_bytes(m)
            bad_v = int(np.count_nonzero(gv != ov))
            bad_m = int(np.count_nonzero(gm != om))
            mism_v += bad_v
            mism_m += bad_m
            if bad_v or bad_m:
                i = int(np.argmax((gm != om).any(axis=1) | (gv != ov).any(axis=1)))
                say(f"chunk {c} {f}: {bad_v} value bytes and {bad_m} metadata bytes differ (first row {i})")
            del v, m, gv, gm
        del d, host, ov, om
        say(f"chunk {c + 1}/{CHUNKS}: groups {base:#x}..{base + n_groups - 1:#x} done, {time.time() - t0:.1f} s")
    assert mism_v == 0 and mism_m == 0, f"{mism_v} value bytes and {mism_m} metadata bytes differ from the oracle"
