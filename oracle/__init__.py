"""CPU oracle for the row-wise-scaled FP8 linear layer with a 2:4 sparse weight.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``sparse_fp8_row_amd``) never imports, links or runs anything here, and this
package never imports the product library.

The arithmetic lives in ``sfr_oracle.c`` (plain C, binary32/binary64, no
contraction, OpenMP over independent outputs only).  This module compiles it
with gcc on first use and wraps it with ctypes + numpy.

Sources, cited per function in ``sfr_oracle.c``:
  * "Add CUTLASS-based row-wise scaled sparse FP8 kernel" (pytorch/ao PR #1671):
    the operator, the sparse converter and its -0.0 rule, no-NaN casts.
  * "Making torchao ABI compatible ..." (pytorch/ao issue #3516), file table:
    the four FP8 dtype pairs.
  * "[float8nocompile] ... atomic_max-based algo ..." (pytorch/ao PR #1455):
    deterministic amax.
  * "promote blocksparse from prototype, make it faster" (pytorch/ao PR
    #1734): the block-sparse (BSR, 64 x 64 blocks) weight and its linear layer.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against library routines, closed forms, brute force and printed fixtures.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

E4M3 = 0
E5M2 = 1
FMAX = {E4M3: 448.0, E5M2: 57344.0}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sfr_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libsfr_oracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-std=c11",
           "-Wall", "-Wextra", "-shared", "-fPIC"]
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle's C source with gcc (host code only)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.orc_fp8_decode.restype = ctypes.c_double
        lib.orc_fp8_decode.argtypes = [ctypes.c_uint8, I]
        lib.orc_fp8_encode.restype = ctypes.c_uint8
        lib.orc_fp8_encode.argtypes = [ctypes.c_float, I]
        lib.orc_bf16_from_double.restype = ctypes.c_uint16
        lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
        for name, args in {
            "orc_fp8_decode_array": [P, I64, I, P],
            "orc_fp8_encode_array": [P, I64, I, P],
            "orc_bf16_from_double_array": [P, I64, P],
            "orc_select_array": [P, I64, I, P, P],
            "orc_quantize_rows": [P, I64, I64, I, P, P],
            "orc_quantize_tensor": [P, I64, I64, I, P, P],
            "orc_compress_2to4": [P, I64, I64, P, P],
            "orc_decompress_2to4": [P, P, I64, I64, P],
            "orc_prune_2to4": [P, I64, I64, P],
            "orc_prune_2to4_bf16": [P, I64, I64, P],
            "orc_check_all_groups": [P, P],
            "orc_linear": [P, I, P, I64, I64, P, P, I, P, I64, P, P, I64, P, I64, P, P, P],
            "orc_bsr_fill": [P, I64, I64, I64, P, P, P],
            "orc_bsr_to_dense": [P, P, P, I64, I64, I64, P],
            "orc_bsr_linear": [P, I64, I64, P, P, P, I64, I64, P, P, I64, P, I64, P, P, P],
        }.items():
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = args
        lib.orc_bsr_count.restype = I64
        lib.orc_bsr_count.argtypes = [P, I64, I64, I64, P]
        lib.orc_num_threads.restype = I
        lib.orc_num_threads.argtypes = []
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


# --------------------------------------------------------------------------
# FP8 and bf16 codecs
# --------------------------------------------------------------------------
def fp8_decode(codes, fmt: int) -> np.ndarray:
    """Exact binary64 value of each FP8 byte."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_fp8_decode_array(_ptr(c), c.size, fmt, _ptr(out))
    return out


def fp8_encode(values, fmt: int) -> np.ndarray:
    """Saturating round-to-nearest-even FP8 code of each binary32 value."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_fp8_encode_array(_ptr(v), v.size, fmt, _ptr(out))
    return out


def bf16_from_double(y) -> np.ndarray:
    """Round binary64 values to bf16 bits (RNE, overflow to inf)."""
    v = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().orc_bf16_from_double_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_float(h) -> np.ndarray:
    """Exact binary32 value of bf16 bits."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Quantization and 2:4 compression
# --------------------------------------------------------------------------
def quantize_rows(x_bf16: np.ndarray, fmt: int):
    """Row-wise dynamic FP8 quantization of bf16 bits [rows, cols].

    Returns (q uint8 [rows, cols], scale float32 [rows])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(rows, np.float32)
    _load().orc_quantize_rows(_ptr(x), rows, cols, fmt, _ptr(q), _ptr(s))
    return q, s


def quantize_tensor(x_bf16: np.ndarray, fmt: int):
    """Tensor-wise dynamic FP8 quantization of bf16 bits [rows, cols].

    Returns (q uint8 [rows, cols], scale float32 [1])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(1, np.float32)
    _load().orc_quantize_tensor(_ptr(x), rows, cols, fmt, _ptr(q), _ptr(s))
    return q, s


def select(groups: np.ndarray, formulation: int = 0):
    """Kept (i0, i1) of each 4-byte group; formulation 0 ranks, 1 tests pairs."""
    g = np.ascontiguousarray(groups, dtype=np.uint8).reshape(-1, 4)
    i0 = np.empty(len(g), np.int32)
    i1 = np.empty(len(g), np.int32)
    _load().orc_select_array(_ptr(g), len(g), formulation, _ptr(i0), _ptr(i1))
    return i0, i1


def compress_2to4(wq: np.ndarray):
    """(values uint8 [n, k/2], meta uint8 [n, k/8]) of FP8 bytes [n, k]."""
    w = np.ascontiguousarray(wq, dtype=np.uint8)
    n, k = w.shape
    assert k % 8 == 0
    values = np.empty((n, k // 2), np.uint8)
    meta = np.empty((n, k // 8), np.uint8)
    _load().orc_compress_2to4(_ptr(w), n, k, _ptr(values), _ptr(meta))
    return values, meta


def decompress_2to4(values: np.ndarray, meta: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.uint8)
    m = np.ascontiguousarray(meta, dtype=np.uint8)
    n, k2 = v.shape
    k = 2 * k2
    assert m.shape == (n, k // 8)
    w = np.empty((n, k), np.uint8)
    _load().orc_decompress_2to4(_ptr(v), _ptr(m), n, k, _ptr(w))
    return w


def prune_2to4(wq: np.ndarray) -> np.ndarray:
    """Dense FP8 bytes with the non-kept entries zeroed (pair formulation)."""
    w = np.ascontiguousarray(wq, dtype=np.uint8)
    n, k = w.shape
    out = np.empty_like(w)
    _load().orc_prune_2to4(_ptr(w), n, k, _ptr(out))
    return out


def prune_2to4_bf16(w_bf16: np.ndarray) -> np.ndarray:
    """2:4 magnitude pruning of bf16 bits [n, k]: in every group of four along
    k the two largest magnitudes keep their bits (ties to the lower index,
    +0.0 and -0.0 equal), the other two become +0.0."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    n, k = w.shape
    assert k % 4 == 0
    out = np.empty_like(w)
    _load().orc_prune_2to4_bf16(_ptr(w), n, k, _ptr(out))
    return out


def prepare_weight(w_bf16: np.ndarray, fmt: int, scaling: str = "row"):
    """The weight's preparation: 2:4 pruning in bf16, FP8 quantization (one
    scale per output row, or one for the tensor), compression.

    Returns (values, meta, scale, pruned bf16 bits)."""
    pruned = prune_2to4_bf16(w_bf16)
    q, s = (quantize_tensor if scaling == "tensor" else quantize_rows)(pruned, fmt)
    v, m = compress_2to4(q)
    return v, m, s, pruned


def check_all_groups():
    """(disagreements, invalid) of the two selection formulations over all 2^32 groups."""
    d = np.zeros(1, np.int64)
    b = np.zeros(1, np.int64)
    _load().orc_check_all_groups(_ptr(d), _ptr(b))
    return int(d[0]), int(b[0])


# --------------------------------------------------------------------------
# The linear layer
# --------------------------------------------------------------------------
def linear(xq, xfmt, xs, values, meta, wfmt, ws, bias=None, rows=None, cols=None):
    """Evaluate out[m,n] = xs[m]*ws[n]*sum_k xq[m,k]*wq[n,k] (+bias[n]).

    Only the positions rows x cols are computed (all by default).  Returns a
    dict of [len(rows), len(cols)] arrays:
      y      binary64 value from the exact dot product
      acc32  dot product summed serially in binary32 (unscaled)
      sabs   sum_k |xq*wq| * xs * ws (the tolerance scale)
      bf16   y rounded once to bf16 bits
    """
    xq = np.ascontiguousarray(xq, np.uint8)
    values = np.ascontiguousarray(values, np.uint8)
    meta = np.ascontiguousarray(meta, np.uint8)
    xs = np.ascontiguousarray(xs, np.float32)
    ws = np.ascontiguousarray(ws, np.float32)
    m, k = xq.shape
    n = values.shape[0]
    assert values.shape == (n, k // 2) and meta.shape == (n, k // 8)
    assert xs.shape == (m,) and ws.shape == (n,)
    rows = np.arange(m, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    cols = np.arange(n, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, np.int64)
    y = np.empty((len(rows), len(cols)), np.float64)
    acc = np.empty((len(rows), len(cols)), np.float32)
    sabs = np.empty((len(rows), len(cols)), np.float64)
    if bias is not None:
        bias = np.ascontiguousarray(bias, np.uint16)
        assert bias.shape == (n,)
    _load().orc_linear(_ptr(xq), xfmt, _ptr(xs), m, k, _ptr(values), _ptr(meta), wfmt, _ptr(ws), n,
                       None if bias is None else _ptr(bias), _ptr(rows), len(rows), _ptr(cols),
                       len(cols), _ptr(y), _ptr(acc), _ptr(sabs))
    return {"y": y, "acc32": acc, "sabs": sabs, "bf16": bf16_from_double(y)}


# --------------------------------------------------------------------------
# Block-sparse (BSR) weight, blocks of 64 x 64
# --------------------------------------------------------------------------
BSR_BLOCK = 64


def bsr_from_dense(w_bf16: np.ndarray, bs: int = BSR_BLOCK):
    """(crow int32 [n/bs + 1], col int32 [nnz], values uint16 [nnz, bs, bs]) of
    bf16 bits [n, k]: the blocks holding any non-zero value, in block-row order
    and ascending block column."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    n, k = w.shape
    assert n % bs == 0 and k % bs == 0
    crow = np.empty(n // bs + 1, np.int32)
    nnz = int(_load().orc_bsr_count(_ptr(w), n, k, bs, _ptr(crow)))
    col = np.empty(nnz, np.int32)
    values = np.empty((nnz, bs, bs), np.uint16)
    _load().orc_bsr_fill(_ptr(w), n, k, bs, _ptr(crow), _ptr(col), _ptr(values))
    return crow, col, values


def bsr_to_dense(crow, col, values, n: int, k: int) -> np.ndarray:
    crow = np.ascontiguousarray(crow, np.int32)
    col = np.ascontiguousarray(col, np.int32)
    values = np.ascontiguousarray(values, np.uint16)
    bs = values.shape[1] if values.ndim == 3 else BSR_BLOCK
    w = np.empty((n, k), np.uint16)
    _load().orc_bsr_to_dense(_ptr(crow), _ptr(col), _ptr(values), n, k, bs, _ptr(w))
    return w


def bsr_linear(x_bf16, crow, col, values, n: int, bias=None, rows=None, cols=None):
    """out[m, n] = sum_k x[m, k] * W[n, k] (+ bias[n]) for the BSR weight W.

    Returns a dict of [len(rows), len(cols)] arrays: y (binary64 sum), acc32
    (serial binary32 sum, no bias), sabs (sum |x * w|), bf16 (y rounded once)."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    crow = np.ascontiguousarray(crow, np.int32)
    col = np.ascontiguousarray(col, np.int32)
    values = np.ascontiguousarray(values, np.uint16)
    m, k = x.shape
    bs = BSR_BLOCK
    assert crow.shape == (n // bs + 1,) and values.shape == (len(col), bs, bs)
    rows = np.arange(m, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    cols = np.arange(n, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, np.int64)
    y = np.empty((len(rows), len(cols)), np.float64)
    acc = np.empty((len(rows), len(cols)), np.float32)
    sabs = np.empty((len(rows), len(cols)), np.float64)
    if bias is not None:
        bias = np.ascontiguousarray(bias, np.uint16)
        assert bias.shape == (n,)
    _load().orc_bsr_linear(_ptr(x), m, k, _ptr(crow), _ptr(col), _ptr(values), n, bs,
                           None if bias is None else _ptr(bias), _ptr(rows), len(rows), _ptr(cols), len(cols),
                           _ptr(y), _ptr(acc), _ptr(sabs))
    return {"y": y, "acc32": acc, "sabs": sabs, "bf16": bf16_from_double(y)}
