"""Row-wise-scaled FP8 linear layer with a 2:4 sparse weight, for MI355X (gfx950).

Thin Python binding of ``libsparse_fp8_row.so`` (C ABI in
``include/sparse_fp8_row.h``).  This module only marshals arguments: every
step of the computation runs in the library's HIP kernels.  PyTorch provides
device memory and the current HIP stream.

    xq, xs = quantize_rowwise_fp8(x)                    # x: bf16 [M, K] on the GPU
    w = prepare_weight(w_bf16, torch.float8_e4m3fn)     # once per weight
    y = sparse_fp8_rowwise_linear(xq, xs, w.values, w.meta, w.scale, bias)

Tensor-wise scaling (one scale per operand): ``quantize_tensorwise_fp8``,
``prepare_weight(..., scaling="tensor")`` and ``sparse_fp8_scaled_linear``.

The operator follows pytorch/ao PR #1671 ("Add CUTLASS-based row-wise scaled
sparse FP8 kernel"); see the header for the exact contract of each call.
There is no fallback: if the library is missing or no GPU is present the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_fp8_row.so")

SFR_E4M3, SFR_E5M2 = 0, 1
SFR_OUT_BF16, SFR_OUT_F32 = 0, 1
SFR_SCALE_ROW, SFR_SCALE_TENSOR = 0, 1
STATUS = {0: "SFR_OK", 1: "SFR_ERR_NULL", 2: "SFR_ERR_SHAPE", 3: "SFR_ERR_ALIGN",
          4: "SFR_ERR_DTYPE", 5: "SFR_ERR_LAUNCH"}
EXPORTED = ("quantize_rowwise_fp8", "quantize_tensorwise_fp8", "sfr_quantize_tensorwise_workspace_bytes",
            "quantize_tensorwise_fp8_noalloc",
            "compress_2to4_fp8", "prune_2to4_bf16", "sparse_fp8_rowwise_linear", "sparse_fp8_scaled_linear",
            "sparse_fp8_rowwise_linear_dynamic", "sparse_fp8_rowwise_linear_dynamic_algo",
            "sparse_fp8_scaled_linear_algo", "sfr_linear_algo_count", "sfr_linear_algo_valid",
            "sfr_linear_algo_name", "sfr_linear_algo_supported", "sfr_linear_default_algo",
            "bsr_count_bf16", "bsr_fill_bf16", "bsr_linear_bf16", "sfr_status_string", "sfr_format_version")

_FP8 = {torch.float8_e4m3fn: SFR_E4M3, torch.float8_e5m2: SFR_E5M2}
_lib = None


class SfrError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (torch is imported first so both share one HIP runtime)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m sparse_fp8_row_amd.build`")
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.quantize_rowwise_fp8.argtypes = [P, I64, I64, I, P, P, P]
    lib.compress_2to4_fp8.argtypes = [P, I64, I64, I, P, P, P]
    lib.prune_2to4_bf16.argtypes = [P, I64, I64, P, P]
    lib.sparse_fp8_rowwise_linear.argtypes = [P, I, P, I64, I64, P, P, I, P, I64, P, P, I, P]
    lib.quantize_tensorwise_fp8.argtypes = [P, I64, I64, I, P, P, P, I64, P]
    lib.quantize_tensorwise_fp8_noalloc.argtypes = [P, I64, I64, I, P, P, P]
    lib.quantize_tensorwise_fp8_noalloc.restype = I
    lib.sparse_fp8_scaled_linear.argtypes = [P, I, P, I, I64, I64, P, P, I, P, I, I64, P, P, I, P]
    lib.sparse_fp8_rowwise_linear_dynamic.argtypes = [P, I, I64, I64, P, P, I, P, I, I64, P, P, I, P, P, P]
    lib.sparse_fp8_rowwise_linear_dynamic_algo.argtypes = [P, I, I64, I64, P, P, I, P, I, I64, P, P, I, P, P, I, P]
    lib.sfr_linear_algo_valid.argtypes = [I]
    lib.sfr_linear_algo_valid.restype = I
    lib.sparse_fp8_scaled_linear_algo.argtypes = [P, I, P, I, I64, I64, P, P, I, P, I, I64, P, P, I, I, P]
    lib.sparse_fp8_scaled_linear_algo.restype = I
    lib.sfr_linear_algo_count.argtypes = []
    lib.sfr_linear_algo_count.restype = I
    lib.sfr_linear_algo_name.argtypes = [I]
    lib.sfr_linear_algo_name.restype = ctypes.c_char_p
    lib.sfr_linear_algo_supported.argtypes = [I, I64, I64, I64]
    lib.sfr_linear_algo_supported.restype = I
    lib.sfr_linear_default_algo.argtypes = [I64, I64, I64]
    lib.sfr_linear_default_algo.restype = I
    lib.bsr_count_bf16.argtypes = [P, I64, I64, P, P]
    lib.bsr_fill_bf16.argtypes = [P, I64, I64, P, P, P, P]
    lib.bsr_linear_bf16.argtypes = [P, I64, I64, P, P, P, I64, P, P, I, P]
    for fn in (lib.quantize_rowwise_fp8, lib.compress_2to4_fp8, lib.prune_2to4_bf16, lib.sparse_fp8_rowwise_linear,
               lib.quantize_tensorwise_fp8, lib.sparse_fp8_scaled_linear, lib.sparse_fp8_rowwise_linear_dynamic,
               lib.sparse_fp8_rowwise_linear_dynamic_algo,
               lib.bsr_count_bf16, lib.bsr_fill_bf16, lib.bsr_linear_bf16):
        fn.restype = I
    lib.sfr_quantize_tensorwise_workspace_bytes.argtypes = [I64, I64]
    lib.sfr_quantize_tensorwise_workspace_bytes.restype = I64
    lib.sfr_status_string.argtypes = [I]
    lib.sfr_status_string.restype = ctypes.c_char_p
    lib.sfr_format_version.argtypes = []
    lib.sfr_format_version.restype = I
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise SfrError(status, where)


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fp8_enum(dtype) -> int:
    if dtype not in _FP8:
        raise ValueError(f"unsupported FP8 dtype {dtype}")
    return _FP8[dtype]


def quantize_rowwise_fp8(x: torch.Tensor, dtype=torch.float8_e4m3fn, stream=None):
    """bf16 [rows, cols] -> (q FP8 [rows, cols], scale float32 [rows])."""
    _dev(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=dtype, device=x.device)
    s = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(load().quantize_rowwise_fp8(x.data_ptr(), rows, cols, _fp8_enum(dtype), q.data_ptr(),
                                       s.data_ptr(), _stream(stream)), "quantize_rowwise_fp8")
    return q, s


def quantize_tensorwise_fp8(x: torch.Tensor, dtype=torch.float8_e4m3fn, stream=None):
    """bf16 [rows, cols] -> (q FP8 [rows, cols], scale float32 [1]): one scale for the tensor."""
    _dev(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    rows, cols = x.shape
    lib = load()
    q = torch.empty((rows, cols), dtype=dtype, device=x.device)
    s = torch.empty((1,), dtype=torch.float32, device=x.device)
    nbytes = max(int(lib.sfr_quantize_tensorwise_workspace_bytes(rows, cols)), 16)
    work = torch.empty((nbytes,), dtype=torch.uint8, device=x.device)
    _check(lib.quantize_tensorwise_fp8(x.data_ptr(), rows, cols, _fp8_enum(dtype), q.data_ptr(), s.data_ptr(),
                                       work.data_ptr(), nbytes, _stream(stream)), "quantize_tensorwise_fp8")
    return q, s


def quantize_tensorwise_fp8_noalloc(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, stream=None):
    """quantize_tensorwise_fp8 into caller-provided q FP8 [rows, cols] and
    scale float32 [1], on the library's own device workspace (the call
    allocates nothing).  Calls that overlap on one GPU must be serialized."""
    for t, nm in ((x, "x"), (q, "q"), (scale, "scale")):
        _dev(t, nm)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or q.shape != x.shape or scale.shape != (1,) or \
            scale.dtype != torch.float32:
        raise ValueError("x bf16 [rows, cols], q FP8 [rows, cols], scale float32 [1]")
    rows, cols = x.shape
    _check(load().quantize_tensorwise_fp8_noalloc(x.data_ptr(), rows, cols, _fp8_enum(q.dtype), q.data_ptr(),
                                                  scale.data_ptr(), _stream(stream)),
           "quantize_tensorwise_fp8_noalloc")
    return q, scale


def compress_2to4_fp8(wq: torch.Tensor, stream=None):
    """FP8 [n, k] -> (values FP8 [n, k/2], meta uint8 [n, k/8])."""
    _dev(wq, "wq")
    n, k = wq.shape
    values = torch.empty((n, k // 2), dtype=wq.dtype, device=wq.device)
    meta = torch.empty((n, k // 8), dtype=torch.uint8, device=wq.device)
    _check(load().compress_2to4_fp8(wq.data_ptr(), n, k, _fp8_enum(wq.dtype), values.data_ptr(),
                                    meta.data_ptr(), _stream(stream)), "compress_2to4_fp8")
    return values, meta


def prune_2to4_bf16(w: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """bf16 [n, k] -> the same with each group of four along k pruned to its
    two largest magnitudes (the others +0.0).  out may be w (in place)."""
    _dev(w, "w")
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise ValueError("w must be a 2-D bfloat16 tensor")
    n, k = w.shape
    if out is None:
        out = torch.empty_like(w)
    elif out.shape != w.shape or out.dtype != w.dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    _check(load().prune_2to4_bf16(w.data_ptr(), n, k, out.data_ptr(), _stream(stream)), "prune_2to4_bf16")
    return out


SFR_ALGO_DEFAULT = -1
# Flag of an algorithm id: FP8 matrix-instruction accumulation (twice the
# instruction rate; the products of one 128-k step are added 13 bits below
# the largest).  Without it the accumulation is binary32-grade.
SFR_ALGO_ACC_F8 = 0x100
# Algorithm table consulted by sparse_fp8_scaled_linear when no algo is given:
# {(m_bucket, n, k): algo}, filled by set_algo_table (see tune.py).
_algo_table = {}
M_BUCKETS = (1, 4, 16, 64, 256, 1024, 4096, 1 << 62)


def m_bucket(m: int) -> int:
    """Upper bound of m's bucket: rows 1, 2-4, 5-16, 17-64, ... share a table entry."""
    for b in M_BUCKETS:
        if m <= b:
            return b
    return M_BUCKETS[-1]


def linear_algos(acc: Optional[str] = None):
    """[(id, name)] of the linear layer's algorithms: every kernel
    configuration with binary32-grade accumulation (acc="f32"), with FP8
    matrix-instruction accumulation (acc="f8"), or both (None)."""
    lib = load()
    flags = {"f32": (0,), "f8": (SFR_ALGO_ACC_F8,), None: (0, SFR_ALGO_ACC_F8)}[acc]
    ids = [i | f for f in flags for i in range(lib.sfr_linear_algo_count())]
    return [(a, lib.sfr_linear_algo_name(a).decode()) for a in ids if lib.sfr_linear_algo_valid(a)]


def algo_acc(algo: int) -> str:
    """Accumulation of an algorithm id: "f8" or "f32"."""
    return "f8" if algo >= 0 and algo & SFR_ALGO_ACC_F8 else "f32"


def algo_supported(algo: int, m: int, n: int, k: int) -> bool:
    return bool(load().sfr_linear_algo_supported(algo, m, n, k))


def default_algo(m: int, n: int, k: int) -> int:
    return int(load().sfr_linear_default_algo(m, n, k))


def set_algo_table(table: dict):
    """Use {(m_bucket, n, k): algo} (e.g. from tune.search) for later calls; an
    entry whose algorithm cannot run a shape is ignored for that shape."""
    _algo_table.clear()
    _algo_table.update({(int(b), int(n), int(k)): int(a) for (b, n, k), a in table.items()})


def _table_algo(m: int, n: int, k: int) -> int:
    a = _algo_table.get((m_bucket(m), n, k), SFR_ALGO_DEFAULT)
    return a if a == SFR_ALGO_DEFAULT or algo_supported(a, m, n, k) else SFR_ALGO_DEFAULT


def sparse_fp8_scaled_linear(xq: torch.Tensor, xs: torch.Tensor, values: torch.Tensor, meta: torch.Tensor,
                             ws: torch.Tensor, bias: Optional[torch.Tensor] = None,
                             out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None, stream=None,
                             algo: Optional[int] = None):
    """out[m, n] = xs * ws * sum_k xq[m, k] * wq[n, k] (+ bias[n]), as bf16 (or float32).

    Each scale is per row (xs [m], ws [n]) or one for the tensor (shape [1]);
    the granularity follows from the scale's length.  `algo` picks the kernel
    configuration (see linear_algos); None uses the table set by
    set_algo_table, else the library's built-in choice."""
    for t, nm in ((xq, "xq"), (xs, "xs"), (values, "values"), (meta, "meta"), (ws, "ws")):
        _dev(t, nm)
    m, k = xq.shape
    n = values.shape[0]
    if values.shape != (n, k // 2) or meta.shape != (n, k // 8):
        raise ValueError("operand shapes do not match")
    if xs.dim() != 1 or ws.dim() != 1 or xs.dtype != torch.float32 or ws.dtype != torch.float32:
        raise ValueError("scales must be 1-D float32")
    xk = SFR_SCALE_ROW if xs.shape[0] == m and m != 1 else SFR_SCALE_TENSOR if xs.shape[0] == 1 else None
    wk = SFR_SCALE_ROW if ws.shape[0] == n and n != 1 else SFR_SCALE_TENSOR if ws.shape[0] == 1 else None
    if xk is None or wk is None:
        raise ValueError("scales must have one entry per row or a single entry")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.bfloat16 or bias.shape != (n,):
            raise ValueError("bias must be bfloat16 [n]")
    od = {torch.bfloat16: SFR_OUT_BF16, torch.float32: SFR_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=xq.device)
    elif out.shape != (m, n) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    if algo is None:
        algo = _table_algo(m, n, k)
    _check(load().sparse_fp8_scaled_linear_algo(
        xq.data_ptr(), _fp8_enum(xq.dtype), xs.data_ptr(), xk, m, k, values.data_ptr(), meta.data_ptr(),
        _fp8_enum(values.dtype), ws.data_ptr(), wk, n, 0 if bias is None else bias.data_ptr(), out.data_ptr(), od,
        int(algo), _stream(stream)), "sparse_fp8_scaled_linear")
    return out


def sparse_fp8_rowwise_linear(xq: torch.Tensor, xs: torch.Tensor, values: torch.Tensor, meta: torch.Tensor,
                              ws: torch.Tensor, bias: Optional[torch.Tensor] = None,
                              out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None, stream=None):
    """out[m, n] = xs[m] * ws[n] * sum_k xq[m, k] * wq[n, k] (+ bias[n]), as bf16 (or float32)."""
    for t, nm in ((xq, "xq"), (xs, "xs"), (values, "values"), (meta, "meta"), (ws, "ws")):
        _dev(t, nm)
    m, k = xq.shape
    n = values.shape[0]
    if values.shape != (n, k // 2) or meta.shape != (n, k // 8) or xs.shape != (m,) or ws.shape != (n,):
        raise ValueError("operand shapes do not match")
    if xs.dtype != torch.float32 or ws.dtype != torch.float32:
        raise ValueError("scales must be float32")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.bfloat16 or bias.shape != (n,):
            raise ValueError("bias must be bfloat16 [n]")
    od = {torch.bfloat16: SFR_OUT_BF16, torch.float32: SFR_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=xq.device)
    elif out.shape != (m, n) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    _check(load().sparse_fp8_rowwise_linear(
        xq.data_ptr(), _fp8_enum(xq.dtype), xs.data_ptr(), m, k, values.data_ptr(), meta.data_ptr(),
        _fp8_enum(values.dtype), ws.data_ptr(), n, 0 if bias is None else bias.data_ptr(), out.data_ptr(), od,
        _stream(stream)), "sparse_fp8_rowwise_linear")
    return out


def sparse_fp8_rowwise_linear_dynamic(x: torch.Tensor, values: torch.Tensor, meta: torch.Tensor, ws: torch.Tensor,
                                      bias: Optional[torch.Tensor] = None, act_dtype=torch.float8_e4m3fn,
                                      out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None, stream=None,
                                      algo: Optional[int] = None):
    """bf16 x [m, k] -> (out [m, n], xq [m, k], xs [m]): row-wise activation
    quantization and the linear layer, fused into one launch for small decode shapes."""
    for t, nm in ((x, "x"), (values, "values"), (meta, "meta"), (ws, "ws")):
        _dev(t, nm)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    m, k = x.shape
    n = values.shape[0]
    if values.shape != (n, k // 2) or meta.shape != (n, k // 8) or ws.dim() != 1:
        raise ValueError("operand shapes do not match")
    wk = SFR_SCALE_ROW if ws.shape[0] == n and n != 1 else SFR_SCALE_TENSOR if ws.shape[0] == 1 else None
    if wk is None or ws.dtype != torch.float32:
        raise ValueError("ws must be float32 [n] or [1]")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.bfloat16 or bias.shape != (n,):
            raise ValueError("bias must be bfloat16 [n]")
    od = {torch.bfloat16: SFR_OUT_BF16, torch.float32: SFR_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    elif out.shape != (m, n) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    xq = torch.empty((m, k), dtype=act_dtype, device=x.device)
    xs = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check(load().sparse_fp8_rowwise_linear_dynamic_algo(
        x.data_ptr(), _fp8_enum(act_dtype), m, k, values.data_ptr(), meta.data_ptr(), _fp8_enum(values.dtype),
        ws.data_ptr(), wk, n, 0 if bias is None else bias.data_ptr(), out.data_ptr(), od, xq.data_ptr(),
        xs.data_ptr(), SFR_ALGO_DEFAULT if algo is None else int(algo), _stream(stream)),
        "sparse_fp8_rowwise_linear_dynamic")
    return out, xq, xs


@dataclass
class SparseFp8Weight:
    """A prepared weight: 2:4-compressed FP8 values, metadata and row scales."""
    values: torch.Tensor   # FP8 [N, K/2]
    meta: torch.Tensor     # uint8 [N, K/8]
    scale: torch.Tensor    # float32 [N]
    format_version: int = 1


def prepare_weight(w: torch.Tensor, dtype=torch.float8_e4m3fn, stream=None, scaling: str = "row") -> SparseFp8Weight:
    """bf16 weight [N, K] -> 2:4 magnitude pruning in bf16, FP8 quantization
    (row-wise, or tensor-wise with scaling="tensor"), 2:4 compression.

    The compressor then keeps each group's two survivors; the row scales are
    those of the dense weight, since a row's largest element always survives."""
    if scaling not in ("row", "tensor"):
        raise ValueError("scaling must be 'row' or 'tensor'")
    pruned = prune_2to4_bf16(w, stream=stream)
    if scaling == "row":
        wq, ws = quantize_rowwise_fp8(pruned, dtype, stream)
    else:
        wq, ws = quantize_tensorwise_fp8(pruned, dtype, stream)
    del pruned
    values, meta = compress_2to4_fp8(wq, stream)
    return SparseFp8Weight(values, meta, ws, int(load().sfr_format_version()))


def linear(x: torch.Tensor, w: SparseFp8Weight, bias: Optional[torch.Tensor] = None,
           act_dtype=torch.float8_e4m3fn, stream=None, act_scaling: str = "row") -> torch.Tensor:
    """bf16 x [M, K] -> bf16 [M, N]: dynamic activation quantization (row- or
    tensor-wise) + sparse FP8 GEMM."""
    if act_scaling == "row":
        xq, xs = quantize_rowwise_fp8(x, act_dtype, stream)
    elif act_scaling == "tensor":
        xq, xs = quantize_tensorwise_fp8(x, act_dtype, stream)
    else:
        raise ValueError("act_scaling must be 'row' or 'tensor'")
    return sparse_fp8_scaled_linear(xq, xs, w.values, w.meta, w.scale, bias, stream=stream)


# --------------------------------------------------------------------------
# Block-sparse (BSR, 64 x 64 blocks) bf16 weight
# --------------------------------------------------------------------------
BSR_BLOCK = 64


@dataclass
class BsrWeight:
    """A bf16 weight [n, k] in block-sparse form: crow int32 [n/64 + 1], col
    int32 [nnz], values bf16 [nnz, 64, 64] (torch's BSR layout)."""
    crow: torch.Tensor
    col: torch.Tensor
    values: torch.Tensor
    n: int
    k: int

    @property
    def nnz(self) -> int:
        return self.col.shape[0]


def bsr_from_dense(w: torch.Tensor, stream=None) -> BsrWeight:
    """Dense bf16 [n, k] -> BsrWeight keeping every 64 x 64 block that holds a
    non-zero value (two kernels, a read of the block count, one kernel)."""
    _dev(w, "w")
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise ValueError("w must be a 2-D bfloat16 tensor")
    n, k = w.shape
    lib, h = load(), _stream(stream)
    crow = torch.empty((n // BSR_BLOCK + 1,), dtype=torch.int32, device=w.device)
    _check(lib.bsr_count_bf16(w.data_ptr(), n, k, crow.data_ptr(), h), "bsr_count_bf16")
    nnz = int(crow[-1].item()) if crow.numel() else 0
    col = torch.empty((nnz,), dtype=torch.int32, device=w.device)
    values = torch.empty((nnz, BSR_BLOCK, BSR_BLOCK), dtype=torch.bfloat16, device=w.device)
    _check(lib.bsr_fill_bf16(w.data_ptr(), n, k, crow.data_ptr(), col.data_ptr() if nnz else None,
                             values.data_ptr() if nnz else None, h), "bsr_fill_bf16")
    return BsrWeight(crow, col, values, n, k)


def bsr_linear(x: torch.Tensor, w: BsrWeight, bias: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """bf16 x [m, k] -> out [m, n] = x @ W^T (+ bias) for the BSR weight W."""
    _dev(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != w.k:
        raise ValueError("x must be bfloat16 [m, k]")
    m = x.shape[0]
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.bfloat16 or bias.shape != (w.n,):
            raise ValueError("bias must be bfloat16 [n]")
    od = {torch.bfloat16: SFR_OUT_BF16, torch.float32: SFR_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((m, w.n), dtype=out_dtype, device=x.device)
    elif out.shape != (m, w.n) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    _check(load().bsr_linear_bf16(x.data_ptr(), m, w.k, w.crow.data_ptr(), w.col.data_ptr() if w.nnz else None,
                                  w.values.data_ptr() if w.nnz else None, w.n,
                                  None if bias is None else bias.data_ptr(), out.data_ptr(), od, _stream(stream)),
           "bsr_linear_bf16")
    return out
