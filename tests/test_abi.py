"""The C ABI on the CPU: the built library loads, exports every function the
header declares, and rejects invalid arguments with the documented status
before anything is launched (so these calls need no GPU)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_fp8_row.h")


@pytest.fixture(scope="module")
def lib():
    import sparse_fp8_row_amd as sfr
    if not os.path.exists(sfr.LIB_PATH):
        from sparse_fp8_row_amd import build
        build.build()
    return sfr.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("quantize_rowwise_fp8", "compress_2to4_fp8", "prune_2to4_bf16", "sparse_fp8_rowwise_linear",
              "sfr_status_string",
              "sfr_format_version", "quantize_tensorwise_fp8", "sfr_quantize_tensorwise_workspace_bytes",
              "sparse_fp8_scaled_linear", "sparse_fp8_rowwise_linear_dynamic", "sparse_fp8_scaled_linear_algo",
              "sparse_fp8_rowwise_linear_dynamic_algo", "sfr_linear_algo_valid",
              "sfr_linear_algo_count", "sfr_linear_algo_name", "sfr_linear_algo_supported", "sfr_linear_default_algo",
              "bsr_count_bf16", "bsr_fill_bf16", "bsr_linear_bf16"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.sfr_format_version() == 1
    assert lib.sfr_status_string(0) == b"ok"
    assert lib.sfr_status_string(2) == b"invalid shape"
    assert lib.sfr_status_string(99) == b"unknown status"


OK, NULL, SHAPE, ALIGN, DTYPE = 0, 1, 2, 3, 4
A = 0x10000          # a 16-byte aligned stand-in address (never dereferenced: every call below fails validation)
U = 0x10001          # a misaligned one


def test_quantize_validation(lib):
    q = lib.quantize_rowwise_fp8
    assert q(A, 4, 16, 2, A, A, None) == DTYPE
    assert q(A, 4, 15, 0, A, A, None) == SHAPE          # cols % 8
    assert q(A, 4, 0, 0, A, A, None) == SHAPE           # no elements
    assert q(A, -1, 16, 0, A, A, None) == SHAPE
    assert q(A, 4, (1 << 30) + 8, 0, A, A, None) == SHAPE
    assert q(None, 0, 16, 0, None, None, None) == OK    # empty: no-op
    assert q(None, 4, 16, 0, A, A, None) == NULL
    assert q(A, 4, 16, 0, A, None, None) == NULL
    assert q(U, 4, 16, 0, A, A, None) == ALIGN
    assert q(A, 4, 16, 1, A, U, None) == ALIGN


def test_compress_validation(lib):
    c = lib.compress_2to4_fp8
    assert c(A, 4, 128, -1, A, A, None) == DTYPE
    assert c(A, 4, 64, 0, A, A, None) == SHAPE          # k % 128
    assert c(A, 4, 0, 0, A, A, None) == SHAPE
    assert c(A, -4, 128, 0, A, A, None) == SHAPE
    assert c(None, 0, 128, 0, None, None, None) == OK
    assert c(A, 4, 128, 0, None, A, None) == NULL
    assert c(A, 4, 128, 0, A, U, None) == ALIGN


def test_linear_validation(lib):
    f = lib.sparse_fp8_rowwise_linear
    good = dict(xq=A, xd=0, xs=A, m=4, k=256, v=A, meta=A, wd=0, ws=A, n=32, bias=None, out=A, od=0)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["xq"], a["xd"], a["xs"], a["m"], a["k"], a["v"], a["meta"], a["wd"], a["ws"], a["n"],
                 a["bias"], a["out"], a["od"], None)

    assert call(xd=2) == DTYPE
    assert call(wd=5) == DTYPE
    assert call(od=3) == DTYPE
    assert call(k=192) == SHAPE
    assert call(k=0) == SHAPE
    assert call(n=24) == SHAPE
    assert call(m=-1) == SHAPE
    assert call(m=(1 << 30) + 1) == SHAPE
    assert call(m=0, xq=None, xs=None, out=None) == OK
    assert call(n=0, v=None, meta=None, ws=None) == OK
    assert call(xq=None) == NULL
    assert call(meta=None) == NULL
    assert call(out=None) == NULL
    assert call(ws=U) == ALIGN
    assert call(bias=U) == ALIGN
    assert call(out=U) == ALIGN


def test_tensorwise_quantize_validation(lib):
    wb = lib.sfr_quantize_tensorwise_workspace_bytes
    assert wb(8192, 4096) == 4096                       # 1024 blocks of 4096 chunks
    assert wb(16, 4096) == 4 * (16 * 4096 // 8 // 256)  # blocks of 256 chunks
    assert wb(1, 8) == 4
    assert wb(4, 15) == 0 and wb(0, 16) == 0 and wb(-1, 16) == 0
    q = lib.quantize_tensorwise_fp8
    need = wb(4, 16)
    assert q(A, 4, 16, 2, A, A, A, need, None) == DTYPE
    assert q(A, 4, 15, 0, A, A, A, need, None) == SHAPE
    assert q(A, 4, 0, 0, A, A, A, need, None) == SHAPE
    assert q(A, 4, 16, 0, A, A, A, need - 1, None) == SHAPE    # workspace too small
    assert q(None, 0, 16, 0, None, None, None, 0, None) == OK   # empty: no-op
    assert q(None, 4, 16, 0, A, A, A, need, None) == NULL
    assert q(A, 4, 16, 0, A, A, None, need, None) == NULL
    assert q(A, 4, 16, 0, A, U, A, need, None) == ALIGN
    assert q(A, 4, 16, 0, A, A, U, need, None) == ALIGN


def test_scaled_linear_validation(lib):
    f = lib.sparse_fp8_scaled_linear
    good = dict(xq=A, xd=0, xs=A, xk=0, m=4, k=256, v=A, meta=A, wd=0, ws=A, wk=1, n=32, bias=None, out=A, od=0)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["xq"], a["xd"], a["xs"], a["xk"], a["m"], a["k"], a["v"], a["meta"], a["wd"], a["ws"], a["wk"],
                 a["n"], a["bias"], a["out"], a["od"], None)

    assert call(xk=2) == DTYPE
    assert call(wk=-1) == DTYPE
    assert call(xd=3) == DTYPE
    assert call(k=192) == SHAPE
    assert call(n=8) == SHAPE
    assert call(m=0, xq=None, xs=None, out=None) == OK
    assert call(xs=None) == NULL
    assert call(ws=U) == ALIGN


def test_dynamic_linear_validation(lib):
    f = lib.sparse_fp8_rowwise_linear_dynamic
    good = dict(x=A, xd=0, m=4, k=1024, v=A, meta=A, wd=1, ws=A, wk=0, n=32, bias=None, out=A, od=0, xq=A, xs=A)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["x"], a["xd"], a["m"], a["k"], a["v"], a["meta"], a["wd"], a["ws"], a["wk"], a["n"], a["bias"],
                 a["out"], a["od"], a["xq"], a["xs"], None)

    assert call(xd=7) == DTYPE
    assert call(wk=3) == DTYPE
    assert call(k=1000) == SHAPE
    assert call(n=40) == SHAPE
    assert call(m=0, x=None, xq=None, xs=None, out=None) == OK
    assert call(xq=None) == NULL
    assert call(xs=None) == NULL
    assert call(xs=U) == ALIGN
    assert call(x=U) == ALIGN


F8 = 0x100   # SFR_ALGO_ACC_F8


def test_prune_validation(lib):
    p = lib.prune_2to4_bf16
    assert p(A, 4, 12, A, None) == SHAPE          # k % 8
    assert p(A, 4, 0, A, None) == SHAPE
    assert p(A, -1, 8, A, None) == SHAPE
    assert p(None, 0, 8, None, None) == OK         # no rows
    assert p(None, 4, 8, A, None) == NULL
    assert p(A, 4, 8, None, None) == NULL
    assert p(U, 4, 8, A, None) == ALIGN
    assert p(A, 4, 8, U, None) == ALIGN


def test_linear_algos(lib):
    names = [lib.sfr_linear_algo_name(i) for i in range(lib.sfr_linear_algo_count())]
    assert names == [b"decode_lds", b"decode_reg", b"tiled_64x64", b"tiled_128x128", b"tiled_256x256",
                     None, b"decode_lds_32", b"tiled_256x128"]
    f8 = [lib.sfr_linear_algo_name(i | F8) for i in range(lib.sfr_linear_algo_count())]
    assert f8 == [n + b"+f8acc" for n in (b"decode_lds", b"decode_reg", b"tiled_64x64", b"tiled_128x128",
                                          b"tiled_256x256", b"wide_256x256", b"decode_lds_32", b"tiled_256x128")]
    for a in (8, -1, 5, 8 | F8, 0x200, 0x300, 1 << 20):
        assert lib.sfr_linear_algo_name(a) is None and lib.sfr_linear_algo_valid(a) == 0, a
    assert all(lib.sfr_linear_algo_valid(a) == 1 for a in (0, 4, 6, 7, 0 | F8, 5 | F8, 6 | F8, 7 | F8))
    sup = lambda a, m, n, k: lib.sfr_linear_algo_supported(a, m, n, k)
    # each accumulation supports the same shapes per configuration (the
    # pipelined kernel only with FP8 accumulation)
    for a in (0, 1, 2, 3, 4, 6, 7):
        for shape in ((64, 4096, 4096), (65, 4096, 4096), (4, 4096, 640), (16, 4096, 640), (17, 4096, 640),
                      (5000, 4096, 256), (4, 4112, 1024)):
            assert sup(a, *shape) == sup(a | F8, *shape), (a, shape)
    assert sup(5, 5000, 4096, 512) == 0 and sup(5 | F8, 5000, 4096, 512) == 1   # pipelined: FP8, k >= 512
    assert sup(5 | F8, 5000, 4096, 384) == 0
    assert sup(0, 64, 4096, 4096) == 1 and sup(0, 65, 4096, 4096) == 0      # unit decode: m <= 64
    assert sup(6, 64, 4096, 4096) == 1 and sup(6, 65, 4096, 4096) == 0
    assert sup(0, 4, 4096, 640) == 0 and sup(0, 4, 4096, 17408) == 1        # unit decode: k % 1024, any K
    assert sup(6, 4, 4096, 1024) == 1 and sup(6, 4, 4112, 1024) == 0        # 32 rows per workgroup: n % 32
    assert sup(1, 16, 4096, 640) == 1 and sup(1, 17, 4096, 640) == 0
    assert all(sup(a, 5000, 4096, 256) == 1 for a in (2, 3, 4, 7))
    assert sup(2, 4, 100, 256) == 0 and sup(8, 4, 128, 256) == 0           # bad n, unknown id
    # the built-in choice
    d = lib.sfr_linear_default_algo
    assert d(1, 4096, 4096) == 0 and d(16, 4096, 14336) == 0 and d(16, 4096, 17408) == 0
    assert d(1, 14336, 4096) == 0 and d(4, 14336, 4096) == 6 and d(16, 6144, 4096) == 6
    assert d(16, 6144, 640) == 1 and d(4, 6160, 4096) == 0
    assert d(8192, 14336, 4096) == 4 and d(8192, 14336, 6144) == 4 and d(8192, 4096, 14336) == 4 and d(8192, 14336, 256) == 4
    assert d(512, 14336, 4096) == 7 and d(512, 4096, 4096) == 2 and d(512, 6144, 4096) == 2
    # 256x256 tiles from 2/3 of the 128x128 configuration's rounds (256 CUs without a GPU)
    assert d(1024, 14336, 4096) == 4 and d(4096, 4096, 14336) == 4 and d(2048, 6144, 4096) == 4
    # one round of 256x128 tiles over 3/4 .. all of the CUs
    assert d(2048, 4096, 4096) == 7 and d(2048, 4096, 14336) == 7 and d(1024, 6144, 4096) == 7
    assert d(1024, 4096, 4096) == 3 and d(1024, 4096, 14336) == 3 and d(3072, 4096, 4096) == 4
    # 17..64 rows: unit decode over 16-row blocks, except above 32 rows when
    # the 64x64 tiles cover about 3/4 of the CUs
    assert d(17, 4096, 4096) == 0 and d(32, 4096, 4096) == 6 and d(64, 6144, 4096) == 6
    assert d(17, 14336, 4096) == 6 and d(48, 14336, 4096) == 2 and d(64, 4096, 14336) == 6
    assert d(64, 4096, 640) == 2 and d(65, 4096, 4096) == 2


def test_linear_algo_validation(lib):
    f = lib.sparse_fp8_scaled_linear_algo
    good = dict(xq=A, xd=0, xs=A, xk=0, m=4, k=256, v=A, meta=A, wd=0, ws=A, wk=0, n=32, bias=None, out=A, od=0,
                algo=-1)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["xq"], a["xd"], a["xs"], a["xk"], a["m"], a["k"], a["v"], a["meta"], a["wd"], a["ws"], a["wk"],
                 a["n"], a["bias"], a["out"], a["od"], a["algo"], None)

    assert call(algo=8) == DTYPE and call(algo=-2) == DTYPE
    assert call(algo=5) == DTYPE                  # the pipelined kernel: FP8 accumulation only
    assert call(algo=0x200) == DTYPE and call(algo=8 | F8) == DTYPE
    assert call(algo=0) == SHAPE                  # k = 256: not a multiple of 1024
    assert call(algo=0 | F8) == SHAPE
    assert call(algo=5 | F8) == SHAPE             # k < 512
    assert call(algo=1, xq=None) == NULL          # supported: validation goes on
    assert call(algo=2, m=0, xq=None, xs=None, out=None) == OK


def test_algo_table_buckets():
    import sparse_fp8_row_amd as sfr
    assert [sfr.m_bucket(m) for m in (1, 2, 4, 5, 16, 17, 8192, 9000)] == [1, 4, 4, 16, 16, 64, 1 << 62, 1 << 62]


def test_binding_rejects_host_tensors():
    import torch
    import sparse_fp8_row_amd as sfr
    with pytest.raises(ValueError):
        sfr.quantize_rowwise_fp8(torch.zeros((2, 16), dtype=torch.bfloat16))


def test_bsr_validation(lib):
    c, fl, li = lib.bsr_count_bf16, lib.bsr_fill_bf16, lib.bsr_linear_bf16
    assert c(A, 96, 128, A, None) == SHAPE               # n % 64
    assert c(A, 64, 100, A, None) == SHAPE               # k % 64
    assert c(A, 64, 0, A, None) == SHAPE
    assert c(A, -64, 64, A, None) == SHAPE
    assert c(A, 64, 64, None, None) == NULL
    assert c(None, 64, 64, A, None) == NULL
    assert c(U, 64, 64, A, None) == ALIGN
    assert c(A, 64, 64, A + 2, None) == ALIGN            # crow: 4-byte aligned
    assert fl(A, 64, 96, A, A, A, None) == SHAPE
    assert fl(None, 0, 64, None, None, None, None) == OK  # no block rows: nothing to do
    assert fl(None, 64, 64, A, A, A, None) == NULL
    assert fl(A, 64, 64, A, A + 1, A, None) == ALIGN
    assert fl(A, 64, 64, A, A, U, None) == ALIGN
    assert li(A, 4, 128, A, A, A, 64, None, A, 2, None) == DTYPE
    assert li(A, 4, 96, A, A, A, 64, None, A, 0, None) == SHAPE      # k % 64
    assert li(A, 4, 128, A, A, A, 80, None, A, 0, None) == SHAPE     # n % 64
    assert li(A, -1, 128, A, A, A, 64, None, A, 0, None) == SHAPE
    assert li(None, 0, 128, None, None, None, 64, None, None, 0, None) == OK   # empty
    assert li(A, 4, 128, A, A, A, 0, None, A, 0, None) == OK
    assert li(None, 4, 128, A, A, A, 64, None, A, 0, None) == NULL
    assert li(A, 4, 128, None, A, A, 64, None, A, 0, None) == NULL
    assert li(A, 4, 128, A, A, A, 64, None, None, 1, None) == NULL
    assert li(U, 4, 128, A, A, A, 64, None, A, 0, None) == ALIGN
    assert li(A, 4, 128, A, A, A, 64, U, A, 0, None) == ALIGN        # bias
    assert li(A, 4, 128, A, A + 2, A, 64, None, A, 0, None) == ALIGN  # col
