"""Pins for the oracle's FP8 and bf16 codecs (CPU only).

The oracle's decode/encode are checked against (a) the OCP FP8 special-value
table in tests/golden/ofp8_table.txt, (b) torch's CPU float8 casts, a library
routine with round-to-nearest-even, and (c) closed forms of saturation, ties and
subnormals.  The bf16 rounding is checked against torch's float32->bfloat16 cast
and against hand-derived binary64 cases that a double rounding would get wrong.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

FMT = {"e4m3": oracle.E4M3, "e5m2": oracle.E5M2}
TORCH_FP8 = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


def torch_decode(codes, fmt):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(TORCH_FP8[fmt])
    return t.to(torch.float32).numpy().astype(np.float64)


def torch_encode(vals, fmt):
    t = torch.from_numpy(np.ascontiguousarray(vals, np.float32)).to(TORCH_FP8[fmt])
    return t.view(torch.uint8).numpy().copy()


def test_decode_matches_ofp8_table(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "ofp8_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    assert len(rows) >= 20
    for fmt_name, code, val in rows:
        got = oracle.fp8_decode(np.array([int(code, 16)]), FMT[fmt_name])[0]
        if val == "nan":
            assert np.isnan(got), (fmt_name, code)
        elif val in ("inf", "-inf"):
            assert got == float(val), (fmt_name, code)
        elif val == "-0":
            assert got == 0 and np.signbit(got), (fmt_name, code)
        else:
            assert Fraction(got) == Fraction(val), (fmt_name, code, got, val)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_all_codes_vs_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes, fmt)
    ref = torch_decode(codes, fmt)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_monotone_codes(fmt):
    # finite non-negative codes are ordered by value (the encoder's bisection relies on it)
    cmax = 0x7E if fmt == oracle.E4M3 else 0x7B
    v = oracle.fp8_decode(np.arange(cmax + 1, dtype=np.uint8), fmt)
    assert np.all(np.diff(v) > 0)
    # and the low-7-bit order is the magnitude order for both signs
    neg = oracle.fp8_decode(np.arange(cmax + 1, dtype=np.uint8) | 0x80, fmt)
    assert np.array_equal(np.abs(neg), v)


def _structured_floats():
    """All binary32 exponents x mantissas around every FP8 rounding point."""
    exps = np.arange(0, 255, dtype=np.uint32)
    hi = np.arange(0, 128, dtype=np.uint32) << 16          # top 7 mantissa bits
    lo = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x3FFF, 0x4000, 0xC000], dtype=np.uint32)
    mant = (hi[:, None] | lo[None, :]).reshape(-1)
    u = (exps[:, None] << 23 | mant[None, :]).reshape(-1)
    u = np.concatenate([u, u | 0x80000000])
    return u.view(np.float32)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_vs_torch_in_range(fmt):
    fmax = oracle.FMAX[fmt]
    rng = np.random.default_rng(7)
    rand = rng.integers(0, 2**32, size=4_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = np.concatenate([_structured_floats(), rand])
    v = v[np.isfinite(v) & (np.abs(v) <= fmax)]
    ours = oracle.fp8_encode(v, fmt)
    ref = torch_encode(v, fmt)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(ours[i]), hex(ref[i])) for i in bad[:8]]


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_saturates(fmt):
    fmax = oracle.FMAX[fmt]
    cmax = 0x7E if fmt == oracle.E4M3 else 0x7B
    v = np.array([fmax, fmax * 1.0001, fmax * 1.5, 1e30, 3.0e38, np.inf], np.float32)
    assert np.all(oracle.fp8_encode(v, fmt) == cmax)
    assert np.all(oracle.fp8_encode(-v, fmt) == (cmax | 0x80))


def test_encode_closed_forms():
    E4, E5 = oracle.E4M3, oracle.E5M2
    enc = lambda x, f: int(oracle.fp8_encode(np.array([x], np.float32), f)[0])
    # subnormal ties to even: 2^-10 is halfway between 0 and 2^-9 -> 0
    assert enc(2.0**-10, E4) == 0x00
    assert enc(3 * 2.0**-11, E4) == 0x01      # 0.75 of a quantum -> 1
    assert enc(3 * 2.0**-10, E4) == 0x02      # 1.5 quanta tie -> even (2)
    assert enc(5 * 2.0**-10, E4) == 0x02      # 2.5 quanta tie -> even (2)
    assert enc(2.0**-17, E5) == 0x00
    assert enc(3 * 2.0**-17, E5) == 0x02
    # normal ties: 1 + 1/16 lies halfway between 1 (0x38) and 1.125 (0x39) -> even 0x38
    assert enc(1.0625, E4) == 0x38
    assert enc(1.1875, E4) == 0x3A            # halfway 1.125/1.25 -> even 0x3A
    assert enc(1.125, E5) == 0x3C             # halfway 1/1.25 -> even 0x3C
    # signed zeros and underflow keep the sign
    assert enc(-0.0, E4) == 0x80 and enc(-0.0, E5) == 0x80
    assert enc(-1e-30, E4) == 0x80 and enc(1e-30, E4) == 0x00
    # 464 is halfway between 448 and the (non-existent) 480: saturates to 448
    assert enc(464.0, E4) == 0x7E and enc(470.0, E4) == 0x7E


def test_bf16_from_float32_vs_torch():
    rng = np.random.default_rng(11)
    rand = rng.integers(0, 2**32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    exps = np.arange(0, 255, dtype=np.uint32)
    lo = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x17FFF, 0x18000, 0x18001], dtype=np.uint32)
    hi = np.arange(0, 128, dtype=np.uint32) << 16
    structured = (exps[:, None] << 23 | (hi[:, None] | lo[None, :]).reshape(-1)[None, :]).reshape(-1)
    u = np.concatenate([rand, structured, structured | 0x80000000])
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.bf16_from_double(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(f[i]), hex(ours[i]), hex(ref[i])) for i in bad[:8]]


def test_bf16_from_double_closed_forms():
    b = lambda y: int(oracle.bf16_from_double(np.array([y]))[0])
    assert b(1.0) == 0x3F80
    assert b(1.0 + 2.0**-8) == 0x3F80               # exact tie -> even
    assert b(1.0 + 2.0**-8 + 2.0**-40) == 0x3F81    # just above the tie (binary32 would lose it)
    assert b(1.0 + 3 * 2.0**-8) == 0x3F82           # tie between 0x3F81 and 0x3F82 -> even
    assert b(-2.0) == 0xC000
    assert b(-0.0) == 0x8000 and b(0.0) == 0x0000
    top = (2 - 2.0**-7) * 2.0**127                  # largest finite bf16, 0x7F7F
    assert b(top) == 0x7F7F
    assert b((2 - 2.0**-8) * 2.0**127) == 0x7F80    # tie with 2^128 -> even -> inf
    assert b((2 - 2.0**-8) * 2.0**127 * (1 - 2.0**-30)) == 0x7F7F
    assert b(2.0**-133) == 0x0001                   # smallest bf16 subnormal
    assert b(2.0**-134) == 0x0000                   # tie -> even (0)
    assert b(2.0**-134 * (1 + 2.0**-20)) == 0x0001
