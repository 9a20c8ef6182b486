"""Pins for the oracle's linear layer (CPU only).

Checks: on the smoke shape, torch's float64 matmul of the decoded operands is
exact (products are multiples of 2^-18 below 2^18, sums stay under 2^53 units),
so it reproduces the oracle's exact result bit for bit; an exact Python-integer
brute force on tiny shapes for all four dtype pairs; one-hot weights gather
single activations; binary32 accumulation stays within the gamma_K bound of
the exact sum; bias enters once; sampled evaluation equals the full one.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import sfr_inputs

FMTS = [oracle.E4M3, oracle.E5M2]


def random_operands(m, n, k, xfmt, wfmt, seed, bias=False):
    rng = np.random.default_rng(seed)
    xb = sfr_inputs.to_bf16_bits(rng.standard_normal((m, k)))
    wb = sfr_inputs.to_bf16_bits(rng.normal(0, 0.02, (n, k)))
    xq, xs = oracle.quantize_rows(xb, xfmt)
    wq, ws = oracle.quantize_rows(wb, wfmt)
    values, meta = oracle.compress_2to4(wq)
    b = sfr_inputs.to_bf16_bits(rng.normal(0, 0.01, n)) if bias else None
    return xq, xs, values, meta, ws, b


def test_smoke_shape_vs_torch_float64():
    case = sfr_inputs.smoke_case()
    xb = sfr_inputs.draw_x(case)
    wb = sfr_inputs.draw_w(case)
    xq, xs = oracle.quantize_rows(xb, oracle.E4M3)
    wq, ws = oracle.quantize_rows(wb, oracle.E4M3)
    values, meta = oracle.compress_2to4(wq)
    r = oracle.linear(xq, oracle.E4M3, xs, values, meta, oracle.E4M3, ws)
    xd = torch.from_numpy(oracle.fp8_decode(xq, oracle.E4M3))
    wd = torch.from_numpy(oracle.fp8_decode(oracle.decompress_2to4(values, meta), oracle.E4M3))
    S = (xd @ wd.T).numpy()
    t = xs.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]
    assert np.array_equal(r["y"], S * t)
    assert np.array_equal(r["bf16"], oracle.bf16_from_double(S * t))


@pytest.mark.parametrize("xfmt,wfmt", list(itertools.product(FMTS, FMTS)))
def test_exact_integer_brute_force(xfmt, wfmt):
    m, n, k = 3, 4, 16
    xq, xs, values, meta, ws, b = random_operands(m, n, k, xfmt, wfmt, 10 + 2 * xfmt + wfmt, bias=True)
    # exaggerate the range: a few large codes
    xq[0, :4] = [0x7E if xfmt == 0 else 0x7B, 0x01, 0x80 | 0x7A, 0x02]
    r = oracle.linear(xq, xfmt, xs, values, meta, wfmt, ws, bias=b)
    wq = oracle.decompress_2to4(values, meta)
    from fractions import Fraction
    xv = oracle.fp8_decode(xq, xfmt)
    wv = oracle.fp8_decode(wq, wfmt)
    for i in range(m):
        for j in range(n):
            S = sum(Fraction(float(xv[i, q])) * Fraction(float(wv[j, q])) for q in range(k))
            Sa = sum(abs(Fraction(float(xv[i, q])) * Fraction(float(wv[j, q]))) for q in range(k))
            t = Fraction(float(xs[i])) * Fraction(float(ws[j]))
            bias = Fraction(float(oracle.bf16_to_float(b[j:j + 1])[0]))
            y = S * t + bias
            assert abs(Fraction(float(r["y"][i, j])) - y) <= abs(y) * Fraction(1, 2**51)
            assert Fraction(float(r["sabs"][i, j])) == Fraction(float(Sa)) * t or \
                abs(Fraction(float(r["sabs"][i, j])) - Sa * t) <= Sa * t / 2**51


def test_one_hot_weight_gathers():
    m, n, k = 5, 8, 64
    rng = np.random.default_rng(3)
    xq = rng.integers(0, 0x7E, (m, k), dtype=np.uint8) | (rng.integers(0, 2, (m, k), dtype=np.uint8) << 7)
    xs = np.ones(m, np.float32)
    ws = np.ones(n, np.float32)
    wq = np.zeros((n, k), np.uint8)
    pos = rng.integers(0, k, n)
    wq[np.arange(n), pos] = 0x38           # 1.0 in e4m3
    values, meta = oracle.compress_2to4(wq)
    r = oracle.linear(xq, oracle.E4M3, xs, values, meta, oracle.E4M3, ws)
    xv = oracle.fp8_decode(xq, oracle.E4M3)
    assert np.array_equal(r["y"], xv[:, pos])


@pytest.mark.parametrize("xfmt,wfmt", [(0, 0), (1, 1), (0, 1)])
def test_acc32_within_gamma_bound(xfmt, wfmt):
    m, n, k = 8, 16, 1024
    xq, xs, values, meta, ws, _ = random_operands(m, n, k, xfmt, wfmt, 4)
    r = oracle.linear(xq, xfmt, xs, values, meta, wfmt, ws)
    t = xs.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]
    S = r["y"] / t
    Sabs = r["sabs"] / t
    kk = k // 2                              # number of non-zero terms
    gamma = kk * 2.0**-24 / (1 - kk * 2.0**-24)
    assert np.all(np.abs(r["acc32"].astype(np.float64) - S) <= gamma * Sabs)


def test_bias_and_sampling_consistency():
    m, n, k = 12, 32, 256
    xq, xs, values, meta, ws, b = random_operands(m, n, k, 0, 0, 8, bias=True)
    full = oracle.linear(xq, 0, xs, values, meta, 0, ws, bias=b)
    nob = oracle.linear(xq, 0, xs, values, meta, 0, ws)
    bf = oracle.bf16_to_float(b).astype(np.float64)
    assert np.array_equal(full["y"], nob["y"] + bf[None, :])
    rows = np.array([11, 0, 5])
    cols = np.array([31, 2, 2, 17])
    part = oracle.linear(xq, 0, xs, values, meta, 0, ws, bias=b, rows=rows, cols=cols)
    for key in ("y", "acc32", "sabs", "bf16"):
        assert np.array_equal(part[key], full[key][np.ix_(rows, cols)])


def test_zero_scale_row_gives_bias():
    m, n, k = 2, 16, 128
    xq, xs, values, meta, ws, b = random_operands(m, n, k, 0, 0, 12, bias=True)
    xq[1] = 0
    xs[1] = 0
    r = oracle.linear(xq, 0, xs, values, meta, 0, ws, bias=b)
    assert np.array_equal(r["y"][1], oracle.bf16_to_float(b).astype(np.float64))
