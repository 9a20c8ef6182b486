"""Pins for the oracle's row-wise FP8 quantization (CPU only).

Checks: hand-derived rows (tests/golden/quantize_rows.txt); an independent
pipeline built from library routines (for the row-wise and the tensor-wise
variant) (numpy binary64 division rounded to
binary32, which equals binary32 division because 53 >= 2*24+2, then torch's
FP8 cast); the invariants scale*fmax == amax within one binary32 rounding, the
amax element hitting +/-fmax, the per-element error bound, -0.0 handling, zero
rows, subnormal scales and column-permutation invariance.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import sfr_inputs

TORCH_FP8 = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}
CMAX = {oracle.E4M3: 0x7E, oracle.E5M2: 0x7B}


def load_golden(golden_dir):
    cases = []
    with open(os.path.join(golden_dir, "quantize_rows.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            if line.startswith("case"):
                _, fmt, sc = line.split()
                cases.append({"fmt": oracle.E4M3 if fmt == "e4m3" else oracle.E5M2,
                              "scale": int(sc, 16), "x": [], "q": []})
            else:
                for pair in line.split():
                    xb, qb = pair.split(":")
                    cases[-1]["x"].append(int(xb, 16))
                    cases[-1]["q"].append(int(qb, 16))
    return cases


def test_golden_rows(golden_dir):
    cases = load_golden(golden_dir)
    assert len(cases) == 5
    for c in cases:
        x = np.array([c["x"]], np.uint16)
        q, s = oracle.quantize_rows(x, c["fmt"])
        assert int(s.view(np.uint32)[0]) == c["scale"]
        assert q[0].tolist() == c["q"]


def independent_pipeline(x_bits, fmt):
    """numpy + torch: amax, scale and codes without the oracle's C code."""
    xf = oracle.bf16_to_float(x_bits).astype(np.float64)
    amax = np.max(np.abs(xf), axis=1)
    fmax = oracle.FMAX[fmt]
    scale = (amax / fmax).astype(np.float32)                       # RN32(RN64(a/b)) == RN32(a/b)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xf / scale.astype(np.float64)[:, None]).astype(np.float32)
    t = np.clip(t, -fmax, fmax)                                    # saturation
    codes = torch.from_numpy(np.ascontiguousarray(t)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    codes = codes.copy()
    zero = amax == 0
    codes[zero] = np.where(np.signbit(xf[zero]), 0x80, 0x00)
    scale[zero] = 0
    return codes, scale


def _rows(kind, rows, cols, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.standard_normal((rows, cols))
    elif kind == "student":
        x = rng.standard_t(3.0, (rows, cols))
        x[:, rng.choice(cols, max(1, cols // 100), replace=False)] *= 50
    elif kind == "wide":          # magnitudes spanning the whole bf16 range
        x = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-120, 120, (rows, 1)))
    elif kind == "tiny":          # amax small enough that the scale is subnormal
        x = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-133, -118, (rows, 1)))
    else:
        raise ValueError(kind)
    bits = sfr_inputs.to_bf16_bits(x)
    # sprinkle exact -0.0 and +0.0
    z = rng.random((rows, cols)) < 0.01
    bits[z] = np.where(rng.random(z.sum()) < 0.5, 0x8000, 0x0000)
    return bits


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("kind", ["normal", "student", "wide", "tiny"])
def test_matches_independent_pipeline(fmt, kind):
    x = _rows(kind, 64, 512, 3 + fmt)
    q, s = oracle.quantize_rows(x, fmt)
    q2, s2 = independent_pipeline(x, fmt)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(q, q2)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_invariants(fmt):
    x = np.concatenate([_rows("normal", 32, 256, 1), _rows("student", 32, 256, 2), _rows("wide", 32, 256, 5)])
    q, s = oracle.quantize_rows(x, fmt)
    xf = oracle.bf16_to_float(x).astype(np.float64)
    amax = np.abs(xf).max(axis=1)
    fmax = oracle.FMAX[fmt]
    # scale * fmax == amax up to the one rounding of the division (half an ulp:
    # relative 2^-24 for a normal scale, absolute 2^-150 for a subnormal one)
    bound = np.maximum(2.0**-24 * amax, 2.0**-150 * fmax)
    assert np.all(np.abs(s.astype(np.float64) * fmax - amax) <= bound)
    # the amax element maps to +/-fmax
    cmax = CMAX[fmt]
    arg = np.abs(xf).argmax(axis=1)
    qa = q[np.arange(len(q)), arg]
    assert np.all((qa & 0x7F) == cmax)
    # no NaN / inf codes
    dq = oracle.fp8_decode(q, fmt)
    assert np.all(np.isfinite(dq))
    assert np.all(np.abs(dq) <= fmax)
    # element error: |dec(q)*s - x| <= (half an FP8 step at x/s  +  the binary32 quotient error)*s
    t = xf / s.astype(np.float64)[:, None]
    at = np.abs(t)
    e = np.floor(np.log2(np.maximum(at, 1e-300)))
    mbits = 3 if fmt == oracle.E4M3 else 2
    emin = -6 if fmt == oracle.E4M3 else -14
    step = np.exp2(np.maximum(e, emin) - mbits)
    err = np.abs(dq - t)
    assert np.all(err <= 0.5 * step + 2.0**-23 * at + 1e-300)
    # signed zeros keep their sign
    nz = x == 0x8000
    assert np.all(q[nz] == 0x80)
    pz = x == 0x0000
    assert np.all(q[pz] == 0x00)


def test_zero_rows_and_subnormal_scale():
    x = np.zeros((3, 16), np.uint16)
    x[1, ::2] = 0x8000
    x[2, 3] = 0x0001                       # bf16 smallest subnormal 2^-133
    x[2, 5] = 0x8001
    for fmt in (oracle.E4M3, oracle.E5M2):
        q, s = oracle.quantize_rows(x, fmt)
        assert s[0] == 0 and s[1] == 0 and np.all(q[0] == 0) and np.all(q[1, ::2] == 0x80)
        assert np.all(q[1, 1::2] == 0)
        # row 2: amax = 2^-133, scale = fl32(2^-133 / fmax) is a binary32 subnormal
        assert 0 < s[2] < np.finfo(np.float32).tiny
        assert (q[2, 3] & 0x7F) == CMAX[fmt] and (q[2, 5] & 0x7F) == CMAX[fmt] and q[2, 5] & 0x80
        q2, s2 = independent_pipeline(x, fmt)
        assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))


def test_column_permutation_invariance():
    x = _rows("student", 16, 384, 9)
    perm = np.random.default_rng(0).permutation(384)
    q, s = oracle.quantize_rows(x, oracle.E4M3)
    qp, sp = oracle.quantize_rows(np.ascontiguousarray(x[:, perm]), oracle.E4M3)
    assert np.array_equal(s, sp)
    assert np.array_equal(q[:, perm], qp)


# ---- tensor-wise variant: one scale for the whole tensor ----

def independent_tensor_pipeline(x_bits, fmt):
    """numpy + torch, one amax over every element (no oracle C code)."""
    xf = oracle.bf16_to_float(x_bits).astype(np.float64)
    amax = np.max(np.abs(xf))
    fmax = oracle.FMAX[fmt]
    if amax == 0:
        return np.where(np.signbit(xf), 0x80, 0x00).astype(np.uint8), np.zeros(1, np.float32)
    scale = np.float32(amax / fmax)
    t = (xf / np.float64(scale)).astype(np.float32)
    t = np.clip(t, -fmax, fmax)
    codes = torch.from_numpy(np.ascontiguousarray(t)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy().copy()
    return codes, np.array([scale], np.float32)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("kind", ["normal", "student", "wide", "tiny"])
def test_tensorwise_matches_independent_pipeline(fmt, kind):
    # "wide" rows differ by up to 2^240 in magnitude: most rows quantize to 0
    x = _rows(kind, 48, 384, 11 + fmt)
    q, s = oracle.quantize_tensor(x, fmt)
    q2, s2 = independent_tensor_pipeline(x, fmt)
    assert s.shape == (1,)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(q, q2)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_tensorwise_special_cases(fmt):
    # one row: the same as the row-wise quantization
    x = _rows("student", 1, 1024, 21)
    q, s = oracle.quantize_tensor(x, fmt)
    qr, sr = oracle.quantize_rows(x, fmt)
    assert np.array_equal(q, qr) and s[0] == sr[0]
    # the row holding the global amax: its codes equal the row-wise ones; the
    # global amax element maps to +/-fmax, every other row's codes are those of
    # its own elements divided by the global scale
    x = _rows("normal", 16, 256, 22)
    xf = oracle.bf16_to_float(x)
    r = int(np.abs(xf).max(axis=1).argmax())
    q, s = oracle.quantize_tensor(x, fmt)
    qr, sr = oracle.quantize_rows(x[r:r + 1], fmt)
    assert s[0] == sr[0] and np.array_equal(q[r], qr[0])
    assert (q.reshape(-1)[np.abs(xf).argmax()] & 0x7F) == CMAX[fmt]
    # all-zero tensor: scale 0, signed zeros kept
    z = np.zeros((3, 64), np.uint16)
    z[1, ::3] = 0x8000
    q, s = oracle.quantize_tensor(z, fmt)
    assert s[0] == 0 and np.array_equal(q, np.where(z == 0x8000, 0x80, 0x00))


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_tensorwise_power_of_two_invariance(fmt):
    # scaling every element by 2^j (exact in bf16 away from its range limits)
    # scales amax and scale by 2^j and leaves every code unchanged
    x = _rows("normal", 24, 256, 23)
    xf = oracle.bf16_to_float(x).astype(np.float64)
    q, s = oracle.quantize_tensor(x, fmt)
    for j in (-20, -3, 5, 40):
        y = sfr_inputs.to_bf16_bits(xf * 2.0**j)
        qy, sy = oracle.quantize_tensor(y, fmt)
        assert np.array_equal(qy, q)
        assert sy[0] == np.float32(s[0] * np.float32(2.0**j))
