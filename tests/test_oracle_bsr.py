"""Pins of the oracle's block-sparse (BSR, 64 x 64 blocks) weight and linear
layer ("promote blocksparse from prototype, make it faster", pytorch/ao PR
#1734), against things other than the oracle itself: scipy's BSR conversion,
numpy's binary64 matrix product over the dense weight, brute force on tiny
inputs, and closed forms."""
import numpy as np
import pytest
import scipy.sparse

import oracle

BS = oracle.BSR_BLOCK


def f32_to_bf16_bits(a):
    """bf16 bits of binary32 values that are exactly bf16 (low half zero)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def block_sparse_bits(rng, n, k, keep, special=True):
    """bf16 bits [n, k]: each 64 x 64 block kept with probability `keep`
    (values ~N(0, 1) rounded to bf16), else all +0.0; with `special`, a few
    dropped blocks hold only -0.0 (must stay dropped) and a few kept blocks
    hold a single subnormal (must be kept)."""
    v = rng.standard_normal((n, k)).astype(np.float32)
    w = f32_to_bf16_bits((v.view(np.uint32) & 0xFFFF0000).view(np.float32))
    mask = rng.random((n // BS, k // BS)) < keep
    full = np.kron(mask, np.ones((BS, BS), bool))
    w = np.where(full, w, np.uint16(0))
    if special:
        zb = np.argwhere(~mask)
        for br, bc in zb[: max(1, len(zb) // 8)]:
            blk = w[br * BS:(br + 1) * BS, bc * BS:(bc + 1) * BS]
            blk[rng.random(blk.shape) < 0.3] = 0x8000
        for br, bc in zb[len(zb) // 8: len(zb) // 8 + 2]:
            w[br * BS + 5, bc * BS + 7] = 0x0001          # smallest subnormal
    return w


@pytest.mark.parametrize("shape,keep,seed", [((128, 192), 0.5, 0), ((256, 512), 0.1, 1), ((64, 64), 1.0, 2),
                                             ((192, 320), 0.0, 3)])
def test_bsr_format_matches_scipy(shape, keep, seed):
    rng = np.random.default_rng(seed)
    n, k = shape
    w = block_sparse_bits(rng, n, k, keep)
    crow, col, values = oracle.bsr_from_dense(w)
    ref = scipy.sparse.bsr_matrix(oracle.bf16_to_float(w), blocksize=(BS, BS))
    ref.sort_indices()
    assert np.array_equal(crow, ref.indptr.astype(np.int32))
    assert np.array_equal(col, ref.indices.astype(np.int32))
    assert np.array_equal(oracle.bf16_to_float(values), ref.data.astype(np.float32))


def test_bsr_round_trip_and_zero_rules():
    rng = np.random.default_rng(5)
    n, k = 256, 384
    w = block_sparse_bits(rng, n, k, 0.3)
    crow, col, values = oracle.bsr_from_dense(w)
    back = oracle.bsr_to_dense(crow, col, values, n, k)
    kept = np.zeros((n // BS, k // BS), bool)
    for br in range(n // BS):
        kept[br, col[crow[br]:crow[br + 1]]] = True
    full = np.kron(kept, np.ones((BS, BS), bool))
    assert np.array_equal(back[full], w[full])              # kept blocks: every bit, -0.0 included
    assert np.all(back[~full] == 0)
    assert np.all((w[~full] & 0x7FFF) == 0)                  # dropped blocks held only zeros
    # a block whose only non-zero element is a NaN or an infinity is kept
    w2 = np.zeros((64, 128), np.uint16)
    w2[3, 70] = 0x7FC0
    w2[9, 2] = 0xFF80
    c2, k2, v2 = oracle.bsr_from_dense(w2)
    assert c2.tolist() == [0, 2] and k2.tolist() == [0, 1]


def test_bsr_linear_matches_numpy():
    rng = np.random.default_rng(7)
    m, n, k = 5, 256, 512
    w = block_sparse_bits(rng, n, k, 0.25, special=False)
    x = f32_to_bf16_bits((rng.standard_normal((m, k)).astype(np.float32).view(np.uint32) & 0xFFFF0000)
                         .view(np.float32))
    bias = f32_to_bf16_bits(np.float32(0.25) * np.arange(n, dtype=np.float32) % 3)
    crow, col, values = oracle.bsr_from_dense(w)
    ref = oracle.bsr_linear(x, crow, col, values, n, bias=bias)
    dense = oracle.bf16_to_float(x).astype(np.float64) @ oracle.bf16_to_float(w).astype(np.float64).T
    y_np = dense + oracle.bf16_to_float(bias).astype(np.float64)
    sabs = np.abs(oracle.bf16_to_float(x).astype(np.float64)) @ np.abs(oracle.bf16_to_float(w).astype(np.float64)).T
    assert np.allclose(ref["sabs"], sabs, rtol=1e-13, atol=0)
    assert np.all(np.abs(ref["y"] - y_np) <= 1e-13 * (sabs + 1))
    assert np.array_equal(ref["bf16"], oracle.bf16_from_double(ref["y"]))
    # a subset of positions gives the same values
    sub = oracle.bsr_linear(x, crow, col, values, n, bias=bias, rows=[4, 0], cols=[255, 3, 64])
    assert np.array_equal(sub["y"], ref["y"][np.ix_([4, 0], [255, 3, 64])])


def test_bsr_linear_brute_force_tiny():
    rng = np.random.default_rng(11)
    m, n, k = 3, 128, 192
    w = block_sparse_bits(rng, n, k, 0.5, special=False)
    x = f32_to_bf16_bits((rng.standard_normal((m, k)).astype(np.float32).view(np.uint32) & 0xFFFF0000)
                         .view(np.float32))
    crow, col, values = oracle.bsr_from_dense(w)
    ref = oracle.bsr_linear(x, crow, col, values, n)
    xf, wf = oracle.bf16_to_float(x), oracle.bf16_to_float(w)
    for i in range(m):
        for j in range(0, n, 7):
            s, f = 0.0, np.float32(0.0)
            for kk in range(k):                      # dense definition, ascending k
                p = float(xf[i, kk]) * float(wf[j, kk])
                s += p
                f = np.float32(f + np.float32(p))
            assert abs(ref["y"][i, j] - s) <= 1e-12 * (abs(s) + 1)
            assert ref["acc32"][i, j] == f


def test_bsr_linear_closed_forms():
    # identity weight: y = x exactly, and its bf16 rounding returns x's bits
    k = 128
    eye = np.zeros((k, k), np.uint16)
    eye[np.arange(k), np.arange(k)] = 0x3F80
    rng = np.random.default_rng(13)
    x = f32_to_bf16_bits((rng.standard_normal((4, k)).astype(np.float32).view(np.uint32) & 0xFFFF0000)
                         .view(np.float32))
    crow, col, values = oracle.bsr_from_dense(eye)
    r = oracle.bsr_linear(x, crow, col, values, k)
    assert np.array_equal(r["bf16"], x)
    # all-zero weight: no blocks, the output is the bias exactly
    z = np.zeros((192, 256), np.uint16)
    crow, col, values = oracle.bsr_from_dense(z)
    assert len(col) == 0 and np.all(crow == 0)
    bias = f32_to_bf16_bits(np.linspace(-2, 2, 192).astype(np.float32).view(np.uint32).__and__(0xFFFF0000)
                            .view(np.float32))
    r = oracle.bsr_linear(np.zeros((2, 256), np.uint16), crow, col, values, 192, bias=bias)
    assert np.array_equal(r["bf16"], np.broadcast_to(bias, (2, 192)))
    assert np.all(r["sabs"] == 0)
