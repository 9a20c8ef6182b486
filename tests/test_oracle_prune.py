"""Pins for the oracle's 2:4 pruning of the bf16 weight (CPU only).

The weight is pruned to 2:4 in bf16, before quantization: in each group of
four along k the two largest magnitudes survive (ties to the lower index,
+0.0 and -0.0 both zero), the others become +0.0 ("Add CUTLASS-based
row-wise scaled sparse FP8 kernel", pytorch/ao PR #1671: a 2:4 sparse
weight; the -0.0 rule of the same PR).

Pins: a Python sort of (-|value|, index) over every group of random,
tie-heavy and special-value inputs; hand-derived groups; and the
invariants at most two non-zeros per group, survivors bit-identical, pruning
idempotent, each row's largest magnitude kept (so a row's FP8 scale does not
change), and groups with at most two non-zero magnitudes keeping them.
"""
import numpy as np
import pytest

import oracle
import sfr_inputs


def bits_to_float(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def brute_prune(w):
    out = np.zeros_like(w)
    vals = np.abs(bits_to_float(w).astype(np.float64))
    n, k = w.shape
    for r in range(n):
        for g in range(k // 4):
            idx = sorted(range(4), key=lambda i: (-vals[r, 4 * g + i], i))[:2]
            for i in idx:
                out[r, 4 * g + i] = w[r, 4 * g + i]
    return out


def random_weights(seed):
    rng = np.random.default_rng(seed)
    normal = sfr_inputs.to_bf16_bits(rng.normal(0.0, 0.02, (64, 256)))
    # tie-heavy: a small alphabet with both zero signs, equal magnitudes of
    # both signs, a subnormal pair and the largest finite bf16
    alphabet = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x3C00, 0xBC00, 0x0001, 0x8001, 0x7F7F, 0xFF7F],
                        np.uint16)
    ties = rng.choice(alphabet, (64, 256))
    hard = normal.copy()
    hard[rng.random(hard.shape) < 0.3] = 0x8000
    hard[rng.random(hard.shape) < 0.1] = 0x0000
    return [normal, ties, hard]


@pytest.mark.parametrize("seed", [1, 2])
def test_matches_brute_force(seed):
    for w in random_weights(seed):
        assert np.array_equal(oracle.prune_2to4_bf16(w), brute_prune(w))


def test_hand_groups():
    cases = [
        # (group, survivors' positions)
        ([0x3F80, 0xBF80, 0x3F80, 0x0000], (0, 1)),      # |1| three times: lower indices
        ([0x8000, 0x0000, 0x0000, 0x4000], (0, 3)),      # 2.0, then the first zero (-0.0)
        ([0x0000, 0x8000, 0x0000, 0x8000], (0, 1)),      # all zero: the first two
        ([0x3C00, 0xC000, 0x0001, 0x4000], (1, 3)),      # -2 and 2 outrank 2^-7 and a subnormal
        ([0x0001, 0x8001, 0x0000, 0x8000], (0, 1)),      # subnormals outrank zeros
        ([0x7F7F, 0x3F80, 0xFF7F, 0x3F80], (0, 2)),      # largest finite of both signs
    ]
    for g, keep in cases:
        w = np.array([g], np.uint16)
        want = np.array([[g[i] if i in keep else 0x0000 for i in range(4)]], np.uint16)
        assert np.array_equal(oracle.prune_2to4_bf16(w), want), (g, keep)


@pytest.mark.parametrize("seed", [3, 4])
def test_invariants(seed):
    for w in random_weights(seed):
        p = oracle.prune_2to4_bf16(w)
        v = bits_to_float(p).reshape(p.shape[0], -1, 4)
        assert ((v != 0).sum(axis=2) <= 2).all()
        kept = p != 0
        assert np.array_equal(p[kept], w[kept])                         # survivors keep their bits
        assert np.array_equal(oracle.prune_2to4_bf16(p), p)              # idempotent
        a_in = np.abs(bits_to_float(w)).max(axis=1)
        a_out = np.abs(bits_to_float(p)).max(axis=1)
        assert np.array_equal(a_in, a_out)                               # row amax survives
        # groups with at most two non-zero magnitudes keep every non-zero
        g_in = bits_to_float(w).reshape(w.shape[0], -1, 4)
        few = (g_in != 0).sum(axis=2) <= 2
        assert np.array_equal(g_in[few] != 0, v[few] != 0)
        # dropped entries are +0.0
        dropped = (p == 0) & (w != 0)
        assert (p[dropped] == 0x0000).all()


def test_row_scale_unchanged_by_pruning():
    # a row's FP8 scale only depends on its largest magnitude, which survives
    rng = np.random.default_rng(6)
    w = sfr_inputs.to_bf16_bits(rng.normal(0.0, 0.02, (32, 512)))
    for fmt in (oracle.E4M3, oracle.E5M2):
        _, s0 = oracle.quantize_rows(w, fmt)
        _, s1 = oracle.quantize_rows(oracle.prune_2to4_bf16(w), fmt)
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))


def test_prepare_weight_compresses_the_survivors():
    # after pruning in bf16, compression only picks survivors: decompressing
    # gives the quantized pruned weight (with -0.0 written as +0.0)
    rng = np.random.default_rng(7)
    w = sfr_inputs.to_bf16_bits(rng.normal(0.0, 0.02, (16, 256)))
    for fmt in (oracle.E4M3, oracle.E5M2):
        v, m, s, pruned = oracle.prepare_weight(w, fmt)
        q, s2 = oracle.quantize_rows(pruned, fmt)
        assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))
        q = np.where(q == 0x80, np.uint8(0), q)
        assert np.array_equal(oracle.decompress_2to4(v, m), q)
