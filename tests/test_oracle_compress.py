"""Pins for the oracle's 2:4 selection, compression and decompression (CPU only).

Checks: the two independent formulations of the selection (ranking, pairs)
agree over the whole 2^32 space of 4-byte groups; a Python sort-based brute
force agrees on random groups; hand-derived groups (tests/golden/
compress_groups.txt); and the invariants exactly two kept per group, valid
nibbles, decompress(compress(w)) == prune(w), prune idempotent, no loss for
groups with at most two non-zero magnitudes, no 0x80 in the values.
"""
import os

import numpy as np
import pytest

import oracle

VALID_NIBBLES = {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}


def brute_select(g):
    keys = [b & 0x7F for b in g]
    order = sorted(range(4), key=lambda i: (-keys[i], i))
    return tuple(sorted(order[:2]))


def test_formulations_agree_on_all_groups():
    disagree, invalid = oracle.check_all_groups()
    assert disagree == 0 and invalid == 0


@pytest.mark.parametrize("formulation", [0, 1])
def test_brute_force_random_groups(formulation):
    rng = np.random.default_rng(5)
    # mix of uniform bytes and few-distinct-value groups (many ties)
    g1 = rng.integers(0, 256, (20000, 4), dtype=np.uint8)
    g2 = rng.choice(np.array([0x00, 0x80, 0x38, 0xB8, 0x01, 0x81], np.uint8), (20000, 4))
    g = np.concatenate([g1, g2])
    i0, i1 = oracle.select(g, formulation)
    for row, a, b in zip(g, i0, i1):
        assert (a, b) == brute_select(row.tolist())


def test_golden_groups(golden_dir):
    n = 0
    with open(os.path.join(golden_dir, "compress_groups.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            lhs, rhs = line.split("->")
            g = np.array([[int(t, 16) for t in lhs.split()]], np.uint8)
            v0, v1, nib = rhs.split()
            values, meta = oracle.compress_2to4(np.tile(g, (1, 2)))   # k = 8: groups 0 and 1
            assert values[0].tolist() == [int(v0, 16), int(v1, 16)] * 2
            assert meta[0, 0] == int(nib, 16) | (int(nib, 16) << 4)
            n += 1
    assert n >= 10


def _weights(n, k, seed):
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 256, (n, k), dtype=np.uint8)
    # finite codes only for half the rows, plenty of zeros / ties
    w[: n // 2] = rng.choice(np.array([0, 0x80, 0x38, 0xB8, 0x3C, 0x20, 0xA0, 0x7E], np.uint8), (n // 2, k))
    return w


def test_invariants():
    w = _weights(64, 512, 1)
    values, meta = oracle.compress_2to4(w)
    assert values.shape == (64, 256) and meta.shape == (64, 64)
    nibbles = np.stack([meta & 0xF, meta >> 4], axis=-1).reshape(64, 128)
    assert set(np.unique(nibbles).tolist()) <= VALID_NIBBLES
    assert not np.any(values == 0x80)
    dense = oracle.decompress_2to4(values, meta)
    pruned = oracle.prune_2to4(w)
    assert np.array_equal(dense, pruned)
    assert np.array_equal(oracle.prune_2to4(pruned), pruned)
    # exactly two slots per group come from the input (the others are 0x00)
    grp = pruned.reshape(64, 128, 4)
    src = w.reshape(64, 128, 4)
    kept_mask = np.zeros_like(grp, dtype=bool)
    i0 = nibbles & 3
    i1 = nibbles >> 2
    np.put_along_axis(kept_mask, i0[..., None], True, axis=2)
    np.put_along_axis(kept_mask, i1[..., None], True, axis=2)
    assert np.all(kept_mask.sum(axis=2) == 2)
    canon = np.where(src == 0x80, 0x00, src)
    assert np.array_equal(np.where(kept_mask, canon, 0), grp)


def test_no_loss_when_already_2to4():
    rng = np.random.default_rng(2)
    w = rng.integers(1, 0x7F, (32, 256), dtype=np.uint8) | (rng.integers(0, 2, (32, 256), dtype=np.uint8) << 7)
    # zero two random positions of each group, alternating +0 / -0
    g = w.reshape(32, 64, 4)
    for r in range(32):
        for j in range(64):
            z = rng.choice(4, 2, replace=False)
            g[r, j, z] = [0x00, 0x80][j % 2]
    values, meta = oracle.compress_2to4(w)
    dense = oracle.decompress_2to4(values, meta)
    assert np.array_equal(dense, np.where(w == 0x80, 0, w))
