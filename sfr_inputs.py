"""Seeded synthetic inputs for the sparse FP8 row-wise linear layer.

This module only draws inputs.  It holds none of the layer's arithmetic (no
quantization, no 2:4 selection, no products) and imports neither the HIP
library nor the CPU oracle, so both sides can take their inputs from it.

Workloads follow the layer shapes of Llama-3.1-8B (hidden 4096, MLP 14336,
fused qkv 6144) that the pytorch/ao pages run the method on through their
``generate.py`` script ("Add CUTLASS-based row-wise scaled sparse FP8 kernel",
PR #1671, item 5 of the ready-for-review comment).  No weights or prompts of
that model are used: values are drawn from the distributions listed per
config below, and the weight is drawn dense; its 2:4 magnitude pruning (in
bf16, before quantization) is the method's own first step, not the
generator's.

Random streams: ``numpy.random.Generator(PCG64(SeedSequence([seed, cfg_id,
tensor_id])))`` with tensor ids X=0, W=1, bias=2, outlier channels=3,
negative-zero positions=4, weight-zero positions=5.  Samples are drawn in
binary64, cast to binary32 by numpy, then to bf16 with torch's
round-to-nearest-even CPU cast.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

E4M3 = 0
E5M2 = 1
DTYPE_NAMES = {E4M3: "e4m3", E5M2: "e5m2"}

T_X, T_W, T_BIAS, T_OUTLIER, T_NEGZERO, T_WZERO = range(6)

# Llama-3.1-8B linear shapes (N, K): fused qkv, attention output, gate/up, down.
LLAMA_SHAPES = {"qkv": (6144, 4096), "o": (4096, 4096), "up": (14336, 4096), "down": (4096, 14336)}


@dataclass(frozen=True)
class Case:
    """One parity / benchmark case."""
    cfg: str
    cfg_id: int
    m: int
    n: int
    k: int
    x_fmt: int = E4M3
    w_fmt: int = E4M3
    bias: bool = False
    seed: int = 0
    hard: bool = False          # Student-t activations with outliers and -0.0 entries

    @property
    def name(self) -> str:
        b = "+bias" if self.bias else ""
        return (f"{self.cfg}:M{self.m}N{self.n}K{self.k}:{DTYPE_NAMES[self.x_fmt]}x"
                f"{DTYPE_NAMES[self.w_fmt]}{b}:s{self.seed}")


def smoke_case() -> Case:
    """Tiny smoke: M=32, K=256, N=128, e4m3 x e4m3, no bias, seed 0."""
    return Case("smoke", 1, 32, 128, 256)


def decode_cases():
    """Decode-shaped: M in {1,4,16} and batched decode M in {32,64}, K=N=4096,
    e4m3 x e4m3, bf16 bias ~N(0,0.01)."""
    return [Case("decode", 2, m, 4096, 4096, bias=True) for m in (1, 4, 16, 32, 64)]


def prefill_up_case() -> Case:
    """Prefill MLP up-projection: M=8192, K=4096, N=14336, e4m3 x e4m3, no bias."""
    return Case("prefill_up", 3, 8192, 14336, 4096)


def prefill_down_hard_case() -> Case:
    """Prefill MLP down-projection with hard values: M=8192, K=14336, N=4096,
    Student-t(3) activations with 1% outlier channels (x50) and 0.1% exact -0.0
    entries, weight with 10% +/-0.0 entries; activation e4m3, weight e5m2."""
    return Case("prefill_down_hard", 4, 8192, 4096, 14336, x_fmt=E4M3, w_fmt=E5M2, hard=True)


def sweep_cases(seeds=(0, 1, 2)):
    """Llama-3.1-8B layer sweep: 4 shapes x M in {1,16,512,8192} x 4 dtype pairs x seeds."""
    out = []
    for _, (n, k) in LLAMA_SHAPES.items():
        for m in (1, 16, 512, 8192):
            for xf in (E4M3, E5M2):
                for wf in (E4M3, E5M2):
                    for s in seeds:
                        out.append(Case("sweep", 5, m, n, k, x_fmt=xf, w_fmt=wf, seed=s))
    return out


def _rng(seed: int, cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, tensor_id])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """binary64/32 samples -> bf16 bit patterns (uint16) via torch's RNE cast."""
    import torch
    f32 = np.ascontiguousarray(a, dtype=np.float32)
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw_x(case: Case, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Activation X as bf16 bits [M, K] (or only the listed rows)."""
    g = _rng(case.seed, case.cfg_id, T_X)
    m, k = case.m, case.k
    if not case.hard:
        x = g.standard_normal((m, k))
    else:
        x = g.standard_t(3.0, size=(m, k))
        n_out = int(0.01 * k)
        ch = _rng(case.seed, case.cfg_id, T_OUTLIER).choice(k, size=n_out, replace=False)
        x[:, ch] *= 50.0
    bits = to_bf16_bits(x)
    if case.hard:
        n_nz = int(0.001 * m * k)
        pos = _rng(case.seed, case.cfg_id, T_NEGZERO).choice(m * k, size=n_nz, replace=False)
        bits.reshape(-1)[pos] = 0x8000
    if rows is not None:
        bits = np.ascontiguousarray(bits[rows])
    return bits


def draw_w(case: Case) -> np.ndarray:
    """Dense weight W as bf16 bits [N, K], ~N(0, 0.02)."""
    g = _rng(case.seed, case.cfg_id, T_W)
    n, k = case.n, case.k
    w = g.normal(0.0, 0.02, size=(n, k))
    if case.hard:
        n_z = int(0.1 * n * k)
        gz = _rng(case.seed, case.cfg_id, T_WZERO)
        pos = gz.choice(n * k, size=n_z, replace=False)
        sign = gz.integers(0, 2, size=n_z)
        w.reshape(-1)[pos] = np.where(sign == 1, -0.0, 0.0)
    return to_bf16_bits(w)


def draw_bias(case: Case) -> Optional[np.ndarray]:
    """bf16 bias bits [N] ~N(0, 0.01), or None."""
    if not case.bias:
        return None
    g = _rng(case.seed, case.cfg_id, T_BIAS)
    return to_bf16_bits(g.normal(0.0, 0.01, size=case.n))


# --------------------------------------------------------------------------
# Block-sparse (BSR) workload ("promote blocksparse from prototype, make it
# faster", pytorch/ao PR #1734): 64 x 64 blocks, sparsity level 0.9, Llama
# shapes, decode batches padded up to 16 rows.  The generator draws a dense
# bf16 weight ~N(0, 0.02) and zeroes every block outside a seeded choice of
# round(keep * blocks) blocks (chosen over the whole matrix, so block rows keep
# different numbers of blocks); with ``special`` some dropped blocks hold -0.0
# entries and one kept block holds a single subnormal.  Stream ids: mask 6,
# special entries 7 (weight values use T_W, activations T_X, bias T_BIAS).
# --------------------------------------------------------------------------
T_BLOCKMASK, T_BLOCKSPECIAL = 6, 7
BSR_BLOCK = 64
BSR_SPARSITY = 0.9


def draw_bsr_w(case: Case, sparsity: float = BSR_SPARSITY, special: bool = False) -> np.ndarray:
    """Block-sparse weight as bf16 bits [N, K] (N, K multiples of 64)."""
    n, k, bs = case.n, case.k, BSR_BLOCK
    assert n % bs == 0 and k % bs == 0
    w = draw_w(Case(case.cfg, case.cfg_id, case.m, n, k, seed=case.seed))
    nb = (n // bs) * (k // bs)
    keep = int(round((1.0 - sparsity) * nb))
    kept = np.zeros(nb, bool)
    kept[_rng(case.seed, case.cfg_id, T_BLOCKMASK).choice(nb, size=keep, replace=False)] = True
    kept = kept.reshape(n // bs, k // bs)
    w = np.where(np.kron(kept, np.ones((bs, bs), bool)), w, np.uint16(0))
    if special:
        g = _rng(case.seed, case.cfg_id, T_BLOCKSPECIAL)
        dropped = np.argwhere(~kept)
        for br, bc in dropped[: max(1, len(dropped) // 10)]:
            blk = w[br * bs:(br + 1) * bs, bc * bs:(bc + 1) * bs]
            blk[g.random((bs, bs)) < 0.2] = 0x8000
        if len(dropped) > 1:
            br, bc = dropped[-1]
            w[br * bs + 3, bc * bs + 60] = 0x0001
    return np.ascontiguousarray(w)
