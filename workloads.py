"""Seeded synthetic workloads shared by the tests, the smoke check and the
benchmark.

This module holds no attention, softmax, quantisation or rotation
arithmetic: it only draws random numbers and names the workload shapes.  Both
the HIP path and the CPU oracle are fed from here.

Recipe (every tensor):
  * numpy Generator(PCG64(seed)) with seed = 1000 * (config_index + 1) + t,
    t = 0 for Q, 1 for K, 2 for V, 3/4/5 for the Q/K/V outlier masks and
    9 for the Hadamard sign vector;
  * standard normal float32 draws, C-contiguous [B, H, N, d] (K and V:
    [B, Hkv, N, d]);
  * outlier workloads: an independent Bernoulli(0.001) mask per entry, and
    the masked entries multiplied by 20;
  * bf16 workloads: the float32 draws cast to bf16 with round-to-nearest-even
    (torch's cast); the oracle reads those exact bf16 values.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed base = 1000 * (index + 1)
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool
    dtype: str          # "bf16" or "fp8"
    outliers: bool = False
    description: str = ""

    @property
    def flops(self) -> float:
        """4 * B * H * N^2 * d, halved for the causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def seed(self, t: int) -> int:
        return 1000 * (self.index + 1) + t


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_d64", 0, 1, 2, 2, 256, 64, False, "bf16",
                 description="B1 H2 N256 d64 non-causal; fp32 N(0,1) draws "
                             "rounded to bf16 for the GPU"),
        Workload("bf16_n4096", 1, 4, 16, 16, 4096, 128, False, "bf16",
                 description="B4 H16 N4096 d128 non-causal bf16"),
        Workload("bf16_causal_n8192", 2, 2, 32, 32, 8192, 128, True, "bf16",
                 description="B2 H32 N8192 d128 causal bf16"),
        Workload("bf16_causal_gqa_n16384", 3, 1, 32, 8, 16384, 128, True,
                 "bf16", description="B1 Hq32 Hkv8 N16384 d128 causal GQA "
                                     "bf16"),
        Workload("fp8_n8192", 4, 4, 16, 16, 8192, 128, False, "fp8",
                 outliers=True,
                 description="B4 H16 N8192 d128 non-causal e4m3, 0.1% x20 "
                             "outliers, with and without Hadamard rotation"),
        Workload("bf16_n8192", 5, 4, 16, 16, 8192, 128, False, "bf16",
                 description="B4 H16 N8192 d128 non-causal bf16 (headline "
                             "throughput shape)"),
    ]
}

HEADLINE = "bf16_n8192"


def draw(shape, seed: int, outliers: bool = False,
         outlier_seed: int | None = None) -> np.ndarray:
    """Standard normal float32 array of `shape`, optionally with 0.1% of the
    entries multiplied by 20 (mask drawn from its own seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if outliers:
        mrng = np.random.Generator(np.random.PCG64(
            outlier_seed if outlier_seed is not None else seed + 3))
        mask = mrng.random(size=shape, dtype=np.float32) < 1e-3
        x[mask] *= np.float32(20.0)
    return x


def qkv(B, H, Hkv, N, d, seed_base: int, outliers: bool = False):
    """float32 Q [B,H,N,d], K/V [B,Hkv,N,d] from seeds seed_base + 0/1/2
    (outlier masks from seed_base + 3/4/5)."""
    q = draw((B, H, N, d), seed_base + 0, outliers, seed_base + 3)
    k = draw((B, Hkv, N, d), seed_base + 1, outliers, seed_base + 4)
    v = draw((B, Hkv, N, d), seed_base + 2, outliers, seed_base + 5)
    return q, k, v


def workload_qkv(w: Workload):
    return qkv(w.B, w.H, w.Hkv, w.N, w.d, w.seed(0), w.outliers)


def hadamard_signs(d: int, seed: int) -> np.ndarray:
    """Random +-1 vector of length d (int8)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)


def to_bf16(x: np.ndarray):
    """float32 numpy -> torch bfloat16 CPU tensor (round to nearest even)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def bf16_values(t) -> np.ndarray:
    """torch bf16 tensor (any device) -> float32 numpy holding the exact same
    values (widening is exact)."""
    import torch
    return t.detach().to("cpu").to(torch.float32).numpy()


def pack_mask(mask) -> np.ndarray:
    """Boolean visibility mask [..., Nq, Nk] -> uint32 [..., Nq, ceil(Nk/32)]
    words: bit j % 32 of word j // 32 is set iff key j is visible.  A data
    format conversion only (the HIP path reads masks in this form)."""
    m = np.asarray(mask, dtype=bool)
    nk = m.shape[-1]
    nw = (nk + 31) // 32
    pad = np.zeros(m.shape[:-1] + (nw * 32,), dtype=bool)
    pad[..., :nk] = m
    bits = pad.reshape(m.shape[:-1] + (nw, 32)).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (bits * weights).sum(axis=-1).astype(np.uint32)


def random_mask(shape, p_visible: float, seed: int) -> np.ndarray:
    """Independent Bernoulli(p_visible) visibility per (query, key)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.random(shape) < p_visible


def block_sparse_mask(Nq: int, Nk: int, block: int, n_random: int,
                      seed: int) -> np.ndarray:
    """Boolean [Nq, Nk] mask made of block x block squares: query block i
    sees key block 0 (global), key blocks i - 1, i, i + 1 (local band) and
    n_random further key blocks drawn without replacement (seeded)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nqb = (Nq + block - 1) // block
    nkb = (Nk + block - 1) // block
    m = np.zeros((Nq, Nk), dtype=bool)
    for i in range(nqb):
        keep = {0, i - 1, i, i + 1}
        rest = [j for j in range(nkb) if j not in keep]
        pick = rng.choice(len(rest), size=min(n_random, len(rest)),
                          replace=False)
        keep |= {rest[t] for t in pick}
        for j in keep:
            if 0 <= j < nkb:
                m[i * block:(i + 1) * block, j * block:(j + 1) * block] = True
    return m
