"""Seeded synthetic inputs for Prof-K exact top-k (shared by tests and bench.py).

This module draws random inputs and nothing else: it holds none of the
selection method's arithmetic.  The workloads stand in for the pages'
inputs ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
Selection": standard-normal float32 tensors in §5, the distributions of
App. E.3 Table 7, the uniform / normal / Pareto grid and the BatchTopK SAE
activation pool of the earlier version's §5); no dataset or model
activations are used.

Recipe.  An input of n values is cut into chunks of CHUNK = 2^24 values;
chunk c is drawn by numpy.random.Generator(PCG64(child_c)) where child_c is
the c-th child of numpy.random.SeedSequence(seed).spawn(n_chunks).  The
result therefore does not depend on how many threads generate it.  All
values are float32.

  uniform      Uniform[0,1) drawn directly in float32 (24-bit grid, so exact
               ties occur at large n)
  normal       standard normal drawn in float32
  pareto       Pareto(alpha=1.5, x_m=1): x = (1-U)^(-1/1.5) evaluated in
               float64 with a 53-bit U, then rounded to float32
  sae          BatchTopK-SAE-shaped pool, 4096 x 12288: bias b_j ~ N(-1, 0.5)
               (0.5 = standard deviation) from SeedSequence(seed) child 0,
               pre-activations N(0,1) float32, x = max(pre + b_j, 0); row r
               is chunk-generated like the others from children 1..
  adv_levels   radix-adversarial: 90% of positions 0x3F800000 | u8 noise
               (uniform u8), 10% (Bernoulli(0.1)) one of 1024 exact levels
               0x3F800000 + ((j+1) << 8), j uniform in 0..1023
  adv_noise    only the 8-bit noise: 0x3F800000 | u8 (256 distinct values)
  uniform12    Uniform[1,2)
  narrow       Uniform[128.6, 128.7]
  lognormal    exp(N(0,1))
  exponential  Exp(1)
  cauchy       standard Cauchy
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 24

SAE_ROWS = 4096
SAE_COLS = 12288


def _chunk(kind: str, rng: np.random.Generator, n: int) -> np.ndarray:
    if kind == "uniform":
        return rng.random(n, dtype=np.float32)
    if kind == "normal":
        return rng.standard_normal(n, dtype=np.float32)
    if kind == "pareto":
        u = rng.random(n)  # float64, 53-bit
        return ((1.0 - u) ** (-1.0 / 1.5)).astype(np.float32)
    if kind == "adv_levels":
        noise = rng.integers(0, 256, n, dtype=np.uint32)
        lvl = rng.integers(0, 1024, n, dtype=np.uint32)
        use_level = rng.random(n) < 0.1
        bits = np.where(use_level, np.uint32(0x3F800000) + ((lvl + np.uint32(1)) << np.uint32(8)),
                        np.uint32(0x3F800000) | noise)
        return bits.astype(np.uint32).view(np.float32)
    if kind == "adv_noise":
        noise = rng.integers(0, 256, n, dtype=np.uint32)
        return (np.uint32(0x3F800000) | noise).view(np.float32)
    if kind == "uniform12":
        return (1.0 + rng.random(n)).astype(np.float32)
    if kind == "narrow":
        return rng.uniform(128.6, 128.7, n).astype(np.float32)
    if kind == "lognormal":
        return np.exp(rng.standard_normal(n)).astype(np.float32)
    if kind == "exponential":
        return rng.standard_exponential(n).astype(np.float32)
    if kind == "cauchy":
        return rng.standard_cauchy(n).astype(np.float32)
    raise ValueError(f"unknown input kind {kind!r}")


KINDS = ("uniform", "normal", "pareto", "adv_levels", "adv_noise", "uniform12", "narrow",
         "lognormal", "exponential", "cauchy")


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(kind: str, n: int, seed: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """n float32 values of the named distribution (recipe in the module docstring)."""
    if kind == "sae":
        if n != SAE_ROWS * SAE_COLS:
            raise ValueError("the sae pool has a fixed size of 4096 x 12288")
        return sae_pool(seed).reshape(-1)
    if out is None:
        out = np.empty(n, dtype=np.float32)
    n_chunks = (n + CHUNK - 1) // CHUNK
    children = np.random.SeedSequence(seed).spawn(max(1, n_chunks))

    def work(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        rng = np.random.Generator(np.random.PCG64(children[c]))
        out[lo:hi] = _chunk(kind, rng, hi - lo)

    if n_chunks <= 1:
        if n:
            work(0)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def sae_pool(seed: int = 0) -> np.ndarray:
    """The 4096 x 12288 BatchTopK-SAE-shaped activation pool (float32)."""
    children = np.random.SeedSequence(seed).spawn(1 + SAE_ROWS // 256)
    b = np.random.Generator(np.random.PCG64(children[0])).normal(-1.0, 0.5, SAE_COLS)
    b = b.astype(np.float32)
    out = np.empty((SAE_ROWS, SAE_COLS), dtype=np.float32)

    def work(c: int) -> None:
        rng = np.random.Generator(np.random.PCG64(children[1 + c]))
        rows = slice(c * 256, (c + 1) * 256)
        pre = rng.standard_normal((256, SAE_COLS), dtype=np.float32)
        np.maximum(pre + b, np.float32(0.0), out=out[rows])

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(work, range(SAE_ROWS // 256)))
    return out


def edge_case(name: str, n: int, seed: int = 0) -> np.ndarray:
    """Small structured inputs for edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "all_equal":
        return np.full(n, 0.5, dtype=np.float32)
    if name == "signed_zeros":
        z = rng.integers(0, 2, n)
        return np.where(z == 1, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    if name == "few_levels":
        return rng.integers(0, 4, n).astype(np.float32)
    if name == "ascending":
        return np.arange(n, dtype=np.float32)
    if name == "descending":
        return np.arange(n, 0, -1, dtype=np.float32)
    if name == "with_inf":
        x = rng.standard_normal(n, dtype=np.float32)
        x[rng.integers(0, n, max(1, n // 100))] = np.inf
        x[rng.integers(0, n, max(1, n // 100))] = -np.inf
        return x
    if name == "with_nan":
        x = rng.standard_normal(n, dtype=np.float32)
        x[rng.integers(0, n, max(1, n // 1000))] = np.nan
        return x
    if name == "two_levels":  # 10% exactly 2.0, 90% exactly 1.0
        return np.where(rng.random(n) < 0.1, np.float32(2.0), np.float32(1.0)).astype(np.float32)
    if name == "negative":
        return -np.abs(rng.standard_normal(n, dtype=np.float32)) - 1.0
    raise ValueError(name)
