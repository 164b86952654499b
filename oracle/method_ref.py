"""Reference for the method-internal quantities of Prof-K: TEST INFRASTRUCTURE ONLY.

Pages: P1 = "Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
Selection" (arXiv HTML page); P2 = the earlier version of the same paper
(bittide mirror).  Plain Python/numpy, slow and direct.  Shares no code with
the GPU library.

* sample_indices: stage 1 of P1 §3 (uniform S-subset of [N] without
  replacement).  The pages do not fix the procedure.  Reading used by both
  sides: draw j = 0, 1, 2, ... maps Philox4x32-10(counter = (j, row,
  attempt, 0), key = (seed mod 2^32, seed div 2^32)) to the 64-bit value
  r = w0 + 2^32 w1 and then to the index floor(r N / 2^64); the sample is
  the set of the first S distinct indices in draw order.  Every S-subset is
  equally likely (the draws are i.i.d. and the rule is symmetric under
  relabelling of [N]); the per-index bias of the 64-bit map is below N/2^64.
* threshold: stage 2 of P1 §3: tau is the t-th largest sampled entry, with
  the total order (value descending, then lower index first) standing in for
  the distinct-entries assumption of P1 §4.
* count: R = number of entries at or before tau in that order (P1 §4
  "Notation and Conventions": R is the rank of tau in the full input).
* rank simulator: R is the t-th smallest rank of a uniform S-subset of
  {1..N} (P2 §4 Lemma 1); drawn here with numpy's own generator, independent
  of Philox.
"""
from __future__ import annotations

import math

import numpy as np

from .philox import philox4x32

_M32 = 0xFFFFFFFF


def draw_indices(N: int, seed: int, attempt: int, row: int, j0: int, count: int) -> np.ndarray:
    """Indices of draws j0 .. j0+count-1 (before removing repeats), as Python ints."""
    j = np.arange(j0, j0 + count, dtype=np.uint64)
    w0, w1, _, _ = philox4x32(j & np.uint64(_M32), np.uint64(row & _M32),
                              np.uint64(attempt & _M32), np.uint64(0),
                              seed & _M32, (seed >> 32) & _M32)
    out = np.empty(count, dtype=np.int64)
    for n in range(count):
        r = int(w0[n]) | (int(w1[n]) << 32)
        out[n] = (r * N) >> 64  # exact integer arithmetic
    return out


def sample_indices(N: int, S: int, seed: int, attempt: int = 0, row: int = 0) -> np.ndarray:
    """The first S distinct draw indices in draw order, returned sorted ascending."""
    if not (1 <= S <= N):
        raise ValueError("need 1 <= S <= N")
    seen: set[int] = set()
    j = 0
    chunk = max(1024, S)
    while len(seen) < S:
        for i in draw_indices(N, seed, attempt, row, j, chunk):
            i = int(i)
            if i not in seen:
                seen.add(i)
                if len(seen) == S:
                    break
        j += chunk
        chunk = 1024
    return np.array(sorted(seen), dtype=np.int64)


def order_key(v: float, i: int):
    """Sort key for the total order: NaN first, then larger value, then lower index."""
    if math.isnan(v):
        return (0, 0.0, i)
    return (1, -v, i)


def threshold(x: np.ndarray, sample: np.ndarray, t: int):
    """tau = the t-th entry (1-based) of the sampled entries in the total order.
    Returns (value as np.float32, index)."""
    if not (1 <= t <= len(sample)):
        raise ValueError("need 1 <= t <= S")
    vals = x[sample]
    entries = sorted(((float(vals[n]), int(sample[n])) for n in range(len(sample))),
                     key=lambda e: order_key(*e))
    v, i = entries[t - 1]
    return np.float32(v), i


def count_at_or_before(x: np.ndarray, tau_val, tau_idx: int) -> int:
    """R(tau) = #{i : (x_i, i) at or before (tau_val, tau_idx) in the total order}."""
    x = np.asarray(x)
    idx = np.arange(x.size, dtype=np.int64)
    tv = float(tau_val)
    if math.isnan(tv):
        m = np.isnan(x) & (idx <= tau_idx)
    else:
        m = np.isnan(x) | (x > tv) | ((x == tv) & (idx <= tau_idx))
    return int(np.count_nonzero(m))


def candidate_set(x: np.ndarray, tau_val, tau_idx: int) -> np.ndarray:
    """Sorted indices of every entry at or before tau (the set the filter keeps)."""
    x = np.asarray(x)
    idx = np.arange(x.size, dtype=np.int64)
    tv = float(tau_val)
    if math.isnan(tv):
        m = np.isnan(x) & (idx <= tau_idx)
    else:
        m = np.isnan(x) | (x > tv) | ((x == tv) & (idx <= tau_idx))
    return idx[m]


def simulate_rank(N: int, S: int, t: int, trials: int, rng: np.random.Generator) -> np.ndarray:
    """R over `trials` independent uniform S-subsets of ranks {1..N}: the t-th smallest
    sampled rank (rank 1 = largest entry).  Uses numpy's generator, not Philox."""
    out = np.empty(trials, dtype=np.int64)
    for n in range(trials):
        ranks = rng.choice(N, size=S, replace=False)
        out[n] = int(np.partition(ranks, t - 1)[t - 1]) + 1
    return out
