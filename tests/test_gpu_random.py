"""Seeded random parity sweep of the HIP path against the CPU oracle: flat calls over
many distributions, sizes, k and parameter options, and batched shapes.  Every case is
bit-exact (indices and value bits) or the test fails; each case prints its draw first.
"""
import numpy as np
import pytest

import oracle
import sampling_threshold_filtering_amd as stf
from workloads import edge_case, generate

pytestmark = pytest.mark.gpu

GEN = ("uniform", "normal", "pareto", "adv_levels", "adv_noise", "uniform12", "narrow", "lognormal",
       "exponential", "cauchy")
EDGE = ("all_equal", "signed_zeros", "few_levels", "ascending", "descending", "with_inf", "with_nan",
        "two_levels", "negative")


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def draw_case(seed: int, max_log2n: int):
    rng = np.random.default_rng(1000 + seed)
    kinds = GEN + EDGE
    kind = kinds[int(rng.integers(len(kinds)))]
    log2n = rng.uniform(10, max_log2n)
    n = int(2 ** log2n) + int(rng.integers(0, 17))
    log2k = rng.uniform(0, min(log2n, 17))
    k = max(1, min(n, int(2 ** log2k)))
    opts = {"s_rule": int(rng.choice([0, 2])), "param_mode": int(rng.integers(0, 2))}
    return kind, n, k, opts


def make_input(kind: str, n: int, seed: int) -> np.ndarray:
    return generate(kind, n, seed=seed) if kind in GEN else edge_case(kind, n, seed)


@pytest.mark.parametrize("seed", range(48))
def test_random_flat_cases(seed):
    kind, n, k, opts = draw_case(seed, 23)
    print("[case] flat", seed, kind, n, k, opts, flush=True)
    x = make_input(kind, n, seed)
    vals, idx, st = stf.topk(dev(x), k, eps=1e-3, seed=seed, options=opts, stats=True)
    ov, oi = oracle.topk(x, k, nthreads=8)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(vals.cpu().numpy().view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("seed", range(16))
def test_random_batched_cases(seed):
    rng = np.random.default_rng(5000 + seed)
    kinds = ("uniform", "normal", "pareto", "few_levels", "with_nan", "narrow")
    kind = kinds[int(rng.integers(len(kinds)))]
    B = int(rng.integers(1, 65))
    n = int(2 ** rng.uniform(9, 18)) + int(rng.integers(0, 9))
    k = max(1, min(n, int(2 ** rng.uniform(0, 10))))
    print("[case] batched", seed, kind, B, n, k, flush=True)
    x = make_input(kind, B * n, seed).reshape(B, n)
    vals, idx = stf.topk_batched(dev(x), k, eps=1e-3, seed=seed)
    ov, oi = oracle.topk_batched(x, k, nthreads=8)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(vals.cpu().numpy().view(np.uint32), ov.view(np.uint32))
