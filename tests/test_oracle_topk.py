"""Pins of the C top-k oracle against definitions that do not reuse its code.

The oracle's result is the plain definition of exact top-k under the total
order (value descending, ties to the lower index, NaN above everything);
see "Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
Selection", §3 (problem statement: the k largest entries with their
indices) and §4 "Notation and Conventions" (rank 1 = largest).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import method_ref
from workloads import edge_case, generate


def brute_force_topk(x, k):
    """O(N^2) rank definition: rank(i) = number of j that come before i."""
    n = len(x)

    def before(j, i):
        a, b = float(x[j]), float(x[i])
        if math.isnan(a) or math.isnan(b):
            if math.isnan(a) and math.isnan(b):
                return j < i
            return math.isnan(a)
        return a > b or (a == b and j < i)

    rank = [sum(1 for j in range(n) if j != i and before(j, i)) for i in range(n)]
    order = sorted(range(n), key=lambda i: rank[i])
    assert sorted(rank) == list(range(n)), "the order must be total"
    return np.array(order[:k], dtype=np.int64)


def tiny_inputs():
    rng = np.random.default_rng(123)
    cases = []
    for n in (1, 2, 3, 7, 16, 33, 64):
        cases.append(rng.standard_normal(n).astype(np.float32))
        cases.append(rng.integers(0, 3, n).astype(np.float32))  # heavy ties
    cases.append(edge_case("signed_zeros", 40, 1))
    cases.append(edge_case("all_equal", 20))
    cases.append(edge_case("with_inf", 50, 2))
    x = rng.standard_normal(30).astype(np.float32)
    x[[3, 7, 20]] = np.nan
    cases.append(x)
    cases.append(edge_case("ascending", 25))
    cases.append(edge_case("descending", 25))
    return cases


@pytest.mark.parametrize("case", range(len(tiny_inputs())))
def test_oracle_matches_brute_force_for_every_k(case):
    x = tiny_inputs()[case]
    n = len(x)
    full = brute_force_topk(x, n)
    for k in range(1, n + 1):
        vals, idx = oracle.topk(x, k)
        np.testing.assert_array_equal(idx, full[:k])
        # values are bit copies of x at those indices
        np.testing.assert_array_equal(vals.view(np.uint32), x[idx].view(np.uint32))


def test_oracle_matches_python_sort_with_order_key():
    rng = np.random.default_rng(7)
    x = rng.integers(-50, 50, 5000).astype(np.float32) / 4
    ref = sorted(range(len(x)), key=lambda i: method_ref.order_key(float(x[i]), i))
    for k in (1, 17, 999, 5000):
        _, idx = oracle.topk(x, k)
        np.testing.assert_array_equal(idx, np.array(ref[:k]))


def test_special_cases():
    x = edge_case("all_equal", 100)
    _, idx = oracle.topk(x, 10)
    np.testing.assert_array_equal(idx, np.arange(10))  # all tie -> lowest indices
    x = np.array([1.0, 5.0, 5.0, 2.0, 5.0], dtype=np.float32)
    _, idx = oracle.topk(x, 1)
    assert idx[0] == 1  # argmax, lowest index among the maxima
    x = np.random.default_rng(1).standard_normal(300).astype(np.float32)
    vals, idx = oracle.topk(x, 300)  # k = N is the full descending sort
    np.testing.assert_array_equal(idx, np.argsort(-x.astype(np.float64), kind="stable"))


def test_adversarial_noise_closed_form():
    # 0x3F800000 | u8: the top-k is the k lowest indices holding the max value
    x = generate("adv_noise", 1 << 20, seed=3)
    k = 1 << 10
    _, idx = oracle.topk(x, k)
    mx = x.max()
    expect = np.flatnonzero(x == mx)[:k]
    assert len(expect) == k
    np.testing.assert_array_equal(idx, expect)


def test_multithreaded_and_batched_agree_with_single_thread():
    x = generate("normal", 1 << 20, seed=5)
    for k in (1, 64, 4096):
        v1, i1 = oracle.topk(x, k, nthreads=1)
        v4, i4 = oracle.topk(x, k, nthreads=4)
        np.testing.assert_array_equal(i1, i4)
        np.testing.assert_array_equal(v1.view(np.uint32), v4.view(np.uint32))
    xb = generate("uniform", 8 * 5000, seed=9).reshape(8, 5000)
    vb, ib = oracle.topk_batched(xb, 33)
    for r in range(8):
        v, i = oracle.topk(xb[r], 33)
        np.testing.assert_array_equal(ib[r], i)
        np.testing.assert_array_equal(vb[r], v)


def test_count_at_or_before_matches_rank_definition():
    rng = np.random.default_rng(11)
    for x in (rng.integers(0, 5, 200).astype(np.float32), edge_case("signed_zeros", 64, 4),
              edge_case("with_nan", 3000, 5)):
        order = brute_force_topk(x, len(x)) if len(x) <= 200 else None
        if order is None:
            order = np.array(sorted(range(len(x)), key=lambda i: method_ref.order_key(float(x[i]), i)))
        for r in (0, 1, len(x) // 3, len(x) - 1):
            tau_i = int(order[r])
            expect = r + 1  # tau is the (r+1)-th entry of the order
            assert oracle.count_at_or_before(x, x[tau_i], tau_i) == expect
            assert method_ref.count_at_or_before(x, x[tau_i], tau_i) == expect
            cand = method_ref.candidate_set(x, x[tau_i], tau_i)
            np.testing.assert_array_equal(cand, np.sort(order[: r + 1]))


def test_bad_arguments_rejected():
    x = np.zeros(4, dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.topk(x, 5)
    with pytest.raises(ValueError):
        oracle.topk(x, 0)


def test_indices_beyond_2p32():
    """64-bit indices: planted values past 2^32 in an otherwise zero input (the
    zero pages are shared, so the 17 GB array costs little memory); the expected
    order is written out from the definition."""
    N = (1 << 32) + 1000
    x = np.zeros(N, dtype=np.float32)
    x[(1 << 32) + 999] = 5.0
    x[1 << 32] = 4.0
    x[3] = 4.0
    x[1 << 31] = -1.0
    v, i = oracle.topk(x, 5, nthreads=8)
    np.testing.assert_array_equal(i, np.array([(1 << 32) + 999, 3, 1 << 32, 0, 1], dtype=np.int64))
    np.testing.assert_array_equal(v, np.array([5.0, 4.0, 4.0, 0.0, 0.0], dtype=np.float32))
