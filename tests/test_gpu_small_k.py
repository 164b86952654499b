"""The one-launch refinement for small k (k <= 64) on the GPU ("Prof-K: Probabilistic
One-Pass Filtering for Efficient Top-k Selection", §3 stage 4: the exact top k of the
candidates that passed the threshold).

Each workgroup keeps the k largest of its share of the candidates and the last one
selects the final k from the union of those lists.  Cases: every k up to the bound and
just past it (k = 65 takes the three-launch refinement), ties broken by index, shares
spanning one and many workgroups, a buffer M large enough that the union of the lists
sits at its bound of 8192 keys, and the approximate mode's partial outcomes (fewer than
k kept, padded with index -1; more hits than the buffer holds).

Bar: bit-exact indices and value bits against the CPU oracle; for partial outcomes the
sorted top of what the buffer kept, checked against the oracle's top-R set.
"""
import numpy as np
import pytest

import oracle
import sampling_threshold_filtering_amd as stf
from workloads import edge_case, generate

pytestmark = pytest.mark.gpu


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def say(*a):
    print("[case]", *a, flush=True)


def check_topk(x, vals, idx, k):
    ov, oi = oracle.topk(x, k, nthreads=8)
    np.testing.assert_array_equal(host(idx), oi)
    np.testing.assert_array_equal(host(vals).view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("k", [1, 2, 3, 17, 32, 33, 63, 64, 65])
@pytest.mark.parametrize("kind,N", [("uniform", (1 << 22) + 77), ("pareto", 1 << 23), ("normal", 1 << 20)])
def test_every_small_k(kind, N, k):
    say("small k", kind, N, k)
    x = generate(kind, N, seed=k)
    vals, idx, st = stf.topk(dev(x), k, seed=k, stats=True)
    check_topk(x, vals, idx, k)
    assert not st["fallback"]


@pytest.mark.parametrize("kind,N,k", [("adv_noise", 1 << 22, 40), ("adv_levels", 1 << 22, 64), ("two_levels", 1 << 21, 50)])
def test_small_k_ties_break_by_index(kind, N, k):
    say("small k ties", kind, N, k)
    x = generate(kind, N, seed=51) if kind != "two_levels" else edge_case(kind, N, 51)
    vals, idx, _ = stf.topk(dev(x), k, seed=2, stats=True)
    check_topk(x, vals, idx, k)


@pytest.mark.parametrize("k,M", [(32, 1 << 20), (33, 1000000), (64, 1 << 19), (64, 600000), (8, 5000), (64, 64)])
def test_small_k_list_union_bounds(k, M):
    """A forced buffer size sets the number of lists, ceil(M / 4096): 256 lists of 32,
    245 of 33 and 128 of 64 keys put the union at or just under 8192 keys; 147 lists of
    64 are past it and take the three-launch refinement.  M = k leaves one list."""
    say("small k union", k, M)
    N = 1 << 24
    x = generate("normal", N, seed=M % 1000)
    vals, idx, st = stf.topk(dev(x), k, seed=3, options={"force_M": M}, stats=True)
    if st["fallback"] or st["attempts"] > 1:
        print("[case] attempts", st["attempts"], "fallback", st["fallback"], flush=True)
    check_topk(x, vals, idx, k)


def assert_valid_partial(x, vals, idx, k, R, M):
    """The sorted top of min(R, M) buffered entries, all of which rank at or above R;
    index -1 and value -inf past them."""
    i = host(idx)
    v = host(vals).view(np.uint32)
    kept = min(R, M, k)
    assert np.all(i[kept:] == -1)
    assert np.all(v[kept:] == np.uint32(0xFF800000))
    got = i[:kept]
    assert len(set(got.tolist())) == kept and got.min() >= 0 and got.max() < x.size
    np.testing.assert_array_equal(v[:kept], x[got].view(np.uint32))
    assert set(got.tolist()) <= set(oracle.topk(x, R, nthreads=8)[1].tolist())
    xv = x[got].astype(np.float64)
    assert np.all((xv[:-1] > xv[1:]) | ((xv[:-1] == xv[1:]) & (got[:-1] < got[1:])))


def test_small_k_approx_recall_failure_pads():
    say("small k approx recall failure")
    N, k = 1 << 16, 60
    x = generate("uniform", N, seed=61)
    # t = 1 on a 4096-sample: R is about N/S = 16 < k
    vals, idx, info = stf.topk_approx(dev(x), k, options={"force_t": 1, "s_override": 4096}, seed=6)
    inf = stf.approx_info(info)
    assert inf["status"] == 1 and 0 < inf["R"] < k
    assert_valid_partial(x, vals, idx, k, inf["R"], inf["M"])
    ov, oi = oracle.topk(x, inf["R"], nthreads=8)
    np.testing.assert_array_equal(host(idx)[:inf["R"]], oi)


def test_small_k_approx_overflow_keeps_a_valid_subset():
    say("small k approx overflow")
    N, k = 1 << 22, 48
    x = generate("normal", N, seed=62)
    vals, idx, info = stf.topk_approx(dev(x), k, options={"force_M": k}, seed=5)
    inf = stf.approx_info(info)
    assert inf["status"] == 2 and inf["R"] > inf["M"] == k
    assert_valid_partial(x, vals, idx, k, inf["R"], inf["M"])


def test_small_k_repeated_calls_leave_state_clean():
    """Back-to-back calls with different k and N on one stream: the election counter
    and the sampler's hash set are left zero by each call."""
    xs = [generate("uniform", 1 << 21, seed=70), generate("pareto", 3 << 20, seed=71)]
    for rep in range(3):
        for j, x in enumerate(xs):
            k = [5, 64, 31][rep] + j
            say("small k repeat", rep, j, k)
            vals, idx, _ = stf.topk(dev(x), k, seed=rep, stats=True)
            check_topk(x, vals, idx, k)
