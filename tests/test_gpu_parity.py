"""GPU parity of every stage of the HIP path against the CPU oracle.

Bar: bit-exact (indices, value bits, counts, sample sets).  Each test prints
its case before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import sampling_threshold_filtering_amd as stf
from oracle import method_ref
from workloads import edge_case, generate

pytestmark = pytest.mark.gpu


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def say(*a):
    print("[case]", *a, flush=True)


def check_topk(x_np, vals, idx, k):
    ov, oi = oracle.topk(x_np, k, nthreads=8)
    np.testing.assert_array_equal(host(idx), oi)
    np.testing.assert_array_equal(host(vals).view(np.uint32), ov.view(np.uint32))


# ----------------------------------------------------------------------------- stage 1
@pytest.mark.parametrize("N,S,seed,attempt", [(1 << 20, 32768, 0, 0), (1 << 20, 32768, 7, 3), (5000, 2500, 1, 0),
                                              (4096, 2048, 2, 1), (123457, 1000, 99, 0), (1 << 22, 131072, 5, 0)])
def test_sample_matches_oracle(N, S, seed, attempt):
    say("sample", N, S, seed, attempt)
    x = generate("uniform", N, seed=1)
    got = np.sort(host(stf.stage_sample(dev(x), S, seed=seed, attempt=attempt)))
    ref = method_ref.sample_indices(N, S, seed=seed, attempt=attempt)
    np.testing.assert_array_equal(got, ref)


# ----------------------------------------------------------------------------- stage 2
@pytest.mark.parametrize("kind,N,S,t,seed", [("uniform", 1 << 20, 32768, 4, 0), ("normal", 1 << 20, 32768, 118, 3),
                                             ("few_levels", 100000, 20000, 500, 1),
                                             ("adv_noise", 1 << 20, 32768, 7, 2),
                                             ("signed_zeros", 50000, 10000, 3000, 4),
                                             ("uniform", 1 << 22, 131072, 1, 9),
                                             # sorted per-block lists (t <= 64): boundary t, ragged last
                                             # block, heavy top-up (S = N/2), special values, ties
                                             ("normal", 100003, 3001, 50, 12),
                                             ("uniform", 5000, 2500, 10, 13),
                                             ("with_inf", 1 << 20, 32768, 20, 14),
                                             ("with_nan", 1 << 20, 32768, 2, 15),
                                             ("all_equal", 100000, 20000, 64, 16),
                                             ("negative", 1 << 20, 32768, 33, 17),
                                             ("ascending", 1 << 20, 8192, 64, 18),
                                             # 256-thread sampling workgroups up to S = 32768, then 1024
                                             ("pareto", 1 << 24, 16357, 1, 21), ("pareto", 1 << 24, 16357, 20, 22),
                                             ("normal", 1 << 20, 32769, 40, 23),
                                             # unordered per-block top-t lists (t <= 1024) in workgroups of
                                             # 256 / 512 / 1024: t just above the sorted lists, the SAE
                                             # pool's and the adversarial workload's (S, t) under the
                                             # default rule, t = 1024, a last block with fewer than t
                                             # draws, large top-ups
                                             ("normal", 1 << 20, 32768, 65, 20), ("normal", 1 << 20, 8192, 100, 24),
                                             ("normal", 1 << 20, 16384, 65, 35), ("normal", 1 << 26, 32768, 118, 34),
                                             ("adv_levels", 1 << 24, 82557, 68, 28), ("normal", 1 << 20, 7000, 1024, 29),
                                             ("uniform", 1 << 20, 9221, 200, 30), ("uniform", 12000, 6000, 300, 25),
                                             ("uniform", 20000, 8000, 200, 26),
                                             # every key slot in LDS (t > 1024, S + top-up <= 8192)
                                             ("uniform", 12000, 5000, 2000, 27),
                                             # multi-block select passes over the key slots: lists beyond
                                             # the LDS (128 x 64 + top-up), t > 1024, ties, top-up ~ S / 4
                                             ("pareto", 1 << 24, 131072, 64, 11), ("uniform", 1 << 22, 131072, 64, 19),
                                             ("normal", 1 << 22, 131072, 5000, 31), ("all_equal", 1 << 20, 65536, 3000, 32),
                                             ("uniform", 40000, 20000, 2000, 33)])
def test_threshold_matches_oracle(kind, N, S, t, seed):
    say("threshold", kind, N, S, t, seed)
    edge = ("few_levels", "signed_zeros", "with_inf", "with_nan", "all_equal", "negative", "ascending")
    x = edge_case(kind, N, 5) if kind in edge else generate(kind, N, seed=5)
    v, i = stf.stage_threshold(dev(x), S, t, seed=seed)
    sample = method_ref.sample_indices(N, S, seed=seed)
    rv, ri = method_ref.threshold(x, sample, t)
    assert int(host(i)[0]) == ri
    assert host(v).view(np.uint32)[0] == np.float32(rv).view(np.uint32)


# ----------------------------------------------------------------------------- stage 3
@pytest.mark.parametrize("kind,N,offset,M,rank", [("normal", 1 << 20, 0, 5000, 3000), ("normal", 1000003, 1, 5000, 3000),
                                                  ("uniform", 1 << 22, 3, 100000, 70000),
                                                  ("few_levels", 65537, 2, 70000, 40000),
                                                  ("normal", 300001, 0, 100, 2000),  # overflow: R > M
                                                  ("normal", 7, 1, 8, 5), ("normal", 3, 0, 4, 2),
                                                  ("with_nan", 100000, 0, 1000, 500)])
def test_filter_matches_oracle(kind, N, offset, M, rank):
    say("filter", kind, N, offset, M, rank)
    x = generate(kind, N + offset, seed=11) if kind in ("normal", "uniform") else edge_case(kind, N + offset, 11)
    xs = x[offset:]
    order = np.array(sorted(range(N), key=lambda i: method_ref.order_key(float(xs[i]), i))) if N < 2000 else None
    if order is not None:
        tau_i = int(order[rank - 1])
    else:
        # tau = the rank-th entry in the total order, from the oracle top-k
        _, oi = oracle.topk(xs, rank, nthreads=8)
        tau_i = int(oi[-1])
    tau_v = xs[tau_i]
    xd = dev(x)[offset:]  # misaligned views exercise the scalar head
    R, cand = stf.stage_filter(xd, float(tau_v), tau_i, M)
    assert R == oracle.count_at_or_before(xs, tau_v, tau_i) == rank
    got = np.sort(host(cand))
    ref = method_ref.candidate_set(xs, tau_v, tau_i)
    if R <= M:
        np.testing.assert_array_equal(got, ref)
    else:
        assert len(got) == M and len(np.unique(got)) == M and np.isin(got, ref).all()


# ----------------------------------------------------------------------------- end to end
SMALL = [
    ("uniform", 1 << 22, 32, {}),                       # first workload, default parameters
    ("normal", 1 << 20, 1, {"s_override": 8192}),
    ("normal", 1 << 20, 1000, {"s_override": 8192}),
    ("normal", 1 << 20, 9000, {"s_override": 16384}),   # multi-block sort path (k > 8192)
    ("few_levels", 300007, 777, {"s_override": 4096}),  # heavy ties
    ("adv_noise", 1 << 20, 5000, {"s_override": 8192}),  # all values share the top 24 bits
    ("adv_levels", 1 << 21, 2048, {"s_override": 8192}),
    ("signed_zeros", 200000, 100, {"s_override": 4096}),
    ("with_inf", 500000, 300, {"s_override": 8192}),
    ("with_nan", 500000, 300, {"s_override": 8192}),
    ("negative", 400000, 64, {"s_override": 8192}),
    ("ascending", 1 << 20, 100, {"s_override": 8192}),
    ("descending", 1 << 20, 100, {"s_override": 8192}),
    # rare hits: the filter's one-block, 8-float4 launch shape (E[R] + 3 sd(R) <= N / 8192)
    ("normal", 1 << 26, 8, {"s_override": 131072}),
    ("normal", (1 << 24) + 13, 5, {"s_override": 65536}),
]


@pytest.mark.parametrize("kind,N,k,opts", SMALL)
def test_topk_matches_oracle(kind, N, k, opts):
    say("topk", kind, N, k, opts)
    x = generate(kind, N, seed=21) if kind in ("uniform", "normal", "adv_noise", "adv_levels") else edge_case(kind, N, 21)
    vals, idx, st = stf.topk(dev(x), k, eps=1e-3, seed=3, options=opts or None, stats=True)
    check_topk(x, vals, idx, k)
    assert not st["fallback"] and st["attempts"] >= 1
    print("[case] refine_multipass", st["refine_multipass"], flush=True)


@pytest.mark.parametrize("kind,N,k,mode,rule", [
    ("normal", 1 << 22, 32, 1, 0), ("uniform", 1 << 22, 2048, 1, 1), ("pareto", 1 << 24, 16384, 1, 1),
    ("normal", 1 << 24, 131072, 0, 1), ("normal", 1 << 23, 300, 1, 0),
])
def test_fast_parameters_and_cost_model_rule_stay_exact(kind, N, k, mode, rule):
    """The closed-form surrogates and the cost-model S rule (P1 Algorithm 1) only change
    (S, t, M); the output is still the exact top-k."""
    say("topk fast params", kind, N, k, mode, rule)
    x = generate(kind, N, seed=23)
    o = stf.make_options(param_mode=mode, s_rule=rule)
    p = stf.solve(N, k, 1e-3, options=o)
    vals, idx, st = stf.topk(dev(x), k, eps=1e-3, seed=4, options=o, stats=True)
    check_topk(x, vals, idx, k)
    assert (st["S"], st["t"], st["M"]) == (p["S"], p["t"], p["M"])


@pytest.mark.parametrize("N,k,offset", [(1, 1, 0), (5, 3, 1), (1000, 1000, 2), (4096, 17, 3), (100003, 5000, 1)])
def test_exact_path_small_and_misaligned(N, k, offset):
    say("exact path", N, k, offset)
    x = generate("normal", N + offset, seed=N)
    vals, idx, st = stf.topk(dev(x)[offset:], k, stats=True)
    check_topk(x[offset:], vals, idx, k)
    # where the sample would not pay off the solver routes the call to the exact selection
    assert st["fallback"] == bool(stf.solve(N, k, 1e-3)["direct_exact"])


def test_binned_and_multipass_refinement_both_run():
    say("refinement paths")
    # continuous values: every needed value bin fits one LDS sort
    x = generate("normal", 1 << 22, seed=40)
    vals, idx, st = stf.topk(dev(x), 3000, stats=True)
    check_topk(x, vals, idx, 3000)
    assert st["refine_multipass"] == 0
    # one tie group: the index part of the keys spreads it over the bins
    x = generate("adv_noise", 1 << 22, seed=41)
    vals, idx, st = stf.topk(dev(x), 3000, stats=True)
    check_topk(x, vals, idx, 3000)
    assert st["refine_multipass"] == 0
    # two values, ~210K copies of the larger within a value range that puts each tie
    # group in one bin: bins beyond one workgroup's LDS sort go to the multi-block radix
    # select (the in-kernel partition of such bins runs in approximate mode,
    # test_gpu_approx.py)
    x = edge_case("two_levels", 1 << 21, 43)
    vals, idx, st = stf.topk(dev(x), 250000, stats=True)
    check_topk(x, vals, idx, 250000)
    assert st["refine_multipass"] >= 1
    # 419K copies of the larger: beyond what one workgroup partitions, so the host hands
    # the bin to the multi-block radix select
    x = edge_case("two_levels", 1 << 22, 42)
    vals, idx, st = stf.topk(dev(x), 500000, stats=True)
    check_topk(x, vals, idx, 500000)
    assert st["refine_multipass"] >= 1


@pytest.mark.parametrize("kind,log2n,k", [("normal", 22, 3000), ("pareto", 24, 1 << 15)])
def test_refinement_wait_that_runs_out_takes_the_multipass_refinement(kind, log2n, k):
    """The fused histogram-and-scatter launch waits once for all of its workgroups; a wait
    that runs out (forced here from the host) must leave no key placed and send the attempt
    to the multi-pass refinement, and the next call must find the launch-wide counter clear."""
    say("refinement wait runs out", kind, log2n, k)
    x = generate(kind, 1 << log2n, seed=44)
    xd = dev(x)
    vals, idx, st = stf.topk(xd, k, seed=5, options={"refine_wait_ticks": -1}, stats=True)
    check_topk(x, vals, idx, k)
    assert st["refine_multipass"] == st["attempts"] >= 1
    for _ in range(2):
        vals, idx, st = stf.topk(xd, k, seed=5, stats=True)
        check_topk(x, vals, idx, k)
        assert st["refine_multipass"] == 0


@pytest.mark.parametrize("kind,log2n,k", [("adv_levels", 26, 1 << 15), ("adv_levels", 24, 5000),
                                         ("adv_levels", 26, 64)])
def test_tie_groups_in_single_bins_take_the_multipass_select(kind, log2n, k):
    """Radix-adversarial levels: ~6500 (2^26) or ~1600 (2^24) copies of each of 1024
    values.  A whole level falls in one value bin of the binned refinement: bins beyond
    one workgroup's LDS sort (4096 keys) go to the multi-block radix select, smaller
    ones stay in the bin sort; k <= 64 takes the one-launch refinement (no bins)."""
    N = 1 << log2n
    say("tie groups", kind, N, k)
    x = generate(kind, N, seed=45)
    vals, idx, st = stf.topk(dev(x), k, stats=True)
    check_topk(x, vals, idx, k)
    print("[case] multipass", st["refine_multipass"], "R", st["R"], flush=True)
    assert st["refine_multipass"] == (1 if (log2n == 26 and k > 64) else 0)


def heavy_bins_input(n: int, seed: int) -> np.ndarray:
    """Background noise below 1.5, plus clusters that each fill one value bin of the
    refinement with more keys than one wavefront sorts: 2000 keys within 512 ulps
    (counting pass, ranks by scan and small sub-bucket sorts), 300 copies of one value
    among 200 neighbours (a sub-bucket sorted by one wavefront), 1000 copies (a
    sub-bucket too large for that: the bin goes to the LDS bitonic sort), 5000 copies
    (a bin beyond one workgroup's LDS: the multi-block radix select in exact mode, the
    in-kernel digit partition in approximate mode), and light bins."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 0.25).astype(np.float32)
    def ulps(base, off):
        return (np.uint32(np.float32(base).view(np.uint32)) + off.astype(np.uint32)).view(np.float32)
    parts = [
        rng.uniform(1.5, 8.0, 50).astype(np.float32),
        ulps(4.0, rng.integers(0, 512, 2000)),
        np.full(300, 5.0, np.float32), ulps(5.0, rng.integers(1, 600, 200)),
        np.full(1000, 6.0, np.float32),
        np.full(5000, 7.0, np.float32),
        rng.uniform(2.0, 3.0, 3000).astype(np.float32),
    ]
    planted = np.concatenate(parts)
    x[rng.choice(n, planted.size, replace=False)] = planted
    return x


@pytest.mark.parametrize("k", [12000, 9000, 2100])
def test_heavy_bins_take_every_sort_path(k):
    say("heavy bins", k)
    x = heavy_bins_input(1 << 21, 44)
    vals, idx, st = stf.topk(dev(x), k, stats=True)
    check_topk(x, vals, idx, k)
    # the 5000-copy bin of 7.0 is needed at every k here; the candidates hold all of it
    # when tau lies below 7.0, else the copies up to tau's index (R minus the values above
    # 7.0): beyond one workgroup's LDS sort (4096 keys) the multi-block radix select takes it
    in_bin = min(5000, st["R"][-1] - int(np.count_nonzero(x > np.float32(7.0))))
    assert st["refine_multipass"] == (1 if in_bin > 4096 else 0) and not st["fallback"]
    # approximate mode has no host to hand it to: the bin sort's digit partition runs
    vals, idx, info = stf.topk_approx(dev(x), k)
    assert stf.approx_info(info)["status"] == 0
    check_topk(x, vals, idx, k)


@pytest.mark.parametrize("kind,log2n,k,rule", [("uniform", 22, 1 << 18, 0), ("normal", 24, 1 << 20, 2)])
def test_large_k_share_thresholds_stay_exact(kind, log2n, k, rule):
    # k a large share of N: under the default rule t = 2194 (S = 32768), so tau comes from
    # the multi-block select passes over the key slots; under the MI355X rule t = 338 from
    # the unordered per-block top-t lists.  Exact and approximate mode.
    N = 1 << log2n
    p = stf.solve(N, k, 1e-3, options={"s_rule": rule})
    say("large k share", kind, N, k, "rule", rule, "S", p["S"], "t", p["t"])
    assert not p["direct_exact"] and p["t"] > 64
    x = generate(kind, N, seed=21)
    xd = dev(x)
    vals, idx, st = stf.topk(xd, k, seed=3, options={"s_rule": rule}, stats=True)
    check_topk(x, vals, idx, k)
    assert not st["fallback"]
    av, ai, info = stf.topk_approx(xd, k, seed=3, options={"s_rule": rule})
    rec = stf.approx_info(info)
    assert rec["status"] in (0, 1, 2)
    if rec["status"] == 0:  # the check held (probability >= 1 - eps): the exact top-k
        check_topk(x, av, ai, k)


def test_forced_overflow_goes_to_fallback_and_stays_exact():
    say("forced overflow M = k")
    N, k = 1 << 22, 4096
    x = generate("adv_levels", N, seed=8)
    vals, idx, st = stf.topk(dev(x), k, options={"force_M": k}, stats=True)
    check_topk(x, vals, idx, k)
    assert st["attempts"] == 6 and st["fallback"]
    assert all(m == 2 for m in st["fail_mode"])  # every attempt overflowed (R > M)


def test_forced_recall_failure_retries():
    say("forced recall failure t = 1")
    N, k = 1 << 22, 1 << 14
    x = generate("normal", N, seed=9)
    vals, idx, st = stf.topk(dev(x), k, options={"force_t": 1}, stats=True)
    check_topk(x, vals, idx, k)
    assert st["fail_mode"][0] == 1  # R < k with t = 1 at this k


def test_forced_fallback_and_max_attempts_zero():
    say("force_fallback")
    x = generate("pareto", 1 << 21, seed=4)
    for opts in ({"force_fallback": 1}, {"use_max_attempts": 1, "max_attempts": 0}):
        vals, idx, st = stf.topk(dev(x), 3000, options=opts, stats=True)
        check_topk(x, vals, idx, 3000)
        assert st["fallback"] and st["attempts"] == 0


def test_fallback_with_huge_tie_group():
    say("fallback, 256-value input")
    x = generate("adv_noise", 1 << 22, seed=6)
    vals, idx = stf.topk(dev(x), 20000, options={"force_fallback": 1})
    check_topk(x, vals, idx, 20000)


@pytest.mark.parametrize("kind,N,k,offset", [("normal", 1000003, 1, 1), ("adv_levels", (1 << 22) + 5, 70000, 2),
                                             ("with_nan", 300001, 1000, 3), ("signed_zeros", 200000, 150000, 0),
                                             ("uniform", 7, 7, 1), ("normal", 5, 1, 3), ("pareto", 1 << 24, 1 << 17, 0),
                                             ("adv_noise", 1 << 20, 5000, 1)])
def test_exact_full_selection_on_ragged_views(kind, N, k, offset):
    """The exact full selection (radix-select passes over x with dwordx4 loads, then the
    filter as the compaction at tau = the k-th key) on misaligned views with scalar
    heads and tails, ties, NaN and signed zeros."""
    say("exact full selection", kind, N, k, offset)
    edge = ("with_nan", "signed_zeros")
    x = edge_case(kind, N + offset, 7) if kind in edge else generate(kind, N + offset, seed=7)
    vals, idx, st = stf.topk(dev(x)[offset:], k, options={"force_fallback": 1}, stats=True)
    check_topk(x[offset:], vals, idx, k)
    assert st["fallback"]


def test_interleaved_calls_leave_the_workspace_clean():
    # Every call must leave the hash set, tickets and histograms zero for the next
    # one, whatever its sizes: alternate shapes, stage calls and batched calls on one
    # stream and check each result.
    xs = {N: generate("normal", N, seed=N % 97) for N in (1 << 22, 1 << 20, 300001)}
    d = {N: dev(x) for N, x in xs.items()}
    for rep in range(2):
        for N, k in ((1 << 22, 32), (1 << 20, 1000), (300001, 64), (1 << 22, 5000)):
            say("interleaved topk", rep, N, k)
            v, i = stf.topk(d[N], k, seed=rep)
            check_topk(xs[N], v, i, k)
        say("interleaved stage_sample", rep)
        got = np.sort(host(stf.stage_sample(d[1 << 20], 60000, seed=rep)))
        np.testing.assert_array_equal(got, method_ref.sample_indices(1 << 20, 60000, seed=rep))
        say("interleaved batched", rep)
        xb = generate("uniform", 64 * 65536, seed=rep).reshape(64, 65536)
        vb, ib = stf.topk_batched(dev(xb), 16, seed=rep)
        ov, oi = oracle.topk_batched(xb, 16, nthreads=8)
        np.testing.assert_array_equal(host(ib), oi)


def test_out_buffers_and_side_stream():
    # The call returns once its run-time check is known; the outputs are complete in
    # stream order.  Reuse caller buffers and run on a non-default stream.
    import torch
    x = generate("normal", 1 << 22, seed=31)
    xd = dev(x)
    s2 = torch.cuda.Stream()
    for k in (7, 2000, 70000):
        say("out= on a side stream", k)
        out = (torch.empty(k, dtype=torch.float32, device="cuda"), torch.empty(k, dtype=torch.int64, device="cuda"))
        torch.cuda.current_stream().synchronize()
        with torch.cuda.stream(s2):
            for rep in range(3):
                v, i = stf.topk(xd, k, seed=rep, out=out)
                assert v.data_ptr() == out[0].data_ptr() and i.data_ptr() == out[1].data_ptr()
            hv, hi = v.cpu(), i.cpu()  # ordered on s2
        ov, oi = oracle.topk(x, k, nthreads=8)
        np.testing.assert_array_equal(hi.numpy(), oi)
        np.testing.assert_array_equal(hv.numpy().view(np.uint32), ov.view(np.uint32))
    with pytest.raises(ValueError):
        stf.topk(xd, 5, out=(torch.empty(4, device="cuda"), torch.empty(5, dtype=torch.int64, device="cuda")))


def test_seed_does_not_change_result_and_repeats_are_identical():
    say("determinism")
    x = generate("normal", 1 << 22, seed=12)
    xd = dev(x)
    v0, i0 = stf.topk(xd, 1000, seed=0)
    for seed in (1, 2, 12345678901234):
        v, i = stf.topk(xd, 1000, seed=seed)
        assert (host(i) == host(i0)).all() and (host(v) == host(v0)).all()
    check_topk(x, v0, i0, 1000)


def test_batched_matches_oracle():
    say("batched 16 x 2^18, k = 64")
    B, N, k = 16, 1 << 18, 64
    x = generate("normal", B * N, seed=13).reshape(B, N)
    vals, idx = stf.topk_batched(dev(x), k, options={"s_override": 4096})
    ov, oi = oracle.topk_batched(x, k)
    np.testing.assert_array_equal(host(idx), oi)
    np.testing.assert_array_equal(host(vals).view(np.uint32), ov.view(np.uint32))


def check_batched(x2d, vals, idx, k):
    ov, oi = oracle.topk_batched(np.ascontiguousarray(x2d), k, nthreads=8)
    np.testing.assert_array_equal(host(idx), oi)
    np.testing.assert_array_equal(host(vals).view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("kind,B,N,k,opts", [
    ("normal", 64, 1 << 20, 64, {}),                   # per-row kernels, default S
    ("few_levels", 40, 200003, 100, {"s_override": 8192}),  # ties inside rows, odd row length
    ("uniform", 300, 5000, 17, {}),                    # short rows: per-row LDS sort
    ("normal", 5, 8192, 8192, {}),                     # k = N at the short-row limit
    ("normal", 7, 1, 1, {}),
    ("normal", 2, 1 << 21, 300, {}),                   # rows longer than the per-row kernels take
    ("normal", 16, 1 << 20, 3000, {"s_override": 32768}),  # radix-select sampler (t > 64), LDS row sorts
    ("with_nan", 24, 100000, 40, {"s_override": 8000}),    # many repeats and a long top-up; NaN at the top
    ("uniform", 4, 1 << 17, 1024, {}),                 # k at the refinement's select-and-sort limit
    ("pareto", 8, 1 << 16, 65, {}),                    # k just above one wavefront's sort
])
def test_batched_shapes(kind, B, N, k, opts):
    say("batched", kind, B, N, k, opts)
    x = (generate(kind, B * N, seed=31) if kind in ("normal", "uniform", "pareto") else edge_case(kind, B * N, 31)).reshape(B, N)
    vals, idx, st = stf.topk_batched(dev(x), k, options=opts or None, stats=True)
    check_batched(x, vals, idx, k)


@pytest.mark.parametrize("B,k", [(128, 512), (64, 1024), (64, 2048), (64, 4096), (16, 8192)])
def test_batched_buffers_past_8192_keys_stay_on_the_batched_kernels(B, k):
    """Rows of 2^20 under the MI355X S rule with k = 512 / 1024 / 2048 need per-row
    buffers of 8710 / 10054 / 13069 keys, which the batched refinement holds in LDS
    (select then sort for k <= 1024, a full LDS sort above); k = 4096 / 8192 need 17667 /
    23840, past LDS, so the refinement selects over the buffer in global memory and sorts
    the k in LDS.  All run on the batched kernels, within twice what the row-by-row loop
    of flat calls would take (B times one row's flat call)."""
    import torch
    say("batched large buffers", B, k)
    N = 1 << 20
    o = stf.make_options(s_rule=2)
    assert stf.solve(N, k, 1e-3 / B, options=o)["M"] > 8192
    x = generate("pareto", B * N, seed=k).reshape(B, N)
    xd = dev(x)

    def timed(kk):
        stf.topk_batched(xd, kk, options=o)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        out = stf.topk_batched(xd, kk, seed=1, options=o)
        e1.record()
        e1.synchronize()
        return out, e0.elapsed_time(e1)

    (vals, idx), tk = timed(k)
    row0 = xd[0].contiguous()
    stf.topk(row0, k, eps=1e-3 / B, options=o)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(4):
        stf.topk(row0, k, eps=1e-3 / B, seed=r, options=o)
    e1.record()
    e1.synchronize()
    t_row = e0.elapsed_time(e1) / 4
    print("[case] ms batched", round(tk, 3), "one row flat", round(t_row, 3), flush=True)
    check_batched(x, vals, idx, k)
    assert tk < 2 * B * t_row


@pytest.mark.parametrize("kind,B,N,k", [("normal", 64, 9000, 1024), ("uniform", 20, 16384, 3000)])
def test_batched_short_rows_without_a_paying_sample_are_sorted_whole(kind, B, N, k):
    """Rows of up to 16384 values for which the solver finds that the sample does not pay
    off (k a large share of the row) are sorted whole in LDS, one workgroup per row,
    instead of running the exact selection row by row."""
    say("batched direct rows", kind, B, N, k)
    assert stf.solve(N, k, 1e-3 / B)["direct_exact"]
    x = generate(kind, B * N, seed=N).reshape(B, N)
    vals, idx, st = stf.topk_batched(dev(x), k, stats=True)
    check_batched(x, vals, idx, k)
    assert st["rows_fallback"] == B and st["attempts"] == 0


def test_batched_strided_rows():
    say("batched strided ld = N + 3")
    B, N, ld, k = 24, 1 << 18, (1 << 18) + 3, 50
    full = generate("normal", B * ld, seed=32).reshape(B, ld)
    xd = dev(full)[:, :N]  # row stride ld, rows misaligned
    vals, idx = stf.topk_batched(xd, k, options={"s_override": 4096})
    check_batched(full[:, :N], vals, idx, k)


def test_batched_forced_overflow_falls_back_per_row():
    say("batched forced overflow")
    B, N, k = 6, 1 << 18, 40
    x = generate("normal", B * N, seed=33).reshape(B, N)
    vals, idx, st = stf.topk_batched(dev(x), k, options={"s_override": 4096, "force_M": k}, stats=True)
    check_batched(x, vals, idx, k)
    assert st["rows_fallback"] == B and st["attempts"] == 6


def test_rejects_bad_arguments_on_device():
    import torch
    x = torch.zeros(100, device="cuda")
    with pytest.raises(stf.ProfkError):
        stf.topk(x, 0)
    with pytest.raises(stf.ProfkError):
        stf.topk(x, 101)
    with pytest.raises(stf.ProfkError):
        stf.topk(x, 10, eps=0.0)


def test_rare_hit_cases_take_the_sparse_filter_shape():
    """The last two SMALL cases are there for the filter's launch shape for rare hits;
    keep them in its regime (the library takes it when E[R] + 3 sd(R) <= N / 8192)."""
    import math
    for kind, N, k, opts in SMALL[-2:]:
        p = stf.solve(N, k, 1e-3, options=opts)
        assert (p["E_R"] + 3 * math.sqrt(p["Var_R"])) * 8192 <= N, (N, k, p["E_R"], p["Var_R"])


@pytest.mark.parametrize("N", [1 << 24, (1 << 20) + 3, 5])
def test_read_ceiling_probe_reads_every_value(N):
    """The measurement helper behind the read ceiling must read every value once: its
    fold is the XOR of all bit patterns."""
    say("read ceiling probe", N)
    x = generate("normal", N, seed=50)
    out = stf.read_ceiling(dev(x))
    want = int(np.bitwise_xor.reduce(x.view(np.uint32)))
    assert int(host(out)[0]) == want
