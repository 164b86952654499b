"""GPU parity of the batched form's own stages and of its per-row retry.

Stages 1-2 per row ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
Selection", §3 stages 1-2, applied to each batch element; App. C: a threshold per
row): every row's sample set and threshold tau from the batched sampler are compared
bit for bit with the oracle's sample_indices(N, S, seed, attempt, row=r) and
threshold(x[r], sample, t), on the register-list path (t <= 64, S <= 8192, with
and without a heavy top-up), on the radix-select path (t > 64, or S > 8192) and on
tie-heavy and strided rows.  The end-to-end result is exact for any sample, so only
these checks catch a biased or repeat-keeping per-row sampler.

Per-row retry (§3 stage 4 per row; App. E.2): with a buffer capacity or a threshold
rank forced so that about half the rows fail each attempt, only those rows are
redrawn; every row, whichever attempt finished it, must match the oracle.
"""
import numpy as np
import pytest

import oracle
import sampling_threshold_filtering_amd as stf
from oracle import method_ref
from workloads import generate

pytestmark = pytest.mark.gpu


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def say(*a):
    print("[case]", *a, flush=True)


STAGE_CASES = [
    # kind, B, N, S, t, seed, attempt, extra columns of row stride
    ("pareto", 64, 1 << 20, 4096, 13, 0, 0, 0),     # the 1024 x 2^20 workload's rows, MI355X rule
    ("normal", 64, 1 << 14, 2048, 20, 1, 0, 0),     # S = N/8: ~130 repeats per row, heavy top-up
    ("uniform", 64, 1 << 18, 8192, 64, 2, 1, 0),    # boundary of the list path (t = 64, S = 8192)
    ("uniform", 64, 1 << 18, 4096, 100, 3, 0, 0),   # t > 64: radix select over the row's keys
    ("pareto", 64, 1 << 20, 32768, 13, 4, 0, 0),    # S > 8192: the default rule's per-row shape
    ("normal", 96, 1 << 16, 1024, 5, 5, 3, 0),      # a later attempt's counter space
    ("adv_noise", 64, 1 << 16, 2048, 30, 6, 0, 0),  # 256 distinct values: tau decided by the index
    ("normal", 64, 100003, 4000, 7, 7, 0, 3),       # ragged, misaligned strided rows
    ("normal", 1, 1 << 20, 4096, 1, 8, 0, 0),       # one row, t = 1
]


@pytest.mark.parametrize("kind,B,N,S,t,seed,attempt,pad", STAGE_CASES)
def test_batched_sample_and_threshold_match_oracle(kind, B, N, S, t, seed, attempt, pad):
    say("batched stages", kind, B, N, S, t, seed, attempt, pad)
    ld = N + pad
    full = generate(kind, B * ld, seed=seed + 100).reshape(B, ld)
    xd = dev(full)[:, :N]
    got_idx, tau_v, tau_i = stf.stage_batched_sample(xd, S, t, seed=seed, attempt=attempt)
    got_idx, tau_v, tau_i = host(got_idx), host(tau_v), host(tau_i)
    for r in range(B):
        ref = method_ref.sample_indices(N, S, seed=seed, attempt=attempt, row=r)
        np.testing.assert_array_equal(np.sort(got_idx[r]), ref, err_msg=f"row {r}")
        rv, ri = method_ref.threshold(full[r, :N], ref, t)
        assert tau_i[r] == ri, (r, tau_i[r], ri)
        assert tau_v[r:r + 1].view(np.uint32)[0] == np.float32(rv).view(np.uint32), r


GRID_CASES = [
    # rows longer than 2^20: the grid sampler (one draw per thread, a hash set per row)
    ("normal", 8, (1 << 21) + 5, 32768, 13, 9, 0, 0),   # sorted block lists (t <= 64), ragged rows
    ("pareto", 4, 1 << 22, 4096, 100, 10, 1, 0),        # unordered top-t block lists (t > 64)
    ("uniform", 4, 1 << 21, 16384, 70, 11, 0, 7),       # the same over 16 blocks, strided rows
    ("uniform", 3, (1 << 21) + 3, 9221, 200, 14, 0, 0),  # a last block with fewer than t draws
    ("adv_noise", 4, 1 << 21, 8192, 30, 12, 2, 0),      # 256 distinct values
    ("normal", 2, 1 << 21, 32768, 2000, 13, 0, 0),      # t > 1024: one workgroup per row over L2
]


@pytest.mark.parametrize("kind,B,N,S,t,seed,attempt,pad", GRID_CASES)
def test_batched_grid_sampler_matches_oracle(kind, B, N, S, t, seed, attempt, pad):
    test_batched_sample_and_threshold_match_oracle(kind, B, N, S, t, seed, attempt, pad)


def check_batched(x, vals, idx, k):
    ov, oi = oracle.topk_batched(x, k, nthreads=16)
    np.testing.assert_array_equal(host(idx), oi)
    np.testing.assert_array_equal(host(vals).view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("mode", ["overflow", "recall"])
def test_batched_retry_with_mixed_passing_and_failing_rows(mode):
    """About half the rows fail each attempt: a capacity M at the median of R (R > M
    in half the rows), or t = 1 with M large (R < k in about 63% of the rows).  Only
    the failed rows are redrawn and the rows finished earlier keep their outputs."""
    B, N, k, S = 128, 1 << 18, 64, 4096
    eps = 1e-3
    x = generate("normal", B * N, seed=41).reshape(B, N)
    base = {"s_override": S}
    p = stf.solve(N, k, eps / B, options=base)
    if mode == "overflow":
        t = p["t"]
        M = int((N + 1) * (t - 1.0 / 3.0) / (S + 1))  # about the median of R (Gamma-like, shape t)
        opts = dict(base, force_M=M)
    else:
        opts = dict(base, force_t=1, force_M=4 * N // S + 8 * k)
    say("batched mixed retry", mode, B, N, k, opts)
    vals, idx, st = stf.topk_batched(dev(x), k, eps=eps, seed=3, options=opts, stats=True)
    print("[case] stats", {kk: st[kk] for kk in ("attempts", "rows_retried", "rows_fallback")}, flush=True)
    check_batched(x, vals, idx, k)
    assert 0 < st["rows_retried"] < B
    assert st["attempts"] >= 2
    assert st["rows_fallback"] < B // 4
    # without statistics the host first takes the filter's summary word, which reports
    # the failed rows; it then reads the per-row records and redraws those rows
    vals, idx = stf.topk_batched(dev(x), k, eps=eps, seed=3, options=opts)
    check_batched(x, vals, idx, k)


@pytest.mark.parametrize("kind,B,N,k,pad", [("pareto", 16, 1 << 22, 64, 0), ("normal", 16, 1 << 22, 1024, 0),
                                           ("uniform", 5, (1 << 21) + 3, 500, 5), ("adv_levels", 4, 1 << 22, 3000, 0),
                                           ("normal", 3, 1 << 21, 20000, 0)])
def test_batched_long_rows(kind, B, N, k, pad):
    """Rows longer than 2^20 (P1 App. E.2 runs N = 2^22 with B = 16) on the batched
    kernels (grid sampler, multi-row filter, per-row refinement); k above 16384 runs
    the flat path row by row."""
    say("batched long rows", kind, B, N, k, pad)
    ld = N + pad
    full = generate(kind, B * ld, seed=N % 1000 + k).reshape(B, ld)
    vals, idx, st = stf.topk_batched(dev(full)[:, :N], k, stats=True)
    print("[case] stats", {kk: st[kk] for kk in ("S", "t", "M", "attempts", "rows_retried", "rows_fallback")},
          flush=True)
    check_batched(np.ascontiguousarray(full[:, :N]), vals, idx, k)


@pytest.mark.parametrize("B,N,k", [(64, 1 << 18, 64), (512, 1 << 16, 32)])
def test_batched_rows_whose_hits_overflow_the_filter_stage(B, N, k):
    """Rows read in the flat order (several rows, positions packed above the index bits)
    stage every wavefront's hits until the end of the stream.  In a row of equal values the
    keys order by index, so the entries at or above tau are the row's first R: whole tiles
    of hits, 1024 per tile, which fill a wavefront's stage and send each further batch
    straight to the row's buffer (a row whose first half holds one value that tops the
    rest does the same).  Every row must match the oracle."""
    x = generate("normal", B * N, seed=B + N).reshape(B, N)
    for r in (3, B // 2, B - 1):
        x[r, :] = np.float32(0.5)  # all ties: tau is decided by the index
    x[B // 2 + 1, : N // 2] = np.float32(1e30)  # the top values: the row's first half
    say("batched stage overflow", B, N, k)
    vals, idx, st = stf.topk_batched(dev(x), k, seed=7, stats=True)
    print("[case] stats", {kk: st[kk] for kk in ("S", "t", "M", "attempts", "rows_retried", "rows_fallback")},
          flush=True)
    check_batched(x, vals, idx, k)
