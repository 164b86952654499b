"""The entry point that allocates nothing, profk_topk_approx_noalloc, against the
entry point it varies, profk_topk_approx (approximate mode: "Prof-K: Probabilistic
One-Pass Filtering for Efficient Top-k Selection", App. D "Cost of the Run-Time
Check").  Same arguments, same seed: the outputs and the check record must be
bit-identical, call after call on the one static scratch array (each call with a
different, also a smaller, input than the one before), and bit-exact against the
CPU oracle whenever the device reports k <= R <= M.
"""
import numpy as np
import pytest

import oracle
import sampling_threshold_filtering_amd as stf
from workloads import generate

pytestmark = pytest.mark.gpu


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def say(*a):
    print("[case]", *a, flush=True)


def same(a, b):
    import torch
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                       b.view(torch.int32) if b.dtype == torch.float32 else b)


# a sequence of calls in a row on the same static array: larger, then smaller inputs,
# a direct exact selection (sample not worth it) in between, and k on both refinements
SEQUENCE = [("pareto", 1 << 24, 4096, 3), ("normal", 1 << 22, 1000, 4), ("uniform", 1 << 26, 32768, 5),
            ("normal", 4096, 17, 6), ("uniform", 1 << 20, 32, 7), ("pareto", 1 << 23, 1 << 17, 8)]


def test_noalloc_matches_approx_call_after_call():
    import torch
    for kind, N, k, seed in SEQUENCE:
        say("noalloc", kind, N, k, seed)
        x = generate(kind, N, seed=seed)
        xd = dev(x)
        rv, ri, rinfo = stf.topk_approx(xd, k, eps=1e-3, seed=seed)
        vals = torch.full((k,), 7.0, dtype=torch.float32, device="cuda")
        idx = torch.full((k,), -9, dtype=torch.int64, device="cuda")
        info = torch.full((stf.APPROX_INFO_WORDS,), -5, dtype=torch.int64, device="cuda")
        stf.topk_approx_noalloc(xd, k, eps=1e-3, seed=seed, out=(vals, idx), info=info)
        torch.cuda.synchronize()
        assert torch.equal(info, rinfo), (stf.approx_info(info), stf.approx_info(rinfo))
        inf = stf.approx_info(info)
        print("[case] info", inf, flush=True)
        assert inf["status"] != 2, "an overflow keeps an unspecified subset: pick another seed"
        assert same(idx, ri) and same(vals, rv), (kind, N, k)
        if inf["status"] == 0:
            ov, oi = oracle.topk(x, k, nthreads=8)
            np.testing.assert_array_equal(host(idx), oi)
            np.testing.assert_array_equal(host(vals).view(np.uint32), ov.view(np.uint32))


def assert_valid_partial(x, vals, idx, k, R, M):
    """The sorted top of min(R, M) entries that all rank at or above the R-th."""
    i = host(idx)
    v = host(vals).view(np.uint32)
    kept = min(R, M, k)
    assert np.all(i[kept:] == -1) and np.all(v[kept:] == np.uint32(0xFF800000))
    got = i[:kept]
    assert len(set(got.tolist())) == kept and got.min() >= 0 and got.max() < x.size
    np.testing.assert_array_equal(v[:kept], x[got].view(np.uint32))
    assert set(got.tolist()) <= set(oracle.topk(x, R, nthreads=8)[1].tolist())
    xv = x[got].astype(np.float64)
    assert np.all((xv[:-1] > xv[1:]) | ((xv[:-1] == xv[1:]) & (got[:-1] < got[1:])))


def test_noalloc_forced_failures_match_approx():
    """Failed checks.  A recall failure (R < k) keeps every hit, so both entry points
    give the same padded output bit for bit.  On an overflow (R > M) which M hits the
    buffer keeps depends on the order in which wavefronts reserve slots (unspecified,
    and different from call to call on either entry point): there the check record must
    match and the output must be a valid sorted top of M entries ranked <= R."""
    import torch
    N = 1 << 22
    x = generate("normal", N, seed=40)
    xd = dev(x)
    for k, opts in ((4096, {"force_t": 1}), (500, {"force_M": 500})):
        say("noalloc forced", k, opts)
        rv, ri, rinfo = stf.topk_approx(xd, k, seed=1, options=opts)
        vals, idx, info = stf.topk_approx_noalloc(xd, k, seed=1, options=opts)
        torch.cuda.synchronize()
        inf = stf.approx_info(info)
        print("[case] info", inf, flush=True)
        assert torch.equal(info, rinfo)
        if inf["status"] == 1:
            assert same(idx, ri) and same(vals, rv)
        else:
            assert inf["status"] == 2
            assert_valid_partial(x, vals, idx, k, inf["R"], inf["M"])


def test_noalloc_graph_capture_and_replay():
    """Captured in a HIP graph after one eager call on the device; every replay, with
    eager work and synchronisations in between, reproduces the eager result."""
    import torch
    say("noalloc graph capture")
    N, k = 1 << 24, 4096
    x = generate("pareto", N, seed=34)
    xd = dev(x)
    s = torch.cuda.Stream()
    vals = torch.empty(k, dtype=torch.float32, device="cuda")
    idx = torch.empty(k, dtype=torch.int64, device="cuda")
    info = torch.empty(stf.APPROX_INFO_WORDS, dtype=torch.int64, device="cuda")
    with torch.cuda.stream(s):
        stf.topk_approx_noalloc(xd, k, seed=3, out=(vals, idx), info=info)
    s.synchronize()
    ev, ei = vals.clone(), idx.clone()
    ov, oi = oracle.topk(x, k, nthreads=8)
    np.testing.assert_array_equal(host(ei), oi)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        stf.topk_approx_noalloc(xd, k, seed=3, out=(vals, idx), info=info)
    for r in range(4):
        vals.fill_(0.0)
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(idx, ei) and same(vals, ev), r
        assert stf.approx_info(info)["status"] == 0
        # a different, smaller call on the same array between replays
        stf.topk_approx_noalloc(xd[: 1 << 20], 64, seed=r)
        _ = (xd[:1000] * 2).sum().item()


def test_noalloc_rejects_calls_beyond_the_static_scratch():
    """k = 2^22 of 2^23 values needs two 32 MiB key buffers plus the rest: more than the
    64 MiB array.  The call is refused before anything is enqueued."""
    import torch
    say("noalloc too large")
    xd = torch.zeros(1 << 23, dtype=torch.float32, device="cuda")
    with pytest.raises(stf.ProfkError) as e:
        stf.topk_approx_noalloc(xd, 1 << 22)
    assert e.value.code == stf.PROFK_ESCRATCH
    assert "static scratch" in str(e.value)
