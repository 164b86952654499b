"""Prof-K exact top-k for MI355X (gfx950): thin Python binding over libprofk.so.

Every step of the selection runs in the library's HIP kernels; this module only
marshals arguments.  PyTorch supplies device memory and the stream handle.
The library must have been built (``python -m
sampling_threshold_filtering_amd.build_native`` or ``__graft_entry__.build()``);
there is no fallback of any kind when it is missing.

Functions mirror include/profk.h:
  topk(x, k, eps=1e-3, seed=0, options=None, stats=False)
  topk_batched(x2d, k, eps=1e-3, seed=0, options=None, stats=False)
  solve(N, k, eps=1e-3, options=None) -> dict
  stage_sample / stage_threshold / stage_filter  (one stage each, for inspection)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprofk.so")

PROFK_OK = 0
PROFK_EINVAL = -1
PROFK_EUNSUPPORTED = -2
PROFK_ENOMEM = -3
PROFK_EHIP = -4
PROFK_EINTERNAL = -5
PROFK_ESCRATCH = -6

STATS_ATTEMPTS = 8

EXPORTED = ("profk_topk", "profk_topk_ex", "profk_topk_approx", "profk_topk_approx_noalloc", "profk_topk_batched",
            "profk_topk_batched_ex", "profk_topk_batched_approx",
            "profk_solve",
            "profk_stage_sample", "profk_stage_threshold", "profk_stage_batched_sample", "profk_stage_filter",
            "profk_read_ceiling", "profk_strerror", "profk_release")


class Options(ctypes.Structure):
    _fields_ = [
        ("s_override", ctypes.c_int64),
        ("s_min", ctypes.c_int64),
        ("s_max", ctypes.c_int64),
        ("s_prefactor", ctypes.c_double),
        ("force_t", ctypes.c_int64),
        ("force_M", ctypes.c_int64),
        ("max_attempts", ctypes.c_int32),
        ("use_max_attempts", ctypes.c_int32),
        ("force_fallback", ctypes.c_int32),
        ("timing", ctypes.c_int32),
        ("param_mode", ctypes.c_int32),
        ("s_rule", ctypes.c_int32),
        ("cost_a", ctypes.c_double),
        ("cost_b", ctypes.c_double),
        ("refine_wait_ticks", ctypes.c_int64),
    ]


PARAMS_EXACT = 0
PARAMS_FAST = 1
S_RULE_CUBE_ROOT = 0
S_RULE_COST_MODEL = 1
S_RULE_MI355X = 2


class Params(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64), ("k", ctypes.c_int64), ("eps", ctypes.c_double),
        ("eps_a", ctypes.c_double), ("eps_b", ctypes.c_double), ("z_a", ctypes.c_double),
        ("z", ctypes.c_double), ("S_raw", ctypes.c_double), ("S", ctypes.c_int64),
        ("t_star", ctypes.c_int64), ("M_star", ctypes.c_int64), ("M_cf", ctypes.c_double),
        ("t_eq6", ctypes.c_int64), ("t", ctypes.c_int64), ("M", ctypes.c_int64),
        ("p_recall", ctypes.c_double), ("p_overflow", ctypes.c_double), ("E_R", ctypes.c_double),
        ("Var_R", ctypes.c_double), ("direct_exact", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class Stats(ctypes.Structure):
    _fields_ = [
        ("attempts", ctypes.c_int32), ("fallback", ctypes.c_int32),
        ("S", ctypes.c_int64), ("t", ctypes.c_int64), ("M", ctypes.c_int64),
        ("R", ctypes.c_int64 * STATS_ATTEMPTS), ("fail_mode", ctypes.c_int32 * STATS_ATTEMPTS),
        ("workspace_bytes", ctypes.c_uint64), ("filter_ms", ctypes.c_double),
        ("rows_retried", ctypes.c_int64), ("rows_fallback", ctypes.c_int64),
        ("refine_multipass", ctypes.c_int64), ("segments", ctypes.c_int64),
    ]


class ProfkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"profk error {code}: {msg}")
        self.code = code


_lib = None


def load_library():
    """Load libprofk.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sampling_threshold_filtering_amd.build_native`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, f64, u64, i32, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p
    lib.profk_topk.argtypes = [vp, i64, i64, f64, u64, vp, vp, vp]
    lib.profk_topk_ex.argtypes = [vp, i64, i64, f64, u64, vp, vp, vp, ctypes.POINTER(Options),
                                  ctypes.POINTER(Stats)]
    lib.profk_topk_approx.argtypes = [vp, i64, i64, f64, u64, vp, vp, vp, vp, ctypes.POINTER(Options)]
    lib.profk_topk_approx_noalloc.argtypes = [vp, i64, i64, f64, u64, vp, vp, vp, vp, ctypes.POINTER(Options)]
    lib.profk_topk_batched.argtypes = [vp, i64, i64, i64, i64, f64, u64, vp, vp, vp]
    lib.profk_topk_batched_ex.argtypes = [vp, i64, i64, i64, i64, f64, u64, vp, vp, vp, ctypes.POINTER(Options),
                                          ctypes.POINTER(Stats)]
    lib.profk_topk_batched_approx.argtypes = [vp, i64, i64, i64, i64, f64, u64, vp, vp, vp, vp,
                                              ctypes.POINTER(Options)]
    lib.profk_solve.argtypes = [i64, i64, f64, ctypes.POINTER(Options), ctypes.POINTER(Params)]
    lib.profk_stage_sample.argtypes = [vp, i64, i64, u64, i32, vp, vp]
    lib.profk_stage_threshold.argtypes = [vp, i64, i64, i64, u64, i32, vp, vp, vp]
    lib.profk_stage_batched_sample.argtypes = [vp, i64, i64, i64, i64, i64, u64, i32, vp, vp, vp, vp]
    lib.profk_stage_filter.argtypes = [vp, i64, ctypes.c_float, i64, i64, vp, vp, vp]
    lib.profk_read_ceiling.argtypes = [vp, i64, i32, vp, vp]
    lib.profk_read_ceiling.restype = ctypes.c_int
    lib.profk_strerror.argtypes = [ctypes.c_int]
    lib.profk_strerror.restype = ctypes.c_char_p
    lib.profk_release.argtypes = []
    lib.profk_release.restype = None
    for name in ("profk_topk", "profk_topk_ex", "profk_topk_approx", "profk_topk_approx_noalloc", "profk_topk_batched",
                 "profk_topk_batched_ex", "profk_topk_batched_approx",
                 "profk_solve",
                 "profk_stage_sample", "profk_stage_threshold", "profk_stage_batched_sample", "profk_stage_filter"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != PROFK_OK:
        msg = load_library().profk_strerror(rc).decode()
        raise ProfkError(rc, msg)


def make_options(**kw) -> Options:
    o = Options()
    for k, v in kw.items():
        if not hasattr(o, k):
            raise KeyError(k)
        setattr(o, k, v)
    return o


def _opt_ptr(options):
    if options is None:
        return None
    if isinstance(options, dict):
        options = make_options(**options)
    return ctypes.byref(options)


def stats_to_dict(st: Stats) -> dict:
    n = min(st.attempts, STATS_ATTEMPTS)
    return dict(attempts=st.attempts, fallback=bool(st.fallback), S=st.S, t=st.t, M=st.M,
                R=[st.R[i] for i in range(n)], fail_mode=[st.fail_mode[i] for i in range(n)],
                workspace_bytes=st.workspace_bytes, filter_ms=st.filter_ms,
                rows_retried=st.rows_retried, rows_fallback=st.rows_fallback,
                refine_multipass=st.refine_multipass, segments=st.segments)


def _stream_ptr(torch, device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _raw_stream(torch, index: int) -> int:
    """The current stream of device `index` as a raw handle (no Stream object is built:
    the per-call host time matters where the call returns before the GPU work ends)."""
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(index)
    return torch.cuda.current_stream(index).cuda_stream


def _current_device(torch) -> int:
    get = getattr(torch._C, "_cuda_getDevice", None)
    return get() if get is not None else torch.cuda.current_device()


def _check_out(out, shape, device):
    import torch
    vals, idx = out
    if (tuple(vals.shape) != shape or tuple(idx.shape) != shape or vals.dtype != torch.float32
            or idx.dtype != torch.int64 or vals.device != device or idx.device != device
            or not vals.is_contiguous() or not idx.is_contiguous()):
        raise ValueError(f"out must be contiguous float32 / int64 tensors of shape {shape} on {device}")
    return vals, idx


def topk(x, k: int, eps: float = 1e-3, seed: int = 0, options=None, stats: bool = False, out=None):
    """Exact top-k of a 1-D float32 CUDA tensor: (values, int64 indices), sorted
    (value descending, ties to the lower index).  `out=(values, indices)` reuses
    caller buffers.  The outputs are complete in stream order on return."""
    import torch
    if x.dim() != 1 or x.dtype != torch.float32 or not x.is_cuda:
        raise ValueError("x must be a 1-D float32 device tensor")
    if not x.is_contiguous():
        x = x.contiguous()
    lib = _lib if _lib is not None else load_library()
    di = x.get_device()
    if out is None:
        vals = torch.empty(k, dtype=torch.float32, device=x.device)
        idx = torch.empty(k, dtype=torch.int64, device=x.device)
    else:
        vals, idx = _check_out(out, (k,), x.device)
    st = Stats() if stats else None
    args = (x.data_ptr(), x.numel(), k, eps, seed & (2**64 - 1), vals.data_ptr(), idx.data_ptr(),
            _raw_stream(torch, di), _opt_ptr(options), ctypes.byref(st) if st is not None else None)
    if di == _current_device(torch):
        rc = lib.profk_topk_ex(*args)
    else:
        with torch.cuda.device(di):
            rc = lib.profk_topk_ex(*args)
    _check(rc)
    if stats:
        return vals, idx, stats_to_dict(st)
    return vals, idx


APPROX_INFO_WORDS = 3  # profk_approx_info: int64 R, int64 M, int32 status, int32 exact_path


def topk_approx(x, k: int, eps: float = 1e-3, seed: int = 0, options=None, out=None, info=None):
    """Approximate mode: one sampled attempt, enqueued without any host wait (so it
    can be captured in a CUDA/HIP graph after a first call).  Returns (values,
    indices, info) where info is an int64 device tensor of 3 words holding the
    profk_approx_info record; decode it with approx_info().  `out` and `info`
    reuse caller buffers."""
    return _topk_approx("profk_topk_approx", x, k, eps, seed, options, out, info)


def topk_approx_noalloc(x, k: int, eps: float = 1e-3, seed: int = 0, options=None, out=None, info=None):
    """profk_topk_approx_noalloc: topk_approx on the library's static scratch (the
    library allocates no device memory).  Pass `out` and `info` to keep torch's
    allocator out of it as well.  Raises ProfkError (code PROFK_ESCRATCH) when the
    call needs more scratch than the static array holds."""
    return _topk_approx("profk_topk_approx_noalloc", x, k, eps, seed, options, out, info)


def _topk_approx(entry, x, k, eps, seed, options, out, info):
    import torch
    if x.dim() != 1 or x.dtype != torch.float32 or not x.is_cuda:
        raise ValueError("x must be a 1-D float32 device tensor")
    if not x.is_contiguous():
        x = x.contiguous()
    lib = _lib if _lib is not None else load_library()
    dev = x.device
    di = x.get_device()
    if out is None:
        vals = torch.empty(k, dtype=torch.float32, device=dev)
        idx = torch.empty(k, dtype=torch.int64, device=dev)
    else:
        vals, idx = _check_out(out, (k,), dev)
    if info is None:
        info = torch.empty(APPROX_INFO_WORDS, dtype=torch.int64, device=dev)
    elif info.dtype != torch.int64 or info.numel() < APPROX_INFO_WORDS or info.device != dev:
        raise ValueError("info must be an int64 device tensor of 3 words on the input's device")
    args = (x.data_ptr(), x.numel(), k, eps, seed & (2**64 - 1), vals.data_ptr(), idx.data_ptr(), info.data_ptr(),
            _raw_stream(torch, di), _opt_ptr(options))
    fn = getattr(lib, entry)
    if di == _current_device(torch):
        rc = fn(*args)
    else:
        with torch.cuda.device(di):
            rc = fn(*args)
    _check(rc)
    return vals, idx, info


def approx_info(info) -> dict:
    """Decode a profk_approx_info record (int64 tensor of 3 words) on the host."""
    w = [int(v) for v in info.detach().cpu().tolist()[:APPROX_INFO_WORDS]]
    st = w[2] & 0xFFFFFFFF
    ex = (w[2] >> 32) & 0xFFFFFFFF
    return {"R": w[0], "M": w[1], "status": st - (1 << 32) if st >= (1 << 31) else st, "exact_path": ex}


def topk_batched(x, k: int, eps: float = 1e-3, seed: int = 0, options=None, stats: bool = False):
    """Row-wise exact top-k of a 2-D float32 CUDA tensor (rows may be strided):
    (values [B,k], int64 column indices [B,k])."""
    import torch
    if x.dim() != 2 or x.dtype != torch.float32 or not x.is_cuda:
        raise ValueError("x must be a 2-D float32 device tensor")
    if x.stride(1) != 1:
        x = x.contiguous()
    B, N = x.shape
    ld = x.stride(0) if B > 1 else N
    lib = load_library()
    vals = torch.empty((B, k), dtype=torch.float32, device=x.device)
    idx = torch.empty((B, k), dtype=torch.int64, device=x.device)
    st = Stats() if stats else None  # statistics make the call wait for every row's record
    with torch.cuda.device(x.device):
        rc = lib.profk_topk_batched_ex(ctypes.c_void_p(x.data_ptr()), B, N, ld, k, eps, seed & (2**64 - 1),
                                       ctypes.c_void_p(vals.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                                       _stream_ptr(torch, x.device), _opt_ptr(options),
                                       ctypes.byref(st) if st is not None else None)
    _check(rc)
    if stats:
        return vals, idx, stats_to_dict(st)
    return vals, idx


def topk_batched_approx(x, k: int, eps: float = 1e-3, seed: int = 0, options=None, out=None, info=None):
    """Batched approximate mode on a 2-D float32 device tensor (rows may be strided):
    one attempt per row, enqueued without any host wait.  Returns (values [B,k],
    column indices [B,k], info) where info is an int64 device tensor [B, 3] of
    profk_approx_info records (decode with approx_info_rows(info)).  `out` and
    `info` reuse caller buffers."""
    import torch
    if x.dim() != 2 or x.dtype != torch.float32 or not x.is_cuda:
        raise ValueError("x must be a 2-D float32 device tensor")
    if x.stride(1) != 1:
        x = x.contiguous()
    B, N = x.shape
    ld = x.stride(0) if B > 1 else N
    dev = x.device
    if out is None:
        vals = torch.empty((B, k), dtype=torch.float32, device=dev)
        idx = torch.empty((B, k), dtype=torch.int64, device=dev)
    else:
        vals, idx = _check_out(out, (B, k), dev)
    if info is None:
        info = torch.empty((B, APPROX_INFO_WORDS), dtype=torch.int64, device=dev)
    elif (info.dtype != torch.int64 or tuple(info.shape) != (B, APPROX_INFO_WORDS) or info.device != dev
          or not info.is_contiguous()):
        raise ValueError("info must be a contiguous int64 device tensor of shape (B, 3)")
    with torch.cuda.device(dev):
        rc = load_library().profk_topk_batched_approx(
            ctypes.c_void_p(x.data_ptr()), B, N, ld, k, eps, seed & (2**64 - 1), ctypes.c_void_p(vals.data_ptr()),
            ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(info.data_ptr()), _stream_ptr(torch, dev),
            _opt_ptr(options))
    _check(rc)
    return vals, idx, info


def approx_info_rows(info) -> list:
    """Decode a [B, 3] batch of profk_approx_info records on the host."""
    return [approx_info(r) for r in info.detach().cpu()]


def solve(N: int, k: int, eps: float = 1e-3, options=None) -> dict:
    """Host-only parameter choice (no GPU needed)."""
    p = Params()
    _check(load_library().profk_solve(N, k, eps, _opt_ptr(options), ctypes.byref(p)))
    return {name: getattr(p, name) for name, _ in Params._fields_ if name != "reserved"}


def stage_sample(x, S: int, seed: int = 0, attempt: int = 0):
    """The S sampled indices (unordered int64 tensor) of (seed, attempt)."""
    import torch
    out = torch.empty(S, dtype=torch.int64, device=x.device)
    with torch.cuda.device(x.device):
        rc = load_library().profk_stage_sample(ctypes.c_void_p(x.data_ptr()), x.numel(), S, seed, attempt,
                                               ctypes.c_void_p(out.data_ptr()), _stream_ptr(torch, x.device))
    _check(rc)
    return out


def stage_threshold(x, S: int, t: int, seed: int = 0, attempt: int = 0):
    """tau = (value, index) of the t-th largest sampled entry."""
    import torch
    v = torch.empty(1, dtype=torch.float32, device=x.device)
    i = torch.empty(1, dtype=torch.int64, device=x.device)
    with torch.cuda.device(x.device):
        rc = load_library().profk_stage_threshold(ctypes.c_void_p(x.data_ptr()), x.numel(), S, t, seed, attempt,
                                                  ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(i.data_ptr()),
                                                  _stream_ptr(torch, x.device))
    _check(rc)
    return v, i


def stage_batched_sample(x, S: int, t: int, seed: int = 0, attempt: int = 0):
    """Batched stages 1-2 on a 2-D float32 device tensor (rows may be strided):
    (sample indices [B, S] int64, each row unordered; tau values [B]; tau indices [B])."""
    import torch
    if x.dim() != 2 or x.dtype != torch.float32 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 device tensor with unit column stride")
    B, N = x.shape
    ld = x.stride(0) if B > 1 else N
    out = torch.empty((B, S), dtype=torch.int64, device=x.device)
    tv = torch.empty(B, dtype=torch.float32, device=x.device)
    ti = torch.empty(B, dtype=torch.int64, device=x.device)
    with torch.cuda.device(x.device):
        rc = load_library().profk_stage_batched_sample(ctypes.c_void_p(x.data_ptr()), B, N, ld, S, t, seed, attempt,
                                                       ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(tv.data_ptr()),
                                                       ctypes.c_void_p(ti.data_ptr()), _stream_ptr(torch, x.device))
    _check(rc)
    return out, tv, ti


def stage_filter(x, tau_val: float, tau_idx: int, M: int):
    """(R, candidate indices of the min(R, M) kept entries, unordered)."""
    import torch
    cand = torch.empty(M, dtype=torch.int64, device=x.device)
    R = torch.empty(1, dtype=torch.int64, device=x.device)
    with torch.cuda.device(x.device):
        rc = load_library().profk_stage_filter(ctypes.c_void_p(x.data_ptr()), x.numel(), ctypes.c_float(tau_val),
                                               tau_idx, M, ctypes.c_void_p(cand.data_ptr()),
                                               ctypes.c_void_p(R.data_ptr()), _stream_ptr(torch, x.device))
    _check(rc)
    r = int(R.item())
    return r, cand[: min(r, M)]


def read_ceiling(x, blocks_per_cu: int = 0, out=None):
    """Measurement helper: one dwordx4 non-temporal read of a 1-D float32 device tensor
    (16-byte aligned), nothing else; enqueued on the current stream.  XORs the XOR
    of all values' bits into `out` (a one-word int64 tensor, or a new zero one) and
    returns it."""
    import torch
    if x.dim() != 1 or x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 1-D float32 device tensor")
    if out is None:
        out = torch.zeros(1, dtype=torch.int64, device=x.device)
    with torch.cuda.device(x.device):
        rc = load_library().profk_read_ceiling(ctypes.c_void_p(x.data_ptr()), x.numel(), blocks_per_cu,
                                               ctypes.c_void_p(out.data_ptr()), _stream_ptr(torch, x.device))
    _check(rc)
    return out


def release():
    load_library().profk_release()
