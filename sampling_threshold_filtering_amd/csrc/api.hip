// Host controller and C ABI of the Prof-K exact top-k library (see include/profk.h).
//
// Control flow of one call ("Prof-K: Probabilistic One-Pass Filtering for Efficient
// Top-k Selection", §3 stages 1-4 and the retry of stage 4):
//   parameters (memoised)          -> S, t, M
//   for attempt a = 0 .. max-1:
//     enqueue sample(seed, a), threshold select, filter (+ check on device),
//             refinement select, compaction, sort + output write
//     copy the 16-byte attempt record back and synchronise the stream once
//     ok -> return; R < k or R > M -> next attempt with a fresh Philox stream
//   exact full selection over all N values (radix select + compaction + sort)
// The refinement is enqueued before the single synchronisation and skips itself
// on device when the check failed, so a successful attempt costs one round trip.
#include <immintrin.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "launch.h"
#include "profk.h"
#include "solver.h"

namespace profk {
namespace {

thread_local std::string t_err;

int hip_fail(hipError_t e, const char* what) {
  t_err = std::string(what) + ": " + hipGetErrorString(e);
  return PROFK_EHIP;
}

#define HIPCHK(call, what)                        \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr int kDefaultAttempts = 6;  // P1 §3 stage 4: exact fallback after six failures
// Needed value bins up to this many keys are partitioned inside the refinement's last
// kernel; a larger one (a tie group of that size within a wide value range) is left to
// the multi-block radix select, which the host enqueues after reading the flag.
constexpr u32 kMsdCapExact = 1u << 18;
// Bound on the fused histogram-and-scatter launch's wait for all of its blocks: 0.25 s of
// the 100 MHz clock (the wait itself takes microseconds when every block is resident).
constexpr u64 kRefineWaitTicks = 25000000;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

u64 pow2_at_least(u64 v) {
  u64 p = 1;
  while (p < v) p <<= 1;
  return p;
}

struct Layout {
  size_t hash = 0, ctl = 0, sel = 0, rec = 0, rtick = 0, ticket = 0, keys = 0, tops = 0, btops = 0, cand = 0, col = 0,
         topk0 = 0, topk1 = 0, hist = 0, rows = 0, scratch = 0, rtmp = 0, rhist = 0, rchunk = 0,
         rcursor = 0, pool = 0, total = 0;
  u64 hash_slots = 0;  // slots of the hash region (the allocation's capacity)
  u64 rows_cap = 0;    // rows of the control regions (the allocation's capacity)
  u64 hash_used = 0;   // slots this request's sample uses (per row with several rows): a power of two >= 2S
};

// Regions that kernels leave zero for the next call (hash set, tickets and counters,
// selection and refinement histograms) and the per-row control blocks sit first, at
// offsets that depend only on the allocation's capacities (hash slots, rows); the
// per-request regions follow.  A later request with other sizes therefore finds them
// where the previous call cleaned them.
// grid_rows > 0: the batched sampler with one hash set, key slots and block lists per
// row of the attempt's list (4 slots per draw, so that B rows' sets stay small), and
// grid_tops words of block lists per row.
Layout make_layout(u64 B, u64 S, u64 M, u64 k, u64 scratch_words, u64 hash_cap, u64 rows_cap, u64 grid_rows = 0,
                   u64 grid_tops = 0) {
  Layout L;
  // hash set of the sample: 16 slots per draw (up to 2^21 slots) keeps probes and
  // contention on the device-scope CAS low; at least 2 per draw for larger samples, and
  // room for the S indices plus a last top-up chunk's kWave new ones on top
  const u64 s1 = S ? S : 1;
  const u64 sparse = 16 * s1 < (1ull << 21) ? 16 * s1 : (1ull << 21);
  const u64 least = 2 * s1 + kWave;
  L.hash_used = grid_rows ? pow2_at_least(4 * s1 > least ? 4 * s1 : least)
                          : pow2_at_least(sparse > least ? sparse : least);
  const u64 hash_need = L.hash_used * (grid_rows ? grid_rows : 1);
  L.hash_slots = hash_need < hash_cap ? hash_cap : hash_need;
  const u64 rows = B < rows_cap ? rows_cap : B;
  L.rows_cap = rows;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.hash = take(L.hash_slots * sizeof(u32));
  L.ctl = take(rows * sizeof(RowCtl));
  L.sel = take(rows * sizeof(SelState));
  L.rec = take(rows * sizeof(AttemptRecord));
  L.rtick = take(rows * sizeof(u64));  // per-row sampling tickets of the batched sampler
  L.ticket = take(kTicketWords * sizeof(u32));
  L.rhist = take(kBins * sizeof(u32));
  L.rcursor = take(kBins * sizeof(u32));
  L.tops = take((size_t)kTopBlocks * kTopT * sizeof(u64));
  // per request
  L.keys = take(2 * (S ? S : 1) * (grid_rows ? grid_rows : 1) * sizeof(u64));  // S draw slots + the top-up
  L.btops = take((grid_rows * grid_tops ? grid_rows * grid_tops : 1) * sizeof(u64));
  L.cand = take(B * (M ? M : 1) * sizeof(u64));
  L.col = take((size_t)kCollectCap * sizeof(u64));
  L.topk0 = take((k ? k : 1) * sizeof(u64));
  L.topk1 = take((k ? k : 1) * sizeof(u64));
  L.hist = take(sort_hist_words(k) * sizeof(u32));
  L.rows = take(B * sizeof(int));
  L.scratch = take((scratch_words ? scratch_words : 1) * sizeof(u64));
  L.rtmp = take((M ? M : 1) * sizeof(u64));
  L.rchunk = take(chunk_entries(M) * 4 * sizeof(u32));
  L.pool = take(msd_pool_words(M) * sizeof(u64));
  L.total = off;
  return L;
}

constexpr u32 kWeightSets = 4;  // die-weight sets, one per filter launch shape (0..3)

struct Workspace {
  int device = -1;
  hipStream_t stream = nullptr;
  char* dev = nullptr;
  size_t bytes = 0;
  u64 hash_cap = 0;  // slots of the hash region at offset 0
  u64 rows_cap = 0;  // rows of the control regions after it
  AttemptRecord* host = nullptr;
  size_t host_n = 0;
  int* host_rows = nullptr;  // pinned list of rows to redraw (batched form)
  size_t host_rows_n = 0;
  HostRecord* hrec = nullptr;      // pinned record the refinement publishes (host address)
  HostRecord* hrec_dev = nullptr;  // the same memory as the device addresses it
  u32 seq = 0;                     // last sequence number asked of the device
  // Set while a call's kernels may have left counters, tickets or the hash set
  // nonzero (an error between launches); the next call then clears them first.
  bool dirty = false;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  // Relative streaming speed of each die, from the filter's per-die times on earlier
  // calls (moving average); the filter sizes the dies' shares of the input by it.  One
  // set per filter launch shape (blocks per CU and tile width change the dies' relative
  // speeds), shared by the flat and the multi-row filter.
  float xw[kWeightSets][kXcds];
  u32 xw_updates[kWeightSets] = {};  // calls that have updated each set
  Workspace() {
    for (u32 c = 0; c < kWeightSets; ++c)
      for (u32 x = 0; x < kXcds; ++x) xw[c][x] = 1.f;
  }
  char* seg = nullptr;  // per-segment top-k lists of inputs of 2^32 values or more
  size_t seg_bytes = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace*> g_ws;

struct Need {
  u64 B, S, M, k;
  u64 scratch_words = 0;
  u64 grid_rows = 0;  // the batched sampler's rows (see make_layout)
  u64 grid_tops = 0;
};

int get_workspace(hipStream_t s, const Need& need, Workspace** out, Layout* out_layout) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev), "hipGetDevice");
  const u64 rows = need.B;
  std::lock_guard<std::mutex> g(g_ws_mu);
  Workspace*& w = g_ws[std::make_pair(dev, s)];
  if (!w) {
    w = new Workspace();
    w->device = dev;
    w->stream = s;
  }
  Layout L = make_layout(need.B, need.S, need.M, need.k, need.scratch_words, w->hash_cap, w->rows_cap,
                         need.grid_rows, need.grid_tops);
  if (w->bytes < L.total || w->hash_cap < L.hash_slots || w->rows_cap < L.rows_cap) {
    if (w->dev) {
      HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
      HIPCHK(hipFree(w->dev), "hipFree");
      w->dev = nullptr;
      w->bytes = 0;
    }
    size_t want = L.total + L.total / 4;
    void* p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) {
      (void)hipGetLastError();
      want = L.total;
      if (hipMalloc(&p, want) != hipSuccess) {
        (void)hipGetLastError();
        t_err = "workspace allocation failed";
        return PROFK_ENOMEM;
      }
    }
    w->dev = (char*)p;
    w->bytes = want;
    w->hash_cap = L.hash_slots;
    w->rows_cap = L.rows_cap;
    // zero everything once: hash set, selection histograms, counters; every kernel
    // leaves what it uses zero again
    HIPCHK(hipMemsetAsync(w->dev, 0, want, s), "hipMemsetAsync");
    w->dirty = false;
  }
  if (w->host_n < rows) {
    if (w->host) (void)hipHostFree(w->host);
    w->host = nullptr;
    w->host_n = 0;
    HIPCHK(hipHostMalloc((void**)&w->host, rows * sizeof(AttemptRecord), hipHostMallocDefault), "hipHostMalloc");
    w->host_n = rows;
  }
  if (w->host_rows_n < rows) {
    if (w->host_rows) (void)hipHostFree(w->host_rows);
    w->host_rows = nullptr;
    w->host_rows_n = 0;
    HIPCHK(hipHostMalloc((void**)&w->host_rows, rows * sizeof(int), hipHostMallocDefault), "hipHostMalloc");
    w->host_rows_n = rows;
  }
  if (!w->hrec) {
    HIPCHK(hipHostMalloc((void**)&w->hrec, sizeof(HostRecord), hipHostMallocMapped | hipHostMallocCoherent),
           "hipHostMalloc");
    std::memset(w->hrec, 0, sizeof(HostRecord));
    HIPCHK(hipHostGetDevicePointer((void**)&w->hrec_dev, w->hrec, 0), "hipHostGetDevicePointer");
    w->seq = 0;
  }
  if (!w->ev0) {
    // timing only: no system-scope fences around the filter
    HIPCHK(hipEventCreateWithFlags(&w->ev0, hipEventDisableSystemFence), "hipEventCreate");
    HIPCHK(hipEventCreateWithFlags(&w->ev1, hipEventDisableSystemFence), "hipEventCreate");
  }
  *out = w;
  *out_layout = L;
  return PROFK_OK;
}

template <class T>
T* at(Workspace* w, size_t off) {
  return reinterpret_cast<T*>(w->dev + off);
}

// After a call that stopped between launches: clear the hash set, tickets, control
// blocks and histograms that its kernels would have left zero.
int clean_if_dirty(Workspace* w, const Layout& L, hipStream_t s) {
  if (!w->dirty) return PROFK_OK;
  HIPCHK(hipMemsetAsync(w->dev + L.hash, 0, L.hash_slots * sizeof(u32), s), "hipMemsetAsync");
  HIPCHK(hipMemsetAsync(w->dev + L.rtick, 0, L.rows_cap * sizeof(u64), s), "hipMemsetAsync");
  HIPCHK(launch_attempt_init(at<RowCtl>(w, L.ctl), at<SelState>(w, L.sel), at<AttemptRecord>(w, L.rec),
                             at<u32>(w, L.ticket), 1, at<u32>(w, L.rhist), s),
         "launch attempt_init");
  w->dirty = false;
  return PROFK_OK;
}

// Waits until the device has published record number `want` (spinning on the pinned
// host word; a stream that finishes without publishing it is an error, not a hang).
// With early_cap: the filter's word is enough when the check failed or R <= early_cap
// (then no value bin can exceed early_cap keys, so nothing later needs the host);
// *early tells which record was taken.
int wait_record(Workspace* w, hipStream_t s, u32 want, u64 early_cap = 0, bool* early = nullptr) {
  const u32* seq = &w->hrec->seq;
  const u64* ew = &w->hrec->early;
  if (early) *early = false;
  // the filter's early word settles the attempt when the check failed or R is small
  // enough; the scan then publishes no record of its own
  auto take_early = [&]() -> bool {
    if (!early_cap) return false;
    const u64 e = __atomic_load_n(ew, __ATOMIC_ACQUIRE);
    if ((u32)(e >> 42) != (want & 0x3FFFFFu)) return false;
    const u64 R = e & ((1ull << 40) - 1);
    const u32 status = (u32)(e >> 40) & 3u;
    if (status == 0 && R > early_cap) return false;
    w->hrec->R = R;  // the fields the caller reads
    w->hrec->status = status;
    w->hrec->error = 0;
    w->hrec->generic = 0;
    if (early) *early = true;
    return true;
  };
  for (u64 it = 0;; ++it) {
    if (take_early()) return PROFK_OK;
    if (__atomic_load_n(seq, __ATOMIC_ACQUIRE) == want) return PROFK_OK;
    if ((it & 255) == 255) {
      const hipError_t q = hipStreamQuery(s);
      if (q == hipSuccess) {
        // everything has run: one of the two words must be there now (the early word
        // may have landed after the first look above)
        if (take_early()) return PROFK_OK;
        if (__atomic_load_n(seq, __ATOMIC_ACQUIRE) == want) return PROFK_OK;
        t_err = "sampled attempt: the attempt record was not published";
        return PROFK_EINTERNAL;
      }
      if (q != hipErrorNotReady) return hip_fail(q, "hipStreamQuery");
    }
    _mm_pause();
  }
}

// Batched form: waits for the filter's summary word of attempt `want` (every listed
// row passed, or how many failed), spinning on the pinned host word like wait_record.
int wait_summary(Workspace* w, hipStream_t s, u32 want, bool* all_ok) {
  const u64* ew = &w->hrec->early;
  auto take = [&]() -> bool {
    const u64 e = __atomic_load_n(ew, __ATOMIC_ACQUIRE);
    if ((u32)(e >> 42) != (want & 0x3FFFFFu)) return false;
    *all_ok = ((e >> 40) & 3u) == 0;
    return true;
  };
  for (u64 it = 0;; ++it) {
    if (take()) return PROFK_OK;
    if ((it & 255) == 255) {
      const hipError_t q = hipStreamQuery(s);
      if (q == hipSuccess) {
        if (take()) return PROFK_OK;
        t_err = "batched attempt: the filter's summary was not published";
        return PROFK_EINTERNAL;
      }
      if (q != hipErrorNotReady) return hip_fail(q, "hipStreamQuery");
    }
    _mm_pause();
  }
}

SampleArgs sample_args(Workspace* w, const Layout& L, const float* x, u64 N, u64 S, u64 t, u64 seed, u32 attempt) {
  SampleArgs a{};
  a.x = x;
  a.N = N;
  a.S = S;
  a.seed = seed;
  a.attempt = attempt;
  a.row = 0;
  a.table = at<u32>(w, L.hash);
  a.tmask = L.hash_used - 1;
  a.keys = at<u64>(w, L.keys);
  a.tops = at<u64>(w, L.tops);
  a.ctl = at<RowCtl>(w, L.ctl);
  a.rec = nullptr;
  a.ticket = reinterpret_cast<u64*>(at<u32>(w, L.ticket) + kTicketSample);
  a.top_hist = at<SelState>(w, L.sel)->hist;
  a.t = t;
  const SampleShape sh = sample_shape(S, t, N, true);
  a.mode = sh.mode;
  a.threads = sh.threads;
  a.sel = at<SelState>(w, L.sel);
  a.col = at<u64>(w, L.col);
  return a;
}

int validate_args(const float* x, int64_t N, int64_t k, double eps, const void* ov, const void* oi) {
  if (!x || !ov || !oi) return PROFK_EINVAL;
  if (N < 1 || k < 1 || k > N) return PROFK_EINVAL;
  if (!(eps > 0.0 && eps < 1.0)) return PROFK_EINVAL;
  return PROFK_OK;
}

// Rows of fewer than 2^32 values (the 32-bit index inside the keys).
int validate(const float* x, int64_t N, int64_t k, double eps, const void* ov, const void* oi) {
  const int rc = validate_args(x, N, k, eps, ov, oi);
  if (rc) return rc;
  if (N >= (int64_t(1) << 32)) return PROFK_EUNSUPPORTED;
  return PROFK_OK;
}

// Inputs of 2^32 values or more are cut into segments of at most kSegMax values (a
// multiple of 64, so every segment starts on the 16-byte phase of x).
constexpr u64 kSegMax = (1ull << 32) - 64;
constexpr u64 kMaxSegmentedN = kSegMax * kMaxSegments;  // about 2^38 values (1 TiB of fp32)

int max_attempts_of(const profk_options* opt) {
  if (opt && opt->force_fallback) return 0;
  if (opt && opt->use_max_attempts) return opt->max_attempts < 0 ? 0 : opt->max_attempts;
  if (opt && opt->max_attempts > 0) return opt->max_attempts;
  return kDefaultAttempts;
}

// Exact full selection of one row (radix select over all N keys formed on the fly).
int run_exact(Workspace* w, const Layout& L, const float* x, u64 N, u64 k, float* out_vals, int64_t* out_idx,
              hipStream_t s, bool sync = true) {
  RowCtl* ctl = at<RowCtl>(w, L.ctl);
  SelState* sel = at<SelState>(w, L.sel);
  AttemptRecord* rec = at<AttemptRecord>(w, L.rec);
  int rc = clean_if_dirty(w, L, s);
  if (rc) return rc;
  w->dirty = true;
  HIPCHK(launch_attempt_init(ctl, sel, rec, at<u32>(w, L.ticket), 1, at<u32>(w, L.rhist), s), "launch attempt_init");
  HIPCHK(launch_arm_select(sel, k, N, ctl, s), "launch arm_select");
  HIPCHK(launch_select_x(x, N, sel, at<u64>(w, L.col), &ctl->kth, &ctl->status, s), "launch select_x");
  HIPCHK(launch_compact_x(x, N, ctl, at<u64>(w, L.topk0), k, at<u32>(w, L.ticket), s), "launch compact_x");
  HIPCHK(launch_sort_and_write(at<u64>(w, L.topk0), at<u64>(w, L.topk1), at<u32>(w, L.hist), (u32)k, x, N,
                               out_vals, out_idx, ctl, rec, s),
         "launch sort");
  if (!sync) {  // approximate mode: stream-ordered, the consistency check is not read back
    w->dirty = false;
    return PROFK_OK;
  }
  HIPCHK(hipMemcpyAsync(w->host, rec, sizeof(AttemptRecord), hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
  HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
  w->dirty = false;
  if (w->host[0].error || w->host[0].status != 0) {
    t_err = "exact selection: device consistency check failed";
    return PROFK_EINTERNAL;
  }
  return PROFK_OK;
}

RefineArgs refine_args(Workspace* w, const Layout& L, const float* x, u64 N, u64 k, u64 M, float* out_vals,
                       int64_t* out_idx) {
  RefineArgs ra{};
  ra.ctl = at<RowCtl>(w, L.ctl);
  ra.cand = at<u64>(w, L.cand);
  ra.M = M;
  ra.k = k;
  ra.N = N;
  ra.x = x;
  ra.tmp = at<u64>(w, L.rtmp);
  ra.hist = at<u32>(w, L.rhist);
  ra.chunk = at<u32>(w, L.rchunk);
  ra.cursor = at<u32>(w, L.rcursor);
  ra.table = at<u32>(w, L.hash);
  ra.table_slots = L.hash_used;
  ra.out_vals = out_vals;
  ra.out_idx = out_idx;
  ra.pool = at<u64>(w, L.pool);
  ra.ticket = at<u32>(w, L.ticket) + kTicketRefine;
  ra.wait_ticks = kRefineWaitTicks;
  return ra;
}

// Passes long enough for their per-die stream times to size the dies' shares.
constexpr u64 kTimedMinN = 1ull << 24;

FilterArgs flat_filter_args(Workspace* w, const Layout& L, const float* x, u64 N, u64 k, u64 M) {
  FilterArgs fa{};
  fa.x = x;
  fa.ld = N;
  fa.N = N;
  fa.rows = nullptr;
  fa.nrows = 1;
  fa.ctls = at<RowCtl>(w, L.ctl);
  fa.cand = at<u64>(w, L.cand);
  fa.M = M;
  fa.k = k;
  fa.ticket = at<u32>(w, L.ticket) + kTicketFilter;
  fa.groups = at<u32>(w, L.ticket) + kTickets;
  // per-die stream times only where the host updates the die weights from them
  fa.xtime = N >= kTimedMinN ? reinterpret_cast<u64*>(at<u32>(w, L.ticket) + kXtimeWord) : nullptr;
  fa.rec = at<AttemptRecord>(w, L.rec);
  fa.sels = at<SelState>(w, L.sel);
  return fa;
}

// The dies' shares for a filter launch of this weight set (its launch shape).
void set_die_weights(Workspace* w, FilterArgs& fa, u32 set) {
  for (u32 x = 0; x < kXcds; ++x) fa.weight[x] = w->xw[set][x];
}

// Moving average of the dies' streaming speeds from the filter's per-die times of the
// attempt just read back (a performance hint only: the shares never change results).
void update_die_weights(Workspace* w, const u64* split, u32 set) {
  const u64* xt = w->hrec->xt;
  if (xt[0] == 0) return;
  double rate[kXcds], mean = 0.0;
  u32 n = 0;
  for (u32 x = 0; x < kXcds; ++x) {
    const u64 work = split[x + 1] - split[x];
    if (work == 0 || xt[1 + x] <= xt[0]) return;  // a die without work or without a time
    // work on die x was in proportion to (its blocks) x (its weight), so its speed per
    // block is in proportion to weight / time
    rate[x] = (double)w->xw[set][x] / (double)(xt[1 + x] - xt[0]);
    mean += rate[x];
    ++n;
  }
  mean /= n;
  // the first measurement sets the weights (the dies keep their relative speeds from call
  // to call); later ones are averaged in
  const double keep = w->xw_updates[set] == 0 ? 0.0 : 0.5;
  ++w->xw_updates[set];
  for (u32 x = 0; x < kXcds; ++x) {
    double v = keep * (double)w->xw[set][x] + (1.0 - keep) * rate[x] / mean;
    v = v < 0.5 ? 0.5 : (v > 2.0 ? 2.0 : v);
    w->xw[set][x] = (float)v;
  }
  for (u32 x = 0; x < kXcds; ++x) w->hrec->xt[x + 1] = 0;
  w->hrec->xt[0] = 0;
}

// The filter's launch shape by the expected density of hits.  The shape for rare hits
// pays off only while few tiles carry a hit; R varies a lot from draw to draw at small t
// (exponential at t = 1), so that test takes a high draw of R, E[R] + 3 sd(R), not its
// mean.  Dense hits (E[R] >= N / 2048, and N / 256) take more blocks per CU.
u32 filter_shape(const profk_params& p, u64 N) {
  const double hi = p.E_R + 3.0 * std::sqrt(p.Var_R > 0.0 ? p.Var_R : 0.0);
  if (hi * 8192.0 <= (double)N) return kShapeSparse;
  if (p.E_R * 256.0 >= (double)N) return kShapeVeryDenseHits;
  return p.E_R * 2048.0 >= (double)N ? kShapeDenseHits : 0u;
}

// One sampled attempt of one row, enqueued; returns after the record is back.
int run_attempt(Workspace* w, const Layout& L, const float* x, u64 N, u64 k, const profk_params& p, u64 seed,
                u32 attempt, float* out_vals, int64_t* out_idx, hipStream_t s, const profk_options* opt,
                AttemptRecord* out_rec, float* filter_ms) {
  const bool timing = opt && opt->timing;
  RowCtl* ctl = at<RowCtl>(w, L.ctl);
  SelState* sel = at<SelState>(w, L.sel);
  AttemptRecord* rec = at<AttemptRecord>(w, L.rec);
  const u64 S = (u64)p.S, M = (u64)p.M, t = (u64)p.t;
  int rc = clean_if_dirty(w, L, s);
  if (rc) return rc;
  // The sampling kernel resets the attempt's control state; every kernel leaves its
  // tickets, counters and histograms zero, and the refinement clears the hash set.
  w->dirty = true;
  SampleArgs sa = sample_args(w, L, x, N, S, t, seed, attempt);
  sa.rec = rec;
  HIPCHK(launch_sample(sa, s), "launch sample");
  const u32 seq = ++w->seq;
  FilterArgs fa = flat_filter_args(w, L, x, N, k, M);
  fa.hrec = w->hrec_dev;
  fa.seq = seq;
  fa.sparse = filter_shape(p, N);
  set_die_weights(w, fa, fa.sparse);
  u64 split[kXcds + 1];
  if (timing) HIPCHK(hipEventRecord(w->ev0, s), "hipEventRecord");
  HIPCHK(launch_filter(fa, 0, s, split), "launch filter");
  if (timing) HIPCHK(hipEventRecord(w->ev1, s), "hipEventRecord");
  RefineArgs ra = refine_args(w, L, x, N, k, M, out_vals, out_idx);
  ra.hrec = w->hrec_dev;
  ra.seq = seq;
  ra.rec = rec;
  // One-launch refinement (small k): no value bins, so the filter's early word settles
  // the attempt (a bin cap of R <= kMsdCapExact is always met there).  Binned
  // refinement: a needed value bin beyond one workgroup's LDS sort (kBinCap keys: a
  // group of equal values, or a narrow value range) goes to the multi-block radix
  // select, which the host enqueues; so the host always takes the scan's record (the
  // next call is still enqueued while the bin sort runs).  The in-kernel partition of
  // such bins (one workgroup per bin: milliseconds for a 10^5-key tie group) is left to
  // approximate mode, which has no host.
  const bool one = refine_one_launch(ra);
  if (opt && opt->refine_wait_ticks)
    ra.wait_ticks = opt->refine_wait_ticks > 0 ? (u64)opt->refine_wait_ticks : 0ull;  // 0: at once
  ra.msd_cap = one ? kMsdCapExact : kBinCap;
  ra.early_cap = one ? kMsdCapExact : 0;  // the same cap wait_record applies to the early word
  HIPCHK(launch_refine(ra, s), "launch refine");
  // The filter publishes R and the check, the scan the full record.  The refinement
  // launches may still run when this returns (outputs are complete in stream order).
  bool early = false;
  rc = wait_record(w, s, seq, ra.early_cap, &early);
  if (rc) return rc;
  if (N >= kTimedMinN) update_die_weights(w, split, fa.sparse);
  w->host[0].R = w->hrec->R;
  w->host[0].status = w->hrec->status;
  w->host[0].error = w->hrec->error;
  w->host[0].generic = w->hrec->generic;
  if (w->host[0].status == 0 && !w->host[0].error && w->host[0].generic) {
    // a needed bin is too large for one LDS sort (ties, narrow ranges): the
    // multi-pass refinement over the same candidates, then one more read-back
    HIPCHK(launch_select_keys(at<u64>(w, L.cand), &ctl->R, M, sel, at<u64>(w, L.col), &ctl->kth, &ctl->status, s),
           "launch select(candidates)");
    HIPCHK(launch_compact_keys(at<u64>(w, L.cand), &ctl->R, M, ctl, at<u64>(w, L.topk0), k, s), "launch compact");
    HIPCHK(launch_sort_and_write(at<u64>(w, L.topk0), at<u64>(w, L.topk1), at<u32>(w, L.hist), (u32)k, x, N,
                                 out_vals, out_idx, ctl, rec, s),
           "launch sort");
    HIPCHK(hipMemcpyAsync(w->host, rec, sizeof(AttemptRecord), hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
    HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
    w->host[0].generic = 1;
  }
  w->dirty = false;
  *out_rec = w->host[0];
  if (timing && filter_ms) {
    float ms = 0.f;
    // the filter's word can arrive before its launch has completed on the stream
    HIPCHK(hipEventSynchronize(w->ev1), "hipEventSynchronize");
    HIPCHK(hipEventElapsedTime(&ms, w->ev0, w->ev1), "hipEventElapsedTime");
    *filter_ms = ms;
  }
  return PROFK_OK;
}

int topk_row(const float* x, u64 N, u64 k, double eps, u64 seed, float* out_vals, int64_t* out_idx, hipStream_t s,
             const profk_options* opt, profk_stats* st) {
  profk_params p{};
  int rc = solve_memo((int64_t)N, (int64_t)k, eps, opt, &p);
  if (rc) return rc;
  const int max_att = max_attempts_of(opt);
  const bool sampled = !p.direct_exact && max_att > 0;
  Layout L;
  Workspace* w = nullptr;
  rc = get_workspace(s, Need{1, sampled ? (u64)p.S : 0, sampled ? (u64)p.M : 0, k}, &w, &L);
  if (rc) return rc;
  if (st) {
    st->S = p.S;
    st->t = p.t;
    st->M = p.M;
    st->workspace_bytes = w->bytes;
  }
  if (sampled) {
    for (int a = 0; a < max_att; ++a) {
      AttemptRecord r{};
      float fms = 0.f;
      rc = run_attempt(w, L, x, N, k, p, seed, (u32)a, out_vals, out_idx, s, opt, &r, &fms);
      if (rc) return rc;
      if (st) {
        st->attempts = a + 1;
        if (a < PROFK_STATS_ATTEMPTS) {
          st->R[a] = (int64_t)r.R;
          st->fail_mode[a] = (int32_t)r.status;
        }
        st->filter_ms = fms;
        if (r.generic) st->refine_multipass++;
      }
      if (r.error || r.status == 3) {
        t_err = "sampled attempt: device consistency check failed";
        return PROFK_EINTERNAL;
      }
      if (r.status == 0) return PROFK_OK;
    }
  }
  if (st) st->fallback = 1;
  return run_exact(w, L, x, N, k, out_vals, out_idx, s);
}

// Device buffer for the per-segment lists, cached with the (device, stream) workspace.
int get_segment_buffer(hipStream_t s, size_t bytes, char** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> g(g_ws_mu);
  Workspace*& w = g_ws[std::make_pair(dev, s)];
  if (!w) {
    w = new Workspace();
    w->device = dev;
    w->stream = s;
  }
  if (w->seg_bytes < bytes) {
    if (w->seg) {
      HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
      HIPCHK(hipFree(w->seg), "hipFree");
      w->seg = nullptr;
      w->seg_bytes = 0;
    }
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
      (void)hipGetLastError();
      t_err = "segment buffer allocation failed";
      return PROFK_ENOMEM;
    }
    w->seg = (char*)p;
    w->seg_bytes = bytes;
  }
  *out = w->seg;
  return PROFK_OK;
}

// Exact top-k of an input of 2^32 values or more (P1 App. D, Table 4): G contiguous
// segments of fewer than 2^32 values, each an exact top-k of its own (the sampled
// path, budget eps / G, so that a retry anywhere in the call stays within eps), into
// G sorted lists; the global top-k lies in their union and one merge launch takes it.
// The segments together read the input once.
int topk_segmented(const float* x, u64 N, u64 k, double eps, u64 seed, float* out_vals, int64_t* out_idx,
                   hipStream_t s, const profk_options* opt, profk_stats* st) {
  if (N > kMaxSegmentedN) {
    t_err = "input longer than the segmented path supports";
    return PROFK_EUNSUPPORTED;
  }
  const u64 G = (N + kSegMax - 1) / kSegMax;
  const u64 seg = (((N + G - 1) / G) + 63) & ~63ull;  // <= kSegMax; (G - 1) seg < N
  const size_t vbytes = align256(G * k * sizeof(float));
  char* buf = nullptr;
  int rc = get_segment_buffer(s, vbytes + G * k * sizeof(int64_t), &buf);
  if (rc) return rc;
  SegmentLists L{};
  L.vals = reinterpret_cast<float*>(buf);
  L.idx = reinterpret_cast<int64_t*>(buf + vbytes);
  L.stride = k;
  L.k = k;
  L.G = (u32)G;
  for (u64 g = 0; g < G; ++g) {
    const u64 base = g * seg;
    const u64 len = base + seg <= N ? seg : N - base;
    const u64 kg = k < len ? k : len;
    L.len[g] = kg;
    L.base[g] = base;
    profk_stats gs{};
    rc = topk_row(x + base, len, kg, eps / (double)G, seed ^ (0x9E3779B97F4A7C15ull * (g + 1)),
                  const_cast<float*>(L.vals) + g * k, const_cast<int64_t*>(L.idx) + g * k, s, opt,
                  st ? &gs : nullptr);
    if (rc) return rc;
    if (!st) continue;
    if (g == 0) {
      *st = gs;
      continue;
    }
    if (gs.attempts > st->attempts) st->attempts = gs.attempts;
    st->fallback |= gs.fallback;
    st->refine_multipass += gs.refine_multipass;
    st->filter_ms += gs.filter_ms;
    if (gs.workspace_bytes > st->workspace_bytes) st->workspace_bytes = gs.workspace_bytes;
  }
  if (st) st->segments = (int64_t)G;
  HIPCHK(launch_merge_segments(L, out_vals, out_idx, s), "launch merge_segments");
  return PROFK_OK;
}

// Approximate mode: one sampled attempt, everything enqueued on the stream, no host
// read (P1 App. D: omitting the check).  The refinement runs on whatever the buffer
// holds and reports the check's outcome in *info.  Enqueues into the workspace w
// laid out as L (the cached one, or the static scratch of the entry point that
// allocates nothing); allocates nothing itself.
int approx_enqueue(Workspace* w, const Layout& L, const profk_params& p, bool sampled, const float* x, u64 N, u64 k,
                   u64 seed, float* out_vals, int64_t* out_idx, ApproxInfo* info, hipStream_t s) {
  int rc = PROFK_OK;
  if (!sampled) {
    rc = run_exact(w, L, x, N, k, out_vals, out_idx, s, false);
    if (rc) return rc;
    if (info) HIPCHK(launch_approx_info_exact(info, N, s), "launch approx_info");
    return PROFK_OK;
  }
  const u64 S = (u64)p.S, M = (u64)p.M, t = (u64)p.t;
  rc = clean_if_dirty(w, L, s);
  if (rc) return rc;
  w->dirty = true;
  SampleArgs sa = sample_args(w, L, x, N, S, t, seed, 0);
  sa.rec = at<AttemptRecord>(w, L.rec);
  HIPCHK(launch_sample(sa, s), "launch sample");
  FilterArgs fa = flat_filter_args(w, L, x, N, k, M);
  fa.sparse = filter_shape(p, N);
  set_die_weights(w, fa, fa.sparse);
  HIPCHK(launch_filter(fa, 0, s), "launch filter");
  RefineArgs ra = refine_args(w, L, x, N, k, M, out_vals, out_idx);
  ra.msd_cap = 0xFFFFFFFFu;  // no host to hand an oversized bin to
  ra.approx = 1;
  ra.info = info;
  HIPCHK(launch_refine(ra, s), "launch refine");
  w->dirty = false;
  return PROFK_OK;
}

int topk_approx_row(const float* x, u64 N, u64 k, double eps, u64 seed, float* out_vals, int64_t* out_idx,
                    ApproxInfo* info, hipStream_t s, const profk_options* opt) {
  profk_params p{};
  int rc = solve_memo((int64_t)N, (int64_t)k, eps, opt, &p);
  if (rc) return rc;
  const bool sampled = !p.direct_exact && !(opt && opt->force_fallback);
  Layout L;
  Workspace* w = nullptr;
  rc = get_workspace(s, Need{1, sampled ? (u64)p.S : 0, sampled ? (u64)p.M : 0, k}, &w, &L);
  if (rc) return rc;
  return approx_enqueue(w, L, p, sampled, x, N, k, seed, out_vals, out_idx, info, s);
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing (profk_topk_approx_noalloc).  Its workspace is
// the static device array `scratch` below: every GPU the library runs on holds its own
// copy for the life of the process.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the device symbol): the device
// address is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept in g_scratch_ptr.
constexpr size_t kStaticScratchBytes = (size_t)PROFK_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

}  // namespace
}  // namespace profk

static __device__ __align__(256) unsigned char scratch[profk::kStaticScratchBytes];

namespace profk {
namespace {

// Device address of this device's copy of `scratch` (looked up on the first call on the
// device).  No allocation: the array exists since the library's code object was loaded.
int static_scratch(char** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    t_err = "device index beyond the static scratch table";
    return PROFK_EINVAL;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HIPCHK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!ptr) {
      t_err = "hipGetSymbolAddress(scratch) returned a null address";
      return PROFK_EHIP;
    }
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return PROFK_OK;
}

// profk_topk_approx on the static scratch.  The array keeps whatever the last call on
// this GPU left in it, so the regions the kernels expect zero (hash set, tickets,
// control blocks, histograms) are cleared first, by kernels (no memset node, so that
// the call stays capturable in a HIP graph).  Calls that overlap in time on one GPU
// share the array and race.
int topk_approx_static(const float* x, u64 N, u64 k, double eps, u64 seed, float* out_vals, int64_t* out_idx,
                       ApproxInfo* info, hipStream_t s, const profk_options* opt) {
  profk_params p{};
  int rc = solve_memo((int64_t)N, (int64_t)k, eps, opt, &p);
  if (rc) return rc;
  const bool sampled = !p.direct_exact && !(opt && opt->force_fallback);
  const Layout L = make_layout(1, sampled ? (u64)p.S : 0, sampled ? (u64)p.M : 0, k, 0, 0, 0);
  if (L.total > kStaticScratchBytes) {
    t_err = "the call needs " + std::to_string(L.total) + " bytes of workspace; the static scratch holds " +
            std::to_string(kStaticScratchBytes);
    return PROFK_ESCRATCH;
  }
  char* base = nullptr;
  rc = static_scratch(&base);
  if (rc) return rc;
  Workspace w;  // a view of the static array; nothing in it is allocated
  w.stream = s;
  w.dev = base;
  w.bytes = kStaticScratchBytes;
  w.hash_cap = L.hash_slots;
  w.rows_cap = L.rows_cap;
  HIPCHK(launch_clear_sample(at<u32>(&w, L.hash), L.hash_slots, at<u32>(&w, L.ticket), s), "launch clear_sample");
  HIPCHK(launch_attempt_init(at<RowCtl>(&w, L.ctl), at<SelState>(&w, L.sel), at<AttemptRecord>(&w, L.rec),
                             at<u32>(&w, L.ticket), 1, at<u32>(&w, L.rhist), s),
         "launch attempt_init");
  return approx_enqueue(&w, L, p, sampled, x, N, k, seed, out_vals, out_idx, info, s);
}

// Which sampler the batched form takes for rows of N values: the per-row workgroup
// with an LDS bitmap of the row (rows of at most kBatchedMaxN values), or the grid of
// one-draw-per-thread blocks per row with a hash set per row in device memory (any
// row length).
bool batched_grid_sampler(u64 N) { return N > kBatchedMaxN; }

// Batched form with per-row kernels (k at most kBatchedMaxM: the refinement holds a
// row's buffer in LDS up to kBatchedMaxM keys, and beyond that selects over it in
// global memory and sorts the k in LDS).  Returns PROFK_EUNSUPPORTED when the shape is
// outside those limits, so that the caller takes the row-by-row path.  With info
// (approximate mode): one attempt per row, everything enqueued on the stream, no host
// wait, each row's check reported in info[row].
int topk_batched_rows(const float* x, u64 B, u64 N, u64 ld, u64 k, double eps, u64 seed, float* out_vals,
                      int64_t* out_idx, hipStream_t s, const profk_options* opt, profk_stats* st,
                      ApproxInfo* info = nullptr) {
  const bool approx = info != nullptr;
  if (B >= (1ull << 31)) return PROFK_EUNSUPPORTED;
  profk_params p{};
  if (N > kSmallSort) {
    const int rc = solve_memo((int64_t)N, (int64_t)k, eps / (double)B, opt, &p);  // P1 App. E.2: eps / B per row
    if (rc) return rc;
  }
  const bool whole = N <= kSmallSort || (N <= kBatchedMaxM && (p.direct_exact || (opt && opt->force_fallback)));
  if (whole) {
    // rows this short, or short rows where the sample would not pay off: exact top-k by
    // an LDS sort of each row
    Layout L;
    Workspace* w = nullptr;
    int rc = get_workspace(s, Need{B, 0, 0, 1}, &w, &L);
    if (rc) return rc;
    BatchedArgs a{};
    a.x = x;
    a.ld = ld;
    a.N = N;
    a.nrows = B;
    a.k = k;
    a.out_vals = out_vals;
    a.out_idx = out_idx;
    HIPCHK(launch_b_rowsort(a, s), "launch b_rowsort");
    if (approx) {
      HIPCHK(launch_b_info_exact(info, B, N, s), "launch b_info_exact");
      return PROFK_OK;
    }
    HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
    if (st) {
      st->fallback = 1;
      st->rows_fallback = (int64_t)B;
    }
    return PROFK_OK;
  }
  int rc = PROFK_OK;
  if (!p.direct_exact && p.M > (int64_t)kBatchedMaxM && k <= kBatchedSelCap && !(opt && opt->s_override)) {
    // A row buffer beyond the refinement's LDS (kBatchedMaxM keys) is selected over in
    // global memory by one workgroup, several times slower than the LDS select that
    // k <= kBatchedSelCap takes; a larger sample shrinks M (about N t / S), so double S
    // while that stays within N/64 and 2^17 (S changes the work of a call, never its
    // result).  Larger k sort the whole buffer when it fits LDS, which costs more than
    // the select over global memory, and keep the rule's S.
    profk_options o{};
    if (opt) o = *opt;
    for (int64_t S2 = 2 * p.S; S2 <= (int64_t)(N / 64) && S2 <= (int64_t)(1 << 17); S2 *= 2) {
      o.s_override = S2;
      profk_params q{};
      rc = solve_memo((int64_t)N, (int64_t)k, eps / (double)B, &o, &q);
      if (rc) return rc;
      if (q.direct_exact) break;
      p = q;
      if (q.M <= (int64_t)kBatchedMaxM) break;
    }
  }
  const int max_att = approx ? 1 : max_attempts_of(opt);
  const bool grid = batched_grid_sampler(N);
  if (p.direct_exact || max_att == 0 || (opt && opt->force_fallback) || k > kBatchedMaxM ||
      (!grid && (N > kBatchedMaxN || (u64)p.S > kBatchedMaxN / 8)))
    return PROFK_EUNSUPPORTED;
  const u64 S = (u64)p.S, M = (u64)p.M, t = (u64)p.t;
  const u64 G = batched_sample_blocks(B);
  // the grid sampler's per-row block lists (each row's tau in its own last block)
  const SampleShape sh = sample_shape(S, t, N, false);
  const u64 tops_per_row = sh.tops_words;
  Layout L;
  Workspace* w = nullptr;
  rc = grid ? get_workspace(s, Need{B, S, M, 1, 0, B, tops_per_row}, &w, &L)
            : get_workspace(s, Need{B, 0, M, 1, G * 2 * S}, &w, &L);  // per sampling workgroup: S slots + top-up
  if (rc) return rc;
  RowCtl* ctl = at<RowCtl>(w, L.ctl);
  SelState* sel = at<SelState>(w, L.sel);
  AttemptRecord* rec = at<AttemptRecord>(w, L.rec);
  int* rows_dev = at<int>(w, L.rows);
  if (st) {
    st->S = p.S;
    st->t = p.t;
    st->M = p.M;
    st->workspace_bytes = w->bytes;
  }
  rc = clean_if_dirty(w, L, s);
  if (rc) return rc;
  w->dirty = true;
  // control blocks, records and (grid sampler) the rows' top-digit histograms; the
  // pipelined sampler sets up every row it samples, and the first attempt samples all
  const bool pipelined = !grid && b_sample_pipelined(S, t, N);
  if (!pipelined)
    HIPCHK(launch_attempt_init(ctl, grid ? sel : nullptr, rec, at<u32>(w, L.ticket), (u32)B, nullptr, s),
           "launch attempt_init");
  const int* rows = nullptr;  // all rows on the first attempt
  u64 nrows = B;
  std::vector<int> failed;
  for (int att = 0; att < max_att && nrows > 0; ++att) {
    BatchedArgs a{};
    a.x = x;
    a.ld = ld;
    a.N = N;
    a.rows = rows;
    a.nrows = nrows;
    a.S = S;
    a.t = t;
    a.seed = seed;
    a.attempt = (u32)att;
    a.ctls = ctl;
    a.scratch = at<u64>(w, L.scratch);
    a.cand = at<u64>(w, L.cand);
    a.M = M;
    a.k = k;
    a.out_vals = out_vals;
    a.out_idx = out_idx;
    a.rec = rec;
    a.approx = approx ? 1u : 0u;
    a.info = info;
    a.tickets = pipelined && att == 0 ? at<u32>(w, L.ticket) : nullptr;
    if (grid) {
      // one grid row of sampling blocks per listed row (at most 65535 per launch)
      a.table = at<u32>(w, L.hash);
      a.table_slots = L.hash_used;
      for (u64 l0 = 0; l0 < nrows; l0 += 65535) {
        SampleArgs sa{};
        sa.x = x;
        sa.N = N;
        sa.S = S;
        sa.seed = seed;
        sa.attempt = (u32)att;
        sa.table = at<u32>(w, L.hash) + l0 * L.hash_used;
        sa.tmask = L.hash_used - 1;
        sa.keys = at<u64>(w, L.keys) + l0 * 2 * S;
        sa.tops = at<u64>(w, L.btops) + l0 * tops_per_row;
        sa.ctl = ctl;
        sa.rec = rec;
        sa.ticket = at<u64>(w, L.rtick) + l0;
        sa.top_hist = sel->hist;
        sa.t = t;
        sa.mode = sh.mode;
        sa.threads = sh.threads;
        sa.rows = rows ? rows + l0 : nullptr;
        sa.nrows = (u32)(nrows - l0 < 65535 ? nrows - l0 : 65535);
        sa.row0 = (u32)l0;
        sa.ld = ld;
        sa.table_stride = L.hash_used;
        sa.keys_stride = 2 * S;
        sa.tops_stride = tops_per_row;
        sa.ticket_stride = 1;
        sa.hist_stride = sizeof(SelState) / sizeof(u32);
        HIPCHK(launch_sample(sa, s), "launch sample (batched)");
      }
    } else {
      HIPCHK(launch_b_sample(a, s), "launch b_sample");
    }
    FilterArgs fa{};
    fa.x = x;
    fa.ld = ld;
    fa.N = N;
    fa.rows = rows;
    fa.nrows = nrows;
    fa.ctls = ctl;
    fa.cand = a.cand;
    fa.M = M;
    fa.k = k;
    fa.ticket = at<u32>(w, L.ticket) + kTicketFilter;
    fa.groups = at<u32>(w, L.ticket) + kTickets;
    fa.rec = rec;
    fa.sels = nullptr;
    fa.sparse = filter_shape(p, N);
    set_die_weights(w, fa, fa.sparse);
    fa.hits_per_row = p.E_R;
    // exact mode without statistics: the filter's last block publishes whether every
    // listed row passed into pinned host memory, and when they all did the call returns
    // on that word while the refinement still runs (outputs complete in stream order)
    const bool summary = !approx && !st;
    u32 seq = 0;
    if (summary) {
      seq = ++w->seq;
      fa.hrec = w->hrec_dev;
      fa.seq = seq;
      fa.summary = 1;
    }
    // the per-die stream times go back with the summary word, as in the flat path: the
    // dies' shares of a long multi-row pass matter as much (1024 x 2^20 at k = 64: about
    // 20 us per call between equal and learned shares)
    const bool timed = summary && N * nrows >= kTimedMinN;
    fa.xtime = timed ? reinterpret_cast<u64*>(at<u32>(w, L.ticket) + kXtimeWord) : nullptr;
    u64 split[kXcds + 1];
    HIPCHK(launch_filter(fa, 0, s, split), "launch filter");
    HIPCHK(launch_b_refine(a, s), "launch b_refine");
    if (approx) break;
    if (summary) {
      bool all_ok = false;
      rc = wait_summary(w, s, seq, &all_ok);
      if (rc) return rc;
      if (timed) update_die_weights(w, split, fa.sparse);
      if (all_ok) {
        nrows = 0;
        break;
      }
    }
    HIPCHK(hipMemcpyAsync(w->host, rec, B * sizeof(AttemptRecord), hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
    HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
    failed.clear();
    for (u64 li = 0; li < nrows; ++li) {
      const int r = rows ? w->host_rows[li] : (int)li;
      const AttemptRecord& rr = w->host[r];
      if (rr.status == 3 || rr.error) {
        t_err = "batched attempt: device consistency check failed";
        return PROFK_EINTERNAL;
      }
      if (rr.status != 0) failed.push_back(r);
    }
    if (st) {
      st->attempts = att + 1;
      if (att < PROFK_STATS_ATTEMPTS) {
        st->R[att] = (int64_t)w->host[rows ? w->host_rows[0] : 0].R;
        st->fail_mode[att] = (int32_t)w->host[rows ? w->host_rows[0] : 0].status;
      }
      if (att == 1) st->rows_retried = (int64_t)nrows;
    }
    nrows = failed.size();
    if (nrows) {
      std::memcpy(w->host_rows, failed.data(), nrows * sizeof(int));
      HIPCHK(hipMemcpyAsync(rows_dev, w->host_rows, nrows * sizeof(int), hipMemcpyHostToDevice, s), "hipMemcpyAsync");
      rows = rows_dev;
    }
  }
  w->dirty = false;
  if (approx || nrows == 0) return PROFK_OK;
  // rows that failed every attempt: exact full selection, row by row
  std::vector<int> rest(failed);
  if (st) st->rows_fallback = (int64_t)rest.size();
  profk_options o{};
  if (opt) o = *opt;
  o.force_fallback = 1;
  for (int r : rest) {
    rc = topk_row(x + (u64)r * ld, N, k, eps / (double)B, seed, out_vals + (u64)r * k, out_idx + (u64)r * k, s, &o,
                  nullptr);
    if (rc) return rc;
  }
  return PROFK_OK;
}

}  // namespace
}  // namespace profk

using namespace profk;

extern "C" {

int profk_solve(int64_t N, int64_t k, double eps, const profk_options* opt, profk_params* out) {
  return solve_memo(N, k, eps, opt, out);
}

int profk_topk_ex(const float* x, int64_t N, int64_t k, double eps, uint64_t seed, float* out_vals,
                  int64_t* out_idx, void* stream, const profk_options* opt, profk_stats* st) {
  int rc = validate_args(x, N, k, eps, out_vals, out_idx);
  if (rc) return rc;
  if (st) std::memset(st, 0, sizeof(*st));
  if (N >= (int64_t(1) << 32))
    return topk_segmented(x, (u64)N, (u64)k, eps, seed, out_vals, out_idx, (hipStream_t)stream, opt, st);
  return topk_row(x, (u64)N, (u64)k, eps, seed, out_vals, out_idx, (hipStream_t)stream, opt, st);
}

int profk_topk_approx(const float* x, int64_t N, int64_t k, double eps, uint64_t seed, float* out_vals,
                      int64_t* out_idx, profk_approx_info* info, void* stream, const profk_options* opt) {
  int rc = validate(x, N, k, eps, out_vals, out_idx);
  if (rc) return rc;
  return topk_approx_row(x, (u64)N, (u64)k, eps, seed, out_vals, out_idx, info, (hipStream_t)stream, opt);
}

int profk_topk_approx_noalloc(const float* x, int64_t N, int64_t k, double eps, uint64_t seed, float* out_vals,
                              int64_t* out_idx, profk_approx_info* info, void* stream, const profk_options* opt) {
  int rc = validate(x, N, k, eps, out_vals, out_idx);
  if (rc) return rc;
  return topk_approx_static(x, (u64)N, (u64)k, eps, seed, out_vals, out_idx, info, (hipStream_t)stream, opt);
}

int profk_topk(const float* x, int64_t N, int64_t k, double eps, uint64_t seed, float* out_vals, int64_t* out_idx,
               void* stream) {
  return profk_topk_ex(x, N, k, eps, seed, out_vals, out_idx, stream, nullptr, nullptr);
}

int profk_topk_batched_ex(const float* x, int64_t B, int64_t N, int64_t ld_x, int64_t k, double eps, uint64_t seed,
                          float* out_vals, int64_t* out_idx, void* stream, const profk_options* opt,
                          profk_stats* st) {
  int rc = validate(x, N, k, eps, out_vals, out_idx);
  if (rc) return rc;
  if (B < 1 || ld_x < N) return PROFK_EINVAL;
  if (st) std::memset(st, 0, sizeof(*st));
  rc = topk_batched_rows(x, (u64)B, (u64)N, (u64)ld_x, (u64)k, eps, seed, out_vals, out_idx, (hipStream_t)stream, opt,
                         st);
  if (rc != PROFK_EUNSUPPORTED) return rc;
  if (st) std::memset(st, 0, sizeof(*st));
  const double eps_row = eps / (double)B;  // P1 App. E.2: budget split per row
  for (int64_t r = 0; r < B; ++r) {
    profk_stats rs{};
    rc = topk_row(x + r * ld_x, (u64)N, (u64)k, eps_row, seed, out_vals + r * k, out_idx + r * k,
                  (hipStream_t)stream, opt, &rs);
    if (rc) return rc;
    if (st) {
      if (r == 0) *st = rs;
      if (rs.attempts > 1) st->rows_retried++;
      if (rs.fallback) st->rows_fallback++;
      if (rs.attempts > st->attempts) st->attempts = rs.attempts;
    }
  }
  return PROFK_OK;
}

int profk_topk_batched_approx(const float* x, int64_t B, int64_t N, int64_t ld_x, int64_t k, double eps,
                              uint64_t seed, float* out_vals, int64_t* out_idx, profk_approx_info* info, void* stream,
                              const profk_options* opt) {
  int rc = validate(x, N, k, eps, out_vals, out_idx);
  if (rc) return rc;
  if (B < 1 || ld_x < N || !info) return PROFK_EINVAL;
  rc = topk_batched_rows(x, (u64)B, (u64)N, (u64)ld_x, (u64)k, eps, seed, out_vals, out_idx, (hipStream_t)stream, opt,
                         nullptr, info);
  if (rc != PROFK_EUNSUPPORTED) return rc;
  // shapes outside the batched kernels: the flat approximate call row by row (budget
  // eps / B each), all stream-ordered
  const double eps_row = eps / (double)B;
  for (int64_t r = 0; r < B; ++r) {
    rc = topk_approx_row(x + r * ld_x, (u64)N, (u64)k, eps_row, seed, out_vals + r * k, out_idx + r * k, info + r,
                         (hipStream_t)stream, opt);
    if (rc) return rc;
  }
  return PROFK_OK;
}

int profk_topk_batched(const float* x, int64_t B, int64_t N, int64_t ld_x, int64_t k, double eps, uint64_t seed,
                       float* out_vals, int64_t* out_idx, void* stream) {
  return profk_topk_batched_ex(x, B, N, ld_x, k, eps, seed, out_vals, out_idx, stream, nullptr, nullptr);
}

int profk_stage_sample(const float* x, int64_t N, int64_t S, uint64_t seed, int32_t attempt, int64_t* out_idx,
                       void* stream) {
  if (!x || !out_idx || N < 2 || S < 1 || 2 * S > N || attempt < 0) return PROFK_EINVAL;
  if (N >= (int64_t(1) << 32)) return PROFK_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  Layout L;
  Workspace* w = nullptr;
  int rc = get_workspace(s, Need{1, (u64)S, 1, 1}, &w, &L);
  if (rc) return rc;
  rc = clean_if_dirty(w, L, s);
  if (rc) return rc;
  w->dirty = true;
  RowCtl* ctl = at<RowCtl>(w, L.ctl);
  u32* tickets = at<u32>(w, L.ticket);
  HIPCHK(launch_sample(sample_args(w, L, x, (u64)N, (u64)S, 0, seed, (u32)attempt), s), "launch sample");
  HIPCHK(launch_keys_to_index_compact(at<u64>(w, L.keys), &ctl->D, 2 * (u64)S, out_idx, tickets + kCountStage, s),
         "launch keys_to_index");
  HIPCHK(launch_clear_sample(at<u32>(w, L.hash), L.hash_used, tickets, s), "launch clear_sample");
  u32 status = 0;
  HIPCHK(hipMemcpyAsync(&status, &ctl->status, sizeof(u32), hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
  HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
  w->dirty = false;
  if (status != 0) {
    t_err = "sample: device consistency check failed";
    return PROFK_EINTERNAL;
  }
  return PROFK_OK;
}

int profk_stage_threshold(const float* x, int64_t N, int64_t S, int64_t t, uint64_t seed, int32_t attempt,
                          float* out_tau_val, int64_t* out_tau_idx, void* stream) {
  if (!x || !out_tau_val || !out_tau_idx || N < 2 || S < 1 || 2 * S > N || t < 1 || t > S || attempt < 0)
    return PROFK_EINVAL;
  if (N >= (int64_t(1) << 32)) return PROFK_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  Layout L;
  Workspace* w = nullptr;
  int rc = get_workspace(s, Need{1, (u64)S, 1, 1}, &w, &L);
  if (rc) return rc;
  rc = clean_if_dirty(w, L, s);
  if (rc) return rc;
  w->dirty = true;
  RowCtl* ctl = at<RowCtl>(w, L.ctl);
  HIPCHK(launch_sample(sample_args(w, L, x, (u64)N, (u64)S, (u64)t, seed, (u32)attempt), s), "launch sample");
  HIPCHK(launch_tau_to_output(x, (u64)N, ctl, out_tau_val, out_tau_idx, s), "launch tau_to_output");
  HIPCHK(launch_clear_sample(at<u32>(w, L.hash), L.hash_used, at<u32>(w, L.ticket), s), "launch clear_sample");
  u32 status = 0;
  HIPCHK(hipMemcpyAsync(&status, &ctl->status, sizeof(u32), hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
  HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
  w->dirty = false;
  if (status != 0) {
    t_err = "threshold: device consistency check failed";
    return PROFK_EINTERNAL;
  }
  return PROFK_OK;
}

int profk_stage_batched_sample(const float* x, int64_t B, int64_t N, int64_t ld_x, int64_t S, int64_t t,
                               uint64_t seed, int32_t attempt, int64_t* out_idx, float* out_tau_val,
                               int64_t* out_tau_idx, void* stream) {
  if (!x || !out_idx || !out_tau_val || !out_tau_idx || B < 1 || N < 2 || ld_x < N || S < 1 || 2 * S > N || t < 1 ||
      t > S || attempt < 0)
    return PROFK_EINVAL;
  const bool grid = batched_grid_sampler((u64)N);
  if (B >= (int64_t(1) << 31) || B > 65535 || (!grid && ((u64)N > kBatchedMaxN || (u64)S > kBatchedMaxN / 8)))
    return PROFK_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  Layout L;
  Workspace* w = nullptr;
  const u64 nb = (u64)B, uS = (u64)S, ut = (u64)t;
  const SampleShape sh = sample_shape(uS, ut, (u64)N, false);
  const u64 tops_per_row = sh.tops_words;
  int rc = grid ? get_workspace(s, Need{nb, uS, 1, 1, 0, nb, tops_per_row}, &w, &L)
                : get_workspace(s, Need{nb, 0, 1, 1, nb * 2 * uS}, &w, &L);
  if (rc) return rc;
  rc = clean_if_dirty(w, L, s);
  if (rc) return rc;
  w->dirty = true;
  RowCtl* ctl = at<RowCtl>(w, L.ctl);
  SelState* sel = at<SelState>(w, L.sel);
  AttemptRecord* rec = at<AttemptRecord>(w, L.rec);
  // row r's 2S key slots (a slice of the per-workgroup scratch, or of the grid
  // sampler's key region) start at zero, so that the nonzero ones are its sample
  u64* keys = grid ? at<u64>(w, L.keys) : at<u64>(w, L.scratch);
  HIPCHK(launch_attempt_init(ctl, grid ? sel : nullptr, rec, at<u32>(w, L.ticket), (u32)nb, nullptr, s),
         "launch attempt_init");
  HIPCHK(launch_clear_sample(reinterpret_cast<u32*>(keys), nb * 4 * uS, at<u32>(w, L.ticket), s), "launch clear keys");
  if (grid) {
    SampleArgs sa{};
    sa.x = x;
    sa.N = (u64)N;
    sa.S = uS;
    sa.seed = seed;
    sa.attempt = (u32)attempt;
    sa.table = at<u32>(w, L.hash);
    sa.tmask = L.hash_used - 1;
    sa.keys = keys;
    sa.tops = at<u64>(w, L.btops);
    sa.ctl = ctl;
    sa.rec = rec;
    sa.ticket = at<u64>(w, L.rtick);
    sa.top_hist = sel->hist;
    sa.t = ut;
    sa.mode = sh.mode;
    sa.threads = sh.threads;
    sa.rows = nullptr;
    sa.nrows = (u32)nb;
    sa.row0 = 0;
    sa.ld = (u64)ld_x;
    sa.table_stride = L.hash_used;
    sa.keys_stride = 2 * uS;
    sa.tops_stride = tops_per_row;
    sa.ticket_stride = 1;
    sa.hist_stride = sizeof(SelState) / sizeof(u32);
    HIPCHK(launch_sample(sa, s), "launch sample (batched)");
  } else {
    BatchedArgs a{};
    a.x = x;
    a.ld = (u64)ld_x;
    a.N = (u64)N;
    a.rows = nullptr;
    a.nrows = nb;
    a.S = uS;
    a.t = ut;
    a.seed = seed;
    a.attempt = (u32)attempt;
    a.ctls = ctl;
    a.scratch = keys;
    a.keep_keys = 1;
    HIPCHK(launch_b_sample(a, s, (u32)nb), "launch b_sample");
  }
  HIPCHK(launch_b_stage_out(x, (u64)ld_x, (u64)N, nb, uS, keys, ctl, out_idx, out_tau_val, out_tau_idx, rec, s),
         "launch b_stage_out");
  if (grid)  // the per-row hash sets back to zero (the refinement does this in a call)
    HIPCHK(launch_clear_sample(at<u32>(w, L.hash), nb * L.hash_used, at<u32>(w, L.ticket), s), "launch clear hash");
  HIPCHK(hipMemcpyAsync(w->host, rec, nb * sizeof(AttemptRecord), hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
  HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
  w->dirty = false;
  for (u64 r = 0; r < nb; ++r)
    if (w->host[r].status != 0) {
      t_err = "batched sample: device consistency check failed in row " + std::to_string(r);
      return PROFK_EINTERNAL;
    }
  return PROFK_OK;
}

int profk_stage_filter(const float* x, int64_t N, float tau_val, int64_t tau_idx, int64_t M, int64_t* out_cand_idx,
                       int64_t* out_R, void* stream) {
  if (!x || !out_cand_idx || !out_R || N < 1 || M < 1 || tau_idx < 0 || tau_idx >= N) return PROFK_EINVAL;
  if (N >= (int64_t(1) << 32)) return PROFK_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  Layout L;
  Workspace* w = nullptr;
  int rc = get_workspace(s, Need{1, 1, (u64)M, 1}, &w, &L);
  if (rc) return rc;
  rc = clean_if_dirty(w, L, s);
  if (rc) return rc;
  w->dirty = true;
  RowCtl* ctl = at<RowCtl>(w, L.ctl);
  u32 bits;
  std::memcpy(&bits, &tau_val, sizeof(bits));
  HIPCHK(launch_set_tau(ctl, at<u32>(w, L.ticket), bits, (u32)tau_idx, s), "launch set_tau");
  FilterArgs fa{};
  fa.x = x;
  fa.ld = (u64)N;
  fa.N = (u64)N;
  fa.nrows = 1;
  fa.ctls = ctl;
  fa.cand = at<u64>(w, L.cand);
  fa.M = (u64)M;
  fa.k = 1;
  fa.ticket = at<u32>(w, L.ticket) + kTicketFilter;
  fa.groups = at<u32>(w, L.ticket) + kTickets;
  set_die_weights(w, fa, 0);
  fa.rec = nullptr;
  fa.sels = nullptr;
  HIPCHK(launch_filter(fa, 0, s), "launch filter");
  HIPCHK(launch_keys_to_index(at<u64>(w, L.cand), &ctl->R, (u64)M, out_cand_idx, s), "launch keys_to_index");
  HIPCHK(launch_r_to_output(ctl, out_R, s), "launch r_to_output");
  HIPCHK(hipStreamSynchronize(s), "hipStreamSynchronize");
  w->dirty = false;
  return PROFK_OK;
}

int profk_read_ceiling(const float* x, int64_t N, int32_t blocks_per_cu, uint64_t* out_fold, void* stream) {
  if (!x || !out_fold || N < 1 || blocks_per_cu < 0 || blocks_per_cu > 16) return PROFK_EINVAL;
  if ((uintptr_t)x & 15u) return PROFK_EINVAL;
  HIPCHK(launch_read_ceiling(x, (u64)N, (u32)blocks_per_cu, reinterpret_cast<unsigned long long*>(out_fold),
                             (hipStream_t)stream),
         "launch read_ceiling");
  return PROFK_OK;
}

const char* profk_strerror(int code) {
  switch (code) {
    case PROFK_OK:
      return "ok";
    case PROFK_EINVAL:
      return "invalid argument";
    case PROFK_EUNSUPPORTED:
      return "unsupported size (N >= 2^32 outside profk_topk / profk_topk_ex, or beyond their limit)";
    case PROFK_ENOMEM:
      return "device workspace allocation failed";
    case PROFK_EHIP:
      return t_err.empty() ? "HIP runtime error" : t_err.c_str();
    case PROFK_EINTERNAL:
      return t_err.empty() ? "device consistency check failed" : t_err.c_str();
    case PROFK_ESCRATCH:
      return t_err.empty() ? "the call needs more workspace than the static scratch holds" : t_err.c_str();
    default:
      return "unknown status";
  }
}

void profk_release(void) {
  std::lock_guard<std::mutex> g(g_ws_mu);
  for (auto& kv : g_ws) {
    Workspace* w = kv.second;
    if (!w) continue;
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(w->device);
    if (w->dev) {
      (void)hipStreamSynchronize(w->stream);
      (void)hipFree(w->dev);
    }
    if (w->host) (void)hipHostFree(w->host);
    if (w->host_rows) (void)hipHostFree(w->host_rows);
    if (w->hrec) (void)hipHostFree(w->hrec);
    if (w->seg) {
      (void)hipStreamSynchronize(w->stream);
      (void)hipFree(w->seg);
    }
    if (w->ev0) (void)hipEventDestroy(w->ev0);
    if (w->ev1) (void)hipEventDestroy(w->ev1);
    (void)hipSetDevice(cur);
    delete w;
  }
  g_ws.clear();
}

}  // extern "C"
