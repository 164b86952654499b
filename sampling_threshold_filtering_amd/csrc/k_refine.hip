// Stage 4 of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
// Selection", §3 stage 4): the exact top-k of the R buffered candidates, sorted.
// The pages call a library top-k here (App. C).  For k <= kSmallK one launch does it
// (refine_small_kernel, below: per-workgroup top-k lists and a select over their union
// by the last workgroup).  Larger k take a binned refinement for gfx950:
//
//   refine_hist_kernel     histogram of the candidates over kBins equal bins of the
//                          key range [tau, cmax] (cmax = the largest candidate key,
//                          tracked by the filter), added into a global histogram.
//   refine_scatter_kernel  every block scans the global histogram from the top bin
//                          down in LDS: the bin b* that holds the k-th largest
//                          candidate and the output offset of every bin >= b*.  If one
//                          of those bins holds more keys than one workgroup sorts in
//                          LDS (ties, narrow-range inputs), the row is marked for the
//                          multi-pass refinement instead.  Otherwise each block writes
//                          its candidates of bins >= b* into bin order: one global
//                          atomic per (block, bin) reserves the run, LDS atomics place
//                          the keys.  Block 0 also publishes the attempt record (R,
//                          check, multi-pass flag) to the host, which needs nothing
//                          later to decide, and the bin sort's chunk boundaries.
//   refine_bin_kernel      exact mode: the two above in one launch (the histogram's
//                          atomics return each block's run start in its bins; one
//                          launch-wide wait between counting and placing).
//   refine_binsort_kernel  sorts every bin >= b* (256-thread workgroups, at least four
//                          per CU; each wavefront the bins that start in its equal
//                          share of the output positions, in registers up to kWaveMax
//                          keys, a workgroup a bin up to kBinCap by one 8-bit counting
//                          pass in LDS) and writes out_vals / out_idx for positions
//                          < k.  A larger bin (large tie groups, narrow ranges) is
//                          partitioned by one workgroup on successive 12-bit digits of
//                          (key - tau), from the top down, until every part that
//                          reaches a position below k fits those sorts.  It also
//                          leaves the histogram and the sampler's hash set zero for
//                          the next attempt.
// Bins larger than RefineArgs::msd_cap are instead left to the multi-pass refinement,
// which the host enqueues after reading the flag (exact mode only).
// Bins partition the keys by value, so sorted bins laid out from the top bin down
// are the sorted candidates; positions < k are the exact top-k in order.
#include "block_select.h"
#include "launch.h"

namespace profk {

namespace {
constexpr u32 kHistThreads = 1024;
constexpr u32 kSortThreads = 256;
constexpr u32 kPer = kBins / kHistThreads;  // bins per thread in the scan

// LDS position of descending bin position q: one spare word per kPer, so that the
// kPer consecutive positions of each thread fall in distinct banks across a wave.
__device__ __forceinline__ u32 pad_q(u32 q) { return q + q / kPer; }

__device__ __forceinline__ u32 bin_of(u64 key, u64 tau, u32 shift) {
  const u64 b = (key - tau) >> shift;
  return b < kBins ? (u32)b : kBins - 1u;
}

__device__ __forceinline__ u32 bin_shift_of(const RowCtl* c) {
  const u64 range = c->cmax - c->tau;
  return range < kBins ? 0u : (u32)(64 - __clzll((long long)range)) - kBinBits;
}

__device__ __forceinline__ u64 cand_count(const RowCtl* c, u64 M) { return c->R < M ? c->R : M; }

// The refinement runs when the check passed, and in approximate mode also when it
// failed (it then refines whatever the buffer holds).
__device__ __forceinline__ bool refine_live(const RefineArgs& a, const RowCtl* c) {
  return c->status == 0 || (a.approx && (c->status == 1u || c->status == 2u));
}

// Attempt record into pinned host memory; seq last, released at system scope.  Skipped
// where the host already has what it needs from the filter's early word.
__device__ __forceinline__ void publish(const RefineArgs& a, const RowCtl* c, u32 generic) {
  if (!a.hrec) return;
  if (a.early_cap && (c->status != 0 || c->R <= a.early_cap)) return;
  HostRecord* h = a.hrec;
  h->R = c->R;
  h->status = c->status;
  h->error = 0;
  h->generic = generic;
  __hip_atomic_store(&h->seq, a.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

constexpr u32 kILP = 8;  // candidate loads in flight per thread

// Block blockIdx.x's contiguous share [lo, hi) of n candidates.
__device__ __forceinline__ void block_range(u64 n, u64* lo, u64* hi) {
  const u64 per = (n + gridDim.x - 1) / gridDim.x;
  *lo = (u64)blockIdx.x * per;
  *hi = *lo + per < n ? *lo + per : n;
  if (*lo > n) *lo = n;
}

// Output value of a candidate key: the value bits follow from the key's order code
// except for the two codes that fold several encodings (+-0, NaN), which are read back.
__device__ __forceinline__ u32 value_bits(u64 key, const float* x, u32 idx) {
  const u32 o = (u32)(key >> 32);
  if (o == 0x80000000u || o == 0xFFFFFFFFu) return reinterpret_cast<const u32*>(x)[idx];
  return bits_of_ord32(o);
}
}  // namespace

__global__ __launch_bounds__(kHistThreads) void refine_hist_kernel(RefineArgs a) {
  __shared__ u32 s_h[kBins];
  // the scatter reserves from zero
  for (u32 b = blockIdx.x * blockDim.x + threadIdx.x; b < kBins; b += gridDim.x * blockDim.x) a.cursor[b] = 0;
  const RowCtl* c = a.ctl;
  if (!refine_live(a, c)) return;
  const u64 n = cand_count(c, a.M);
  const u64 tau = c->tau;
  const u32 shift = bin_shift_of(c);
  for (u32 b = threadIdx.x; b < kBins; b += blockDim.x) s_h[b] = 0;
  __syncthreads();
  u64 lo, hi;
  block_range(n, &lo, &hi);
  for (u64 base = lo; base < hi; base += (u64)blockDim.x * kILP) {
    u64 kk[kILP];
#pragma unroll
    for (u32 q = 0; q < kILP; ++q) {
      const u64 i = base + (u64)q * blockDim.x + threadIdx.x;
      kk[q] = i < hi ? a.cand[i] : 0ull;
    }
#pragma unroll
    for (u32 q = 0; q < kILP; ++q)
      if (base + (u64)q * blockDim.x + threadIdx.x < hi) atomicAdd(&s_h[bin_of(kk[q], tau, shift)], 1u);
  }
  __syncthreads();
  for (u32 b = threadIdx.x; b < kBins; b += blockDim.x)
    if (s_h[b]) atomicAdd(&a.hist[b], s_h[b]);
}

namespace {
struct ScanLds {
  u32 off[kBins + kBins / kPer + 1];  // by padded descending position; last = total
  u32 wsum[kHistThreads / kWave];
  u32 q, big;
};

// The bin sort's chunk boundaries from the scan in LDS (every block holds it whole), split
// over the blocks by bin: boundary m gets the bin that holds output position m P - 1
// (P = ceil(T / W) for the T keys of the bins >= b*), written by the thread of that bin.
__device__ void write_chunks(const RefineArgs& a, const ScanLds* S, u32 qstar) {
  const u32 T = S->off[pad_q(qstar + 1)];
  const u32 W = a.sort_waves;
  const u32 P = T > W ? (T + W - 1) / W : 1u;
  const u64 inv = ((1ull << 32) + P - 1) / P;
  auto chunk_of = [&](u32 e) {  // floor(e / P) by a multiply, corrected
    u32 m = (u32)(((u64)e * inv) >> 32);
    if ((u64)m * P > e) --m;
    if ((u64)(m + 1) * P <= e) ++m;
    return m;
  };
  uint4* ch = reinterpret_cast<uint4*>(a.chunk);
  const u32 per = (qstar + gridDim.x) / gridDim.x;  // bins 0..qstar per block
  for (u32 q = blockIdx.x * per + threadIdx.x; q < (blockIdx.x + 1) * per && q <= qstar; q += blockDim.x) {
    const u32 e = S->off[pad_q(q)], f = S->off[pad_q(q + 1)];
    if (f == e) continue;
    const u32 mf = chunk_of(f), m2 = mf < W ? mf : W;
    for (u32 m = chunk_of(e) + 1; m <= m2; ++m) ch[m] = make_uint4(e, f, q, 0u);
  }
  for (u32 m = (T + P) / P + blockIdx.x * blockDim.x + threadIdx.x; m <= W; m += gridDim.x * blockDim.x)
    ch[m] = make_uint4(T, T, qstar + 1u, 0u);
  if (blockIdx.x == 0 && threadIdx.x == 0) ch[0] = make_uint4(0u, 0u, 0u, 0u);
}

// Every block of the scatter: the global histogram (loaded by ld(b)) scanned from the top
// bin down in LDS, the bin b* that holds the k-th largest candidate (returned as its
// descending position q*) and whether a bin at or above it is too large for the in-kernel
// sorts (then the attempt takes the multi-pass refinement).  Block 0 publishes b* and
// the record.  Returns true for the multi-pass case.
template <class Load>
__device__ bool bin_scan(const RefineArgs& a, RowCtl* c, u32 shift, Load&& ld, ScanLds* S, u32* qstar_out) {
  const u32 tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  {
    u32 v[kPer];  // all loads in flight, then the LDS stores
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) v[j] = ld(j * kHistThreads + tid);
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) S->off[pad_q(kBins - 1u - (j * kHistThreads + tid))] = v[j];
  }
  if (tid == 0) {
    S->q = 0xFFFFFFFFu;
    S->big = 0;
  }
  __syncthreads();
  // exclusive offsets over descending positions: thread tid owns q = tid*kPer + j
  u32 cnt[kPer];
  u32 sum = 0;
#pragma unroll
  for (u32 j = 0; j < kPer; ++j) {
    cnt[j] = S->off[pad_q(tid * kPer + j)];
    sum += cnt[j];
  }
  u32 incl = sum;
#pragma unroll
  for (u32 d = 1; d < (u32)kWave; d <<= 1) {
    const u32 v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) S->wsum[wid] = incl;
  __syncthreads();
  u32 run = incl - sum;
  for (u32 w = 0; w < wid; ++w) run += S->wsum[w];
  const u64 k = a.k;
#pragma unroll
  for (u32 j = 0; j < kPer; ++j) {
    const u32 q = tid * kPer + j;
    S->off[pad_q(q)] = run;
    if (run < k && run + cnt[j] >= k) S->q = q;  // exactly one bin holds the k-th largest
    run += cnt[j];
  }
  if (tid == blockDim.x - 1) S->off[pad_q(kBins)] = run;
  __syncthreads();
  // fewer than k candidates (approximate mode only): every bin is needed
  const u32 qstar = S->q == 0xFFFFFFFFu && a.approx ? kBins - 1u : S->q;
  // every bin at or above b* must fit the in-kernel sorts and partition
  bool big = qstar == 0xFFFFFFFFu;
#pragma unroll
  for (u32 j = 0; j < kPer; ++j)
    if (tid * kPer + j <= qstar && cnt[j] > a.msd_cap) big = true;
  if (big) S->big = 1;
  __syncthreads();
  const bool generic = S->big != 0;
  if (blockIdx.x == 0 && tid == 0) {
    c->bin_shift = shift;
    c->bstar = generic ? 0u : kBins - 1u - qstar;
    c->c_above = generic ? 0u : S->off[pad_q(qstar)];
    c->generic = generic ? 1u : 0u;
    if (a.rec) a.rec->generic = generic ? 1u : 0u;
    publish(a, c, generic ? 1u : 0u);
  }
  *qstar_out = qstar;
  return generic;
}
}  // namespace

__global__ __launch_bounds__(kHistThreads) void refine_scatter_kernel(RefineArgs a) {
  __shared__ ScanLds s_scan;
  __shared__ u32 s_pos[kBins];
  RowCtl* c = a.ctl;
  if (!refine_live(a, c)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) publish(a, c, 0u);
    return;
  }
  const u32 tid = threadIdx.x;
  const u64 n = cand_count(c, a.M);
  const u64 tau = c->tau;
  const u32 shift = bin_shift_of(c);
  u32 qstar;
  const bool generic = bin_scan(a, c, shift, [&](u32 b) { return a.hist[b]; }, &s_scan, &qstar);
  const u32* s_off = s_scan.off;
  if (generic) return;
  const u32 bstar = kBins - 1u - qstar;

  // this block's contiguous range of candidates, counted per bin >= b*
  u64 lo, hi;
  block_range(n, &lo, &hi);
  for (u32 b = bstar + tid; b < kBins; b += blockDim.x) s_pos[b] = 0;
  __syncthreads();
  for (u64 base = lo; base < hi; base += (u64)blockDim.x * kILP) {
    u64 kk[kILP];
#pragma unroll
    for (u32 q = 0; q < kILP; ++q) {
      const u64 i = base + (u64)q * blockDim.x + tid;
      kk[q] = i < hi ? a.cand[i] : 0ull;
    }
#pragma unroll
    for (u32 q = 0; q < kILP; ++q) {
      const u32 b = bin_of(kk[q], tau, shift);
      if (base + (u64)q * blockDim.x + tid < hi && b >= bstar) atomicAdd(&s_pos[b], 1u);
    }
  }
  __syncthreads();
  {
    // reserve each (block, bin) run: all of this thread's atomics in flight together
    u32 m[kPer], got[kPer];
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) {
      const u32 b = bstar + tid + j * kHistThreads;
      m[j] = b < kBins ? s_pos[b] : 0u;
    }
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) got[j] = m[j] ? atomicAdd(&a.cursor[bstar + tid + j * kHistThreads], m[j]) : 0u;
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) {
      const u32 b = bstar + tid + j * kHistThreads;
      if (m[j]) s_pos[b] = s_off[pad_q(kBins - 1u - b)] + got[j];
    }
  }
  __syncthreads();
  for (u64 base = lo; base < hi; base += (u64)blockDim.x * kILP) {
    u64 kk[kILP];
#pragma unroll
    for (u32 q = 0; q < kILP; ++q) {
      const u64 i = base + (u64)q * blockDim.x + tid;
      kk[q] = i < hi ? a.cand[i] : 0ull;
    }
#pragma unroll
    for (u32 q = 0; q < kILP; ++q) {
      const u32 b = bin_of(kk[q], tau, shift);
      if (base + (u64)q * blockDim.x + tid < hi && b >= bstar) {
        const u32 pos = atomicAdd(&s_pos[b], 1u);
        if (pos < a.M) a.tmp[pos] = kk[q];
      }
    }
  }
  write_chunks(a, &s_scan, qstar);
}

namespace {
constexpr u32 kGridMark = 1u << 30;  // added to the launch-wide counter when a wait ran out
constexpr u32 kGoOffset = 16;        // the go word, u32 words after the counter: the next 128-byte line
constexpr u32 kKeep = 16;            // candidates per thread refine_bin_kernel keeps in registers

// Thread 0 of each block: arrive at the launch-wide counter ctr (zero on entry) and wait
// until all G blocks have: the last to arrive sets the go word (zero on entry), which
// the others poll.  A wait longer than `limit` ticks of the 100 MHz clock (a block could
// not be made resident) marks the counter, which only succeeds while some block has not
// arrived, so no block can have passed it yet; the marking block tells the waiters
// through the go word, and the late blocks see the mark in the value their own arrival
// returns.  True: all arrived.  limit = 0: the wait counts as run out at once (every
// block marks the counter).
__device__ bool grid_wait(u32* ctr, u32* go, u32 G, u64 limit) {
  if (limit == 0) {  // the wait counts as run out at once (every block marks the counter)
    __hip_atomic_fetch_or(ctr, kGridMark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  // arrivals add to ctr; the last one raises `go` (another line, which the waiters poll,
  // so that their loads do not queue in front of the arrivals' atomics)
  u32 v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  if (v >= kGridMark) return false;
  if (v == G) {
    atomic_store_agent(go, 1u);
    return true;
  }
  const u64 t0 = wall_clock64();
  for (;;) {
    const u32 g = atomic_load_agent(go);
    if (g) return g == 1u;
    if (wall_clock64() - t0 >= limit) {
      // mark the counter while some block has not arrived (then none has passed), and
      // tell the other waiters
      u32 seen = atomic_load_agent(ctr);
      while (seen < G) {
        if (__hip_atomic_compare_exchange_strong(ctr, &seen, seen + kGridMark, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
          atomic_store_agent(go, 2u);
          return false;
        }
      }
      // every block arrived meanwhile (the last one raises go) or another block marked
      if (seen >= kGridMark) return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}
}  // namespace

// Exact mode: the histogram and the scatter in one launch.  Each block counts its
// contiguous share of the candidates per bin in LDS and adds the counts into the global
// histogram with returning atomics: the value each returns is where the block's run
// starts within that bin, so no second reservation is needed.  The blocks then wait for
// each other once (a counter in the workspace; at most one 1024-thread block per two
// CUs, so all are resident), scan the finished histogram as refine_scatter_kernel does
// and place their candidates of the bins >= b*.  A wait that runs out (a.wait_ticks)
// sends the attempt to the multi-pass refinement instead, before any block has placed a
// key.  The bin sort clears the counter.
__global__ __launch_bounds__(kHistThreads) void refine_bin_kernel(RefineArgs a) {
  __shared__ ScanLds s_scan;
  __shared__ u32 s_pos[kBins];  // this block's count per bin, then its next position in it
  __shared__ u32 s_ok;
  RowCtl* c = a.ctl;
  if (!refine_live(a, c)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) publish(a, c, 0u);
    return;
  }
  const u32 tid = threadIdx.x;
  const u64 n = cand_count(c, a.M);
  const u64 tau = c->tau;
  const u32 shift = bin_shift_of(c);
  for (u32 b = tid; b < kBins; b += kHistThreads) s_pos[b] = 0;
  __syncthreads();
  u64 lo, hi;
  block_range(n, &lo, &hi);
  // a share of up to kKeep keys per thread stays in registers until the placement, with
  // each key's rank among the block's keys of its bin (from the counting atomic)
  const bool kept = hi - lo <= (u64)kKeep * kHistThreads;
  u64 kk[kKeep];
  u32 rk[kKeep];
  if (kept) {
#pragma unroll
    for (u32 q = 0; q < kKeep; ++q) {
      const u64 i = lo + (u64)q * kHistThreads + tid;
      kk[q] = i < hi ? a.cand[i] : 0ull;
    }
#pragma unroll
    for (u32 q = 0; q < kKeep; ++q)
      rk[q] = lo + (u64)q * kHistThreads + tid < hi ? atomicAdd(&s_pos[bin_of(kk[q], tau, shift)], 1u) : 0u;
  } else {
    for (u64 base = lo; base < hi; base += (u64)kHistThreads * kILP) {
      u64 kl[kILP];
#pragma unroll
      for (u32 q = 0; q < kILP; ++q) {
        const u64 i = base + (u64)q * kHistThreads + tid;
        kl[q] = i < hi ? a.cand[i] : 0ull;
      }
#pragma unroll
      for (u32 q = 0; q < kILP; ++q)
        if (base + (u64)q * kHistThreads + tid < hi) atomicAdd(&s_pos[bin_of(kl[q], tau, shift)], 1u);
    }
  }
  __syncthreads();
  {
    // all of this thread's atomics in flight together; storing their results waits for
    // them, so they are complete at the barrier below
    u32 m[kPer], got[kPer];
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) m[j] = s_pos[j * kHistThreads + tid];
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) got[j] = m[j] ? atomicAdd(&a.hist[j * kHistThreads + tid], m[j]) : 0u;
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) s_pos[j * kHistThreads + tid] = got[j];
  }
  __syncthreads();
  if (tid == 0) s_ok = grid_wait(a.ticket, a.ticket + kGoOffset, gridDim.x, a.wait_ticks) ? 1u : 0u;
  __syncthreads();
  if (!s_ok) {
    if (blockIdx.x == 0 && tid == 0) {
      c->bin_shift = shift;
      c->bstar = 0;
      c->c_above = 0;
      c->generic = 1;
      if (a.rec) a.rec->generic = 1u;
      publish(a, c, 1u);
    }
    return;
  }
  u32 qstar;
  const bool generic = bin_scan(a, c, shift, [&](u32 b) { return atomic_load_agent(&a.hist[b]); }, &s_scan, &qstar);
  if (generic) return;
  const u32 bstar = kBins - 1u - qstar;
  for (u32 b = bstar + tid; b < kBins; b += kHistThreads) s_pos[b] += s_scan.off[pad_q(kBins - 1u - b)];
  __syncthreads();
  if (kept) {
#pragma unroll
    for (u32 q = 0; q < kKeep; ++q) {
      const u32 b = bin_of(kk[q], tau, shift);
      if (lo + (u64)q * kHistThreads + tid < hi && b >= bstar) {
        const u32 pos = s_pos[b] + rk[q];
        if (pos < a.M) a.tmp[pos] = kk[q];
      }
    }
    write_chunks(a, &s_scan, qstar);  // for the next launch, off this launch's critical path
    return;
  }
  for (u64 base = lo; base < hi; base += (u64)kHistThreads * kILP) {
    u64 kl[kILP];
#pragma unroll
    for (u32 q = 0; q < kILP; ++q) {
      const u64 i = base + (u64)q * kHistThreads + tid;
      kl[q] = i < hi ? a.cand[i] : 0ull;
    }
#pragma unroll
    for (u32 q = 0; q < kILP; ++q) {
      const u32 b = bin_of(kl[q], tau, shift);
      if (base + (u64)q * kHistThreads + tid < hi && b >= bstar) {
        const u32 pos = atomicAdd(&s_pos[b], 1u);
        if (pos < a.M) a.tmp[pos] = kl[q];
      }
    }
  }
  write_chunks(a, &s_scan, qstar);
}

#ifndef PROFK_WAVE_MAX
#define PROFK_WAVE_MAX 256
#endif
// Bins up to kWaveMax keys are sorted by one wavefront; larger ones by the workgroup
// (a register sort of 8 keys per lane is a chain of some 4000 instructions on one
// SIMD, the workgroup's counting pass a few LDS round trips).
constexpr u32 kWaveMax = PROFK_WAVE_MAX;
constexpr u32 kSubDigits = 256;  // digit of the workgroup's counting pass (8 bits)
constexpr u32 kRankScan = 32;    // sub-buckets up to this size are ranked by a scan
constexpr u32 kHeavyPer = kBinCap / kSortThreads;

__device__ __forceinline__ void write_out(const RefineArgs& a, u64 p, u64 key) {
  const u32 idx = key_index(key);
  a.out_idx[p] = idx < a.N ? (int64_t)idx : -1;
  if (idx < a.N) reinterpret_cast<u32*>(a.out_vals)[p] = value_bits(key, a.x, idx);
}

// n <= 64*M keys at src[0..n) (global memory or LDS), sorted by one wavefront in
// registers; sorted position i goes to output position out0 + i when that is below k.
template <int M>
__device__ __forceinline__ void wave_bin(const RefineArgs& a, const u64* src, u32 n, u64 out0) {
  const u32 lane = lane_id();
  u64 v[M];
#pragma unroll
  for (int r = 0; r < M; ++r) {
    const u32 i = (u32)r * kWave + lane;
    v[r] = i < n ? src[i] : 0ull;
  }
  wave_sort_regs_desc<M>(v);
#pragma unroll
  for (int r = 0; r < M; ++r) {
    const u32 i = (u32)r * kWave + lane;
    if (i < n && out0 + i < a.k) write_out(a, out0 + i, v[r]);
  }
}

// 1 <= n <= kWaveBin keys at src[0..n) to output positions from out0 (wave-uniform
// arguments).
__device__ __forceinline__ void wave_part(const RefineArgs& a, const u64* src, u32 n, u64 out0) {
  if (n <= 64) wave_bin<1>(a, src, n, out0);
  else if (n <= 128) wave_bin<2>(a, src, n, out0);
  else if (n <= 256) wave_bin<4>(a, src, n, out0);
  else wave_bin<8>(a, src, n, out0);
}

// A light bin of 1 <= n <= 64*M keys already loaded (v[r], element r*64 + lane),
// sorted by the wavefront in registers and written from output position out0.
template <int M>
__device__ __forceinline__ void light_sort(const RefineArgs& a, const u64 (&v)[4], u32 n, u64 out0) {
  const u32 lane = lane_id();
  u64 w[M];
#pragma unroll
  for (int r = 0; r < M; ++r) w[r] = v[r];
  wave_sort_regs_desc<M>(w);
#pragma unroll
  for (int r = 0; r < M; ++r) {
    const u32 i = (u32)r * kWave + lane;
    if (i < n && out0 + i < a.k) write_out(a, out0 + i, w[r]);
  }
}

constexpr u32 kTieCap = 16;  // largest digit bucket wave_range_sort ranks by comparisons
constexpr u32 kWaveLds = 8 * kWave;  // u64 words of LDS per wavefront: 256 keys, counts, starts

// A range of kWave < n <= R kWave keys (v[r], element r*64 + lane) sorted by one
// wavefront and written from output position out0: one counting pass on an 8-bit digit
// of g = (key - tau) >> sub (g is monotone in the key), scaled to the range's span of g,
// then each key's position is its digit bucket's start plus the number of larger keys
// in the bucket.  About 250 instructions for 256 keys against some 1350 for the
// register bitonic sort.  Returns false, writing nothing, when a bucket holds more than
// kTieCap keys (runs of near-equal values).  w: the wavefront's kWaveLds words of LDS.
// (Bins of 257..512 keys sorted this way, 8 keys per lane in twice the LDS, measured no
// faster than the workgroup's counting pass.)
template <int R>
__device__ bool wave_range_sort(const RefineArgs& a, const u64 (&v)[R], u32 n, u64 out0, u64 tau, u32 sub, u64* w) {
  static_assert(R * kWave + 2 * 2 * kWave <= kWaveLds, "keys, counts and starts fit the wavefront's LDS");
  const u32 lane = lane_id();
  u32* cnt = reinterpret_cast<u32*>(w + 4 * kWave);
  u32* beg = cnt + 4 * kWave;
  u32 g[R];
  bool ok[R];
  u32 gmin = 0xFFFFFFFFu, gmax = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    ok[r] = (u32)r * kWave + lane < n;
    g[r] = (u32)((v[r] - tau) >> sub);
    if (ok[r]) {
      gmin = g[r] < gmin ? g[r] : gmin;
      gmax = g[r] > gmax ? g[r] : gmax;
    }
  }
  gmin = wave_reduce_u32(gmin, [](u32 x, u32 y) { return x < y ? x : y; });
  gmax = wave_reduce_u32(gmax, [](u32 x, u32 y) { return x > y ? x : y; });
  const u32 span = gmax - gmin;
  const u32 extra = span < 256u ? 0u : 24u - (u32)__clz(span);  // (span >> extra) < 256
#pragma unroll
  for (u32 j = 0; j < 4; ++j) cnt[4 * lane + j] = 0;
  wave_lds_sync();
  u32 d[R], rk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    d[r] = ok[r] ? (g[r] - gmin) >> extra : 0u;
    rk[r] = ok[r] ? atomicAdd(&cnt[d[r]], 1u) : 0u;
  }
  wave_lds_sync();
  // bucket starts over descending digits: lane owns digits 255 - 4 lane - j
  u32 c[4], sum = 0, cm = 0;
#pragma unroll
  for (u32 j = 0; j < 4; ++j) {
    c[j] = cnt[255u - 4 * lane - j];
    sum += c[j];
    cm = c[j] > cm ? c[j] : cm;
  }
  u32 run = wave_incl_scan_add(sum, lane) - sum;
#pragma unroll
  for (u32 j = 0; j < 4; ++j) {
    beg[255u - 4 * lane - j] = run;
    run += c[j];
  }
  const u32 maxb = wave_reduce_u32(cm, [](u32 x, u32 y) { return x > y ? x : y; });
  wave_lds_sync();
  if (maxb > kTieCap) return false;
  u32 b0[R], bc[R], gt[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    b0[r] = beg[d[r]];
    bc[r] = ok[r] ? cnt[d[r]] : 0u;
    gt[r] = 0;
    if (ok[r]) w[b0[r] + rk[r]] = v[r];
  }
  wave_lds_sync();
  for (u32 it = 0; it < maxb; ++it) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (it < bc[r]) gt[r] += w[b0[r] + it] > v[r] ? 1u : 0u;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const u64 p = out0 + b0[r] + gt[r];
    if (ok[r] && p < a.k) write_out(a, p, v[r]);
  }
  wave_lds_sync();  // the next range reuses w
  return true;
}

// A part of cnt <= kBinCap keys at src[start..), sorted by the workgroup in LDS.
__device__ void lds_part(const RefineArgs& a, u64* s, const u64* src, u32 start, u32 cnt) {
  u32 P = 1;
  while (P < cnt) P <<= 1;
  __syncthreads();
  for (u32 i = threadIdx.x; i < P; i += blockDim.x) s[i] = i < cnt ? src[start + i] : 0ull;
  __syncthreads();
  block_bitonic_desc(s, P);
  const u64 lim = a.k - start < cnt ? a.k - start : cnt;
  for (u32 i = threadIdx.x; i < lim; i += blockDim.x) write_out(a, start + i, s[i]);
}

struct HeavyLds {
  u32 cnt[kSubDigits];  // keys per sub-digit
  u32 beg[kSubDigits];  // start of each sub-bucket within the bin, descending digits first
  u32 cur[kSubDigits];  // placement cursors
  u32 big[kSubDigits];  // sub-digits whose bucket is ranked by a wavefront sort
  u32 nbig;
  u32 over;             // some sub-bucket exceeds kWaveBin
};

// A bin of kWaveMax < cnt <= kBinCap keys at tmp[start..), by the workgroup: one
// counting pass on the next 8 bits below the bin's own (bits [sub, sub + 8) of
// key - tau; higher bits are equal within the bin, so the digit orders the keys
// coarsely), the keys placed in LDS by descending digit, then each key's position
// is its sub-bucket's start plus the number of larger keys in the sub-bucket (a scan
// of at most kRankScan keys); sub-buckets of up to kWaveBin keys are sorted by one
// wavefront each, and a larger one (long runs of equal values) sends the bin to the
// LDS bitonic sort.
__device__ void heavy_part(const RefineArgs& a, u64* s, HeavyLds* L, u32 start, u32 cnt, u64 tau, u32 sub) {
  const u32 tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const u64* src = a.tmp + start;
  __syncthreads();  // the previous user of s and L is done
  for (u32 d = tid; d < kSubDigits; d += blockDim.x) L->cnt[d] = 0;
  if (tid == 0) {
    L->nbig = 0;
    L->over = 0;
  }
  __syncthreads();
  // the keys are read twice from tmp (L2) rather than held in registers, which would
  // cost the kernel its occupancy
#pragma unroll 4
  for (u32 i = tid; i < cnt; i += kSortThreads) atomicAdd(&L->cnt[(u32)((src[i] - tau) >> sub) & (kSubDigits - 1u)], 1u);
  __syncthreads();
  if (wid == 0) {
    // descending exclusive offsets: lane owns descending positions 4*lane .. 4*lane + 3
    constexpr u32 kPerL = kSubDigits / kWave;
    u32 c[kPerL], sum = 0;
#pragma unroll
    for (u32 r = 0; r < kPerL; ++r) {
      c[r] = L->cnt[kSubDigits - 1u - (lane * kPerL + r)];
      sum += c[r];
    }
    u32 incl = sum;
#pragma unroll
    for (u32 d = 1; d < (u32)kWave; d <<= 1) {
      const u32 o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    u32 run = incl - sum;
#pragma unroll
    for (u32 r = 0; r < kPerL; ++r) {
      const u32 d = kSubDigits - 1u - (lane * kPerL + r);
      L->beg[d] = run;
      L->cur[d] = run;
      if (c[r] > kWaveBin) L->over = 1;
      else if (c[r] > kRankScan) L->big[atomicAdd(&L->nbig, 1u)] = d;
      run += c[r];
    }
  }
  __syncthreads();
  if (L->over) {
    lds_part(a, s, a.tmp, start, cnt);
    return;
  }
#pragma unroll 4
  for (u32 i = tid; i < cnt; i += kSortThreads) {
    const u64 key = src[i];
    s[atomicAdd(&L->cur[(u32)((key - tau) >> sub) & (kSubDigits - 1u)], 1u)] = key;
  }
  __syncthreads();
  for (u32 i = tid; i < cnt; i += kSortThreads) {
    const u64 key = s[i];
    const u32 d = (u32)((key - tau) >> sub) & (kSubDigits - 1u);
    const u32 c = L->cnt[d];
    if (c > kRankScan) continue;
    const u32 b0 = L->beg[d];
    u32 r = 0;
    for (u32 q = 0; q < c; ++q) r += s[b0 + q] > key ? 1u : 0u;
    const u64 p = (u64)start + b0 + r;
    if (p < a.k) write_out(a, p, key);
  }
  const u32 nbig = L->nbig;
  if (nbig == 0) return;
  // the placed bin back into its own range of tmp, so that one wavefront per large
  // sub-bucket sorts it from there
  for (u32 i = tid; i < cnt; i += blockDim.x) a.tmp[start + i] = s[i];
  __syncthreads();
  for (u32 e = wid; e < nbig; e += kSortThreads / kWave) {
    const u32 d = L->big[e];
    const u32 b0 = L->beg[d];
    if ((u64)start + b0 < a.k) wave_part(a, a.tmp + start + b0, L->cnt[d], (u64)start + b0);
  }
}

__device__ __forceinline__ u32 msd_digit(u64 key, u64 tau, u32 sub) {
  return (u32)((key - tau) >> sub) & (kMsdDigits - 1u);
}

constexpr u32 kMsdMaxLevels = (64 + kMsdBits - 1) / kMsdBits + 1;

struct MsdLds {
  u32 nlist;  // entries appended to the next level's list
  u64 ent;    // entry being processed (broadcast)
  u32 wsum[kSortThreads / kWave];
};

// Splits the part of c0 keys at src[s0..) by the digit of (key - tau) at bit `sub`
// into dst[s0..), parts in descending digit order.  Parts of at most kWaveBin keys
// that reach a position below k are sorted at once by one wavefront; larger ones are
// appended to nxt.  The digit cursors live in the LDS sort buffer s.
__device__ void msd_split(const RefineArgs& a, u64* s, const u64* src, u64* dst, u32 s0, u32 c0, u32 sub,
                          u64 tau, u64* nxt, MsdLds* m) {
  u32* cur = reinterpret_cast<u32*>(s);
  const u32 tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  constexpr u32 kPerT = kMsdDigits / kSortThreads;
  for (u32 d = tid; d < kMsdDigits; d += blockDim.x) cur[d] = 0;
  __syncthreads();
  for (u32 i = tid; i < c0; i += blockDim.x) atomicAdd(&cur[msd_digit(src[s0 + i], tau, sub)], 1u);
  __syncthreads();
  // start of every part: thread tid owns descending positions [tid*kPerT, tid*kPerT + kPerT)
  u32 v[kPerT];
  u32 sum = 0;
#pragma unroll
  for (u32 j = 0; j < kPerT; ++j) {
    v[j] = cur[kMsdDigits - 1u - (tid * kPerT + j)];
    sum += v[j];
  }
  u32 incl = sum;
#pragma unroll
  for (u32 d = 1; d < (u32)kWave; d <<= 1) {
    const u32 o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) m->wsum[wid] = incl;
  __syncthreads();
  u32 run = s0 + incl - sum;
  for (u32 w = 0; w < wid; ++w) run += m->wsum[w];
#pragma unroll
  for (u32 j = 0; j < kPerT; ++j) {
    cur[kMsdDigits - 1u - (tid * kPerT + j)] = run;
    run += v[j];
  }
  __syncthreads();
  for (u32 i = tid; i < c0; i += blockDim.x) {
    const u64 key = src[s0 + i];
    dst[atomicAdd(&cur[msd_digit(key, tau, sub)], 1u)] = key;
  }
  __syncthreads();
  // part d now spans [end of part d + 1, cur[d]); each wavefront takes 64 digits at a time
  for (u32 ch = wid; ch < kMsdDigits / kWave; ch += kSortThreads / kWave) {
    const u32 d = kMsdDigits - 1u - (ch * kWave + lane);
    const u32 en = cur[d];
    const u32 st = d == kMsdDigits - 1u ? s0 : cur[d + 1];
    const u32 c = en - st;
    const bool need = c != 0 && (u64)st < a.k;
    if (need && c > kWaveBin) nxt[atomicAdd(&m->nlist, 1u)] = (u64)st | ((u64)c << 32);
    u64 small = __ballot(need && c <= kWaveBin);
    while (small) {
      const int l = __ffsll((unsigned long long)small) - 1;
      small &= small - 1;
      const u32 ps = (u32)__shfl((int)st, l), pc = (u32)__shfl((int)c, l);
      wave_part(a, dst + ps, pc, ps);
    }
  }
  __syncthreads();
}

// Bin b of cnt > kBinCap keys at tmp[start..), of key width 2^width: partitioned level
// by level (ping-pong between tmp and the candidate buffer, which the scatter no longer
// needs) until every part below position k is sorted.  Parts at one level are disjoint
// and hold more than kWaveBin keys, so a list never exceeds cnt / kWaveBin + 1 entries;
// bins' lists are disjoint pool ranges.  Each level lowers the width by kMsdBits, and a
// part of width 2^kMsdBits holds at most kMsdDigits <= kBinCap distinct keys, so at most
// ceil(64 / kMsdBits) levels run.
__device__ void msd_bin(const RefineArgs& a, u64* s, u32 b, u32 start, u32 cnt, u32 width, u64 tau, MsdLds* m) {
  const u32 cap = (cnt >> kWaveBinBits) + 1u;
  u64* cur = a.pool + 2ull * ((u64)(start >> kWaveBinBits) + (kBins - 1u - b));
  u64* nxt = cur + cap;
  u64* src = a.tmp;
  u64* dst = a.cand;
  if (threadIdx.x == 0) atomic_store_agent(&cur[0], (u64)start | ((u64)cnt << 32));
  u32 ncur = 1;
  u32 w = width;
  // keys are distinct, so a part of width 1 holds one key: the level bound only
  // guarantees termination
  for (u32 level = 0; ncur && level < kMsdMaxLevels; ++level) {
    const u32 sub = w > kMsdBits ? w - kMsdBits : 0u;
    if (threadIdx.x == 0) m->nlist = 0;
    __syncthreads();
    for (u32 e = 0; e < ncur; ++e) {
      if (threadIdx.x == 0) m->ent = atomic_load_agent(&cur[e]);
      __syncthreads();
      const u64 ent = m->ent;
      __syncthreads();
      const u32 s0 = (u32)ent, c0 = (u32)(ent >> 32);
      if (c0 <= kBinCap)
        lds_part(a, s, src, s0, c0);
      else
        msd_split(a, s, src, dst, s0, c0, sub, tau, nxt, m);
    }
    __syncthreads();
    ncur = m->nlist;
    __syncthreads();  // every thread has the count before thread 0 resets it
    u64* t = cur;
    cur = nxt;
    nxt = t;
    t = src;
    src = dst;
    dst = t;
    w = sub;
  }
}

// Wavefront w of the launch takes output chunk w: the bins that start in positions
// [w P, (w + 1) P), from the chunk boundaries the scan wrote, so that every wavefront
// sorts about P keys whatever the bins' sizes.  Ranges of up to kWaveMax keys are
// sorted in registers; a last bin beyond that goes to the whole workgroup after its
// wavefronts are done (at most one per wavefront): the counting pass above up to
// kBinCap keys, else the partition by 12-bit digits.

__global__ __launch_bounds__(kSortThreads) void refine_binsort_kernel(RefineArgs a) {
  __shared__ u64 s[kBinCap];
  __shared__ uint4 s_big[kSortThreads / kWave];  // {start, end, position} of the block's heavy bins
  __shared__ u32 s_nbig;
  __shared__ MsdLds s_msd;
  __shared__ HeavyLds s_heavy;
  constexpr u32 kWaves = kSortThreads / kWave;
  const u32 lane = lane_id();
  const u32 wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // this wavefront's chunk boundaries, loaded with the control block (they are only
  // used when the scan wrote them: a live attempt with no oversized bin).  A workgroup
  // takes four consecutive chunks (dealing them out across the workgroups, so that the
  // heavy bins near b* meet different workgroups, measured slower: their counting
  // passes then share every CU's LDS at once).
  const u32 m = blockIdx.x * kWaves + wid;
  const uint4* ch = reinterpret_cast<const uint4*>(a.chunk);
  const uint4 c0 = ch[m], c1 = ch[m + 1];
  {  // leave the histogram and the sampler's hash set zero for the next attempt
    const u64 gt = (u64)blockIdx.x * blockDim.x + threadIdx.x, gs = (u64)gridDim.x * blockDim.x;
    for (u64 i = gt; i < kBins; i += gs) a.hist[i] = 0;
    if (gt == 0 && a.ticket) {  // refine_bin_kernel's counter and go word
      a.ticket[0] = 0;
      a.ticket[kGoOffset] = 0;
    }
    if (a.table)
      for (u64 i = gt; i < a.table_slots; i += gs) a.table[i] = 0;
  }
  const RowCtl* c = a.ctl;
  if (a.approx) {
    // approximate mode: the outcome of the check, and padding where fewer than k
    // candidates were kept
    const u64 gt = (u64)blockIdx.x * blockDim.x + threadIdx.x, gs = (u64)gridDim.x * blockDim.x;
    if (gt == 0 && a.info) {
      a.info->R = (int64_t)c->R;
      a.info->M = (int64_t)a.M;
      a.info->status = (int32_t)c->status;
      a.info->exact_path = 0;
    }
    const u64 n = refine_live(a, c) ? cand_count(c, a.M) : 0;
    for (u64 p = n + gt; p < a.k; p += gs) {
      a.out_idx[p] = -1;
      reinterpret_cast<u32*>(a.out_vals)[p] = 0xFF800000u;  // -inf
    }
  }
  if (!refine_live(a, c) || c->generic) return;
  const u64 k = a.k;
  const u64 tau = c->tau;
  const u32 width = c->bin_shift;
  const u32 sub = width > 8u ? width - 8u : 0u;
  if (threadIdx.x == 0) s_nbig = 0;
  __syncthreads();
  {
    // The chunk's bins occupy tmp[rs, re).  Every bin but the last holds fewer than
    // kChunkKeys keys (it starts and ends inside the chunk); the last one, [ls, re),
    // may run past it.  Up to kWaveMax keys: one sort of the whole range (the bins are
    // ordered, so sorting them together sorts each); else the bins before the last,
    // then the last one if it is light, or the workgroup takes it below.
    const u32 rs = c0.y, re = c1.y, ls = c1.x;
    u32 st[2] = {rs, ls}, n[2] = {0u, 0u};
    bool heavy = false;
    if (re > rs && rs < k && re <= a.M) {
      if (re - rs <= kWaveMax) {
        n[0] = re - rs;
      } else {
        n[0] = ls - rs;
        if (ls < k) {
          if (re - ls <= kWaveMax) n[1] = re - ls;
          else heavy = true;
        }
      }
    }
    static_assert(kWaveMax == 4 * kWave && kChunkKeys <= kWaveMax, "light ranges take 4 keys per lane");
    u64* wl = s + wid * kWaveLds;
    u64 v[2][4];
#pragma unroll
    for (u32 r = 0; r < 2; ++r)
#pragma unroll
      for (u32 j = 0; j < 4; ++j) {
        const u32 e = j * kWave + lane;
        v[r][j] = e < n[r] ? a.tmp[st[r] + e] : 0ull;
      }
    // one range at a time from the front, which then moves up: one copy of each sort
#pragma unroll 1
    for (u32 r = 0; r < 2; ++r) {
      const u32 nn = n[0], s0 = st[0];
      const u64 cur[4] = {v[0][0], v[0][1], v[0][2], v[0][3]};
      n[0] = n[1];
      st[0] = st[1];
#pragma unroll
      for (u32 j = 0; j < 4; ++j) v[0][j] = v[1][j];
      n[1] = 0;
      if (nn == 0) continue;
      if (nn <= kWave) light_sort<1>(a, cur, nn, s0);
      else if (!wave_range_sort<4>(a, cur, nn, s0, tau, sub, wl)) {
        if (nn <= 2 * kWave) light_sort<2>(a, cur, nn, s0);
        else light_sort<4>(a, cur, nn, s0);
      }
    }
    if (heavy && lane == 0) s_big[atomicAdd(&s_nbig, 1u)] = make_uint4(ls, re, c1.z, 0u);
  }
  __syncthreads();
  const u32 nbig = s_nbig;
  for (u32 q = 0; q < nbig; ++q) {
    const uint4 h = s_big[q];
    const u32 start = h.x, cnt = h.y - h.x;
    if (cnt <= kBinCap)
      heavy_part(a, s, &s_heavy, start, cnt, tau, sub);
    else
      msd_bin(a, s, kBins - 1u - h.z, start, cnt, width, tau, &s_msd);
  }
}

// One launch for small k (k <= kSmallK), in place of the three above.  When at most
// kSmallShare candidates were kept (the usual case), workgroup 0 takes them all into
// registers, selects the k-th largest (an 8-bit radix select) and sorts the k keys at
// or above it (one wavefront, in registers).  Otherwise each of the first G workgroups
// takes a contiguous share of at most kSmallShare candidates and keeps its k largest
// in a list of k slots in tmp, zero-padded; the last of them to finish takes the G
// lists, selects the k-th largest of their union the same way and sorts.  The k
// largest candidates are among the lists, since each is among the k largest of its
// own share.
// The workgroups past the first G only clear the sampler's hash set (16-byte stores).
constexpr u32 kSmallK = 64;
constexpr u32 kSmallThreads = 256;
constexpr u32 kSmallPer = 16;                               // candidates per thread
constexpr u32 kSmallShare = kSmallThreads * kSmallPer;      // per workgroup
constexpr u32 kSmallLists = 2 * kSmallShare;                // keys of the union
constexpr u32 kClearPerBlock = kSmallThreads * 4;           // 16-byte words per clearing workgroup

// The lists pass between workgroups through agent-scope atomic stores and loads and a
// store-completion wait before the election counter's increment (ld_agent, st_agent,
// drain_memory_ops): an agent-scope release / acquire fence would also write back /
// invalidate the whole L2 of the die, which the hash-set clearing workgroups have just
// filled with dirty lines, about 4 us per call.

// g[0..m) into registers, thread t taking g[t + q * kSmallThreads]; zero past m.
// kShared: g holds another workgroup's lists, read with agent-scope atomic loads.
template <bool kShared, u32 P>
__device__ __forceinline__ void small_load(u64 (&v)[P], const u64* g, u32 m) {
#pragma unroll
  for (u32 q = 0; q < P; ++q) {
    const u32 i = q * kSmallThreads + threadIdx.x;
    v[q] = i < m ? (kShared ? ld_agent(g + i) : g[i]) : 0ull;
  }
}

// The keys of v at or above kth (all nonzero ones when kth is 0) into dst, at most cap.
// kShared: dst is a list another workgroup reads, written with agent-scope atomic stores.
template <bool kShared, u32 P>
__device__ __forceinline__ void small_gather(const u64 (&v)[P], u64 kth, u64* dst, u32 cap, u32* n) {
#pragma unroll
  for (u32 q = 0; q < P; ++q)
    if (v[q] != 0 && v[q] >= kth) {
      const u32 slot = atomicAdd(n, 1u);
      if (slot < cap) {
        if (kShared) st_agent(dst + slot, v[q]);
        else dst[slot] = v[q];
      }
    }
}

// The k largest of g[0..m) (all of them when fewer than k are nonzero) into dst, in no
// particular order, P keys per thread in registers; *cnt is zero on entry.  The number of
// registers is a template constant, so the caller picks the smallest P that holds m.
// kIn / kOut: g / dst are lists shared between workgroups (see small_load, small_gather).
template <bool kIn, bool kOut, u32 P>
__device__ __forceinline__ void small_keep(const u64* g, u32 m, u32 k, u64* dst, LdsSelect* L, u32* cnt) {
  u64 v[P];
  small_load<kIn>(v, g, m);
  // distinct nonzero keys: exactly k of them are at or above the k-th
  const u64 kth = reg_select_desc(v, k, L);
  small_gather<kOut>(v, kth, dst, k, cnt);
}

__global__ __launch_bounds__(kSmallThreads) void refine_small_kernel(RefineArgs a, u32 G) {
  __shared__ LdsSelect s_sel;
  __shared__ u64 s_top[kSmallK];
  __shared__ u32 s_n, s_last;
  const u32 tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  if (blockIdx.x >= G) {  // leave the sampler's hash set zero for the next attempt
    uint4* t = reinterpret_cast<uint4*>(a.table);
    const u64 words = a.table_slots / 4, gs = (u64)(gridDim.x - G) * kSmallThreads;
    for (u64 i = (u64)(blockIdx.x - G) * kSmallThreads + tid; i < words; i += gs) t[i] = make_uint4(0, 0, 0, 0);
    return;
  }
  const RowCtl* c = a.ctl;
  if (blockIdx.x == 0 && tid == 0) {
    if (a.rec) a.rec->generic = 0;
    publish(a, c, 0u);
  }
  const bool live = refine_live(a, c);
  const u64 n = live ? cand_count(c, a.M) : 0;
  const u32 k = (u32)a.k;
  if (a.approx) {
    const u64 gt = (u64)blockIdx.x * kSmallThreads + tid, gs = (u64)G * kSmallThreads;
    if (gt == 0 && a.info) {
      a.info->R = (int64_t)c->R;
      a.info->M = (int64_t)a.M;
      a.info->status = (int32_t)c->status;
      a.info->exact_path = 0;
    }
    for (u64 p = n + gt; p < a.k; p += gs) {
      a.out_idx[p] = -1;
      reinterpret_cast<u32*>(a.out_vals)[p] = 0xFF800000u;  // -inf
    }
  }
  if (!live) return;
  if (n <= kSmallShare) {
    // every candidate fits one workgroup's registers (the usual case: R is mostly well
    // below M): workgroup 0 selects and sorts alone, with no lists, no hand-off and no
    // second select; the election counter is left untouched (zero)
    if (blockIdx.x != 0) return;
    if (tid == 0) s_n = 0;
    __syncthreads();
    if (n <= 4 * kSmallThreads) small_keep<false, false, 4>(a.cand, (u32)n, k, s_top, &s_sel, &s_n);
    else small_keep<false, false, kSmallPer>(a.cand, (u32)n, k, s_top, &s_sel, &s_n);
    __syncthreads();
    const u32 nt1 = s_n < k ? s_n : k;
    if (wid == 0) {
      const u64 key = wave_sort_desc(lane < nt1 ? s_top[lane] : 0ull);
      if (lane < nt1) write_out(a, lane, key);
    }
    return;
  }
  // this workgroup's share (at most kSmallShare: the grid is sized to M) and its k largest
  const u64 per = (n + G - 1) / G;
  const u64 lo = (u64)blockIdx.x * per < n ? (u64)blockIdx.x * per : n;
  const u32 m = (u32)((lo + per < n ? lo + per : n) - lo);
  if (tid == 0) s_n = 0;
  __syncthreads();
  {
    u64* list = a.tmp + (u64)blockIdx.x * k;
    if (m <= k) {
      for (u32 i = tid; i < k; i += kSmallThreads) st_agent(list + i, i < m ? a.cand[lo + i] : 0ull);
    } else if (m <= 4 * kSmallThreads) {
      small_keep<false, true, 4>(a.cand + lo, m, k, list, &s_sel, &s_n);
    } else {
      small_keep<false, true, kSmallPer>(a.cand + lo, m, k, list, &s_sel, &s_n);
    }
  }
  // every thread's list stores complete; then elect the last workgroup
  drain_memory_ops();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(a.ticket, 1u) == G - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) s_n = 0;
  // the k-th largest of the union; with fewer than k candidates (approximate mode) all
  const u32 nl = G * k;  // <= kSmallLists: the grid is sized for it
  if (nl <= 4 * kSmallThreads) small_keep<true, false, 4>(a.tmp, nl, k, s_top, &s_sel, &s_n);
  else if (nl <= kSmallPer * kSmallThreads) small_keep<true, false, kSmallPer>(a.tmp, nl, k, s_top, &s_sel, &s_n);
  else small_keep<true, false, kSmallLists / kSmallThreads>(a.tmp, nl, k, s_top, &s_sel, &s_n);
  __syncthreads();
  const u32 nt = s_n < k ? s_n : k;
  if (wid == 0) {
    const u64 key = wave_sort_desc(lane < nt ? s_top[lane] : 0ull);
    if (lane < nt) write_out(a, lane, key);
  }
  if (tid == 0) atomic_store_agent(a.ticket, 0u);
}

__global__ void approx_info_exact_kernel(ApproxInfo* info, u64 N) {
  if (threadIdx.x == 0) {
    info->R = (int64_t)N;
    info->M = 0;
    info->status = 0;
    info->exact_path = 1;
  }
}

hipError_t launch_approx_info_exact(ApproxInfo* info, u64 N, hipStream_t s) {
  approx_info_exact_kernel<<<1, 64, 0, s>>>(info, N);
  return hipGetLastError();
}

bool refine_one_launch(const RefineArgs& a) {
  // small k: one launch, when the union of the workgroups' lists fits in LDS
  const u64 gsm = (a.M + kSmallShare - 1) / kSmallShare;
  return a.k <= kSmallK && gsm * a.k <= kSmallLists;
}

hipError_t launch_refine(const RefineArgs& a, hipStream_t s) {
  const u64 gsm = (a.M + kSmallShare - 1) / kSmallShare;
  if (refine_one_launch(a)) {
    const u32 G = (u32)(gsm ? gsm : 1);
    const u64 words = a.table ? a.table_slots / 4 : 0;  // slots: a power of two >= 16
    const u64 z = (words + kClearPerBlock - 1) / kClearPerBlock;
    refine_small_kernel<<<G + (u32)(z < 256 ? z : 256), kSmallThreads, 0, s>>>(a, G);
    return hipGetLastError();
  }
  // the bin sort: four workgroups per CU, and enough wavefronts for chunks of at most
  // kChunkKeys keys (the needed bins hold T <= M keys, and T < k + msd_cap, since a
  // needed bin beyond msd_cap keys takes the multi-pass refinement)
  const u64 tmax = a.k + (u64)a.msd_cap < a.M ? a.k + a.msd_cap : a.M;
  u64 gs = 4ull * device_cu_count();
  if (gs > kSortBlocksCap) gs = kSortBlocksCap;
  const u64 gneed = (tmax + 4ull * kChunkKeys - 1) / (4ull * kChunkKeys);
  if (gs < gneed) gs = gneed;
  RefineArgs b = a;
  b.sort_waves = (u32)(4 * gs);
  // about 4 candidates per thread at R = M (R is mostly well below M): more blocks keep
  // more candidate loads in flight, but each adds its nonzero bins to the global
  // histogram and reserves its runs with atomics (measured on MI355X over 2^30 Pareto
  // values, k = 2^5..2^19: 64..128 blocks best, 512 worse than 32)
  u32 gh = (u32)((a.M + 4095) / 4096);
  if (gh < 1) gh = 1;
  if (gh > 128) gh = 128;
  if (a.approx) {
    refine_hist_kernel<<<gh, kHistThreads, 0, s>>>(b);
    refine_scatter_kernel<<<gh, kHistThreads, 0, s>>>(b);
  } else {
    // one block per two CUs at most: every block of the fused launch is resident
    u32 half = device_cu_count() / 2;
#ifdef PROFK_BIN_GRID
    if (half > PROFK_BIN_GRID) half = PROFK_BIN_GRID;
#endif
    if (gh > half) gh = half > 0 ? half : 1;
    refine_bin_kernel<<<gh, kHistThreads, 0, s>>>(b);
  }
  refine_binsort_kernel<<<(u32)gs, kSortThreads, 0, s>>>(b);
  return hipGetLastError();
}

}  // namespace profk
