// Stage 4 of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
// Selection", §3 stage 4): the exact top-k of the R buffered candidates, sorted.
// The pages call a library top-k here (App. C); this is a binned refinement for
// gfx950 that takes three launches whatever k is:
//
//   refine_hist_kernel     histogram of the candidates over kBins equal bins of the
//                          key range [tau, cmax] (cmax = the largest candidate key,
//                          tracked by the filter).  The last block scans the bins
//                          from the top: the bin b* that holds the k-th largest
//                          candidate, the candidates above it, and the output
//                          offset of every bin >= b*.  If one of those bins holds
//                          more keys than one workgroup sorts in LDS (ties,
//                          narrow-range inputs), it marks the row for the
//                          multi-pass refinement instead.
//   refine_scatter_kernel  writes the candidates of bins >= b* into bin order.
//   refine_binsort_kernel  sorts every bin >= b* in LDS (four 256-thread workgroups
//                          per CU) and writes out_vals / out_idx for positions < k.
// Bins partition the keys by value, so sorted bins laid out from the top bin down
// are the sorted candidates; positions < k are the exact top-k in order.
#include "block_select.h"
#include "launch.h"

namespace profk {

namespace {
constexpr u32 kHistThreads = 1024;
constexpr u32 kSortThreads = 256;

__device__ __forceinline__ u32 bin_of(u64 key, u64 tau, u32 shift) {
  const u64 b = (key - tau) >> shift;
  return b < kBins ? (u32)b : kBins - 1u;
}

__device__ __forceinline__ u64 cand_count(const RowCtl* c, u64 M) { return c->R < M ? c->R : M; }
}  // namespace

__global__ __launch_bounds__(kHistThreads) void refine_hist_kernel(RefineArgs a) {
  __shared__ u32 s_h[kBins];
  __shared__ u32 s_part[kHistThreads];
  __shared__ u32 s_last;
  RowCtl* c = a.ctl;
  if (c->status != 0) return;
  const u64 n = cand_count(c, a.M);
  const u64 tau = c->tau;
  const u64 range = c->cmax - tau;
  const u32 shift = range < kBins ? 0u : (u32)(64 - __clzll((long long)range)) - kBinBits;
  for (u32 b = threadIdx.x; b < kBins; b += blockDim.x) s_h[b] = 0;
  __syncthreads();
  const u64 stride = (u64)gridDim.x * blockDim.x;
  for (u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    atomicAdd(&s_h[bin_of(a.cand[i], tau, shift)], 1u);
  __syncthreads();
  for (u32 b = threadIdx.x; b < kBins; b += blockDim.x)
    if (s_h[b]) atomicAdd(&a.hist[b], s_h[b]);
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    s_last = (atomicAdd(a.ticket, 1u) == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // Last block.  Thread t owns the kBins / kHistThreads bins counted from the top:
  // descending position q = kBins-1-b.  Suffix sums over descending positions give
  // each bin's output offset.
  constexpr u32 per = kBins / kHistThreads;
  u32 cnt[per];
  u32 sum = 0;
#pragma unroll
  for (u32 j = 0; j < per; ++j) {  // independent loads, all in flight together
    const u32 b = kBins - 1u - (threadIdx.x * per + j);
    cnt[j] = atomic_load_agent(&a.hist[b]);
  }
#pragma unroll
  for (u32 j = 0; j < per; ++j) {
    a.hist[kBins - 1u - (threadIdx.x * per + j)] = 0;  // left zero for the next call
    sum += cnt[j];
  }
  s_part[threadIdx.x] = sum;
  __syncthreads();
  for (u32 off = 1; off < kHistThreads; off <<= 1) {  // inclusive scan of the parts
    const u32 v = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0u;
    __syncthreads();
    s_part[threadIdx.x] += v;
    __syncthreads();
  }
  u32 run = threadIdx.x ? s_part[threadIdx.x - 1] : 0u;  // keys in the bins above this thread's
  if (threadIdx.x == 0) {
    s_h[0] = 0xFFFFFFFFu;  // b* (as a descending position)
    s_h[1] = 0;            // generic flag
  }
  __syncthreads();
  const u64 k = a.k;
  u32 offs[per];
#pragma unroll
  for (u32 j = 0; j < per; ++j) {
    const u32 q = threadIdx.x * per + j;
    offs[j] = run;
    if (run < k && run + cnt[j] >= k) {  // exactly one bin holds the k-th largest
      s_h[0] = q;
      c->bstar = kBins - 1u - q;
      c->c_above = run;
    }
    run += cnt[j];
  }
  __syncthreads();
  const u32 qstar = s_h[0];
  // offsets and counts are read only for the bins at or above b*
#pragma unroll
  for (u32 j = 0; j < per; ++j) {
    const u32 q = threadIdx.x * per + j;
    if (q <= qstar) {
      const u32 b = kBins - 1u - q;
      a.bin_off[b] = offs[j];
      a.bin_cnt[b] = cnt[j];
      a.cursor[b] = 0;
    }
  }
  // every bin at or above b* must fit one sorting workgroup
  bool big = qstar == 0xFFFFFFFFu;
#pragma unroll
  for (u32 j = 0; j < per; ++j) {
    const u32 q = threadIdx.x * per + j;
    if (q <= qstar && cnt[j] > kBinCap) big = true;
  }
  if (big) s_h[1] = 1;
  __syncthreads();
  if (threadIdx.x == 0) {
    c->bin_shift = shift;
    c->generic = s_h[1];
    if (a.rec) a.rec->generic = s_h[1];
    *a.ticket = 0;
  }
}

// Each block owns a contiguous range of candidates: it counts them per bin in LDS,
// reserves each (block, bin) run with ONE global atomic, then places its keys with
// LDS atomics.
constexpr u32 kScatterThreads = 1024;
__global__ __launch_bounds__(kScatterThreads) void refine_scatter_kernel(RefineArgs a) {
  __shared__ u32 s_pos[kBins];
  const RowCtl* c = a.ctl;
  if (c->status != 0 || c->generic) return;
  const u64 n = cand_count(c, a.M);
  const u64 tau = c->tau;
  const u32 shift = c->bin_shift, bstar = c->bstar;
  const u64 per = (n + gridDim.x - 1) / gridDim.x;
  const u64 lo = (u64)blockIdx.x * per;
  const u64 hi = lo + per < n ? lo + per : n;
  for (u32 b = threadIdx.x; b < kBins; b += blockDim.x) s_pos[b] = 0;
  __syncthreads();
  for (u64 i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const u32 b = bin_of(a.cand[i], tau, shift);
    if (b >= bstar) atomicAdd(&s_pos[b], 1u);
  }
  __syncthreads();
  for (u32 b = threadIdx.x; b < kBins; b += blockDim.x) {
    const u32 cnt = s_pos[b];
    if (cnt) s_pos[b] = a.bin_off[b] + atomicAdd(&a.cursor[b], cnt);
  }
  __syncthreads();
  for (u64 i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const u64 key = a.cand[i];
    const u32 b = bin_of(key, tau, shift);
    if (b >= bstar) {
      const u32 pos = atomicAdd(&s_pos[b], 1u);
      if (pos < a.M) a.tmp[pos] = key;
    }
  }
}

__global__ __launch_bounds__(kSortThreads) void refine_binsort_kernel(RefineArgs a) {
  __shared__ u64 s[kBinCap];
  const RowCtl* c = a.ctl;
  if (c->status != 0 || c->generic) return;
  const int bstar = (int)c->bstar;
  const u64 k = a.k;
  for (int b = (int)kBins - 1 - (int)blockIdx.x; b >= bstar; b -= (int)gridDim.x) {
    const u32 cnt = a.bin_cnt[b];
    const u32 start = a.bin_off[b];
    if (cnt == 0 || start >= k || cnt > kBinCap || start + (u64)cnt > a.M) continue;  // uniform per workgroup
    u32 P = 1;
    while (P < cnt) P <<= 1;
    __syncthreads();
    for (u32 i = threadIdx.x; i < P; i += blockDim.x) s[i] = i < cnt ? a.tmp[start + i] : 0ull;
    __syncthreads();
    block_bitonic_desc(s, P);
    const u64 lim = k - start < cnt ? k - start : cnt;
    for (u32 i = threadIdx.x; i < lim; i += blockDim.x) {
      const u32 idx = key_index(s[i]);
      const u64 p = start + i;
      a.out_idx[p] = idx < a.N ? (int64_t)idx : -1;
      if (idx < a.N) reinterpret_cast<u32*>(a.out_vals)[p] = reinterpret_cast<const u32*>(a.x)[idx];
    }
  }
}

hipError_t launch_refine(const RefineArgs& a, hipStream_t s) {
  u32 gh = (u32)((a.M + 16383) / 16384);  // about 16 candidates per thread
  if (gh < 1) gh = 1;
  if (gh > 32) gh = 32;  // each block adds its nonzero bins to the global histogram
  refine_hist_kernel<<<gh, kHistThreads, 0, s>>>(a);
  refine_scatter_kernel<<<gh, kScatterThreads, 0, s>>>(a);
  refine_binsort_kernel<<<4 * device_cu_count(), kSortThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace profk
