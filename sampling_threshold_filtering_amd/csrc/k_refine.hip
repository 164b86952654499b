// Stage 4 of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
// Selection", §3 stage 4): the exact top-k of the R buffered candidates, sorted.
// The pages call a library top-k here (App. C).  For k <= kSmallK one launch does it
// (refine_small_kernel, below: per-workgroup top-k lists and a select over their union
// by the last workgroup).  Larger k take a binned refinement for gfx950 in three
// launches:
//
//   refine_hist_kernel     histogram of the candidates over kBins equal bins of the
//                          key range [tau, cmax] (cmax = the largest candidate key,
//                          tracked by the filter), added into a global histogram.
//   refine_scatter_kernel  every block scans the global histogram from the top bin
//                          down in LDS: the bin b* that holds the k-th largest
//                          candidate and the output offset of every bin >= b*
//                          (block 0 publishes them).  If one of those bins holds more
//                          keys than one workgroup sorts in LDS (ties, narrow-range
//                          inputs), the row is marked for the multi-pass refinement
//                          instead.  Otherwise each block writes its candidates of
//                          bins >= b* into bin order: one global atomic per (block,
//                          bin) reserves the run, LDS atomics place the keys.  Block 0
//                          also publishes the attempt record (R, check, multi-pass
//                          flag) to the host, which needs nothing later to decide.
//   refine_binsort_kernel  sorts every bin >= b* (four 256-thread workgroups per CU:
//                          one wavefront in registers up to kWaveMax keys, a workgroup
//                          up to kBinCap by one 8-bit counting pass in LDS) and writes
//                          out_vals / out_idx for positions < k.  A larger bin (large
//                          tie groups, narrow ranges) is partitioned by one workgroup
//                          on successive 12-bit digits of (key - tau), from the top
//                          down, until every part that reaches a position below k fits
//                          those sorts.  It also leaves the histogram and the
//                          sampler's hash set zero for the next attempt.
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

__global__ __launch_bounds__(kHistThreads) void refine_scatter_kernel(RefineArgs a) {
  __shared__ u32 s_off[kBins + kBins / kPer + 1];  // by padded descending position; last = total
  __shared__ u32 s_pos[kBins];
  __shared__ u32 s_wsum[kHistThreads / kWave];
  __shared__ u32 s_q, s_big;
  RowCtl* c = a.ctl;
  if (!refine_live(a, c)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) publish(a, c, 0u);
    return;
  }
  const u32 tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const u64 n = cand_count(c, a.M);
  const u64 tau = c->tau;
  const u32 shift = bin_shift_of(c);
  {
    u32 v[kPer];  // all loads in flight, then the LDS stores
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) v[j] = a.hist[j * kHistThreads + tid];
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) s_off[pad_q(kBins - 1u - (j * kHistThreads + tid))] = v[j];
  }
  if (tid == 0) {
    s_q = 0xFFFFFFFFu;
    s_big = 0;
  }
  __syncthreads();
  // exclusive offsets over descending positions: thread tid owns q = tid*kPer + j
  u32 cnt[kPer];
  u32 sum = 0;
#pragma unroll
  for (u32 j = 0; j < kPer; ++j) {
    cnt[j] = s_off[pad_q(tid * kPer + j)];
    sum += cnt[j];
  }
  u32 incl = sum;
#pragma unroll
  for (u32 d = 1; d < (u32)kWave; d <<= 1) {
    const u32 v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) s_wsum[wid] = incl;
  __syncthreads();
  u32 run = incl - sum;
  for (u32 w = 0; w < wid; ++w) run += s_wsum[w];
  const u64 k = a.k;
#pragma unroll
  for (u32 j = 0; j < kPer; ++j) {
    const u32 q = tid * kPer + j;
    s_off[pad_q(q)] = run;
    if (run < k && run + cnt[j] >= k) s_q = q;  // exactly one bin holds the k-th largest
    run += cnt[j];
  }
  if (tid == blockDim.x - 1) s_off[pad_q(kBins)] = run;
  __syncthreads();
  // fewer than k candidates (approximate mode only): every bin is needed
  const u32 qstar = s_q == 0xFFFFFFFFu && a.approx ? kBins - 1u : s_q;
  // every bin at or above b* must fit the in-kernel sorts and partition
  bool big = qstar == 0xFFFFFFFFu;
#pragma unroll
  for (u32 j = 0; j < kPer; ++j)
    if (tid * kPer + j <= qstar && cnt[j] > a.msd_cap) big = true;
  if (big) s_big = 1;
  __syncthreads();
  const bool generic = s_big != 0;
  if (blockIdx.x == 0) {
    if (!generic)
      for (u32 q = tid; q <= qstar; q += blockDim.x) {
        const u32 b = kBins - 1u - q;
        a.bin_off[b] = s_off[pad_q(q)];
        a.bin_cnt[b] = s_off[pad_q(q + 1)] - s_off[pad_q(q)];
      }
    if (tid == 0) {
      c->bin_shift = shift;
      c->bstar = generic ? 0u : kBins - 1u - qstar;
      c->c_above = generic ? 0u : s_off[pad_q(qstar)];
      c->generic = generic ? 1u : 0u;
      if (a.rec) a.rec->generic = generic ? 1u : 0u;
      publish(a, c, generic ? 1u : 0u);
    }
  }
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

// Bin q (descending position; bin kBins - 1 - q) belongs to workgroup q mod G, and
// within it to wavefront (q / G) mod 4: the heavy bins, which are neighbours (next to
// tau on skewed inputs), go to different workgroups.  Bins of up to kWaveMax keys are
// sorted by their wavefront in registers; larger ones by the whole workgroup, after
// its wavefronts are done: the counting pass above up to kBinCap keys, else the
// partition by 12-bit digits.
constexpr u32 kPrefetch = 4;  // bins whose extent a wavefront loads at once

__global__ __launch_bounds__(kSortThreads) void refine_binsort_kernel(RefineArgs a) {
  __shared__ u64 s[kBinCap];
  __shared__ u32 s_big[kSortThreads];
  __shared__ u32 s_nbig;
  __shared__ MsdLds s_msd;
  __shared__ HeavyLds s_heavy;
  {  // leave the histogram and the sampler's hash set zero for the next attempt
    const u64 gt = (u64)blockIdx.x * blockDim.x + threadIdx.x, gs = (u64)gridDim.x * blockDim.x;
    for (u64 i = gt; i < kBins; i += gs) a.hist[i] = 0;
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
  const u32 qmax = kBins - 1u - c->bstar;
  const u64 k = a.k;
  const u32 lane = lane_id();
  const u32 wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  constexpr u32 kWaves = kSortThreads / kWave;
  const u32 G = gridDim.x;
  if (threadIdx.x == 0) s_nbig = 0;
  __syncthreads();
  for (u32 i = wid; blockIdx.x + (u64)G * i <= qmax; i += kWaves * kPrefetch) {
    u32 cnt[kPrefetch], start[kPrefetch], bin[kPrefetch];
#pragma unroll
    for (u32 r = 0; r < kPrefetch; ++r) {  // unconditional loads, all in flight
      const u64 q = blockIdx.x + (u64)G * (i + kWaves * r);
      bin[r] = q <= qmax ? kBins - 1u - (u32)q : kBins;
      const u32 bl = bin[r] < kBins ? bin[r] : kBins - 1u;
      cnt[r] = a.bin_cnt[bl];
      start[r] = a.bin_off[bl];
    }
    // the keys of every light bin of the group in flight before the first sort
    static_assert(kWaveMax <= 4 * kWave, "light bins take at most 4 keys per lane");
    u64 v[kPrefetch][4];
    u32 n[kPrefetch];
#pragma unroll
    for (u32 r = 0; r < kPrefetch; ++r) {
      n[r] = bin[r] < kBins ? cnt[r] : 0u;
      if (start[r] >= k || start[r] + (u64)n[r] > a.M) n[r] = 0;  // uniform per wavefront
      const bool light = n[r] <= kWaveMax;
#pragma unroll
      for (u32 j = 0; j < 4; ++j) {
        const u32 e = j * kWave + lane;
        v[r][j] = light && e < n[r] ? a.tmp[start[r] + e] : 0ull;
      }
    }
#pragma unroll
    for (u32 r = 0; r < kPrefetch; ++r) {
      if (n[r] == 0) continue;
      if (n[r] > kWaveMax) {
        if (lane == 0) s_big[atomicAdd(&s_nbig, 1u)] = bin[r];  // the block meets at most kSortThreads bins
        continue;
      }
      if (n[r] <= kWave) light_sort<1>(a, v[r], n[r], start[r]);
      else if (n[r] <= 2 * kWave) light_sort<2>(a, v[r], n[r], start[r]);
      else light_sort<4>(a, v[r], n[r], start[r]);
    }
  }
  __syncthreads();
  const u32 nbig = s_nbig;
  const u64 tau = c->tau;
  const u32 width = c->bin_shift;
  const u32 sub = width > 8u ? width - 8u : 0u;
  for (u32 q = 0; q < nbig; ++q) {
    const u32 b = s_big[q];
    const u32 cnt = a.bin_cnt[b];
    const u32 start = a.bin_off[b];
    if (cnt <= kBinCap)
      heavy_part(a, s, &s_heavy, start, cnt, tau, sub);
    else
      msd_bin(a, s, b, start, cnt, width, tau, &s_msd);
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
  // about 4 candidates per thread at R = M (R is mostly well below M): more blocks keep
  // more candidate loads in flight, but each adds its nonzero bins to the global
  // histogram and reserves its runs with atomics (measured on MI355X over 2^30 Pareto
  // values, k = 2^5..2^19: 64..128 blocks best, 512 worse than 32)
  u32 gh = (u32)((a.M + 4095) / 4096);
  if (gh < 1) gh = 1;
  if (gh > 128) gh = 128;
  refine_hist_kernel<<<gh, kHistThreads, 0, s>>>(a);
  refine_scatter_kernel<<<gh, kHistThreads, 0, s>>>(a);
  // at least 64 workgroups: a workgroup then owns at most kBins / 64 = kSortThreads
  // bins (s_big)
  u32 gs = 4 * device_cu_count();
  if (gs < 64) gs = 64;
  refine_binsort_kernel<<<gs, kSortThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace profk
