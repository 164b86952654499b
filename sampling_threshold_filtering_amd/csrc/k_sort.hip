// Final ordering of the k selected keys (descending composite key = value
// descending, then lower index first) and the output write.
//
// The pages hand the buffer to a library top-k (torch.topk, "Prof-K:
// Probabilistic One-Pass Filtering for Efficient Top-k Selection", App. C), which
// returns sorted values; the output here is sorted the same way.
//
//   * k <= kSmallSort: one workgroup, bitonic sort in LDS (64 KB), writes outputs.
//   * larger k: LSD radix sort with 8-bit digits across blocks, three launches per
//     digit (per-block digit counts; one-block scan; stable scatter with
//     wavefront match-ranking), skipping every digit that is equal across all
//     k keys (known from the OR / AND folded by the compaction); then the output
//     write.  The buffer a pass reads is the parity of the varying digits below
//     it, so skipped digits cost nothing but an early return.
#include "launch.h"

namespace profk {

namespace {
constexpr int kSortThreads = 256;
constexpr int kSortItems = 8;
constexpr u32 kSortTile = kSortThreads * kSortItems;  // keys per block

__device__ __forceinline__ bool digit_varies(const RowCtl* c, u32 d) {
  return (((c->key_or ^ c->key_and) >> (8u * d)) & 0xFFull) != 0;
}

// Which ping-pong buffer holds the keys before digit d is processed: every digit
// that varies moves them once, the others are skipped.
__device__ __forceinline__ u32 buffer_before(const RowCtl* c, u32 d) {
  u32 moves = 0;
  for (u32 i = 0; i < d; ++i) moves += digit_varies(c, i) ? 1u : 0u;
  return moves & 1u;
}

__device__ __forceinline__ void write_one(const u64 key, u64 i, const float* row, u64 N, float* out_vals,
                                          int64_t* out_idx) {
  const u32 idx = key_index(key);
  out_idx[i] = idx < N ? (int64_t)idx : -1;
  if (idx < N) reinterpret_cast<u32*>(out_vals)[i] = reinterpret_cast<const u32*>(row)[idx];  // bit copy
}
}  // namespace

__global__ __launch_bounds__(1024) void sort_small_kernel(const u64* __restrict__ keys, u32 k, const float* row,
                                                          u64 N, float* out_vals, int64_t* out_idx, RowCtl* ctl,
                                                          AttemptRecord* rec) {
  __shared__ u64 s[kSmallSort];
  if (ctl->status != 0) {
    if (threadIdx.x == 0 && rec) rec->status = ctl->status;
    return;
  }
  if (ctl->nsel != k) {
    if (threadIdx.x == 0 && rec) rec->error = 1;
    return;
  }
  u32 P = 1;
  while (P < k) P <<= 1;
  for (u32 i = threadIdx.x; i < P; i += blockDim.x) s[i] = i < k ? keys[i] : 0ull;
  __syncthreads();
  for (u32 kk = 2; kk <= P; kk <<= 1) {
    for (u32 j = kk >> 1; j > 0; j >>= 1) {
      for (u32 i = threadIdx.x; i < P; i += blockDim.x) {
        const u32 ixj = i ^ j;
        if (ixj > i) {
          const u64 a = s[i], b = s[ixj];
          const bool up = (i & kk) == 0;
          if (up ? (a < b) : (a > b)) {
            s[i] = b;
            s[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (u32 i = threadIdx.x; i < k; i += blockDim.x) write_one(s[i], i, row, N, out_vals, out_idx);
}

// Per-block counts of the (descending) digit d: hist[dd * G + b].
__global__ __launch_bounds__(kSortThreads) void lsd_hist_kernel(u64* buf0, u64* buf1, u32 n, u32 d, u32* hist,
                                                                const RowCtl* ctl) {
  __shared__ u32 s_h[256];
  if (ctl->status != 0 || !digit_varies(ctl, d)) return;
  const u64* src = buffer_before(ctl, d) ? buf1 : buf0;
  for (u32 b = threadIdx.x; b < 256; b += blockDim.x) s_h[b] = 0;
  __syncthreads();
  const u32 lo = blockIdx.x * kSortTile;
  u64 keys[kSortItems];
#pragma unroll
  for (u32 c = 0; c < kSortItems; ++c) {  // all loads in flight before any ballot
    const u32 i = lo + c * kSortThreads + threadIdx.x;
    keys[c] = i < n ? src[i] : 0ull;
  }
#pragma unroll
  for (u32 c = 0; c < kSortItems; ++c) {
    const u32 i = lo + c * kSortThreads + threadIdx.x;
    const bool in = i < n;
    const u32 dd = in ? 255u - (u32)((keys[c] >> (8u * d)) & 0xFFu) : 0u;
    wave_hist_add(s_h, dd, in);
  }
  __syncthreads();
  const u32 G = gridDim.x;
  for (u32 b = threadIdx.x; b < 256; b += blockDim.x) hist[b * G + blockIdx.x] = s_h[b];
}

// Exclusive scan over (digit, block) in digit-major order: hist -> offsets.  The
// digit-major layout makes this one exclusive scan of the 256*G words in array
// order: each thread scans a contiguous run, the run totals are scanned in LDS.
constexpr int kScanThreads = 1024;
constexpr u32 kScanRegWords = 64;  // runs up to this many words stay in registers
__global__ __launch_bounds__(kScanThreads) void lsd_scan_kernel(u32* hist, u32 G, u32 d, const RowCtl* ctl) {
  __shared__ u32 s_tot[kScanThreads];
  if (ctl->status != 0 || !digit_varies(ctl, d)) return;
  // Each thread's run is a whole number of 16-word groups (256 * G is a multiple
  // of 256), read as uint4 so that all of a thread's loads are in flight at once.
  const u32 total = 256u * G;
  const u32 per = ((total + kScanThreads - 1) / kScanThreads + 15u) & ~15u;
  const u32 lo = threadIdx.x * per < total ? threadIdx.x * per : total;
  const u32 hi = lo + per < total ? lo + per : total;
  if (per <= kScanRegWords) {
    // the thread's run (at most kScanRegWords words) loaded at once and kept in
    // registers for the rewrite: one round trip each way
    uint4 q[kScanRegWords / 4];
#pragma unroll
    for (u32 j = 0; j < kScanRegWords / 4; ++j)
      q[j] = lo + 4 * j < hi ? reinterpret_cast<const uint4*>(hist + lo)[j] : make_uint4(0, 0, 0, 0);
    u32 run = 0;
#pragma unroll
    for (u32 j = 0; j < kScanRegWords / 4; ++j) run += q[j].x + q[j].y + q[j].z + q[j].w;
    // exclusive scan of the run totals: within each wavefront by DPP, then over the
    // sixteen wavefront totals
    const u32 lane = lane_id(), w = threadIdx.x / kWave;
    const u32 incl = wave_incl_scan_add(run, lane);
    if (lane == kWave - 1) s_tot[w] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
      u32 a = 0;
      for (u32 i = 0; i < kScanThreads / kWave; ++i) {
        const u32 t = s_tot[i];
        s_tot[i] = a;
        a += t;
      }
    }
    __syncthreads();
    u32 acc = s_tot[w] + incl - run;
#pragma unroll
    for (u32 j = 0; j < kScanRegWords / 4; ++j) {
      const uint4 c = q[j];
      uint4 o;
      o.x = acc;
      o.y = acc + c.x;
      o.z = acc + c.x + c.y;
      o.w = acc + c.x + c.y + c.z;
      acc += c.x + c.y + c.z + c.w;
      if (lo + 4 * j < hi) reinterpret_cast<uint4*>(hist + lo)[j] = o;
    }
    return;
  }
  u32 run = 0;
  for (u32 i = lo; i < hi; i += 16) {
    const uint4* p = reinterpret_cast<const uint4*>(hist + i);
    const uint4 a = p[0], b = p[1], c = p[2], e = p[3];
    run += a.x + a.y + a.z + a.w + b.x + b.y + b.z + b.w + c.x + c.y + c.z + c.w + e.x + e.y + e.z + e.w;
  }
  s_tot[threadIdx.x] = run;
  __syncthreads();
  // Hillis-Steele inclusive scan of the run totals
  for (u32 off = 1; off < kScanThreads; off <<= 1) {
    const u32 v = threadIdx.x >= off ? s_tot[threadIdx.x - off] : 0u;
    __syncthreads();
    s_tot[threadIdx.x] += v;
    __syncthreads();
  }
  u32 acc = threadIdx.x ? s_tot[threadIdx.x - 1] : 0u;
  for (u32 i = lo; i < hi; i += 16) {
    uint4* p = reinterpret_cast<uint4*>(hist + i);
    uint4 q[4] = {p[0], p[1], p[2], p[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 c = q[j];
      q[j].x = acc;
      q[j].y = acc + c.x;
      q[j].z = acc + c.x + c.y;
      q[j].w = acc + c.x + c.y + c.z;
      acc += c.x + c.y + c.z + c.w;
    }
    p[0] = q[0];
    p[1] = q[1];
    p[2] = q[2];
    p[3] = q[3];
  }
}

// Stable scatter of digit d.
__global__ __launch_bounds__(kSortThreads) void lsd_scatter_kernel(u64* buf0, u64* buf1, u32 n, u32 d,
                                                                   const u32* hist, const RowCtl* ctl) {
  __shared__ u32 s_run[256];
  __shared__ u32 s_cnt[kSortThreads / kWave][256];
  if (ctl->status != 0 || !digit_varies(ctl, d)) return;
  const u32 cur = buffer_before(ctl, d);
  const u64* src = cur ? buf1 : buf0;
  u64* dst = cur ? buf0 : buf1;
  const u32 w = threadIdx.x / kWave;
  const u32 G = gridDim.x;
  for (u32 b = threadIdx.x; b < 256; b += blockDim.x) {
    s_run[b] = hist[b * G + blockIdx.x];
    for (u32 ww = 0; ww < kSortThreads / kWave; ++ww) s_cnt[ww][b] = 0;
  }
  __syncthreads();
  const u32 lo = blockIdx.x * kSortTile;
  u64 keys[kSortItems];
#pragma unroll
  for (u32 c = 0; c < kSortItems; ++c) {  // all loads in flight before any ballot
    const u32 i = lo + c * kSortThreads + threadIdx.x;
    keys[c] = i < n ? src[i] : 0ull;
  }
#pragma unroll
  for (u32 c = 0; c < kSortItems; ++c) {
    const u32 i = lo + c * kSortThreads + threadIdx.x;
    const bool in = i < n;
    const u64 key = keys[c];
    const u32 dd = in ? 255u - (u32)((key >> (8u * d)) & 0xFFu) : 0u;
    const u64 same = wave_match8(dd, in);
    const u32 r = count_below(same);
    if (in && r == 0) s_cnt[w][dd] = (u32)__popcll(same);
    __syncthreads();
    // per digit: offsets of each wave's group inside the running position
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x) {
      u32 acc = s_run[b];
      for (u32 ww = 0; ww < kSortThreads / kWave; ++ww) {
        const u32 cc = s_cnt[ww][b];
        s_cnt[ww][b] = acc;
        acc += cc;
      }
      s_run[b] = acc;
    }
    __syncthreads();
    const u32 pos = s_cnt[w][dd] + r;
    if (in && pos < n) dst[pos] = key;
    __syncthreads();
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x)
      for (u32 ww = 0; ww < kSortThreads / kWave; ++ww) s_cnt[ww][b] = 0;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void write_outputs_kernel(u64* buf0, u64* buf1, u32 k, const float* row,
                                                            u64 N, float* out_vals, int64_t* out_idx, const RowCtl* ctl,
                                                            AttemptRecord* rec) {
  if (ctl->status != 0) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && rec) rec->status = ctl->status;
    return;
  }
  if (ctl->nsel != k) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && rec) rec->error = 1;
    return;
  }
  const u64* src = buffer_before(ctl, 8) ? buf1 : buf0;
  for (u32 i = blockIdx.x * blockDim.x + threadIdx.x; i < k; i += gridDim.x * blockDim.x)
    write_one(src[i], i, row, N, out_vals, out_idx);
}

hipError_t launch_sort_and_write(u64* buf0, u64* buf1, u32* hist, u32 k, const float* row, u64 N, float* out_vals,
                                 int64_t* out_idx, RowCtl* ctl, AttemptRecord* rec, hipStream_t s) {
  if (k <= kSmallSort) {
    sort_small_kernel<<<1, 1024, 0, s>>>(buf0, k, row, N, out_vals, out_idx, ctl, rec);
    return hipGetLastError();
  }
  const u32 G = (k + kSortTile - 1) / kSortTile;
  for (u32 d = 0; d < 8; ++d) {
    lsd_hist_kernel<<<G, kSortThreads, 0, s>>>(buf0, buf1, k, d, hist, ctl);
    lsd_scan_kernel<<<1, kScanThreads, 0, s>>>(hist, G, d, ctl);
    lsd_scatter_kernel<<<G, kSortThreads, 0, s>>>(buf0, buf1, k, d, hist, ctl);
  }
  u32 wg = (k + 255) / 256;
  if (wg > 4096) wg = 4096;
  write_outputs_kernel<<<wg, 256, 0, s>>>(buf0, buf1, k, row, N, out_vals, out_idx, ctl, rec);
  return hipGetLastError();
}

u64 sort_hist_words(u64 k) {
  const u64 G = (k + kSortTile - 1) / kSortTile;
  return 256ull * (G ? G : 1);
}

}  // namespace profk
