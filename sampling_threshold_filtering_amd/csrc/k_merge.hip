// Inputs of 2^32 values or more ("Prof-K: Probabilistic One-Pass Filtering for
// Efficient Top-k Selection", App. D, Table 4: inputs beyond 32-bit indexing, up to
// about 4.3e9 values and k = 2^22).
//
// The keys of the hot path carry a 32-bit index, so a longer input is cut into G
// contiguous segments of fewer than 2^32 values.  Each segment gets its own exact
// top-k (the whole sampled path, budget eps/G), which together still read the input
// once.  Every element of the global top-k is in the top-k of its own segment, so
// the global top-k is the top-k of the union of the G sorted lists; this kernel
// takes it exactly.
//
//   merge_segments_kernel  one thread per list entry.  Its rank in the union is its
//                          position in its own list plus, for every other list h, the
//                          number of entries of h that come before it: entries of a
//                          larger value, and, from a segment with lower indices
//                          (h < g), entries of equal value too (ties go to the lower
//                          global index).  Lists are sorted by value descending, so
//                          each count is one binary search.  Ranks in the union are
//                          distinct; entries of rank < k are written to their rank.
#include "launch.h"

namespace profk {

namespace {

__device__ __forceinline__ u32 ord_at(const float* v, u64 i) {
  return ord32(__float_as_uint(v[i]));
}

// Entries of list (v, n) whose order code is > o (strict) or >= o (!strict).
__device__ __forceinline__ u64 count_before(const float* v, u64 n, u32 o, bool strict) {
  u64 lo = 0, hi = n;  // the list is sorted by order code descending
  while (lo < hi) {
    const u64 mid = lo + ((hi - lo) >> 1);
    const u32 m = ord_at(v, mid);
    const bool before = strict ? (m > o) : (m >= o);
    if (before)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

}  // namespace

__global__ __launch_bounds__(256) void merge_segments_kernel(SegmentLists L, float* __restrict__ out_vals,
                                                             int64_t* __restrict__ out_idx) {
  const u64 total = (u64)L.G * L.stride;
  for (u64 e = (u64)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (u64)gridDim.x * blockDim.x) {
    const u32 g = (u32)(e / L.stride);
    const u64 p = e - (u64)g * L.stride;
    if (p >= L.len[g]) continue;
    const float* vg = L.vals + (u64)g * L.stride;
    const u32 o = ord_at(vg, p);
    u64 rank = p;
    for (u32 h = 0; h < L.G && rank < L.k; ++h) {
      if (h == g) continue;
      rank += count_before(L.vals + (u64)h * L.stride, L.len[h], o, h > g);
    }
    if (rank < L.k) {
      out_vals[rank] = vg[p];
      out_idx[rank] = L.idx[(u64)g * L.stride + p] + (int64_t)L.base[g];
    }
  }
}

hipError_t launch_merge_segments(const SegmentLists& L, float* out_vals, int64_t* out_idx, hipStream_t s) {
  const u64 total = (u64)L.G * L.stride;
  u64 blocks = (total + 255) / 256;
  const u64 cap = (u64)device_cu_count() * 8;
  if (blocks > cap) blocks = cap;
  if (blocks == 0) blocks = 1;
  merge_segments_kernel<<<(u32)blocks, 256, 0, s>>>(L, out_vals, out_idx);
  return hipGetLastError();
}

}  // namespace profk
