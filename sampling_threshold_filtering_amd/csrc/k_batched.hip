// Batched Prof-K: the same four stages applied to every row of a B x N matrix
// ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k Selection", §3:
// batched inputs are handled per row; App. C: per-row threshold, buffer and
// counter; App. E.2: the budget is split eps/B per row).
//
//   b_sample_kernel   one workgroup per row (persistent over the listed rows):
//                     the row's sample without replacement is tracked in an LDS
//                     bitmap of N bits (N <= 2^20: 128 KB), draws are made four at a
//                     time per thread, the keys go to a per-workgroup scratch, the
//                     top-digit histogram is built on the way, wavefront 0 tops the
//                     sample up, and the workgroup selects tau (LDS reused as the
//                     sort buffer).  It also clears the row's counter for the filter.
//   filter_kernel     (k_filter.hip) one streaming pass over all listed rows.
//   b_refine_kernel   one 256-thread workgroup per row: the min(R, M) <= 8192
//                     candidates are sorted in LDS (sized to M) and the first k
//                     written out.
//   b_rowsort_kernel  rows of at most 8192 values: exact top-k by sorting the row
//                     in LDS (the sample would not pay off there).
#include "block_select.h"
#include "launch.h"

namespace profk {

namespace {
constexpr u32 kBThreads = 1024;
constexpr u32 kBitmapWords = kBatchedMaxN / 32;  // 128 KB of LDS
constexpr u32 kDrawILP = 4;

__device__ __forceinline__ void write_row_out(u64 key, u64 j, const float* row, u64 N, float* ov, int64_t* oi) {
  const u32 idx = key_index(key);
  oi[j] = idx < N ? (int64_t)idx : -1;
  if (idx < N) reinterpret_cast<u32*>(ov)[j] = reinterpret_cast<const u32*>(row)[idx];
}
}  // namespace

__global__ __launch_bounds__(kBThreads) void b_sample_kernel(BatchedArgs a) {
  __shared__ u32 s_bits[kBitmapWords];
  __shared__ BlockSelectLds s_sel;
  __shared__ u32 s_D;
  __shared__ u32 s_fail;
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  u64* keys = a.scratch + (u64)blockIdx.x * a.S;
  const u32 nwords = (u32)((a.N + 31) / 32);
  for (u64 li = blockIdx.x; li < a.nrows; li += gridDim.x) {
    const u32 row = a.rows ? (u32)a.rows[li] : (u32)li;
    const float* xr = a.x + (u64)row * a.ld;
    __syncthreads();  // the previous row's users of s_bits / s_sel are done
    for (u32 w = threadIdx.x; w < nwords; w += blockDim.x) s_bits[w] = 0;
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x) s_sel.hist[b] = 0;
    if (threadIdx.x == 0) {
      s_D = 0;
      s_fail = 0;
    }
    __syncthreads();
    // draws 0..S-1, kDrawILP per thread per round
    const u64 span = (u64)blockDim.x * kDrawILP;
    for (u64 base = 0; base < a.S; base += span) {
      u32 idx[kDrawILP];
      bool fresh[kDrawILP];
#pragma unroll
      for (u32 q = 0; q < kDrawILP; ++q) {
        const u64 j = base + (u64)q * blockDim.x + threadIdx.x;
        fresh[q] = false;
        idx[q] = 0;
        if (j < a.S) {
          idx[q] = (u32)sample_draw(j, row, a.attempt, a.seed, a.N);
          const u32 bit = 1u << (idx[q] & 31u);
          fresh[q] = (atomicOr(&s_bits[idx[q] >> 5], bit) & bit) == 0;
        }
      }
      float v[kDrawILP];
#pragma unroll
      for (u32 q = 0; q < kDrawILP; ++q) v[q] = fresh[q] ? xr[idx[q]] : 0.f;  // gathers in flight together
#pragma unroll
      for (u32 q = 0; q < kDrawILP; ++q) {
        const u64 m = __ballot(fresh[q]);
        u32 slot = 0;
        if (m) {
          const u32 leader = __ffsll((long long)m) - 1;
          if (lane == leader) slot = atomicAdd(&s_D, (u32)__popcll(m));
          slot = __shfl(slot, leader) + count_below(m);
        }
        const u64 key = fresh[q] ? make_key(__float_as_uint(v[q]), idx[q]) : 0ull;
        if (fresh[q] && slot < a.S) keys[slot] = key;
        wave_hist_add(s_sel.hist, (u32)(key >> 56), fresh[q]);
      }
    }
    __syncthreads();
    // top-up by wavefront 0: further draws in order until S distinct are held
    if (wid == 0) {
      u64 D = s_D;
      u64 j0 = a.S;
      u32 guard = 0;
      while (D < a.S) {
        const u32 id2 = (u32)sample_draw(j0 + lane, row, a.attempt, a.seed, a.N);
        const bool held = (s_bits[id2 >> 5] >> (id2 & 31u)) & 1u;
        bool repeat = false;
        for (int d = 1; d < kWave; ++d) {
          const u32 other = __shfl_up(id2, d, kWave);
          if ((int)lane >= d && other == id2) repeat = true;
        }
        const bool ok2 = !held && !repeat;
        const u64 m2 = __ballot(ok2);
        const u64 need = a.S - D;
        const u32 r = count_below(m2);
        if (ok2 && r < need) {
          atomicOr(&s_bits[id2 >> 5], 1u << (id2 & 31u));
          const u64 key2 = make_key(__float_as_uint(xr[id2]), id2);
          keys[D + r] = key2;
          atomicAdd(&s_sel.hist[key2 >> 56], 1u);
        }
        const u64 got = (u64)__popcll(m2);
        D += got < need ? got : need;
        j0 += kWave;
        if (++guard > (1u << 22)) {  // bounded: S <= N/2 makes each draw new with prob >= 1/2
          if (lane == 0) s_fail = 1;
          break;
        }
      }
      if (lane == 0) s_D = (u32)D;
    }
    __syncthreads();
    const bool sample_ok = !s_fail && s_D == a.S;
    if (threadIdx.x == 0) block_select_start_from_top_hist(&s_sel, s_sel.hist, sample_ok ? a.S : 0, a.t);
    __syncthreads();
    bool ok = false;
    // the bitmap is no longer needed: its LDS holds the final sort (16384 keys)
    const u64 tau = block_select_finish(keys, a.S, reinterpret_cast<u64*>(s_bits), kBitmapWords / 2, &s_sel, &ok);
    if (threadIdx.x == 0) {
      RowCtl* c = &a.ctls[row];
      c->tau = tau;
      c->R = 0;
      c->status = ok ? 0u : 3u;
    }
  }
}

// LDS: pow2(M) keys (dynamic), so that several rows share a compute unit.
constexpr u32 kRefineThreads = 256;
__global__ __launch_bounds__(kRefineThreads) void b_refine_kernel(BatchedArgs a) {
  extern __shared__ u64 s[];
  for (u64 li = blockIdx.x; li < a.nrows; li += gridDim.x) {
    const u32 row = a.rows ? (u32)a.rows[li] : (u32)li;
    const RowCtl* c = &a.ctls[row];
    if (c->status != 0) continue;  // uniform: one row per workgroup
    const u64 R = c->R;
    const u32 n = (u32)(R < a.M ? R : a.M);
    const u64* cand = a.cand + (u64)row * a.M;
    u32 P = 1;
    while (P < n) P <<= 1;
    __syncthreads();
    for (u32 i = threadIdx.x; i < P; i += blockDim.x) s[i] = i < n ? cand[i] : 0ull;
    __syncthreads();
    block_bitonic_desc(s, P);
    const float* xr = a.x + (u64)row * a.ld;
    for (u32 j = threadIdx.x; j < a.k; j += blockDim.x)
      write_row_out(s[j], j, xr, a.N, a.out_vals + (u64)row * a.k, a.out_idx + (u64)row * a.k);
  }
}

__global__ __launch_bounds__(kBThreads) void b_rowsort_kernel(BatchedArgs a) {
  __shared__ u64 s[kSmallSort];
  u32 P = 1;
  while (P < a.N) P <<= 1;
  for (u64 li = blockIdx.x; li < a.nrows; li += gridDim.x) {
    const u32 row = a.rows ? (u32)a.rows[li] : (u32)li;
    const float* xr = a.x + (u64)row * a.ld;
    __syncthreads();
    for (u32 i = threadIdx.x; i < P; i += blockDim.x)
      s[i] = i < a.N ? make_key(__float_as_uint(xr[i]), i) : 0ull;
    __syncthreads();
    block_bitonic_desc(s, P);
    for (u32 j = threadIdx.x; j < a.k; j += blockDim.x)
      write_row_out(s[j], j, xr, a.N, a.out_vals + (u64)row * a.k, a.out_idx + (u64)row * a.k);
  }
}

namespace {
u32 row_grid(u64 nrows, u32 per_cu) {
  u64 g = (u64)device_cu_count() * per_cu;
  if (g > nrows) g = nrows;
  return (u32)(g ? g : 1);
}
}  // namespace

u32 batched_sample_blocks(u64 nrows) { return row_grid(nrows, 1); }

hipError_t launch_b_sample(const BatchedArgs& a, hipStream_t s) {
  b_sample_kernel<<<batched_sample_blocks(a.nrows), kBThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_b_refine(const BatchedArgs& a, hipStream_t s) {
  u32 P = 1;
  while (P < a.M) P <<= 1;  // M <= kSmallSort: at most 64 KB
  b_refine_kernel<<<row_grid(a.nrows, 8), kRefineThreads, (size_t)P * sizeof(u64), s>>>(a);
  return hipGetLastError();
}

hipError_t launch_b_rowsort(const BatchedArgs& a, hipStream_t s) {
  b_rowsort_kernel<<<row_grid(a.nrows, 2), kBThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace profk
