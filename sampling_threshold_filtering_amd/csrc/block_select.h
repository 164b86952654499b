// Radix selection by ONE workgroup: the key of a given rank (descending) among n
// distinct 64-bit keys in global memory, and an LDS bitonic sort.
//
// Used where the whole selection is small enough for one compute unit: the
// threshold tau of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient
// Top-k Selection", §3 stage 2: the t-th largest of the S sampled values, S at most
// 131072) and the per-row stages of the batched form.  Each pass reads the keys
// that still match the fixed prefix from L2 (eight loads in flight per thread),
// histograms the next 8-bit digit in LDS (one LDS atomic per distinct digit per
// wavefront) and fixes it; once at most `cap` keys match they are gathered into
// LDS and sorted, and the answer is read off.
#pragma once

#include "profk_device.h"

namespace profk {

// Descending bitonic sort of s[0..P), P a power of two, by the whole block.
__device__ inline void block_bitonic_desc(u64* s, u32 P) {
  for (u32 k = 2; k <= P; k <<= 1) {
    for (u32 j = k >> 1; j > 0; j >>= 1) {
      for (u32 i = threadIdx.x; i < P; i += blockDim.x) {
        const u32 ixj = i ^ j;
        if (ixj > i) {
          const u64 a = s[i], b = s[ixj];
          const bool up = (i & k) == 0;
          if (up ? (a < b) : (a > b)) {
            s[i] = b;
            s[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Lists j = 0..nl-1 of T keys each (T a power of two), each sorted descending, at
// s + j*T.  Leaves the T largest keys of their union, sorted descending, in s[0..T).
// Pairwise tree: merging descending lists A and B, max(A[i], B[T-1-i]) holds exactly
// the T largest of A and B as a bitonic sequence (the first half-cleaner of the
// bitonic merge of A followed by B reversed), and log2 T half-cleaners sort it.
__device__ inline void block_merge_lists(u64* s, u32 nl, u32 T) {
  u32 lt = 0;
  while ((1u << lt) < T) ++lt;
  for (u32 l = 0; nl > 1; ++l) {
    const u32 pairs = nl >> 1;
    for (u32 e = threadIdx.x; e < (pairs << lt); e += blockDim.x) {
      const u32 p = e >> lt, i = e & (T - 1);
      u64* A = s + ((u64)(2 * p) << (l + lt));
      const u64* B = s + ((u64)(2 * p + 1) << (l + lt));
      const u64 a = A[i], b = B[T - 1 - i];
      A[i] = a > b ? a : b;
    }
    __syncthreads();
    for (u32 h = T >> 1; h > 0; h >>= 1) {
      for (u32 e = threadIdx.x; e < (pairs << lt) >> 1; e += blockDim.x) {
        const u32 p = e >> (lt - 1), r = e & ((T >> 1) - 1);
        const u32 i = ((r & ~(h - 1)) << 1) | (r & (h - 1));  // the pair (i, i + h), bit h of i clear
        u64* A = s + ((u64)(2 * p) << (l + lt));
        const u64 x0 = A[i], x1 = A[i + h];
        if (x0 < x1) {
          A[i] = x1;
          A[i + h] = x0;
        }
      }
      __syncthreads();
    }
    nl = (nl + 1) >> 1;
  }
}

struct BlockSelectLds {
  u32 hist[256];
  u32 ncol;
  u32 digit;
  u64 prefix, mask, rank, count;
  u32 ok;
};

// State after the top digit has been fixed from a histogram of it (hist[b] = number
// of keys whose top 8 bits are b).  Called by thread 0 only.
__device__ inline void block_select_start_from_top_hist(BlockSelectLds* L, const u32* hist, u64 n, u64 rank) {
  L->ok = (rank >= 1 && rank <= n) ? 1u : 0u;
  L->prefix = 0;
  L->mask = 0;
  L->rank = rank;
  L->count = n;
  L->digit = 0;
  if (!L->ok) return;
  u64 cum = 0;
  int b = 255;
  for (; b >= 0; --b) {
    const u64 c = hist[b];
    if (cum + c >= rank) break;
    cum += c;
  }
  if (b < 0) {
    L->ok = 0;
    return;
  }
  L->rank = rank - cum;
  L->count = hist[b];
  L->prefix = (u64)b << 56;
  L->mask = 0xFFull << 56;
  L->digit = 1;
}

__device__ inline void block_select_start(BlockSelectLds* L, u64 n, u64 rank) {
  L->ok = (rank >= 1 && rank <= n) ? 1u : 0u;
  L->prefix = 0;
  L->mask = 0;
  L->rank = rank;
  L->count = n;
  L->digit = 0;
}

constexpr u32 kBlockSelectILP = 8;

// Finishes the selection whose state is in *L (set by one of the start functions and
// visible to every thread); returns the key of the requested rank to all threads.
// keys[0..n) may hold empty slots (key 0, which no valid key equals); the count given
// to the start functions is that of the valid keys.  `buf` is an LDS array of `cap`
// keys (cap a power of two).  *ok_out is false when the state turned out inconsistent
// (never for distinct keys).
__device__ inline u64 block_select_finish(const u64* keys, u64 n, u64* buf, u32 cap, BlockSelectLds* L,
                                          bool* ok_out) {
  const u64 span = (u64)blockDim.x * kBlockSelectILP;
  while (L->ok && L->digit < 8 && L->count > cap) {
    const u64 prefix = L->prefix, mask = L->mask;
    const u32 shift = 56u - 8u * L->digit;
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x) L->hist[b] = 0;
    __syncthreads();
    for (u64 base = 0; base < n; base += span) {
      u64 kk[kBlockSelectILP];
#pragma unroll
      for (u32 q = 0; q < kBlockSelectILP; ++q) {
        const u64 i = base + (u64)q * blockDim.x + threadIdx.x;
        kk[q] = i < n ? keys[i] : 0ull;
      }
#pragma unroll
      for (u32 q = 0; q < kBlockSelectILP; ++q) {
        const u64 i = base + (u64)q * blockDim.x + threadIdx.x;
        const bool match = i < n && kk[q] != 0 && ((kk[q] & mask) == prefix);
        wave_hist_add(L->hist, (u32)(kk[q] >> shift) & 255u, match);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      u64 cum = 0;
      int b = 255;
      for (; b >= 0; --b) {
        const u64 c = L->hist[b];
        if (cum + c >= L->rank) break;
        cum += c;
      }
      if (b < 0) {
        L->ok = 0;
      } else {
        L->rank -= cum;
        L->count = L->hist[b];
        L->prefix = prefix | ((u64)b << shift);
        L->mask = mask | (0xFFull << shift);
        L->digit += 1;
      }
    }
    __syncthreads();
  }
  if (L->ok) {
    const u64 prefix = L->prefix, mask = L->mask, count = L->count;
    if (count > cap || count == 0) {
      __syncthreads();
      if (threadIdx.x == 0) L->ok = 0;
    } else {
      if (threadIdx.x == 0) L->ncol = 0;
      __syncthreads();
      for (u64 base = 0; base < n; base += span) {
        u64 kk[kBlockSelectILP];
#pragma unroll
        for (u32 q = 0; q < kBlockSelectILP; ++q) {
          const u64 i = base + (u64)q * blockDim.x + threadIdx.x;
          kk[q] = i < n ? keys[i] : 0ull;
        }
#pragma unroll
        for (u32 q = 0; q < kBlockSelectILP; ++q) {
          const u64 i = base + (u64)q * blockDim.x + threadIdx.x;
          const bool match = i < n && kk[q] != 0 && ((kk[q] & mask) == prefix);
          const u64 m = __ballot(match);
          u32 slot = 0;
          if (m) {
            const u32 leader = __ffsll((long long)m) - 1;
            if (lane_id() == leader) slot = atomicAdd(&L->ncol, (u32)__popcll(m));
            slot = __shfl(slot, leader) + count_below(m);
          }
          if (match && slot < cap) buf[slot] = kk[q];
        }
      }
      __syncthreads();
      const u32 m = L->ncol;
      if (m != count) {
        __syncthreads();
        if (threadIdx.x == 0) L->ok = 0;
      } else {
        u32 P = 1;
        while (P < m) P <<= 1;
        for (u32 i = m + threadIdx.x; i < P; i += blockDim.x) buf[i] = 0ull;
        __syncthreads();
        block_bitonic_desc(buf, P);
      }
    }
  }
  __syncthreads();
  const bool ok = L->ok != 0;
  const u64 result = ok ? buf[L->rank - 1] : 0ull;
  __syncthreads();
  *ok_out = ok;
  return result;
}

// Convenience: the whole selection from scratch.
__device__ inline u64 block_select_rank(const u64* keys, u64 n, u64 rank, u64* buf, u32 cap, BlockSelectLds* L,
                                        bool* ok_out) {
  if (threadIdx.x == 0) block_select_start(L, n, rank);
  __syncthreads();
  return block_select_finish(keys, n, buf, cap, L, ok_out);
}

}  // namespace profk
