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

struct LdsSelect {
  u32 hist[256];
  u64 prefix, mask;
  u32 rank, count, state;  // state: 0 = running, 1 = at most kWave keys match, 2 = too few keys
  u32 nsmall;
  u64 small[kWave];
  u64 result;
};

// The key of descending rank `rank` (1-based) among the nonzero, distinct keys
// s[0..n) held in LDS, by the whole block: 8-bit digits from the top, each pass a
// histogram of the keys that match the digits fixed so far, until at most kWave keys
// match; those are ranked against each other by one wavefront.  Returns 0 when fewer
// than `rank` nonzero keys are present.
__device__ inline u64 lds_select_desc(const u64* s, u32 n, u32 rank, LdsSelect* L) {
  const u32 tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  if (tid == 0) {
    L->prefix = 0;
    L->mask = 0;
    L->rank = rank;
    L->count = 0xFFFFFFFFu;
    L->state = 0;
    L->nsmall = 0;
    L->result = 0;
  }
  for (u32 d = 0; d < 8; ++d) {
    for (u32 b = tid; b < 256; b += blockDim.x) L->hist[b] = 0;
    __syncthreads();
    const u64 prefix = L->prefix, mask = L->mask;
    const u32 shift = 56u - 8u * d;
    for (u32 i = tid; i < n; i += blockDim.x) {
      const u64 k = s[i];
      if (k != 0 && (k & mask) == prefix) atomicAdd(&L->hist[(u32)(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wid == 0) {
      // descending digits: lane owns 255 - 4*lane .. 255 - 4*lane - 3
      u32 c[4], sum = 0;
#pragma unroll
      for (u32 r = 0; r < 4; ++r) {
        c[r] = L->hist[255u - (4u * lane + r)];
        sum += c[r];
      }
      u32 incl = sum;
#pragma unroll
      for (u32 o = 1; o < (u32)kWave; o <<= 1) {
        const u32 v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      const u32 want = L->rank;
      const u32 total = __shfl(incl, kWave - 1);
      u32 run = incl - sum;
#pragma unroll
      for (u32 r = 0; r < 4; ++r) {
        if (run < want && run + c[r] >= want) {
          const u32 dg = 255u - (4u * lane + r);
          L->rank = want - run;
          L->count = c[r];
          L->prefix = prefix | ((u64)dg << shift);
          L->mask = mask | (0xFFull << shift);
          L->state = c[r] <= (u32)kWave ? 1u : 0u;
        }
        run += c[r];
      }
      if (lane == 0 && total < want) L->state = 2;
    }
    __syncthreads();
    if (L->state != 0) break;
  }
  if (L->state == 1) {
    const u64 prefix = L->prefix, mask = L->mask;
    for (u32 i = tid; i < n; i += blockDim.x) {
      const u64 k = s[i];
      if (k != 0 && (k & mask) == prefix) {
        const u32 slot = atomicAdd(&L->nsmall, 1u);
        if (slot < (u32)kWave) L->small[slot] = k;
      }
    }
    __syncthreads();
    const u32 m = L->nsmall < (u32)kWave ? L->nsmall : (u32)kWave;
    if (wid == 0 && lane < m) {
      const u64 k = L->small[lane];
      u32 r = 0;
      for (u32 j = 0; j < m; ++j) r += L->small[j] > k ? 1u : 0u;
      if (r + 1u == L->rank) L->result = k;
    }
  }
  __syncthreads();
  const u64 result = L->result;
  __syncthreads();
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
