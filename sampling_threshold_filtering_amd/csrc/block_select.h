// Radix selection by ONE workgroup: the key of a given rank (descending) among n
// distinct 64-bit keys in global memory, and an LDS bitonic sort.
//
// Used where the whole selection is small enough for one compute unit: the
// threshold tau of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient
// Top-k Selection", §3 stage 2: the t-th largest of the S sampled values) from block
// lists or key slots staged in LDS (lds_select_desc), a block's own t-th largest
// (reg_select_desc), the per-row stages of the batched form, and, from L2, the
// threshold of batched rows whose sample exceeds LDS with t > 1024.  Each pass reads the keys
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

constexpr u32 kMaxWaves = 16;  // wavefronts of a 1024-thread block

constexpr u32 kSelCopies = 8;  // interleaved copies of the digit histogram, by lane & 7

struct alignas(16) LdsSelect {
  // digit d's count in hist[d * kSelCopies .. + kSelCopies); past them one slot per lane
  // for keys that do not match
  u32 hist[256 * kSelCopies + kWave];
  u64 prefix;
  u32 rank, state;  // state: 0 = running, 1 = at most kWave keys match, 2 = too few keys
  u32 nsmall;
  u64 small[kWave];
  u64 result;
  // per wavefront: AND / OR / count of its nonzero keys (one record, so that one
  // address register serves the three fields)
  struct alignas(8) Wave {
    u64 vand, vor;
    u32 nz, pad;
  } w[kMaxWaves];
};

// Radix selection of the key of descending rank `rank` (1-based) among distinct nonzero
// keys, by the whole block (256 to 1024 threads), in steps that share this state: the
// leading bits that all the keys share (where their AND and OR agree) are fixed first;
// 8-bit digits follow from there, each pass a histogram of the keys that match the
// digits fixed so far, until at most kWave keys match; those are ranked against each
// other.  With one wavefront per SIMD nothing hides latency, so the steps avoid
// dependent chains: cross-lane work goes through DPP and readlane rather than the LDS
// crossbar, counting is branch-free, and the gather reserves one range per wavefront.
struct SelPass {
  u64 prefix, mask;
  u32 want, state, d0;
};

__device__ __forceinline__ u64 wave_and64(u64 v) {
  auto f = [](u32 x, u32 y) { return x & y; };
  return ((u64)wave_reduce_u32((u32)(v >> 32), f) << 32) | wave_reduce_u32((u32)v, f);
}
__device__ __forceinline__ u64 wave_or64(u64 v) {
  auto f = [](u32 x, u32 y) { return x | y; };
  return ((u64)wave_reduce_u32((u32)(v >> 32), f) << 32) | wave_reduce_u32((u32)v, f);
}
__device__ __forceinline__ u32 wave_sum32(u32 v) {
  return wave_reduce_u32(v, [](u32 x, u32 y) { return x + y; });
}

// Per-thread AND / OR / count of its nonzero keys in; the block's combined state out.
__device__ __forceinline__ SelPass sel_begin(u64 va, u64 vo, u32 nz, u32 rank, LdsSelect* L) {
  const u32 tid = opaque_u32(threadIdx.x), lane = tid & (kWave - 1), wid = tid / kWave;
  const u32 nw = blockDim.x / kWave;
  va = wave_and64(va);
  vo = wave_or64(vo);
  nz = wave_sum32(nz);
  if (lane == 0) {
    L->w[wid].vand = va;
    L->w[wid].vor = vo;
    L->w[wid].nz = nz;
  }
  if (tid == 0) {
    L->nsmall = 0;
    L->result = 0;
  }
  __syncthreads();
  // lane w takes wavefront w's values; then the same reductions over the lanes
  const bool in = lane < nw;
  const u64 a = wave_and64(in ? L->w[lane].vand : ~0ull);
  const u64 o = wave_or64(in ? L->w[lane].vor : 0ull);
  const u32 n = wave_sum32(in ? L->w[lane].nz : 0u);
  // bits above the highest one where the keys differ are common to all of them
  const u64 diff = a ^ o;
  SelPass p;
  p.d0 = diff ? (u32)__clzll((long long)diff) / 8u : 8u;
  p.mask = p.d0 ? ~0ull << (64u - 8u * p.d0) : 0ull;
  p.prefix = a & p.mask;
  p.want = rank;
  p.state = n < rank ? 2u : n <= (u32)kWave ? 1u : 0u;
  return p;
}

// After a digit histogram in L->hist: wavefront 0 finds the digit that holds the rank;
// every thread takes the new state.  Ends with the block synchronised.
__device__ __forceinline__ void sel_choose(SelPass& p, u32 shift, LdsSelect* L) {
  const u32 tid = opaque_u32(threadIdx.x), lane = tid & (kWave - 1);
  if (tid < (u32)kWave) {
    if (lane == 0) L->state = 2u;  // replaced by the lane whose digit holds the rank
    // descending digits: lane owns 255 - 4*lane .. 255 - 4*lane - 3
    u32 c[4], sum = 0;
#pragma unroll
    for (u32 r = 0; r < 4; ++r) {
      const uint4* h = reinterpret_cast<const uint4*>(L->hist + (255u - (4u * lane + r)) * kSelCopies);
      const uint4 x = h[0], y = h[1];
      c[r] = x.x + x.y + x.z + x.w + y.x + y.y + y.z + y.w;
      sum += c[r];
    }
    u32 run = wave_incl_scan_add(sum, lane) - sum;
#pragma unroll
    for (u32 r = 0; r < 4; ++r) {
      if (run < p.want && run + c[r] >= p.want) {
        const u32 dg = 255u - (4u * lane + r);
        L->rank = p.want - run;
        L->prefix = p.prefix | ((u64)dg << shift);
        L->state = c[r] <= (u32)kWave ? 1u : 0u;
      }
      run += c[r];
    }
  }
  __syncthreads();
  p.prefix = L->prefix;
  p.mask |= 0xFFull << shift;
  p.want = L->rank;
  p.state = L->state;
}

__device__ __forceinline__ bool sel_match(u64 k, const SelPass& p) { return k != 0 && (k & p.mask) == p.prefix; }

// Key k's digit counted into L->hist with no branch and one LDS atomic: lane l adds to
// copy l & 7 of the digit's count, so a digit that a whole wavefront shares costs
// eight-way conflicts on eight banks rather than 64 on one address; a key that does
// not match adds to its lane's spare slot.
__device__ __forceinline__ void sel_count(u64 k, const SelPass& p, u32 shift, u32 lane, LdsSelect* L) {
  const u32 b = sel_match(k, p) ? ((u32)(k >> shift) & 255u) * kSelCopies + (lane & (kSelCopies - 1)) : 256u * kSelCopies + lane;
  atomicAdd(&L->hist[b], 1u);
}

__device__ __forceinline__ void sel_clear_hist(LdsSelect* L) {
  uint4* h = reinterpret_cast<uint4*>(L->hist);
  for (u32 b = opaque_u32(threadIdx.x); b < 256 * kSelCopies / 4; b += blockDim.x) h[b] = make_uint4(0, 0, 0, 0);
  __syncthreads();
}

// Slot in L->small of a thread's first matching key, the wavefront's keys taking one
// contiguous range: an exclusive scan of the per-thread counts and one LDS atomic.
__device__ __forceinline__ u32 sel_reserve(u32 cnt, u32 lane, LdsSelect* L) {
  const u32 incl = wave_incl_scan_add(cnt, lane);
  const u32 total = (u32)__builtin_amdgcn_readlane((int)incl, kWave - 1);
  u32 base = 0;
  if (total != 0 && lane == 0) base = atomicAdd(&L->nsmall, total);
  return (u32)__builtin_amdgcn_readlane((int)base, 0) + incl - cnt;
}

// The (at most kWave) keys gathered in L->small are ranked against each other, four
// threads per key, sixteen comparisons each; the key of rank p.want is the result.
__device__ __forceinline__ u64 sel_finish(const SelPass& p, LdsSelect* L) {
  __syncthreads();
  if (p.state == 1) {
    const u32 m = L->nsmall < (u32)kWave ? L->nsmall : (u32)kWave;
    for (u32 t = opaque_u32(threadIdx.x); t < 4u * kWave; t += blockDim.x) {
      const u32 i = t >> 2, part = t & 3u;
      const u64 k = L->small[i];
      u64 o[16];
#pragma unroll
      for (u32 j = 0; j < 16; ++j) o[j] = L->small[part * 16u + j];
      u32 r = 0;
#pragma unroll
      for (u32 j = 0; j < 16; ++j) r += (part * 16u + j < m && o[j] > k) ? 1u : 0u;
      r += (u32)__builtin_amdgcn_update_dpp(0, (int)r, 0xB1, 0xF, 0xF, false);
      r += (u32)__builtin_amdgcn_update_dpp(0, (int)r, 0x4E, 0xF, 0xF, false);
      if (part == 0 && i < m && r + 1u == p.want) L->result = k;
    }
  }
  __syncthreads();
  const u64 result = L->result;
  __syncthreads();
  return result;
}

// The key of descending rank `rank` (1-based) among the nonzero, distinct keys s[0..n)
// held in LDS.  Returns 0 when fewer than `rank` nonzero keys are present.
__device__ inline u64 lds_select_desc(const u64* s, u32 n, u32 rank, LdsSelect* L) {
  const u32 tid = opaque_u32(threadIdx.x), lane = tid & (kWave - 1);
  u64 va = ~0ull, vo = 0;
  u32 nz = 0;
  for (u32 i = tid; i < n; i += blockDim.x) {
    const u64 k = s[i];
    const bool h = k != 0;
    va &= h ? k : ~0ull;
    vo |= k;
    nz += h ? 1u : 0u;
  }
  SelPass p = sel_begin(va, vo, nz, rank, L);
  for (u32 d = p.d0; d < 8 && p.state == 0; ++d) {
    sel_clear_hist(L);
    const u32 shift = 56u - 8u * d;
    for (u32 i = tid; i < n; i += blockDim.x) sel_count(s[i], p, shift, lane, L);
    __syncthreads();
    sel_choose(p, shift, L);
  }
  if (p.state == 1) {
    u32 cnt = 0;
    for (u32 i = tid; i < n; i += blockDim.x) cnt += sel_match(s[i], p) ? 1u : 0u;
    u32 slot = sel_reserve(cnt, lane, L);
    for (u32 i = tid; i < n && cnt; i += blockDim.x) {
      const u64 k = s[i];
      if (sel_match(k, p)) {
        if (slot < (u32)kWave) L->small[slot] = k;
        ++slot;
        --cnt;
      }
    }
  }
  return sel_finish(p, L);
}

// The same selection with the keys in registers: thread t holds v[0..P), zero for no
// key.  A pass then reads no keys, it only counts digits.  `after_begin` runs once, by
// every thread, after the first barrier (a caller's independent work, such as loads it
// wants issued while the select runs).
template <u32 P, class Hook>
__device__ inline u64 reg_select_desc(const u64 (&v)[P], u32 rank, LdsSelect* L, Hook&& after_begin) {
  const u32 lane = opaque_u32(threadIdx.x) & (kWave - 1);
  u64 va = ~0ull, vo = 0;
  u32 nz = 0;
#pragma unroll
  for (u32 q = 0; q < P; ++q) {
    const bool h = v[q] != 0;
    va &= h ? v[q] : ~0ull;
    vo |= v[q];
    nz += h ? 1u : 0u;
  }
  SelPass p = sel_begin(va, vo, nz, rank, L);
  after_begin();
  for (u32 d = p.d0; d < 8 && p.state == 0; ++d) {
    sel_clear_hist(L);
    const u32 shift = 56u - 8u * d;
#pragma unroll
    for (u32 q = 0; q < P; ++q) sel_count(v[q], p, shift, lane, L);
    __syncthreads();
    sel_choose(p, shift, L);
  }
  if (p.state == 1) {
    u32 cnt = 0;
#pragma unroll
    for (u32 q = 0; q < P; ++q) cnt += sel_match(v[q], p) ? 1u : 0u;
    u32 slot = sel_reserve(cnt, lane, L);
#pragma unroll
    for (u32 q = 0; q < P; ++q)
      if (sel_match(v[q], p)) {
        if (slot < (u32)kWave) L->small[slot] = v[q];
        ++slot;
      }
  }
  return sel_finish(p, L);
}

template <u32 P>
__device__ inline u64 reg_select_desc(const u64 (&v)[P], u32 rank, LdsSelect* L) {
  return reg_select_desc(v, rank, L, [] {});
}

// Convenience: the whole selection from scratch.
__device__ inline u64 block_select_rank(const u64* keys, u64 n, u64 rank, u64* buf, u32 cap, BlockSelectLds* L,
                                        bool* ok_out) {
  if (threadIdx.x == 0) block_select_start(L, n, rank);
  __syncthreads();
  return block_select_finish(keys, n, buf, cap, L, ok_out);
}

}  // namespace profk
