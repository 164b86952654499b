// Device-side building blocks shared by the Prof-K kernels (gfx950, wave64).
//
// Keys.  Every entry x_i of a row is compared through the 64-bit composite key
//     key(i) = (ord32(x_i) << 32) | (~i & 0xFFFFFFFF)
// where ord32 maps the fp32 bits to an unsigned integer of the same order
// (-0.0 folded onto +0.0, every NaN onto the largest code).  A larger key ranks
// first; equal values are ordered by lower index first.  All keys of a row are
// distinct, which makes the pages' distinct-entries assumption ("Prof-K:
// Probabilistic One-Pass Filtering for Efficient Top-k Selection", §4 "Notation
// and Conventions") hold for every input: the rank law of the threshold and the
// exact parameters of Theorem 4 then apply unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include "profk.h"

namespace profk {

typedef unsigned long long u64;
typedef unsigned int u32;

constexpr int kWave = 64;

__device__ __forceinline__ u32 ord32(u32 bits) {
  if (bits == 0x80000000u) bits = 0u;                          // -0.0 -> +0.0
  if ((bits & 0x7FFFFFFFu) > 0x7F800000u) bits = 0x7FFFFFFFu;  // NaN -> one code above +inf
  return bits ^ ((u32)((int)bits >> 31) | 0x80000000u);
}

__device__ __forceinline__ u64 make_key(u32 bits, u32 idx) {
  return ((u64)ord32(bits) << 32) | (u64)(~idx);
}

__device__ __forceinline__ u32 key_index(u64 key) { return ~(u32)key; }

// Inverse of ord32 on the canonical codes (used for the fast float pre-test).
__device__ __forceinline__ u32 bits_of_ord32(u32 o) {
  return (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11), written from its published definition:
// per round, with A = 0xD2511F53 and B = 0xCD9E8D57,
//   (c0,c1,c2,c3) -> (hi(B c2) ^ c1 ^ k0, lo(B c2), hi(A c0) ^ c3 ^ k1, lo(A c0)),
// and the key advances by (0x9E3779B9, 0xBB67AE85) between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, u32 k0, u32 k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const u32 hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const u32 hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Draw j of the sample stream of (seed, attempt, row): counter (j, row, attempt, 0),
// key (seed lo, seed hi); r = w0 + 2^32 w1 is mapped to floor(r * N / 2^64).
__device__ __forceinline__ u64 sample_draw(u64 j, u32 row, u32 attempt, u64 seed, u64 N) {
  const uint4 w = philox4x32_10(make_uint4((u32)j, row, attempt, 0u), (u32)seed, (u32)(seed >> 32));
  const u64 r = (u64)w.x | ((u64)w.y << 32);
  return __umul64hi(r, N);
}

// ---------------------------------------------------------------------------
// Wave helpers
__device__ __forceinline__ u32 lane_id() { return __lane_id(); }

// v unchanged, but opaque to the optimiser: expressions of it stay where they are
// written instead of being hoisted out of an enclosing loop and held in registers
// across it (used where a loop body is register-bound).
__device__ __forceinline__ u32 opaque_u32(u32 v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ u32 count_below(u64 mask) {
  // number of set bits of mask in lanes below this one
  return __builtin_amdgcn_mbcnt_hi((u32)(mask >> 32), __builtin_amdgcn_mbcnt_lo((u32)mask, 0u));
}

// Order the wave's LDS accesses around a cross-lane exchange through LDS.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <class T>
__device__ __forceinline__ T atomic_load_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T>
__device__ __forceinline__ void atomic_store_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One atomicAdd per wave for the lanes with pred set; returns this lane's slot.
__device__ __forceinline__ u64 wave_reserve(u64* counter, bool pred) {
  const u64 m = __ballot(pred);
  u64 base = 0;
  if (m) {
    const u32 leader = __ffsll((long long)m) - 1;
    if (lane_id() == leader) base = atomicAdd(counter, (u64)__popcll(m));
    base = __shfl(base, leader);
  }
  return base + count_below(m);
}

__device__ __forceinline__ u32 wave_reserve32(u32* counter, bool pred) {
  const u64 m = __ballot(pred);
  u32 base = 0;
  if (m) {
    const u32 leader = __ffsll((long long)m) - 1;
    if (lane_id() == leader) base = atomicAdd(counter, (u32)__popcll(m));
    base = __shfl(base, leader);
  }
  return base + count_below(m);
}

// Exchange with lane ^ J.  Strides 1, 2, 4, 8 use DPP lane moves (plain ALU
// operations); 16 and 32 go through the LDS crossbar (ds_bpermute).
// Hand-off of data between workgroups without cache maintenance.  Agent-scope atomic
// loads and stores are issued with the device-coherence cache bit (stores written
// through, loads served from the coherence point), so they need no L2 writeback or
// invalidate; a writer makes its stores complete (drain_memory_ops) before the atomic
// that publishes them, and the reader reads them with ld_agent after seeing that
// atomic.  An agent-scope release / acquire fence orders the same way but also writes
// back / invalidates the die's whole L2 (every dirty line in it, not just the writer's).
__device__ __forceinline__ u64 ld_agent(const u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_agent(u64* p, u64 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// All of this thread's memory operations complete (s_waitcnt 0), with compiler fences
// around it so that none of them moves past it.
__device__ __forceinline__ void drain_memory_ops() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Reduction over the whole wavefront with an associative, commutative f: DPP within
// rows of 16 (quad_perm xor 1 and xor 2, then row_ror 4 and 8), then the four row
// results read out to scalars.  Every lane gets the result.
template <class F>
__device__ __forceinline__ u32 wave_reduce_u32(u32 v, F f) {
  v = f(v, (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = f(v, (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = f(v, (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = f(v, (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  const u32 r0 = (u32)__builtin_amdgcn_readlane((int)v, 0), r1 = (u32)__builtin_amdgcn_readlane((int)v, 16);
  const u32 r2 = (u32)__builtin_amdgcn_readlane((int)v, 32), r3 = (u32)__builtin_amdgcn_readlane((int)v, 48);
  return f(f(r0, r1), f(r2, r3));
}

// Inclusive prefix sum over the wavefront: row_shr 1, 2, 4, 8 within rows of 16 (lanes
// whose source falls before the row start add zero), then the totals of the rows below.
__device__ __forceinline__ u32 wave_incl_scan_add(u32 v, u32 lane) {
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);
  const u32 s1 = (u32)__builtin_amdgcn_readlane((int)v, 15), s2 = (u32)__builtin_amdgcn_readlane((int)v, 31);
  const u32 s3 = (u32)__builtin_amdgcn_readlane((int)v, 47);
  const u32 row = lane >> 4;
  return v + (row >= 1 ? s1 : 0u) + (row >= 2 ? s2 : 0u) + (row >= 3 ? s3 : 0u);
}

template <u32 J>
__device__ __forceinline__ u32 lane_xor_u32(u32 v, u32 lane) {
  if constexpr (J == 1) {  // quad_perm [1,0,3,2]
    return (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  } else if constexpr (J == 2) {  // quad_perm [2,3,0,1]
    return (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  } else if constexpr (J == 4 || J == 8) {  // within rows of 16: row_shl:J where bit J is clear, row_shr:J else
    const u32 up = (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 | J, 0xF, 0xF, true);
    const u32 dn = (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 | J, 0xF, 0xF, true);
    return (lane & J) ? dn : up;
  } else {
    return (u32)__shfl_xor((int)v, (int)J);
  }
}

template <u32 J>
__device__ __forceinline__ u64 lane_xor(u64 v, u32 lane) {
  const u32 lo = lane_xor_u32<J>((u32)v, lane);
  const u32 hi = lane_xor_u32<J>((u32)(v >> 32), lane);
  return ((u64)hi << 32) | lo;
}

// One stage (K, J) of a descending bitonic sort of 64*M keys held M per lane
// (element i = r*64 + lane is v[r]), then the stages (K, J/2) ... (K, 1).  All
// strides are template constants, so every exchange is resolved at compile time.
template <int M, u32 K, u32 J>
__device__ __forceinline__ void bitonic_stage_regs(u64 (&v)[M], u32 lane) {
  if constexpr (J < (u32)kWave) {
    // all M exchanges first, then the compare-exchanges
    u64 p[M];
#pragma unroll
    for (int r = 0; r < M; ++r) p[r] = lane_xor<J>(v[r], lane);
    __builtin_amdgcn_sched_barrier(0);  // keep the exchanges ahead of their uses
#pragma unroll
    for (int r = 0; r < M; ++r) {
      const u32 i = (u32)r * kWave + lane;
      const bool keep_max = ((i & J) == 0) == ((i & K) == 0);
      if ((v[r] < p[r]) == keep_max) v[r] = p[r];  // take the partner's key
    }
  } else {
    constexpr u32 rj = J / kWave;
#pragma unroll
    for (int r = 0; r < M; ++r) {
      if ((r & rj) == 0) {
        const int r2 = r | (int)rj;
        const bool up = (((u32)r * kWave) & K) == 0;  // lower element's block direction
        const u64 x0 = v[r], x1 = v[r2];
        const u64 hi = x0 > x1 ? x0 : x1, lo = x0 > x1 ? x1 : x0;
        v[r] = up ? hi : lo;
        v[r2] = up ? lo : hi;
      }
    }
  }
  if constexpr (J > 1) bitonic_stage_regs<M, K, J / 2>(v, lane);
}

template <int M, u32 K>
__device__ __forceinline__ void bitonic_levels_regs(u64 (&v)[M], u32 lane) {
  bitonic_stage_regs<M, K, K / 2>(v, lane);
  if constexpr (K < 64u * (u32)M) bitonic_levels_regs<M, K * 2>(v, lane);
}

// Descending bitonic sort of 64*M keys held M per lane: afterwards element
// i = r*64 + lane (v[r] of that lane) is the i-th largest.
template <int M>
__device__ __forceinline__ void wave_sort_regs_desc(u64 (&v)[M]) {
  bitonic_levels_regs<M, 2>(v, lane_id());
}

// Descending bitonic sort of one key per lane across the wavefront, in registers.
__device__ __forceinline__ u64 wave_sort_desc(u64 v) {
  u64 a[1] = {v};
  wave_sort_regs_desc<1>(a);
  return a[0];
}

// Descending bitonic sort of the M keys of one lane (registers only).
template <int M>
__device__ __forceinline__ void lane_sort_desc(u64 (&v)[M]) {
#pragma unroll
  for (int k = 2; k <= M; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const bool desc = (i & k) == 0;
          const u64 a = v[i], b = v[l];
          const u64 hi = a > b ? a : b, lo = a > b ? b : a;
          v[i] = desc ? hi : lo;
          v[l] = desc ? lo : hi;
        }
      }
    }
  }
}

// Merge step of the lane lists: with v this lane's T largest (descending) and the
// partner lane ^ D holding another such list, leaves the T largest of both, sorted,
// in v (max(A[i], B[T-1-i]) is their bitonic top half; log2 T half-cleaners sort it).
template <int T, u32 D>
__device__ __forceinline__ void lane_merge_top(u64 (&v)[T], u32 lane) {
  u64 p[T];
#pragma unroll
  for (int i = 0; i < T; ++i) p[i] = lane_xor<D>(v[T - 1 - i], lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < T; ++i) v[i] = v[i] > p[i] ? v[i] : p[i];
#pragma unroll
  for (int h = T >> 1; h > 0; h >>= 1) {
#pragma unroll
    for (int i = 0; i < T; ++i) {
      if ((i & h) == 0) {
        const u64 a = v[i], b = v[i + h];
        v[i] = a > b ? a : b;
        v[i + h] = a > b ? b : a;
      }
    }
  }
}

// The T largest of the wavefront's 64*M keys (M per lane, T <= M), sorted
// descending, in top[0..T) of every lane.
template <int M, int T>
__device__ __forceinline__ void wave_top_lanes(u64 (&v)[M], u64 (&top)[T]) {
  static_assert(T <= M, "lists longer than the keys per lane");
  const u32 lane = lane_id();
  lane_sort_desc<M>(v);
#pragma unroll
  for (int i = 0; i < T; ++i) top[i] = v[i];
  lane_merge_top<T, 1>(top, lane);
  lane_merge_top<T, 2>(top, lane);
  lane_merge_top<T, 4>(top, lane);
  lane_merge_top<T, 8>(top, lane);
  lane_merge_top<T, 16>(top, lane);
  lane_merge_top<T, 32>(top, lane);
}

// Lanes with equal 8-bit digit (among those with active set): mask of those lanes.
__device__ __forceinline__ u64 wave_match8(u32 digit, bool active) {
  u64 same = __ballot(active);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (digit >> b) & 1u;
    const u64 bb = __ballot(bit);
    same &= bit ? bb : ~bb;
  }
  return same;
}

// Histogram increment of an LDS histogram, one LDS atomic per distinct digit in the wave.
__device__ __forceinline__ void wave_hist_add(u32* hist, u32 digit, bool active) {
  const u64 same = wave_match8(digit, active);
  if (active && lane_id() == (u32)(__ffsll((long long)same) - 1)) atomicAdd(&hist[digit], (u32)__popcll(same));
}

// ---------------------------------------------------------------------------
// Device-resident control blocks.

// State of one multi-pass radix selection ("which key has rank `rank` in
// descending order among n distinct keys").  Each pass either fixes the next
// 8-bit digit (histogram of the keys that match the fixed prefix) or, once at
// most kCollectCap keys match, collects them and finishes in LDS.
constexpr u32 kCollectCap = 2048;

struct SelState {
  u64 prefix;   // fixed high bits
  u64 mask;     // which bits are fixed
  u64 rank;     // 1-based rank of the target among the keys matching prefix
  u64 count;    // number of keys matching prefix
  u32 done;     // 1: result holds the exact key
  u32 digit;    // digits fixed so far (0..8)
  u32 ticket;   // last-block election
  u32 ncol;     // collected keys
  u32 error;    // inconsistent state seen (should never happen)
  u32 pad[3];
  u32 hist[256];
};

// Per-row control of one sampled attempt.
struct RowCtl {
  u64 D;        // distinct sample indices drawn so far
  u64 tau;      // composite threshold key
  u64 R;        // exact filter count
  u64 kth;      // composite key of the k-th largest candidate
  u64 nsel;     // keys written by the compaction
  u64 key_or;   // OR / AND of the selected keys (which digits vary)
  u64 key_and;
  u64 cmax;     // largest candidate key (filter)
  u32 status;   // 0 ok, 1 R < k, 2 R > M, 3 internal error
  u32 cur;      // ping-pong buffer of the sort
  u32 ticket;   // last-block election of the sort passes
  u32 bin_shift;  // refinement bins: bin = min(kBins - 1, (key - tau) >> bin_shift)
  u32 bstar;      // bin holding the k-th largest candidate
  u32 c_above;    // candidates in the bins above bstar
  u32 generic;    // 1: a needed bin is larger than one workgroup sorts in LDS
  u32 pad;
};

// Host-visible summary of an attempt, copied back once per attempt.
struct AttemptRecord {
  u64 R;
  u32 status;
  u32 error;
  u32 generic;  // the binned refinement deferred to the multi-pass one
  u32 pad;
};

// The attempt record as published into pinned host memory by the refinement: the
// host waits for `seq` to reach the value of its call instead of synchronising the
// stream, and returns while the last refinement launch is still writing outputs.
// Device-side outcome of an approximate-mode call (the public profk_approx_info).
using ApproxInfo = profk_approx_info;

constexpr u32 kXcds = 8;  // accelerator complex dies of the part; blocks go round-robin over them

struct HostRecord {
  u64 R;
  u32 status;
  u32 error;
  u32 generic;
  u32 seq;  // written last, with system-scope release
  u64 pad;
  // the filter's stream, 100 MHz clock: [0] first block start, [1 + x] last block end of
  // the blocks on die x (written by the filter's last block; 0 = not measured)
  u64 xt[kXcds + 1];
  // the check as soon as the filter knows it, one 64-bit word written by one store:
  // (seq mod 2^22) << 42 | status << 40 | R  (R < 2^32)
  u64 early;
};

}  // namespace profk
