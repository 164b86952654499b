// Batched Prof-K: the same four stages applied to every row of a B x N matrix
// ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k Selection", §3:
// batched inputs are handled per row; App. C: per-row threshold, buffer and
// counter; App. E.2: the budget is split eps/B per row).
//
//   b_sample_pipe_kernel  rows of at most 2^20 values with S <= 4096: one 1024-thread
//                     workgroup per CU, persistent over the listed rows.  Each row's
//                     sample is tracked in an LDS hash set (two, used in turn); its
//                     keys stay in registers (four draws per thread), and the top-up
//                     keys fill the register slots that repeats left empty before one
//                     register radix select gives tau.  A row's top-up and select run
//                     while the next row's gathers are in flight.
//   b_sample_kernel   the other rows of at most 2^20 values, one workgroup per row
//                     (persistent over the listed rows): the row's sample without
//                     replacement is tracked in an LDS bitmap of N bits (128 KB) and the
//                     keys go to a per-workgroup scratch.  With S <= 8192 every thread
//                     holds its draws' keys in registers and one register radix select
//                     over them and the top-up keys gives tau; otherwise draws are made
//                     four at a time per thread, the top-digit histogram is built on the
//                     way and tau comes from a radix select (LDS reused as the sort
//                     buffer).  Wavefront 0 tops the sample up.  Both samplers also
//                     clear the row's counter for the filter.  Longer rows take
//                     sample_kernel (k_sample.hip) with a row dimension instead: one
//                     hash set per row in device memory.
//   filter_kernel     (k_filter.hip) one streaming pass over all listed rows.
//   b_refine_kernel   one 256-thread workgroup per row, dynamic LDS sized per path.
//                     Buffers of up to kBatchedMaxM = 16384 keys are loaded into LDS:
//                     for k <= kSelCap the k-th largest is found by a radix select
//                     there and the k keys at or above it are sorted (one wavefront in
//                     registers up to 64, else an LDS bitonic sort); for larger k the
//                     whole buffer is sorted (LDS of pow2(M) keys).  Larger buffers
//                     select the k-th over global memory (the one-workgroup radix
//                     select over L2) and sort the k keys at or above it in LDS; an
//                     inconsistent select is reported in the row's attempt record.
//   b_rowsort_kernel  rows of up to 16384 values where the sample would not pay off
//                     (all rows of at most 8192): exact top-k by sorting the whole row
//                     in LDS.
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

constexpr u32 kDrawMax = 8;  // draws per thread held in registers on the fast path

// One row of the fast path; s_bits / s_D / s_fail are clear on entry.  Every thread
// holds its draws' keys in registers; after the top-up (whose keys wavefront 0 also
// stages in s_list) one radix select over the registers and the staged keys gives the
// t-th largest, with the select's state in the bitmap's LDS (the row is drawn by then).
// (Sorting each wavefront's keys in registers and merging the sixteen lists took about
// 20 us per row, the select a few.)
__device__ __forceinline__ void b_sample_fast_row(const BatchedArgs& a, u32 row, const float* xr, u64* keys,
                                                  u32* s_bits, u64* s_list, BlockSelectLds* s_sel, u32* s_D,
                                                  u32* s_fail) {
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  u32 idx[kDrawMax];
  bool fr[kDrawMax];
#pragma unroll
  for (u32 q = 0; q < kDrawMax; ++q) {
    const u64 j = (u64)q * blockDim.x + threadIdx.x;
    fr[q] = false;
    idx[q] = 0;
    if (j < a.S) {
      idx[q] = (u32)sample_draw(j, row, a.attempt, a.seed, a.N);
      const u32 bit = 1u << (idx[q] & 31u);
      fr[q] = (atomicOr(&s_bits[idx[q] >> 5], bit) & bit) == 0;
    }
  }
  u32 vb[kDrawMax];
#pragma unroll
  for (u32 q = 0; q < kDrawMax; ++q) vb[q] = fr[q] ? reinterpret_cast<const u32*>(xr)[idx[q]] : 0u;  // in flight together
  u64 key[kDrawMax];
  u32 nf = 0;
#pragma unroll
  for (u32 q = 0; q < kDrawMax; ++q) {
    key[q] = fr[q] ? make_key(vb[q], idx[q]) : 0ull;  // 0: a repeat (no valid key is 0)
    const u64 j = (u64)q * blockDim.x + threadIdx.x;
    if (j < a.S) keys[j] = key[q];
    nf += (u32)__popcll(__ballot(fr[q]));
  }
  if (lane == 0 && nf) atomicAdd(s_D, nf);
  __syncthreads();
  const u32 D0 = *s_D;
  // top-up by wavefront 0 into keys[S..]
  if (wid == 0) {
    u64 D = D0;
    u64 j0 = a.S;
    u32 guard = 0;
    while (D < a.S) {
      const u32 id2 = (u32)sample_draw(j0 + lane, row, a.attempt, a.seed, a.N);
      // a draw whose bit another lane of this chunk set first repeats within the chunk;
      // only then do the lanes compare indices (see pipe_finish)
      const u32 bit = 1u << (id2 & 31u);
      const bool held = (s_bits[id2 >> 5] & bit) != 0u;
      const bool dup = !held && (atomicOr(&s_bits[id2 >> 5], bit) & bit) != 0u;
      bool repeat = dup;
      if (__ballot(dup)) {
        repeat = false;
        for (int d = 1; d < kWave; ++d) {
          const u32 other = __shfl_up(id2, d, kWave);
          if ((int)lane >= d && other == id2) repeat = true;
        }
      }
      const bool ok2 = !held && !repeat;
      const u64 m2 = __ballot(ok2);
      const u64 need = a.S - D;
      const u32 r = count_below(m2);
      if (ok2 && r < need) {
        const u64 k2 = make_key(__float_as_uint(xr[id2]), id2);
        keys[a.S + (D - D0) + r] = k2;
        if ((D - D0) + r < kBThreads) s_list[(D - D0) + r] = k2;
      }
      const u64 got = (u64)__popcll(m2);
      D += got < need ? got : need;
      j0 += kWave;
      if (++guard > (1u << 22)) {  // bounded: S <= N/2 makes each draw new with prob >= 1/2
        if (lane == 0) *s_fail = 1;
        break;
      }
    }
    if (lane == 0) *s_D = (u32)D;
  }
  __syncthreads();
  const bool sample_ok = !*s_fail && *s_D == a.S;
  const u64 E = sample_ok ? a.S - D0 : 0;
  u64 tau = 0;
  bool ok = sample_ok;
  if (sample_ok && E <= kBThreads) {
    u64 v[kDrawMax + 1];
#pragma unroll
    for (u32 q = 0; q < kDrawMax; ++q) v[q] = key[q];
    v[kDrawMax] = threadIdx.x < E ? s_list[threadIdx.x] : 0ull;  // top-up key threadIdx.x
    tau = reg_select_desc(v, (u32)a.t, reinterpret_cast<LdsSelect*>(s_bits));
    ok = tau != 0;
  } else if (sample_ok) {
    // many top-up keys: radix select over all key slots (repeats are empty slots)
    if (threadIdx.x == 0) block_select_start(s_sel, a.S, a.t);
    __syncthreads();
    tau = block_select_finish(keys, a.S + E, reinterpret_cast<u64*>(s_bits), kBitmapWords / 2, s_sel, &ok);
  }
  if (threadIdx.x == 0) {
    RowCtl* c = &a.ctls[row];
    c->tau = tau;
    c->R = 0;
    c->status = ok && tau != 0 ? 0u : 3u;
  }
}

__global__ __launch_bounds__(kBThreads) void b_sample_kernel(BatchedArgs a) {
  __shared__ __align__(16) u32 s_bits[kBitmapWords];
  __shared__ BlockSelectLds s_sel;
  __shared__ u64 s_list[kBThreads];  // fast path: the top-up keys
  __shared__ u32 s_D;
  __shared__ u32 s_fail;
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  u64* keys = a.scratch + (u64)blockIdx.x * 2 * a.S;  // S draw slots + the top-up
  const u32 nwords = (u32)((a.N + 31) / 32);
  // Fast path (S <= 1024 * kDrawMax): every thread holds its draws' keys in registers
  // and one register radix select gives tau (b_sample_fast_row).
  const bool fast = a.t >= 1 && a.S <= (u64)kBThreads * kDrawMax;
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
    if (fast) {
      b_sample_fast_row(a, row, xr, keys, s_bits, s_list, &s_sel, &s_D, &s_fail);
      continue;
    }
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
        const u32 bit = 1u << (id2 & 31u);
        const bool held = (s_bits[id2 >> 5] & bit) != 0u;
        const bool dup = !held && (atomicOr(&s_bits[id2 >> 5], bit) & bit) != 0u;
        bool repeat = dup;
        if (__ballot(dup)) {
          repeat = false;
          for (int d = 1; d < kWave; ++d) {
            const u32 other = __shfl_up(id2, d, kWave);
            if ((int)lane >= d && other == id2) repeat = true;
          }
        }
        const bool ok2 = !held && !repeat;
        const u64 m2 = __ballot(ok2);
        const u64 need = a.S - D;
        const u32 r = count_below(m2);
        if (ok2 && r < need) {
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

// One workgroup per row (persistent over the listed rows).  A row of at most 64
// candidates is sorted by one wavefront in registers.  Otherwise the candidates are
// loaded into LDS, the k-th largest is found by a radix select there, the k keys at or
// above it are gathered and sorted (one wavefront in registers up to 64, else an LDS
// bitonic sort) and written out; for k above kSelCap the whole row is sorted in LDS.
constexpr u32 kRefineThreads = 256;
constexpr u32 kSelCap = kBatchedSelCap;

// ---------------------------------------------------------------------------------
// Pipelined sampler for S <= kPipeMaxS: while one row's top-up and threshold select
// run, the next row's draws are already in their own LDS hash set and their gathers are
// in flight, so the memory system is not left idle between a workgroup's rows (a
// barrier does not wait for vector loads on this part, so they stay in flight across
// the select's barriers).  Membership is a linear-probing hash set of row indices
// (kPipeH slots, load at most one half) instead of an N-bit map, so that two rows' sets
// fit in LDS at once.
// Wavefront 0 gathers the first kWave top-up draws of a row together with the row's
// own draws; the top-up then needs a further gather only when more than those are
// needed (rows whose sample repeats itself a lot: S close to N / 2).
constexpr u32 kPipeDraws = 4;                    // draws per thread
constexpr u32 kPipeMaxS = kBThreads * kPipeDraws;  // 4096
constexpr u32 kPipeHBits = 13;
constexpr u32 kPipeH = 1u << kPipeHBits;  // >= 2 kPipeMaxS: the set is never full
constexpr u32 kPipeEmpty = ~0u;           // no row index (N <= 2^20)

__device__ __forceinline__ u32 pipe_slot(u32 idx) { return (idx * 0x9E3779B1u) >> (32u - kPipeHBits); }

// Adds idx to the set; true when it was not there.  Ends: the set holds at most
// kPipeMaxS < kPipeH indices, so the probe reaches an empty slot.
__device__ __forceinline__ bool pipe_insert(u32* T, u32 idx) {
  u32 s = pipe_slot(idx);
  for (;;) {
    const u32 old = atomicCAS(&T[s], kPipeEmpty, idx);
    if (old == kPipeEmpty) return true;
    if (old == idx) return false;
    s = (s + 1u) & (kPipeH - 1u);
  }
}

__device__ __forceinline__ bool pipe_held(const u32* T, u32 idx) {
  u32 s = pipe_slot(idx);
  for (;;) {
    const u32 v = T[s];
    if (v == idx) return true;
    if (v == kPipeEmpty) return false;
    s = (s + 1u) & (kPipeH - 1u);
  }
}

// One row in flight: its draws, their gathered bits (loads possibly outstanding), which
// draws were new to the set, and (wavefront 0) the first top-up draw and its bits.
struct PipeRow {
  u32 row;
  u32 idx[kPipeDraws];
  u32 val[kPipeDraws];
  u32 fresh;  // bit q: draw q put its index into the set (one draw per distinct index)
  u32 sidx, sval;
};

struct PipeLds {
  u32 T[2][kPipeH];
  u64 list[kPipeMaxS];  // top-up keys of the row being selected
  LdsSelect sel;
  u32 wempty[kBThreads / kWave];  // per wavefront: its empty register slots
  u32 D[2];                        // distinct indices among a row's S draws
  u32 Dfin, fail;
};

// Row `row`'s draws (indices only).  S = 0 (no next row) draws nothing, and its loads
// (pipe_gather) then read index 0, so that the number of loads in flight does not depend
// on the path taken.
__device__ __forceinline__ void pipe_draw(const BatchedArgs& a, u32 row, u64 S, PipeRow& p) {
  const u32 wid = threadIdx.x / kWave;
  p.row = row;
  // opaque thread index: otherwise the row-independent part of each draw's first
  // round is hoisted out of the row loop and held in registers across it
  const u32 tid = opaque_u32(threadIdx.x);
#pragma unroll
  for (u32 q = 0; q < kPipeDraws; ++q) {
    const u64 j = (u64)q * kBThreads + tid;
    p.idx[q] = j < S ? (u32)sample_draw(j, row, a.attempt, a.seed, a.N) : 0u;
  }
  // wavefront 0: the first top-up draw
  p.sidx = wid == 0 && S ? (u32)sample_draw(a.S + (tid & (kWave - 1)), row, a.attempt, a.seed, a.N) : 0u;
}

// Draws Q0..Q1-1 of the drawn row: their gathers issued, then the draws added to set T
// (cleared, and the block synchronised since); the count of new indices is added to *D.
template <u32 Q0, u32 Q1>
__device__ __forceinline__ void pipe_gather(const BatchedArgs& a, u64 S, u32* T, u32* D, PipeRow& p) {
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  const u32* xr = reinterpret_cast<const u32*>(a.x + (u64)p.row * a.ld);
#pragma unroll
  for (u32 q = Q0; q < Q1; ++q) p.val[q] = xr[p.idx[q]];
  if (Q0 == 0) {
    // only wavefront 0 takes the top-up's first draw: every load is another request
    // in the CU's queue, which the gathers of a row fill
    p.sval = wid == 0 ? xr[p.sidx] : 0u;
    p.fresh = 0;
  }
  u32 nf = 0;
#pragma unroll
  for (u32 q = Q0; q < Q1; ++q) {
    const u64 j = (u64)q * kBThreads + threadIdx.x;
    if (j < S && pipe_insert(T, p.idx[q])) p.fresh |= 1u << q;
    nf += (u32)__popcll(__ballot((p.fresh >> q) & 1u));
  }
  if (lane == 0 && nf) atomicAdd(D, nf);
}

// Every wavefront waits here for all of row p's loads, on every path, so that none is
// still in flight when its register is next written.
__device__ __forceinline__ void pipe_wait(const PipeRow& p) {
  static_assert(kPipeDraws == 4, "the wait names every draw");
  asm volatile("" ::"v"(p.val[0]), "v"(p.val[1]), "v"(p.val[2]), "v"(p.val[3]), "v"(p.sval));
}

// The row's top-up (wavefront 0), its threshold and its control block; p's set is T,
// its count of new indices D0.  The kPipeMaxS register slots of the block hold the D0
// distinct draws and kPipeMaxS - D0 >= S - D0 empty slots (repeats, and draws past
// S), so the top-up keys, staged in L.list, fill empty slots: a block-wide scan of the
// empty slots gives each thread its range of L.list, and one register radix select over
// the slots gives tau.
// `mid` runs once the top-up is done, before the select, and `late` inside the select
// after its first barrier (they issue the next row's remaining gathers).
template <class Mid, class Late>
__device__ __forceinline__ void pipe_finish(const BatchedArgs& a, PipeRow& p, u32* T, PipeLds& L, u32 D0,
                                            bool has_row, Mid&& mid, Late&& late) {
  // has_row is false (block-uniformly) in a workgroup's last step, whose row is the
  // loads of index 0 that stand in for a next row; mid() still runs, in the one place
  // both cases share, so that the wait analysis sees one path through the loads
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  u64 key[kPipeDraws];
#pragma unroll
  for (u32 q = 0; q < kPipeDraws; ++q) key[q] = (p.fresh >> q) & 1u ? make_key(p.val[q], p.idx[q]) : 0ull;
  u64* keep = a.keep_keys && has_row ? a.scratch + (u64)p.row * 2 * a.S : nullptr;
  if (keep) {
#pragma unroll
    for (u32 q = 0; q < kPipeDraws; ++q) {
      const u64 j = (u64)q * kBThreads + threadIdx.x;
      if (j < a.S) keep[j] = key[q];
    }
  }
  const u32 empty = kPipeDraws - (u32)__popc(p.fresh);
  const u32 incl = wave_incl_scan_add(empty, lane);
  if (lane == kWave - 1) L.wempty[wid] = incl;
  if (has_row && wid == 0) {
    const u32* xr = reinterpret_cast<const u32*>(a.x + (u64)p.row * a.ld);
    u64 D = D0;
    u64 j0 = a.S;
    u32 guard = 0;
    bool first = true;
    while (D < a.S) {
      u32 id2, v2;
      if (first) {
        id2 = p.sidx;
        v2 = p.sval;
      } else {
        id2 = (u32)sample_draw(j0 + lane, p.row, a.attempt, a.seed, a.N);
        v2 = xr[id2];
        asm volatile("" ::"v"(v2));  // waited here even where no lane takes it
      }
      first = false;
      // A draw is taken when its index is neither in the set nor drawn by a lower lane
      // of this chunk.  Every draw not in the set is inserted; a draw that then finds
      // its index inserted by another lane of the chunk is a repeat within the chunk,
      // and only then (about one chunk in 500 at S = 4096, N = 2^20) do the lanes
      // compare indices to find which of the equal draws is the first.  The set then
      // holds the chunk's new indices, the taken ones among them; the others can only
      // be there when the chunk is the last one.
      const bool held = pipe_held(T, id2);
      const bool dup = !held && !pipe_insert(T, id2);
      bool repeat = dup;
      if (__ballot(dup)) {
        repeat = false;
        for (int d = 1; d < kWave; ++d) {
          const u32 other = __shfl_up(id2, d, kWave);
          if ((int)lane >= d && other == id2) repeat = true;
        }
      }
      const bool ok2 = !held && !repeat;
      const u64 m2 = __ballot(ok2);
      const u64 need = a.S - D;
      const u32 r = count_below(m2);
      if (ok2 && r < need) {
        L.list[(D - D0) + r] = make_key(v2, id2);
        if (keep) keep[a.S + (D - D0) + r] = make_key(v2, id2);
      }
      const u64 got = (u64)__popcll(m2);
      D += got < need ? got : need;
      j0 += kWave;
      if (++guard > (1u << 22)) {  // bounded: S <= N/2 makes each draw new with prob >= 1/2
        if (lane == 0) L.fail = 1;
        break;
      }
    }
    if (lane == 0) L.Dfin = (u32)D;
  }
  __syncthreads();
  mid();
  const bool sample_ok = has_row && !L.fail && L.Dfin == a.S;
  if (sample_ok) {
    const u32 E = (u32)(a.S - D0);
    // first empty slot of this thread in the block's order (wavefronts, then lanes)
    u32 e = incl - empty + wave_sum32(lane < wid ? L.wempty[lane] : 0u);
#pragma unroll
    for (u32 q = 0; q < kPipeDraws; ++q)
      if (key[q] == 0) {
        if (e < E) key[q] = L.list[e];
        ++e;
      }
  } else {
#pragma unroll
    for (u32 q = 0; q < kPipeDraws; ++q) key[q] = 0;  // no keys: the select returns 0
  }
  // the select runs on every path (also with no row: its barriers order the reads of
  // L.fail / L.Dfin before their reset, and `late` has one place)
  const u64 tau = reg_select_desc(key, (u32)a.t, &L.sel, late);
  if (!has_row) return;
  if (threadIdx.x == 0) {
    // the row's whole control block, as attempt_init leaves it, with tau and its status
    RowCtl c{};
    c.key_and = ~0ull;
    c.tau = tau;
    c.status = tau != 0 ? 0u : 3u;
    a.ctls[p.row] = c;
    if (a.rec) a.rec[p.row] = AttemptRecord{0ull, 0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void pipe_clear(u32* T) {
  uint4* t = reinterpret_cast<uint4*>(T);
  for (u32 i = threadIdx.x; i < kPipeH / 4; i += kBThreads) t[i] = make_uint4(kPipeEmpty, kPipeEmpty, kPipeEmpty, kPipeEmpty);
}

// Listed row l, read through the scalar cache: its wait then does not wait for the
// gathers in flight (the list is not written while the kernel runs).
__device__ __forceinline__ u32 pipe_row_of(const BatchedArgs& a, u64 l) {
  if (!a.rows) return (u32)l;
  const __attribute__((address_space(4))) int* r = (const __attribute__((address_space(4))) int*)a.rows;
  return (u32)r[l];
}

// One step: row `cur` (set T[c]; none when !has_cur) is finished while listed row li2
// (set T[c ^ 1]) is drawn and gathered into `nxt`, if there is one.
__device__ __forceinline__ void pipe_step(const BatchedArgs& a, PipeLds& L, u32 c, PipeRow& cur, PipeRow& nxt,
                                          bool has_cur, u64 li2) {
  const bool more = li2 < a.nrows;
  pipe_clear(L.T[c ^ 1u]);
  if (threadIdx.x == 0) {
    L.D[c ^ 1u] = 0;
    L.fail = 0;
  }
  __syncthreads();  // cur's count complete; T[c ^ 1] clear; the last select's users done
  const u32 D0 = L.D[c];
  const u64 S2 = more ? a.S : 0;
  pipe_draw(a, more ? pipe_row_of(a, li2) : cur.row, S2, nxt);
  // One row's gathers in flight at a time: with two, random gathers ran at about 42 G/s
  // against about 49 G/s with one (a probe of this launch shape on MI355X).  The next
  // row's gathers are issued as soon as cur's have arrived, and cur's top-up and
  // threshold run while they are in flight.
  pipe_wait(cur);
  // in three slices: now, after cur's top-up, and inside cur's select (a wavefront that
  // issues a load while the CU's request queue is full stalls, and with it every
  // barrier of the block)
  pipe_gather<0, 1>(a, S2, L.T[c ^ 1u], &L.D[c ^ 1u], nxt);
  pipe_finish(
      a, cur, L.T[c], L, D0, has_cur, [&] { pipe_gather<1, 2>(a, S2, L.T[c ^ 1u], &L.D[c ^ 1u], nxt); },
      [&] { pipe_gather<2, kPipeDraws>(a, S2, L.T[c ^ 1u], &L.D[c ^ 1u], nxt); });
}

__global__ __launch_bounds__(kBThreads) void b_sample_pipe_kernel(BatchedArgs a) {
  __shared__ PipeLds L;
  PipeRow ra, rb;
  u64 li = blockIdx.x;
  if (blockIdx.x == 0 && a.tickets)
    for (u32 i = threadIdx.x; i < kTicketWords; i += kBThreads) a.tickets[i] = 0;
  if (li >= a.nrows) return;
  pipe_clear(L.T[0]);
  if (threadIdx.x == 0) {
    L.D[0] = 0;
    L.fail = 0;
  }
  __syncthreads();
  pipe_draw(a, pipe_row_of(a, li), a.S, ra);
  pipe_gather<0, kPipeDraws>(a, a.S, L.T[0], &L.D[0], ra);
  // two register sets used in turn, so that no row's in-flight loads are copied.  The
  // loop's one exit is at the bottom: an exit between the two steps would give the wait
  // analysis a path from the first step's loads to the loop head, where it would then
  // wait for them before the first step issues the next row's.
  for (;;) {
    const u64 li2 = li + gridDim.x, li3 = li2 + gridDim.x;
    pipe_step(a, L, 0, ra, rb, true, li2);
    pipe_step(a, L, 1, rb, ra, li2 < a.nrows, li3);
    if (li3 >= a.nrows) return;
    li = li3;
  }
}

namespace {
// Value bits from a key's order code, except the codes that fold encodings (+-0, NaN).
__device__ __forceinline__ u32 row_value_bits(u64 key, const float* row, u32 idx) {
  const u32 o = (u32)(key >> 32);
  if (o == 0x80000000u || o == 0xFFFFFFFFu) return reinterpret_cast<const u32*>(row)[idx];
  return bits_of_ord32(o);
}

__device__ __forceinline__ u64 cand_at(const BatchedArgs& a, u32 row, u32 i) { return a.cand[(u64)row * a.M + i]; }

__device__ __forceinline__ void write_row_key(u64 key, u64 j, const float* row, u64 N, float* ov, int64_t* oi) {
  const u32 idx = key_index(key);
  oi[j] = idx < N ? (int64_t)idx : -1;
  if (idx < N) reinterpret_cast<u32*>(ov)[j] = row_value_bits(key, row, idx);
}
}  // namespace

__global__ __launch_bounds__(kRefineThreads) void b_refine_kernel(BatchedArgs a) {
  extern __shared__ u64 s[];  // M keys (k <= kSelCap), pow2(M) (k > kSelCap) or kBatchedMaxM (M above it)
  __shared__ u64 s_top[kSelCap];
  __shared__ LdsSelect s_sel;
  __shared__ BlockSelectLds s_bsel;
  __shared__ u32 s_n;
  const u32 tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  for (u64 li = blockIdx.x; li < a.nrows; li += gridDim.x) {
    const u32 row = a.rows ? (u32)a.rows[li] : (u32)li;
    if (a.table) {  // this position's sample hash set, zero again for the next attempt
      uint4* t = reinterpret_cast<uint4*>(a.table + li * a.table_slots);
      for (u64 i = tid; i < a.table_slots / 4; i += kRefineThreads) t[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    const RowCtl* c = &a.ctls[row];
    const u32 status = c->status;  // uniform per workgroup
    // exact mode refines rows whose check held; approximate mode also the others
    const bool live = status == 0 || (a.approx && (status == 1u || status == 2u));
    const u64 R = c->R;
    const u32 n = live ? (u32)(R < a.M ? R : a.M) : 0u;
    const float* xr = a.x + (u64)row * a.ld;
    float* ov = a.out_vals + (u64)row * a.k;
    int64_t* oi = a.out_idx + (u64)row * a.k;
    if (a.approx) {
      if (tid == 0 && a.info) {
        ApproxInfo inf;
        inf.R = (int64_t)R;
        inf.M = (int64_t)a.M;
        inf.status = (int32_t)status;
        inf.exact_path = 0;
        a.info[row] = inf;
      }
      for (u64 p = n + tid; p < a.k; p += kRefineThreads) {  // fewer than k kept
        oi[p] = -1;
        reinterpret_cast<u32*>(ov)[p] = 0xFF800000u;  // -inf
      }
    }
    if (n == 0) continue;
    const u32 kk = (u32)(a.k < n ? a.k : n);  // outputs this row gets (k unless fewer were kept)
    if (n <= (u32)kWave) {
      if (wid == 0) {
        const u64 v = wave_sort_desc(lane < n ? cand_at(a, row, lane) : 0ull);
        if (lane < kk) write_row_key(v, lane, xr, a.N, ov, oi);
      }
      continue;
    }
    const u64* cand = a.cand + (u64)row * a.M;
    __syncthreads();  // the previous row's users of s are done
    if (n > kBatchedMaxM) {
      // more candidates than LDS holds: the k-th largest by the one-workgroup radix
      // select over the buffer in global memory, then the k keys at or above it (k <=
      // kBatchedMaxM, the host's bound) are gathered into LDS and sorted there
      bool ok = false;
      const u64 kth = block_select_rank(cand, n, kk, s, (u32)kBatchedMaxM, &s_bsel, &ok);
      if (!ok) {
        // the select came back inconsistent (never expected): report it instead of
        // writing k arbitrary keys; the host turns it into PROFK_EINTERNAL
        if (tid == 0 && a.rec) a.rec[row].error = 1u;
        continue;  // uniform per workgroup
      }
      if (tid == 0) s_n = 0;
      __syncthreads();
      for (u32 i = tid; i < n; i += kRefineThreads) {
        const u64 key = cand[i];
        if (key >= kth) {
          const u32 slot = atomicAdd(&s_n, 1u);
          if (slot < (u32)kBatchedMaxM) s[slot] = key;
        }
      }
      __syncthreads();
      const u32 m = s_n < kk ? s_n : kk;  // exactly kk: the keys are distinct
      u32 P = 1;
      while (P < m) P <<= 1;
      for (u32 i = m + tid; i < P; i += kRefineThreads) s[i] = 0ull;
      __syncthreads();
      block_bitonic_desc(s, P);
      for (u32 j = tid; j < m; j += kRefineThreads) write_row_key(s[j], j, xr, a.N, ov, oi);
      continue;
    }
    constexpr u32 kILP = 8;
    for (u32 base = 0; base < n; base += kRefineThreads * kILP) {
      u64 kv[kILP];
#pragma unroll
      for (u32 q = 0; q < kILP; ++q) {
        const u32 i = base + q * kRefineThreads + tid;
        kv[q] = i < n ? cand[i] : 0ull;
      }
#pragma unroll
      for (u32 q = 0; q < kILP; ++q) {
        const u32 i = base + q * kRefineThreads + tid;
        if (i < n) s[i] = kv[q];
      }
    }
    __syncthreads();
    if (a.k <= kSelCap) {
      const u64 kth = lds_select_desc(s, n, kk, &s_sel);
      if (tid == 0) s_n = 0;
      __syncthreads();
      for (u32 i = tid; i < n; i += kRefineThreads) {
        const u64 key = s[i];
        if (key >= kth) {
          const u32 slot = atomicAdd(&s_n, 1u);
          if (slot < kSelCap) s_top[slot] = key;
        }
      }
      __syncthreads();
      const u32 m = s_n < kk ? s_n : kk;  // exactly kk: the keys are distinct
      if (m <= (u32)kWave) {
        if (wid == 0) {
          const u64 v = wave_sort_desc(lane < m ? s_top[lane] : 0ull);
          if (lane < m) write_row_key(v, lane, xr, a.N, ov, oi);
        }
      } else {
        u32 P = 1;
        while (P < m) P <<= 1;
        for (u32 i = m + tid; i < P; i += kRefineThreads) s_top[i] = 0ull;
        __syncthreads();
        block_bitonic_desc(s_top, P);
        for (u32 j = tid; j < m; j += kRefineThreads) write_row_key(s_top[j], j, xr, a.N, ov, oi);
      }
    } else {
      u32 P = 1;
      while (P < n) P <<= 1;
      for (u32 i = n + tid; i < P; i += kRefineThreads) s[i] = 0ull;
      __syncthreads();
      block_bitonic_desc(s, P);
      for (u32 j = tid; j < kk; j += kRefineThreads) write_row_key(s[j], j, xr, a.N, ov, oi);
    }
  }
}

__global__ __launch_bounds__(kBThreads) void b_rowsort_kernel(BatchedArgs a) {
  extern __shared__ u64 s[];  // pow2(N) keys, N <= kBatchedMaxM
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

// Approximate mode, rows sorted whole (the exact result): info[r] = {N, 0, 0, 1}.
__global__ void b_info_exact_kernel(ApproxInfo* info, u64 nrows, u64 N) {
  for (u64 r = (u64)blockIdx.x * blockDim.x + threadIdx.x; r < nrows; r += (u64)gridDim.x * blockDim.x) {
    ApproxInfo inf;
    inf.R = (int64_t)N;
    inf.M = 0;
    inf.status = 0;
    inf.exact_path = 1;
    info[r] = inf;
  }
}

hipError_t launch_b_info_exact(ApproxInfo* info, u64 nrows, u64 N, hipStream_t s) {
  u64 g = (nrows + 255) / 256;
  if (g > 1024) g = 1024;
  b_info_exact_kernel<<<(u32)(g ? g : 1), 256, 0, s>>>(info, nrows, N);
  return hipGetLastError();
}

namespace {
u32 row_grid(u64 nrows, u32 per_cu) {
  u64 g = (u64)device_cu_count() * per_cu;
  if (g > nrows) g = nrows;
  return (u32)(g ? g : 1);
}
}  // namespace

u32 batched_sample_blocks(u64 nrows) { return row_grid(nrows, 1); }

bool b_sample_pipelined(u64 S, u64 t, u64 N) { return t >= 1 && S <= kPipeMaxS && N <= kBatchedMaxN; }

hipError_t launch_b_sample(const BatchedArgs& a, hipStream_t s, u32 grid) {
  if (b_sample_pipelined(a.S, a.t, a.N)) {
    b_sample_pipe_kernel<<<batched_sample_blocks(a.nrows), kBThreads, 0, s>>>(a);
    return hipGetLastError();
  }
  if (!grid) grid = batched_sample_blocks(a.nrows);
  b_sample_kernel<<<grid, kBThreads, 0, s>>>(a);
  return hipGetLastError();
}

// Stage entry point of the batched sampler (one sampling workgroup per row, so row r's
// keys stay in scratch[r * 2S .. r * 2S + 2S), zero on entry): row r's sample indices
// in any order to out_idx[r * S ..], its threshold to out_tau_*[r], its status to rec[r].
__global__ __launch_bounds__(256) void b_stage_out_kernel(const float* x, u64 ld, u64 N, u64 S, const u64* scratch,
                                                          const RowCtl* ctls, int64_t* out_idx, float* out_tau_val,
                                                          int64_t* out_tau_idx, AttemptRecord* rec) {
  __shared__ u32 s_cnt;
  const u32 row = blockIdx.x;
  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();
  const u64* keys = scratch + (u64)row * 2 * S;
  for (u64 i0 = 0; i0 < 2 * S; i0 += blockDim.x) {
    const u64 i = i0 + threadIdx.x;
    const u64 key = i < 2 * S ? keys[i] : 0ull;
    const u32 slot = wave_reserve32(&s_cnt, key != 0);
    if (key != 0 && slot < S) out_idx[(u64)row * S + slot] = (int64_t)key_index(key);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const RowCtl* c = &ctls[row];
    const u32 idx = key_index(c->tau);
    const bool ok = c->status == 0 && idx < N && s_cnt == S;
    out_tau_idx[row] = ok ? (int64_t)idx : -1;
    if (ok) reinterpret_cast<u32*>(out_tau_val)[row] = reinterpret_cast<const u32*>(x + (u64)row * ld)[idx];
    rec[row].status = ok ? 0u : 3u;
  }
}

hipError_t launch_b_stage_out(const float* x, u64 ld, u64 N, u64 B, u64 S, const u64* scratch, const RowCtl* ctls,
                              int64_t* out_idx, float* out_tau_val, int64_t* out_tau_idx, AttemptRecord* rec,
                              hipStream_t s) {
  b_stage_out_kernel<<<(u32)B, 256, 0, s>>>(x, ld, N, S, scratch, ctls, out_idx, out_tau_val, out_tau_idx, rec);
  return hipGetLastError();
}

hipError_t launch_b_refine(const BatchedArgs& a, hipStream_t s) {
  // keys of LDS the rows need: the select path holds at most M, the whole-buffer sort
  // pow2(M), and a buffer past kBatchedMaxM is selected over in global memory with an
  // LDS buffer of kBatchedMaxM.  Two workgroups per CU while this stays near 64 KB.
  u64 keys = a.M;
  if (a.M > kBatchedMaxM) {
    keys = kBatchedMaxM;
  } else if (a.k > kSelCap) {
    keys = 1;
    while (keys < a.M) keys <<= 1;
  }
  const size_t lds = (size_t)keys * sizeof(u64);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&b_refine_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  b_refine_kernel<<<row_grid(a.nrows, 2), kRefineThreads, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_b_rowsort(const BatchedArgs& a, hipStream_t s) {
  if (a.N > kBatchedMaxM) return hipErrorInvalidValue;
  u32 P = 1;
  while (P < a.N) P <<= 1;
  const size_t lds = (size_t)P * sizeof(u64);  // at most 128 KB
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&b_rowsort_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  b_rowsort_kernel<<<row_grid(a.nrows, 2), kBThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace profk
