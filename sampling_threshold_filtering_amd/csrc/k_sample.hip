// Stage 1 of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
// Selection", §3, stage 1): S indices drawn uniformly without replacement.
//
// The pages leave the procedure open.  The sample here is the set of the first S
// distinct indices of the Philox stream of (seed, attempt, row) in draw order
// (see profk_device.h for the draw).  That rule is symmetric under relabelling of
// [N], so every S-subset is equally likely, and it is deterministic per seed.
//
//   sample_kernel   one thread per draw 0..S-1: each index goes into a hash set in
//                   device memory (open addressing, 64-bit slots tagged with a
//                   per-attempt generation so the table never needs clearing); the
//                   first insert of each index gathers x[idx] into a key, and each
//                   block reserves its key slots with one atomic.  The last block
//                   then (a) tops up: while fewer than S distinct indices are held,
//                   wavefront 0 takes further draws S, S+1, ... in order, 64 at a
//                   time, keeping those that are new and not repeated earlier in the
//                   same chunk (expected extra draws about S^2 / (2N)); and (b) selects
//                   tau, the t-th largest of the S keys, by a one-workgroup radix
//                   select (stage 2), so stages 1 and 2 cost a single launch.
#include "block_select.h"
#include "launch.h"

namespace profk {

namespace {

__device__ __forceinline__ u32 mix32(u32 h) {
  // murmur3 finalizer
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// Returns true when idx was not in the set (and is now).
__device__ bool hash_insert(u64* table, u64 tmask, u32 gen, u32 idx) {
  const u64 mine = ((u64)gen << 32) | idx;
  u64 h = mix32(idx) & tmask;
  for (u64 probe = 0; probe <= tmask; ++probe) {
    u64 cur = atomic_load_agent(&table[h]);
    while ((u32)(cur >> 32) != gen) {  // stale slot of an older generation: free
      const u64 prev = atomicCAS(&table[h], cur, mine);
      if (prev == cur) return true;
      cur = prev;
    }
    if ((u32)cur == idx) return false;
    h = (h + 1) & tmask;
  }
  return false;  // unreachable: the table holds at least 2S slots
}

__device__ bool hash_contains(const u64* table, u64 tmask, u32 gen, u32 idx) {
  u64 h = mix32(idx) & tmask;
  for (u64 probe = 0; probe <= tmask; ++probe) {
    const u64 cur = atomic_load_agent(&table[h]);
    if ((u32)(cur >> 32) != gen) return false;
    if ((u32)cur == idx) return true;
    h = (h + 1) & tmask;
  }
  return false;
}

}  // namespace

// Clears every per-attempt counter, record and selection state (histograms
// included) so that nothing depends on what the workspace held before.
__global__ __launch_bounds__(1024) void attempt_init_kernel(RowCtl* ctl, SelState* sel, AttemptRecord* rec,
                                                          u32* tickets, u32 nrows, u32* refine_hist) {
  if (tickets && threadIdx.x < kTickets) tickets[threadIdx.x] = 0;
  if (refine_hist)
    for (u32 b = threadIdx.x; b < kBins; b += blockDim.x) refine_hist[b] = 0;
  if (sel)
    for (u32 r = 0; r < nrows; ++r)
      for (u32 b = threadIdx.x; b < 256; b += blockDim.x) sel[r].hist[b] = 0;
  for (u32 r = threadIdx.x; r < nrows; r += blockDim.x) {
    RowCtl c{};
    c.key_and = ~0ull;
    ctl[r] = c;
    if (rec) rec[r] = AttemptRecord{0ull, 0u, 0u, 0u, 0u};
    if (!sel) continue;
    SelState* s = &sel[r];
    s->prefix = 0;
    s->mask = 0;
    s->rank = 1;
    s->count = 0;
    s->done = 1;
    s->digit = 0;
    s->ticket = 0;
    s->ncol = 0;
    s->error = 0;
  }
}

constexpr u32 kSampleThreads = 1024;
constexpr u32 kTauCap = 8192;  // keys the last block sorts in LDS (64 KB)

// Draws 0..S-1 (one per thread), dedupes them through the hash set and gathers
// the keys of the first inserts; the block reserves its slots with ONE atomic.
// The last block to finish then tops the sample up to exactly S distinct indices
// (wavefront 0, draws S, S+1, ... in order) and, when t > 0, selects
// tau = the t-th largest sampled key (P1 §3 stage 2) into ctl->tau.
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(const float* __restrict__ x, u64 N, u64 S,
                                                                u64 seed, u32 attempt, u32 row, u64* table,
                                                                u64 tmask, u32 gen, u64* __restrict__ keys,
                                                                RowCtl* ctl, u32* ticket, u32* top_hist, u64 t) {
  __shared__ u64 s_buf[kTauCap];
  __shared__ BlockSelectLds s_sel;
  __shared__ u32 s_wcnt[kSampleThreads / kWave];
  __shared__ u64 s_base;
  __shared__ u64 s_D;
  __shared__ u32 s_last;
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  const u64 j = (u64)blockIdx.x * kSampleThreads + threadIdx.x;
  bool fresh = false;
  u32 idx = 0;
  if (j < S) {
    idx = (u32)sample_draw(j, row, attempt, seed, N);
    fresh = hash_insert(table, tmask, gen, idx);
  }
  const u64 m = __ballot(fresh);
  if (lane == 0) s_wcnt[wid] = (u32)__popcll(m);
  __syncthreads();
  if (threadIdx.x == 0) {
    u32 tot = 0;
    for (u32 w = 0; w < kSampleThreads / kWave; ++w) {
      const u32 c = s_wcnt[w];
      s_wcnt[w] = tot;
      tot += c;
    }
    s_base = tot ? atomicAdd(&ctl->D, (u64)tot) : 0ull;
  }
  __syncthreads();
  u64 key = 0;
  if (fresh) {
    key = make_key(__float_as_uint(x[idx]), idx);
    const u64 slot = s_base + s_wcnt[wid] + count_below(m);
    if (slot < S) keys[slot] = key;
  }
  // histogram of the top 8 bits of this block's keys: the first digit of the
  // threshold selection, so the last block starts one pass further on
  for (u32 b = threadIdx.x; b < 256; b += blockDim.x) s_sel.hist[b] = 0;
  __syncthreads();
  wave_hist_add(s_sel.hist, (u32)(key >> 56), fresh);
  __syncthreads();
  for (u32 b = threadIdx.x; b < 256; b += blockDim.x)
    if (s_sel.hist[b]) atomicAdd(&top_hist[b], s_sel.hist[b]);
  // release this block's keys, then elect the last block
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    s_last = (atomicAdd(ticket, 1u) == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // top-up by wavefront 0
  if (wid == 0) {
    u64 D = atomicAdd(&ctl->D, 0ull);
    u64 j0 = S;
    u32 guard = 0;
    bool failed = false;
    while (D < S) {
      const u32 idx2 = (u32)sample_draw(j0 + lane, row, attempt, seed, N);
      const bool held = hash_contains(table, tmask, gen, idx2);
      bool repeat = false;
      for (int d = 1; d < kWave; ++d) {
        const u32 other = __shfl_up(idx2, d, kWave);
        if ((int)lane >= d && other == idx2) repeat = true;
      }
      const bool ok2 = !held && !repeat;
      const u64 m2 = __ballot(ok2);
      const u64 need = S - D;
      const u32 r = count_below(m2);
      if (ok2 && r < need) {
        hash_insert(table, tmask, gen, idx2);
        const u64 key2 = make_key(__float_as_uint(x[idx2]), idx2);
        keys[D + r] = key2;
        atomicAdd(&top_hist[key2 >> 56], 1u);
      }
      const u64 got = (u64)__popcll(m2);
      D += got < need ? got : need;
      j0 += kWave;
      if (++guard > (1u << 22)) {  // bounded: S <= N/2 makes each draw new with prob >= 1/2
        failed = true;
        break;
      }
    }
    if (lane == 0) {
      s_D = failed ? ~0ull : D;
      ctl->D = D;
    }
  }
  __syncthreads();
  const bool sample_ok = s_D == S;
  for (u32 b = threadIdx.x; b < 256; b += blockDim.x) {
    s_sel.hist[b] = atomicAdd(&top_hist[b], 0u);
    top_hist[b] = 0;  // left zero for the next attempt
  }
  __syncthreads();
  if (t > 0) {
    if (threadIdx.x == 0) block_select_start_from_top_hist(&s_sel, s_sel.hist, sample_ok ? S : 0, t);
    __syncthreads();
    bool ok = false;
    const u64 tau = block_select_finish(keys, S, s_buf, kTauCap, &s_sel, &ok);
    if (threadIdx.x == 0) {
      ctl->tau = tau;
      if (!ok) ctl->status = 3;
    }
  } else if (threadIdx.x == 0 && !sample_ok) {
    ctl->status = 3;
  }
  if (threadIdx.x == 0) *ticket = 0;
}

// Stage-level helpers: keys -> int64 indices, tau -> (value, index).
__global__ void keys_to_index_kernel(const u64* __restrict__ keys, const u64* n_ptr, u64 n_cap,
                                     int64_t* __restrict__ out) {
  u64 n = *n_ptr;
  if (n > n_cap) n = n_cap;
  for (u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (u64)gridDim.x * blockDim.x)
    out[i] = (int64_t)key_index(keys[i]);
}

__global__ void tau_to_output_kernel(const float* __restrict__ x, u64 N, const RowCtl* ctl, float* out_val,
                                     int64_t* out_idx) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const u32 idx = key_index(ctl->tau);
    if (ctl->status != 0 || idx >= N) {  // no threshold was selected
      out_idx[0] = -1;
      return;
    }
    out_idx[0] = (int64_t)idx;
    out_val[0] = x[idx];
  }
}

__global__ void set_tau_kernel(RowCtl* ctl, u32* tickets, u32 tau_bits, u32 tau_idx) {
  if (blockIdx.x == 0 && threadIdx.x < kTickets) tickets[threadIdx.x] = 0;
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    RowCtl c{};
    c.key_and = ~0ull;
    c.tau = make_key(tau_bits, tau_idx);
    *ctl = c;
  }
}

__global__ void r_to_output_kernel(const RowCtl* ctl, int64_t* out_R) {
  if (threadIdx.x == 0 && blockIdx.x == 0) out_R[0] = (int64_t)ctl->R;
}

// ---------------------------------------------------------------------------
hipError_t launch_attempt_init(RowCtl* ctl, SelState* sel, AttemptRecord* rec, u32* tickets, u32 nrows,
                               u32* refine_hist, hipStream_t s) {
  attempt_init_kernel<<<1, 1024, 0, s>>>(ctl, sel, rec, tickets, nrows, refine_hist);
  return hipGetLastError();
}

hipError_t launch_sample(const float* x, u64 N, u64 S, u64 seed, u32 attempt, u32 row, u64* table, u64 tmask,
                         u32 gen, u64* keys, RowCtl* ctl, u32* ticket, u32* top_hist, u64 t, hipStream_t s) {
  const u32 blocks = (u32)((S + kSampleThreads - 1) / kSampleThreads);
  sample_kernel<<<blocks, kSampleThreads, 0, s>>>(x, N, S, seed, attempt, row, table, tmask, gen, keys, ctl, ticket,
                                                  top_hist, t);
  return hipGetLastError();
}

hipError_t launch_keys_to_index(const u64* keys, const u64* n_ptr, u64 n_cap, int64_t* out, hipStream_t s) {
  u32 blocks = (u32)((n_cap + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  keys_to_index_kernel<<<blocks, 256, 0, s>>>(keys, n_ptr, n_cap, out);
  return hipGetLastError();
}

hipError_t launch_tau_to_output(const float* x, u64 N, const RowCtl* ctl, float* out_val, int64_t* out_idx,
                                hipStream_t s) {
  tau_to_output_kernel<<<1, 64, 0, s>>>(x, N, ctl, out_val, out_idx);
  return hipGetLastError();
}

hipError_t launch_set_tau(RowCtl* ctl, u32* tickets, u32 tau_bits, u32 tau_idx, hipStream_t s) {
  set_tau_kernel<<<1, 64, 0, s>>>(ctl, tickets, tau_bits, tau_idx);
  return hipGetLastError();
}

hipError_t launch_r_to_output(const RowCtl* ctl, int64_t* out_R, hipStream_t s) {
  r_to_output_kernel<<<1, 64, 0, s>>>(ctl, out_R);
  return hipGetLastError();
}

}  // namespace profk
