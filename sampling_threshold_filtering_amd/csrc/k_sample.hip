// Stage 1 of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
// Selection", §3, stage 1): S indices drawn uniformly without replacement.
//
// The pages leave the procedure open.  The sample here is the set of the first S
// distinct indices of the Philox stream of (seed, attempt, row) in draw order
// (see profk_device.h for the draw).  That rule is symmetric under relabelling of
// [N], so every S-subset is equally likely, and it is deterministic per seed.
//
//   sample_draw_kernel   draws 0..S-1 in parallel; each index goes into a hash set in
//                        device memory (open addressing, 64-bit slots tagged with a
//                        per-attempt generation so the table never needs clearing);
//                        the first insert of each index gathers x[idx] into a key.
//   sample_topup_kernel  one wavefront: while fewer than S distinct indices are held,
//                        takes further draws S, S+1, ... in order, 64 at a time,
//                        keeping those that are new and not repeated earlier in the
//                        same chunk, until exactly S are held.  Expected extra draws
//                        are about S^2 / (2N).
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
__global__ __launch_bounds__(64) void attempt_init_kernel(RowCtl* ctl, SelState* sel, AttemptRecord* rec,
                                                          u32* tickets, u32 nrows) {
  if (tickets && threadIdx.x < kTickets) tickets[threadIdx.x] = 0;
  for (u32 r = 0; r < nrows; ++r)
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x) sel[r].hist[b] = 0;
  for (u32 r = threadIdx.x; r < nrows; r += blockDim.x) {
    RowCtl c{};
    c.key_and = ~0ull;
    ctl[r] = c;
    if (rec) rec[r] = AttemptRecord{0ull, 0u, 0u};
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

__global__ __launch_bounds__(256) void sample_draw_kernel(const float* __restrict__ x, u64 N, u64 S, u64 seed,
                                                          u32 attempt, u32 row, u64* table, u64 tmask, u32 gen,
                                                          u64* __restrict__ keys, RowCtl* ctl) {
  const u64 j = (u64)blockIdx.x * blockDim.x + threadIdx.x;
  bool fresh = false;
  u32 idx = 0;
  if (j < S) {
    idx = (u32)sample_draw(j, row, attempt, seed, N);
    fresh = hash_insert(table, tmask, gen, idx);
  }
  const u64 slot = wave_reserve(&ctl->D, fresh);
  if (fresh && slot < S) keys[slot] = make_key(__float_as_uint(x[idx]), idx);
}

// One wavefront.  Also arms the threshold selection (rank t among the S keys).
__global__ __launch_bounds__(64) void sample_topup_kernel(const float* __restrict__ x, u64 N, u64 S, u64 seed,
                                                          u32 attempt, u32 row, u64* table, u64 tmask, u32 gen,
                                                          u64* __restrict__ keys, RowCtl* ctl, SelState* sel,
                                                          u64 t) {
  const u32 lane = lane_id();
  u64 D = ctl->D;
  u64 j0 = S;
  u32 guard = 0;
  bool failed = false;
  while (D < S) {
    const u32 idx = (u32)sample_draw(j0 + lane, row, attempt, seed, N);
    const bool held = hash_contains(table, tmask, gen, idx);
    bool repeat = false;
    for (int d = 1; d < kWave; ++d) {
      const u32 other = __shfl_up(idx, d, kWave);
      if ((int)lane >= d && other == idx) repeat = true;
    }
    const bool fresh = !held && !repeat;
    const u64 m = __ballot(fresh);
    const u64 need = S - D;
    const u32 r = count_below(m);
    if (fresh && r < need) {
      hash_insert(table, tmask, gen, idx);
      keys[D + r] = make_key(__float_as_uint(x[idx]), idx);
    }
    const u64 got = (u64)__popcll(m);
    D += got < need ? got : need;
    j0 += kWave;
    if (++guard > (1u << 22)) {  // bounded: S <= N/2 makes each draw new with prob >= 1/2
      failed = true;
      break;
    }
  }
  if (lane == 0) {
    ctl->D = D;
    if (failed) ctl->status = 3;
    sel->prefix = 0;
    sel->mask = 0;
    sel->rank = t;
    sel->count = D;
    sel->done = failed ? 1u : 0u;
    sel->digit = 0;
    sel->ticket = 0;
    sel->ncol = 0;
    sel->error = failed ? 1u : 0u;
  }
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
                               hipStream_t s) {
  attempt_init_kernel<<<1, 64, 0, s>>>(ctl, sel, rec, tickets, nrows);
  return hipGetLastError();
}

hipError_t launch_sample(const float* x, u64 N, u64 S, u64 seed, u32 attempt, u32 row, u64* table, u64 tmask,
                         u32 gen, u64* keys, RowCtl* ctl, SelState* sel, u64 t, hipStream_t s) {
  const u32 blocks = (u32)((S + 255) / 256);
  sample_draw_kernel<<<blocks, 256, 0, s>>>(x, N, S, seed, attempt, row, table, tmask, gen, keys, ctl);
  sample_topup_kernel<<<1, 64, 0, s>>>(x, N, S, seed, attempt, row, table, tmask, gen, keys, ctl, sel, t);
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
