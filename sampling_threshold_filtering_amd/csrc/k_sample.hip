// Stage 1 of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
// Selection", §3, stage 1): S indices drawn uniformly without replacement, and
// stage 2: tau = the t-th largest sampled entry.
//
// The pages leave the procedure open.  The sample here is the set of the first S
// distinct indices of the Philox stream of (seed, attempt, row) in draw order
// (see profk_device.h for the draw).  That rule is symmetric under relabelling of
// [N], so every S-subset is equally likely, and it is deterministic per seed.
//
//   sample_kernel   one thread per draw 0..S-1, in workgroups of 256 threads when
//                   the per-block lists below apply and S <= 32768 (the random
//                   gathers then spread over 4x as many CUs, which halves their
//                   latency on MI355X), else 1024.  Each index goes into a hash set of
//                   32-bit slots in device memory (idx + 1, 0 = empty, one CAS per
//                   probe; the set is zero on entry and cleared again after the
//                   attempt), while the gather of x[idx] is already in flight.  Draw
//                   j keeps its key in keys[j], or 0 when it repeats an earlier draw
//                   (no valid key is 0).  For t <= kTopT each block also sorts its
//                   wavefronts' keys in registers and stores its own t largest keys.
//                   Each block adds itself and its distinct draws to one 64-bit ticket.
//                   The last block (a) tops up: while fewer than S distinct indices
//                   are held, wavefront 0 takes further draws S, S+1, ... in order,
//                   64 at a time, keeping those that are new and not repeated earlier
//                   in the same chunk (expected extra draws about S^2 / (2N)), into
//                   keys[S..]; and (b) selects tau.  With the per-block lists, only
//                   the first t keys of each list (and the top-up keys) can be among
//                   the t largest: those are loaded into LDS and a radix select
//                   there finds the t-th.  Otherwise, while all key slots fit in
//                   LDS, the same select runs over them, and beyond that a
//                   one-workgroup radix select reads them from L2 pass by pass.
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

// Open-addressing set of 32-bit slots holding idx + 1 (0 = empty), linear probing.
// Returns true when idx was not in the set (and is now).
__device__ bool hash_insert(u32* table, u64 tmask, u32 idx) {
  const u32 mine = idx + 1u;
  u64 h = mix32(idx) & tmask;
  for (u64 probe = 0; probe <= tmask; ++probe) {
    const u32 prev = atomicCAS(&table[h], 0u, mine);
    if (prev == 0u || prev == mine) return prev == 0u;
    h = (h + 1) & tmask;
  }
  return false;  // unreachable: the table holds at least 2S slots
}

__device__ bool hash_contains(const u32* table, u64 tmask, u32 idx) {
  const u32 mine = idx + 1u;
  u64 h = mix32(idx) & tmask;
  for (u64 probe = 0; probe <= tmask; ++probe) {
    const u32 cur = atomic_load_agent(&table[h]);
    if (cur == 0u || cur == mine) return cur == mine;
    h = (h + 1) & tmask;
  }
  return false;
}

}  // namespace

// Clears every per-attempt counter, record and selection state (histograms
// included) so that nothing depends on what the workspace held before.
__global__ __launch_bounds__(1024) void attempt_init_kernel(RowCtl* ctl, SelState* sel, AttemptRecord* rec,
                                                          u32* tickets, u32 nrows, u32* refine_hist) {
  if (tickets)
    for (u32 i = threadIdx.x; i < kTicketWords; i += blockDim.x) tickets[i] = 0;
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

constexpr u32 kTauCap = 8192;  // keys the last block sorts or selects from in LDS (64 KB)

template <u32 kSampleThreads>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(SampleArgs a0) {
  constexpr u32 kSampleWaves = kSampleThreads / kWave;
  SampleArgs a = a0;  // this row's view (wave-uniform)
  if (a0.nrows) {
    const u64 li = blockIdx.y;
    const u32 row = a0.rows ? (u32)a0.rows[li] : a0.row0 + (u32)li;
    a.row = row;
    a.x = a0.x + (u64)row * a0.ld;
    a.ctl = a0.ctl + row;
    a.rec = a0.rec ? a0.rec + row : nullptr;
    a.top_hist = a0.top_hist + (u64)row * a0.hist_stride;
    a.table = a0.table + li * a0.table_stride;
    a.keys = a0.keys + li * a0.keys_stride;
    a.tops = a0.tops + li * a0.tops_stride;
    a.ticket = a0.ticket + li * a0.ticket_stride;
  }
  __shared__ u64 s_buf[kTauCap];
  __shared__ BlockSelectLds s_sel;
  __shared__ LdsSelect s_lsel;
  __shared__ u32 s_wcnt[kSampleWaves];
  __shared__ u32 s_n;
  __shared__ u32 s_last;
  __shared__ u64 s_D, s_E;
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  const bool select = a.t > 0;
  const bool use_hist = select && !a.fast;
  for (u32 b = threadIdx.x; b < 256; b += blockDim.x) s_sel.hist[b] = 0;
  if (threadIdx.x == 0) s_n = 0;

  // one draw per thread
  const u64 j = (u64)blockIdx.x * kSampleThreads + threadIdx.x;
  bool fresh = false;
  u64 key = 0;
  if (j < a.S) {
    const u32 idx = (u32)sample_draw(j, a.row, a.attempt, a.seed, a.N);
    const u32 bits = __float_as_uint(a.x[idx]);  // issued before the insert: both in flight
    fresh = hash_insert(a.table, a.tmask, idx);
    if (fresh) key = make_key(bits, idx);
    st_agent(a.keys + j, key);
  }
  const u64 fm = __ballot(fresh);
  if (lane == 0) s_wcnt[wid] = (u32)__popcll(fm);
  // fast path: lists of T = pow2(t) keys, each sorted descending
  u32 T = 1;
  while (T < a.t) T <<= 1;
  if (a.fast) {
    key = wave_sort_desc(key);
    if (lane < T) s_buf[wid * T + lane] = key;  // this wavefront's T largest (0-padded)
  }
  __syncthreads();
  if (use_hist) {
    // histogram of the top 8 bits: the first digit of the radix select
    wave_hist_add(s_sel.hist, (u32)(key >> 56), fresh);
    __syncthreads();
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x)
      if (s_sel.hist[b]) atomicAdd(&a.top_hist[b], s_sel.hist[b]);
  } else if (a.fast) {
    block_merge_lists(s_buf, kSampleWaves, T);  // the block's T largest keys
    for (u32 i = threadIdx.x; i < T; i += blockDim.x) st_agent(a.tops + (u64)blockIdx.x * T + i, s_buf[i]);
  }
  // this block's keys and lists complete (written through at agent scope), then elect
  // the last block: one atomic adds the block to the ticket and its distinct draws to
  // the count, so the last block has the total from the atomic's return value
  drain_memory_ops();
  __syncthreads();
  if (threadIdx.x == 0) {
    u32 tot = 0;
    for (u32 w = 0; w < kSampleWaves; ++w) tot += s_wcnt[w];
    const u64 old = atomicAdd(a.ticket, (1ull << 32) | (u64)tot);
    const bool last = (u32)(old >> 32) == gridDim.x - 1;
    s_last = last ? 1u : 0u;
    s_D = (u64)(u32)old + tot;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // top-up by wavefront 0
  if (wid == 0) {
    const u64 D = s_D;
    u64 E = 0, j0 = a.S;
    u32 guard = 0;
    bool failed = false;
    while (D + E < a.S) {
      const u32 idx2 = (u32)sample_draw(j0 + lane, a.row, a.attempt, a.seed, a.N);
      const bool held = hash_contains(a.table, a.tmask, idx2);
      bool repeat = false;
      for (int d = 1; d < kWave; ++d) {
        const u32 other = __shfl_up(idx2, d, kWave);
        if ((int)lane >= d && other == idx2) repeat = true;
      }
      const bool ok2 = !held && !repeat;
      const u64 m2 = __ballot(ok2);
      const u64 need = a.S - D - E;
      const u32 r = count_below(m2);
      if (ok2 && r < need) {
        hash_insert(a.table, a.tmask, idx2);
        const u64 key2 = make_key(__float_as_uint(a.x[idx2]), idx2);
        a.keys[a.S + E + r] = key2;
        if (use_hist) atomicAdd(&a.top_hist[key2 >> 56], 1u);
      }
      const u64 got = (u64)__popcll(m2);
      E += got < need ? got : need;
      j0 += kWave;
      if (++guard > (1u << 22)) {  // bounded: S <= N/2 makes each draw new with prob >= 1/2
        failed = true;
        break;
      }
    }
    if (lane == 0) s_E = failed ? ~0ull : E;
  }
  __syncthreads();
  const u64 E = s_E;
  const bool sample_ok = E != ~0ull && s_D + E == a.S;
  const u64 nslots = a.S + (sample_ok ? E : 0ull);
  bool ok = sample_ok;
  u64 tau = 0;
  if (select) {
    if (a.fast && sample_ok && (u64)gridDim.x * a.t + E <= kTauCap) {
      // each block's list holds its T largest draws in descending order, so only its
      // first t can be among the t largest; with the top-up keys they go into LDS
      const u32 G = gridDim.x, tt = (u32)a.t, nl = G * tt;
      constexpr u32 kILP = 8;
      for (u32 base = 0; base < nl; base += blockDim.x * kILP) {
        u64 kk[kILP];
#pragma unroll
        for (u32 q = 0; q < kILP; ++q) {
          const u32 i = base + q * blockDim.x + threadIdx.x;
          const u32 b = i / tt;
          kk[q] = i < nl ? a.tops[(u64)b * T + (i - b * tt)] : 0ull;
        }
#pragma unroll
        for (u32 q = 0; q < kILP; ++q) {
          const u32 i = base + q * blockDim.x + threadIdx.x;
          if (i < nl) s_buf[i] = kk[q];
        }
      }
      for (u64 i = threadIdx.x; i < E; i += blockDim.x) s_buf[nl + i] = a.keys[a.S + i];
      __syncthreads();
      tau = lds_select_desc(s_buf, nl + (u32)E, tt, &s_lsel);
      ok = tau != 0;
    } else if (sample_ok && nslots <= kTauCap) {
      // every key slot fits in LDS: select there
      constexpr u32 kILP = 8;
      for (u64 base = 0; base < nslots; base += (u64)blockDim.x * kILP) {
        u64 kk[kILP];
#pragma unroll
        for (u32 q = 0; q < kILP; ++q) {
          const u64 i = base + (u64)q * blockDim.x + threadIdx.x;
          kk[q] = i < nslots ? a.keys[i] : 0ull;
        }
#pragma unroll
        for (u32 q = 0; q < kILP; ++q) {
          const u64 i = base + (u64)q * blockDim.x + threadIdx.x;
          if (i < nslots) s_buf[i] = kk[q];
        }
      }
      if (use_hist)
        for (u32 b = threadIdx.x; b < 256; b += blockDim.x) a.top_hist[b] = 0;  // left zero for the next launch
      __syncthreads();
      tau = lds_select_desc(s_buf, (u32)nslots, (u32)a.t, &s_lsel);
      ok = tau != 0;
    } else {
      if (use_hist) {
        for (u32 b = threadIdx.x; b < 256; b += blockDim.x) {
          s_sel.hist[b] = atomicAdd(&a.top_hist[b], 0u);
          a.top_hist[b] = 0;  // left zero for the next launch
        }
        __syncthreads();
        if (threadIdx.x == 0) block_select_start_from_top_hist(&s_sel, s_sel.hist, sample_ok ? a.S : 0, a.t);
      } else if (threadIdx.x == 0) {
        block_select_start(&s_sel, sample_ok ? a.S : 0, a.t);
      }
      __syncthreads();
      bool ok2 = false;
      tau = block_select_finish(a.keys, nslots, s_buf, kTauCap, &s_sel, &ok2);
      ok = ok && ok2;
    }
  }
  if (threadIdx.x == 0) {
    // per-attempt control state for the filter and the refinement
    RowCtl* c = a.ctl;
    c->D = nslots;
    c->tau = tau;
    c->R = 0;
    c->kth = 0;
    c->nsel = 0;
    c->key_or = 0;
    c->key_and = ~0ull;
    c->cmax = 0;
    c->status = ok ? 0u : 3u;
    c->cur = 0;
    c->ticket = 0;
    c->bin_shift = 0;
    c->bstar = 0;
    c->c_above = 0;
    c->generic = 0;
    if (a.rec) {
      a.rec->R = 0;
      a.rec->status = ok ? 0u : 3u;
      a.rec->error = 0;
      a.rec->generic = 0;
    }
    *a.ticket = 0ull;
  }
}

// Zeroes the hash slots a sampling launch used and the tickets (stage entry points,
// which do not run the refinement that clears them otherwise).
__global__ void clear_sample_kernel(u32* table, u64 slots, u32* tickets) {
  const u64 gs = (u64)gridDim.x * blockDim.x;
  for (u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x; i < slots; i += gs) table[i] = 0;
  if (blockIdx.x == 0)
    for (u32 i = threadIdx.x; i < kTicketWords; i += blockDim.x) tickets[i] = 0;
}

// Indices of the nonzero keys among keys[0 .. min(*n_ptr, n_cap)), appended in any order.
__global__ void keys_to_index_compact_kernel(const u64* __restrict__ keys, const u64* n_ptr, u64 n_cap,
                                             int64_t* __restrict__ out, u32* counter) {
  u64 n = *n_ptr;
  if (n > n_cap) n = n_cap;
  for (u64 i0 = (u64)blockIdx.x * blockDim.x; i0 < n; i0 += (u64)gridDim.x * blockDim.x) {
    const u64 i = i0 + threadIdx.x;
    const u64 key = i < n ? keys[i] : 0ull;
    const u32 slot = wave_reserve32(counter, key != 0);
    if (key != 0) out[slot] = (int64_t)key_index(key);
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
  if (blockIdx.x == 0)
    for (u32 i = threadIdx.x; i < kTicketWords; i += blockDim.x) tickets[i] = 0;
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

u32 sample_threads(u64 S, u64 t) {
  const bool lists = t == 0 || t <= kTopT;
  return lists && (S + 255) / 256 <= kTopBlocks ? 256u : 1024u;
}

u32 sample_blocks(u64 S, u64 t) {
  const u32 th = sample_threads(S, t);
  return (u32)((S + th - 1) / th);
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
  const u32 th = sample_threads(a.S, a.t), blocks = sample_blocks(a.S, a.t);
  const dim3 grid(blocks, a.nrows ? a.nrows : 1u);
  if (th == 256)
    sample_kernel<256><<<grid, 256, 0, s>>>(a);
  else
    sample_kernel<1024><<<grid, 1024, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_clear_sample(u32* table, u64 slots, u32* tickets, hipStream_t s) {
  u64 blocks = (slots + 1023) / 1024;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  clear_sample_kernel<<<(u32)blocks, 1024, 0, s>>>(table, slots, tickets);
  return hipGetLastError();
}

hipError_t launch_keys_to_index_compact(const u64* keys, const u64* n_ptr, u64 n_cap, int64_t* out, u32* counter,
                                        hipStream_t s) {
  u32 blocks = (u32)((n_cap + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  keys_to_index_compact_kernel<<<blocks, 256, 0, s>>>(keys, n_ptr, n_cap, out, counter);
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
