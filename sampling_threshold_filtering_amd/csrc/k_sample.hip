// Stage 1 of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
// Selection", §3, stage 1): S indices drawn uniformly without replacement, and
// stage 2: tau = the t-th largest sampled entry.
//
// The pages leave the procedure open.  The sample here is the set of the first S
// distinct indices of the Philox stream of (seed, attempt, row) in draw order
// (see profk_device.h for the draw).  That rule is symmetric under relabelling of
// [N], so every S-subset is equally likely, and it is deterministic per seed.
//
//   sample_kernel   one thread per draw 0..S-1, in workgroups of 256, 512 or 1024
//                   threads (sample_shape).  Each index goes into a hash set of
//                   32-bit slots in device memory (idx + 1, 0 = empty, one CAS per
//                   probe; the set is zero on entry and cleared again after the
//                   attempt), while the gather of x[idx] is already in flight.  Draw
//                   j keeps its key in keys[j], or 0 when it repeats an earlier draw
//                   (no valid key is 0).  Each block adds itself and its distinct
//                   draws to one 64-bit ticket.  The last block tops up: while fewer
//                   than S distinct indices are held, wavefront 0 takes further draws
//                   S, S+1, ... in order, 64 at a time, keeping those that are new and
//                   not repeated earlier in the same chunk (expected extra draws about
//                   S^2 / (2N)), into keys[S..].
//
// tau (stage 2) is found in one of four ways (sample_shape picks the first that fits):
//   sorted lists    t <= 64: each block sorts its wavefronts' keys in registers and
//                   merges them into its pow2(t) largest, sorted;
//   top-t lists     t <= 1024: each block finds its own t-th largest key by a radix
//                   select on the keys in registers and keeps the t keys at or above
//                   it, in no order.
//                   In both, only a block's t largest draws can be among the t largest
//                   of all: the last block stages the lists in LDS (its other
//                   wavefronts load them while wavefront 0 tops up), appends the top-up
//                   keys, and a radix select in LDS finds the t-th.  The lists are sized
//                   so that they and a bound on the top-up fit in LDS.
//   key slots       every draw slot fits in LDS: the same select over all of them;
//   select passes   (one row) beyond that: the last block arms the multi-block radix
//                   select of k_select.hip over the key slots, whose passes follow this
//                   launch on the stream and leave tau in the row's control block.
// Rows of the batched form whose slots exceed LDS with t > 1024 keep one workgroup per
// row reading the slots from L2 (the rows run side by side); so does a list launch
// whose top-up ever exceeds its bound.

#include <cmath>

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
// included) so that nothing depends on what the workspace held before.  Block b
// takes rows b, b + gridDim.x, ...; block 0 also the tickets and the refinement's
// histogram.
__global__ __launch_bounds__(1024) void attempt_init_kernel(RowCtl* ctl, SelState* sel, AttemptRecord* rec,
                                                          u32* tickets, u32 nrows, u32* refine_hist) {
  if (blockIdx.x == 0) {
    if (tickets)
      for (u32 i = threadIdx.x; i < kTicketWords; i += blockDim.x) tickets[i] = 0;
    if (refine_hist)
      for (u32 b = threadIdx.x; b < kBins; b += blockDim.x) refine_hist[b] = 0;
  }
  if (sel)
    for (u32 r = blockIdx.x; r < nrows; r += gridDim.x)
      for (u32 b = threadIdx.x; b < 256; b += blockDim.x) sel[r].hist[b] = 0;
  for (u32 r = blockIdx.x * blockDim.x + threadIdx.x; r < nrows; r += gridDim.x * blockDim.x) {
    RowCtl c{};
    c.key_and = ~0ull;
    ctl[r] = c;
    if (rec) rec[r] = AttemptRecord{0ull, 0u, 0u, 0u, 0u};
    if (!sel) continue;
    SelState* q = &sel[r];
    q->prefix = 0;
    q->mask = 0;
    q->rank = 1;
    q->count = 0;
    q->done = 1;
    q->digit = 0;
    q->ticket = 0;
    q->ncol = 0;
    q->error = 0;
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
  __shared__ u32 s_wkeep[kSampleWaves];
  __shared__ u32 s_n;
  __shared__ u32 s_last;
  __shared__ u64 s_D, s_E;
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  const bool select = a.t > 0;
  const u32 mode = select ? a.mode : kTauKeys;
  // the top-digit histogram starts the one-workgroup select over L2 (key slots beyond LDS)
  const bool use_hist = mode == kTauKeys && select && a.S > kTauCap;
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
  if (mode == kTauSortedLists) {
    const u64 sk = wave_sort_desc(key);
    if (lane < T) s_buf[wid * T + lane] = sk;  // this wavefront's T largest (0-padded)
  }
  __syncthreads();
  if (use_hist) {
    // histogram of the top 8 bits: the first digit of the radix select
    wave_hist_add(s_sel.hist, (u32)(key >> 56), fresh);
    __syncthreads();
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x)
      if (s_sel.hist[b]) atomicAdd(&a.top_hist[b], s_sel.hist[b]);
  } else if (mode == kTauSortedLists) {
    block_merge_lists(s_buf, kSampleWaves, T);  // the block's T largest keys
    for (u32 i = threadIdx.x; i < T; i += blockDim.x) st_agent(a.tops + (u64)blockIdx.x * T + i, s_buf[i]);
  } else if (mode == kTauTopLists) {
    // the block's t largest keys, in no order: the t-th largest by a radix select on
    // the keys in registers (0 when the block holds fewer than t), then every key at
    // or above it (exactly t of them, the keys being distinct), zero-padded to t
    const u64 v1[1] = {key};
    const u64 kb = reg_select_desc(v1, (u32)a.t, &s_lsel);
    const bool keep = key != 0 && key >= kb;
    const u64 km = __ballot(keep);
    if (lane == 0) s_wkeep[wid] = (u32)__popcll(km);
    __syncthreads();
    u32 off = 0, tot = 0;
    for (u32 w = 0; w < kSampleWaves; ++w) {
      off += w < wid ? s_wkeep[w] : 0u;
      tot += s_wkeep[w];
    }
    u64* dst = a.tops + (u64)blockIdx.x * a.t;
    const u32 slot = off + count_below(km);
    if (keep && slot < a.t) st_agent(dst + slot, key);
    for (u32 i = tot + threadIdx.x; i < a.t; i += blockDim.x) st_agent(dst + i, 0ull);
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
  // What the select reads, known before the top-up: the block lists (only a block's t
  // largest draws can be among the t largest of all: the first t of each sorted list,
  // stride T, or each unordered top-t list, stride t), or every draw slot when they
  // fit.  The other wavefronts stage it in LDS while wavefront 0 tops the sample up
  // and appends the top-up keys behind it.
  const bool lists = mode == kTauSortedLists || mode == kTauTopLists;
  const u32 tt = (u32)a.t;
  const u64 nbase = lists ? (u64)gridDim.x * tt : (mode == kTauKeys && select && a.S <= kTauCap ? a.S : 0ull);
  const bool staged = select && nbase > 0 && nbase <= kTauCap;
  if (wid == 0) {
    const u64 D = s_D;
    u64 E = 0, j0 = a.S;
    u32 guard = 0;
    bool failed = false;
    while (D + E < a.S) {
      const u32 idx2 = (u32)sample_draw(j0 + lane, a.row, a.attempt, a.seed, a.N);
      // every new draw is inserted; one that finds its index inserted by another lane of
      // this chunk repeats within the chunk, and only then (rare: 64^2 / 2N per chunk) do
      // the lanes compare indices to find which of the equal draws came first.  The set
      // then holds the chunk's new indices; those not taken can only be there when the
      // chunk is the last one.
      const bool held = hash_contains(a.table, a.tmask, idx2);
      const bool dup = !held && !hash_insert(a.table, a.tmask, idx2);
      bool repeat = dup;
      if (__ballot(dup)) {
        repeat = false;
        for (int d = 1; d < kWave; ++d) {
          const u32 other = __shfl_up(idx2, d, kWave);
          if ((int)lane >= d && other == idx2) repeat = true;
        }
      }
      const bool ok2 = !held && !repeat;
      const u64 m2 = __ballot(ok2);
      const u64 need = a.S - D - E;
      const u32 r = count_below(m2);
      if (ok2 && r < need) {
        const u64 key2 = make_key(__float_as_uint(a.x[idx2]), idx2);
        a.keys[a.S + E + r] = key2;
        if (staged && nbase + E + r < kTauCap) s_buf[nbase + E + r] = key2;
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
  } else if (staged) {
    const u64 ls = mode == kTauSortedLists ? (u64)T : (u64)tt;
    const u32 nl = (u32)nbase, lt = threadIdx.x - kWave, nt = kSampleThreads - kWave;
    constexpr u32 kILP = 8;
    for (u32 base = 0; base < nl; base += nt * kILP) {
      u64 kk[kILP];
#pragma unroll
      for (u32 q = 0; q < kILP; ++q) {
        const u32 i = base + q * nt + lt;
        u64 src = i;
        if (lists) {
          const u32 b = i / tt;
          src = (u64)b * ls + (i - b * tt);
        }
        kk[q] = i < nl ? (lists ? a.tops[src] : a.keys[src]) : 0ull;
      }
#pragma unroll
      for (u32 q = 0; q < kILP; ++q) {
        const u32 i = base + q * nt + lt;
        if (i < nl) s_buf[i] = kk[q];
      }
    }
  }
  __syncthreads();
  const u64 E = s_E;
  const bool sample_ok = E != ~0ull && s_D + E == a.S;
  const u64 nslots = a.S + (sample_ok ? E : 0ull);
  bool ok = sample_ok;
  u64 tau = 0;
  if (select) {
    if (staged && sample_ok && nbase + E <= kTauCap) {
      tau = lds_select_desc(s_buf, (u32)(nbase + E), tt, &s_lsel);
      ok = tau != 0;
    } else if (mode == kTauPasses) {
      // the select passes that follow this launch find tau over the nslots key slots
      // (zero for the repeated draws: below every key, so the rank t <= S still lands
      // on a drawn key); a failed sample leaves them nothing to do
      if (threadIdx.x == 0) {
        SelState* q = a.sel;
        q->prefix = 0;
        q->mask = 0;
        q->rank = a.t;
        q->count = nslots;
        q->done = sample_ok ? 0u : 1u;
        q->digit = 0;
        q->ticket = 0;
        q->ncol = 0;
        q->error = 0;
      }
    } else {
      // one workgroup over the key slots in L2 (a top-up beyond the room in LDS, or
      // rows of the batched form with t > 1024): starting from the top-digit
      // histogram the sampling blocks built, if they built one
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
  // the rows' histograms (256 words each) over up to 256 blocks; without them one
  // thread per row
  u32 blocks = sel ? (nrows < 256 ? nrows : 256u) : (nrows + 1023) / 1024;
  if (blocks < 1) blocks = 1;
  attempt_init_kernel<<<blocks, 1024, 0, s>>>(ctl, sel, rec, tickets, nrows, refine_hist);
  return hipGetLastError();
}

namespace {
// Blocks of the sorted-list path: 256 threads while at most kTopBlocks of them cover S.
u32 list_threads(u64 S) { return (S + 255) / 256 <= kTopBlocks ? 256u : 1024u; }

// A bound on the top-up draws E (the repeats among the first S draws): their mean is
// at most S^2 / (2N) (the first term of an alternating series), their spread about
// its square root; six of those past it are not reached in practice.  A launch whose
// top-up does exceed the room left in LDS still ends correctly (the select over the
// key slots).
u64 topup_bound(u64 S, u64 N) {
  const double mu = (double)S * (double)S / (2.0 * (double)(N ? N : 1));
  return (u64)(mu + 6.0 * std::sqrt(mu) + 64.0);
}
}  // namespace

SampleShape sample_shape(u64 S, u64 t, u64 N, bool passes) {
  SampleShape sh{kTauKeys, 1024u, 0u, 1ull};
  const u64 E = topup_bound(S, N);
  const u32 tl = list_threads(S);
  const u64 gl = (S + tl - 1) / tl;
  if (t == 0) {
    sh.threads = tl;
  } else if (t <= kTopT && gl <= kTopBlocks && gl * t + E <= kTauCap) {
    u64 T = 1;
    while (T < t) T <<= 1;
    sh.mode = kTauSortedLists;
    sh.threads = tl;
    sh.tops_words = gl * T;
  } else {
    // unordered top-t lists: the smallest workgroups (the most CUs gathering) whose
    // lists still fit in LDS beside the top-up
    for (u32 th = 256; th <= 1024; th <<= 1) {
      const u64 g = (S + th - 1) / th;
      if (t <= 1024 && g * t + E <= kTauCap) {
        sh.mode = kTauTopLists;
        sh.threads = th;
        sh.tops_words = g * t;
        break;
      }
    }
    // else the key slots (S plus the top-up): in LDS when they fit, else several
    // workgroups read them, pass by pass (one row), or one workgroup per row over L2
    if (sh.mode == kTauKeys && S + E > kTauCap && passes) sh.mode = kTauPasses;
  }
  sh.blocks = (u32)((S + sh.threads - 1) / sh.threads);
  return sh;
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
  const u32 th = a.threads;
  const dim3 grid((u32)((a.S + th - 1) / th), a.nrows ? a.nrows : 1u);
  if (a.mode == kTauPasses && (a.nrows || !a.sel || !a.col)) return hipErrorInvalidValue;
  if (th == 256)
    sample_kernel<256><<<grid, 256, 0, s>>>(a);
  else if (th == 512)
    sample_kernel<512><<<grid, 512, 0, s>>>(a);
  else if (th == 1024)
    sample_kernel<1024><<<grid, 1024, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.mode != kTauPasses || a.t == 0) return e;
  // tau into ctl->tau by the multi-block passes (a failed check into ctl->status)
  return launch_select_keys(a.keys, &a.ctl->D, 2 * a.S, a.sel, a.col, &a.ctl->tau, &a.ctl->status, s);
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
