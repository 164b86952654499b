// Multi-pass radix selection over 64-bit composite keys, and the compaction of
// the selected keys.
//
// Used three times on the hot path of Prof-K ("Prof-K: Probabilistic One-Pass
// Filtering for Efficient Top-k Selection"):
//   * stage 2 (§3): tau = the t-th largest of the S sampled keys;
//   * stage 4 (§3): the k-th largest of the R buffered candidates, after which the
//     compaction keeps exactly the k keys at or above it;
//   * the exact full selection after the last failed attempt (§3 stage 4), over all
//     N entries with keys formed on the fly (select_pass_x_kernel: dwordx4 loads), after
//     which the compaction is the filter itself with tau = the k-th key (k_filter.hip).
// The pages use a library top-k for these steps (App. C); this is a radix select
// written for gfx950.
//
// One pass = one launch over the keys.  While more than kCollectCap keys share
// the fixed prefix, a pass histograms the next 8-bit digit of those keys (LDS
// histogram, one LDS atomic per distinct digit per wavefront, then one global
// atomic per nonzero bin per block) and the last block to finish picks the
// digit bucket holding the target rank.  Once at most kCollectCap keys remain,
// the next pass appends them to a small array and the last block sorts it in LDS
// and reads off the exact key.  Eight launches always suffice (8 digits); the
// launches after completion return at once.
#include "launch.h"

namespace profk {

struct KeyArraySrc {
  const u64* keys;
  const u64* n_ptr;  // device count; the size is min(*n_ptr, n_cap)
  u64 n_cap;
  __device__ __forceinline__ u64 size() const {
    const u64 n = *n_ptr;
    return n < n_cap ? n : n_cap;
  }
  __device__ __forceinline__ u64 key(u64 i) const { return keys[i]; }
};

namespace {

constexpr int kSelThreads = 256;

// Descending bitonic sort of s[0..P) (P a power of two) by the whole block.
__device__ void bitonic_desc(u64* s, u32 P) {
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

}  // namespace

// One digit of one pass: the histogram of the digit of the matching keys (or, in
// collect mode, the matching keys themselves) for a wavefront's keys.  Every lane of
// the wavefront calls it (wave-collective).
__device__ __forceinline__ void select_take(u64 key, bool match, bool collect, u32 shift, u32* s_hist, SelState* st,
                                            u64* col) {
  if (collect) {
    const u32 slot = wave_reserve32(&st->ncol, match);
    if (match && slot < kCollectCap) col[slot] = key;
    return;
  }
  const u32 d = (u32)(key >> shift) & 255u;
  // The lanes on the wavefront's most common digit (one of the first and the last
  // matching lane's digits: inputs whose values share their leading bits put most lanes
  // on one digit) add with one LDS atomic; the others add one each (the LDS serialises
  // lanes on one address, so a shared digit must not be left to per-lane atomics).
  const u64 m = __ballot(match);
  if (!m) return;
  const int la = __ffsll((long long)m) - 1, lb = 63 - __clzll((long long)m);
  const u32 da = (u32)__builtin_amdgcn_readlane((int)d, la);
  u64 g = __ballot(match && d == da);
  u32 dg = da;
  int lg = la;
  if (2 * __popcll(g) < __popcll(m)) {
    const u32 db = (u32)__builtin_amdgcn_readlane((int)d, lb);
    const u64 gb = __ballot(match && d == db);
    if (__popcll(gb) > __popcll(g)) {
      g = gb;
      dg = db;
      lg = lb;
    }
  }
  if ((int)lane_id() == lg) atomicAdd(&s_hist[dg], (u32)__popcll(g));
  if (match && d != dg) atomicAdd(&s_hist[d], 1u);
}

// End of a pass: the block's histogram into the global one, then the last block fixes
// the digit (or, in collect mode, sorts the collected keys and reads off the result).
__device__ void select_finish(SelState* st, u64* col, u64* result, u32* status, bool collect, u64 prefix, u64 mask,
                              u64 count, u32 digit, u32 shift, u32* s_hist, u64* s_col, u32* s_last) {
  if (!collect) {
    __syncthreads();
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x)
      if (s_hist[b]) atomicAdd(&st->hist[b], s_hist[b]);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) *s_last = (atomicAdd(&st->ticket, 1u) == gridDim.x - 1) ? 1u : 0u;
  __syncthreads();
  if (!*s_last) return;
  __threadfence();

  if (!collect) {
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x) {
      s_hist[b] = atomic_load_agent(&st->hist[b]);
      atomic_store_agent(&st->hist[b], 0u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const u64 rank = st->rank;
      u64 cum = 0;
      int b = 255;
      for (; b >= 0; --b) {
        const u64 c = s_hist[b];
        if (cum + c >= rank) break;
        cum += c;
      }
      if (b < 0 || (digit == 7 && s_hist[b] != 1)) {
        st->error = 1;
        st->done = 1;
        *status = 3;
      } else {
        st->rank = rank - cum;
        st->count = s_hist[b];
        st->prefix = prefix | ((u64)b << shift);
        st->mask = mask | (0xFFull << shift);
        st->digit = digit + 1;
        if (digit + 1 == 8) {
          st->done = 1;
          *result = st->prefix;
        }
      }
      st->ticket = 0;
    }
    return;
  }

  // collect mode: the last block finishes in LDS
  const u32 m = atomic_load_agent(&st->ncol);
  const bool ok = (u64)m == count && m <= kCollectCap && st->rank >= 1 && st->rank <= count;
  if (!ok) {
    if (threadIdx.x == 0) {
      st->error = 1;
      st->done = 1;
      st->ncol = 0;
      st->ticket = 0;
      *status = 3;
    }
    return;
  }
  u32 P = 1;
  while (P < m) P <<= 1;
  for (u32 i = threadIdx.x; i < P; i += blockDim.x) s_col[i] = i < m ? atomic_load_agent(&col[i]) : 0ull;
  __syncthreads();
  bitonic_desc(s_col, P);
  if (threadIdx.x == 0) {
    const u64 ans = s_col[st->rank - 1];
    st->prefix = ans;
    st->mask = ~0ull;
    st->count = 1;
    st->rank = 1;
    st->done = 1;
    st->ncol = 0;
    st->ticket = 0;
    *result = ans;
  }
}

template <class Src>
__global__ __launch_bounds__(kSelThreads) void select_pass_kernel(Src src, SelState* st, u64* col, u64* result,
                                                                  u32* status) {
  __shared__ u32 s_hist[256];
  __shared__ u64 s_col[kCollectCap];
  __shared__ u32 s_last;
  if (st->done) return;
  const u64 n = src.size();
  const u64 prefix = st->prefix, mask = st->mask, count = st->count;
  const bool collect = count <= kCollectCap;
  const u32 digit = st->digit;
  const u32 shift = 56u - 8u * digit;
  if (!collect) {
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x) s_hist[b] = 0;
    __syncthreads();
  }
  // kSelILP keys per thread in flight, then taken
  constexpr u32 kSelILP = 8;
  const u64 stride = (u64)gridDim.x * blockDim.x * kSelILP;
  for (u64 base = (u64)blockIdx.x * blockDim.x * kSelILP; base < n; base += stride) {
    u64 kk[kSelILP];
#pragma unroll
    for (u32 q = 0; q < kSelILP; ++q) {
      const u64 i = base + (u64)q * blockDim.x + threadIdx.x;
      kk[q] = i < n ? src.key(i) : 0ull;
    }
#pragma unroll
    for (u32 q = 0; q < kSelILP; ++q) {
      const u64 i = base + (u64)q * blockDim.x + threadIdx.x;
      select_take(kk[q], i < n && ((kk[q] & mask) == prefix), collect, shift, s_hist, st, col);
    }
  }
  select_finish(st, col, result, status, collect, prefix, mask, count, digit, shift, s_hist, s_col, &s_last);
}

// The same pass over the input values themselves (the exact full selection), with the
// keys formed on the fly: dwordx4 loads, wave-tiles of 64 lanes x kSelXU float4 in a
// grid-stride order, the next tile's loads issued before the current tile's keys are
// taken (two register sets); the scalar head (before the first 16-byte boundary) and
// tail by the first wavefront.
constexpr u32 kSelXU = 4;
typedef float f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kSelThreads) void select_pass_x_kernel(const float* x, u64 N, SelState* st, u64* col,
                                                                    u64* result, u32* status) {
  __shared__ u32 s_hist[256];
  __shared__ u64 s_col[kCollectCap];
  __shared__ u32 s_last;
  if (st->done) return;
  const u64 prefix = st->prefix, mask = st->mask, count = st->count;
  const bool collect = count <= kCollectCap;
  const u32 digit = st->digit;
  const u32 shift = 56u - 8u * digit;
  if (!collect) {
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x) s_hist[b] = 0;
    __syncthreads();
  }
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  u64 head = (4ull - (((u64)(uintptr_t)x >> 2) & 3ull)) & 3ull;
  if (head > N) head = N;
  const u64 nvec = (N - head) >> 2, tail = N - head - 4 * nvec;
  const f4* xv = reinterpret_cast<const f4*>(x + head);
  const u64 per_tile = (u64)kSelXU * kWave;
  const u64 ntiles = (nvec + per_tile - 1) / per_tile;
  const u64 nw = (u64)gridDim.x * (kSelThreads / kWave);
  auto load = [&](u64 tl, f4 (&v)[kSelXU]) {
#pragma unroll
    for (u32 u = 0; u < kSelXU; ++u) {
      const u64 vi = tl * per_tile + (u64)u * kWave + lane;
      v[u] = vi < nvec ? __builtin_nontemporal_load(xv + vi) : f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto take = [&](u64 tl, const f4 (&v)[kSelXU]) {
#pragma unroll
    for (u32 u = 0; u < kSelXU; ++u) {
      const u64 vi = tl * per_tile + (u64)u * kWave + lane;
      const u32 i0 = (u32)(head + 4 * vi);
      const float c[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (u32 q = 0; q < 4; ++q) {
        const u64 key = make_key(__float_as_uint(c[q]), i0 + q);
        select_take(key, vi < nvec && ((key & mask) == prefix), collect, shift, s_hist, st, col);
      }
    }
  };
  f4 va[kSelXU], vb[kSelXU];
  u64 tile = (u64)blockIdx.x * (kSelThreads / kWave) + wid;
  if (tile < ntiles) load(tile, va);
  while (tile < ntiles) {
    const u64 t1 = tile + nw;
    if (t1 < ntiles) load(t1, vb);
    take(tile, va);
    if (t1 >= ntiles) break;
    const u64 t2 = t1 + nw;
    if (t2 < ntiles) load(t2, va);
    take(t1, vb);
    tile = t2;
  }
  if (blockIdx.x == 0 && wid == 0 && (head | tail)) {
    u64 i = N;
    if (lane < head) i = lane;
    else if (lane < head + tail) i = head + 4 * nvec + (lane - head);
    const bool in = i < N;
    const u64 key = in ? make_key(__float_as_uint(x[i]), (u32)i) : 0ull;
    select_take(key, in && ((key & mask) == prefix), collect, shift, s_hist, st, col);
  }
  select_finish(st, col, result, status, collect, prefix, mask, count, digit, shift, s_hist, s_col, &s_last);
}

// Writes every key >= *kth_ptr (exactly k of them when the selection is
// consistent) to out[], and folds the OR / AND of the written keys into ctl
// (which digits vary, for the sort).
// Each block owns a contiguous range of the keys: it counts its selected keys,
// reserves them with ONE atomic, then writes them in range order.
template <class Src>
__global__ __launch_bounds__(256) void compact_kernel(Src src, RowCtl* ctl, u64* __restrict__ out, u64 k) {
  __shared__ u32 s_w[256 / kWave];
  __shared__ u64 s_base;
  if (ctl->status != 0) return;
  const u64 kth = ctl->kth;
  const u64 n = src.size();
  const u64 per = (n + gridDim.x - 1) / gridDim.x;
  const u64 lo = (u64)blockIdx.x * per;
  const u64 hi = lo + per < n ? lo + per : n;
  const u32 wid = threadIdx.x / kWave;
  u32 cnt = 0;
  for (u64 i = lo + threadIdx.x; i < hi; i += blockDim.x) cnt += src.key(i) >= kth ? 1u : 0u;
  for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d);
  if (lane_id() == 0) s_w[wid] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32 tot = 0;
    for (u32 w = 0; w < blockDim.x / kWave; ++w) tot += s_w[w];
    s_base = tot ? atomicAdd(&ctl->nsel, (u64)tot) : 0ull;
  }
  __syncthreads();
  u64 run = s_base;
  u64 v_or = 0, v_and = ~0ull;
  bool any = false;
  for (u64 base = lo; base < hi; base += blockDim.x) {
    const u64 i = base + threadIdx.x;
    const bool in = i < hi;
    const u64 key = in ? src.key(i) : 0ull;
    const bool sel = in && key >= kth;
    const u64 m = __ballot(sel);
    __syncthreads();
    if (lane_id() == 0) s_w[wid] = (u32)__popcll(m);
    __syncthreads();
    u64 off = run;
    u32 tot = 0;
    for (u32 w = 0; w < blockDim.x / kWave; ++w) {
      if (w < wid) off += s_w[w];
      tot += s_w[w];
    }
    if (sel) {
      const u64 slot = off + count_below(m);
      if (slot < k) out[slot] = key;
      v_or |= key;
      v_and &= key;
      any = true;
    }
    run += tot;
  }
  // wave reduction of or / and
  for (int d = 32; d >= 1; d >>= 1) {
    v_or |= __shfl_xor(v_or, d);
    v_and &= __shfl_xor(v_and, d);
  }
  const bool wave_any = __ballot(any) != 0;
  if (wave_any && lane_id() == 0) {
    atomicOr(&ctl->key_or, v_or);
    atomicAnd(&ctl->key_and, v_and);
  }
}

// ---------------------------------------------------------------------------
namespace {
// Few blocks per selection pass: every block adds its nonzero bins to the global
// histogram with atomics, and hundreds of blocks contend on the same 256 words.
constexpr u32 kSelMaxBlocks = 128;
constexpr u32 kCompactMaxBlocks = 256;

u32 select_grid(u64 n_max, u32 cap) {
  u64 g = (n_max + 1023) / 1024;  // about four keys per thread
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (u32)g;
}
}  // namespace

hipError_t launch_select_keys(const u64* keys, const u64* n_ptr, u64 n_cap, SelState* st, u64* col, u64* result,
                              u32* status, hipStream_t s) {
  KeyArraySrc src{keys, n_ptr, n_cap};
  const u32 g = select_grid(n_cap, kSelMaxBlocks);
  for (int p = 0; p < 8; ++p) select_pass_kernel<KeyArraySrc><<<g, kSelThreads, 0, s>>>(src, st, col, result, status);
  return hipGetLastError();
}

hipError_t launch_select_x(const float* x, u64 N, SelState* st, u64* col, u64* result, u32* status, hipStream_t s) {
  // a persistent grid of four blocks per CU (fewer for short inputs): each block adds
  // its nonzero bins to the global histogram and takes the ticket once per pass
  u64 g = (N + 4095) / 4096;
  const u64 cap = 4ull * device_cu_count();
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  for (int p = 0; p < 8; ++p) select_pass_x_kernel<<<(u32)g, kSelThreads, 0, s>>>(x, N, st, col, result, status);
  return hipGetLastError();
}

hipError_t launch_compact_keys(const u64* keys, const u64* n_ptr, u64 n_cap, RowCtl* ctl, u64* out, u64 k,
                               hipStream_t s) {
  KeyArraySrc src{keys, n_ptr, n_cap};
  const u32 g = select_grid(n_cap, kCompactMaxBlocks);
  compact_kernel<KeyArraySrc><<<g, 256, 0, s>>>(src, ctl, out, k);
  return hipGetLastError();
}

// The exact full selection's compaction is the filter itself (one streaming pass with
// tau = the k-th key and capacity k, k_filter.hip); these two kernels frame it.
__global__ void arm_compact_kernel(RowCtl* ctl) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    RowCtl* c = ctl;
    c->tau = c->kth;  // keep exactly the keys at or above the k-th
    c->R = 0;
    c->cmax = 0;
    c->nsel = 0;
    c->key_or = 0;
    c->key_and = ~0ull;
  }
}

// After the filter: the count must be exactly k (the keys are distinct); the OR / AND
// of the k keys tells the sort which digits vary.
__global__ __launch_bounds__(256) void finish_compact_kernel(RowCtl* ctl, const u64* __restrict__ keys, u64 k) {
  const RowCtl* c = ctl;
  if (c->status != 0) return;
  if (c->R != k) {
    if (blockIdx.x == 0 && threadIdx.x == 0) ctl->status = 3u;
    return;
  }
  u64 v_or = 0, v_and = ~0ull;
  for (u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x; i < k; i += (u64)gridDim.x * blockDim.x) {
    v_or |= keys[i];
    v_and &= keys[i];
  }
  for (int d = 32; d >= 1; d >>= 1) {
    v_or |= __shfl_xor(v_or, d);
    v_and &= __shfl_xor(v_and, d);
  }
  if (lane_id() == 0) {
    atomicOr(&ctl->key_or, v_or);
    atomicAnd(&ctl->key_and, v_and);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) ctl->nsel = k;
}

hipError_t launch_compact_x(const float* x, u64 N, RowCtl* ctl, u64* out, u64 k, u32* tickets, hipStream_t s) {
  arm_compact_kernel<<<1, 64, 0, s>>>(ctl);
  FilterArgs fa{};
  fa.x = x;
  fa.ld = N;
  fa.N = N;
  fa.rows = nullptr;
  fa.nrows = 1;
  fa.ctls = ctl;
  fa.cand = out;
  fa.M = k;
  fa.k = k;
  fa.ticket = tickets + kTicketFilter;
  fa.groups = tickets + kTickets;
  fa.xtime = nullptr;
  fa.hrec = nullptr;
  fa.rec = nullptr;
  fa.sels = nullptr;
  // launch shape by the density of the k hits, as for a sampled attempt
  fa.sparse = (double)k * 8192.0 <= (double)N ? kShapeSparse
              : (double)k * 256.0 >= (double)N ? kShapeVeryDenseHits
              : (double)k * 2048.0 >= (double)N ? kShapeDenseHits : 0u;
  hipError_t e = launch_filter(fa, 0, s);
  if (e != hipSuccess) return e;
  u64 g = (k + 1023) / 1024;
  if (g > 256) g = 256;
  if (g < 1) g = 1;
  finish_compact_kernel<<<(u32)g, 256, 0, s>>>(ctl, out, k);
  return hipGetLastError();
}

__global__ void arm_select_kernel(SelState* st, u64 rank, u64 count, RowCtl* ctl) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    st->prefix = 0;
    st->mask = 0;
    st->rank = rank;
    st->count = count;
    st->done = 0;
    st->digit = 0;
    st->ticket = 0;
    st->ncol = 0;
    st->error = 0;
    for (int b = 0; b < 256; ++b) st->hist[b] = 0;
    RowCtl c{};
    c.key_and = ~0ull;
    *ctl = c;
  }
}

hipError_t launch_arm_select(SelState* st, u64 rank, u64 count, RowCtl* ctl, hipStream_t s) {
  arm_select_kernel<<<1, 64, 0, s>>>(st, rank, count, ctl);
  return hipGetLastError();
}

}  // namespace profk
