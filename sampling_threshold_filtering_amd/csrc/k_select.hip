// Multi-pass radix selection over 64-bit composite keys, and the compaction of
// the selected keys.
//
// Used three times on the hot path of Prof-K ("Prof-K: Probabilistic One-Pass
// Filtering for Efficient Top-k Selection"):
//   * stage 2 (§3): tau = the t-th largest of the S sampled keys;
//   * stage 4 (§3): the k-th largest of the R buffered candidates, after which the
//     compaction keeps exactly the k keys at or above it;
//   * the exact full selection after the last failed attempt (§3 stage 4), over all
//     N entries with keys formed on the fly.
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

struct FloatSrc {
  const float* x;
  u64 N;
  __device__ __forceinline__ u64 size() const { return N; }
  __device__ __forceinline__ u64 key(u64 i) const { return make_key(__float_as_uint(x[i]), (u32)i); }
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
  const u64 stride = (u64)gridDim.x * blockDim.x;
  for (u64 base = (u64)blockIdx.x * blockDim.x; base < n; base += stride) {
    const u64 i = base + threadIdx.x;
    const bool in = i < n;
    const u64 key = in ? src.key(i) : 0ull;
    const bool match = in && ((key & mask) == prefix);
    if (collect) {
      const u32 slot = wave_reserve32(&st->ncol, match);
      if (match && slot < kCollectCap) col[slot] = key;
    } else {
      wave_hist_add(s_hist, (u32)(key >> shift) & 255u, match);
    }
  }
  if (!collect) {
    __syncthreads();
    for (u32 b = threadIdx.x; b < 256; b += blockDim.x)
      if (s_hist[b]) atomicAdd(&st->hist[b], s_hist[b]);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&st->ticket, 1u) == gridDim.x - 1) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
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
  FloatSrc src{x, N};
  const u32 g = select_grid(N, 4096);
  for (int p = 0; p < 8; ++p) select_pass_kernel<FloatSrc><<<g, kSelThreads, 0, s>>>(src, st, col, result, status);
  return hipGetLastError();
}

hipError_t launch_compact_keys(const u64* keys, const u64* n_ptr, u64 n_cap, RowCtl* ctl, u64* out, u64 k,
                               hipStream_t s) {
  KeyArraySrc src{keys, n_ptr, n_cap};
  const u32 g = select_grid(n_cap, kCompactMaxBlocks);
  compact_kernel<KeyArraySrc><<<g, 256, 0, s>>>(src, ctl, out, k);
  return hipGetLastError();
}

hipError_t launch_compact_x(const float* x, u64 N, RowCtl* ctl, u64* out, u64 k, hipStream_t s) {
  FloatSrc src{x, N};
  const u32 g = select_grid(N, 4 * kCompactMaxBlocks);
  compact_kernel<FloatSrc><<<g, 256, 0, s>>>(src, ctl, out, k);
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
