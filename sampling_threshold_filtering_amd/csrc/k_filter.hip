// Stage 3 of Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
// Selection", §3 stage 3 and App. C "The Filter Kernel"): one streaming pass over
// every row keeps each entry at or above the row's threshold tau in a candidate
// buffer of capacity M and counts them exactly.  The counter R is incremented by
// the full number of kept entries while stores stop at M, so R is the exact rank
// of tau even when the buffer overflows, and the run-time check k <= R <= M needs
// no second pass (App. C).
//
// gfx950 design (the page's Triton kernel is prior art for another GPU):
//   * Work unit: a wave-tile of 64 lanes x U float4 (U = 4: 1024 values, 4 KB)
//     read with dwordx4 loads; wavefronts stride over the wave-tiles of all rows.
//   * Fast pre-test per value: !(x < tau_value), one float compare.  Only a
//     wavefront whose tile has a hit evaluates the exact key test
//     key(x_i, i) >= tau (value, then lower index first: the total order that makes
//     every key distinct).
//   * Compaction: ballot + mbcnt give each hit its slot; hits are staged in a
//     per-wavefront LDS ring (512 keys) and flushed with ONE global atomic on the
//     row counter per flush, so dense tiles cost one atomic per ~512 hits.
//   * Several rows (the batched form): up to 1024 rows whose list positions fit in the
//     index word above the index are read in the flat order too (FO), their thresholds
//     from an LDS copy of the row list; staged keys carry their row's position, and the
//     block places them at the end of the stream with one atomic per row it holds.
//     Other row sets are read in chunks of up to 64 tiles, flushing at row changes.
//   * The last block to finish (ticket) evaluates k <= R <= M per row, writes the
//     host-visible record, and arms the refinement selection of each row.
#include "launch.h"

namespace profk {

namespace {

constexpr int kFilterThreads = 256;
constexpr int kWavesPerBlock = kFilterThreads / kWave;
constexpr u32 kStageCap = 512;

typedef float f4 __attribute__((ext_vector_type(4)));

struct RowGeom {
  const float* row;  // row base
  u64 head;          // scalar values before the first 16-byte boundary
  u64 nvec;          // float4 vectors after it
  u64 tail;          // scalar values after the vectors
};

__device__ __forceinline__ RowGeom row_geom(const float* x, u64 ld, u64 N, u64 r) {
  RowGeom g;
  g.row = x + r * ld;
  const u64 mis = ((u64)(uintptr_t)g.row >> 2) & 3ull;
  u64 head = (4ull - mis) & 3ull;
  if (head > N) head = N;
  g.head = head;
  g.nvec = (N - head) >> 2;
  g.tail = N - head - 4 * g.nvec;
  return g;
}

struct Stage {
  u64* buf;  // this wavefront's LDS ring
  u32 n;     // staged keys
  u32 row;   // row the staged keys belong to
  u64 kmax;  // per lane: largest key staged by this lane (0 when the stage is empty)
};

__device__ __forceinline__ u64 wave_max_u64(u64 v) {
  for (int d = 32; d >= 1; d >>= 1) {
    const u64 o = __shfl_xor(v, d);
    v = o > v ? o : v;
  }
  return v;
}

// The largest candidate key of this block's ticket group (one row): a u64 on the group
// counter's 128-byte line; zero, left zero.
__device__ __forceinline__ u64* group_max(const FilterArgs& a) {
  const u32 ng = gridDim.x < kFilterGroups ? gridDim.x : kFilterGroups;
  return reinterpret_cast<u64*>(a.groups + (u64)(blockIdx.x % ng) * kFilterGroupStride + 2);
}

__device__ __forceinline__ void stage_flush(Stage& st, RowCtl* ctls, u64* cand, u64 M) {
  if (st.n == 0) return;
  wave_lds_sync();
  const u64 mx = wave_max_u64(st.kmax);
  u64 base = 0;
  if (lane_id() == 0) {
    base = atomicAdd(&ctls[st.row].R, (u64)st.n);
    atomicMax(&ctls[st.row].cmax, mx);
  }
  base = __shfl(base, 0);
  st.kmax = 0;
  u64* dst = cand + (u64)st.row * M;
  for (u32 j = lane_id(); j < st.n; j += kWave)
    if (base + j < M) dst[base + j] = st.buf[j];
  wave_lds_sync();
  st.n = 0;
}

// Route the hits of one batch (nmask ballots, hits[] per lane) into the stage.
template <int NB>
__device__ __forceinline__ void stage_hits(Stage& st, u32 row, const u64 (&masks)[NB], const bool (&hit)[NB],
                                           const u64 (&key)[NB], RowCtl* ctls, u64* cand, u64 M) {
  u32 total = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) total += (u32)__popcll(masks[b]);
  if (total == 0) return;
  if (st.n != 0 && (st.row != row || st.n + total > kStageCap)) stage_flush(st, ctls, cand, M);
  if (total > kStageCap) {
    // dense batch: straight to the row's buffer with one atomic
    u64 lmax = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (hit[b] && key[b] > lmax) lmax = key[b];
    const u64 mx = wave_max_u64(lmax);
    u64 base = 0;
    if (lane_id() == 0) {
      base = atomicAdd(&ctls[row].R, (u64)total);
      atomicMax(&ctls[row].cmax, mx);
    }
    base = __shfl(base, 0);
    u64* dst = cand + (u64)row * M;
    u32 run = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (hit[b]) {
        const u64 pos = base + run + count_below(masks[b]);
        if (pos < M) dst[pos] = key[b];
      }
      run += (u32)__popcll(masks[b]);
    }
    return;
  }
  st.row = row;
  u32 run = st.n;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (hit[b]) {
      st.buf[run + count_below(masks[b])] = key[b];
      if (key[b] > st.kmax) st.kmax = key[b];
    }
    run += (u32)__popcll(masks[b]);
  }
  st.n = run;
}

// Several rows, read in the flat pass's order (FO): a wavefront's tiles change rows every
// few tiles, so its stage holds the keys of many rows.  Each staged key carries its row's
// list position l in the index word's bits above the index (all set in ~i, i < N: the
// launch takes this order only where the positions fit there); the block places its
// wavefronts' keys at the end of the stream.
constexpr u32 kFoRows = 1024;  // listed rows whose positions and thresholds a block holds in LDS

// The index word's bits at and above `shift` (= the bits of N - 1) hold the position.
__device__ __forceinline__ u64 fo_high(u32 shift) { return (u64)(0xFFFFFFFFu << shift); }
__device__ __forceinline__ u64 fo_pack(u64 key, u32 l, u32 shift) { return (key & ~fo_high(shift)) | ((u64)l << shift); }
__device__ __forceinline__ u32 fo_list(u64 p, u32 shift) { return (u32)p >> shift; }
__device__ __forceinline__ u64 fo_unpack(u64 p, u32 shift) { return p | fo_high(shift); }

template <int NB>
__device__ __forceinline__ void stage_hits_fo(Stage& st, u32 l, const u64 (&masks)[NB], const bool (&hit)[NB],
                                              const u64 (&key)[NB], const u32* lrow, u32 shift, RowCtl* ctls, u64* cand,
                                              u64 M) {
  u32 total = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) total += (u32)__popcll(masks[b]);
  if (total == 0) return;
  if (st.n + total > kStageCap) {
    // stage full (the launch takes this order only while a wavefront's expected hits
    // fill at most 80% of it): this batch straight to its row's buffer with one atomic; the
    // stage itself is flushed at the end of the stream, where few registers are live
    const u32 row = lrow[l];
    u64 base = 0;
    if (lane_id() == 0) base = atomicAdd(&ctls[row].R, (u64)total);
    base = __shfl(base, 0);
    u64* dst = cand + (u64)row * M;
    u32 run = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (hit[b]) {
        const u64 pos = base + run + count_below(masks[b]);
        if (pos < M) dst[pos] = key[b];
      }
      run += (u32)__popcll(masks[b]);
    }
    return;
  }
  u32 run = st.n;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (hit[b]) st.buf[run + count_below(masks[b])] = fo_pack(key[b], l, shift);
    run += (u32)__popcll(masks[b]);
  }
  st.n = run;
}

}  // namespace

// One wave-tile's place: its row, the row's threshold and the tile's first float4.
struct TileAt {
  u32 row;
  RowGeom geo;
  u64 tau;
  u64 v0;
  u64 tile;
  u32 lr;  // the row's list position
};

// The current row of a wavefront, reloaded only when the row changes: the row list
// and the threshold are read with vector loads (the kernel's atomics on the same
// control blocks rule out scalar ones), and waiting for them would also wait for the
// tile loads in flight.  In the flat order (FO) rows change every few tiles, and the
// block holds every listed row's index and threshold in LDS instead (lrow, ltau).
template <bool FO>
struct RowLds {};
template <>
struct RowLds<true> {
  const u32* lrow = nullptr;
  const u64* ltau = nullptr;
};
template <bool FO>
struct RowCache : RowLds<FO> {
  u64 lr = ~0ull;
  u32 row = 0;
  RowGeom geo{};
  u64 tau = 0;
  __device__ __forceinline__ TileAt at(const FilterArgs& a, u64 l, u64 tile, u32 U) {
    if (l != lr) {
      lr = l;
      if constexpr (FO) {
        row = this->lrow[l];
        geo = row_geom(a.x, a.ld, a.N, row);
        tau = this->ltau[l];
      } else {
        row = a.rows ? (u32)a.rows[l] : (u32)l;
        geo = row_geom(a.x, a.ld, a.N, row);
        tau = a.ctls[row].tau;
      }
    }
    TileAt t;
    t.row = row;
    t.geo = geo;
    t.tau = tau;
    t.v0 = tile * (u64)(U * kWave);
    t.tile = tile;
    t.lr = (u32)l;
    return t;
  }
};

// Issues exactly U dwordx4 loads per lane whatever the tile (a lane past the row's
// vectors reads an in-bounds address and is masked), so the compiler can wait for an
// older tile with a partial count while this one is in flight.  `safe` is any
// readable 16 bytes, for rows too short to hold a float4.
template <int U, bool NT>
__device__ __forceinline__ void load_tile(const TileAt& t, f4 (&v)[U], bool (&valid)[U], const f4* safe) {
  const f4* pv = reinterpret_cast<const f4*>(t.geo.row + t.geo.head);
  const f4* p0 = t.geo.nvec ? pv : safe;
  const u32 lane = lane_id();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const u64 vi = t.v0 + (u64)u * kWave + lane;
    valid[u] = vi < t.geo.nvec;
    const f4* p = valid[u] ? pv + vi : p0;
    v[u] = NT ? __builtin_nontemporal_load(p) : *p;
  }
}

// FO: the block's row list and its per-position counters for the end of the stream.
struct FoCtx {
  u32* cnt;
  const u32* lrow;
  u32 shift;  // bits of N - 1: the position's place in the index word
};

// Stage one batch of hits of tile t (FO: with the tile's list position).
template <bool FO, int NB>
__device__ __forceinline__ void stage_tile_hits(const FilterArgs& a, Stage& st, const FoCtx& fo, const TileAt& t,
                                                const u64 (&masks)[NB], const bool (&hit)[NB], const u64 (&key)[NB]) {
  if constexpr (FO)
    stage_hits_fo<NB>(st, t.lr, masks, hit, key, fo.lrow, fo.shift, a.ctls, a.cand, a.M);
  else
    stage_hits<NB>(st, t.row, masks, hit, key, a.ctls, a.cand, a.M);
}

// Tests one loaded wave-tile (and, on a row's first tile, the row's scalar edges).
template <int U, bool FO>
__device__ __forceinline__ void test_tile(const FilterArgs& a, Stage& st, const FoCtx& fo, const TileAt& t,
                                          const f4 (&v)[U], const bool (&valid)[U]) {
  const u32 lane = lane_id();
  const u32 tk = (u32)(t.tau >> 32);
  const u32 ti = key_index(t.tau);
  const float tv = __uint_as_float(bits_of_ord32(tk));
  bool maybe = false;
  bool mu[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool m = !(v[u].x < tv) | !(v[u].y < tv) | !(v[u].z < tv) | !(v[u].w < tv);
    mu[u] = valid[u] & m;
    maybe |= mu[u];
  }
  if (__ballot(maybe)) {
    // candidate components of this lane (passing the pre-test), bit 4u + q
    u32 cm = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cm |= (u32)(valid[u] && !(v[u].x < tv)) << (4 * u);
      cm |= (u32)(valid[u] && !(v[u].y < tv)) << (4 * u + 1);
      cm |= (u32)(valid[u] && !(v[u].z < tv)) << (4 * u + 2);
      cm |= (u32)(valid[u] && !(v[u].w < tv)) << (4 * u + 3);
    }
    if (!__ballot((cm & (cm - 1u)) != 0u)) {
      // no lane holds two candidates (all but about 1% of the tiles with any at 1.25 hits
      // per tile): each lane picks its candidate with selects, and one batch stages them
      const bool has = cm != 0u;
      const u32 e = has ? (u32)__builtin_ctz(cm) : 0u;
      const u32 eu = e >> 2, eq = e & 3u;
      f4 vs = v[0];
#pragma unroll
      for (int u = 1; u < U; ++u) vs = eu == (u32)u ? v[u] : vs;
      const float c = eq == 0u ? vs.x : eq == 1u ? vs.y : eq == 2u ? vs.z : vs.w;
      const u32 o = ord32(__float_as_uint(c));
      const u32 i = (u32)(t.geo.head + 4 * (t.v0 + (u64)eu * kWave + lane)) + eq;
      u64 masks[1];
      bool hit[1];
      u64 key[1];
      hit[0] = has && (o > tk || (o == tk && i <= ti));
      key[0] = ((u64)o << 32) | (u64)(~i);
      masks[0] = __ballot(hit[0]);
      stage_tile_hits<FO, 1>(a, st, fo, t, masks, hit, key);
    } else {
    // exact test only for the float4 slots, and within them the components, where some
    // lane may hold a hit: when hits are dense (one in a few hundred values) a slot
    // usually has one such component, and the exact keys of the other three would
    // cost three times the instructions
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!__ballot(mu[u])) continue;
      const u64 vi = t.v0 + (u64)u * kWave + lane;
      const u32 i0 = (u32)(t.geo.head + 4 * vi);
      const float c[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!__ballot(valid[u] && !(c[q] < tv))) continue;
        const u32 o = ord32(__float_as_uint(c[q]));
        const u32 i = i0 + q;
        u64 masks[1];
        bool hit[1];
        u64 key[1];
        hit[0] = valid[u] && (o > tk || (o == tk && i <= ti));
        key[0] = ((u64)o << 32) | (u64)(~i);
        masks[0] = __ballot(hit[0]);
        stage_tile_hits<FO, 1>(a, st, fo, t, masks, hit, key);
      }
    }
    }
  }
  if (t.tile == 0 && (t.geo.head | t.geo.tail)) {
    // scalar edge values of this row: lanes [0, head) take the head, then the tail
    const u64 e = lane;
    bool in = false;
    u32 i = 0;
    if (e < t.geo.head) {
      in = true;
      i = (u32)e;
    } else if (e < t.geo.head + t.geo.tail) {
      in = true;
      i = (u32)(t.geo.head + 4 * t.geo.nvec + (e - t.geo.head));
    }
    u64 masks[1];
    bool hit[1];
    u64 key[1];
    const u32 o = in ? ord32(__float_as_uint(t.geo.row[i])) : 0u;
    hit[0] = in && (o > tk || (o == tk && i <= ti));
    key[0] = ((u64)o << 32) | (u64)(~i);
    masks[0] = __ballot(hit[0]);
    stage_tile_hits<FO, 1>(a, st, fo, t, masks, hit, key);
  }
}

template <int U, bool NT, bool FO>
__global__ __launch_bounds__(kFilterThreads) void filter_kernel(FilterArgs a) {
  __shared__ u64 s_stage[kWavesPerBlock][kStageCap];
  __shared__ u32 s_last, s_fwd;
  __shared__ u32 s_nfail;  // last block: listed rows whose check failed
  // wave-uniform: tile coordinates, row, threshold live in scalar registers, and their
  // loads wait on the scalar counter, not behind the tile's vector loads
  const u32 wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const u32 lane = lane_id();
  Stage st{s_stage[wid], 0u, 0u, 0ull};

  // Tile order: chunks of `run` consecutive tiles (run = 1 for one row).  Die x (the
  // blocks b with b mod kXcds = x, which the dispatcher places round-robin on the dies)
  // owns the contiguous chunk range [split[x], split[x+1]) and deals it block-cyclically
  // over its wavefronts, which sweep it together.  The dies stream at different rates
  // on MI355X (up to 15% apart, the same dies every call), so equal shares leave the
  // slowest die to set the end; the host sizes the ranges from the per-die stream times
  // this kernel reports.  Several rows: short runs keep a wavefront's reads together
  // while it changes rows (and flushes its stage) only between chunks.
  const u32 xcd = blockIdx.x % kXcds;
  const u64 nbx = (gridDim.x - xcd + kXcds - 1) / kXcds;      // blocks on this die
  const u64 nwx = nbx * kWavesPerBlock;                        // their wavefronts
  const u64 wx = (u64)(blockIdx.x / kXcds) * kWavesPerBlock + wid;
  const u64 cend = a.split[xcd + 1];
  const u64 run = a.run, gend = a.total_tiles, tpr = a.tiles_per_row;
  // earliest start kept as the largest complement, so that the resting value is zero;
  // taken from the first block of each die only (one address takes an atomic every
  // ~12 ns, and every block's would queue for ~9 us, which short passes wait out)
  if (a.xtime && threadIdx.x == 0 && blockIdx.x < kXcds) atomicMax(&a.xtime[0], ~wall_clock64());
  struct Cursor {
    u64 g, lr, tile, in, chunk;
  };
  auto place = [&](Cursor& c) {
    if (c.chunk >= cend) {
      c.g = gend;
      return;
    }
    c.g = c.chunk * run;
    if (a.nrows == 1) {
      c.lr = 0;
      c.tile = c.g;
    } else {
      c.lr = c.g / tpr;
      c.tile = c.g - c.lr * tpr;
    }
  };
  auto advance = [&](Cursor& c) {
    if constexpr (FO) {
      // one tile per chunk: the next is nwx tiles on, the row kept by subtraction
      c.chunk += nwx;
      if (c.chunk >= cend) {
        c.g = gend;
        return;
      }
      c.g = c.chunk;
      c.tile += nwx;
      while (c.tile >= tpr) {
        c.tile -= tpr;
        ++c.lr;
      }
      return;
    }
    if (c.in + 1 < run && c.g + 1 < gend) {
      ++c.in;
      ++c.g;
      if (++c.tile == tpr) {
        c.tile = 0;
        ++c.lr;
      }
    } else {
      c.in = 0;
      c.chunk += nwx;
      place(c);
    }
  };
  Cursor cur{0, 0, 0, 0, a.split[xcd] + wx};
  place(cur);
  // Software pipeline over two register sets (A, B) used in turn, so that no loaded
  // register is copied: the next tile's loads are issued before the current tile is
  // tested, and the wavefront keeps U dwordx4 loads in flight while it stages hits.
  TileAt ta{}, tb{};
  f4 va[U], vb[U];
  bool oka[U], okb[U];
  RowCache<FO> rc;
  FoCtx fo{nullptr, nullptr, 0u};
  if constexpr (FO) {
    // every listed row's index and threshold, and a counter per list position
    __shared__ u64 s_ltau[kFoRows];
    __shared__ u32 s_lrow[kFoRows];
    __shared__ u32 s_cnt[kFoRows];
    for (u32 l = threadIdx.x; l < (u32)a.nrows; l += kFilterThreads) {
      const u32 row = a.rows ? (u32)a.rows[l] : l;
      s_lrow[l] = row;
      s_ltau[l] = a.ctls[row].tau;
    }
    __syncthreads();
    rc.lrow = s_lrow;
    rc.ltau = s_ltau;
    fo.cnt = s_cnt;
    fo.lrow = s_lrow;
    fo.shift = 32u - (u32)__clz((u32)(a.N - 1));  // N >= 2
  }
  const f4* safe = reinterpret_cast<const f4*>(a.ctls);
  if (cur.g < gend) {
    ta = rc.at(a, cur.lr, cur.tile, U);
    load_tile<U, NT>(ta, va, oka, safe);
  }
  while (cur.g < gend) {
    Cursor nx = cur;
    advance(nx);
    // past the end: reload the current tile (the loads stay unconditional)
    tb = nx.g < gend ? rc.at(a, nx.lr, nx.tile, U) : ta;
    load_tile<U, NT>(tb, vb, okb, safe);
    test_tile<U, FO>(a, st, fo, ta, va, oka);
    cur = nx;
    if (cur.g >= gend) break;
    advance(nx);
    ta = nx.g < gend ? rc.at(a, nx.lr, nx.tile, U) : tb;
    load_tile<U, NT>(ta, va, oka, safe);
    test_tile<U, FO>(a, st, fo, tb, vb, okb);
    cur = nx;
  }
  if (a.xtime) {
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(&a.xtime[1 + xcd], wall_clock64());
  }
  if constexpr (FO) {
    // End of the stream: the block's keys per list position counted in LDS, one atomic
    // on R per position the block holds, then every key placed from its position's run
    // (the block's four wavefronts sweep the same rows side by side)
    u32* cnt = fo.cnt;
    __syncthreads();
    for (u32 l = threadIdx.x; l < (u32)a.nrows; l += kFilterThreads) cnt[l] = 0;
    __syncthreads();
    for (u32 j = lane; j < st.n; j += kWave) atomicAdd(&cnt[fo_list(st.buf[j], fo.shift)], 1u);
    __syncthreads();
    for (u32 l = threadIdx.x; l < (u32)a.nrows; l += kFilterThreads)
      if (cnt[l]) cnt[l] = (u32)atomicAdd(&a.ctls[fo.lrow[l]].R, (u64)cnt[l]);  // R < 2^32: rows of <= 2^20
    __syncthreads();
    for (u32 j = lane; j < st.n; j += kWave) {
      const u64 p = st.buf[j];
      const u32 l = fo_list(p, fo.shift);
      const u64 pos = atomicAdd(&cnt[l], 1u);
      if (pos < a.M) a.cand[(u64)fo.lrow[l] * a.M + pos] = fo_unpack(p, fo.shift);
    }
  } else {
  // End of the stream: the block's waves reserve their staged keys with one
  // atomic per row they hold (one in the flat case) instead of one per wave.
  __shared__ u32 s_n[kWavesPerBlock], s_row[kWavesPerBlock];
  __shared__ u64 s_base[kWavesPerBlock], s_max[kWavesPerBlock];
  const u64 wmax = wave_max_u64(st.kmax);
  if (lane == 0) {
    s_n[wid] = st.n;
    s_row[wid] = st.row;
    s_max[wid] = wmax;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 0; w < kWavesPerBlock; ++w) {
      if (s_n[w] == 0) continue;
      bool first = true;
      for (int v = 0; v < w; ++v)
        if (s_n[v] && s_row[v] == s_row[w]) first = false;
      if (!first) continue;
      u64 tot = 0, mx = 0;
      for (int v = w; v < kWavesPerBlock; ++v)
        if (s_n[v] && s_row[v] == s_row[w]) {
          s_base[v] = tot;
          tot += s_n[v];
          mx = s_max[v] > mx ? s_max[v] : mx;
        }
      // R's atomic returns, so it is performed before this block's ticket; cmax is
      // only read by the next kernel.  One row: the block raises its ticket group's
      // maximum, and the group's last block raises the row's once (where all blocks end
      // together, on short inputs, one atomic per block on the line of R and cmax
      // queues them all)
      // (the group maximum's atomic goes first: the wait for R's result, in issue
      // order, also covers it, so it is in place before this block's ticket)
      if (a.nrows == 1) atomicMax(group_max(a), mx);
      const u64 b = atomicAdd(&a.ctls[s_row[w]].R, tot);
      if (a.nrows != 1) atomicMax(&a.ctls[s_row[w]].cmax, mx);
      for (int v = w; v < kWavesPerBlock; ++v)
        if (s_n[v] && s_row[v] == s_row[w]) s_base[v] += b;
    }
  }
  __syncthreads();
  if (st.n) {
    const u64 base = s_base[wid];
    u64* dst = a.cand + (u64)st.row * a.M;
    for (u32 j = lane; j < st.n; j += kWave)
      if (base + j < a.M) dst[base + j] = st.buf[j];
  }
  }

  // Last block: run-time check per row, host record, arm the refinement selection.
  // Every R update above and in stage_flush is an atomic whose result was consumed
  // before this block's ticket, so the counts are complete when the last ticket is
  // drawn; no release fence (an L2 write-back on this part) is needed per block.
  // The ticket has two levels: block b counts into group b mod G, and the block that
  // completes its group counts into the single ticket, so that no one counter takes
  // an atomic from every block when all blocks end at once (short inputs).
  __syncthreads();
  if (threadIdx.x == 0) {
    const u32 ng = gridDim.x < kFilterGroups ? gridDim.x : kFilterGroups;
    const u32 g = blockIdx.x % ng;
    const u32 gsize = (gridDim.x - g + ng - 1) / ng;  // blocks b with b mod ng = g
    u32 last = 0;
    u32* gc = a.groups + (u64)g * kFilterGroupStride;
    u32 fwd = 0;
    if (atomicAdd(gc, 1u) == gsize - 1) {
      atomic_store_agent(gc, 0u);  // every block of the group has counted: left zero
      last = atomicAdd(a.ticket, 1u) == ng - 1 ? 1u : 0u;
      fwd = 1;
    }
    s_last = last;
    s_fwd = fwd;
  }
  __syncthreads();
  // One row: the group's last block raises the row's maximum by the group's, off the
  // last block's path to the check (the next kernel reads cmax)
  auto forward_group_max = [&]() {
    if constexpr (!FO) {
      if (threadIdx.x == 0 && s_fwd && a.nrows == 1) {
        const u64 gm = atomicExch(group_max(a), 0ull);  // the word left zero
        if (gm) atomicMax(&a.ctls[a.rows ? (u32)a.rows[0] : 0u].cmax, gm);
      }
    }
  };
  if (!s_last) {
    forward_group_max();
    return;
  }
  // No fence: what the last block reads from other blocks (R, the die times) it reads
  // with atomics at the coherence point, and each row's status (written by an earlier
  // launch) with agent-scope loads; its own writes are read by later launches only.
  if (threadIdx.x == 0 && a.xtime) {
    // hand the timing to the host with the attempt record, and leave the words zero
    for (u32 i = 0; i <= kXcds; ++i) {
      const u64 t = atomicExch(&a.xtime[i], 0ull);
      if (a.hrec) a.hrec->xt[i] = i == 0 ? (t ? ~t : 0ull) : t;
    }
  }
  if (threadIdx.x == 0) s_nfail = 0;
  __syncthreads();
  if constexpr (FO) {
    // up to kFoRows rows: each thread reads its rows' counts and statuses together (one
    // round trip to L2, not one per row), then checks them
    constexpr u32 kTail = kFoRows / kFilterThreads;
    u32 rowv[kTail];
    u64 Rv[kTail];
    u32 sv[kTail];
#pragma unroll
    for (u32 q = 0; q < kTail; ++q) {
      const u32 lr = q * kFilterThreads + threadIdx.x;
      rowv[q] = 0;
      Rv[q] = 0;
      sv[q] = 0;
      if (lr < a.nrows) {
        rowv[q] = rc.lrow[lr];
        Rv[q] = atomicAdd(&a.ctls[rowv[q]].R, 0ull);  // read at the coherence point
        sv[q] = atomic_load_agent(&a.ctls[rowv[q]].status);
      }
    }
#pragma unroll
    for (u32 q = 0; q < kTail; ++q) {
      const u32 lr = q * kFilterThreads + threadIdx.x;
      if (lr >= a.nrows) continue;
      const u32 row = rowv[q];
      const u64 R = Rv[q];
      u32 status = sv[q];
      if (status == 0) status = R < a.k ? 1u : (R > a.M ? 2u : 0u);
      a.ctls[row].status = status;
      if (status) atomicAdd(&s_nfail, 1u);
      if (a.rec) {
        a.rec[row].R = R;
        a.rec[row].status = status;
      }
      if (lr == 0 && a.hrec && a.seq && !a.summary) {
        const u64 word = ((u64)(a.seq & 0x3FFFFFu) << 42) | ((u64)(status & 3u) << 40) | (R & ((1ull << 40) - 1));
        __hip_atomic_store(&a.hrec->early, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      if (a.sels) {
        SelState* s = &a.sels[row];
        s->prefix = 0;
        s->mask = 0;
        s->rank = a.k;
        s->count = R < a.M ? R : a.M;
        s->done = status ? 1u : 0u;
        s->digit = 0;
        s->ticket = 0;
        s->ncol = 0;
      }
    }
  } else
  for (u64 lr = threadIdx.x; lr < a.nrows; lr += blockDim.x) {
    const u32 row = a.rows ? (u32)a.rows[lr] : (u32)lr;
    RowCtl* c = &a.ctls[row];
    const u64 R = atomicAdd(&c->R, 0ull);  // read at the coherence point
    u32 status = atomic_load_agent(&c->status);
    if (status == 0) status = R < a.k ? 1u : (R > a.M ? 2u : 0u);
    c->status = status;
    if (status) atomicAdd(&s_nfail, 1u);
    if (a.rec) {
      a.rec[row].R = R;
      a.rec[row].status = status;
    }
    if (lr == 0 && a.hrec && a.seq && !a.summary) {
      // the host learns the check here, before the refinement runs
      const u64 word = ((u64)(a.seq & 0x3FFFFFu) << 42) | ((u64)(status & 3u) << 40) | (R & ((1ull << 40) - 1));
      __hip_atomic_store(&a.hrec->early, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    if (a.sels) {
      SelState* s = &a.sels[row];
      s->prefix = 0;
      s->mask = 0;
      s->rank = a.k;
      s->count = R < a.M ? R : a.M;
      s->done = status ? 1u : 0u;
      s->digit = 0;
      s->ticket = 0;
      s->ncol = 0;
    }
  }
  if (a.summary && a.hrec && a.seq) {
    // several rows: the host learns here whether every row passed (status 0, and the
    // number of rows listed), else the number that failed (status 1)
    __syncthreads();
    if (threadIdx.x == 0) {
      const u32 nf = s_nfail;
      const u64 cnt = nf ? (u64)nf : a.nrows;
      const u64 word = ((u64)(a.seq & 0x3FFFFFu) << 42) | ((u64)(nf ? 1u : 0u) << 40) | (cnt & ((1ull << 40) - 1));
      __hip_atomic_store(&a.hrec->early, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
  if (threadIdx.x == 0) atomic_store_agent(a.ticket, 0u);
  forward_group_max();
}

namespace {
template <int U>
hipError_t launch_filter_shape(const FilterArgs& a0, u32 grid, u32 blocks_per_cu, hipStream_t s, u64* split_out) {
  FilterArgs a = a0;
  const u64 vec_per_tile = (u64)U * kWave;
  const u64 max_vec = (a.N >> 2) + 1;
  a.tiles_per_row = (max_vec + vec_per_tile - 1) / vec_per_tile;
  if (a.tiles_per_row == 0) a.tiles_per_row = 1;
  a.total_tiles = a.tiles_per_row * a.nrows;
  u64 need = (a.total_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  if (need < 1) need = 1;
  if (grid == 0) grid = blocks_per_cu * device_cu_count();
  if ((u64)grid > need) grid = (u32)need;
  // several rows: chunks of up to kFilterRun tiles, but short enough that every
  // wavefront gets about four (16 rows of 2^22 values are only 256 chunks of 64 tiles,
  // which would leave most wavefronts idle); rows of at most 2^20 values, up to
  // kFoRows of them, are read in the flat pass's order instead (FO)
  // positions fit above the index: bits(N - 1) + bits(nrows - 1) <= 32
  auto bits = [](u64 v) { u32 b = 0; while (v) { ++b; v >>= 1; } return b; };
  const bool fo = a.nrows > 1 && a.nrows <= kFoRows && a.N >= 2 && bits(a.N - 1) + bits(a.nrows - 1) <= 32 &&
                  a.hits_per_row * (double)a.nrows <= 0.8 * kStageCap * (double)grid * kWavesPerBlock;
  a.run = 1;
  if (a.nrows > 1 && !fo) {
    const u64 per = a.total_tiles / ((u64)grid * kWavesPerBlock * 4);
    a.run = per < 1 ? 1 : (per > kFilterRun ? kFilterRun : per);
  }
  // chunk ranges per die, in proportion to (blocks on the die) x (the die's weight)
  const u64 nchunks = (a.total_tiles + a.run - 1) / a.run;
  double share[kXcds], tot = 0.0;
  for (u32 x = 0; x < kXcds; ++x) {
    const u64 nb = grid > x ? (grid - x + kXcds - 1) / kXcds : 0;
    const float w = a0.weight[x] > 0.f ? a0.weight[x] : 1.f;
    share[x] = (double)nb * (double)w;
    tot += share[x];
  }
  double acc = 0.0;
  a.split[0] = 0;
  for (u32 x = 0; x < kXcds; ++x) {
    acc += share[x];
    a.split[x + 1] = x + 1 == kXcds ? nchunks : (u64)((double)nchunks * acc / tot + 0.5);
    if (a.split[x + 1] < a.split[x]) a.split[x + 1] = a.split[x];
    if (a.split[x + 1] > nchunks) a.split[x + 1] = nchunks;
  }
  if (split_out)
    for (u32 x = 0; x <= kXcds; ++x) split_out[x] = a.split[x];
  if (fo)
    filter_kernel<U, true, true><<<grid, kFilterThreads, 0, s>>>(a);
  else
    filter_kernel<U, true, false><<<grid, kFilterThreads, 0, s>>>(a);
  return hipGetLastError();
}
}  // namespace

// Launch shape by the expected share of hits (measured on MI355X; 1..8 blocks per CU,
// 4..16 float4 per lane).  One block of four wavefronts per CU with 8-float4 tiles
// streams fastest while hits are rare (598 us per 2^30 values at k = 32), but a
// wavefront that stages hits stops issuing loads, and with one wavefront per SIMD
// nothing covers for it (939 us at k = 2^19).  Two blocks of 4-float4 tiles keep the
// rate when tiles carry hits; a third costs 3-4 us per 2^30 values at k <= 2^15 and
// 5-10% at 2^22..2^28 values (more blocks queue their end-of-stream reservations on R).
// Four blocks per CU cover for the wavefronts that stage hits when hits come in one
// value in 256 or more over 2^25 values or more (k = 2^19 over 2^26 values: 0.144
// against 0.168 ms per call), or in one in 2048 or more over 2^29 values or more (k = 2^19
// over 2^30 values under the MI355X rule: one in ~820, 692-696 against 706-708 us; the
// batched rows).  Shorter passes keep two even then (2^22 values, k = 2^15: 0.068
// against 0.078 ms).
hipError_t launch_filter(const FilterArgs& a, u32 grid, hipStream_t s, u64* split_out) {
  if (a.sparse == kShapeSparse) return launch_filter_shape<8>(a, grid, 1, s, split_out);
  const u64 n = a.N * a.nrows;
  const bool four = (a.sparse == kShapeVeryDenseHits && n >= (1ull << 25)) ||
                    (a.sparse == kShapeDenseHits && n >= (1ull << 29));
#ifndef PROFK_SHORT_FILTER_LOG2
#define PROFK_SHORT_FILTER_LOG2 23
#endif
  // short inputs: one block per CU (the blocks end their streams together, and each adds
  // to R once)
  const bool short_in = n <= (1ull << PROFK_SHORT_FILTER_LOG2);
  const u32 bpc = four ? 2 * kFilterBlocksPerCU : (short_in ? 1u : kFilterBlocksPerCU);
  return launch_filter_shape<4>(a, grid, bpc, s, split_out);
}

}  // namespace profk
