// Host-side launchers of the Prof-K kernels (one declaration per launch group).
#pragma once

#include "profk_device.h"

namespace profk {

constexpr u32 kSmallSort = 8192;  // keys sorted by one workgroup in LDS (64 KB)
constexpr u32 kTickets = 64;      // u32 tickets / counters in the workspace; each user leaves its own zero
// The filter's two-level ticket: kFilterGroups counters, each on its own 128-byte line,
// after the tickets.  Cleared together with them.
constexpr u32 kFilterGroups = 32;
constexpr u32 kFilterGroupStride = 32;  // u32 words between group counters
constexpr u32 kTicketWords = kTickets + kFilterGroups * kFilterGroupStride + 32;
constexpr u32 kXtimeWord = kTickets + kFilterGroups * kFilterGroupStride;  // u64-aligned, 2 x (kXcds + 1) words
constexpr u32 kFilterBlocksPerCU = 2;  // persistent filter grid: 2 blocks x 4 waves per CU (4 for dense hits)
constexpr u32 kShapeSparse = 1;        // filter launch shapes by expected hit density
constexpr u32 kShapeDenseHits = 2;     // hits in one value in 2048 or more
constexpr u32 kShapeVeryDenseHits = 3; // hits in one value in 256 or more
constexpr u64 kFilterRun = 64;         // consecutive tiles per chunk when there are several rows

// Compute units of the current device (cached per device).
inline u32 device_cu_count() {
  static u32 cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = (u32)n;
  }
  return cache[dev];
}

struct FilterArgs {
  const float* x;      // row 0
  u64 ld;              // row stride (elements)
  u64 N;               // values per row
  const int* rows;     // rows to process (device), or nullptr for rows 0..nrows-1
  u64 nrows;
  RowCtl* ctls;        // per row: tau in, R / status out
  u64* cand;           // per row M keys, row stride M
  u64 M;
  u64 k;
  u32* ticket;         // zero before the launch; left zero after it
  u32* groups;         // kFilterGroups counters kFilterGroupStride words apart; zero, left zero
  u64* xtime;          // kXcds + 1 words: start (min) and per-die stream ends (max); zero, left zero
  HostRecord* hrec;    // where the last block copies xtime for the host, or nullptr
  u32 seq;             // with hrec: the attempt's sequence number for hrec->early (row 0)
  u32 summary;         // with hrec, several rows: hrec->early says whether every listed row
                       // passed its check instead of row 0's R
  u64 split[kXcds + 1];  // chunk ranges per die (set by launch_filter from weights)
  float weight[kXcds];   // relative speed of each die (input to launch_filter; 0 = equal)
  u32 sparse;            // launch shape by the expected density of hits: kShapeSparse (fewer
                         // than one value in 8192), kShapeDenseHits, kShapeVeryDenseHits, or 0
  AttemptRecord* rec;  // per row, or nullptr
  SelState* sels;      // per row refinement selection to arm, or nullptr
  u64 tiles_per_row;   // set by launch_filter
  u64 total_tiles;
  u64 run;             // tiles per chunk of the block-cyclic order (set by launch_filter)
  double hits_per_row; // several rows: the expected hits per row, E[R] (0: unknown)
};

hipError_t launch_attempt_init(RowCtl* ctl, SelState* sel, AttemptRecord* rec, u32* tickets, u32 nrows,
                               u32* refine_hist, hipStream_t s);
// Stages 1-2 (k_sample.hip).  Ticket slots of the workspace's ticket array:
constexpr u32 kTicketFilter = 0;  // filter kernel
constexpr u32 kTicketSample = 8;  // sampling kernel: one u64 at slots 8-9 (8-byte aligned),
                                  // (blocks done << 32) | distinct draws so far
constexpr u32 kCountStage = 4;    // output counter of the stage entry points
constexpr u32 kTicketRefine = 16; // one-launch refinement for small k
constexpr u32 kTopT = 64;         // largest t of the sorted per-block lists
constexpr u32 kTopBlocks = 128;   // most sampling blocks of that path (S <= 131072)
// How a sampling launch finds tau, the t-th largest of its S draws (sample_mode):
constexpr u32 kTauKeys = 0;         // from the key slots: in LDS when they fit, else one workgroup over L2
constexpr u32 kTauSortedLists = 1;  // per-block sorted lists of pow2(t) keys (t <= kTopT), merged in LDS
constexpr u32 kTauTopLists = 2;     // per-block unordered top t (t <= 1024), selected from in LDS
constexpr u32 kTauPasses = 3;       // multi-block radix select passes over the key slots (one row)

struct SampleArgs {
  const float* x;
  u64 N, S;
  u64 seed;
  u32 attempt, row;
  u32* table;       // hash set, tmask + 1 slots, zero on entry
  u64 tmask;
  u64* keys;        // 2S slots: draw j < S at keys[j] (0 = repeat), top-up from keys[S]
  u64* tops;        // per-block lists (kTauSortedLists, kTauTopLists): tops_words of sample_shape
  RowCtl* ctl;      // tau out; the per-attempt fields are reset
  AttemptRecord* rec;  // reset, or nullptr
  u64* ticket;      // (blocks done << 32) | distinct draws; zero on entry, left zero
  u32* top_hist;    // 256 words, zero on entry, left zero
  u64 t;            // threshold rank (0: sample only)
  u32 mode;         // how tau is found: one of kTau* (sample_shape)
  u32 threads;      // workgroup size (sample_shape)
  SelState* sel;    // kTauPasses: armed by the last block for the select passes (one row)
  u64* col;         // kTauPasses: kCollectCap keys of collect space for the passes
  // Several rows at once (the batched form): the grid has one row of blocks per row
  // in the list (blockIdx.y is the position in it).  The pointers above are for row 0
  // (x, ctl, rec, top_hist, indexed by row id) or list position 0 (table, keys, tops,
  // ticket) and advance by these strides; the Philox counter takes the row id.
  // nrows = 0: one row, the fields above as they are.
  const int* rows;  // row ids, or nullptr for rows row0 .. row0 + nrows - 1
  u32 nrows;
  u32 row0;
  u64 ld;           // elements between rows of x
  u64 table_stride; // u32 slots between positions' hash sets
  u64 keys_stride;  // u64 words between positions' key slots
  u64 tops_stride;  // u64 words between positions' block lists
  u64 ticket_stride;  // u64 words between positions' tickets
  u64 hist_stride;  // u32 words between rows' top-digit histograms
};

// Sampling launch shape for (S, t): 256-thread workgroups while the per-block-list
// threshold path applies and needs at most kTopBlocks of them, else 1024 threads.
// The launch for S draws of N and rank t: how tau is found (kTau*; kTauPasses only
// where `passes`: one row with a SelState), the workgroup size and count, and the u64
// words of per-block lists one row needs (at least 1).
struct SampleShape {
  u32 mode, threads, blocks;
  u64 tops_words;
};
SampleShape sample_shape(u64 S, u64 t, u64 N, bool passes);
hipError_t launch_sample(const SampleArgs& a, hipStream_t s);
hipError_t launch_clear_sample(u32* table, u64 slots, u32* tickets, hipStream_t s);
hipError_t launch_keys_to_index_compact(const u64* keys, const u64* n_ptr, u64 n_cap, int64_t* out, u32* counter,
                                        hipStream_t s);
hipError_t launch_keys_to_index(const u64* keys, const u64* n_ptr, u64 n_cap, int64_t* out, hipStream_t s);
hipError_t launch_tau_to_output(const float* x, u64 N, const RowCtl* ctl, float* out_val, int64_t* out_idx,
                                hipStream_t s);
hipError_t launch_set_tau(RowCtl* ctl, u32* tickets, u32 tau_bits, u32 tau_idx, hipStream_t s);
hipError_t launch_r_to_output(const RowCtl* ctl, int64_t* out_R, hipStream_t s);

hipError_t launch_select_keys(const u64* keys, const u64* n_ptr, u64 n_cap, SelState* st, u64* col, u64* result,
                              u32* status, hipStream_t s);
hipError_t launch_select_x(const float* x, u64 N, SelState* st, u64* col, u64* result, u32* status,
                           hipStream_t s);
hipError_t launch_compact_keys(const u64* keys, const u64* n_ptr, u64 n_cap, RowCtl* ctl, u64* out, u64 k,
                               hipStream_t s);
// The compaction of the exact full selection: the filter with tau = ctl->kth and
// capacity k (tickets: the workspace's ticket words, zero, left zero).
hipError_t launch_compact_x(const float* x, u64 N, RowCtl* ctl, u64* out, u64 k, u32* tickets, hipStream_t s);
hipError_t launch_arm_select(SelState* st, u64 rank, u64 count, RowCtl* ctl, hipStream_t s);

// split_out (host, kXcds + 1 words, or nullptr): the per-die chunk ranges used.
hipError_t launch_filter(const FilterArgs& a, u32 grid, hipStream_t s, u64* split_out = nullptr);

// Binned refinement (k_refine.hip).
constexpr u32 kBinBits = 14;
constexpr u32 kBins = 1u << kBinBits;
constexpr u32 kBinCap = 4096;  // keys one sorting workgroup holds in LDS (32 KB)

constexpr u32 kMsdBits = 12;  // digit of the in-kernel partition of oversized bins
constexpr u32 kMsdDigits = 1u << kMsdBits;

// Largest part one wavefront sorts in registers (8 keys per lane): a wider register
// sort would set the bin sort kernel's register count, and with it its occupancy.
constexpr u32 kWaveBinBits = 9;
constexpr u32 kWaveBin = 1u << kWaveBinBits;

// Work-list entries (start | count << 32) of the in-kernel partition of oversized
// bins: two lists per oversized bin, at most kBins + M / kWaveBin + 2 pairs in all.
__host__ __device__ inline u64 msd_pool_words(u64 M) { return 2 * (M / kWaveBin + kBins + 2); }
// The bin sort's wavefront w sorts the bins that start in output positions
// [w P, (w + 1) P), P = ceil(T / W) for the T keys of the needed bins.  Chunk boundary m
// (0 <= m <= W) holds {start, end, descending position} of the bin that holds position
// m P - 1 ({T, T, -} past T).  The launch makes W >= T_max / kChunkKeys, so that the bins
// before the last one of a chunk hold fewer than kChunkKeys keys; at most kSortBlocksCap
// workgroups of four wavefronts beyond that.
constexpr u32 kChunkKeys = 128;
constexpr u32 kSortBlocksCap = 1024;
__host__ __device__ inline u64 chunk_entries(u64 M) { return 4ull * kSortBlocksCap + M / kChunkKeys + 8; }

struct RefineArgs {
  RowCtl* ctl;
  u64* cand;        // min(R, M) candidate keys; reused as the partition's second buffer
  u64 M;
  u64 k;
  u64 N;
  const float* x;   // the row (outputs copy x[idx])
  u64* tmp;         // M keys: candidates of bins >= b* in bin order
  u32* hist;        // kBins, zero on entry, left zero
  u32* chunk;       // chunk_entries(M) x 4 words: the bin sort's output chunks (below)
  u32 sort_waves;   // W, wavefronts of the bin sort; set by launch_refine
  u32* cursor;      // kBins
  u32* table;       // sampler hash set cleared by the last launch, or nullptr
  u64 table_slots;
  HostRecord* hrec;  // pinned host record published by the scan, or nullptr
  u32 seq;
  u64 early_cap;    // nonzero: the host takes R and the check from the filter's early
                    // word when the check failed or R <= early_cap, and the scan then
                    // skips its record (a system-scope release); 0: always published
  AttemptRecord* rec;
  float* out_vals;
  int64_t* out_idx;
  u64* pool;        // msd_pool_words(M) words: work lists of the oversized-bin partition
  u32* ticket;      // zero, left zero: the one-launch refinement's last-block election, the
                    // fused histogram-and-scatter launch's counter
  u64 wait_ticks;   // bound on that launch's wait for its blocks (100 MHz clock ticks; 0: the
                    // wait counts as run out at once)
  u32 msd_cap;      // largest needed bin partitioned in-kernel; larger ones defer to the
                    // multi-pass refinement (the host reads the flag)
  u32 approx;       // 1: no run-time check (approximate mode): refine whatever the buffer
                    // holds, pad missing outputs, and report R and the check in *info
  ApproxInfo* info; // approximate mode: device result of the check, or nullptr
};

hipError_t launch_refine(const RefineArgs& a, hipStream_t s);
// Whether launch_refine takes the one-launch refinement for small k (else the binned one).
bool refine_one_launch(const RefineArgs& a);
// Approximate mode routed to the exact selection: *info = {N, 0, 0, 1}.
hipError_t launch_approx_info_exact(ApproxInfo* info, u64 N, hipStream_t s);

// Batched form (k_batched.hip): rows of at most kBatchedMaxN values.
constexpr u64 kBatchedMaxN = 1ull << 20;
// Batched refinement: a row buffer of up to this many keys is held in LDS (128 KB); k
// is at most this.
constexpr u64 kBatchedMaxM = 1ull << 14;
// Batched refinement: up to this k the k-th largest is selected in LDS and only the k
// keys at or above it are sorted; above it the whole buffer is sorted.
constexpr u32 kBatchedSelCap = 1024;

struct BatchedArgs {
  const float* x;  // row 0
  u64 ld;          // row stride (elements)
  u64 N;           // values per row
  const int* rows; // rows to process (device), or nullptr for rows 0..nrows-1
  u64 nrows;
  u64 S, t;        // sample size and threshold rank per row
  u64 seed;
  u32 attempt;
  RowCtl* ctls;    // per row
  u64* scratch;    // sample keys: 2S per sampling workgroup
  u64* cand;       // per row M keys (row stride M)
  u64 M;
  u64 k;
  float* out_vals; // B x k
  int64_t* out_idx;
  AttemptRecord* rec;  // per row: the refinement flags an internal error here, or nullptr
  u32* table;      // the batched sampler's hash sets, one per list position, which the
                   // refinement clears; nullptr with the per-row bitmap sampler
  u64 table_slots; // slots per position (a multiple of 4)
  u32 approx;      // 1: approximate mode (refine whatever each row's buffer holds, pad,
                   // and report each row's check in info[row])
  ApproxInfo* info;
  u32 keep_keys;   // stage entry point: row r's sample keys stay in scratch[r * 2S ..)
  u32* tickets;    // pipelined sampler: kTicketWords words it zeroes (nullptr: none)
};

// Whether launch_b_sample runs the pipelined sampler, which also leaves every row it
// samples with a fresh control block and attempt record (what attempt_init does).
bool b_sample_pipelined(u64 S, u64 t, u64 N);

u32 batched_sample_blocks(u64 nrows);

// The pipelined sampler (S <= 4096 and t >= 1) runs on the persistent grid
// (batched_sample_blocks) and keeps no keys unless keep_keys is set; otherwise the
// bitmap sampler runs on `grid` workgroups (0: the persistent grid), and the stage entry
// point gives it one workgroup per row so that every row keeps its keys in its own
// scratch slice.
hipError_t launch_b_sample(const BatchedArgs& a, hipStream_t s, u32 grid = 0);
hipError_t launch_b_stage_out(const float* x, u64 ld, u64 N, u64 B, u64 S, const u64* scratch, const RowCtl* ctls,
                              int64_t* out_idx, float* out_tau_val, int64_t* out_tau_idx, AttemptRecord* rec,
                              hipStream_t s);
hipError_t launch_b_refine(const BatchedArgs& a, hipStream_t s);
hipError_t launch_b_rowsort(const BatchedArgs& a, hipStream_t s);
hipError_t launch_b_info_exact(ApproxInfo* info, u64 nrows, u64 N, hipStream_t s);

// Inputs of 2^32 values or more (k_merge.hip): G sorted per-segment top-k lists.
constexpr u32 kMaxSegments = 64;
struct SegmentLists {
  const float* vals;         // list g at vals + g * stride, sorted by the total order
  const int64_t* idx;        // indices inside segment g, same layout
  u64 stride;                // = k
  u64 k;                     // outputs wanted
  u32 G;                     // lists
  u64 len[kMaxSegments];     // entries of list g (min(k, segment length))
  u64 base[kMaxSegments];    // first global index of segment g
};
hipError_t launch_merge_segments(const SegmentLists& L, float* out_vals, int64_t* out_idx, hipStream_t s);

// Measurement helper (k_probe.hip): one dwordx4 non-temporal streaming read of x.
hipError_t launch_read_ceiling(const float* x, u64 N, u32 blocks_per_cu, unsigned long long* out, hipStream_t s);

hipError_t launch_sort_and_write(u64* buf0, u64* buf1, u32* hist, u32 k, const float* row, u64 N, float* out_vals,
                                 int64_t* out_idx, RowCtl* ctl, AttemptRecord* rec, hipStream_t s);
u64 sort_hist_words(u64 k);

}  // namespace profk
