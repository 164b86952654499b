/*
 * Exact top-k oracle: TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this library.  It shares no code, header or table with the GPU
 * library: it is the plain definition of the result, written out.
 *
 * What it computes.  Prof-K ("Prof-K: Probabilistic One-Pass Filtering for
 * Efficient Top-k Selection", arXiv HTML page, §3 "Problem Setup and
 * Algorithm Overview") returns the k largest entries of x with their
 * indices, and the abstract and §3 stage 4 state that the returned set is
 * always the exact top-k.  The pages assume distinct entries (§4 "Notation
 * and Conventions"); with ties we use the total order
 *
 *     i before j  <=>  x_i > x_j,  or  x_i == x_j and i < j
 *
 * (IEEE comparison, so -0.0 == +0.0; every NaN ranks above +inf and NaNs
 * tie with each other, broken by index).  The output is the first k indices
 * in that order, values copied bit for bit from x.
 *
 * How: a bounded min-heap of the k best seen so far (root = the element
 * that ranks last among them).  Each input element is compared with the
 * root and replaces it when it ranks before it.  At the end the heap is
 * sorted into output order.  O(N log k) worst case, no cleverness.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  float v;
  int64_t i;
} entry_t;

/* 1 when a ranks strictly before b in the total order above. */
static int ranks_before(entry_t a, entry_t b) {
  int an = isnan(a.v), bn = isnan(b.v);
  if (an || bn) {
    if (an && bn) return a.i < b.i;
    return an; /* the NaN one ranks first */
  }
  if (a.v > b.v) return 1;
  if (a.v < b.v) return 0;
  return a.i < b.i; /* equal values (including -0.0 vs +0.0) */
}

/* Heap ordered so that heap[0] is the entry that ranks LAST. */
static void sift_down(entry_t* h, int64_t n, int64_t p) {
  for (;;) {
    int64_t l = 2 * p + 1, r = l + 1, w = p;
    if (l < n && ranks_before(h[w], h[l])) w = l; /* l ranks later than w */
    if (r < n && ranks_before(h[w], h[r])) w = r;
    if (w == p) return;
    entry_t t = h[p];
    h[p] = h[w];
    h[w] = t;
    p = w;
  }
}

static void sift_up(entry_t* h, int64_t c) {
  while (c > 0) {
    int64_t p = (c - 1) / 2;
    if (!ranks_before(h[p], h[c])) return; /* parent already ranks later */
    entry_t t = h[p];
    h[p] = h[c];
    h[c] = t;
    c = p;
  }
}

/* Push candidate e into the bounded heap (capacity k, current size *n). */
static void offer(entry_t* h, int64_t* n, int64_t k, entry_t e) {
  if (*n < k) {
    h[*n] = e;
    sift_up(h, *n);
    (*n)++;
  } else if (ranks_before(e, h[0])) {
    h[0] = e;
    sift_down(h, *n, 0);
  }
}

static int cmp_output(const void* pa, const void* pb) {
  entry_t a = *(const entry_t*)pa, b = *(const entry_t*)pb;
  if (ranks_before(a, b)) return -1;
  if (ranks_before(b, a)) return 1;
  return 0;
}

/* Scan x[lo:hi) (row-relative indices lo..hi-1) into the heap. */
static void scan_range(const float* x, int64_t lo, int64_t hi, entry_t* h, int64_t* n,
                       int64_t k) {
  for (int64_t i = lo; i < hi; ++i) {
    entry_t e = {x[i], i};
    offer(h, n, k, e);
  }
}

typedef struct {
  const float* x;
  int64_t lo, hi, k;
  entry_t* heap;
  int64_t n;
} chunk_job_t;

static void* chunk_worker(void* arg) {
  chunk_job_t* j = (chunk_job_t*)arg;
  j->n = 0;
  scan_range(j->x, j->lo, j->hi, j->heap, &j->n, j->k);
  return NULL;
}

/*
 * oracle_topk: exact top-k of one row x[0..N), 1 <= k <= N.
 * out_vals[j] is the bit copy of x[out_idx[j]]; j = 0 is the first in order.
 * nthreads <= 1 runs single-threaded; otherwise the row is cut into nthreads
 * contiguous chunks, each keeps its own top-k heap, and the union of the
 * chunk heaps is reduced by one more heap (the global top-k is contained
 * in that union).  Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_topk(const float* x, int64_t N, int64_t k, int nthreads, float* out_vals,
                int64_t* out_idx) {
  if (!x || !out_vals || !out_idx || N < 1 || k < 1 || k > N) return -1;
  entry_t* heap = (entry_t*)malloc((size_t)k * sizeof(entry_t));
  if (!heap) return -1;
  int64_t n = 0;
  if (nthreads <= 1 || N < (int64_t)nthreads * 4096) {
    scan_range(x, 0, N, heap, &n, k);
  } else {
    int T = nthreads;
    chunk_job_t* jobs = (chunk_job_t*)calloc((size_t)T, sizeof(chunk_job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)T, sizeof(pthread_t));
    if (!jobs || !th) {
      free(heap);
      free(jobs);
      free(th);
      return -1;
    }
    int ok = 1;
    for (int t = 0; t < T; ++t) {
      jobs[t].x = x;
      jobs[t].lo = N * t / T;
      jobs[t].hi = N * (t + 1) / T;
      jobs[t].k = k;
      jobs[t].heap = (entry_t*)malloc((size_t)k * sizeof(entry_t));
      if (!jobs[t].heap) ok = 0;
    }
    if (ok) {
      for (int t = 0; t < T; ++t) pthread_create(&th[t], NULL, chunk_worker, &jobs[t]);
      for (int t = 0; t < T; ++t) pthread_join(th[t], NULL);
      for (int t = 0; t < T; ++t)
        for (int64_t j = 0; j < jobs[t].n; ++j) offer(heap, &n, k, jobs[t].heap[j]);
    }
    for (int t = 0; t < T; ++t) free(jobs[t].heap);
    free(jobs);
    free(th);
    if (!ok) {
      free(heap);
      return -1;
    }
  }
  qsort(heap, (size_t)n, sizeof(entry_t), cmp_output);
  for (int64_t j = 0; j < n; ++j) {
    memcpy(&out_vals[j], &x[heap[j].i], sizeof(float));
    out_idx[j] = heap[j].i;
  }
  free(heap);
  return 0;
}

/*
 * oracle_topk_batched: the same definition applied to each of B rows
 * independently (§3 of the arXiv page: batched inputs are handled row by
 * row).  Row r starts at x + r*ld; indices are column indices in [0, N).
 */
int oracle_topk_batched(const float* x, int64_t B, int64_t N, int64_t ld, int64_t k,
                        int nthreads, float* out_vals, int64_t* out_idx) {
  if (B < 1 || ld < N) return -1;
  for (int64_t r = 0; r < B; ++r) {
    int rc = oracle_topk(x + r * ld, N, k, nthreads, out_vals + r * k, out_idx + r * k);
    if (rc) return rc;
  }
  return 0;
}

/*
 * oracle_count_ranked_before_or_at: R(tau) = #{ i : i is at or before tau }
 * in the total order, where tau = (tau_val, tau_idx) is a position in that
 * order.  This is the count the filter of §3 stage 3 produces when ties are
 * broken by index (the pages' R, §4 "Notation and Conventions").
 */
int64_t oracle_count_at_or_before(const float* x, int64_t N, float tau_val, int64_t tau_idx) {
  entry_t tau = {tau_val, tau_idx};
  int64_t c = 0;
  for (int64_t i = 0; i < N; ++i) {
    entry_t e = {x[i], i};
    if (e.i == tau.i || ranks_before(e, tau)) c++;
  }
  return c;
}
