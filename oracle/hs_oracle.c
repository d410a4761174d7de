/*
 * ORACLE — test infrastructure, not product code.
 *
 * A plain, slow, single-threaded CPU model of the HiSparse swap-in step,
 * written so that each step can be checked against the pages by eye. Only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark may load
 * it; the HIP library never calls, links or includes anything here, and this
 * file includes nothing from the HIP library.
 *
 * What one resolve computes, per request (pages: "HiSparse: Turbocharging
 * Sparse Attention with Hierarchical Memory", section 2, the three steps of
 * the swap-in kernel; the Japanese review of the same post, section
 * 「効率的なSwap-inカーネル」; and "vLLM GLM 5.3 最適化: Hybrid HiSparse
 * オフローディング", section 2 Mixed Residency):
 *   1. find which selected ids miss the hot device buffer (resident tail ids
 *      resolve in place, ids already in a slot are hits);
 *   2. pick LRU eviction victims among slots not hit this step;
 *   3. update the page table and fetch each missed row from the host pool into
 *      its victim slot; hit slots have their last-use step refreshed.
 * The pages say only "LRU". The tie-breaks this model fixes are:
 *   - eviction order is ascending (stamp, slot), an empty slot having stamp -1,
 *     so empty slots go first, lowest index first;
 *   - misses are paired with victims in ascending token-id order;
 *   - the stamp of a hit slot and of a newly filled slot becomes the step t.
 * With these rules the outcome is unique.
 *
 * The pages compare LRU with another eviction strategy they do not name
 * ("HiSparse: Turbocharging Sparse Attention with Hierarchical Memory",
 * section 2, and the Japanese review, section 「効率的なSwap-inカーネル」). The
 * model also runs FIFO as that alternative: the same steps, except that a hit
 * leaves its slot's stamp alone, so a slot's stamp is the step it was filled.
 *
 * Invalid ids never trap: -1 is padding (output -1, no effect), an id outside
 * [0, host_rows) or at/after tail0 but outside the tail window sets
 * ORACLE_BAD_ID, a repeat of an earlier valid id in the same step sets
 * ORACLE_DUP_ID; both give output -1.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BAD_ID 1
#define ORACLE_DUP_ID 2

#define ORACLE_LRU 0
#define ORACLE_FIFO 1

typedef struct {
  int32_t B;          /* hot slots per request */
  int32_t k;          /* selected ids per step */
  int32_t H;          /* host rows per request */
  int32_t T;          /* device-resident tail rows per request (0: none) */
  int64_t row_bytes;  /* bytes per KV row */
  int32_t policy;     /* ORACLE_LRU or ORACLE_FIFO */
} oracle_dims;

typedef struct { int32_t key; int32_t val; } pair_t;

static int by_key_then_val(const void* a, const void* b) {
  const pair_t* p = (const pair_t*)a;
  const pair_t* q = (const pair_t*)b;
  if (p->key != q->key) return p->key < q->key ? -1 : 1;
  if (p->val != q->val) return p->val < q->val ? -1 : 1;
  return 0;
}

/* Reset one request: no token in any slot, no stamps, empty page table, step 0.
 * The hot buffer's bytes are left as they are. */
void oracle_reset(const oracle_dims* d, int32_t* slot_tok, int32_t* stamp, int32_t* page, int32_t* t) {
  for (int32_t s = 0; s < d->B; ++s) { slot_tok[s] = -1; stamp[s] = -1; }
  for (int32_t x = 0; x < d->H; ++x) page[x] = -1;
  *t = 0;
}

/*
 * One resolve of one request.
 *   slot_tok[B], stamp[B], page[H], t, hot[B*row_bytes]: the request's state, updated in place.
 *   host[H*row_bytes]: the request's host pool rows; tail[T*row_bytes]: its device tail rows
 *     (may be NULL when has_tail == 0).
 *   ids[k]: the selected token ids; tail0: first resident token when has_tail != 0.
 *   out[k]: slot for a hit or miss, B + (id mod T) for a resident id, -1 otherwise. The device tail is a
 *     ring of T rows: it holds the tokens [tail0, tail0 + T), token x in row x mod T.
 *   gather[k*row_bytes] (optional): the row each output names; zeros for -1.
 * Returns 0, or -1 when a request has more misses than free slots (needs B < k).
 */
int oracle_resolve(const oracle_dims* d, int32_t* slot_tok, int32_t* stamp, int32_t* page, int32_t* t_io,
                   uint8_t* hot, const uint8_t* host, const uint8_t* tail, const int32_t* ids, int32_t has_tail,
                   int32_t tail0, int32_t* out, int32_t* miss_out, int32_t* status_out, uint8_t* gather) {
  const int32_t B = d->B, k = d->k, H = d->H, T = d->T;
  const int64_t rb = d->row_bytes;
  const int32_t t = *t_io;
  int32_t status = 0;
  uint8_t* seen = (uint8_t*)calloc((size_t)H, 1);
  uint8_t* hit = (uint8_t*)calloc((size_t)B, 1);
  pair_t* misses = (pair_t*)malloc(sizeof(pair_t) * (size_t)(k > 0 ? k : 1));
  pair_t* cand = (pair_t*)malloc(sizeof(pair_t) * (size_t)B);
  if (!seen || !hit || !misses || !cand) { free(seen); free(hit); free(misses); free(cand); return -2; }

  /* step 1: classify every selected id; collect the misses as (token, position) */
  int32_t m = 0;
  for (int32_t i = 0; i < k; ++i) {
    const int32_t x = ids[i];
    out[i] = -1;
    if (x == -1) continue;
    if (x < 0 || x >= H) { status |= ORACLE_BAD_ID; continue; }
    const int resident = has_tail && (int64_t)x >= (int64_t)tail0;
    if (resident && (int64_t)x - (int64_t)tail0 >= (int64_t)T) { status |= ORACLE_BAD_ID; continue; }
    /* repeats are looked for among valid ids only */
    if (seen[x]) { status |= ORACLE_DUP_ID; continue; }
    seen[x] = 1;
    if (resident) { out[i] = B + x % T; continue; }
    if (page[x] != -1) {
      out[i] = page[x];
      hit[page[x]] = 1;
      continue;
    }
    misses[m].key = x;
    misses[m].val = i;
    ++m;
  }
  /* misses in ascending token-id order */
  qsort(misses, (size_t)m, sizeof(pair_t), by_key_then_val);

  /* step 2: eviction candidates = slots not hit this step, in ascending (stamp, slot) */
  int32_t c = 0;
  for (int32_t s = 0; s < B; ++s) {
    if (hit[s]) continue;
    cand[c].key = stamp[s];
    cand[c].val = s;
    ++c;
  }
  qsort(cand, (size_t)c, sizeof(pair_t), by_key_then_val);
  if (m > c) { free(seen); free(hit); free(misses); free(cand); return -1; }

  /* step 3: the j-th smallest missed id takes the j-th victim; page table, slot table,
   * stamp, and the row copied from the host pool */
  for (int32_t j = 0; j < m; ++j) {
    const int32_t v = cand[j].val;
    const int32_t x = misses[j].key;
    const int32_t y = slot_tok[v];
    if (y != -1) page[y] = -1;
    slot_tok[v] = x;
    page[x] = v;
    stamp[v] = t;
    memcpy(hot + (int64_t)v * rb, host + (int64_t)x * rb, (size_t)rb);
    out[misses[j].val] = v;
  }
  /* LRU: hit slots were used at step t too; FIFO: a slot keeps the step it was filled */
  if (d->policy == ORACLE_LRU)
    for (int32_t s = 0; s < B; ++s)
      if (hit[s]) stamp[s] = t;

  *miss_out = m;
  *status_out = status;
  *t_io = t + 1;

  if (gather) {
    for (int32_t i = 0; i < k; ++i) {
      uint8_t* g = gather + (int64_t)i * rb;
      const int32_t o = out[i];
      if (o < 0) memset(g, 0, (size_t)rb);
      else if (o < B) memcpy(g, hot + (int64_t)o * rb, (size_t)rb);
      else memcpy(g, tail + (int64_t)(o - B) * rb, (size_t)rb);
    }
  }
  free(seen); free(hit); free(misses); free(cand);
  return 0;
}

/*
 * The same step for n requests laid out back to back (request r at offset r times each
 * per-request size). tail0s may be NULL (no tail); tail and gather may be NULL.
 * Returns 0, or the first failing request's code.
 */
int oracle_resolve_batch(const oracle_dims* d, int32_t n, int32_t* slot_tok, int32_t* stamp, int32_t* page,
                         int32_t* t, uint8_t* hot, const uint8_t* host, const uint8_t* tail, const int32_t* ids,
                         const int32_t* tail0s, int32_t* out, int32_t* miss, int32_t* status, uint8_t* gather) {
  const int64_t rb = d->row_bytes;
  for (int32_t r = 0; r < n; ++r) {
    int rc = oracle_resolve(d, slot_tok + (int64_t)r * d->B, stamp + (int64_t)r * d->B, page + (int64_t)r * d->H,
                            t + r, hot + (int64_t)r * d->B * rb, host + (int64_t)r * d->H * rb,
                            tail ? tail + (int64_t)r * d->T * rb : NULL, ids + (int64_t)r * d->k,
                            tail0s != NULL, tail0s ? tail0s[r] : 0, out + (int64_t)r * d->k, miss + r, status + r,
                            gather ? gather + (int64_t)r * d->k * rb : NULL);
    if (rc) return rc;
  }
  return 0;
}

/*
 * Offload of device rows into one request's host pool: row j becomes host row pos + j, and a slot that
 * holds that token gets the same row (inactive KV lives in host memory, "HiSparse: Turbocharging Sparse
 * Attention with Hierarchical Memory", section 2; finished prefix pages are copied to host memory ahead of
 * eviction, "vLLM GLM 5.3 最適化: Hybrid HiSparse オフローディング", section 1 Full Residency). Rows outside
 * [0, H) are skipped; returns ORACLE_BAD_ID if any was, else 0.
 */
int oracle_offload(const oracle_dims* d, uint8_t* host, uint8_t* hot, const int32_t* page, const uint8_t* rows,
                   int32_t pos, int32_t n) {
  const int64_t rb = d->row_bytes;
  int status = 0;
  for (int32_t j = 0; j < n; ++j) {
    const int64_t x = (int64_t)pos + j;
    if (x < 0 || x >= d->H) { status = ORACLE_BAD_ID; continue; }
    memcpy(host + x * rb, rows + (int64_t)j * rb, (size_t)rb);
    if (page[x] != -1) memcpy(hot + (int64_t)page[x] * rb, rows + (int64_t)j * rb, (size_t)rb);
  }
  return status;
}

/*
 * Advance one request's device tail by n tokens (the Mixed-residency tail migrating to host memory under
 * pressure, "vLLM GLM 5.3 最適化: Hybrid HiSparse オフローディング", section 2): tokens tail0 .. tail0+n-1
 * leave the ring; their rows (ring row x mod T) are written to host rows x, and into the hot slot of a token
 * that has one. n is clamped to [0, T]; tokens at or past H are skipped (ORACLE_BAD_ID). tail0 advances by n.
 */
int oracle_advance_tail(const oracle_dims* d, uint8_t* host, const uint8_t* tail, uint8_t* hot, const int32_t* page,
                        int32_t* tail0, int32_t n) {
  const int64_t rb = d->row_bytes;
  int status = 0;
  if (n < 0) n = 0;
  if (n > d->T) n = d->T;
  for (int32_t j = 0; j < n; ++j) {
    const int64_t x = (int64_t)*tail0 + j;
    if (x < 0 || x >= d->H) { status = ORACLE_BAD_ID; continue; }
    memcpy(host + x * rb, tail + (x % d->T) * rb, (size_t)rb);
    if (page[x] != -1) memcpy(hot + (int64_t)page[x] * rb, tail + (x % d->T) * rb, (size_t)rb);
  }
  *tail0 += n;
  return status;
}
