#define _GNU_SOURCE
/*
 * Seeded synthetic inputs for the HiSparse swap-in path: per-step top-k token
 * streams and the bf16 KV rows of the host pool.
 *
 * This module only *draws inputs*. It holds none of the swap-in method's own
 * arithmetic (no hit test, no LRU, no page table); both the CPU oracle and the
 * HIP path consume what it produces.
 *
 * Random numbers come from SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): a 64-bit counter advanced by
 * the golden-ratio increment and passed through the published finaliser.
 * Every request-step owns its own counter, so results do not depend on thread
 * count or on the order in which requests are generated.
 *
 * Stream recipe (one request, one step t, context length L_t):
 *   step 0  : optional forced current token L_t-1, then uniform distinct draws
 *             from [0, L_t) up to k ids, then a Fisher-Yates shuffle;
 *   step t>0: keep floor(keep_permille*k/1000) ids of the previous step chosen
 *             by a partial Fisher-Yates shuffle, add the forced current token,
 *             then refill to k ids in two parts drawn without repetition:
 *             part A uniform over range A, part B uniform over range B, where
 *             |B| = floor(partB_permille * n_new / 1000) and |A| = n_new - |B|;
 *             finally a full Fisher-Yates shuffle fixes the order.
 * Ranges: plain workloads use A = [0, L_t) and B = the last `window` tokens of
 * [0, L_t); hybrid-residency workloads use A = [0, L - T) (the host region)
 * and B = [L - T, L) (the device tail).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

typedef struct { uint64_t s; } rng_t;

static inline uint64_t rng_next(rng_t* g) { g->s += GOLDEN; return sm64_mix(g->s); }

/* uniform integer in [0, n), n < 2^32: high 32 bits scaled by n */
static inline uint32_t rng_below(rng_t* g, uint32_t n) {
  return (uint32_t)(((rng_next(g) >> 32) * (uint64_t)n) >> 32);
}

/* the counter of (seed, request, step) */
static inline rng_t rng_for(uint64_t seed, uint32_t r, uint32_t t) {
  rng_t g;
  g.s = sm64_mix(seed ^ sm64_mix(((uint64_t)r << 32) | (uint64_t)t));
  return g;
}

typedef struct {
  int32_t k;              /* ids per step */
  int32_t L0;             /* context length at step 0 */
  int32_t grow;           /* 1: L_t = L0 + t and token L_t-1 is forced into every step */
  int32_t keep_permille;  /* retained share of the previous step, in 1/1000 */
  int32_t window;         /* recent window for part B (plain workloads) */
  int32_t tail;           /* T > 0: hybrid workload, part B drawn from [L-T, L) */
  int32_t partB_permille; /* share of the refill drawn from range B, in 1/1000 */
} ws_spec;

/* marks: one byte per token of [0, L_max); cleared entry by entry after use */
static int draw_distinct(rng_t* g, int32_t lo, int32_t hi, int32_t n, int32_t* dst, int32_t* cnt,
                         uint8_t* mark) {
  int32_t span = hi - lo;
  if (n <= 0) return 0;
  if (span <= 0) return -1;
  /* the range must still hold n unmarked tokens, else rejection would not end */
  int32_t taken = 0;
  for (int32_t i = 0; i < *cnt; ++i) taken += (dst[i] >= lo && dst[i] < hi);
  if (span - taken < n) return -1;
  while (n > 0) {
    int32_t x = lo + (int32_t)rng_below(g, (uint32_t)span);
    if (mark[x]) continue;
    mark[x] = 1;
    dst[(*cnt)++] = x;
    --n;
  }
  return 0;
}

static void shuffle(rng_t* g, int32_t* a, int32_t n) {
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)rng_below(g, (uint32_t)(i + 1));
    int32_t tmp = a[i]; a[i] = a[j]; a[j] = tmp;
  }
}

/*
 * Generate steps [0, n_steps) of request r. out: [n_steps][k] int32.
 * Returns 0, or -1 if a range cannot supply the ids asked for.
 */
int ws_request_stream(const ws_spec* sp, uint64_t seed, int32_t r, int32_t n_steps, int32_t* out) {
  const int32_t k = sp->k;
  int32_t L_max = sp->L0 + (sp->grow ? n_steps : 0);
  uint8_t* mark = (uint8_t*)calloc((size_t)L_max, 1);
  int32_t* cur = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  int rc = 0;
  if (!mark || !cur || !tmp) { rc = -2; goto done; }
  for (int32_t t = 0; t < n_steps; ++t) {
    rng_t g = rng_for(seed, (uint32_t)r, (uint32_t)t);
    const int32_t L = sp->L0 + (sp->grow ? t : 0);
    int32_t cnt = 0;
    if (t == 0) {
      if (sp->grow) { cur[cnt++] = L - 1; mark[L - 1] = 1; }
      if (draw_distinct(&g, 0, L, k - cnt, cur, &cnt, mark)) { rc = -1; goto done; }
    } else {
      const int32_t keep = (int32_t)(((int64_t)sp->keep_permille * k) / 1000);
      memcpy(tmp, out + (size_t)(t - 1) * k, sizeof(int32_t) * (size_t)k);
      for (int32_t i = 0; i < keep; ++i) {
        int32_t j = i + (int32_t)rng_below(&g, (uint32_t)(k - i));
        int32_t v = tmp[i]; tmp[i] = tmp[j]; tmp[j] = v;
        cur[cnt++] = tmp[i];
        mark[tmp[i]] = 1;
      }
      if (sp->grow) { cur[cnt++] = L - 1; mark[L - 1] = 1; }
      const int32_t n_new = k - cnt;
      const int32_t nB = (int32_t)(((int64_t)sp->partB_permille * n_new) / 1000);
      const int32_t nA = n_new - nB;
      int32_t loA, hiA, loB, hiB;
      if (sp->tail > 0) { loA = 0; hiA = L - sp->tail; loB = L - sp->tail; hiB = L; }
      else { loA = 0; hiA = L; loB = L - sp->window < 0 ? 0 : L - sp->window; hiB = L; }
      if (draw_distinct(&g, loA, hiA, nA, cur, &cnt, mark)) { rc = -1; goto done; }
      if (draw_distinct(&g, loB, hiB, nB, cur, &cnt, mark)) { rc = -1; goto done; }
    }
    shuffle(&g, cur, k);
    for (int32_t i = 0; i < k; ++i) mark[cur[i]] = 0;
    memcpy(out + (size_t)t * k, cur, sizeof(int32_t) * (size_t)k);
  }
done:
  free(mark); free(cur); free(tmp);
  return rc;
}

/* All requests: out [n_req][n_steps][k]. Requests are independent, so they run in parallel. */
int ws_streams(const ws_spec* sp, uint64_t seed, int32_t n_req, int32_t n_steps, int32_t* out) {
  int rc = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
  for (int32_t r = 0; r < n_req; ++r)
    rc |= ws_request_stream(sp, seed, r, n_steps, out + (size_t)r * n_steps * sp->k) ? 1 : 0;
  return rc ? -1 : 0;
}

/* float32 -> bf16, round to nearest even (inputs are finite) */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/*
 * Fill rows [row0, row0 + n_rows) of a pool laid out as [rows][row_elems] bf16,
 * where the global row index g = row0 + i names the row. Each pair of elements
 * comes from one SplitMix64 output at counter g*row_elems/2 + q through the
 * Box-Muller transform (float32), then is rounded to bf16.
 */
int ws_fill_rows(uint16_t* dst, int64_t row0, int64_t n_rows, int32_t row_elems, uint64_t seed) {
  if (row_elems <= 0 || (row_elems & 1)) return -1;
  const int64_t pairs = row_elems / 2;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_rows; ++i) {
    uint16_t* row = dst + i * row_elems;
    const uint64_t base = (uint64_t)(row0 + i) * (uint64_t)pairs;
    for (int64_t q = 0; q < pairs; ++q) {
      uint64_t z = sm64_mix(seed + (base + (uint64_t)q + 1) * GOLDEN);
      float u1 = (float)((z >> 40) + 1) * (1.0f / 16777216.0f); /* (0, 1] */
      float u2 = (float)((z >> 16) & 0xFFFFFF) * (1.0f / 16777216.0f);
      float rad = sqrtf(-2.0f * logf(u1));
      float s, c;
      sincosf(6.2831853071795864f * u2, &s, &c);
      row[2 * q] = f32_to_bf16(rad * c);
      row[2 * q + 1] = f32_to_bf16(rad * s);
    }
  }
  return 0;
}
