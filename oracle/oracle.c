/*
 * oracle.c -- TEST INFRASTRUCTURE: the reference rule of the "Effort"
 * approximate vector-matrix multiply, written out step by step.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this file's library.  It is independent of the GPU library: no shared code,
 * headers, tables or helpers.  Single-threaded, brute force, double-precision
 * sums; build with -O2 -ffp-contract=off and without fast-math so that every
 * fp32 product below is one IEEE round-to-nearest-even multiply and fp16
 * subnormals are kept.
 *
 * Sources (web pages; cited by title and passage):
 *  [HN] "Show HN: Speeding up LLM inference 2x times (possibly)", Hacker News
 *       thread (Gopher archive and the forum repost of the post text).
 *  [HT] hntin item 40095016, the author's reply on algorithmic complexity.
 *
 * Parity pins for every function are in tests/test_oracle_pins.py; each
 * function below is pinned there against brute force, closed forms, invariants
 * or a library routine.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
   exponent 0: subnormal f * 2^-24; exponent 31: inf/NaN; else (1024+f) * 2^(e-25). */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double mag;
  if (e == 0)
    mag = ldexp((double)f, -24);
  else if (e == 31)
    mag = f ? NAN : INFINITY;
  else
    mag = ldexp((double)(1024 + f), e - 25);
  return sign ? -mag : mag;
}

/* splitmix64 output function (Steele, Lea, Flood 2014) of state x. */
uint64_t oracle_pair_hash(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* |w| as fp32.  The magnitude of a binary16 value is its bit pattern with the
   sign cleared; the conversion to fp32 is exact. */
static float magnitude_f32(uint16_t h) { return (float)oracle_f16_to_f64((uint16_t)(h & 0x7FFF)); }

static int cmp_u16_desc(const void* a, const void* b) {
  uint16_t x = *(const uint16_t*)a, y = *(const uint16_t*)b;
  return (x < y) - (x > y);
}

static int cmp_f32_desc(const void* a, const void* b) {
  float x = *(const float*)a, y = *(const float*)b;
  return (x < y) - (x > y);
}

/* Step "get_probes" of the precompute in the [HN] pseudocode (gcy's quote).
   The pages give only the name; the reading used here: each stored row is
   sorted by |w| descending (the author's reply to bigcat12345678: all entries
   kept, ordered from the highest absolute value down) and cut into P rank
   segments (the reply to marmaduke: each row split into 16 parts).  probe k is
   the magnitude at rank ceil((k+1) n / P), i.e. the smallest magnitude of
   segment k.  For finite fp16 the unsigned order of (bits & 0x7FFF) is the
   order of magnitudes, so the sort is done on those keys. */
int oracle_probes(const uint16_t* W, int64_t m, int64_t n, int32_t P, float* probes) {
  if (!W || !probes || m <= 0 || n <= 0 || P < 1 || P > n) return 1;
  uint16_t* keys = (uint16_t*)malloc((size_t)n * sizeof(uint16_t));
  if (!keys) return 1;
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t j = 0; j < n; ++j) keys[j] = (uint16_t)(W[i * n + j] & 0x7FFF);
    qsort(keys, (size_t)n, sizeof(uint16_t), cmp_u16_desc);
    for (int32_t k = 0; k < P; ++k) {
      int64_t rank = ((int64_t)(k + 1) * n + P - 1) / P; /* ceil((k+1) n / P), 1-based */
      probes[i * P + k] = (float)oracle_f16_to_f64(keys[rank - 1]);
    }
  }
  free(keys);
  return 0;
}

/* "cutoff_chart = v * probes" in the [HN] pseudocode.  Ranking is by magnitude
   (the method keeps the largest |v_i * W_ij|), so the chart holds |v_i| times
   each probe, one fp32 multiply each. */
int oracle_chart(const float* v, const float* probes, int64_t m, int32_t P, float* chart) {
  if (!v || !probes || !chart || m <= 0 || P < 1) return 1;
  for (int64_t i = 0; i < m; ++i) {
    float av = fabsf(v[i]);
    for (int32_t k = 0; k < P; ++k) chart[i * P + k] = av * probes[i * P + k];
  }
  return 0;
}

/* The top-K step over the chart in the [HN] pseudocode: effort is the
   fraction of the chart that lies at or above the cutoff.  K rounds up so the
   kept fraction never falls below effort; the cutoff is the K-th largest chart
   value (a value, so ties need no rule).  A full descending sort stands in for
   a selection. */
int oracle_cutoff(const float* chart, int64_t N, float effort, int64_t* K, float* cutoff,
                  int64_t* Kprime) {
  if (!chart || N <= 0 || !(effort > 0.0f) || !(effort <= 1.0f)) return 1;
  double kd = ceil((double)effort * (double)N);
  int64_t k = (int64_t)kd;
  if (k < 1) k = 1;
  if (k > N) k = N;
  float* s = (float*)malloc((size_t)N * sizeof(float));
  if (!s) return 1;
  memcpy(s, chart, (size_t)N * sizeof(float));
  qsort(s, (size_t)N, sizeof(float), cmp_f32_desc);
  float c = s[k - 1];
  free(s);
  int64_t kp = 0;
  for (int64_t t = 0; t < N; ++t) kp += (chart[t] >= c);
  if (K) *K = k;
  if (cutoff) *cutoff = c;
  if (Kprime) *Kprime = kp;
  return 0;
}

/* bucketMul of the [HN] pseudocode, done without buckets: every product whose
   fp32 magnitude reaches the cutoff is kept (O(effort * inDim * outDim)
   multiplications in the real method, [HT]); each kept product is added into
   the output element its column names (the scatter step of the write-up that
   bigcat12345678 quotes in [HN]).  Here all m*n pairs are swept. */
int oracle_keep_sum(const uint16_t* W, int64_t m, int64_t n, const float* v, float cutoff,
                    double* y_double, int64_t* row_kept, uint64_t* fingerprint, uint8_t* mask,
                    int64_t* total_kept) {
  if (!W || !v || !y_double || m <= 0 || n <= 0) return 1;
  for (int64_t j = 0; j < n; ++j) y_double[j] = 0.0;
  uint64_t fp = 0;
  int64_t total = 0;
  for (int64_t i = 0; i < m; ++i) {
    float av = fabsf(v[i]);
    double vi = (double)v[i];
    int64_t cnt = 0;
    for (int64_t j = 0; j < n; ++j) {
      uint16_t h = W[i * n + j];
      float p = av * magnitude_f32(h);
      int keep = (p >= cutoff);
      if (mask) mask[i * n + j] = (uint8_t)keep;
      if (keep) {
        y_double[j] += vi * oracle_f16_to_f64(h);
        fp += oracle_pair_hash((uint64_t)(i * n + j));
        ++cnt;
      }
    }
    if (row_kept) row_kept[i] = cnt;
    total += cnt;
  }
  if (fingerprint) *fingerprint = fp;
  if (total_kept) *total_kept = total;
  return 0;
}

/* The stored part of a cropped layout (the [HN] post text: the data format
   lets one load only part of the model, leaving out a share of the
   smallest-magnitude weights; the author runs Mixtral from its top ~70 %).  Reading
   used here: rows are cut into the same P rank segments as the probes, and
   segments 0..crop-1 -- the ceil(crop n / P) largest magnitudes of the row,
   ties going to the lower column -- are stored.  stored[i*n+j] = 1 for those. */
typedef struct {
  uint16_t key;
  int64_t col;
} key_col;

static int cmp_key_desc_col_asc(const void* a, const void* b) {
  const key_col* x = (const key_col*)a;
  const key_col* y = (const key_col*)b;
  if (x->key != y->key) return (x->key < y->key) - (x->key > y->key);
  return (x->col > y->col) - (x->col < y->col);
}

int oracle_stored_mask(const uint16_t* W, int64_t m, int64_t n, int32_t P, int32_t crop,
                       uint8_t* stored) {
  if (!W || !stored || m <= 0 || n <= 0 || P < 1 || P > n || crop < 1 || crop > P) return 1;
  key_col* kc = (key_col*)malloc((size_t)n * sizeof(key_col));
  if (!kc) return 1;
  int64_t keep = ((int64_t)crop * n + P - 1) / P; /* ceil(crop n / P) */
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      kc[j].key = (uint16_t)(W[i * n + j] & 0x7FFF);
      kc[j].col = j;
      stored[i * n + j] = 0;
    }
    qsort(kc, (size_t)n, sizeof(key_col), cmp_key_desc_col_asc);
    for (int64_t r = 0; r < keep; ++r) stored[i * n + kc[r].col] = 1;
  }
  free(kc);
  return 0;
}

/* The rule on a cropped layout: probes, chart and cutoff of the whole matrix
   (the crop drops entries, not the statistics that place the cutoff); kept =
   the stored pairs whose product reaches the cutoff; *crop_reached = 1 when a
   pair that is not stored reaches it too (the uncropped rule would keep it). */
int oracle_run_cropped(const uint16_t* W, int64_t m, int64_t n, const float* probes, int32_t P,
                       int32_t crop, const float* v, float effort, float* cutoff, int64_t* K,
                       int64_t* Kprime, double* y_double, int64_t* row_kept, uint64_t* fingerprint,
                       uint8_t* mask, int64_t* total_kept, int32_t* crop_reached) {
  if (!W || !probes || !v || !y_double || m <= 0 || n <= 0 || P < 1 || P > n) return 1;
  int64_t N = m * P;
  float* chart = (float*)malloc((size_t)N * sizeof(float));
  uint8_t* stored = (uint8_t*)malloc((size_t)(m * n));
  if (!chart || !stored) {
    free(chart);
    free(stored);
    return 1;
  }
  float c = 0.0f;
  int rc = oracle_chart(v, probes, m, P, chart);
  if (!rc) rc = oracle_cutoff(chart, N, effort, K, &c, Kprime);
  if (!rc) rc = oracle_stored_mask(W, m, n, P, crop, stored);
  free(chart);
  if (rc) {
    free(stored);
    return rc;
  }
  for (int64_t j = 0; j < n; ++j) y_double[j] = 0.0;
  uint64_t fp = 0;
  int64_t total = 0;
  int32_t reached = 0;
  for (int64_t i = 0; i < m; ++i) {
    float av = fabsf(v[i]);
    double vi = (double)v[i];
    int64_t cnt = 0;
    for (int64_t j = 0; j < n; ++j) {
      uint16_t h = W[i * n + j];
      int keep = (av * magnitude_f32(h) >= c);
      if (keep && !stored[i * n + j]) reached = 1;
      keep = keep && stored[i * n + j];
      if (mask) mask[i * n + j] = (uint8_t)keep;
      if (keep) {
        y_double[j] += vi * oracle_f16_to_f64(h);
        fp += oracle_pair_hash((uint64_t)(i * n + j));
        ++cnt;
      }
    }
    if (row_kept) row_kept[i] = cnt;
    total += cnt;
  }
  free(stored);
  if (cutoff) *cutoff = c;
  if (fingerprint) *fingerprint = fp;
  if (total_kept) *total_kept = total;
  if (crop_reached) *crop_reached = reached;
  return 0;
}

/* The Q8 bucketed form (the [HN] post text: Q8 is in the works; the author's
   reply to kwikiel: in a bucketed Q8 entry 4 bits store the weight, 1 bit the
   sign and 3 bits the location, and the 4 bits only have to cover the range
   of the weight's bucket).  Reading used here: the buckets are the P rank
   segments of each row; bucket k covers magnitude keys from lo = probe k (its
   smallest) to hi = probe k-1 (for k = 0: the row's largest), and its 16
   levels are lo + c 2^s (c = 0..15, s the smallest shift with 15 2^s >= hi -
   lo) capped at hi, in the integer order of binary16 magnitude bits -- a
   quasi-logarithmic grid.  A weight takes the level nearest to its key (ties
   to the upper level) and keeps its sign.  wq[m][n] receives the quantized
   fp16 bits.  The levels include lo and stay within [lo, hi], so the
   quantized rows have the same probes as the original ones. */
static int cmp_u16_desc_col(const void* a, const void* b) { return cmp_key_desc_col_asc(a, b); }

int oracle_quantize_q8(const uint16_t* W, int64_t m, int64_t n, int32_t P, uint16_t* wq) {
  if (!W || !wq || m <= 0 || n <= 0 || P < 1 || P > n) return 1;
  key_col* kc = (key_col*)malloc((size_t)n * sizeof(key_col));
  if (!kc) return 1;
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      kc[j].key = (uint16_t)(W[i * n + j] & 0x7FFF);
      kc[j].col = j;
    }
    qsort(kc, (size_t)n, sizeof(key_col), cmp_u16_desc_col);
    int64_t start = 0; /* first rank (0-based) of bucket k */
    for (int32_t k = 0; k < P; ++k) {
      int64_t end = ((int64_t)(k + 1) * n + P - 1) / P; /* one past its last rank */
      uint32_t lo = kc[end - 1].key;
      uint32_t hi = k == 0 ? kc[0].key : kc[start - 1].key;
      uint32_t d = hi - lo, sh = 0;
      while (15u * (1u << sh) < d) ++sh;
      for (int64_t r = start; r < end; ++r) {
        /* the two levels around the key (the top one capped at hi), the
           nearer taken, ties to the upper */
        uint32_t x = kc[r].key;
        uint32_t c = (x - lo) >> sh;
        if (c > 15u) c = 15u;
        uint32_t below = lo + (c << sh);
        if (below > hi) below = hi;
        uint32_t q = below;
        if (c < 15u) {
          uint32_t above = lo + ((c + 1u) << sh);
          if (above > hi) above = hi;
          if (above - x <= x - below) q = above;
        }
        int64_t j = kc[r].col;
        wq[i * n + j] = (uint16_t)((W[i * n + j] & 0x8000) | q);
      }
      start = end;
    }
  }
  free(kc);
  return 0;
}

int oracle_run(const uint16_t* W, int64_t m, int64_t n, const float* probes, int32_t P,
               const float* v, float effort, float* cutoff, int64_t* K, int64_t* Kprime,
               double* y_double, int64_t* row_kept, int64_t* row_chart_kept,
               uint64_t* fingerprint, uint8_t* mask, int64_t* total_kept) {
  if (!W || !probes || !v || !y_double || m <= 0 || n <= 0 || P < 1 || P > n) return 1;
  int64_t N = m * P;
  float* chart = (float*)malloc((size_t)N * sizeof(float));
  if (!chart) return 1;
  int rc = oracle_chart(v, probes, m, P, chart);
  float c = 0.0f;
  if (!rc) rc = oracle_cutoff(chart, N, effort, K, &c, Kprime);
  if (!rc && row_chart_kept) {
    for (int64_t i = 0; i < m; ++i) {
      int64_t cnt = 0;
      for (int32_t k = 0; k < P; ++k) cnt += (chart[i * P + k] >= c);
      row_chart_kept[i] = cnt;
    }
  }
  free(chart);
  if (rc) return rc;
  if (cutoff) *cutoff = c;
  return oracle_keep_sum(W, m, n, v, c, y_double, row_kept, fingerprint, mask, total_kept);
}

int oracle_dense(const uint16_t* W, int64_t m, int64_t n, const float* v, double* y_double) {
  if (!W || !v || !y_double || m <= 0 || n <= 0) return 1;
  for (int64_t j = 0; j < n; ++j) y_double[j] = 0.0;
  for (int64_t i = 0; i < m; ++i) {
    double vi = (double)v[i];
    for (int64_t j = 0; j < n; ++j) y_double[j] += vi * oracle_f16_to_f64(W[i * n + j]);
  }
  return 0;
}
