/*
 * oracle.h -- reference implementation of the "Effort" approximate
 * vector-matrix multiply, used ONLY as test infrastructure.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  It shares no code, header, table or helper with the GPU
 * library; it is plain, single-threaded, slow and written to be checked by eye.
 *
 * What it computes (the method's defining rule, each step done by brute force):
 *   W   fp16 [m][n] row-major; row i multiplies v_i ("W = W.T": the stored
 *       matrix is the transposed weight, one row per input element).
 *   probes   per row, P order statistics of |W_i,:| at ranks ceil((k+1) n / P),
 *            k = 0..P-1 (each rank-segment's smallest magnitude).
 *   chart    c[i*P+k] = fl32(|v_i| * probe_i[k]).
 *   K        min(N, max(1, ceil(effort * N))), N = m*P, evaluated in double.
 *   cutoff   the K-th largest chart value.
 *   kept     {(i,j) : fl32(|v_i| * |W_ij|) >= cutoff}.
 *   y_j      sum over kept (i,j) of v_i * W_ij, in double, i ascending.
 *
 * Status codes: 0 ok, 1 invalid argument.
 */
#ifndef EFFORT_ORACLE_H
#define EFFORT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* exact value of an IEEE-754 binary16 bit pattern */
double oracle_f16_to_f64(uint16_t h);

/* splitmix64 output function of x: the per-(i,j) hash of the kept-set fingerprint */
uint64_t oracle_pair_hash(uint64_t x);

/* probes[m][P] (fp32 magnitudes), 1 <= P <= n */
int oracle_probes(const uint16_t* W, int64_t m, int64_t n, int32_t P, float* probes);

/* chart[m][P] = fl32(|v_i| * probe_i[k]) */
int oracle_chart(const float* v, const float* probes, int64_t m, int32_t P, float* chart);

/* K, cutoff = K-th largest of chart[0..N-1], Kprime = #{chart >= cutoff} */
int oracle_cutoff(const float* chart, int64_t N, float effort, int64_t* K, float* cutoff,
                  int64_t* Kprime);

/* Brute-force kept set and sums.  Outputs other than y_double may be NULL.
   row_kept[m]: kept count per row; mask[m][n]: 1 where kept;
   fingerprint: sum of oracle_pair_hash(i*n+j) over kept pairs, mod 2^64. */
int oracle_keep_sum(const uint16_t* W, int64_t m, int64_t n, const float* v, float cutoff,
                    double* y_double, int64_t* row_kept, uint64_t* fingerprint, uint8_t* mask,
                    int64_t* total_kept);

/* Whole rule for one vector.  probes must come from oracle_probes(W, m, n, P).
   row_chart_kept[m] (nullable): #{k : chart[i][k] >= cutoff}. */
int oracle_run(const uint16_t* W, int64_t m, int64_t n, const float* probes, int32_t P,
               const float* v, float effort, float* cutoff, int64_t* K, int64_t* Kprime,
               double* y_double, int64_t* row_kept, int64_t* row_chart_kept,
               uint64_t* fingerprint, uint8_t* mask, int64_t* total_kept);

/* Cropped layouts: stored[m][n] = 1 for the ceil(crop n / P) largest
   magnitudes of each row (ties: lower column first), 1 <= crop <= P. */
int oracle_stored_mask(const uint16_t* W, int64_t m, int64_t n, int32_t P, int32_t crop,
                       uint8_t* stored);

/* The rule with only the stored pairs of a cropped layout kept: cutoff from
   the whole matrix's probes; kept = stored pairs reaching it; *crop_reached =
   1 when an unstored pair reaches it.  Outputs as oracle_run. */
int oracle_run_cropped(const uint16_t* W, int64_t m, int64_t n, const float* probes, int32_t P,
                       int32_t crop, const float* v, float effort, float* cutoff, int64_t* K,
                       int64_t* Kprime, double* y_double, int64_t* row_kept, uint64_t* fingerprint,
                       uint8_t* mask, int64_t* total_kept, int32_t* crop_reached);

/* Q8 bucketed form: wq[m][n] = W with each magnitude moved to the nearest of
   its rank bucket's 16 levels (see oracle.c); the rule then runs on wq. */
int oracle_quantize_q8(const uint16_t* W, int64_t m, int64_t n, int32_t P, uint16_t* wq);

/* plain dense y_j = sum_i v_i W_ij in double, i ascending */
int oracle_dense(const uint16_t* W, int64_t m, int64_t n, const float* v, double* y_double);

#ifdef __cplusplus
}
#endif
#endif
