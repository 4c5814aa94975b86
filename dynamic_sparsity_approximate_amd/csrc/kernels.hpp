// kernels.hpp -- kernel argument blocks and launchers (implemented in kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "effort.h"

namespace effort {

// Cutoff, first pass: chart = fl32(|v_i| * probe_i[k]); a histogram of the
// top 12 bits (exponent + 4 fraction bits) of the chart values, accumulated in
// a global 4096-bin array; one thread per row.
constexpr int HIST_BINS = 4096;
constexpr int HIST_SHIFT = 19;
struct SelectArgs {
  const float* v;
  const uint16_t* probes;  // [m][P] fp16 magnitude bits
  int64_t m;
  int32_t P;
  int64_t N;         // m * P
  uint32_t* hist;    // [HIST_BINS], zero on entry (the multiply clears it)
  uint32_t* hist2;   // [1024] cleared here for the dispatch
  uint32_t* result;  // candidate count and flags, cleared here
  float* y;          // zeroed here (the multiply accumulates into it)
  int64_t n;
  uint32_t* bsum;        // [bsum_words] zeroed here (the dispatch may accumulate into it)
  int64_t bsum_words;
  // several vectors in one launch (grid y): vector k reads v + k m, writes
  // y + k n and uses the workspace words hist/hist2/result + k vec_ws
  uint64_t vec_ws;
};

// result words of the workspace
constexpr int RES_CUTOFF = 0, RES_KPRIME = 1, RES_K = 2, RES_NCAND = 3, RES_BIN = 4, RES_ABOVE = 5,
              RES_FLAGS = 6;
// RES_FLAGS bit 0: a cropped layout left out an entry the keep rule keeps
constexpr uint32_t FLAG_CROP_REACHED = 1u;

// The lane-per-segment-quad dispatch (P = 16 or 32, at most 8 column groups)
// gives a row P / 4 lanes and takes quad_rows(P) rows per block: 64 for
// P = 16, 32 for P = 32.  When its blocks number at most 64 (in_dim <= 4096
// for P = 16, 2048 for P = 32), block r keeps the chart values in the
// cutoff's bin in a region of RCAP = quad_rows(P) * P candidate slots of its
// own, from slot r * RCAP, and their count in result word RES_RCOUNT + r: no
// slot reservation.  Otherwise the candidates form one list of
// result[RES_NCAND] values.
constexpr int QUAD_ROWS = 64;  // rows per block at P = 16
constexpr int RCAP = QUAD_ROWS * 16;
constexpr int RES_RCOUNT = 64;  // 64 region counts after the 64 result words
__host__ __device__ inline bool quad_dispatch_ok(int32_t P, int32_t G) {
  return (P == 16 || P == 32) && G >= 1 && G <= 8;
}
__host__ __device__ inline int32_t quad_rows(int32_t P) { return P == 32 ? QUAD_ROWS / 2 : QUAD_ROWS; }
__host__ __device__ inline bool cand_regions(int32_t P, int32_t G, int64_t m) {
  return quad_dispatch_ok(P, G) && m <= 64 * (int64_t)quad_rows(P);
}
// words of the candidate list: in_dim rounded up to QUAD_ROWS, times P (this
// also covers P = 32's regions: ceil(m / 32) * RCAP <= ceil(m / 64) * 64 * 32)
__host__ __device__ inline uint64_t cand_capacity(int64_t m, int32_t P) {
  return (uint64_t)((m + QUAD_ROWS - 1) / QUAD_ROWS * QUAD_ROWS) * (uint64_t)P;
}

// Dispatch: per (group, row) read length from a lower bound of the cutoff (the
// low edge of the histogram bin b1 that holds the K-th largest chart value),
// per block of DSP_ROWS rows the sum of the read lengths of each group and the
// bound sum |v_i| * rowmax_i; the chart values that fall in bin b1 go to a
// candidate list and a 1024-bin histogram of their next 10 bits.
constexpr int DSP_ROWS = 256;
constexpr int DSP_T = 256;
struct DispatchArgs {
  const float* v;
  const uint16_t* probes;   // [m][P]
  const uint32_t* counts;   // [m][P][G4]
  const uint16_t* rowmax;   // [m] largest magnitude key per row
  const uint32_t* hist;     // [HIST_BINS]
  uint32_t* hist2;          // [1024], zero on entry
  uint32_t* cand;           // [m * P] candidate chart values (bit patterns)
  uint32_t* result;         // RES_NCAND (zero on entry), RES_BIN, RES_ABOVE written here
  uint32_t* runlen;         // [G][m]
  uint32_t* bsum;           // [ceil(m / DSP_ROWS)][G + 1]
  int64_t m;
  int32_t P, G, G4;
  uint32_t K;
  uint64_t vec_ws;  // grid y = vector: its v + k m and workspace words + k vec_ws
};

// Union of several vectors' read lengths (batched multiply): per (group, row)
// the largest read length over the vectors, and its per-256-row sums.
struct UnionArgs {
  const uint32_t* runlen;  // vector 0's [G][m]; vector k at + k vec_ws
  uint64_t vec_ws;
  int32_t nv, G;
  int64_t m;
  uint32_t* urunlen;  // [G][m]
  uint32_t* ubsum;    // [ceil(m / DSP_ROWS)][G + 1] (the last column unused)
};

// bucketMul: every block first finishes the exact cutoff (histograms + the
// candidate list), then streams each (row, group) run prefix, keeps entries
// whose magnitude reaches the row threshold, scatters v_i * w into an LDS tile
// of the group's output columns and adds the tile to y.  The entries of a
// group, concatenated over rows, are split evenly over the group's waves.  The
// tile holds 32-bit fixed-point sums (integer LDS atomics); the scale comes from
// the bound sum_i |v_i| * rowmax_i >= |any partial sum|.
//
// Batched (nv > 1 vectors of one pass): runlen/bsum are the union read lengths;
// vector k's v, y, cutoff inputs, bound column and histogram to clear are at
// v + k m, y + k n and the workspace words + k vec_ws; one tile per vector.
struct MulArgs {
  const float* v;
  const uint32_t* entries;  // units [m][G][gstride] (u32 format: one word per unit)
  int64_t gstride;          // units per (row, group) run
  int32_t format;           // EFFORT_ENTRY_* (all pairs of a multi launch alike)
  const uint16_t* floor;    // cropped layouts: [m] largest magnitude key not stored (else null)
  const uint16_t* probes;   // [m][P] probe keys, rowmax [m]: the q8 format's bucket bounds
  const uint16_t* rowmax;
  int32_t regions;          // the dispatch put the candidates in per-block regions (quad
                            // dispatch with cand_regions), else in one list
  const uint32_t* runlen;   // [G][m]
  const uint32_t* bsum;     // [nbd][G + 1]
  uint32_t* hist;           // [HIST_BINS], cleared here for the next call
  const uint32_t* hist2;    // [1024]
  const uint32_t* cand;     // candidate chart values
  uint32_t* result;         // reads RES_NCAND, RES_BIN, RES_ABOVE; writes the cutoff, K', K
  float* y;                 // [n]
  int64_t m, n, row_stride;
  int32_t G, TW, nbd, P;
  uint32_t K;
  int32_t nv;              // vectors of this pass (1: the single-vector path)
  uint32_t bpg_recip;       // floor(2^32 / blocks per group), set by launch_bucketmul
  uint64_t vec_ws;
  const uint32_t* vbsum;    // vector 0's own per-256-row sums: column G is its bound
                            // (bsum, the partition's sums, is the union when batched)
  // parity recording (null in the timed path); a batched pass records
  // vector p of the pass at row_kept + p m, fingerprint + p, mask + p m n
  int32_t* row_kept;
  unsigned long long* fingerprint;
  uint8_t* mask;
};

// Optional timing: when `start` is set, the kernel is launched with
// hipExtLaunchKernelGGL and the runtime stamps `start`/`stop` with the kernel's
// own begin and end.
struct EventPair {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_select(const SelectArgs& a, hipStream_t s, const EventPair* ev = nullptr,
                         int nvec = 1);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s, const EventPair* ev = nullptr,
                           int nvec = 1);
hipError_t launch_union(const UnionArgs& a, hipStream_t s);
// vectors per pass of the batched multiply that the LDS holds for groups of
// TW columns (0: none, use single-vector calls)
int bucketmul_pass_width(int32_t TW, int32_t batch, int32_t format);
// Several matrices that share the input vector (one vector each): argument
// tables indexed by grid y (chart, dispatch) or by block range (multiply).
struct SelectMulti {
  SelectArgs a[EFFORT_MAX_MULTI];
};
struct DispatchMulti {
  DispatchArgs a[EFFORT_MAX_MULTI];
};
struct MulMulti {
  MulArgs a[EFFORT_MAX_MULTI];
  uint32_t first[EFFORT_MAX_MULTI + 1];  // matrix j owns blocks [first[j], first[j + 1])
  int32_t count;
};
hipError_t launch_select_multi(const SelectMulti& mm, int count, hipStream_t s);
hipError_t launch_dispatch_multi(const DispatchMulti& mm, int count, hipStream_t s);
// whether launch_dispatch_multi runs the quad-lane dispatch for these pairs
// (all of them qualify); otherwise every pair gets the row-per-thread one
bool dispatch_multi_quad(const DispatchMulti& mm, int count);
// blocks_per_group[j]: matrix j's blocks per column group (its grid is G_j times that)
hipError_t launch_bucketmul_multi(const MulMulti& mm, int count, const int* blocks_per_group,
                                  bool record, hipStream_t s);
hipError_t launch_bucketmul(const MulArgs& a, bool record, int blocks_per_group, hipStream_t s,
                            const EventPair* ev = nullptr);
hipError_t launch_dense_gemv(const uint16_t* W, const float* v, int64_t m, int64_t n, float* y,
                             int lanes_per_row, int row_splits, hipStream_t s);
// Dense GEMV over 128-column strips with split rows (y zero-filled, then one
// atomic per column and split); serves out_dim a multiple of 8 with W 16-byte
// aligned (dense_split_serves).
bool dense_split_serves(int64_t n, const uint16_t* W);
hipError_t launch_dense_split(const uint16_t* W, const float* v, int64_t m, int64_t n, float* y,
                              hipStream_t s);
hipError_t launch_dense_gemm_small(const uint16_t* W, const float* v, int batch, int64_t m,
                                   int64_t n, float* y, hipStream_t s);
hipError_t launch_silu_mul(const float* h1, const float* h3, int64_t n, float* out, hipStream_t s);
hipError_t launch_axpby(const float* a, float ga, const float* b, float gb, int64_t n, float* out,
                        hipStream_t s);
hipError_t launch_zero_bytes(void* p, uint64_t bytes, hipStream_t s);
// count vectors' cutoffs and (K, K') from their result words, vector k's at
// result + k * stride (u32 words)
hipError_t launch_debug_result(const uint32_t* result, uint64_t stride, int count, float* cutoff,
                               int64_t* K, uint32_t* status, hipStream_t s);
// *status |= 1 when any of v[0..m) is a NaN or an infinity (status cleared by the caller).
hipError_t launch_check_finite(const float* v, int64_t m, uint32_t* status, hipStream_t s);

// The device workspace of effort_matvec_noalloc on the current device (its
// address, set up on the first call: the symbol's address and a zero fill on
// `s`).  kNoallocScratchBytes bytes; calls on one device share it.
constexpr uint64_t kNoallocScratchBytes = EFFORT_NOALLOC_WORKSPACE_BYTES;
hipError_t noalloc_workspace(hipStream_t s, uint8_t** ws);

}  // namespace effort
