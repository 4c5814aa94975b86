// kernels.hpp -- kernel argument blocks and launchers (implemented in kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace effort {

// Select: chart = fl32(|v_i| * probe_i[k]); cutoff = K-th largest chart value.
// Block b owns chart entries [b*SEL_VALS, (b+1)*SEL_VALS).
constexpr int SEL_VALS = 4096;   // chart values per select block
constexpr int SEL_BINS = 256;    // first digit: the fp32 exponent field
struct SelectArgs {
  const float* v;
  const uint16_t* probes;  // [m][P] fp16 magnitude bits
  int64_t m;
  int32_t P;
  int64_t N;         // m * P
  uint32_t K;
  uint32_t* done;    // last-block counter (zero on entry, left zero)
  uint32_t* boff;    // [blocks][SEL_BINS + 1] per-block exclusive bin offsets
  float* sorted;     // [blocks * SEL_VALS] chart slice of each block, ordered by bin
  uint32_t* result;  // [0] cutoff bits, [1] K', [2] K
  float* y;          // zeroed here (the multiply accumulates into it)
  int64_t n;
};

// Dispatch: per row threshold and per (group, row) read length, plus the sum
// of the read lengths of each block of DSP_ROWS rows per group.
constexpr int DSP_ROWS = 256;
struct DispatchArgs {
  const float* v;
  const uint16_t* probes;   // [m][P]
  const uint32_t* counts;   // [m][P][G]
  const uint16_t* rowmax;   // [m] largest magnitude key per row
  const uint32_t* result;   // cutoff bits
  uint32_t* thresh;         // [m]
  uint32_t* runlen;         // [G][m]
  uint32_t* bsum;           // [ceil(m / DSP_ROWS)][G + 1]
  int32_t* row_chart_kept;  // [m] or null
  int64_t m;
  int32_t P, G;
};

// bucketMul: stream each (row, group) run prefix, keep entries whose magnitude
// reaches the row threshold, scatter v_i * w into an LDS tile of the group's
// output columns, then add the tile to y.  The entries of a group, concatenated
// over rows, are split evenly over the group's waves.  The tile holds 64-bit
// fixed-point sums (integer LDS atomics); the scale comes from the bound
// sum_i |v_i| * rowmax_i >= |any partial sum|.
struct MulArgs {
  const float* v;
  const uint32_t* entries;  // [m][row_stride]
  const uint32_t* thresh;   // [m]
  const uint32_t* runlen;   // [G][m]
  const uint32_t* bsum;     // [nbd][G + 1]
  float* y;                 // [n]
  int64_t m, n, row_stride;
  int32_t G, TW, nbd;
  // parity recording (null in the timed path)
  int32_t* row_kept;
  unsigned long long* fingerprint;
  uint8_t* mask;
};

hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
hipError_t launch_bucketmul(const MulArgs& a, bool record, int blocks_per_group, hipStream_t s);
hipError_t launch_dense_gemv(const uint16_t* W, const float* v, int64_t m, int64_t n, float* y,
                             int lanes_per_row, int row_splits, hipStream_t s);
hipError_t launch_dense_gemm_small(const uint16_t* W, const float* v, int batch, int64_t m,
                                   int64_t n, float* y, hipStream_t s);
hipError_t launch_silu_mul(const float* h1, const float* h3, int64_t n, float* out, hipStream_t s);
hipError_t launch_zero_bytes(void* p, uint64_t bytes, hipStream_t s);
hipError_t launch_debug_result(const uint32_t* result, float* cutoff, int64_t* K, hipStream_t s);

}  // namespace effort
