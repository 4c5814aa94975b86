// kernels.hpp -- kernel argument blocks and launchers (implemented in kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace effort {

// Cutoff: chart = fl32(|v_i| * probe_i[k]); cutoff = K-th largest chart value.
struct SelectArgs {
  const float* v;
  const uint16_t* probes;  // [m][P] fp16 magnitude bits
  int64_t m;
  int32_t P;
  uint32_t K;
  uint32_t* done;    // last-block counter (zero on entry, left zero)
  uint32_t* hist;    // [2048] first-digit histogram (zero on entry, left zero)
  float* chart;      // [m*P] scratch
  uint32_t* result;  // [0] cutoff bits, [1] K', [2] K
  float* y;          // zeroed here (the multiply accumulates into it)
  int64_t n;
  int32_t rows_per_block;
};

// Dispatch: per row threshold and per (group, row) read length.
struct DispatchArgs {
  const float* v;
  const uint16_t* probes;   // [m][P]
  const uint32_t* counts;   // [m][P][G]
  const uint32_t* result;   // cutoff bits
  uint32_t* thresh;         // [m]
  uint32_t* runlen;         // [G][m]
  uint32_t* rowctr;         // [G] zeroed here
  int32_t* row_chart_kept;  // [m] or null
  int64_t m;
  int32_t P, G;
};

// bucketMul: stream each (row, group) run prefix, keep entries whose magnitude
// reaches the row threshold, scatter v_i * w into an LDS tile of the group's
// output columns, then add the tile to y.
struct MulArgs {
  const float* v;
  const uint32_t* entries;  // [m][row_stride]
  const uint32_t* thresh;   // [m]
  const uint32_t* runlen;   // [G][m]
  uint32_t* rowctr;         // [G]
  float* y;                 // [n]
  int64_t m, n, row_stride;
  int32_t G, TW;
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
