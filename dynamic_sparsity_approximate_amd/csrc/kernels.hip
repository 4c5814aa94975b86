// kernels.hip -- gfx950 kernels of the Effort approximate vector-matrix multiply.
//
// Method: HN thread "Show HN: Speeding up LLM inference 2x times (possibly)"
// (pseudocode precompute/approxMul quoted by gcy; sorted (index, value) rows in
// the reply to bigcat12345678; 16-part row split of bucketMul in the reply to
// marmaduke) and hntin item 40095016 (cutoff O(inDim log inDim), dispatch
// O(inDim), multiply O(effort inDim outDim)).
//
// Three kernels per call, all on one stream:
//   k_select    chart |v_i| * probe_i[k] -> radix select of the K-th largest
//               (11/10/10-bit digits of the fp32 bit pattern; the last block to
//               finish the first digit finishes the selection) and zeroing of y.
//   k_dispatch  per row the smallest fp16 magnitude key that passes the keep
//               test, and per (group, row) how many rank-ordered entries to read.
//   k_bucketmul per output-column group an LDS tile of y; waves take rows from a
//               per-group counter, stream the run prefix with 16-byte loads, keep
//               entries whose key reaches the threshold, ds_add_f32 v_i * w into
//               the tile, and finally add the tile to y.
// No MFMA: the multiply is a bandwidth-bound gather-scatter, not a contraction.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace effort {

__device__ __forceinline__ float h2f(uint32_t bits) {
  return __half2float(__ushort_as_half((unsigned short)(bits & 0xFFFFu)));
}

// splitmix64 output function: per-(i, j) hash of the kept-set fingerprint.
__device__ __forceinline__ uint64_t pair_hash(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Exclusive scan over the block (NT threads); tmp holds NT/64 + 1 words.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t x, uint32_t* tmp, uint32_t* total) {
  constexpr int NWAVE = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(x);
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    const uint32_t w = lane < NWAVE ? tmp[lane] : 0u;
    const uint32_t wi = wave_incl_scan(w);
    if (lane < NWAVE) tmp[lane] = wi - w;
    if (lane == NWAVE - 1) tmp[NWAVE] = wi;
  }
  __syncthreads();
  const uint32_t r = inc - x + tmp[wid];
  *total = tmp[NWAVE];
  __syncthreads();
  return r;
}

// h[0..nb) in LDS.  Finds the bin b with above(b) < K <= above(b) + h[b], where
// above(b) counts the entries of all higher bins; writes out[0] = b,
// out[1] = above(b).  Requires 1 <= K <= sum(h).
template <int NT>
__device__ void find_from_top(const uint32_t* h, int nb, uint32_t K, uint32_t* tmp, uint32_t* out) {
  const int per = (nb + NT - 1) / NT;
  if (threadIdx.x == 0) {
    out[0] = 0u;
    out[1] = 0u;
  }
  uint32_t s = 0;
  for (int u = 0; u < per; ++u) {
    const int b = nb - 1 - ((int)threadIdx.x * per + u);
    if (b >= 0) s += h[b];
  }
  uint32_t tot;
  uint32_t above = block_excl_scan<NT>(s, tmp, &tot);
  for (int u = 0; u < per; ++u) {
    const int b = nb - 1 - ((int)threadIdx.x * per + u);
    if (b < 0) break;
    const uint32_t c = h[b];
    if (above < K && K <= above + c) {
      out[0] = (uint32_t)b;
      out[1] = above;
    }
    above += c;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- cutoff

constexpr int SEL_T = 1024;
constexpr uint32_t CAND_CAP = 12288;

__global__ __launch_bounds__(SEL_T) void k_select(SelectArgs a) {
  __shared__ uint32_t h[2048];
  __shared__ uint32_t tmp[SEL_T / 64 + 1];
  __shared__ uint32_t sres[8];
  __shared__ uint32_t cand[CAND_CAP];
  const int tid = threadIdx.x;

  for (int64_t j = (int64_t)blockIdx.x * SEL_T + tid; j < a.n; j += (int64_t)gridDim.x * SEL_T)
    a.y[j] = 0.0f;
  for (int b = tid; b < 2048; b += SEL_T) h[b] = 0u;
  __syncthreads();

  // first digit (bits 30..20; bit 31 is the sign, always 0 here) of this block's chart slice
  const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_block;
  const int64_t r1 = r0 + a.rows_per_block < a.m ? r0 + a.rows_per_block : a.m;
  for (int64_t e = r0 * a.P + tid; e < r1 * a.P; e += SEL_T) {
    const int64_t i = e / a.P;
    const float c = __fmul_rn(fabsf(a.v[i]), h2f(a.probes[e]));
    a.chart[e] = c;
    atomicAdd(&h[__float_as_uint(c) >> 20], 1u);
  }
  __syncthreads();
  for (int b = tid; b < 2048; b += SEL_T)
    if (h[b]) atomicAdd(&a.hist[b], h[b]);
  __threadfence();
  __syncthreads();
  if (tid == 0) sres[7] = (atomicAdd(a.done, 1u) == gridDim.x - 1) ? 1u : 0u;
  __syncthreads();
  if (sres[7] == 0u) return;
  __threadfence();

  // ---- last block: finish the selection over all m*P chart values
  for (int b = tid; b < 2048; b += SEL_T)
    h[b] = __hip_atomic_load(&a.hist[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  find_from_top<SEL_T>(h, 2048, a.K, tmp, sres);
  const uint32_t b1 = sres[0] & 2047u, above1 = sres[1];
  const uint32_t K1 = a.K - above1;
  const uint32_t n1 = h[b1];
  __syncthreads();

  for (int b = tid; b < 1024; b += SEL_T) h[b] = 0u;
  if (tid == 0) sres[6] = 0u;
  __syncthreads();
  const int64_t N = a.m * (int64_t)a.P;
  const bool use_cand = n1 <= CAND_CAP;
  for (int64_t e = tid; e < N; e += SEL_T) {
    const uint32_t bits = __float_as_uint(a.chart[e]);
    if ((bits >> 20) == b1) {
      atomicAdd(&h[(bits >> 10) & 1023u], 1u);
      if (use_cand) {
        const uint32_t pos = atomicAdd(&sres[6], 1u);
        if (pos < CAND_CAP) cand[pos] = bits;
      }
    }
  }
  __syncthreads();
  find_from_top<SEL_T>(h, 1024, K1, tmp, sres);
  const uint32_t b2 = sres[0] & 1023u, above2 = sres[1];
  const uint32_t K2 = K1 - above2;
  __syncthreads();

  for (int b = tid; b < 1024; b += SEL_T) h[b] = 0u;
  __syncthreads();
  const uint32_t pre = (b1 << 10) | b2;
  if (use_cand) {
    for (uint32_t e = tid; e < n1 && e < CAND_CAP; e += SEL_T) {
      const uint32_t bits = cand[e];
      if ((bits >> 10) == pre) atomicAdd(&h[bits & 1023u], 1u);
    }
  } else {
    for (int64_t e = tid; e < N; e += SEL_T) {
      const uint32_t bits = __float_as_uint(a.chart[e]);
      if ((bits >> 10) == pre) atomicAdd(&h[bits & 1023u], 1u);
    }
  }
  __syncthreads();
  find_from_top<SEL_T>(h, 1024, K2, tmp, sres);
  const uint32_t b3 = sres[0] & 1023u, above3 = sres[1];
  if (tid == 0) {
    a.result[0] = (pre << 10) | b3;
    a.result[1] = above1 + above2 + above3 + h[b3];
    a.result[2] = a.K;
    *a.done = 0u;
  }
  for (int b = tid; b < 2048; b += SEL_T) a.hist[b] = 0u;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int64_t blocks = (a.m + a.rows_per_block - 1) / a.rows_per_block;
  hipLaunchKernelGGL(k_select, dim3((unsigned)blocks), dim3(SEL_T), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dispatch

constexpr int DSP_T = 256;

__global__ __launch_bounds__(DSP_T) void k_dispatch(DispatchArgs a) {
  if (blockIdx.x == 0)
    for (int g = threadIdx.x; g < a.G; g += DSP_T) a.rowctr[g] = 0u;
  const int64_t i = (int64_t)blockIdx.x * DSP_T + threadIdx.x;
  if (i >= a.m) return;
  const float c = __uint_as_float(a.result[0]);
  const float av = fabsf(a.v[i]);
  // smallest finite fp16 magnitude key whose product with |v_i| reaches the
  // cutoff (0x7C00 = none); the product is monotone in the key
  uint32_t lo = 0u, hi = 0x7C00u;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (__fmul_rn(av, h2f(mid)) >= c)
      hi = mid;
    else
      lo = mid + 1u;
  }
  const uint32_t t = lo;
  // q = number of probes (descending keys) at or above the threshold = number of
  // fully kept segments; segment q (if any) is the one that is partly kept
  const uint16_t* pr = a.probes + i * a.P;
  int32_t qlo = 0, qhi = a.P;
  while (qlo < qhi) {
    const int32_t mid = (qlo + qhi) >> 1;
    if ((uint32_t)pr[mid] >= t)
      qlo = mid + 1;
    else
      qhi = mid;
  }
  const int32_t q = qlo;
  const int32_t qc = q < a.P ? q : a.P - 1;
  const uint32_t* cr = a.counts + ((size_t)i * a.P + qc) * a.G;
  for (int g = 0; g < a.G; ++g) a.runlen[(size_t)g * a.m + i] = cr[g];
  a.thresh[i] = t;
  if (a.row_chart_kept) a.row_chart_kept[i] = q;
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const int64_t blocks = (a.m + DSP_T - 1) / DSP_T;
  hipLaunchKernelGGL(k_dispatch, dim3((unsigned)blocks), dim3(DSP_T), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bucketMul

constexpr int MUL_T = 512;

template <bool REC>
__global__ __launch_bounds__(MUL_T) void k_bucketmul(
    const float* __restrict__ vvec, const uint32_t* __restrict__ entries,
    const uint32_t* __restrict__ thresh, const uint32_t* __restrict__ runlen,
    uint32_t* __restrict__ rowctr, float* __restrict__ y, MulArgs a) {
  extern __shared__ float tile[];
  const int g = (int)(blockIdx.x % (unsigned)a.G);
  const int64_t col0 = (int64_t)g * a.TW;
  const int tw = (int)((int64_t)a.TW < a.n - col0 ? (int64_t)a.TW : a.n - col0);
  for (int c = threadIdx.x; c < tw; c += MUL_T) tile[c] = 0.0f;
  __syncthreads();

  const int lane = threadIdx.x & 63;
  uint32_t* ctr = rowctr + g;
  const uint32_t* rl = runlen + (size_t)g * a.m;
  const uint32_t m = (uint32_t)a.m;
  uint32_t row = 0u;
  if (lane == 0) row = atomicAdd(ctr, 1u);
  row = __builtin_amdgcn_readfirstlane(row);
  while (row < m) {
    uint32_t nxt = 0u;
    if (lane == 0) nxt = atomicAdd(ctr, 1u);  // next row, fetched while this one streams
    const uint32_t L = min(rl[row], (uint32_t)tw);  // never past the group's slot
    const uint32_t t = thresh[row];
    const float vi = vvec[row];
    const uint4* base =
        reinterpret_cast<const uint4*>(entries + (size_t)row * (size_t)a.row_stride + col0);
    uint32_t cnt = 0u;
    uint64_t fp = 0u;
    for (uint32_t off = (uint32_t)lane * 4u; off < L; off += 1024u) {
      uint4 e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t o = off + (uint32_t)u * 256u;
        e[u] = o < L ? base[o >> 2] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t o = off + (uint32_t)u * 256u;
        const uint32_t ev[4] = {e[u].x, e[u].y, e[u].z, e[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t w = ev[k];
          if (o + (uint32_t)k < L && (w & 0x7FFFu) >= t) {
            atomicAdd(&tile[w >> 16], vi * h2f(w));
            if (REC) {
              const uint64_t col = (uint64_t)col0 + (w >> 16);
              const uint64_t flat = (uint64_t)row * (uint64_t)a.n + col;
              if (a.mask) a.mask[flat] = 1u;
              fp += pair_hash(flat);
              ++cnt;
            }
          }
        }
      }
    }
    if (REC) {
      uint32_t flo = (uint32_t)fp, fhi = (uint32_t)(fp >> 32);
      for (int off = 32; off > 0; off >>= 1) {
        cnt += __shfl_xor(cnt, off, 64);
        const uint32_t olo = __shfl_xor(flo, off, 64);
        const uint32_t ohi = __shfl_xor(fhi, off, 64);
        const uint64_t s = ((uint64_t)fhi << 32 | flo) + ((uint64_t)ohi << 32 | olo);
        flo = (uint32_t)s;
        fhi = (uint32_t)(s >> 32);
      }
      if (lane == 0) {
        if (cnt && a.row_kept) atomicAdd(&a.row_kept[row], (int32_t)cnt);
        if (a.fingerprint) atomicAdd(a.fingerprint, ((unsigned long long)fhi << 32) | flo);
      }
    }
    row = __builtin_amdgcn_readlane(nxt, 0);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < tw; c += MUL_T) {
    const float s = tile[c];
    if (s != 0.0f) atomicAdd(&y[col0 + c], s);
  }
}

hipError_t launch_bucketmul(const MulArgs& a, bool record, int blocks_per_group, hipStream_t s) {
  const unsigned grid = (unsigned)(a.G * blocks_per_group);
  const size_t lds = (size_t)a.TW * sizeof(float);
  if (record)
    hipLaunchKernelGGL(k_bucketmul<true>, dim3(grid), dim3(MUL_T), lds, s, a.v, a.entries,
                       a.thresh, a.runlen, a.rowctr, a.y, a);
  else
    hipLaunchKernelGGL(k_bucketmul<false>, dim3(grid), dim3(MUL_T), lds, s, a.v, a.entries,
                       a.thresh, a.runlen, a.rowctr, a.y, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dense comparator

constexpr int DN_T = 512;

// Block (x, y) owns columns [x*8*LPR, (x+1)*8*LPR) and rows [y*rps, (y+1)*rps).
// LPR lanes cover one row of the strip with 16-byte loads (8 fp16 each); a wave
// covers 64/LPR rows per load; partial sums are reduced with shuffles and LDS.
template <int LPR, int B>
__global__ __launch_bounds__(DN_T) void k_dense(const uint16_t* __restrict__ W,
                                                const float* __restrict__ v, int64_t m, int64_t n,
                                                float* __restrict__ y, int64_t rps, int atomic_out,
                                                int aligned) {
  constexpr int RPW = 64 / LPR;
  constexpr int NW = DN_T / 64;
  constexpr int CPB = 8 * LPR;
  constexpr int STEP = NW * RPW;
  constexpr int UNR = 4;
  __shared__ float red[NW][B][CPB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cl = lane % LPR, rs = lane / LPR;
  const int64_t col = (int64_t)blockIdx.x * CPB + cl * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rps;
  const int64_t r1 = r0 + rps < m ? r0 + rps : m;
  const bool vec = (col + 8 <= n) && aligned;
  float acc[B][8];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[b][k] = 0.0f;

  for (int64_t rb = r0 + wave * RPW + rs; rb < r1; rb += (int64_t)STEP * UNR) {
    uint4 q[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t r = rb + (int64_t)u * STEP;
      if (vec) {
        q[u] = r < r1 ? *reinterpret_cast<const uint4*>(W + r * n + col) : make_uint4(0u, 0u, 0u, 0u);
      } else {
        uint32_t hw[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) hw[k] = (r < r1 && col + k < n) ? W[r * n + col + k] : 0u;
        q[u] = make_uint4(hw[0] | hw[1] << 16, hw[2] | hw[3] << 16, hw[4] | hw[5] << 16,
                          hw[6] | hw[7] << 16);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t r = rb + (int64_t)u * STEP;
      if (r < r1) {
        const uint32_t qq[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
        float wv[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          wv[2 * k] = h2f(qq[k]);
          wv[2 * k + 1] = h2f(qq[k] >> 16);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float vb = v[(int64_t)b * m + r];
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[b][k] = __builtin_fmaf(vb, wv[k], acc[b][k]);
        }
      }
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[b][k] += __shfl_xor(acc[b][k], off, 64);
  if (rs == 0)
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int k = 0; k < 8; ++k) red[wave][b][cl * 8 + k] = acc[b][k];
  __syncthreads();
  for (int idx = threadIdx.x; idx < B * CPB; idx += DN_T) {
    const int b = idx / CPB, c = idx % CPB;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w][b][c];
    const int64_t cc = (int64_t)blockIdx.x * CPB + c;
    if (cc < n) {
      if (atomic_out)
        atomicAdd(&y[(int64_t)b * n + cc], s);
      else
        y[(int64_t)b * n + cc] = s;
    }
  }
}

template <int LPR, int B>
static hipError_t dense_launch(const uint16_t* W, const float* v, int64_t m, int64_t n, float* y,
                               int row_splits, hipStream_t s) {
  constexpr int CPB = 8 * LPR;
  const int64_t gx = (n + CPB - 1) / CPB;
  if (row_splits < 1) row_splits = 1;
  if ((int64_t)row_splits > m) row_splits = (int)m;
  const int64_t rps = (m + row_splits - 1) / row_splits;
  const int gy = (int)((m + rps - 1) / rps);
  if (gy > 1) {
    hipError_t e = launch_zero_bytes(y, (uint64_t)B * n * sizeof(float), s);
    if (e != hipSuccess) return e;
  }
  const int aligned = ((n & 7) == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0) ? 1 : 0;
  hipLaunchKernelGGL((k_dense<LPR, B>), dim3((unsigned)gx, (unsigned)gy), dim3(DN_T), 0, s, W, v,
                     m, n, y, rps, gy > 1 ? 1 : 0, aligned);
  return hipGetLastError();
}

hipError_t launch_dense_gemv(const uint16_t* W, const float* v, int64_t m, int64_t n, float* y,
                             int lanes_per_row, int row_splits, hipStream_t s) {
  switch (lanes_per_row) {
    case 4: return dense_launch<4, 1>(W, v, m, n, y, row_splits, s);
    case 8: return dense_launch<8, 1>(W, v, m, n, y, row_splits, s);
    case 16: return dense_launch<16, 1>(W, v, m, n, y, row_splits, s);
    case 32: return dense_launch<32, 1>(W, v, m, n, y, row_splits, s);
    case 64: return dense_launch<64, 1>(W, v, m, n, y, row_splits, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dense_gemm_small(const uint16_t* W, const float* v, int batch, int64_t m,
                                   int64_t n, float* y, hipStream_t s) {
  // one pass over W per launch; batch split into supported widths
  int done = 0;
  while (done < batch) {
    const int left = batch - done;
    const int b = left >= 16 ? 16 : left >= 8 ? 8 : left >= 4 ? 4 : left >= 2 ? 2 : 1;
    const float* vb = v + (int64_t)done * m;
    float* yb = y + (int64_t)done * n;
    hipError_t e;
    const int64_t gx = (n + 63) / 64;
    const int rs = gx >= 256 ? 1 : (int)((512 + gx - 1) / gx);
    switch (b) {
      case 16: e = dense_launch<8, 16>(W, vb, m, n, yb, rs, s); break;
      case 8: e = dense_launch<8, 8>(W, vb, m, n, yb, rs, s); break;
      case 4: e = dense_launch<8, 4>(W, vb, m, n, yb, rs, s); break;
      case 2: e = dense_launch<8, 2>(W, vb, m, n, yb, rs, s); break;
      default: e = dense_launch<8, 1>(W, vb, m, n, yb, rs, s); break;
    }
    if (e != hipSuccess) return e;
    done += b;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- parity outputs

__global__ void k_debug_result(const uint32_t* result, float* cutoff, int64_t* K) {
  if (threadIdx.x == 0) {
    if (cutoff) *cutoff = __uint_as_float(result[0]);
    if (K) {
      K[0] = (int64_t)result[2];
      K[1] = (int64_t)result[1];
    }
  }
}

hipError_t launch_debug_result(const uint32_t* result, float* cutoff, int64_t* K, hipStream_t s) {
  hipLaunchKernelGGL(k_debug_result, dim3(1), dim3(64), 0, s, result, cutoff, K);
  return hipGetLastError();
}

// ---------------------------------------------------------------- glue

__global__ void k_silu_mul(const float* __restrict__ h1, const float* __restrict__ h3, int64_t n,
                           float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float x = h1[i];
    out[i] = x / (1.0f + expf(-x)) * h3[i];
  }
}

hipError_t launch_silu_mul(const float* h1, const float* h3, int64_t n, float* out, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_silu_mul, dim3((unsigned)blocks), dim3(256), 0, s, h1, h3, n, out);
  return hipGetLastError();
}

__global__ void k_zero_bytes(uint8_t* p, uint64_t bytes, int aligned) {
  const uint64_t nvec = aligned ? bytes / 16 : 0;
  uint4* p16 = reinterpret_cast<uint4*>(p);
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec;
       i += (uint64_t)gridDim.x * blockDim.x)
    p16[i] = make_uint4(0u, 0u, 0u, 0u);
  for (uint64_t i = nvec * 16 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero_bytes(void* p, uint64_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  uint64_t blocks = (bytes / 16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  const int aligned = (reinterpret_cast<uintptr_t>(p) & 15) == 0 ? 1 : 0;
  hipLaunchKernelGGL(k_zero_bytes, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<uint8_t*>(p), bytes, aligned);
  return hipGetLastError();
}

}  // namespace effort
