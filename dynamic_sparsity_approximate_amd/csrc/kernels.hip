// kernels.hip -- gfx950 kernels of the Effort approximate vector-matrix multiply.
//
// Method: HN thread "Show HN: Speeding up LLM inference 2x times (possibly)"
// (pseudocode precompute/approxMul quoted by gcy; sorted (index, value) rows in
// the reply to bigcat12345678; 16-part row split of bucketMul in the reply to
// marmaduke) and hntin item 40095016 (cutoff O(inDim log inDim), dispatch
// O(inDim), multiply O(effort inDim outDim)).
//
// Three kernels per call, all on one stream:
//   k_chart_hist chart |v_i| * probe_i[k] and a histogram of its top 12 bits;
//                zeroes y.
//   k_dispatch   per (group, row) how many rank-ordered entries to read, from the
//                low edge of the bin holding the K-th largest chart value; one
//                extra block finishes the exact radix selection of the cutoff.
//   k_bucketmul  per output-column group an LDS tile of y; each wave streams an
//                equal share of the group's run prefixes with 16-byte loads,
//                keeps entries whose key reaches the row threshold (from the
//                exact cutoff), adds v_i * w as 64-bit fixed point into the tile,
//                and finally adds the tile to y.
// No MFMA: the multiply is a bandwidth-bound gather-scatter, not a contraction.
#include <hip/hip_fp16.h>
#include <hip/hip_ext.h>
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

// Wave-level scans and sums with DPP row shifts (rows of 16 lanes) and
// readlane for the four row totals; no LDS traffic.
__device__ __forceinline__ uint32_t row_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
  return x;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x = row_incl_scan(x);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  const uint32_t add = row == 0 ? 0u : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2;
  return x + add;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  x = row_incl_scan(x);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 15) +
         (uint32_t)__builtin_amdgcn_readlane((int)x, 31) +
         (uint32_t)__builtin_amdgcn_readlane((int)x, 47) +
         (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ float wave_sum_f(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
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
// The P <= PM probe keys of row i in registers (16-byte loads when P % 8 == 0).
constexpr int PMAXR = 32;
template <int PM>
__device__ __forceinline__ void load_row_keys(const uint16_t* probes, int32_t P, int64_t i,
                                              uint32_t* key) {
  const uint16_t* pr = probes + i * P;
  if ((P & 7) == 0) {
#pragma unroll
    for (int c = 0; c < PM / 8; ++c) {
      uint4 q = make_uint4(0u, 0u, 0u, 0u);
      if (c * 8 < P) q = *reinterpret_cast<const uint4*>(pr + c * 8);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        key[c * 8 + 2 * j] = w[j] & 0xFFFFu;
        key[c * 8 + 2 * j + 1] = w[j] >> 16;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < PM; ++k) key[k] = k < P ? (uint32_t)pr[k] : 0u;
  }
}

constexpr int CH_T = 256;  // rows per block of the histogram kernel

__global__ __launch_bounds__(CH_T) void k_chart_hist(SelectArgs a) {
  __shared__ uint32_t hist[HIST_BINS];
  const int tid = threadIdx.x;
  for (int b = tid; b < HIST_BINS; b += CH_T) hist[b] = 0u;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * CH_T + tid;
  if (i < a.m) {
    const float av = fabsf(a.v[i]);
    if (a.P <= PMAXR) {
      uint32_t key[PMAXR];
      load_row_keys<PMAXR>(a.probes, a.P, i, key);
#pragma unroll
      for (int k = 0; k < PMAXR; ++k)
        if (k < a.P) atomicAdd(&hist[__float_as_uint(__fmul_rn(av, h2f(key[k]))) >> HIST_SHIFT], 1u);
    } else {
      const uint16_t* pr = a.probes + i * a.P;
      for (int k = 0; k < a.P; ++k)
        atomicAdd(&hist[__float_as_uint(__fmul_rn(av, h2f(pr[k]))) >> HIST_SHIFT], 1u);
    }
  }
  __syncthreads();
  for (int b = tid; b < HIST_BINS; b += CH_T)
    if (hist[b]) atomicAdd(&a.hist[b], hist[b]);
  // y is accumulated by the multiply; global stores come last (no barrier waits on them)
  for (int64_t j = (int64_t)blockIdx.x * CH_T + tid; j < a.n; j += (int64_t)gridDim.x * CH_T)
    a.y[j] = 0.0f;
  if (blockIdx.x == 0) {  // the dispatch accumulates into these
    for (int b = tid; b < 1024; b += CH_T) a.hist2[b] = 0u;
    if (tid == 0) a.result[RES_NCAND] = 0u;
  }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s, const EventPair* ev) {
  const int64_t blocks = (a.m + CH_T - 1) / CH_T;
  if (ev && ev->start)
    hipExtLaunchKernelGGL(k_chart_hist, dim3((unsigned)blocks), dim3(CH_T), 0, s, ev->start, ev->stop,
                          0, a);
  else
    hipLaunchKernelGGL(k_chart_hist, dim3((unsigned)blocks), dim3(CH_T), 0, s, a);
  return hipGetLastError();
}

// Smallest finite fp16 magnitude key k with fl32(av * k) >= c (0x7C00: none).
// The product is monotone in the key, so bisection finds it.
__device__ __forceinline__ uint32_t key_threshold(float av, float c) {
  uint32_t lo = 0u, hi = 0x7C00u;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (__fmul_rn(av, h2f(mid)) >= c)
      hi = mid;
    else
      lo = mid + 1u;
  }
  return lo;
}

__global__ __launch_bounds__(DSP_T) void k_dispatch(DispatchArgs a) {
  __shared__ uint32_t hist[HIST_BINS];
  __shared__ uint32_t h2[1024];
  __shared__ uint32_t tmp[DSP_T / 64 + 1];
  __shared__ uint32_t sres[8];
  __shared__ uint32_t red[16 * (DSP_T / 64)];
  __shared__ float redf[DSP_T / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int64_t i = (int64_t)blockIdx.x * DSP_T + tid;
  const bool valid = i < a.m;
  const int G1 = a.G + 1;
  // row data first (independent of the cutoff), then the histogram
  float av = 0.0f;
  uint32_t rmax = 0u;
  uint32_t pk[PMAXR];
  if (valid) {
    av = fabsf(a.v[i]);
    rmax = a.rowmax[i];
    if (a.P <= PMAXR) load_row_keys<PMAXR>(a.probes, a.P, i, pk);
  }
  for (int b = tid; b < HIST_BINS; b += DSP_T) hist[b] = a.hist[b];
  for (int b = tid; b < 1024; b += DSP_T) h2[b] = 0u;
  __syncthreads();
  find_from_top<DSP_T>(hist, HIST_BINS, a.K, tmp, sres);
  const uint32_t b1 = sres[0] & (HIST_BINS - 1);
  const uint32_t above1 = sres[1];
  // the K-th largest chart value lies in bin b1: its low edge bounds the cutoff below
  const float lo = __uint_as_float(b1 << HIST_SHIFT);
  const uint32_t t = key_threshold(av, lo);
  const bool none = !valid || rmax < t;  // no entry of the row can pass
  int32_t q = 0;
  uint32_t hits = 0u;  // chart entries of this row in bin b1 (P <= PMAXR)
  if (valid) {
    if (a.P <= PMAXR) {
#pragma unroll
      for (int k = 0; k < PMAXR; ++k) {
        if (k < a.P) {
          q += pk[k] >= t ? 1 : 0;  // probes are descending keys: q = segments kept whole
          const uint32_t bits = __float_as_uint(__fmul_rn(av, h2f(pk[k])));
          if ((bits >> HIST_SHIFT) == b1) {
            hits |= 1u << k;
            atomicAdd(&h2[(bits >> 9) & 1023u], 1u);
          }
        }
      }
    } else {
      const uint16_t* pr = a.probes + i * a.P;
      for (int k = 0; k < a.P; ++k) {
        const uint32_t key = pr[k];
        q += key >= t ? 1 : 0;
        const uint32_t bits = __float_as_uint(__fmul_rn(av, h2f(key)));
        if ((bits >> HIST_SHIFT) == b1) atomicAdd(&h2[(bits >> 9) & 1023u], 1u);
      }
    }
  }
  const int32_t qc = q < a.P ? q : a.P - 1;
  const uint32_t* cr = a.counts + ((size_t)(valid ? i : 0) * a.P + qc) * a.G4;
  constexpr int GCH = 16;  // groups per pass: their counts are loaded before any store
  constexpr int SUBS = DSP_T / DSP_ROWS;
  constexpr int WPS = DSP_ROWS / 64;
  // bound on |any sum of products| of the row
  const float bs = wave_sum_f(valid ? av * h2f(rmax) : 0.0f);
  if (lane == 0) redf[wid] = bs;
  for (int g0 = 0; g0 < a.G; g0 += GCH) {
    uint32_t L[GCH];
#pragma unroll
    for (int u4 = 0; u4 < GCH / 4; ++u4) {
      uint4 c4 = make_uint4(0u, 0u, 0u, 0u);
      if (!none && g0 + u4 * 4 < a.G) c4 = *reinterpret_cast<const uint4*>(cr + g0 + u4 * 4);
      L[u4 * 4 + 0] = c4.x;
      L[u4 * 4 + 1] = c4.y;
      L[u4 * 4 + 2] = c4.z;
      L[u4 * 4 + 3] = c4.w;
    }
#pragma unroll
    for (int u = 0; u < GCH; ++u) {
      if (g0 + u >= a.G) L[u] = 0u;
      const uint32_t s = wave_sum(L[u]);
      if (lane == 0) red[u * (DSP_T / 64) + wid] = s;
    }
    __syncthreads();  // no global store is outstanding here
    if (valid)
#pragma unroll
      for (int u = 0; u < GCH; ++u)
        if (g0 + u < a.G) a.runlen[(size_t)(g0 + u) * a.m + i] = L[u];
    for (int x = tid; x < GCH * SUBS; x += DSP_T) {
      const int u = x / SUBS, sub = x % SUBS;
      const int64_t sbt = (int64_t)blockIdx.x * SUBS + sub;
      if (g0 + u < a.G && sbt * DSP_ROWS < a.m) {
        uint32_t tot = 0;
        for (int w = 0; w < WPS; ++w) tot += red[u * (DSP_T / 64) + sub * WPS + w];
        a.bsum[(size_t)sbt * G1 + g0 + u] = tot;
      }
    }
    if (g0 == 0 && tid < SUBS) {
      const int64_t sbt = (int64_t)blockIdx.x * SUBS + tid;
      if (sbt * DSP_ROWS < a.m) {
        float tot = 0.0f;
        for (int w = 0; w < WPS; ++w) tot += redf[tid * WPS + w];
        a.bsum[(size_t)sbt * G1 + a.G] = __float_as_uint(tot);
      }
    }
    if (g0 + GCH < a.G) __syncthreads();  // red[] is reused (more than GCH groups)
  }
  // the bin's refinement histogram and its values, for the exact cutoff
  if (blockIdx.x == 0 && tid == 0) {
    a.result[RES_BIN] = b1;
    a.result[RES_ABOVE] = above1;
  }
  for (int b = tid; b < 1024; b += DSP_T)
    if (h2[b]) atomicAdd(&a.hist2[b], h2[b]);
  if (a.P <= PMAXR) {
    const uint32_t c = (uint32_t)__popc(hits);
    const uint32_t incl = wave_incl_scan(c);
    uint32_t base = 0u;
    if (lane == 63 && incl) base = atomicAdd(&a.result[RES_NCAND], incl);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, 63) + incl - c;
#pragma unroll
    for (int k = 0; k < PMAXR; ++k)
      if ((hits >> k) & 1u) a.cand[base++] = __float_as_uint(__fmul_rn(av, h2f(pk[k])));
  } else if (valid) {
    const uint16_t* pr = a.probes + i * a.P;
    for (int k = 0; k < a.P; ++k) {
      const uint32_t bits = __float_as_uint(__fmul_rn(av, h2f(pr[k])));
      if ((bits >> HIST_SHIFT) == b1) a.cand[atomicAdd(&a.result[RES_NCAND], 1u)] = bits;
    }
  }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s, const EventPair* ev) {
  const int64_t blocks = (a.m + DSP_T - 1) / DSP_T;
  if (ev && ev->start)
    hipExtLaunchKernelGGL(k_dispatch, dim3((unsigned)blocks), dim3(DSP_T), 0, s, ev->start, ev->stop,
                          0, a);
  else
    hipLaunchKernelGGL(k_dispatch, dim3((unsigned)blocks), dim3(DSP_T), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bucketMul

constexpr int MUL_T = 1024;
constexpr int MUL_W = MUL_T / 64;

// Finds, among `count` non-negative values x[0..count) (x(j) loads one), the
// index j with prefix(j) <= target < prefix(j) + x[j] and x[j] > 0; returns
// j and prefix(j).  Wave-uniform; requires target < sum.
template <typename X>
__device__ __forceinline__ void wave_locate(uint32_t count, uint32_t target, X x, uint32_t* idx,
                                            uint32_t* before) {
  const int lane = threadIdx.x & 63;
  uint32_t acc = 0;
  for (uint32_t j0 = 0; j0 < count; j0 += 256) {
    uint32_t s[4];  // 256 values loaded together, then scanned in order
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t j = j0 + (uint32_t)u * 64u + (uint32_t)lane;
      s[u] = j < count ? x(j) : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t inc = wave_incl_scan(s[u]);
      const uint32_t lo = acc + inc - s[u];
      const unsigned long long hit = __ballot(s[u] > 0u && lo <= target && target < lo + s[u]);
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        *idx = j0 + (uint32_t)u * 64u + (uint32_t)l;
        *before = (uint32_t)__builtin_amdgcn_readlane((int)lo, l);
        return;
      }
      acc += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    }
  }
  *idx = count;
  *before = acc;
}

// Fixed-point accumulation: with B >= |any sum of kept products| and B < 2^eB,
// scale S = 50 - eB puts every scaled sum below 2^50 in magnitude.  A product
// w * v * 2^S is exact in double (11 + 24 significant bits); adding 1.5 * 2^52
// rounds it to an integer held in the low mantissa bits, which are then read
// as an int64.
constexpr double kMagic = 6755399441055744.0;  // 1.5 * 2^52

__device__ __forceinline__ int64_t fixed_product(uint32_t w, double vs) {
  const double d = __builtin_fma((double)h2f(w), vs, kMagic);
  return (int64_t)(__double_as_longlong(d) - __double_as_longlong(kMagic));
}

// Exact cutoff from the bin b1 (and the count of values above it), the 1024-bin
// histogram of the bin's next 10 bits and the bin's values: two more radix
// digits.  Every block computes it; all get the same value.
__device__ uint32_t exact_cutoff(const MulArgs& a, uint32_t* hs, uint32_t* tmp, uint32_t* sres,
                                 uint32_t* kprime) {
  const int tid = threadIdx.x;
  const uint32_t b1 = a.result[RES_BIN], above1 = a.result[RES_ABOVE];
  const uint32_t nc = a.result[RES_NCAND];
  for (int b = tid; b < 1024; b += MUL_T) hs[b] = a.hist2[b];
  __syncthreads();
  const uint32_t K1 = a.K - above1;
  find_from_top<MUL_T>(hs, 1024, K1, tmp, sres);
  const uint32_t b2 = sres[0] & 1023u, above2 = sres[1];
  const uint32_t K2 = K1 - above2;
  const uint32_t pre = (b1 << 10) | b2;  // bits 30..9
  __syncthreads();
  for (int b = tid; b < 512; b += MUL_T) hs[b] = 0u;
  __syncthreads();
  for (uint32_t p0 = 0; p0 < nc; p0 += MUL_T * 4u) {
    uint32_t bits[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t p = p0 + (uint32_t)u * MUL_T + tid;
      bits[u] = p < nc ? a.cand[p] : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (bits[u] != 0xFFFFFFFFu && (bits[u] >> 9) == pre) atomicAdd(&hs[bits[u] & 511u], 1u);
  }
  __syncthreads();
  find_from_top<MUL_T>(hs, 512, K2, tmp, sres);
  const uint32_t b3 = sres[0] & 511u, above3 = sres[1];
  *kprime = above1 + above2 + above3 + hs[b3];
  __syncthreads();
  return (pre << 9) | b3;
}

template <bool REC>
__global__ __launch_bounds__(MUL_T) void k_bucketmul(
    const float* __restrict__ vvec, const uint32_t* __restrict__ entries,
    const uint32_t* __restrict__ runlen, const uint32_t* __restrict__ bsum,
    const uint32_t* __restrict__ result, float* __restrict__ y, MulArgs a) {
  extern __shared__ unsigned long long tile[];
  __shared__ uint32_t hs[1024];
  __shared__ uint32_t ctmp[MUL_T / 64 + 1];
  __shared__ uint32_t csres[8];
  (void)result;
  uint32_t kprime;
  const uint32_t cut_bits = exact_cutoff(a, hs, ctmp, csres, &kprime);
  const float cutoff = __uint_as_float(cut_bits);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.result[RES_CUTOFF] = cut_bits;
    a.result[RES_KPRIME] = kprime;
    a.result[RES_K] = a.K;
  }
  const int G = a.G;
  const int G1 = G + 1;
  const int g = (int)(blockIdx.x % (unsigned)G);
  const uint32_t bslot = blockIdx.x / (unsigned)G;
  const uint32_t bpg = gridDim.x / (unsigned)G;
  const int64_t col0 = (int64_t)g * a.TW;
  const int tw = (int)((int64_t)a.TW < a.n - col0 ? (int64_t)a.TW : a.n - col0);
  for (int c = threadIdx.x; c < tw; c += MUL_T) tile[c] = 0ull;

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t m = (uint32_t)a.m;
  const uint32_t nbd = (uint32_t)a.nbd;
  const uint32_t* rl = runlen + (size_t)g * a.m;

  // group total and the fixed-point scale
  uint32_t T = 0;
  float B = 0.0f;
  for (uint32_t b0 = 0; b0 < nbd; b0 += 64) {
    const uint32_t b = b0 + lane;
    T += wave_sum(b < nbd ? bsum[(size_t)b * G1 + g] : 0u);
    B += wave_sum_f(b < nbd ? __uint_as_float(bsum[(size_t)b * G1 + G]) : 0.0f);
  }
  int eB = 0;
  frexpf(B * 1.001f + 1e-38f, &eB);  // B * 1.001 < 2^eB; the margin covers float summation
  const int S = __builtin_amdgcn_readfirstlane(50 - eB);
  __syncthreads();

  // this wave's share [start, end) of the group's entries, concatenated over rows
  const uint64_t nslots = (uint64_t)bpg * MUL_W;
  const uint64_t slot = (uint64_t)bslot * MUL_W + wid;
  const uint32_t start = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)T * slot / nslots));
  const uint32_t end = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)T * (slot + 1) / nslots));

  if (start < end) {
    uint32_t bstar, before_b;
    wave_locate(nbd, start, [&](uint32_t b) { return bsum[(size_t)b * G1 + g]; }, &bstar, &before_b);
    const uint32_t r0 = bstar < nbd ? bstar * DSP_ROWS : m;
    const uint32_t nr = r0 < m ? (m - r0 < (uint32_t)DSP_ROWS ? m - r0 : (uint32_t)DSP_ROWS) : 0u;
    uint32_t jrow = 0, before_r = 0;
    if (nr > 0u)
      wave_locate(nr, start - before_b, [&](uint32_t j) { return rl[r0 + j]; }, &jrow, &before_r);
    uint32_t rowb = __builtin_amdgcn_readfirstlane(jrow < nr ? r0 + jrow : m);
    uint32_t offb = __builtin_amdgcn_readfirstlane(start - before_b - before_r);
    uint32_t remaining = end - start;

    while (remaining > 0u && rowb < m) {
      // metadata of up to 64 rows, one per lane
      const uint32_t r = rowb + (uint32_t)lane;
      uint32_t Lj = 0u;
      float vj = 0.0f;
      if (r < m) {
        Lj = min(rl[r], (uint32_t)tw);
        vj = vvec[r];
      }
      const uint32_t tj = Lj ? key_threshold(fabsf(vj), cutoff) : 0x7C00u;
      const uint32_t aj = lane == 0 ? offb : 0u;
      const uint32_t lenj = Lj > aj ? Lj - aj : 0u;
      const uint32_t incl = wave_incl_scan(lenj);
      const uint32_t excl = incl - lenj;
      const uint32_t takej = excl >= remaining ? 0u : min(lenj, remaining - excl);
      const uint32_t batch_take =
          min((uint32_t)__builtin_amdgcn_readlane((int)incl, 63), remaining);
      // clamped: only a row whose weights are all zero can exceed it, and its
      // products stay 0
      const double vsj = fmin(fmax(ldexp((double)vj, S), -0x1p100), 0x1p100);
      unsigned long long todo = __ballot(takej > 0u);

      // chunks of <= 1024 entries of one row; the next chunk's loads are in
      // flight while the current one is processed
      uint32_t cj = 0, cs0 = 0, cs1 = 0, ce = 0;
      bool have = false;
      uint4 cur[4], nxt[4];
      auto first_of = [&](uint32_t j, uint32_t* s0, uint32_t* e) {
        *s0 = (uint32_t)__builtin_amdgcn_readlane((int)aj, j);
        *e = *s0 + (uint32_t)__builtin_amdgcn_readlane((int)takej, j);
      };
      auto issue = [&](uint32_t j, uint32_t s0, uint32_t s1, uint4* buf) {
        const uint4* base = reinterpret_cast<const uint4*>(
            entries + (size_t)(rowb + j) * (size_t)a.row_stride + col0);
        const uint32_t o = (s0 & ~3u) + (uint32_t)lane * 4u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t p = o + (uint32_t)u * 256u;
          buf[u] = p < s1 ? base[p >> 2] : make_uint4(0u, 0u, 0u, 0u);
        }
      };
      if (todo) {
        cj = (uint32_t)(__ffsll((long long)todo) - 1);
        todo &= todo - 1ull;
        first_of(cj, &cs0, &ce);
        cs1 = min(ce, (cs0 & ~3u) + 1024u);
        issue(cj, cs0, cs1, cur);
        have = true;
      }
      while (have) {
        // next chunk: rest of this row, else the next row with entries
        uint32_t nj = cj, ns0 = cs1, ne = ce;
        bool nhave = true;
        if (cs1 >= ce) {
          if (todo) {
            nj = (uint32_t)(__ffsll((long long)todo) - 1);
            todo &= todo - 1ull;
            first_of(nj, &ns0, &ne);
          } else {
            nhave = false;
          }
        }
        const uint32_t ns1 = min(ne, (ns0 & ~3u) + 1024u);
        if (nhave) issue(nj, ns0, ns1, nxt);

        // process the current chunk
        const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)tj, cj);
        const double vs = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(vsj), cj),
                                           __builtin_amdgcn_readlane(__double2loint(vsj), cj));
        const uint32_t row = rowb + cj;
        uint32_t cnt = 0u;
        uint64_t fp = 0u;
        const uint32_t o = (cs0 & ~3u) + (uint32_t)lane * 4u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t p = o + (uint32_t)u * 256u;
          const uint32_t ev[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2) {
            const uint32_t w = ev[k2];
            const uint32_t pos = p + (uint32_t)k2;
            if (pos >= cs0 && pos < cs1 && (w & 0x7FFFu) >= t) {
              atomicAdd(&tile[w >> 16], (unsigned long long)fixed_product(w, vs));
              if (REC) {
                const uint64_t flat = (uint64_t)row * (uint64_t)a.n + (uint64_t)col0 + (w >> 16);
                if (a.mask) a.mask[flat] = 1u;
                fp += pair_hash(flat);
                ++cnt;
              }
            }
          }
        }
        if (REC) {
          uint32_t flo = (uint32_t)fp, fhi = (uint32_t)(fp >> 32);
          for (int sh = 32; sh > 0; sh >>= 1) {
            cnt += __shfl_xor(cnt, sh, 64);
            const uint32_t olo = __shfl_xor(flo, sh, 64);
            const uint32_t ohi = __shfl_xor(fhi, sh, 64);
            const uint64_t sum = ((uint64_t)fhi << 32 | flo) + ((uint64_t)ohi << 32 | olo);
            flo = (uint32_t)sum;
            fhi = (uint32_t)(sum >> 32);
          }
          if (lane == 0) {
            if (cnt && a.row_kept) atomicAdd(&a.row_kept[row], (int32_t)cnt);
            if (a.fingerprint) atomicAdd(a.fingerprint, ((unsigned long long)fhi << 32) | flo);
          }
        }
        cj = nj;
        cs0 = ns0;
        cs1 = ns1;
        ce = ne;
        have = nhave;
#pragma unroll
        for (int u = 0; u < 4; ++u) cur[u] = nxt[u];
      }
      remaining -= batch_take;
      rowb += 64u;
      offb = 0u;
    }
  }
  __syncthreads();
  const double unscale = ldexp(1.0, -S);
  for (int c = threadIdx.x; c < tw; c += MUL_T) {
    const long long acc = (long long)tile[c];
    if (acc != 0) atomicAdd(&y[col0 + c], (float)((double)acc * unscale));
  }
  if (blockIdx.x == 0)  // only the dispatch reads it: ready for the next call
    for (int b = threadIdx.x; b < HIST_BINS; b += MUL_T) a.hist[b] = 0u;
}

hipError_t launch_bucketmul(const MulArgs& a, bool record, int blocks_per_group, hipStream_t s,
                            const EventPair* ev) {
  const unsigned grid = (unsigned)(a.G * blocks_per_group);
  const size_t lds = (size_t)a.TW * sizeof(unsigned long long);
  if (ev && ev->start && !record)
    hipExtLaunchKernelGGL(k_bucketmul<false>, dim3(grid), dim3(MUL_T), (uint32_t)lds, s, ev->start,
                          ev->stop, 0, a.v, a.entries, a.runlen, a.bsum, a.result, a.y, a);
  else if (record)
    hipLaunchKernelGGL(k_bucketmul<true>, dim3(grid), dim3(MUL_T), lds, s, a.v, a.entries,
                       a.runlen, a.bsum, a.result, a.y, a);
  else
    hipLaunchKernelGGL(k_bucketmul<false>, dim3(grid), dim3(MUL_T), lds, s, a.v, a.entries,
                       a.runlen, a.bsum, a.result, a.y, a);
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
