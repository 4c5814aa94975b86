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
//                low edge of the bin holding the K-th largest chart value; the
//                chart values in that bin go to a candidate list and a
//                histogram of their next 10 bits.
//   k_bucketmul  one wave finishes the exact radix selection of the cutoff;
//                per output-column group an LDS tile of y; the other waves
//                stream their shares of the group's run prefixes with 16-byte
//                loads, keep entries whose key reaches the row threshold (from
//                the exact cutoff), add v_i * w as 32-bit fixed point into the
//                tile, and finally add the tile to y.
// The *_multi kernels run the same bodies for up to four matrices that share
// the input vector.
// No MFMA: the multiply is a bandwidth-bound gather-scatter, not a contraction.
#include <hip/hip_fp16.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "effort.h"
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

// Wave-level scans and sums with DPP: row shifts within rows of 16 lanes,
// then the row broadcasts of lanes 15 and 31 across rows; no LDS traffic and
// no branches.
__device__ __forceinline__ uint32_t row_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
  return x;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x = row_incl_scan(x);
  // rows 1 and 3 add the last lane of rows 0 and 2 (row_bcast:15), then rows
  // 2 and 3 add lane 31, the total of rows 0 and 1 (row_bcast:31); rows
  // outside the row mask add the old value 0
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
  return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), 63);
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

// ---------------------------------------------------------------- cutoff

// The P <= PM probe keys of row i in registers, two per word: key 2t in the
// low half of kw[t] (16-byte loads when P % 8 == 0).  Callers unpack a key
// where they use it (key_at), so every load of the row is in flight before
// the first wait; unpacking right after each load had serialized them.
constexpr int PMAXR = 32;
template <int PM>
__device__ __forceinline__ void load_row_keys(const uint16_t* probes, int32_t P, int64_t i,
                                              uint32_t* kw) {
  const uint16_t* pr = probes + i * P;
  if ((P & 7) == 0) {
#pragma unroll
    for (int c = 0; c < PM / 8; ++c) {
      uint4 q = make_uint4(0u, 0u, 0u, 0u);
      if (c * 8 < P) q = *reinterpret_cast<const uint4*>(pr + c * 8);
      kw[4 * c] = q.x;
      kw[4 * c + 1] = q.y;
      kw[4 * c + 2] = q.z;
      kw[4 * c + 3] = q.w;
    }
  } else {
    uint32_t h[PM];
#pragma unroll
    for (int k = 0; k < PM; ++k) h[k] = k < P ? (uint32_t)pr[k] : 0u;
#pragma unroll
    for (int t = 0; t < PM / 2; ++t) kw[t] = h[2 * t] | (h[2 * t + 1] << 16);
  }
}

// Keys pr[0 .. count) of a row, count <= PM, two per word (zero past count):
// 16-byte loads when vec (pr 16-byte aligned and the row's P a multiple of
// 8), else one load per key.  Used for rows with more than PM probes, a
// chunk of PM keys at a time.
template <int PM>
__device__ __forceinline__ void load_keys(const uint16_t* pr, int count, bool vec, uint32_t* kw) {
  if (vec) {
#pragma unroll
    for (int c = 0; c < PM / 8; ++c) {
      uint4 q = make_uint4(0u, 0u, 0u, 0u);
      if (c * 8 < count) q = *reinterpret_cast<const uint4*>(pr + c * 8);
      kw[4 * c] = q.x;
      kw[4 * c + 1] = q.y;
      kw[4 * c + 2] = q.z;
      kw[4 * c + 3] = q.w;
    }
  } else {
    uint32_t h[PM];
#pragma unroll
    for (int k = 0; k < PM; ++k) h[k] = k < count ? (uint32_t)pr[k] : 0u;
#pragma unroll
    for (int t = 0; t < PM / 2; ++t) kw[t] = h[2 * t] | (h[2 * t + 1] << 16);
  }
}

__device__ __forceinline__ uint32_t key_at(const uint32_t* kw, int k) {
  return (kw[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
}

constexpr int CH_T = 256;  // rows per block of the histogram kernel

// PM: probes per row held in registers (16 or 32); rows with more are read
// PM keys at a time.
template <int PM>
__device__ __forceinline__ void chart_hist_body(const SelectArgs& a) {
  __shared__ uint32_t hist[HIST_BINS + 1];  // + a slot for the keys past P
  const int tid = threadIdx.x;
  // the row's loads are issued before the histogram is cleared
  const int64_t i = (int64_t)blockIdx.x * CH_T + tid;
  const bool valid = i < a.m;
  float vi = 0.0f;
  uint32_t kw[PM / 2];
  if (valid) {
    vi = a.v[i];
    if (a.P <= PM) load_row_keys<PM>(a.probes, a.P, i, kw);
  }
  for (int b = tid; b < HIST_BINS; b += CH_T) hist[b] = 0u;
  __syncthreads();
  if (valid) {
    const float av = fabsf(vi);
    if (a.P <= PM) {
      // straight-line: the keys past P go to the spare slot, never merged
#pragma unroll
      for (int k = 0; k < PM; ++k) {
        const uint32_t bin = __float_as_uint(__fmul_rn(av, h2f(key_at(kw, k)))) >> HIST_SHIFT;
        atomicAdd(&hist[k < a.P ? bin : (uint32_t)HIST_BINS], 1u);
      }
    } else {
      // PM keys at a time; the keys past P go to the spare slot
      const uint16_t* pr = a.probes + i * a.P;
      const bool vec = (a.P & 7) == 0;
      for (int k0 = 0; k0 < a.P; k0 += PM) {
        load_keys<PM>(pr + k0, min(PM, a.P - k0), vec, kw);
#pragma unroll
        for (int k = 0; k < PM; ++k) {
          const uint32_t bin = __float_as_uint(__fmul_rn(av, h2f(key_at(kw, k)))) >> HIST_SHIFT;
          atomicAdd(&hist[k0 + k < a.P ? bin : (uint32_t)HIST_BINS], 1u);
        }
      }
    }
  }
  __syncthreads();
  // merge into the global histogram: every bin read first (one LDS wait, not
  // one per bin), then one atomic per non-empty bin
  constexpr int BPT = HIST_BINS / CH_T;
  uint32_t hv[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) hv[j] = hist[tid + j * CH_T];
#pragma unroll
  for (int j = 0; j < BPT; ++j)
    if (hv[j]) atomicAdd(&a.hist[tid + j * CH_T], hv[j]);
  // y is accumulated by the multiply; global stores come last (no barrier waits on them)
  for (int64_t j = (int64_t)blockIdx.x * CH_T + tid; j < a.n; j += (int64_t)gridDim.x * CH_T)
    a.y[j] = 0.0f;
  if (blockIdx.x == 0) {  // the dispatch accumulates into these
    for (int b = tid; b < 1024; b += CH_T) a.hist2[b] = 0u;
    if (tid == 0) {
      a.result[RES_NCAND] = 0u;
      a.result[RES_FLAGS] = 0u;
    }
  }
  for (int64_t j = (int64_t)blockIdx.x * CH_T + tid; j < a.bsum_words; j += (int64_t)gridDim.x * CH_T)
    a.bsum[j] = 0u;
}

template <int PM>
__global__ __launch_bounds__(CH_T) void k_chart_hist(SelectArgs a) {
  if (blockIdx.y) {  // vector blockIdx.y of a batch
    const uint64_t k = blockIdx.y;
    a.v += k * a.m;
    a.y += k * a.n;
    a.hist += k * a.vec_ws;
    a.hist2 += k * a.vec_ws;
    a.result += k * a.vec_ws;
    a.bsum += k * a.vec_ws;
  }
  chart_hist_body<PM>(a);
}

// Several matrices sharing v: blockIdx.y picks the matrix.
template <int PM>
__global__ __launch_bounds__(CH_T) void k_chart_hist_multi(SelectMulti mm) {
  chart_hist_body<PM>(mm.a[blockIdx.y]);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s, const EventPair* ev, int nvec) {
  const int64_t blocks = (a.m + CH_T - 1) / CH_T;
  const dim3 grid((unsigned)blocks, (unsigned)nvec);
  auto kern = a.P <= 16 ? k_chart_hist<16> : k_chart_hist<PMAXR>;
  if (ev && ev->start)
    hipExtLaunchKernelGGL(kern, grid, dim3(CH_T), 0, s, ev->start, ev->stop, 0, a);
  else
    hipLaunchKernelGGL(kern, grid, dim3(CH_T), 0, s, a);
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

// The same threshold from an estimate: k = fp16(c / av) is within one key of
// it (the fp32 quotient is far finer than an fp16 step), so checking the exact
// products at k - 2 .. k + 1 settles it; out-of-range quotients, tiny av and
// any check that does not bracket the answer fall back to bisection.
__device__ __forceinline__ uint32_t key_threshold_fast(float av, float c) {
  if (!(c > 0.0f)) return 0u;
  const float q = c * __builtin_amdgcn_rcpf(av);
  if (av >= 0x1p-100f && q <= 65504.0f) {
    const uint32_t k = (uint32_t)__half_as_ushort(__float2half_rn(q));
    auto ok = [&](uint32_t key) { return __fmul_rn(av, h2f(key)) >= c; };
    const bool o1 = k > 0u && ok(k - 1u);
    const bool o2 = k > 1u && ok(k - 2u);
    const bool o0 = ok(k);
    const bool p1 = k + 1u >= 0x7C00u || ok(k + 1u);
    if (o1 && !o2) return k - 1u;
    if (!o1 && o0) return k;
    if (!o0 && p1) return k + 1u;
  }
  return key_threshold(av, c);
}

static_assert(DSP_T == DSP_ROWS, "one dispatch block per block of rows");
static_assert(HIST_BINS == 16 * DSP_T, "each dispatch thread holds 16 histogram bins");

// One block per DSP_ROWS rows, one thread per row.  Every block finds the bin
// b1 of the K-th largest chart value from the histogram (16 bins per thread in
// registers, one block scan).  With lo = the bin's low edge (a lower bound of
// the cutoff), a row keeps whole the probe segments whose chart value is >= lo
// (probes are descending, so these are segments 0..q-1), and the read length
// of (row, group) covers segments 0..min(q, P-1) through the counts table.
// PM: probes per row held in registers (16 or 32); rows with more are read
// PM keys at a time (one round trip per chunk), their candidates' slots
// reserved once per wave as for the others.
template <int PM>
__device__ __forceinline__ void dispatch_body(const DispatchArgs& a) {
  __shared__ uint32_t tmp[DSP_T / 64 + 1];
  __shared__ uint32_t sres[2];
  __shared__ uint32_t red[4 * (DSP_T / 64)];
  __shared__ float redf[DSP_T / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int64_t i = (int64_t)blockIdx.x * DSP_T + tid;
  const bool valid = i < a.m;
  const int G1 = a.G + 1;
  // capacity of the candidate list: the count cannot exceed it when the select
  // kernel has reset it, and stores beyond it are dropped if it has not
  const uint64_t capc = cand_capacity(a.m, a.P);
  // this thread's 16 histogram bins and the row's data, all loads issued
  // together (|v| is taken after the histogram loads are issued, so that its
  // wait does not hold them back)
  const int hb = HIST_BINS - 16 * (tid + 1);  // bins hb .. hb + 15, thread 0 holds the top
  uint32_t h[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 q4 = *reinterpret_cast<const uint4*>(a.hist + hb + 4 * c);
    h[4 * c] = q4.x;
    h[4 * c + 1] = q4.y;
    h[4 * c + 2] = q4.z;
    h[4 * c + 3] = q4.w;
  }
  float vi = 0.0f;
  uint32_t rmax = 0u;
  uint32_t pk[PM / 2];  // the row's probe keys, two per word (zero past P)
#pragma unroll
  for (int t = 0; t < PM / 2; ++t) pk[t] = 0u;
  if (valid) {
    vi = a.v[i];
    rmax = a.rowmax[i];
    if (a.P <= PM) load_row_keys<PM>(a.probes, a.P, i, pk);
  }
  uint32_t hs = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) hs += h[k];
  uint32_t tot;
  uint32_t above = block_excl_scan<DSP_T>(hs, tmp, &tot);
  if (above < a.K && a.K <= above + hs) {
    // from the top bin down, the bins whose running total stays below K lie
    // wholly above the K-th value: count them (no branches)
    uint32_t acc = above, nb = 0u, before = above;
#pragma unroll
    for (int k = 15; k >= 0; --k) {
      const uint32_t nxt = acc + h[k];
      const bool below = nxt < a.K;
      nb += below ? 1u : 0u;
      before = below ? nxt : before;
      acc = nxt;
    }
    sres[0] = (uint32_t)(hb + 15) - nb;
    sres[1] = before;
  }
  __syncthreads();
  const float av = fabsf(vi);
  const uint32_t b1 = sres[0] & (HIST_BINS - 1);
  const uint32_t above1 = sres[1];
  const uint32_t lo_bits = b1 << HIST_SHIFT;
  const bool none = !valid || __float_as_uint(__fmul_rn(av, h2f(rmax))) < lo_bits;
  // bin b1 holds the chart bits [lo_bits, hi_bits); no chart reaches 2^31
  const uint32_t hi_bits = (b1 + 1u) << HIST_SHIFT;
  int32_t q = 0;
  uint32_t hits = 0u;  // chart entries of this row in bin b1 (P <= PM)
  uint32_t rlo = 0u, rhi = 0u;  // P > PM: those entries are keys rhi .. rlo - 1
  if (valid) {
    if (a.P <= PM) {
      // A row's probes do not increase with k, so neither do its chart
      // values: the ones at or above a bound form a prefix, and the ones in
      // bin b1 the range [chi, clo).  The keys past P are 0 and only count
      // toward clo when lo_bits is 0; the counts are clamped to P.
      uint32_t clo = 0u, chi = 0u;
#pragma unroll
      for (int k = 0; k < PM; ++k) {
        const uint32_t bits = __float_as_uint(__fmul_rn(av, h2f(key_at(pk, k))));
        clo += bits >= lo_bits ? 1u : 0u;
        chi += bits >= hi_bits ? 1u : 0u;
      }
      clo = min(clo, (uint32_t)a.P);
      chi = min(chi, (uint32_t)a.P);
      q = (int32_t)clo;
      // bits chi .. clo - 1 (clo <= 32; shifts of 32 go through 64 bits)
      hits = (uint32_t)((1ull << clo) - (1ull << chi));
    } else {
      // more probes than registers: the same prefix counts, PM keys at a
      // time (the chunks' loads wait one round trip each)
      const uint16_t* pr = a.probes + i * a.P;
      const bool vec = (a.P & 7) == 0;
      uint32_t clo = 0u, chi = 0u;
      for (int k0 = 0; k0 < a.P; k0 += PM) {
        uint32_t kw[PM / 2];
        load_keys<PM>(pr + k0, min(PM, a.P - k0), vec, kw);
#pragma unroll
        for (int k = 0; k < PM; ++k) {
          const uint32_t bits = __float_as_uint(__fmul_rn(av, h2f(key_at(kw, k))));
          const bool in = k0 + k < a.P;
          clo += in && bits >= lo_bits ? 1u : 0u;
          chi += in && bits >= hi_bits ? 1u : 0u;
        }
      }
      q = (int32_t)clo;
      rlo = clo;
      rhi = chi;
    }
  }
  // The chart values in bin b1, for the exact cutoff: their slots are
  // reserved here, so that the reservation's round trip overlaps the work on
  // the read lengths; the values are stored at the end.
  uint32_t cnt = 0u, cpos = 0u, cret = 0u;
  {
    cnt = a.P <= PM ? (uint32_t)__popc(hits) : rlo - rhi;
    const uint32_t incl = wave_incl_scan(cnt);
    cpos = incl - cnt;
    if (lane == 63 && incl) cret = atomicAdd(&a.result[RES_NCAND], incl);
  }
  const int32_t qc = q < a.P ? q : a.P - 1;
  const uint32_t* cr = a.counts + ((size_t)(valid ? i : 0) * a.P + qc) * a.G4;
  constexpr int NW = DSP_T / 64;
  // bound on |any sum of products| of the row
  const float bs = wave_sum_f(valid ? av * h2f(rmax) : 0.0f);
  if (lane == 0) redf[wid] = bs;
  for (int g0 = 0; g0 < a.G; g0 += 4) {  // 4 groups (one 16-byte slice) a pass
    uint4 c4 = make_uint4(0u, 0u, 0u, 0u);
    if (!none) c4 = *reinterpret_cast<const uint4*>(cr + g0);
    const uint32_t L[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (g0 + u < a.G) {
        const uint32_t s = wave_sum(L[u]);
        if (lane == 0) red[u * NW + wid] = s;
      }
    }
    __syncthreads();
    if (valid)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (g0 + u < a.G) a.runlen[(size_t)(g0 + u) * a.m + i] = L[u];
    if (tid < 4 && g0 + tid < a.G) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += red[tid * NW + w];
      a.bsum[(size_t)blockIdx.x * G1 + g0 + tid] = t;
    }
    if (g0 == 0 && tid == 0) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += redf[w];
      a.bsum[(size_t)blockIdx.x * G1 + a.G] = __float_as_uint(t);
    }
    if (g0 + 4 < a.G) __syncthreads();  // red[] is reused (more than 4 groups)
  }
  if (blockIdx.x == 0 && tid == 0) {
    a.result[RES_BIN] = b1;
    a.result[RES_ABOVE] = above1;
  }
  // Last, the chart values in bin b1: into the candidate list and the
  // refinement histogram of their bits 18..9 (memory instructions inside the
  // keep loop above, even rarely taken ones, made it 0.4 us slower).
  uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)cret, 63) + cpos;
  if (a.P <= PM) {
#pragma unroll
    for (int k = 0; k < PM; ++k) {
      if ((hits >> k) & 1u) {
        const uint32_t bits = __float_as_uint(__fmul_rn(av, h2f(key_at(pk, k))));
        if ((uint64_t)base < capc) a.cand[base] = bits;
        ++base;
        atomicAdd(&a.hist2[(bits >> 9) & 1023u], 1u);
      }
    }
  } else if (valid) {
    const uint16_t* pr = a.probes + i * a.P;
    for (uint32_t k = rhi; k < rlo; ++k) {
      const uint32_t bits = __float_as_uint(__fmul_rn(av, h2f(pr[k])));
      if ((uint64_t)base < capc) a.cand[base] = bits;
      ++base;
      atomicAdd(&a.hist2[(bits >> 9) & 1023u], 1u);
    }
  }
}

template <int PM>
__global__ __launch_bounds__(DSP_T) void k_dispatch(DispatchArgs a) {
  if (blockIdx.y) {  // vector blockIdx.y of a batch
    const uint64_t k = blockIdx.y;
    a.v += k * a.m;
    a.hist += k * a.vec_ws;
    a.hist2 += k * a.vec_ws;
    a.cand += k * a.vec_ws;
    a.result += k * a.vec_ws;
    a.runlen += k * a.vec_ws;
    a.bsum += k * a.vec_ws;
  }
  dispatch_body<PM>(a);
}

// Several matrices sharing v: blockIdx.y picks the matrix.
template <int PM>
__global__ __launch_bounds__(DSP_T) void k_dispatch_multi(DispatchMulti mm) {
  const DispatchArgs& a = mm.a[blockIdx.y];
  // past this matrix's rows (a taller one sized the grid): no rows, and no
  // per-256-row sums to write (the matrix's sum array ends before this block)
  if ((int64_t)blockIdx.x * DSP_T >= a.m) return;
  dispatch_body<PM>(a);
}


// The dispatch for P = 16 and 32 with the read lengths of every segment
// loaded up front: a block holds QR rows of LPR = P / 4 lanes (64 rows of 4,
// or 32 of 8), lane s of a row holding probes 4s .. 4s + 3 and the counts
// slices of those four segments, loaded with the histogram, so no load waits
// for the bin b1 (the slice used, at segment min(q, P - 1), is already in its
// lane's registers).  m / QR blocks; the per-256-row sums are accumulated
// with atomics into words the chart kernel zeroed, and the candidate slots
// are reserved once per block.  QG4: words of a counts slice (G4), 4 for up
// to 4 column groups, 8 for up to 8; a segment's slice is QG4 / 4 16-byte
// words.
template <int LPR>
constexpr int quad_block_rows() {
  return DSP_T / LPR;
}
static_assert(quad_block_rows<4>() == QUAD_ROWS, "four lanes per row at P = 16");
static_assert(DSP_ROWS % quad_block_rows<8>() == 0, "a block's rows lie in one 256-row block");
static_assert(quad_block_rows<8>() * 32 == RCAP, "P = 32 regions hold RCAP slots too");

template <int QG4, int LPR>
__device__ __forceinline__ void dispatch_quad_body(const DispatchArgs& a) {
  static_assert(QG4 == 4 || QG4 == 8, "counts slices of 4 or 8 words");
  static_assert(LPR == 4 || LPR == 8, "P = 16 or 32");
  constexpr int QR = quad_block_rows<LPR>();  // rows per block
  constexpr int PQ = 4 * LPR;                 // probes per row
  constexpr int QH = QG4 / 4;  // 16-byte words per segment slice
  constexpr int NW = DSP_T / 64;
  __shared__ uint32_t tmp[NW + 1];
  __shared__ uint32_t sres[2];
  __shared__ uint32_t red[NW][QG4];
  __shared__ float redf[NW];
  __shared__ uint32_t sbase;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int sub = tid & (LPR - 1);                            // segments 4 sub .. 4 sub + 3
  const int64_t i = (int64_t)blockIdx.x * QR + (tid / LPR);  // row
  const bool valid = i < a.m;
  const int G1 = a.G + 1;
  const uint64_t capc = cand_capacity(a.m, a.P);
  const bool regions = cand_regions(a.P, a.G, a.m);
  // every load first: 16 histogram bins, the row's v and max key, this lane's
  // four probe keys and four counts slices
  const int hb = HIST_BINS - 16 * (tid + 1);  // bins hb .. hb + 15, thread 0 holds the top
  uint32_t h[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 q4 = *reinterpret_cast<const uint4*>(a.hist + hb + 4 * c);
    h[4 * c] = q4.x;
    h[4 * c + 1] = q4.y;
    h[4 * c + 2] = q4.z;
    h[4 * c + 3] = q4.w;
  }
  float vi = 0.0f;
  uint32_t rmax = 0u;
  uint2 kq = make_uint2(0u, 0u);  // keys 4 sub .. 4 sub + 3, two per word
  // the counts slices of the four segments: words 0..3 of segment j in cj,
  // words 4..7 (8 groups) in cjh -- named values, not arrays, so that the
  // selection below stays in registers
  uint4 c0 = make_uint4(0u, 0u, 0u, 0u), c1 = c0, c2 = c0, c3 = c0;
  uint4 c0h = c0, c1h = c0, c2h = c0, c3h = c0;
  if (valid) {
    vi = a.v[i];
    rmax = a.rowmax[i];
    kq = *reinterpret_cast<const uint2*>(a.probes + i * PQ + 4 * sub);
    const uint4* cr = reinterpret_cast<const uint4*>(a.counts + ((size_t)i * PQ + 4 * sub) * QG4);
    c0 = cr[0];
    c1 = cr[QH];
    c2 = cr[2 * QH];
    c3 = cr[3 * QH];
    if constexpr (QH == 2) {
      c0h = cr[1];
      c1h = cr[QH + 1];
      c2h = cr[2 * QH + 1];
      c3h = cr[3 * QH + 1];
    }
  }
  uint32_t hs = 0;
#pragma unroll
  for (int t = 0; t < 16; ++t) hs += h[t];
  uint32_t tot;
  uint32_t above = block_excl_scan<DSP_T>(hs, tmp, &tot);
  if (above < a.K && a.K <= above + hs) {
    // from the top bin down, the bins whose running total stays below K lie
    // wholly above the K-th value: count them (no branches)
    uint32_t acc = above, nb = 0u, before = above;
#pragma unroll
    for (int t = 15; t >= 0; --t) {
      const uint32_t nxt = acc + h[t];
      const bool below = nxt < a.K;
      nb += below ? 1u : 0u;
      before = below ? nxt : before;
      acc = nxt;
    }
    sres[0] = (uint32_t)(hb + 15) - nb;
    sres[1] = before;
  }
  __syncthreads();
  const float av = fabsf(vi);
  const uint32_t b1 = sres[0] & (HIST_BINS - 1);
  const uint32_t above1 = sres[1];
  const uint32_t lo_bits = b1 << HIST_SHIFT;
  const uint32_t hi_bits = (b1 + 1u) << HIST_SHIFT;  // no chart reaches 2^31
  // this lane's four chart values (probes do not increase with k: the kept
  // segments of a row are 0 .. q - 1, the ones in bin b1 a range of them)
  uint32_t bits[4];
  bits[0] = __float_as_uint(__fmul_rn(av, h2f(kq.x)));
  bits[1] = __float_as_uint(__fmul_rn(av, h2f(kq.x >> 16)));
  bits[2] = __float_as_uint(__fmul_rn(av, h2f(kq.y)));
  bits[3] = __float_as_uint(__fmul_rn(av, h2f(kq.y >> 16)));
  uint32_t nk = 0u, nh = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    nk += valid && bits[k] >= lo_bits ? 1u : 0u;
    nh += valid && bits[k] >= lo_bits && bits[k] < hi_bits ? 1u : 0u;
  }
  // the candidates' slots: one reservation per block, issued now so that its
  // round trip overlaps the sums below; the values are stored last
  const uint32_t cpos = block_excl_scan<DSP_T>(nh, tmp, &tot);
  uint32_t ret = 0u;  // thread 0: the block's first slot, used (waited for) only at the end
  if (regions) {
    if (tid == 0) a.result[RES_RCOUNT + blockIdx.x] = tot;
  } else if (tid == 0 && tot) {
    ret = atomicAdd(&a.result[RES_NCAND], tot);
  }
  // q: the row's kept segments, summed over its LPR lanes
  uint32_t q = nk;
  q += (uint32_t)__shfl_xor((int)q, 1, 64);
  q += (uint32_t)__shfl_xor((int)q, 2, 64);
  if constexpr (LPR == 8) q += (uint32_t)__shfl_xor((int)q, 4, 64);
  const uint32_t qc = q < (uint32_t)PQ ? q : (uint32_t)PQ - 1u;
  const bool none = !valid || __float_as_uint(__fmul_rn(av, h2f(rmax))) < lo_bits;
  const bool owner = valid && (qc >> 2) == (uint32_t)sub;
  const uint32_t kk = qc & 3u;
  const bool use = owner && !none;
  uint32_t L[QG4];
  const uint4 x = kk == 0u ? c0 : kk == 1u ? c1 : kk == 2u ? c2 : c3;
  L[0] = use ? x.x : 0u;
  L[1] = use ? x.y : 0u;
  L[2] = use ? x.z : 0u;
  L[3] = use ? x.w : 0u;
  if constexpr (QH == 2) {
    const uint4 xh = kk == 0u ? c0h : kk == 1u ? c1h : kk == 2u ? c2h : c3h;
    L[4] = use ? xh.x : 0u;
    L[5] = use ? xh.y : 0u;
    L[6] = use ? xh.z : 0u;
    L[7] = use ? xh.w : 0u;
  }
  if (owner)
#pragma unroll
    for (int g = 0; g < QG4; ++g)
      if (g < a.G) a.runlen[(size_t)g * a.m + i] = L[g];
  // per-256-row sums: per wave, per block, then one atomic per column
#pragma unroll
  for (int g = 0; g < QG4; ++g)
    if (g < a.G) {
      const uint32_t sg = wave_sum(L[g]);
      if (lane == 0) red[wid][g] = sg;
    }
  const float bnd = wave_sum_f(valid && sub == 0 ? av * h2f(rmax) : 0.0f);
  if (lane == 0) redf[wid] = bnd;
  __syncthreads();
  const size_t brow = (size_t)((uint64_t)blockIdx.x * QR / DSP_ROWS) * G1;
  if (tid < a.G) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w][tid];
    if (t) atomicAdd(&a.bsum[brow + tid], t);
  } else if (tid == a.G) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += redf[w];
    if (t != 0.0f) atomicAdd(reinterpret_cast<float*>(&a.bsum[brow + a.G]), t);
  }
  if (blockIdx.x == 0 && tid == 0) {
    a.result[RES_BIN] = b1;
    a.result[RES_ABOVE] = above1;
  }
  // last, the chart values in bin b1: into the candidate list and the
  // refinement histogram of their bits 18..9
  uint32_t base;
  if (regions) {
    base = blockIdx.x * (uint32_t)RCAP + cpos;
  } else {
    if (tid == 0) sbase = ret;
    __syncthreads();
    base = sbase + cpos;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (valid && bits[k] >= lo_bits && bits[k] < hi_bits) {
      if ((uint64_t)base < capc) a.cand[base] = bits[k];
      ++base;
      atomicAdd(&a.hist2[(bits[k] >> 9) & 1023u], 1u);
    }
  }
}

template <int QG4, int LPR>
__global__ __launch_bounds__(DSP_T) void k_dispatch_quad(DispatchArgs a) {
  if (blockIdx.y) {  // vector blockIdx.y of a batch
    const uint64_t k = blockIdx.y;
    a.v += k * a.m;
    a.hist += k * a.vec_ws;
    a.hist2 += k * a.vec_ws;
    a.cand += k * a.vec_ws;
    a.result += k * a.vec_ws;
    a.runlen += k * a.vec_ws;
    a.bsum += k * a.vec_ws;
  }
  dispatch_quad_body<QG4, LPR>(a);
}

// whether the quad-lane dispatch serves these arguments (G4 is 4 or 8 then)
static bool quad_dispatch(const DispatchArgs& a) { return quad_dispatch_ok(a.P, a.G); }

// The pairs of one launch share P (dispatch_multi_quad), hence the rows per block.
template <int LPR>
__global__ __launch_bounds__(DSP_T) void k_dispatch_quad_multi(DispatchMulti mm) {
  const DispatchArgs& a = mm.a[blockIdx.y];
  // past this matrix's rows (a taller one sized the grid): nothing to do
  if ((int64_t)blockIdx.x * quad_block_rows<LPR>() >= a.m) return;
  if (a.G4 == 4)
    dispatch_quad_body<4, LPR>(a);
  else
    dispatch_quad_body<8, LPR>(a);
}

hipError_t launch_select_multi(const SelectMulti& mm, int count, hipStream_t s) {
  if (count < 1 || count > EFFORT_MAX_MULTI) return hipErrorInvalidValue;
  int P = 0;
  int64_t m = 0;
  for (int j = 0; j < count; ++j) {
    P = mm.a[j].P > P ? mm.a[j].P : P;
    m = mm.a[j].m > m ? mm.a[j].m : m;
  }
  // sized for the tallest matrix; a shorter one's extra blocks hold no rows
  const dim3 grid((unsigned)((m + CH_T - 1) / CH_T), (unsigned)count);
  if (P <= 16)
    hipLaunchKernelGGL(k_chart_hist_multi<16>, grid, dim3(CH_T), 0, s, mm);
  else
    hipLaunchKernelGGL(k_chart_hist_multi<PMAXR>, grid, dim3(CH_T), 0, s, mm);
  return hipGetLastError();
}

bool dispatch_multi_quad(const DispatchMulti& mm, int count) {
  bool quad = true;
  for (int j = 0; j < count; ++j) quad = quad && quad_dispatch(mm.a[j]) && mm.a[j].P == mm.a[0].P;
  return quad;
}

hipError_t launch_dispatch_multi(const DispatchMulti& mm, int count, hipStream_t s) {
  if (count < 1 || count > EFFORT_MAX_MULTI) return hipErrorInvalidValue;
  int P = 0;
  int64_t m = 0;
  for (int j = 0; j < count; ++j) {
    P = mm.a[j].P > P ? mm.a[j].P : P;
    m = mm.a[j].m > m ? mm.a[j].m : m;
  }
  if (dispatch_multi_quad(mm, count)) {
    const int qr = quad_rows(P);
    const dim3 gq((unsigned)((m + qr - 1) / qr), (unsigned)count);
    if (P == 32)
      hipLaunchKernelGGL(k_dispatch_quad_multi<8>, gq, dim3(DSP_T), 0, s, mm);
    else
      hipLaunchKernelGGL(k_dispatch_quad_multi<4>, gq, dim3(DSP_T), 0, s, mm);
    return hipGetLastError();
  }
  // sized for the tallest matrix; a shorter one's extra blocks return at once
  const dim3 grid((unsigned)((m + DSP_T - 1) / DSP_T), (unsigned)count);
  if (P <= 16)
    hipLaunchKernelGGL(k_dispatch_multi<16>, grid, dim3(DSP_T), 0, s, mm);
  else
    hipLaunchKernelGGL(k_dispatch_multi<PMAXR>, grid, dim3(DSP_T), 0, s, mm);
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s, const EventPair* ev, int nvec) {
  if (quad_dispatch(a)) {
    const int qr = quad_rows(a.P);
    const dim3 gq((unsigned)((a.m + qr - 1) / qr), (unsigned)nvec);
    auto kern = a.P == 32 ? (a.G4 == 4 ? k_dispatch_quad<4, 8> : k_dispatch_quad<8, 8>)
                          : (a.G4 == 4 ? k_dispatch_quad<4, 4> : k_dispatch_quad<8, 4>);
    if (ev && ev->start)
      hipExtLaunchKernelGGL(kern, gq, dim3(DSP_T), 0, s, ev->start, ev->stop, 0, a);
    else
      hipLaunchKernelGGL(kern, gq, dim3(DSP_T), 0, s, a);
    return hipGetLastError();
  }
  const int64_t blocks = (a.m + DSP_T - 1) / DSP_T;
  const dim3 grid((unsigned)blocks, (unsigned)nvec);
  // probes in registers: 16 when they fit (the common P), else 32
  auto kern = a.P <= 16 ? k_dispatch<16> : k_dispatch<PMAXR>;
  if (ev && ev->start)
    hipExtLaunchKernelGGL(kern, grid, dim3(DSP_T), 0, s, ev->start, ev->stop, 0, a);
  else
    hipLaunchKernelGGL(kern, grid, dim3(DSP_T), 0, s, a);
  return hipGetLastError();
}

// Union read lengths of nv vectors: one thread per row, one block per 256 rows.
__global__ __launch_bounds__(DSP_T) void k_union(UnionArgs a) {
  __shared__ uint32_t red[DSP_T / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t i = (int64_t)blockIdx.x * DSP_T + tid;
  const bool valid = i < a.m;
  for (int g = 0; g < a.G; ++g) {
    uint32_t L = 0u;
    if (valid)
      for (int k = 0; k < a.nv; ++k)
        L = max(L, a.runlen[(size_t)k * a.vec_ws + (size_t)g * a.m + i]);
    if (valid) a.urunlen[(size_t)g * a.m + i] = L;
    const uint32_t sw = wave_sum(L);
    if (lane == 0) red[wid] = sw;
    __syncthreads();
    if (tid == 0) {
      uint32_t t = 0;
      for (int w = 0; w < DSP_T / 64; ++w) t += red[w];
      a.ubsum[(size_t)blockIdx.x * (a.G + 1) + g] = t;
    }
    __syncthreads();
  }
}

hipError_t launch_union(const UnionArgs& a, hipStream_t s) {
  const int64_t blocks = (a.m + DSP_T - 1) / DSP_T;
  hipLaunchKernelGGL(k_union, dim3((unsigned)blocks), dim3(DSP_T), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bucketMul

// threads per bucketMul block.  One vector: 9 waves, wave 0 computing the
// cutoff and 8 streaming (measured faster than 7 or 9 streaming waves);
// a batched pass: 16 waves (waves 0..7 compute the pass's cutoffs, wave 8 the
// partition sums, then all stream).
template <int BP>
constexpr int mul_threads() {
  return BP == 1 ? 576 : 1024;
}
constexpr int CH = 256;  // u32 format: entries per chunk, one 16-byte quad per lane
// Units per chunk: a quad of 4 entries per lane (u32), two records of 4
// entries per lane (r12: 12 bytes each, q8: 8 bytes).
// Loads per lane of one chunk (records, u32: quads of 4 entries).  r12 and
// q8 chunks are two: 128 records, 1536 (r12) or 1024 (q8) contiguous bytes
// per wave, loaded as two halves; the larger pieces of a run in flight
// measured 0.2 us (r12) and 0.6 us (q8) faster at 4096x14336 than one record
// per lane (three or four per lane, and two quads per lane for u32, were
// slower or no faster).
template <int FMT>
constexpr int records_per_lane() {
  return FMT == EFFORT_ENTRY_U32 ? 1 : 2;
}
template <int FMT>
constexpr uint32_t chunk_units() {
  return (FMT == EFFORT_ENTRY_U32 ? (uint32_t)CH : 64u) * (uint32_t)records_per_lane<FMT>();
}

// Chunks in flight per wave: a ring of loads, a slot processed and then
// refilled, so RING - 1 chunks stay outstanding while one is used.  4-byte
// entries: 4 (measured faster than 2, 6 or 8).  r12: 3 chunks of 1536 bytes
// (2 was slower, 4 the same); q8: 3 of 1024 (4 the same).
#ifndef EFFORT_RING_U32
#define EFFORT_RING_U32 4
#endif
#ifndef EFFORT_RING_R12
#define EFFORT_RING_R12 3
#endif
#ifndef EFFORT_RING_Q8
#define EFFORT_RING_Q8 3
#endif
template <int FMT>
constexpr int ring_depth() {
  return FMT == EFFORT_ENTRY_R12 ? EFFORT_RING_R12 : FMT == EFFORT_ENTRY_Q8 ? EFFORT_RING_Q8 : EFFORT_RING_U32;
}

// A scaled product to the tile's integer unit, floor(x + 0.5) in one
// instruction (checked against the host's floor(x + 0.5) over 10^5 values on
// gfx950): a fixed rounding, so the tile sums stay independent of order.
__device__ __forceinline__ int32_t to_fixed(float x) {
  int32_t r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// The q8 format: per wave, a table of the bucket bounds of its batch's 64
// rows, 17 slots a row (16 segments, padded so that the rows' slots spread
// over the LDS banks).  One vector: {lo | hi << 16, shift}; a batched pass,
// whose LDS holds several tiles: lo | hi << 16 only, the shift recomputed.
constexpr int Q8_ROW_SLOTS = 17;
template <int BP>
struct Q8Slot {
  using T = uint32_t;
};
template <>
struct Q8Slot<1> {
  using T = uint2;
};
// The level shift of a bucket with key range d = hi - lo: the smallest s with
// 15 * 2^s >= d, i.e. the bit length of floor((d - 1) / 15) for d >= 1, and 0
// for d = 0.  floor(x / 15) = (x * 0x8889) >> 19 for x < 2^15.
__device__ __forceinline__ uint32_t q8_shift(uint32_t d) {
  const uint32_t q = ((max(d, 1u) - 1u) * 0x8889u) >> 19;
  return 31u - (uint32_t)__builtin_clz(2u * q + 1u);
}
__device__ __forceinline__ void q8_make(uint32_t lo, uint32_t hi, uint2& t) {
  t = make_uint2(lo | (hi << 16), q8_shift(hi - lo));
}
__device__ __forceinline__ void q8_make(uint32_t lo, uint32_t hi, uint32_t& t) { t = lo | (hi << 16); }
// The bounds as one word lo | hi << 16, and the shift.
__device__ __forceinline__ void q8_packed(uint2 t, uint32_t& lohi, uint32_t& sh) {
  lohi = t.x;
  sh = t.y;
}
__device__ __forceinline__ void q8_packed(uint32_t t, uint32_t& lohi, uint32_t& sh) {
  lohi = t;
  sh = q8_shift((t >> 16) - (t & 0xFFFFu));
}
// Two levels at once in the 16-bit halves: min(lo + (code << sh), hi) per
// half (packed 16-bit integer operations).  Keys stay below 2^15 and
// lo + (15 << sh) below 2^16, so no half overflows.
typedef unsigned short q8_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t q8_levels2(uint32_t codes, uint32_t lo2, uint32_t hi2, uint32_t sh) {
  const q8_u16x2 c = __builtin_bit_cast(q8_u16x2, codes);
  const q8_u16x2 l = __builtin_bit_cast(q8_u16x2, lo2);
  const q8_u16x2 h = __builtin_bit_cast(q8_u16x2, hi2);
  const q8_u16x2 s = {(unsigned short)sh, (unsigned short)sh};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(l + (c << s), h));
}

// A chunk of one row's run: units [s0, s1), at most chunk_units; `run` is the
// row's run, `tf` / `vf` the row's fp32 magnitude threshold and scaled
// activation (one vector), all wave-uniform.
struct Chunk {
  const uint32_t* run;
  uint32_t j, s0, s1;  // row of the batch, units [s0, s1) of its run
  float tf, vf;
  bool valid;
};

// Word 3 of a raw buffer descriptor on gfx9-family chips: 32-bit data format
// (a zero format would make every access out of range).
constexpr int kBufferDword3 = 0x00020000;

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

// Radix selection of the exact cutoff by one wave.  The dispatch found the
// bin b1 of the K-th largest chart value (bits 30..19) and the count above1 of
// larger values; the refinement histogram hist2 of the bin's values (bits
// 18..9) gives the second digit, and the candidate values that share bits
// 30..9 give the last nine bits through a 512-bin histogram in the wave's own
// LDS words h3[512].  Every step keeps the bin holding the remaining rank, so
// the result is the K-th largest value itself.

// The second digit from the refinement histogram (lane l holds bins
// [1008 - 16 l, 1024 - 16 l), lane 0 the top): every lane counts, from its top
// bin down, the bins whose running total stays below K1 (selects, no
// branches), and lane L's answer is kept.  Returns bits 30..9 of the cutoff;
// *above2 counts the values above its bin within b1.  Wave-uniform.
__device__ __forceinline__ uint32_t second_digit(const uint32_t* h, uint32_t b1, uint32_t K1,
                                                 uint32_t* above2) {
  const int lane = threadIdx.x & 63;
  uint32_t sum = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) sum += h[k];
  const uint32_t above = wave_incl_scan(sum) - sum;
  const unsigned long long hit = __ballot(above < K1 && K1 <= above + sum);
  const int L = __ffsll((long long)hit) - 1;
  uint32_t acc = above, nb = 0u, before = above;
#pragma unroll
  for (int k = 15; k >= 0; --k) {
    const uint32_t nxt = acc + h[k];
    const bool below = nxt < K1;
    nb += below ? 1u : 0u;
    before = below ? nxt : before;
    acc = nxt;
  }
  const uint32_t b2 = (uint32_t)__builtin_amdgcn_readlane((int)((uint32_t)(1008 - 16 * lane + 15) - nb), L);
  *above2 = (uint32_t)__builtin_amdgcn_readlane((int)before, L);
  return (b1 << 10) | b2;
}

// The last digit from h3 (filled by the caller with the matching candidates'
// bits 8..0): returns the cutoff's bit pattern; *kprime = the number of chart
// values >= it.  Wave-uniform.
__device__ __forceinline__ uint32_t third_digit(const uint32_t* h3, uint32_t pre, uint32_t K2,
                                                uint32_t above12, uint32_t* kprime) {
  const int lane = threadIdx.x & 63;
  // lane l holds bins [504 - 8 l, 512 - 8 l)
  uint32_t g[8];
  uint32_t sum = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    g[k] = h3[504 - 8 * lane + k];
    sum += g[k];
  }
  const uint32_t above = wave_incl_scan(sum) - sum;
  const unsigned long long hit3 = __ballot(above < K2 && K2 <= above + sum);
  const int L3 = __ffsll((long long)hit3) - 1;
  // as for the second digit; c3 is the count of the first bin whose running
  // total reaches K2
  uint32_t acc = above, nb = 0u, before = above, c3 = 0u;
  bool found = false;
#pragma unroll
  for (int k = 7; k >= 0; --k) {
    const uint32_t nxt = acc + g[k];
    const bool below = nxt < K2;
    nb += below ? 1u : 0u;
    before = below ? nxt : before;
    c3 = !below && !found ? g[k] : c3;
    found = found || !below;
    acc = nxt;
  }
  const uint32_t b3 = (uint32_t)__builtin_amdgcn_readlane((int)((uint32_t)(504 - 8 * lane + 7) - nb), L3);
  const uint32_t above3 = (uint32_t)__builtin_amdgcn_readlane((int)before, L3);
  c3 = (uint32_t)__builtin_amdgcn_readlane((int)c3, L3);
  *kprime = above12 + above3 + c3;
  return (pre << 9) | b3;
}

// The candidates as one list of nc values (ncap: capacity of the first
// loads, words past it read as zero).  The first CB * 64 are loaded with the
// histogram, the next RB * 64 as soon as the count is known, so that their
// round trip overlaps the second digit's work; more come in rounds.
__device__ uint32_t wave_exact_cutoff(const uint32_t* __restrict__ hist2,
                                      const uint32_t* __restrict__ cand, uint32_t ncap, uint32_t nc,
                                      uint32_t b1, uint32_t above1, uint32_t K, uint32_t* h3,
                                      uint32_t* kprime) {
  const int lane = threadIdx.x & 63;
  uint32_t h[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 q = *reinterpret_cast<const uint4*>(hist2 + 1008 - 16 * lane + 4 * c);
    h[4 * c] = q.x;
    h[4 * c + 1] = q.y;
    h[4 * c + 2] = q.z;
    h[4 * c + 3] = q.w;
  }
  constexpr int CB = 16;
  uint32_t cv[CB];
  {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)cand, (short)0, (int)(ncap * 4u), kBufferDword3);
#pragma unroll
    for (int u = 0; u < CB; ++u) cv[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, (u * 64 + lane) * 4, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) h3[k * 64 + lane] = 0u;
  constexpr int RB = 48;
  const bool more = nc > CB * 64u;
  uint32_t rv[RB];
  if (more) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)cand, (short)0, (int)(nc * 4u), kBufferDword3);
#pragma unroll
    for (int u = 0; u < RB; ++u)
      rv[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, ((CB + u) * 64 + lane) * 4, 0, 0);
  }
  const uint32_t K1 = K - above1;
  uint32_t above2;
  const uint32_t pre = second_digit(h, b1, K1, &above2);  // bits 30..9 of the cutoff
  const uint32_t K2 = K1 - above2;
  // last digit: histogram of the matching candidates' bits 8..0
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    const uint32_t p = (uint32_t)(u * 64 + lane);
    if (p < nc && (cv[u] >> 9) == pre) atomicAdd(&h3[cv[u] & 511u], 1u);
  }
  if (more) {
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const uint32_t p = (uint32_t)((CB + u) * 64 + lane);
      if (p < nc && (rv[u] >> 9) == pre) atomicAdd(&h3[rv[u] & 511u], 1u);
    }
    // still more: CB per lane a round
    for (uint32_t p0 = (CB + RB) * 64u; p0 < nc; p0 += CB * 64u) {
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const uint32_t p = p0 + (uint32_t)(u * 64 + lane);
        cv[u] = p < nc ? cand[p] : 0u;
      }
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const uint32_t p = p0 + (uint32_t)(u * 64 + lane);
        if (p < nc && (cv[u] >> 9) == pre) atomicAdd(&h3[cv[u] & 511u], 1u);
      }
    }
  }
  return third_digit(h3, pre, K2, above1 + above2, kprime);
}

// The candidates in nreg <= 64 regions of RCAP slots (region r: the chart
// values in the cutoff's bin of dispatch block r, counts[r] of them).  Lane r
// loads its region's count and first RSPEC slots with the histogram (one
// round trip); a region with more takes further rounds.
constexpr int RSPEC = 32;
__device__ uint32_t wave_exact_cutoff_regions(const uint32_t* __restrict__ hist2,
                                              const uint32_t* __restrict__ cand, uint32_t capw,
                                              const uint32_t* __restrict__ counts, uint32_t nreg,
                                              uint32_t b1, uint32_t above1, uint32_t K,
                                              uint32_t* h3, uint32_t* kprime) {
  const int lane = threadIdx.x & 63;
  uint32_t h[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 q = *reinterpret_cast<const uint4*>(hist2 + 1008 - 16 * lane + 4 * c);
    h[4 * c] = q.x;
    h[4 * c + 1] = q.y;
    h[4 * c + 2] = q.z;
    h[4 * c + 3] = q.w;
  }
  // counts past nreg read as zero, and so do slots past the list's capacity
  const uint32_t rc = (uint32_t)lane < nreg ? counts[lane] : 0u;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)cand, (short)0, (int)(capw * 4u), kBufferDword3);
  const int rbase = lane * RCAP * 4;  // bytes
  uint32_t cv[RSPEC];
#pragma unroll
  for (int c = 0; c < RSPEC / 4; ++c) {
    const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, rbase + c * 16, 0, 0);
    cv[4 * c] = q[0];
    cv[4 * c + 1] = q[1];
    cv[4 * c + 2] = q[2];
    cv[4 * c + 3] = q[3];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) h3[k * 64 + lane] = 0u;
  const uint32_t K1 = K - above1;
  uint32_t above2;
  const uint32_t pre = second_digit(h, b1, K1, &above2);  // bits 30..9 of the cutoff
  const uint32_t K2 = K1 - above2;
#pragma unroll
  for (int u = 0; u < RSPEC; ++u)
    if ((uint32_t)u < rc && (cv[u] >> 9) == pre) atomicAdd(&h3[cv[u] & 511u], 1u);
  // regions with more than RSPEC candidates: RSPEC more per round
  for (uint32_t s0 = RSPEC; __ballot(rc > s0); s0 += RSPEC) {
#pragma unroll
    for (int c = 0; c < RSPEC / 4; ++c) {
      const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, rbase + (int)(s0 * 4u) + c * 16, 0, 0);
      cv[4 * c] = q[0];
      cv[4 * c + 1] = q[1];
      cv[4 * c + 2] = q[2];
      cv[4 * c + 3] = q[3];
    }
#pragma unroll
    for (int u = 0; u < RSPEC; ++u)
      if (s0 + (uint32_t)u < rc && (cv[u] >> 9) == pre) atomicAdd(&h3[cv[u] & 511u], 1u);
  }
  return third_digit(h3, pre, K2, above1 + above2, kprime);
}

// Where share wave j's part of a block's entries starts, in 128ths of them.
// One vector: 8 share waves, waves 1..9 of the block.  A workgroup's waves are
// spread over the CU's 4 SIMDs in turn and a SIMD issues its older wave first,
// so share waves 0..3 (the first share wave on their SIMD) stream faster than
// 4..7; share waves 3 and 7 also share their SIMD with the cutoff wave and
// start streaming last.  The weights make the waves finish together (fitted to
// per-wave timestamps, then measured).  A batched pass: 16 equal shares.
constexpr uint32_t kShareW1[8] = {18, 18, 17, 17, 15, 15, 15, 13};
static_assert(kShareW1[0] + kShareW1[1] + kShareW1[2] + kShareW1[3] + kShareW1[4] + kShareW1[5] +
                  kShareW1[6] + kShareW1[7] == 128,
              "one vector's share weights cover the block");
// byte j: the sum of the weights before share wave j (j < 8)
constexpr uint64_t share_cum_bytes() {
  uint64_t r = 0;
  uint32_t c = 0;
  for (int k = 0; k < 8; ++k) {
    r |= (uint64_t)c << (8 * k);
    c += kShareW1[k];
  }
  return r;
}
constexpr uint64_t kShareCum1 = share_cum_bytes();
// share_cum(j) for j below the number of share waves (8 or 16); a few scalar
// instructions
template <int BP>
__device__ __forceinline__ uint32_t share_cum(uint32_t j) {
  if constexpr (BP == 1)
    return (uint32_t)(kShareCum1 >> (8u * j)) & 0xFFu;
  else
    return j * 8u;
}

// Block (g, s) of the grid: group g's LDS tile, share s of its entries.
//
// Prologue, three dependent rounds of global loads:
//   (1) the per-256-row sums that place each wave's share (and, for one
//       vector, give the fixed-point scale); for the cutoff, its bin, the
//       refinement histogram and the candidate chart values, from which the
//       exact cutoff is computed (every block gets the same value);
//   (2) per wave, the run lengths and activations of the 256 rows where its
//       share starts;
//   (3) the share's first chunks of entries, in flight while each row's fp16
//       key threshold is derived from the cutoff.
// One vector: wave 0 only computes the cutoff, while the other waves run the
// three rounds; each waits for the cutoff (an LDS flag) only after load round 3.
// Batched: waves 0..nv-1 compute the cutoffs and wave PW the partition sums
// before a barrier, then every wave runs rounds 2 and 3.
//
// Accumulation: with B >= |any sum of kept products| and B * 1.001 < 2^eB,
// the scale 2^S, S = 30 - eB, keeps every tile sum below 2^30 in magnitude.
// A kept product is fl32(w * v * 2^S) rounded to an integer (relative error
// 2^-24 plus half a unit of 2^-S) and added to the column's int32 LDS word;
// integer adds make the tile independent of order.
// The kernel's body for block `bid` of `nblk` (the grid, or one matrix's
// part of a multi-matrix grid).
template <bool REC, int BP, int FMT>
__device__ __forceinline__ void bucketmul_body(
    const uint32_t bid, const uint32_t nblk, const float* __restrict__ vvec,
    const uint32_t* __restrict__ entries, const uint32_t* __restrict__ runlen,
    const uint32_t* __restrict__ bsum, const uint32_t* __restrict__ result,
    float* __restrict__ y, const MulArgs& a) {
  static_assert(BP >= 1 && BP <= 8, "at most 8 vectors per pass");
  constexpr int MUL_T = mul_threads<BP>();
  constexpr int MUL_W = MUL_T / 64;
  static_assert(BP == 1 || MUL_W > BP, "a wave for each cutoff and one for the partition");
  static_assert(BP == 1 ? MUL_W == 9 : MUL_W == 16, "share_cum splits a block over 8 or 16 share waves");
  constexpr int PW = BP == 1 ? 1 : BP;  // the wave that scans the partition sums
  // tiles: one vector's in a static array, several vectors' in dynamic LDS
  // (vector p's at p * TW)
  __shared__ int32_t tile1[BP == 1 ? EFFORT_MAX_GROUP_WIDTH : 1];
  extern __shared__ int32_t tiled[];
  int32_t* const tile = BP == 1 ? tile1 : tiled;
  __shared__ uint32_t h3w[BP][512];  // wave p: histogram of vector p's last cutoff digit
  __shared__ uint32_t pfx[256];      // inclusive prefix sums of the group's per-256-row sums
  __shared__ uint32_t sT;
  __shared__ uint32_t sReady;  // one vector: set once the cutoff is in sCut[0]
  __shared__ uint32_t sCut[BP];
  __shared__ int32_t sS[BP];
  __shared__ uint32_t mrl[MUL_W][DSP_ROWS];           // per wave: run lengths of its first 256 rows
  __shared__ float mv[BP == 1 ? MUL_W : 1][DSP_ROWS];  // and (one vector) their activations
  constexpr bool Q8 = FMT == EFFORT_ENTRY_Q8;
  using QT = typename Q8Slot<BP>::T;
  __shared__ QT qtab[Q8 ? MUL_W : 1][Q8 ? 64 * Q8_ROW_SLOTS : 1];  // q8: the batch's bucket bounds
  const int tid = threadIdx.x;
  // the wave index made provably uniform: descriptors and per-wave offsets
  // derived from it stay in scalar registers
  const int lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.G;
  const int G1 = G + 1;
  const int g = (int)(bid % (unsigned)G);
  const uint32_t bslot = bid / (unsigned)G;
  const uint32_t bpg = nblk / (unsigned)G;
  const int64_t col0 = (int64_t)g * a.TW;
  const int tw = (int)((int64_t)a.TW < a.n - col0 ? (int64_t)a.TW : a.n - col0);
  const uint32_t m = (uint32_t)a.m;
  const uint32_t nbd = (uint32_t)a.nbd;
  const uint32_t* rl = runlen + (size_t)g * a.m;
  const int nv = BP == 1 ? 1 : a.nv;

  // The chart histogram is read only by the dispatch, which has finished:
  // cleared here, spread over the grid, ready for the next call.
  for (int p = 0; p < nv; ++p)
    for (int b = (int)bid * MUL_T + tid; b < HIST_BINS; b += (int)nblk * MUL_T)
      a.hist[(size_t)p * a.vec_ws + b] = 0u;

  // ---- load round 1
  // wave p < nv: the exact cutoff of vector p (batched: and its fixed-point scale)
  auto cutoff_wave = [&]() {
    const uint64_t vo = (uint64_t)wid * a.vec_ws;
    const uint32_t* res = result + vo;
    const uint32_t b1 = res[RES_BIN], above1 = res[RES_ABOVE];
    const uint64_t cap = cand_capacity(a.m, a.P);
    uint32_t kp, cut;
    if (a.regions) {  // where the dispatch put them
      const uint32_t nreg = (uint32_t)((a.m + quad_rows(a.P) - 1) / quad_rows(a.P));
      cut = wave_exact_cutoff_regions(a.hist2 + vo, a.cand + vo, (uint32_t)cap, res + RES_RCOUNT,
                                      nreg, b1, above1, a.K, h3w[wid], &kp);
    } else {
      // the count never exceeds the list's capacity; clamped so that no read can
      const uint32_t nc = (uint32_t)min((uint64_t)res[RES_NCAND], cap);
      const uint32_t ncap = (uint32_t)(cap < 1024u ? cap : 1024u);
      cut = wave_exact_cutoff(a.hist2 + vo, a.cand + vo, ncap, nc, b1, above1, a.K, h3w[wid], &kp);
    }
    if (lane == 0) {
      sCut[wid] = cut;
      if (bid == 0) {
        a.result[vo + RES_CUTOFF] = cut;
        a.result[vo + RES_KPRIME] = kp;
        a.result[vo + RES_K] = a.K;
      }
    }
    if (BP > 1) {
      float B = 0.0f;
      for (uint32_t b0 = 0; b0 < nbd; b0 += 64) {
        const uint32_t b = b0 + lane;
        B += wave_sum_f(b < nbd ? __uint_as_float(a.vbsum[vo + (size_t)b * G1 + G]) : 0.0f);
      }
      if (lane == 0) {
        int eB = 0;
        frexpf(B * 1.001f + 1e-38f, &eB);  // the margin covers float summation
        sS[wid] = 30 - eB;
      }
    }
  };
  // The group's per-256-row sums: index u * 64 + lane in sb[u] (one vector).
  uint32_t sb[4] = {0u, 0u, 0u, 0u};
  uint32_t sp[4] = {0u, 0u, 0u, 0u};
  uint32_t T = 0u;  // the group's entry count
  int S1 = 0;       // one vector: the fixed-point scale, computed by every share wave
  // One vector: load round 1 also loads the run lengths and activations of two
  // 256-row blocks from w0, around the row where the wave's share would start
  // if the group's entries were spread evenly over its rows; load round 2 loads
  // only when the share starts outside them.
  uint32_t w0 = nbd;
  uint32_t slr[8];
  float slv[8];
  if constexpr (BP == 1) {
    // Wave 0 only computes the cutoff and then publishes it through sReady.
    // Every other wave sums the group's per-256-row sums itself (the same
    // loads and the same order of addition in every wave, so the same T and
    // scale), stages its rows, issues its first chunks and waits for the
    // cutoff only then, each at its own pace.  The one barrier here clears the
    // tile and the flag before anyone uses them.
    for (int c = tid; c < tw; c += MUL_T) tile[c] = 0;
    if (tid == 0) sReady = 0u;
    __syncthreads();
    if (wid == 0) {
      cutoff_wave();
      if (lane == 0) __hip_atomic_store(&sReady, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      float sf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t b = (uint32_t)u * 64u + (uint32_t)lane;
        sb[u] = b < nbd ? bsum[(size_t)b * G1 + g] : 0u;
        sf[u] = b < nbd ? __uint_as_float(a.vbsum[(size_t)b * G1 + G]) : 0.0f;
      }
      // 16-byte loads: byte offsets within 32 bits, both arrays 16-byte aligned
      if (m <= (1u << 28) && ((reinterpret_cast<uintptr_t>(rl) | reinterpret_cast<uintptr_t>(vvec)) & 15u) == 0u) {
        // the guessed start row: m times the share's start as a fraction of
        // the group, (bslot + share_cum / 128) / bpg, in 32-bit fixed point;
        // the window holds its block and the nearer neighbour
        const uint32_t F = bslot * a.bpg_recip +
                           __umulhi(a.bpg_recip, share_cum<1>((uint32_t)(wid - 1)) << 25);
        const uint32_t gr = __umulhi(m, F);
        const uint32_t bg = gr / DSP_ROWS;
        uint32_t lo = gr % DSP_ROWS < DSP_ROWS / 2 && bg > 0u ? bg - 1u : bg;
        if (lo + 2u > nbd) lo = nbd >= 2u ? nbd - 2u : 0u;
        w0 = __builtin_amdgcn_readfirstlane(lo);
        // lane l: rows 4l .. 4l + 3 of each block; words past m read as zero
        const __amdgpu_buffer_rsrc_t rr =
            __builtin_amdgcn_make_buffer_rsrc((void*)rl, (short)0, (int)(m * 4u), kBufferDword3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)vvec, (short)0, (int)(m * 4u), kBufferDword3);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int off = (int)((w0 * DSP_ROWS + (uint32_t)h * DSP_ROWS + 4u * (uint32_t)lane) * 4u);
          const auto qr = __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0);
          const auto qv = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            slr[4 * h + k] = qr[k];
            slv[4 * h + k] = __uint_as_float(qv[k]);
          }
        }
      }
      // inclusive prefix sums of the first 256 block sums (sp), kept for the
      // search of the share's block
      float B = 0.0f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sp[u] = T;
        if ((uint32_t)u * 64u < nbd) {  // rounds past the last block hold zeros
          const uint32_t inc = wave_incl_scan(sb[u]);
          sp[u] = T + inc;
          T += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
          B += wave_sum_f(sf[u]);
        }
      }
      for (uint32_t b0 = 256; b0 < nbd; b0 += 64) {  // more than 256 blocks of rows
        const uint32_t b = b0 + lane;
        T += wave_sum(b < nbd ? bsum[(size_t)b * G1 + g] : 0u);
        B += wave_sum_f(b < nbd ? __uint_as_float(a.vbsum[(size_t)b * G1 + G]) : 0.0f);
      }
      int eB = 0;
      frexpf(B * 1.001f + 1e-38f, &eB);  // the margin covers float summation
      S1 = 30 - eB;
      if (wid == 1 && lane == 0) sS[0] = S1;  // for the flush
    }
  } else {
    // Batched: waves 0..nv-1 the cutoffs, wave PW the partition sums, then a
    // barrier.
    if (wid < nv) {
      cutoff_wave();
    } else if (wid == PW) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t b = (uint32_t)u * 64u + (uint32_t)lane;
        sb[u] = b < nbd ? bsum[(size_t)b * G1 + g] : 0u;
      }
      uint32_t acc = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t inc = wave_incl_scan(sb[u]);
        pfx[u * 64 + lane] = acc + inc;
        acc += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
      }
      for (uint32_t b0 = 256; b0 < nbd; b0 += 64) {  // more than 256 blocks of rows
        const uint32_t b = b0 + lane;
        acc += wave_sum(b < nbd ? bsum[(size_t)b * G1 + g] : 0u);
      }
      if (lane == 0) sT = acc;
    }
    for (int p = 0; p < nv; ++p)
      for (int c = tid; c < tw; c += MUL_T) tile[p * a.TW + c] = 0;
    __syncthreads();
    T = sT;
  }

  // this wave's share [start, end) of the group's entries, concatenated over rows
  constexpr int NCW = BP == 1 ? 1 : 0;  // waves without a share
  // Block boundaries bound(b) = floor(T * b R / 2^32) with R = floor(2^32 /
  // bpg) for b < bpg, and bound(bpg) = T: 32 x 32-bit products (the high word
  // of each), non-decreasing, the same in every block; block sizes differ by
  // at most 1 + T bpg / 2^32 entries.  Within the block, share wave j gets
  // the fraction (share_cum(j + 1) - share_cum(j)) / 128 of the block's
  // entries (share_cum(j) < 128 below the last share, so share_cum(j) << 25
  // fits 32 bits).
  constexpr uint32_t NSH = BP == 1 ? 8u : 16u;  // share waves
  uint32_t start = 0u, end = 0u;
  if (wid >= NCW) {
    const uint32_t Tu = __builtin_amdgcn_readfirstlane(T);
    const uint32_t bs = __umulhi(Tu, bslot * a.bpg_recip);
    const uint32_t be = bslot + 1u >= bpg ? Tu : __umulhi(Tu, (bslot + 1u) * a.bpg_recip);
    const uint32_t d = be - bs;
    const uint32_t j = (uint32_t)(wid - NCW);
    start = j == 0u ? bs : bs + __umulhi(d, share_cum<BP>(j) << 25);
    end = j + 1u >= NSH ? be : bs + __umulhi(d, share_cum<BP>(j + 1u) << 25);
    start = __builtin_amdgcn_readfirstlane(start);
    end = __builtin_amdgcn_readfirstlane(end);
  }
  const bool active = start < end;

  // the 256-row block where the share starts: first prefix above start
  uint32_t bstar = nbd, before_b = 0;
  if (active) {
    if (nbd <= 256u) {
      if constexpr (BP == 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t lo = sp[u] - sb[u];
          const unsigned long long hit = __ballot(sb[u] > 0u && lo <= start && start < sp[u]);
          if (hit) {
            const int l = __ffsll((long long)hit) - 1;
            bstar = (uint32_t)u * 64u + (uint32_t)l;
            before_b = (uint32_t)__builtin_amdgcn_readlane((int)lo, l);
            break;
          }
        }
      } else {
        for (int u = 0; u < 4; ++u) {
          const uint32_t b = (uint32_t)u * 64u + (uint32_t)lane;
          const unsigned long long hit = __ballot(b < nbd && pfx[b] > start);
          if (hit) {
            bstar = (uint32_t)u * 64u + (uint32_t)(__ffsll((long long)hit) - 1);
            before_b = bstar > 0u ? pfx[bstar - 1u] : 0u;
            break;
          }
        }
      }
    } else {
      wave_locate(nbd, start, [&](uint32_t b) { return bsum[(size_t)b * G1 + g]; }, &bstar, &before_b);
    }
  }
  const uint32_t r0 = bstar < nbd ? bstar * DSP_ROWS : m;
  const uint32_t nr = r0 < m ? (m - r0 < (uint32_t)DSP_ROWS ? m - r0 : (uint32_t)DSP_ROWS) : 0u;

  // ---- load round 2 (one vector: unless the window of load round 1 holds the block);
  // lane l holds rows r0 + 4l .. r0 + 4l + 3
  uint32_t lr[4];
  float lv[4];
  bool spec = false;
  if constexpr (BP == 1) spec = bstar == w0 || bstar == w0 + 1u;
  if (spec) {
    const bool second = bstar != w0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      lr[u] = second ? slr[u + 4] : slr[u];
      lv[u] = second ? slv[u + 4] : slv[u];
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t j = 4u * (uint32_t)lane + (uint32_t)u;
      lr[u] = j < nr ? rl[r0 + j] : 0u;
      lv[u] = BP == 1 && j < nr ? vvec[r0 + j] : 0.0f;
    }
  }

  // ---- load round 3: the share's first rows, their chunks in flight
  uint32_t remaining = end - start;
  uint32_t rowb = m, offb = 0;
  if (active) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      mrl[wid][4 * lane + u] = lr[u];
      if (BP == 1) mv[wid][4 * lane + u] = lv[u];
    }
    // the row: one scan over the lanes' sums of four, then lane L's four rows
    // (the first with prefix <= t < prefix + length; zero lengths are passed)
    const uint32_t t = start - before_b;
    const uint32_t s4 = lr[0] + lr[1] + lr[2] + lr[3];
    const uint32_t inc = wave_incl_scan(s4);
    const uint32_t lo4 = inc - s4;
    const unsigned long long hit = __ballot(s4 > 0u && lo4 <= t && t < inc);
    uint32_t jrow = nr, before_r = 0u;
    if (hit) {
      const int L = __ffsll((long long)hit) - 1;
      uint32_t acc = (uint32_t)__builtin_amdgcn_readlane((int)lo4, L);
      uint32_t k = 3u;
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)lr[u], L);
        if (k == 3u) {
          if (t < acc + x) k = (uint32_t)u;
          else acc += x;
        }
      }
      jrow = 4u * (uint32_t)L + k;
      before_r = acc;
    }
    rowb = __builtin_amdgcn_readfirstlane(jrow < nr ? r0 + jrow : m);
    offb = __builtin_amdgcn_readfirstlane(t - before_r);
  }

  // batch state: up to 64 rows from rowb, one per lane
  uint32_t Lj = 0u, aj = 0u, takej = 0u, batch_take = 0u;
  float vj[BP];  // the row's activation in each vector of the pass
  uint32_t pkj[Q8 ? 17 : 1];  // q8: the row's largest key and its probe keys
  unsigned long long todo = 0ull;
  // chunk sequence: row sj of the batch, entries [ss, se) not yet issued
  uint32_t sj = 0u, ss = 0u, se = 0u;

  auto batch_meta = [&]() {
    const uint32_t r = rowb + (uint32_t)lane;
    Lj = 0u;
#pragma unroll
    for (int p = 0; p < BP; ++p) vj[p] = 0.0f;
    if (r < m) {
      if (r >= r0 && r - r0 < nr) {
        Lj = mrl[wid][r - r0];
        if (BP == 1) vj[0] = mv[wid][r - r0];
      } else {
        Lj = rl[r];
        if (BP == 1) vj[0] = vvec[r];
      }
      if (BP > 1)
#pragma unroll
        for (int p = 0; p < BP; ++p)
          if (p < nv) vj[p] = vvec[(size_t)p * a.m + r];
      Lj = (uint32_t)min((int64_t)Lj, a.gstride);  // a run holds gstride units
    }
    if constexpr (Q8) {
      // loaded here, written to the table after the batch's first chunks are
      // in flight
      const bool ok = r < m;
      pkj[0] = ok ? (uint32_t)a.rowmax[r] : 0u;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        pkj[k + 1] = ok && k < a.P ? (uint32_t)a.probes[(size_t)r * (uint32_t)a.P + (uint32_t)k] : 0u;
    }
    aj = lane == 0 ? offb : 0u;
    const uint32_t lenj = Lj > aj ? Lj - aj : 0u;
    const uint32_t incl = wave_incl_scan(lenj);
    const uint32_t excl = incl - lenj;
    takej = excl >= remaining ? 0u : min(lenj, remaining - excl);
    batch_take = min((uint32_t)__builtin_amdgcn_readlane((int)incl, 63), remaining);
    todo = __ballot(takej > 0u);
    sj = 0u;
    ss = 0u;
    se = 0u;
  };
  // Next chunk of the batch: <= chunk_units units of one row.  What depends
  // only on the row -- its run's address, threshold and activation -- is read
  // once when the row starts, not per chunk.  Wave-uniform.
  constexpr uint32_t UW = FMT == EFFORT_ENTRY_R12 ? 3u : FMT == EFFORT_ENTRY_Q8 ? 2u : 1u;  // words per unit
  const uint32_t* srun = entries;
  float stf = 0.0f, svf = 0.0f;
  uint32_t tfj[BP];  // per lane: the row's threshold as fp32 bits (from thresholds())
  uint32_t tj[BP];   // per vector: the row's fp16 key threshold and scaled activation
  float vfj[BP];
  auto take = [&](Chunk& c) {
    if (ss >= se && todo) {
      sj = (uint32_t)(__ffsll((long long)todo) - 1);
      todo &= todo - 1ull;
      ss = (uint32_t)__builtin_amdgcn_readlane((int)aj, sj);
      se = ss + (uint32_t)__builtin_amdgcn_readlane((int)takej, sj);
      const uint32_t row = rowb + sj;
      srun = entries + ((size_t)row * (size_t)a.row_stride + (size_t)g * (size_t)a.gstride) * UW;
      if constexpr (BP == 1) {
        stf = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)tfj[0], sj));
        svf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vfj[0]), sj));
      }
    }
    c.valid = ss < se;
    c.j = sj;
    c.s0 = ss;
    c.run = srun;
    c.tf = stf;
    c.vf = svf;
    // u32: chunk ends on quad boundaries of the run (a share's first chunk
    // in a row may start inside a quad); r12, q8: whole records
    const uint32_t cs = FMT == EFFORT_ENTRY_U32 ? (ss & ~3u) : ss;
    c.s1 = c.valid ? min(se, cs + chunk_units<FMT>()) : 0u;
    ss = c.valid ? c.s1 : ss;
  };
  // Loads the chunk for this lane through a buffer descriptor that starts at
  // unit s0 and ends at s1: lane l reads records s0 + l and s0 + 64 + l
  // (r12, q8) or words from s0 + 4l (u32: four entries).
  // Words past s1 read as zero without a memory access (the range is checked
  // per 4-byte word), so every lane issues the load and the wait counters
  // stay exact; an empty chunk accesses no memory.
  constexpr int RPL = records_per_lane<FMT>();
  auto issue = [&](const Chunk& c, uint4* buf) {
    const uint32_t units = c.valid ? c.s1 - c.s0 : 0u;
    const uint32_t* p0 = c.run + (size_t)c.s0 * UW;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)p0, (short)0, (int)(units * UW * 4u), kBufferDword3);
    if constexpr (FMT == EFFORT_ENTRY_R12) {
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const auto q = __builtin_amdgcn_raw_buffer_load_b96(rs, (64 * r + lane) * 12, 0, 0);
        buf[r] = make_uint4(q[0], q[1], q[2], 0u);
      }
    } else if constexpr (FMT == EFFORT_ENTRY_Q8) {
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const auto q = __builtin_amdgcn_raw_buffer_load_b64(rs, (64 * r + lane) * 8, 0, 0);
        buf[r] = make_uint4(q[0], q[1], 0u, 0u);
      }
    } else {
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, (64 * r + lane) * 16, 0, 0);
        buf[r] = make_uint4(q[0], q[1], q[2], q[3]);
      }
    }
  };
  // sub: which load of the lane (unit 64 sub + lane of the chunk, u32: quad)
  auto process = [&](const Chunk& c, const uint4& buf, int sub) {
    if (!c.valid) return;
    float tf[BP], vf[BP];
    if constexpr (BP == 1) {
      tf[0] = c.tf;
      vf[0] = c.vf;
    } else {
#pragma unroll
      for (int p = 0; p < BP; ++p) {
        tf[p] = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)tfj[p], c.j));
        vf[p] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vfj[p]), c.j));
      }
    }
    // The 4 entries of this lane's load `sub`: fp16 value bits (low half) and
    // the column inside the group; `in` whether they are units of the chunk
    // (words past s1 read as zero).
    uint32_t ev[4], col[4];
    bool entry[4], unit[4];  // an entry of the chunk; a unit of the chunk (pads included)
    if constexpr (FMT == EFFORT_ENTRY_R12) {
      // One record: two words of values, then the first column (12 bits) and
      // three steps (7, 7, 6 bits).  Pads (0x8000, step 0) have key 0.
      ev[0] = buf.x;
      ev[1] = buf.x >> 16;
      ev[2] = buf.y;
      ev[3] = buf.y >> 16;
      col[0] = buf.z & 0xFFFu;
      col[1] = col[0] + ((buf.z >> 12) & 0x7Fu);
      col[2] = col[1] + ((buf.z >> 19) & 0x7Fu);
      col[3] = col[2] + (buf.z >> 26);
      const bool in = (uint32_t)lane + 64u * (uint32_t)sub < c.s1 - c.s0;
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        unit[k2] = in;
        entry[k2] = in && (ev[k2] & 0xFFFFu) != 0x8000u;
      }
    } else if constexpr (FMT == EFFORT_ENTRY_Q8) {
      // One record: a header (segment, entries - 1, first 8-column cell, cell
      // steps of 6, 6 and 5 bits) and one byte per entry (sign, level code,
      // column in the cell).  The level: min(lo + (code << shift), hi) in the
      // bucket of the record's segment.  Unused slots and words past the
      // chunk are not entries: the keep test below excludes them.
      const uint32_t H = buf.x, E = buf.y;
      const bool in = (uint32_t)lane + 64u * (uint32_t)sub < c.s1 - c.s0;
      const uint32_t trow = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.j) * (uint32_t)Q8_ROW_SLOTS;
      const uint32_t last = (H >> 4) & 3u;
      uint32_t cell = (H >> 6) & 511u;
      // the four levels two at a time: the bounds and the codes spread over
      // the 16-bit halves with byte permutes (selector byte 0x0c gives zero),
      // the signs moved to bits 15 and 31 the same way
      uint32_t lohi, sh;
      q8_packed(qtab[wid][trow + (H & 15u)], lohi, sh);
      const uint32_t lo2 = __builtin_amdgcn_perm(0u, lohi, 0x01000100u);
      const uint32_t hi2 = __builtin_amdgcn_perm(0u, lohi, 0x03020302u);
      const uint32_t cw = (E >> 3) & 0x0F0F0F0Fu;
      const uint32_t sw = E & 0x80808080u;
      const uint32_t k01 = q8_levels2(__builtin_amdgcn_perm(0u, cw, 0x0c010c00u), lo2, hi2, sh) |
                           __builtin_amdgcn_perm(0u, sw, 0x010c000cu);
      const uint32_t k23 = q8_levels2(__builtin_amdgcn_perm(0u, cw, 0x0c030c02u), lo2, hi2, sh) |
                           __builtin_amdgcn_perm(0u, sw, 0x030c020cu);
      ev[0] = k01;
      ev[1] = k01 >> 16;
      ev[2] = k23;
      ev[3] = k23 >> 16;
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        if (k2 == 1) cell += (H >> 15) & 63u;
        if (k2 == 2) cell += (H >> 21) & 63u;
        if (k2 == 3) cell += H >> 27;
        unit[k2] = in;
        entry[k2] = in && (uint32_t)k2 <= last;
        col[k2] = (cell << 3) | ((E >> (8 * k2)) & 7u);
      }
    } else {
      ev[0] = buf.x;
      ev[1] = buf.y;
      ev[2] = buf.z;
      ev[3] = buf.w;
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        col[k2] = ev[k2] >> 16;
        entry[k2] = 4u * ((uint32_t)lane + 64u * (uint32_t)sub) + (uint32_t)k2 < c.s1 - c.s0;
        unit[k2] = entry[k2];
      }
    }
    // The keep test and the accumulation are the same with and without
    // recording; recording only adds the stores of the kept (row, column)
    // pairs.  Every slot adds: a kept product, or 0 -- to its own column,
    // or (a word past the chunk, column 0 for all such lanes) to a word of
    // its own lane, so that the zero adds do not all meet at one address.
    // r12, q8: a lane's whole record is in the chunk or past it, and past it
    // every column decodes to 0, so the lane's offset is added once per
    // record (lsub) instead of a select per slot.
    uint32_t cnt[BP];
    uint64_t fp[BP];
#pragma unroll
    for (int p = 0; p < BP; ++p) {
      cnt[p] = 0u;
      fp[p] = 0u;
    }
    const uint32_t lsub = FMT == EFFORT_ENTRY_U32 || unit[0] ? 0u : (uint32_t)lane;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const float x = h2f(ev[k2]);
      const uint32_t addr = FMT == EFFORT_ENTRY_U32 ? (unit[k2] ? col[k2] : (uint32_t)lane) : col[k2];
#pragma unroll
      for (int p = 0; p < BP; ++p) {
        // |w| >= t, exact: the fp16 -> fp32 widening is monotone (q8: the
        // record's unused slots decode to levels, and are not entries)
        const bool keep = (FMT != EFFORT_ENTRY_Q8 || entry[k2]) && fabsf(x) >= tf[p];
        const int32_t add = to_fixed(__fmul_rn(x, vf[p]));
        atomicAdd(&tile[p * a.TW + lsub + addr], keep ? add : 0);
        if constexpr (REC) {
          if (keep && entry[k2]) {
            const uint64_t flat = (uint64_t)(rowb + c.j) * (uint64_t)a.n + (uint64_t)col0 + col[k2];
            if (a.mask) a.mask[(uint64_t)p * (uint64_t)a.m * (uint64_t)a.n + flat] = 1u;
            fp[p] += pair_hash(flat);
            ++cnt[p];
          }
        }
      }
    }
    if constexpr (REC) {
      const uint32_t row = rowb + c.j;
#pragma unroll
      for (int p = 0; p < BP; ++p) {
        uint32_t cn = cnt[p];
        uint32_t flo = (uint32_t)fp[p], fhi = (uint32_t)(fp[p] >> 32);
        for (int sh = 32; sh > 0; sh >>= 1) {
          cn += __shfl_xor(cn, sh, 64);
          const uint32_t olo = __shfl_xor(flo, sh, 64);
          const uint32_t ohi = __shfl_xor(fhi, sh, 64);
          const uint64_t sum = ((uint64_t)fhi << 32 | flo) + ((uint64_t)ohi << 32 | olo);
          flo = (uint32_t)sum;
          fhi = (uint32_t)(sum >> 32);
        }
        if (lane == 0 && p < nv) {
          if (cn && a.row_kept) atomicAdd(&a.row_kept[(size_t)p * a.m + row], (int32_t)cn);
          if (a.fingerprint) atomicAdd(a.fingerprint + p, ((unsigned long long)fhi << 32) | flo);
        }
      }
    }
  };
  auto thresholds = [&]() {
    if constexpr (Q8) {
      // lane l: row rowb + l's buckets; read back by every lane of this wave
      // only (a wave's LDS accesses take effect in order)
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < a.P) q8_make(pkj[k + 1], pkj[k], qtab[wid][lane * Q8_ROW_SLOTS + k]);
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int p = 0; p < BP; ++p) {
      tj[p] = p < nv && Lj ? key_threshold_fast(fabsf(vj[p]), __uint_as_float(sCut[p])) : 0x7C00u;
      tfj[p] = __float_as_uint(h2f(tj[p]));
      // clamped: only a row whose weights are all zero can exceed it, and its
      // products stay 0
      vfj[p] = p < nv ? fminf(fmaxf(ldexpf(vj[p], BP == 1 ? S1 : sS[p]), -0x1p100f), 0x1p100f) : 0.0f;
    }
    // A cropped layout: a row whose largest dropped magnitude reaches its
    // threshold has kept products that are not stored (every row with kept
    // products has a nonzero read length in some group, so some wave sees it).
    if (a.floor) {
      const uint32_t r = rowb + (uint32_t)lane;
      const uint32_t fl = Lj && r < m ? (uint32_t)a.floor[r] : 0u;
#pragma unroll
      for (int p = 0; p < BP; ++p)
        if (__ballot(Lj && fl >= tj[p]) && lane == 0)
          atomicOr(&a.result[(size_t)p * a.vec_ws + RES_FLAGS], FLAG_CROP_REACHED);
    }
  };
  // The ring of chunks in flight (ring_depth).
  constexpr int RING = ring_depth<FMT>();
  Chunk d[RING];
  uint4 q[RING][RPL];
  auto fill = [&]() {
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      take(d[k]);
      issue(d[k], q[k]);
    }
  };
  // The ring is filled before the rows' thresholds are known (their loads
  // overlap the threshold work); the chunks already taken get the row values
  // afterwards.
  auto refresh = [&]() {
    if constexpr (BP == 1) {
#pragma unroll
      for (int k = 0; k < RING; ++k) {
        d[k].tf = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)tfj[0], d[k].j));
        d[k].vf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vfj[0]), d[k].j));
      }
      stf = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)tfj[0], sj));
      svf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vfj[0]), sj));
    }
  };
  // unconditional, so that the wait counters stay exact: a wave without a
  // share (rowb = m, remaining = 0) gets empty chunks that access no memory
  batch_meta();
  fill();
  if (BP == 1) {
    // the cutoff: wave 0 sets the flag unconditionally once sCut[0] is
    // written, so this wait ends
    while (__hip_atomic_load(&sReady, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u)
      __builtin_amdgcn_s_sleep(1);
  }
  thresholds();
  refresh();

  // ---- stream
  while (active && rowb < m) {
    for (;;) {
      bool any = false;
#pragma unroll
      for (int k = 0; k < RING; ++k) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) process(d[k], q[k][r], r);
        take(d[k]);
        issue(d[k], q[k]);
        any = any || d[k].valid;
      }
      if (!any) break;
    }
    remaining -= batch_take;
    rowb += 64u;
    offb = 0u;
    if (remaining == 0u || rowb >= m) break;
    batch_meta();
    fill();
    thresholds();
    refresh();
  }
  __syncthreads();
  // Flush: FU tile words per thread are read before any is used (one LDS
  // wait per round instead of one per word: a group of 3584 columns is one
  // round), then the non-zero ones are added to y.
  constexpr int FU = 8;
  for (int p = 0; p < nv; ++p) {
    const double unscale = ldexp(1.0, -sS[p]);
    for (int c0 = tid; c0 < tw; c0 += MUL_T * FU) {
      int32_t acc[FU];
#pragma unroll
      for (int u = 0; u < FU; ++u) {
        const int c = c0 + u * MUL_T;
        acc[u] = c < tw ? tile[p * a.TW + c] : 0;
      }
#pragma unroll
      for (int u = 0; u < FU; ++u) {
        const int c = c0 + u * MUL_T;
        if (acc[u] != 0) atomicAdd(&y[(size_t)p * a.n + col0 + c], (float)((double)acc[u] * unscale));
      }
    }
  }
}

template <bool REC, int BP, int FMT>
__global__ __launch_bounds__(mul_threads<BP>()) void k_bucketmul(
    const float* __restrict__ vvec, const uint32_t* __restrict__ entries,
    const uint32_t* __restrict__ runlen, const uint32_t* __restrict__ bsum,
    const uint32_t* __restrict__ result, float* __restrict__ y, MulArgs a) {
  bucketmul_body<REC, BP, FMT>(blockIdx.x, gridDim.x, vvec, entries, runlen, bsum, result, y, a);
}

// Several matrices sharing v, one vector each: matrix j owns blocks
// [first[j], first[j + 1]) of the grid.
template <bool REC, int FMT>
__global__ __launch_bounds__(mul_threads<1>()) void k_bucketmul_multi(MulMulti mm) {
  int j = 0;
  for (int k = 1; k < mm.count; ++k)
    if (blockIdx.x >= mm.first[k]) j = k;
  const MulArgs& a = mm.a[j];
  bucketmul_body<REC, 1, FMT>(blockIdx.x - mm.first[j], mm.first[j + 1] - mm.first[j], a.v, a.entries,
                              a.runlen, a.bsum, a.result, a.y, a);
}

// LDS of a workgroup on gfx950; the batched kernel's static LDS (cutoff
// histograms, prefix sums, row staging) stays under kMulStaticLds for 8 vectors.
constexpr size_t kLdsBytes = 160 * 1024;
constexpr size_t kMulStaticLds = 24 * 1024;

// The q8 bucket table of a batched pass (16 waves).
constexpr size_t kQ8PassTable = 16 * 64 * Q8_ROW_SLOTS * sizeof(uint32_t);

// Largest dynamic LDS (the vectors' tiles) a pass of bp vectors may request.
static size_t pass_tile_budget(int bp, int format) {
  const size_t per = (kLdsBytes - kMulStaticLds) / (size_t)bp;  // tile + cutoff histogram
  return (size_t)bp * (per - 2048) - (format == EFFORT_ENTRY_Q8 ? kQ8PassTable : 0);
}

int bucketmul_pass_width(int32_t TW, int32_t batch, int32_t format) {
  if (batch < 2) return 0;
  for (int bp = 8; bp >= 2; bp >>= 1)
    if ((size_t)bp * ((size_t)TW * 4) <= pass_tile_budget(bp, format)) return bp;
  return 0;
}

template <bool REC, int BP, int FMT>
static hipError_t launch_mul_bp(const MulArgs& a, unsigned grid, hipStream_t s) {
  const size_t lds = (size_t)BP * a.TW * sizeof(int32_t);
  if (lds > pass_tile_budget(BP, FMT)) return hipErrorInvalidValue;
  // the attribute is set on every launch: a per-instantiation flag would be
  // per device state, and the call costs no device work
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bucketmul<REC, BP, FMT>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)pass_tile_budget(BP, FMT));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_bucketmul<REC, BP, FMT>), dim3(grid), dim3(mul_threads<BP>()), lds, s, a.v,
                     a.entries, a.runlen, a.bsum, a.result, a.y, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_mul_fmt(const MulArgs& a, bool record, unsigned grid, hipStream_t s,
                                 const EventPair* ev) {
  if (a.nv > 1) {
    if (a.nv > 8) return hipErrorInvalidValue;
    if (record) {
      if (a.nv > 4) return launch_mul_bp<true, 8, FMT>(a, grid, s);
      if (a.nv > 2) return launch_mul_bp<true, 4, FMT>(a, grid, s);
      return launch_mul_bp<true, 2, FMT>(a, grid, s);
    }
    if (a.nv > 4) return launch_mul_bp<false, 8, FMT>(a, grid, s);
    if (a.nv > 2) return launch_mul_bp<false, 4, FMT>(a, grid, s);
    return launch_mul_bp<false, 2, FMT>(a, grid, s);
  }
  if (ev && ev->start && !record)
    hipExtLaunchKernelGGL((k_bucketmul<false, 1, FMT>), dim3(grid), dim3(mul_threads<1>()), 0, s,
                          ev->start, ev->stop, 0, a.v, a.entries, a.runlen, a.bsum, a.result, a.y, a);
  else if (record)
    hipLaunchKernelGGL((k_bucketmul<true, 1, FMT>), dim3(grid), dim3(mul_threads<1>()), 0, s, a.v,
                       a.entries, a.runlen, a.bsum, a.result, a.y, a);
  else
    hipLaunchKernelGGL((k_bucketmul<false, 1, FMT>), dim3(grid), dim3(mul_threads<1>()), 0, s, a.v,
                       a.entries, a.runlen, a.bsum, a.result, a.y, a);
  return hipGetLastError();
}

hipError_t launch_bucketmul(const MulArgs& args, bool record, int blocks_per_group, hipStream_t s,
                            const EventPair* ev) {
  if (blocks_per_group < 1) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(args.G * blocks_per_group);
  MulArgs a = args;
  a.bpg_recip = blocks_per_group >= 2 ? (uint32_t)((1ull << 32) / (uint64_t)blocks_per_group) : 0u;
  if (a.format == EFFORT_ENTRY_R12) return launch_mul_fmt<EFFORT_ENTRY_R12>(a, record, grid, s, ev);
  if (a.format == EFFORT_ENTRY_Q8) return launch_mul_fmt<EFFORT_ENTRY_Q8>(a, record, grid, s, ev);
  return launch_mul_fmt<EFFORT_ENTRY_U32>(a, record, grid, s, ev);
}

hipError_t launch_bucketmul_multi(const MulMulti& mm_in, int count, const int* blocks_per_group,
                                  bool record, hipStream_t s) {
  if (count < 1 || count > EFFORT_MAX_MULTI || !blocks_per_group) return hipErrorInvalidValue;
  MulMulti mm = mm_in;
  uint32_t total = 0;
  for (int j = 0; j < count; ++j) {
    const int bpg = blocks_per_group[j];
    if (bpg < 1 || mm.a[j].nv != 1) return hipErrorInvalidValue;
    mm.a[j].bpg_recip = bpg >= 2 ? (uint32_t)((1ull << 32) / (uint64_t)bpg) : 0u;
    mm.first[j] = total;
    total += (uint32_t)(mm.a[j].G * bpg);
  }
  for (int j = count; j <= EFFORT_MAX_MULTI; ++j) mm.first[j] = total;
  mm.count = count;
  for (int j = 1; j < count; ++j)  // one instantiation per launch: the pairs share a format
    if (mm.a[j].format != mm.a[0].format) return hipErrorInvalidValue;
  const int f = mm.a[0].format;
  const dim3 gr(total), bl(mul_threads<1>());
  if (f == EFFORT_ENTRY_R12) {
    if (record) hipLaunchKernelGGL((k_bucketmul_multi<true, EFFORT_ENTRY_R12>), gr, bl, 0, s, mm);
    else hipLaunchKernelGGL((k_bucketmul_multi<false, EFFORT_ENTRY_R12>), gr, bl, 0, s, mm);
  } else if (f == EFFORT_ENTRY_Q8) {
    if (record) hipLaunchKernelGGL((k_bucketmul_multi<true, EFFORT_ENTRY_Q8>), gr, bl, 0, s, mm);
    else hipLaunchKernelGGL((k_bucketmul_multi<false, EFFORT_ENTRY_Q8>), gr, bl, 0, s, mm);
  } else {
    if (record) hipLaunchKernelGGL((k_bucketmul_multi<true, EFFORT_ENTRY_U32>), gr, bl, 0, s, mm);
    else hipLaunchKernelGGL((k_bucketmul_multi<false, EFFORT_ENTRY_U32>), gr, bl, 0, s, mm);
  }
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
  constexpr int UNR = 1;  // one load in flight per lane measured fastest (4.5 vs 3.9 TB/s at 4)
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

// Dense GEMV over 256-column strips (512 bytes of each row, line aligned)
// with the rows split so that the grid holds about one block per CU: lane l
// of a wave reads 16 bytes (8 fp16) of row l / 32, a wave 2 rows per load,
// UNR loads in flight per lane; 16 waves per block take interleaved rows; the
// partial sums are reduced over the waves and the rows of a load in LDS and
// added to y with one atomic per column and split (y zero-filled first).
// Swept on MI355X (strips of 128/256/512 columns, 2-32 splits, 256-1024
// threads, 1-8 loads in flight): this shape was fastest at 4096x14336,
// 14336x4096 and 4096x4096 (about 19.5 us at the first two without the fill);
// full-height strips of n / 8 / CUs octets, one block per CU without atomics,
// took 24.5 us (128-byte rows) to 43 us (112-byte rows sharing cache lines
// between CUs).
constexpr int DS_T = 1024;
constexpr int DS_W = DS_T / 64;
constexpr int DS_LPR = 32;  // lanes per row: 32 x 16 bytes = 256 columns
template <int UNR>
__global__ __launch_bounds__(DS_T) void k_dense_split(const uint16_t* __restrict__ W,
                                                      const float* __restrict__ v, int64_t m,
                                                      int64_t n, float* __restrict__ y, int64_t rps) {
  constexpr int RPW = 64 / DS_LPR;  // rows per wave load
  __shared__ float red[DS_W][64 * 8 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = lane / DS_LPR, oc = lane % DS_LPR;
  const int64_t col = ((int64_t)blockIdx.x * DS_LPR + oc) * 8;
  const bool ok = col < n;
  const int64_t r0 = (int64_t)blockIdx.y * rps;
  const int64_t r1 = r0 + rps < m ? r0 + rps : m;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
  constexpr int64_t STEP = (int64_t)DS_W * RPW;
  for (int64_t rb = r0 + wave * RPW + rl; rb < r1; rb += STEP * UNR) {
    uint4 q[UNR];
    float vr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t r = rb + u * STEP;
      q[u] = ok && r < r1 ? *reinterpret_cast<const uint4*>(W + r * n + col) : make_uint4(0u, 0u, 0u, 0u);
      vr[u] = r < r1 ? v[r] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const uint32_t qq[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = __builtin_fmaf(vr[u], h2f(qq[k]), acc[2 * k]);
        acc[2 * k + 1] = __builtin_fmaf(vr[u], h2f(qq[k] >> 16), acc[2 * k + 1]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[wave][lane * 8 + k] = acc[k];
  __syncthreads();
  // over the waves: thread t < 512 sums slot t of every wave
  if (tid < 64 * 8) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < DS_W; ++w) t += red[w][tid];
    red[0][tid] = t;
  }
  __syncthreads();
  // over the rows of a wave load: column o * 8 + k of the strip
  if (tid < DS_LPR * 8) {
    const int o = tid >> 3, k = tid & 7;
    float t = 0.0f;
#pragma unroll
    for (int r = 0; r < RPW; ++r) t += red[0][(r * DS_LPR + o) * 8 + k];
    const int64_t c = ((int64_t)blockIdx.x * DS_LPR + o) * 8 + k;
    if (c < n) atomicAdd(&y[c], t);
  }
}

bool dense_split_serves(int64_t n, const uint16_t* W) {
  return (n & 7) == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0;
}

hipError_t launch_dense_split(const uint16_t* W, const float* v, int64_t m, int64_t n, float* y,
                              hipStream_t s) {
  if (!dense_split_serves(n, W)) return hipErrorInvalidValue;
  const int64_t strips = (n + DS_LPR * 8 - 1) / (DS_LPR * 8);
  int64_t splits = 256 / strips;
  const int64_t max_splits = (m + 63) / 64;  // at least 64 rows per split
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  const int64_t rps = (m + splits - 1) / splits;
  hipError_t e = launch_zero_bytes(y, (uint64_t)n * sizeof(float), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dense_split<2>, dim3((unsigned)strips, (unsigned)splits), dim3(DS_T), 0, s, W, v,
                     m, n, y, rps);
  return hipGetLastError();
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

// Vector k's result words at result + k * stride (u32 words): its cutoff to
// cutoff[k], K and K' to K[2k], K[2k + 1]; a reached crop to bit 1 of
// status[k].
__global__ void k_debug_result(const uint32_t* result, uint64_t stride, int count, float* cutoff,
                               int64_t* K, uint32_t* status) {
  const int k = (int)threadIdx.x;
  if (k < count) {
    const uint32_t* r = result + (uint64_t)k * stride;
    if (cutoff) cutoff[k] = __uint_as_float(r[RES_CUTOFF]);
    if (K) {
      K[2 * k] = (int64_t)r[RES_K];
      K[2 * k + 1] = (int64_t)r[RES_KPRIME];
    }
    if (status && (r[RES_FLAGS] & FLAG_CROP_REACHED)) status[k] |= 2u;
  }
}

__global__ void k_check_finite(const float* __restrict__ v, int64_t m, uint32_t* status) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool bad = i < m && (__float_as_uint(v[i]) & 0x7F800000u) == 0x7F800000u;
  if (__ballot(bad) && (threadIdx.x & 63) == 0) atomicOr(status, 1u);
}

hipError_t launch_check_finite(const float* v, int64_t m, uint32_t* status, hipStream_t s) {
  const int64_t blocks = (m + 255) / 256;
  hipLaunchKernelGGL(k_check_finite, dim3((unsigned)blocks), dim3(256), 0, s, v, m, status);
  return hipGetLastError();
}

hipError_t launch_debug_result(const uint32_t* result, uint64_t stride, int count, float* cutoff,
                               int64_t* K, uint32_t* status, hipStream_t s) {
  if (count < 1 || count > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_debug_result, dim3(1), dim3(64), 0, s, result, stride, count, cutoff, K,
                     status);
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

__global__ void k_axpby(const float* __restrict__ a, float ga, const float* __restrict__ b, float gb,
                        int64_t n, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = __fadd_rn(__fmul_rn(ga, a[i]), __fmul_rn(gb, b[i]));
}

hipError_t launch_axpby(const float* a, float ga, const float* b, float gb, int64_t n, float* out,
                        hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_axpby, dim3((unsigned)blocks), dim3(256), 0, s, a, ga, b, gb, n, out);
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

// ---------------------------------------------------------------- allocation-free workspace

// The workspace of effort_matvec_noalloc: a file-scope device array, one copy
// per device, held until the process ends.  Host code never uses the array's
// name as an address (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and is kept per device.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t noalloc_workspace(hipStream_t s, uint8_t** ws) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the words every call expects to find zero start at zero (a fill kernel,
    // stream-ordered before this device's first call)
    e = launch_zero_bytes(p, kNoallocScratchBytes, s);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ws = static_cast<uint8_t*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

}  // namespace effort
