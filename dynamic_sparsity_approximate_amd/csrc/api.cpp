// api.cpp -- C ABI of libeffort: argument validation, workspace carving and
// kernel launches.  Every check happens before the first enqueue.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "effort.h"
#include "kernels.hpp"
#include "layout.hpp"

namespace effort {
int prepare_host(const uint16_t* W, int64_t m, int64_t n, int32_t P, int32_t groups, int32_t format,
                 int32_t crop, void* layout, uint64_t layout_bytes, effort_desc* desc_out);
int plan_layout(const uint16_t* W, int64_t m, int64_t n, int32_t P, int32_t groups, int32_t format,
                int32_t crop, Geometry* g);
uint64_t blob_checksum(const void* blob, uint64_t total);
}  // namespace effort

using namespace effort;

namespace {

constexpr int kMaxDevices = 64;
thread_local hipError_t t_last_hip_error = hipSuccess;  // what effort_last_hip_error() reports

// Records a failed HIP status for effort_last_hip_error().
bool hip_failed(hipError_t e) {
  if (e == hipSuccess) return false;
  t_last_hip_error = e;
  return true;
}
// Device property cache (immutable per device; threads may fill it concurrently
// with the same value).
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int status_of(hipError_t e) { return hip_failed(e) ? EFFORT_EHIP : EFFORT_OK; }

bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_desc(const effort_desc* d, Geometry* g) {
  if (!d) return EFFORT_EINVAL;
  if (d->magic != EFFORT_MAGIC || d->version != EFFORT_VERSION) return EFFORT_ECORRUPT;
  if (d->desc_check != desc_check_of(*d)) return EFFORT_ECORRUPT;
  if (!geometry_from_desc(d, g)) return EFFORT_ECORRUPT;
  return EFFORT_OK;
}

bool effort_ok(float e) { return e > 0.0f && e <= 1.0f; }  // false for NaN

// Entry formats the multiply reads.
bool format_supported(const Geometry& g) {
  return g.format == EFFORT_ENTRY_U32 || g.format == EFFORT_ENTRY_R12 || g.format == EFFORT_ENTRY_Q8;
}

uint32_t k_of(float effort, int64_t N) {
  double k = ceil((double)effort * (double)N);
  if (k < 1.0) k = 1.0;
  if (k > (double)N) k = (double)N;
  return (uint32_t)k;
}

// Parity outputs of one vector (or one matrix of a multi-matrix call); every
// pointer may be null.
struct Rec {
  float* cutoff;                    // [1]
  int64_t* K;                       // [2]: K, K'
  int32_t* row_kept;                // [in_dim]
  unsigned long long* fingerprint;  // [1]
  uint8_t* mask;                    // [in_dim][out_dim]
  bool records() const { return row_kept || fingerprint || mask; }
};

// Parity outputs of a call with `count` vectors of one matrix: vector k's at
// cutoff + k, K + 2k, row_kept + k m, fingerprint + k, mask + k m n.
struct DebugOut {
  float* cutoff;
  int64_t* K;
  int32_t* row_kept;
  uint64_t* fingerprint;
  uint8_t* mask;
  uint32_t* status;
  Rec of(const Geometry& g, int32_t k) const {
    Rec r;
    r.cutoff = cutoff ? cutoff + k : nullptr;
    r.K = K ? K + 2 * k : nullptr;
    r.row_kept = row_kept ? row_kept + (uint64_t)k * g.m : nullptr;
    r.fingerprint = fingerprint ? reinterpret_cast<unsigned long long*>(fingerprint) + k : nullptr;
    r.mask = mask ? mask + (uint64_t)k * g.m * g.n : nullptr;
    return r;
  }
};

// Clears a vector's recording outputs (stream-ordered, before the kernels).
hipError_t clear_rec(const Geometry& g, const Rec& r, int32_t count, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (r.row_kept && (e = launch_zero_bytes(r.row_kept, (uint64_t)count * g.m * 4, s)) != hipSuccess)
    return e;
  if (r.fingerprint && (e = launch_zero_bytes(r.fingerprint, (uint64_t)count * 8, s)) != hipSuccess)
    return e;
  if (r.mask && (e = launch_zero_bytes(r.mask, (uint64_t)count * g.m * g.n, s)) != hipSuccess) return e;
  return e;
}

// The three kernels' arguments for one vector and one matrix, its workspace
// slice at `ws`.
struct CallArgs {
  SelectArgs sa;
  DispatchArgs da;
  MulArgs ma;
};

void build_args(const Geometry& g, const uint8_t* layout, const float* v, float effort, float* y,
                uint8_t* ws, CallArgs* c) {
  const WsLayout w = ws_layout(g);
  uint32_t* result = reinterpret_cast<uint32_t*>(ws + w.result);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + w.hist);
  uint32_t* hist2 = reinterpret_cast<uint32_t*>(ws + w.hist2);
  uint32_t* cand = reinterpret_cast<uint32_t*>(ws + w.cand);
  uint32_t* runlen = reinterpret_cast<uint32_t*>(ws + w.runlen);
  uint32_t* bsum = reinterpret_cast<uint32_t*>(ws + w.bsum);
  const uint16_t* probes = reinterpret_cast<const uint16_t*>(layout + g.off_probes);
  const uint32_t* counts = reinterpret_cast<const uint32_t*>(layout + g.off_counts);
  const uint32_t* entries = reinterpret_cast<const uint32_t*>(layout + g.off_entries);
  const uint16_t* rowmax = reinterpret_cast<const uint16_t*>(layout + g.off_rowmax);
  const uint16_t* floor = g.off_floor ? reinterpret_cast<const uint16_t*>(layout + g.off_floor) : nullptr;
  const int64_t N = g.m * (int64_t)g.P;
  const uint32_t K = k_of(effort, N);

  SelectArgs& sa = c->sa;
  sa = SelectArgs();
  sa.v = v;
  sa.probes = probes;
  sa.m = g.m;
  sa.P = g.P;
  sa.N = N;
  sa.hist = hist;
  sa.hist2 = hist2;
  sa.result = result;
  sa.y = y;
  sa.n = g.n;
  sa.bsum = bsum;
  sa.bsum_words = (g.m + kDspRows - 1) / kDspRows * (g.G + 1);
  sa.vec_ws = 0;

  DispatchArgs& da = c->da;
  da = DispatchArgs();
  da.v = v;
  da.probes = probes;
  da.counts = counts;
  da.rowmax = rowmax;
  da.hist = hist;
  da.hist2 = hist2;
  da.cand = cand;
  da.result = result;
  da.runlen = runlen;
  da.bsum = bsum;
  da.m = g.m;
  da.P = g.P;
  da.G = g.G;
  da.G4 = g.G4;
  da.K = K;
  da.vec_ws = 0;

  MulArgs& ma = c->ma;
  ma = MulArgs();
  ma.v = v;
  ma.entries = entries;
  ma.gstride = g.gstride;
  ma.format = g.format;
  ma.floor = floor;
  ma.probes = probes;
  ma.rowmax = rowmax;
  ma.regions = cand_regions(g.P, g.G, g.m) ? 1 : 0;  // launch_dispatch's choice for one matrix
  ma.runlen = runlen;
  ma.bsum = bsum;
  ma.hist = hist;
  ma.hist2 = hist2;
  ma.cand = cand;
  ma.result = result;
  ma.y = y;
  ma.m = g.m;
  ma.n = g.n;
  ma.row_stride = g.row_stride;
  ma.G = g.G;
  ma.TW = g.TW;
  ma.nbd = (int32_t)((g.m + kDspRows - 1) / kDspRows);
  ma.P = g.P;
  ma.K = K;
  ma.nv = 1;
  ma.vec_ws = 0;
  ma.vbsum = bsum;
  ma.row_kept = nullptr;
  ma.fingerprint = nullptr;
  ma.mask = nullptr;
}

// After a failed launch part-way through a call, the workspace words that
// every call expects to find zero (histograms, counters) may be left set:
// they are cleared again (best effort: if launches keep failing, the caller
// must run effort_workspace_init before the next call).
void reset_after_failure(uint8_t* ws, uint64_t bytes, hipStream_t s) {
  (void)launch_zero_bytes(ws, bytes, s);
}

// One vector: select, dispatch, bucketMul on `s`.
int run_one(const Geometry& g, const uint8_t* layout, const float* v, float effort, float* y,
            uint8_t* ws, hipStream_t s, const Rec* rec, uint32_t* status, const EventPair* ev) {
  CallArgs c;
  build_args(g, layout, v, effort, y, ws, &c);
  const uint64_t slice = ws_layout(g).slice;

  if (rec && hip_failed(clear_rec(g, *rec, 1, s))) return EFFORT_EHIP;
  if (status && (hip_failed(launch_zero_bytes(status, 4, s)) ||
                 hip_failed(launch_check_finite(v, g.m, status, s))))
    return EFFORT_EHIP;

  if (hip_failed(launch_select(c.sa, s, ev ? &ev[0] : nullptr))) {
    reset_after_failure(ws, slice, s);
    return EFFORT_EHIP;
  }
  if (hip_failed(launch_dispatch(c.da, s, ev ? &ev[1] : nullptr))) {
    reset_after_failure(ws, slice, s);
    return EFFORT_EHIP;
  }
  MulArgs& ma = c.ma;
  ma.row_kept = rec ? rec->row_kept : nullptr;
  ma.fingerprint = rec ? rec->fingerprint : nullptr;
  ma.mask = rec ? rec->mask : nullptr;
  const bool record = rec && rec->records();
  int bpg = cu_count() / g.G;  // at most one block per CU: a larger grid runs a second round
  if (bpg < 1) bpg = 1;
  if (hip_failed(launch_bucketmul(ma, record, bpg, s, ev ? &ev[2] : nullptr))) {
    reset_after_failure(ws, slice, s);
    return EFFORT_EHIP;
  }
  if (((rec && (rec->cutoff || rec->K)) || status) &&
      hip_failed(launch_debug_result(ma.result, 0, 1, rec ? rec->cutoff : nullptr,
                                     rec ? rec->K : nullptr, status, s)))
    return EFFORT_EHIP;
  return EFFORT_OK;
}

// Several vectors in one pass over the union of their read lengths: cutoff
// and dispatch kernels for all vectors at once, then per pass of up to
// bucketmul_pass_width vectors the union kernel and the multiply.
int run_batched(const Geometry& g, const uint8_t* layout, const float* v, int32_t batch, float effort,
                float* y, uint8_t* ws, hipStream_t s, const DebugOut* dbg) {
  const WsLayout w = ws_layout(g);
  const uint64_t ws_total = w.slice * (uint64_t)batch + w.union_bytes;
  const Rec rec0 = dbg ? dbg->of(g, 0) : Rec{};
  if (dbg && hip_failed(clear_rec(g, rec0, batch, s))) return EFFORT_EHIP;
  const uint64_t vec_ws = w.slice / 4;  // u32 words between consecutive vectors' slices
  const uint16_t* probes = reinterpret_cast<const uint16_t*>(layout + g.off_probes);
  const uint32_t* counts = reinterpret_cast<const uint32_t*>(layout + g.off_counts);
  const uint32_t* entries = reinterpret_cast<const uint32_t*>(layout + g.off_entries);
  const uint16_t* rowmax = reinterpret_cast<const uint16_t*>(layout + g.off_rowmax);
  auto u32 = [&](int32_t b, uint64_t off) {
    return reinterpret_cast<uint32_t*>(ws + (uint64_t)b * w.slice + off);
  };
  const int64_t N = g.m * (int64_t)g.P;
  const uint32_t K = k_of(effort, N);

  SelectArgs sa;
  sa.v = v;
  sa.probes = probes;
  sa.m = g.m;
  sa.P = g.P;
  sa.N = N;
  sa.hist = u32(0, w.hist);
  sa.hist2 = u32(0, w.hist2);
  sa.result = u32(0, w.result);
  sa.y = y;
  sa.n = g.n;
  sa.bsum = u32(0, w.bsum);
  sa.bsum_words = (g.m + kDspRows - 1) / kDspRows * (g.G + 1);
  sa.vec_ws = vec_ws;
  if (hip_failed(launch_select(sa, s, nullptr, batch))) {
    reset_after_failure(ws, ws_total, s);
    return EFFORT_EHIP;
  }

  DispatchArgs da;
  da.v = v;
  da.probes = probes;
  da.counts = counts;
  da.rowmax = rowmax;
  da.hist = u32(0, w.hist);
  da.hist2 = u32(0, w.hist2);
  da.cand = u32(0, w.cand);
  da.result = u32(0, w.result);
  da.runlen = u32(0, w.runlen);
  da.bsum = u32(0, w.bsum);
  da.m = g.m;
  da.P = g.P;
  da.G = g.G;
  da.G4 = g.G4;
  da.K = K;
  da.vec_ws = vec_ws;
  if (hip_failed(launch_dispatch(da, s, nullptr, batch))) {
    reset_after_failure(ws, ws_total, s);
    return EFFORT_EHIP;
  }

  uint32_t* urunlen = reinterpret_cast<uint32_t*>(ws + (uint64_t)batch * w.slice + w.urunlen);
  uint32_t* ubsum = reinterpret_cast<uint32_t*>(ws + (uint64_t)batch * w.slice + w.ubsum);
  const int bp = bucketmul_pass_width(g.TW, batch, g.format);
  int bpg = cu_count() / g.G;  // at most one block per CU: a larger grid runs a second round
  if (bpg < 1) bpg = 1;
  for (int32_t b0 = 0; b0 < batch; b0 += bp) {
    const int32_t nv = batch - b0 < bp ? batch - b0 : bp;
    UnionArgs ua;
    ua.runlen = u32(b0, w.runlen);
    ua.vec_ws = vec_ws;
    ua.nv = nv;
    ua.G = g.G;
    ua.m = g.m;
    ua.urunlen = urunlen;
    ua.ubsum = ubsum;
    if (hip_failed(launch_union(ua, s))) {
      reset_after_failure(ws, ws_total, s);
      return EFFORT_EHIP;
    }

    MulArgs ma;
    ma.v = v + (int64_t)b0 * g.m;
    ma.entries = entries;
    ma.gstride = g.gstride;
    ma.format = g.format;
    ma.floor = g.off_floor ? reinterpret_cast<const uint16_t*>(layout + g.off_floor) : nullptr;
    ma.probes = probes;
    ma.rowmax = rowmax;
    ma.regions = cand_regions(g.P, g.G, g.m) ? 1 : 0;
    ma.runlen = urunlen;
    ma.bsum = ubsum;
    ma.hist = u32(b0, w.hist);
    ma.hist2 = u32(b0, w.hist2);
    ma.cand = u32(b0, w.cand);
    ma.result = u32(b0, w.result);
    ma.y = y + (int64_t)b0 * g.n;
    ma.m = g.m;
    ma.n = g.n;
    ma.row_stride = g.row_stride;
    ma.G = g.G;
    ma.TW = g.TW;
    ma.nbd = (int32_t)((g.m + kDspRows - 1) / kDspRows);
    ma.P = g.P;
    ma.K = K;
    ma.nv = nv;
    ma.vec_ws = vec_ws;
    ma.vbsum = u32(b0, w.bsum);
    const Rec rec = dbg ? dbg->of(g, b0) : Rec{};
    ma.row_kept = rec.row_kept;
    ma.fingerprint = rec.fingerprint;
    ma.mask = rec.mask;
    if (hip_failed(launch_bucketmul(ma, rec.records(), bpg, s))) {
      reset_after_failure(ws, ws_total, s);
      return EFFORT_EHIP;
    }
  }
  if (dbg && (dbg->cutoff || dbg->K) &&
      hip_failed(launch_debug_result(u32(0, w.result), vec_ws, batch, dbg->cutoff, dbg->K, nullptr, s)))
    return EFFORT_EHIP;
  return EFFORT_OK;
}

// Workspace bytes of a multi-matrix call: matrix j's one-vector slice at a
// 256-byte aligned offset.
uint64_t multi_ws_offsets(const Geometry* g, int32_t count, uint64_t* off) {
  uint64_t total = 0;
  for (int32_t j = 0; j < count; ++j) {
    off[j] = total;
    total = align_up(total + ws_layout(g[j]).slice, kAlign);
  }
  return total;
}

int check_multi(const effort_desc* descs, int32_t count, Geometry* g) {
  if (!descs || count < 1 || count > EFFORT_MAX_MULTI) return EFFORT_EINVAL;
  for (int32_t j = 0; j < count; ++j) {
    const int rc = check_desc(&descs[j], &g[j]);
    if (rc) return rc;
  }
  return EFFORT_OK;
}

// One launch serves one entry format: the pairs of a multi-matrix call share it.
int check_multi_formats(const Geometry* g, int32_t count) {
  for (int32_t j = 0; j < count; ++j)
    if (!format_supported(g[j]) || g[j].format != g[0].format) return EFFORT_EUNSUPPORTED;
  return EFFORT_OK;
}

// Several (matrix, vector) pairs -- matrices sharing v, one matrix with
// several vectors, or any mix: each kernel launched once for all of them.
// The multiply's CUs are shared out by output width (the kept bytes of each
// matrix are about proportional to it at one effort), whole blocks per group.
int run_multi(const Geometry* g, int32_t count, const uint8_t* const* layouts,
              const float* const* vs, const float* efforts, float* const* ys, uint8_t* ws,
              const uint64_t* off, hipStream_t s, const Rec* recs) {
  bool record = false;
  if (recs)
    for (int32_t j = 0; j < count; ++j) {
      if (hip_failed(clear_rec(g[j], recs[j], 1, s))) return EFFORT_EHIP;
      record = record || recs[j].records();
    }
  auto fail = [&]() {
    for (int32_t j = 0; j < count; ++j) reset_after_failure(ws + off[j], ws_layout(g[j]).slice, s);
    return EFFORT_EHIP;
  };
  SelectMulti sm;
  DispatchMulti dm;
  MulMulti mm;
  int bpg[EFFORT_MAX_MULTI];
  int64_t ntot = 0;
  for (int32_t j = 0; j < count; ++j) ntot += g[j].n;
  const int cus = cu_count();
  for (int32_t j = 0; j < count; ++j) {
    CallArgs c;
    build_args(g[j], layouts[j], vs[j], efforts[j], ys[j], ws + off[j], &c);
    sm.a[j] = c.sa;
    dm.a[j] = c.da;
    mm.a[j] = c.ma;
    if (recs) {
      mm.a[j].row_kept = recs[j].row_kept;
      mm.a[j].fingerprint = recs[j].fingerprint;
      mm.a[j].mask = recs[j].mask;
    }
    const int64_t share = (int64_t)cus * g[j].n / ntot;
    bpg[j] = (int)(share / g[j].G);
    if (bpg[j] < 1) bpg[j] = 1;
  }
  // a pair the quad dispatch cannot serve sends every pair to the
  // row-per-thread dispatch, whose candidates form one list
  if (!dispatch_multi_quad(dm, count))
    for (int32_t j = 0; j < count; ++j) mm.a[j].regions = 0;
  if (hip_failed(launch_select_multi(sm, count, s))) return fail();
  if (hip_failed(launch_dispatch_multi(dm, count, s))) return fail();
  if (hip_failed(launch_bucketmul_multi(mm, count, bpg, record, s))) return fail();
  if (recs)
    for (int32_t j = 0; j < count; ++j)
      if ((recs[j].cutoff || recs[j].K) &&
          hip_failed(launch_debug_result(mm.a[j].result, 0, 1, recs[j].cutoff, recs[j].K, nullptr, s)))
        return EFFORT_EHIP;
  return EFFORT_OK;
}

// Batches from kUnionMinBatch vectors at an effort of at least
// kUnionMinEffort read the union of the vectors' read lengths once
// (run_batched); other batches run each vector's own multiply, up to four in
// one launch of each kernel.  At 4096x14336 (r12), b = 8 in two launches of
// four against one union pass takes 193 / 167 / 128 / 108 / 92 us against
// 155 / 155 / 144 / 136 / 127 us at effort 1 / 0.75 / 0.5 / 0.35 / 0.25: the
// union pass does every vector's keep test and LDS add for each entry it
// reads, which costs about the same at any effort, so it wins only where
// the vectors' prefixes are long.
constexpr int32_t kUnionMinBatch = 5;
constexpr float kUnionMinEffort = 0.625f;

int matvec_common(const effort_desc* desc, const void* layout_dev, const float* v_dev, int32_t batch,
                  float effort, float* y_dev, void* ws_dev, uint64_t ws_bytes, void* stream,
                  const DebugOut* dbg, void* const* events) {
  Geometry g;
  int rc = check_desc(desc, &g);
  if (rc) return rc;
  if (!layout_dev || !v_dev || !y_dev || !ws_dev) return EFFORT_EINVAL;
  if (!aligned(layout_dev, 256) || !aligned(ws_dev, 256) || !aligned(v_dev, 4) || !aligned(y_dev, 4))
    return EFFORT_EINVAL;
  if (batch < 1 || batch > EFFORT_MAX_BATCH) return EFFORT_EINVAL;
  if (!effort_ok(effort)) return EFFORT_EINVAL;
  if (!format_supported(g)) return EFFORT_EUNSUPPORTED;
  const WsLayout w = ws_layout(g);
  if (ws_bytes < w.slice * (uint64_t)batch + (batch > 1 ? w.union_bytes : 0)) return EFFORT_ENOSPACE;
  if (dbg) {
    if (dbg->K && !aligned(dbg->K, 8)) return EFFORT_EINVAL;
    if (dbg->fingerprint && !aligned(dbg->fingerprint, 8)) return EFFORT_EINVAL;
    if (dbg->row_kept && !aligned(dbg->row_kept, 4)) return EFFORT_EINVAL;
    if (dbg->cutoff && !aligned(dbg->cutoff, 4)) return EFFORT_EINVAL;
    if (dbg->status && !aligned(dbg->status, 4)) return EFFORT_EINVAL;
  }
  EventPair ev[3];
  if (events) {
    for (int k = 0; k < 3; ++k) {
      ev[k].start = static_cast<hipEvent_t>(events[2 * k]);
      ev[k].stop = static_cast<hipEvent_t>(events[2 * k + 1]);
      if (!ev[k].start != !ev[k].stop) return EFFORT_EINVAL;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* layout = static_cast<const uint8_t*>(layout_dev);
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  // a call with parity outputs takes the same route as one without
  if (batch > 1 && !events && batch >= kUnionMinBatch && effort >= kUnionMinEffort &&
      bucketmul_pass_width(g.TW, batch, g.format) > 0)
    return run_batched(g, layout, v_dev, batch, effort, y_dev, ws, s, dbg);
  if (batch > 1 && !events) {
    // up to EFFORT_MAX_MULTI vectors per launch, each its own single-vector
    // multiply over its own read lengths (the slices are the batch's)
    for (int32_t b0 = 0; b0 < batch; b0 += EFFORT_MAX_MULTI) {
      const int32_t cnt = batch - b0 < EFFORT_MAX_MULTI ? batch - b0 : EFFORT_MAX_MULTI;
      Geometry gs[EFFORT_MAX_MULTI];
      const uint8_t* ls[EFFORT_MAX_MULTI];
      const float* vs[EFFORT_MAX_MULTI];
      float* ys[EFFORT_MAX_MULTI];
      float es[EFFORT_MAX_MULTI];
      uint64_t off[EFFORT_MAX_MULTI];
      Rec recs[EFFORT_MAX_MULTI];
      for (int32_t j = 0; j < cnt; ++j) {
        if (dbg) recs[j] = dbg->of(g, b0 + j);
        gs[j] = g;
        ls[j] = layout;
        vs[j] = v_dev + (int64_t)(b0 + j) * g.m;
        ys[j] = y_dev + (int64_t)(b0 + j) * g.n;
        es[j] = effort;
        off[j] = (uint64_t)(b0 + j) * w.slice;
      }
      rc = run_multi(gs, cnt, ls, vs, es, ys, ws, off, s, dbg ? recs : nullptr);
      if (rc) return rc;
    }
    return EFFORT_OK;
  }
  for (int32_t b = 0; b < batch; ++b) {
    const Rec rec = dbg ? dbg->of(g, b) : Rec{};
    rc = run_one(g, layout, v_dev + (int64_t)b * g.m, effort, y_dev + (int64_t)b * g.n,
                 ws + (uint64_t)b * w.slice, s, dbg ? &rec : nullptr, dbg ? dbg->status : nullptr,
                 events ? ev : nullptr);
    if (rc) return rc;
  }
  return EFFORT_OK;
}

}  // namespace

extern "C" {

const char* effort_last_hip_error(void) { return hipGetErrorName(t_last_hip_error); }

const char* effort_strerror(int status) {
  switch (status) {
    case EFFORT_OK: return "ok";
    case EFFORT_EINVAL: return "invalid argument";
    case EFFORT_ENOSPACE: return "buffer too small";
    case EFFORT_EHIP: return "HIP error";
    case EFFORT_EUNSUPPORTED: return "unsupported";
    case EFFORT_ECORRUPT: return "corrupt descriptor or layout";
    default: return "unknown status";
  }
}

int32_t effort_default_groups(int64_t out_dim) { return default_groups(out_dim); }

int effort_layout_bytes_ex(int64_t in_dim, int64_t out_dim, int32_t P, int32_t groups, uint64_t* bytes) {
  if (!bytes) return EFFORT_EINVAL;
  Geometry g;
  int rc = make_geometry(in_dim, out_dim, P, groups, &g);
  if (rc) return rc;
  *bytes = g.total;
  return EFFORT_OK;
}

int effort_layout_bytes(int64_t in_dim, int64_t out_dim, int32_t P, uint64_t* bytes) {
  return effort_layout_bytes_ex(in_dim, out_dim, P, 0, bytes);
}

int effort_workspace_bytes(const effort_desc* desc, int32_t batch, uint64_t* bytes) {
  if (!bytes) return EFFORT_EINVAL;
  Geometry g;
  int rc = check_desc(desc, &g);
  if (rc) return rc;
  if (batch < 1 || batch > EFFORT_MAX_BATCH) return EFFORT_EINVAL;
  const WsLayout w = ws_layout(g);
  *bytes = w.slice * (uint64_t)batch + (batch > 1 ? w.union_bytes : 0);
  return EFFORT_OK;
}

int effort_workspace_bytes_multi(const effort_desc* descs, int32_t count, uint64_t* bytes) {
  if (!bytes) return EFFORT_EINVAL;
  Geometry g[EFFORT_MAX_MULTI];
  const int rc = check_multi(descs, count, g);
  if (rc) return rc;
  uint64_t off[EFFORT_MAX_MULTI];
  *bytes = multi_ws_offsets(g, count, off);
  return EFFORT_OK;
}

int effort_matvec_multi(const effort_desc* descs, const void* const* layouts_dev, int32_t count,
                        const float* const* vs_dev, const float* efforts, float* const* ys_dev,
                        void* ws_dev, uint64_t ws_bytes, void* stream) {
  Geometry g[EFFORT_MAX_MULTI];
  int rc = check_multi(descs, count, g);
  if (rc) return rc;
  if ((rc = check_multi_formats(g, count)) != EFFORT_OK) return rc;
  if (!layouts_dev || !vs_dev || !ys_dev || !efforts || !ws_dev) return EFFORT_EINVAL;
  if (!aligned(ws_dev, 256)) return EFFORT_EINVAL;
  const uint8_t* layouts[EFFORT_MAX_MULTI];
  const float* vs[EFFORT_MAX_MULTI];
  float* ys[EFFORT_MAX_MULTI];
  for (int32_t j = 0; j < count; ++j) {
    if (!effort_ok(efforts[j])) return EFFORT_EINVAL;
    if (!layouts_dev[j] || !vs_dev[j] || !ys_dev[j]) return EFFORT_EINVAL;
    if (!aligned(layouts_dev[j], 256) || !aligned(vs_dev[j], 4) || !aligned(ys_dev[j], 4))
      return EFFORT_EINVAL;
    layouts[j] = static_cast<const uint8_t*>(layouts_dev[j]);
    vs[j] = vs_dev[j];
    ys[j] = ys_dev[j];
  }
  uint64_t off[EFFORT_MAX_MULTI];
  if (ws_bytes < multi_ws_offsets(g, count, off)) return EFFORT_ENOSPACE;
  return run_multi(g, count, layouts, vs, efforts, ys, static_cast<uint8_t*>(ws_dev), off,
                   static_cast<hipStream_t>(stream), nullptr);
}

int effort_matvec_multi_debug(const effort_desc* descs, const void* const* layouts_dev, int32_t count,
                              const float* const* vs_dev, const float* efforts, float* const* ys_dev,
                              void* ws_dev, uint64_t ws_bytes, float* cutoff_dev, int64_t* K_dev,
                              int32_t* const* row_kept_dev, uint64_t* fingerprint_dev, void* stream) {
  Geometry g[EFFORT_MAX_MULTI];
  int rc = check_multi(descs, count, g);
  if (rc) return rc;
  if ((rc = check_multi_formats(g, count)) != EFFORT_OK) return rc;
  if (!layouts_dev || !vs_dev || !ys_dev || !efforts || !ws_dev) return EFFORT_EINVAL;
  if (!aligned(ws_dev, 256)) return EFFORT_EINVAL;
  if ((cutoff_dev && !aligned(cutoff_dev, 4)) || (K_dev && !aligned(K_dev, 8)) ||
      (fingerprint_dev && !aligned(fingerprint_dev, 8)))
    return EFFORT_EINVAL;
  const uint8_t* layouts[EFFORT_MAX_MULTI];
  const float* vs[EFFORT_MAX_MULTI];
  float* ys[EFFORT_MAX_MULTI];
  Rec recs[EFFORT_MAX_MULTI];
  for (int32_t j = 0; j < count; ++j) {
    if (!effort_ok(efforts[j])) return EFFORT_EINVAL;
    if (!layouts_dev[j] || !vs_dev[j] || !ys_dev[j]) return EFFORT_EINVAL;
    if (!aligned(layouts_dev[j], 256) || !aligned(vs_dev[j], 4) || !aligned(ys_dev[j], 4))
      return EFFORT_EINVAL;
    int32_t* rk = row_kept_dev ? row_kept_dev[j] : nullptr;
    if (rk && !aligned(rk, 4)) return EFFORT_EINVAL;
    layouts[j] = static_cast<const uint8_t*>(layouts_dev[j]);
    vs[j] = vs_dev[j];
    ys[j] = ys_dev[j];
    recs[j].cutoff = cutoff_dev ? cutoff_dev + j : nullptr;
    recs[j].K = K_dev ? K_dev + 2 * j : nullptr;
    recs[j].row_kept = rk;
    recs[j].fingerprint =
        fingerprint_dev ? reinterpret_cast<unsigned long long*>(fingerprint_dev) + j : nullptr;
    recs[j].mask = nullptr;
  }
  uint64_t off[EFFORT_MAX_MULTI];
  if (ws_bytes < multi_ws_offsets(g, count, off)) return EFFORT_ENOSPACE;
  return run_multi(g, count, layouts, vs, efforts, ys, static_cast<uint8_t*>(ws_dev), off,
                   static_cast<hipStream_t>(stream), recs);
}

int effort_workspace_init(void* ws_dev, uint64_t ws_bytes, void* stream) {
  if (!ws_dev || !aligned(ws_dev, 256)) return EFFORT_EINVAL;
  return status_of(launch_zero_bytes(ws_dev, ws_bytes, static_cast<hipStream_t>(stream)));
}

int effort_prepare_host_ex(const uint16_t* w_fp16, int64_t in_dim, int64_t out_dim, int32_t P,
                           int32_t groups, void* layout_host, uint64_t layout_bytes,
                           effort_desc* desc_out) {
  return prepare_host(w_fp16, in_dim, out_dim, P, groups, EFFORT_ENTRY_U32, P, layout_host,
                      layout_bytes, desc_out);
}

int effort_prepare_host(const uint16_t* w_fp16, int64_t in_dim, int64_t out_dim, int32_t P,
                        void* layout_host, uint64_t layout_bytes, effort_desc* desc_out) {
  return prepare_host(w_fp16, in_dim, out_dim, P, 0, EFFORT_ENTRY_U32, P, layout_host, layout_bytes,
                      desc_out);
}

int effort_layout_bytes_opts(const uint16_t* w_fp16, int64_t in_dim, int64_t out_dim, int32_t P,
                             const effort_prepare_opts* opts, uint64_t* bytes) {
  if (!opts || !bytes) return EFFORT_EINVAL;
  Geometry g;
  const int rc = plan_layout(w_fp16, in_dim, out_dim, P, opts->groups, opts->entry_format,
                             opts->crop_segments, &g);
  if (rc) return rc;
  *bytes = g.total;
  return EFFORT_OK;
}

int effort_prepare_host_opts(const uint16_t* w_fp16, int64_t in_dim, int64_t out_dim, int32_t P,
                             const effort_prepare_opts* opts, void* layout_host,
                             uint64_t layout_bytes, effort_desc* desc_out) {
  if (!opts) return EFFORT_EINVAL;
  return prepare_host(w_fp16, in_dim, out_dim, P, opts->groups, opts->entry_format,
                      opts->crop_segments, layout_host, layout_bytes, desc_out);
}

int effort_prepare(const uint16_t* w_fp16_host, int64_t in_dim, int64_t out_dim, int32_t P,
                   void* layout_dev, uint64_t layout_bytes, effort_desc* desc_out, void* stream) {
  if (!w_fp16_host || !layout_dev || !desc_out || !aligned(layout_dev, 256)) return EFFORT_EINVAL;
  Geometry g;
  int rc = make_geometry(in_dim, out_dim, P, 0, &g);
  if (rc) return rc;
  if (layout_bytes < g.total) return EFFORT_ENOSPACE;
  void* tmp = aligned_alloc(256, (size_t)g.total);
  if (!tmp) return EFFORT_ENOSPACE;
  rc = prepare_host(w_fp16_host, in_dim, out_dim, P, 0, EFFORT_ENTRY_U32, P, tmp, g.total, desc_out);
  if (!rc) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hip_failed(hipMemcpyAsync(layout_dev, tmp, (size_t)g.total, hipMemcpyHostToDevice, s)) ||
        hip_failed(hipStreamSynchronize(s)))
      rc = EFFORT_EHIP;
  }
  free(tmp);
  return rc;
}

int effort_layout_check(const effort_desc* desc, const void* layout_host) {
  Geometry g;
  int rc = check_desc(desc, &g);
  if (rc) return rc;
  if (!layout_host || !aligned(layout_host, 8)) return EFFORT_EINVAL;
  if (memcmp(layout_host, desc, sizeof *desc) != 0) return EFFORT_ECORRUPT;
  if (blob_checksum(layout_host, g.total) != desc->checksum) return EFFORT_ECORRUPT;
  return EFFORT_OK;
}

int effort_matvec(const effort_desc* desc, const void* layout_dev, const float* v_dev, float effort,
                  float* y_dev, void* ws_dev, uint64_t ws_bytes, void* stream) {
  return matvec_common(desc, layout_dev, v_dev, 1, effort, y_dev, ws_dev, ws_bytes, stream, nullptr,
                       nullptr);
}

int effort_matvec_noalloc(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                          float effort, float* y_dev, void* stream) {
  Geometry g;
  int rc = check_desc(desc, &g);
  if (rc) return rc;
  if (!layout_dev || !v_dev || !y_dev) return EFFORT_EINVAL;
  if (!aligned(layout_dev, 256) || !aligned(v_dev, 4) || !aligned(y_dev, 4)) return EFFORT_EINVAL;
  if (!effort_ok(effort)) return EFFORT_EINVAL;
  if (!format_supported(g)) return EFFORT_EUNSUPPORTED;
  const uint64_t need = ws_layout(g).slice;
  if (need > kNoallocScratchBytes) return EFFORT_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = nullptr;
  if (hip_failed(noalloc_workspace(s, &ws))) return EFFORT_EHIP;
  return matvec_common(desc, layout_dev, v_dev, 1, effort, y_dev, ws, need, stream, nullptr, nullptr);
}

int effort_matvec_batched(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                          int32_t batch, float effort, float* y_dev, void* ws_dev, uint64_t ws_bytes,
                          void* stream) {
  return matvec_common(desc, layout_dev, v_dev, batch, effort, y_dev, ws_dev, ws_bytes, stream,
                       nullptr, nullptr);
}

int effort_matvec_debug(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                        float effort, float* y_dev, void* ws_dev, uint64_t ws_bytes,
                        float* cutoff_dev, int64_t* K_dev, int32_t* row_kept_dev,
                        uint64_t* fingerprint_dev, uint8_t* kept_mask_dev, uint32_t* status_dev,
                        void* stream) {
  DebugOut d{cutoff_dev, K_dev, row_kept_dev, fingerprint_dev, kept_mask_dev, status_dev};
  return matvec_common(desc, layout_dev, v_dev, 1, effort, y_dev, ws_dev, ws_bytes, stream, &d,
                       nullptr);
}

int effort_matvec_batched_debug(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                                int32_t batch, float effort, float* y_dev, void* ws_dev,
                                uint64_t ws_bytes, float* cutoff_dev, int64_t* K_dev,
                                int32_t* row_kept_dev, uint64_t* fingerprint_dev,
                                uint8_t* kept_mask_dev, void* stream) {
  DebugOut d{cutoff_dev, K_dev, row_kept_dev, fingerprint_dev, kept_mask_dev, nullptr};
  return matvec_common(desc, layout_dev, v_dev, batch, effort, y_dev, ws_dev, ws_bytes, stream, &d,
                       nullptr);
}

int effort_matvec_timed(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                        float effort, float* y_dev, void* ws_dev, uint64_t ws_bytes, void* stream,
                        void* const* events) {
  if (stream_capturing(static_cast<hipStream_t>(stream))) return EFFORT_EUNSUPPORTED;
  return matvec_common(desc, layout_dev, v_dev, 1, effort, y_dev, ws_dev, ws_bytes, stream, nullptr,
                       events);
}

int dense_gemv(const uint16_t* w_dev, const float* v_dev, int64_t in_dim, int64_t out_dim,
               float* y_dev, void* stream) {
  if (!w_dev || !v_dev || !y_dev || in_dim < 1 || out_dim < 1) return EFFORT_EINVAL;
  if (!aligned(w_dev, 2) || !aligned(v_dev, 4) || !aligned(y_dev, 4)) return EFFORT_EINVAL;
  const int cus = cu_count();
  if (dense_split_serves(out_dim, w_dev))
    return status_of(launch_dense_split(w_dev, v_dev, in_dim, out_dim, y_dev,
                                        static_cast<hipStream_t>(stream)));
  const int64_t strips = (out_dim + 63) / 64;
  int rs = 1;
  if (strips < cus) {
    int64_t want = (2 * cus + strips - 1) / strips;
    int64_t cap = (in_dim + 255) / 256;
    rs = (int)(want < cap ? want : cap);
    if (rs < 1) rs = 1;
  }
  return status_of(launch_dense_gemv(w_dev, v_dev, in_dim, out_dim, y_dev, 8, rs,
                           static_cast<hipStream_t>(stream)));
}

int dense_gemm_small(const uint16_t* w_dev, const float* v_dev, int32_t batch, int64_t in_dim,
                     int64_t out_dim, float* y_dev, void* stream) {
  if (!w_dev || !v_dev || !y_dev || in_dim < 1 || out_dim < 1) return EFFORT_EINVAL;
  if (batch < 1 || batch > EFFORT_MAX_BATCH) return EFFORT_EINVAL;
  if (!aligned(w_dev, 2) || !aligned(v_dev, 4) || !aligned(y_dev, 4)) return EFFORT_EINVAL;
  return status_of(launch_dense_gemm_small(w_dev, v_dev, batch, in_dim, out_dim, y_dev,
                                 static_cast<hipStream_t>(stream)));
}

int effort_silu_mul(const float* h1_dev, const float* h3_dev, int64_t n, float* out_dev, void* stream) {
  if (!h1_dev || !h3_dev || !out_dev || n < 1) return EFFORT_EINVAL;
  if (!aligned(h1_dev, 4) || !aligned(h3_dev, 4) || !aligned(out_dev, 4)) return EFFORT_EINVAL;
  return status_of(launch_silu_mul(h1_dev, h3_dev, n, out_dev, static_cast<hipStream_t>(stream)));
}

int effort_axpby(const float* a_dev, float ga, const float* b_dev, float gb, int64_t n, float* out_dev,
                 void* stream) {
  if (!a_dev || !b_dev || !out_dev || n < 1) return EFFORT_EINVAL;
  if (!aligned(a_dev, 4) || !aligned(b_dev, 4) || !aligned(out_dev, 4)) return EFFORT_EINVAL;
  return status_of(launch_axpby(a_dev, ga, b_dev, gb, n, out_dev, static_cast<hipStream_t>(stream)));
}

int effort_event_create(void** event_out) {
  if (!event_out) return EFFORT_EINVAL;
  hipEvent_t e;
  if (hip_failed(hipEventCreate(&e))) return EFFORT_EHIP;
  *event_out = e;
  return EFFORT_OK;
}

int effort_event_record(void* event, void* stream) {
  if (!event) return EFFORT_EINVAL;
  return status_of(hipEventRecord(static_cast<hipEvent_t>(event), static_cast<hipStream_t>(stream)));
}

int effort_event_elapsed_ms(void* start, void* end, float* ms_out) {
  if (!start || !end || !ms_out) return EFFORT_EINVAL;
  if (hip_failed(hipEventSynchronize(static_cast<hipEvent_t>(end)))) return EFFORT_EHIP;
  return status_of(hipEventElapsedTime(ms_out, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(end)));
}

int effort_event_destroy(void* event) {
  if (!event) return EFFORT_EINVAL;
  return status_of(hipEventDestroy(static_cast<hipEvent_t>(event)));
}

int effort_stream_synchronize(void* stream) {
  return status_of(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
}

}  // extern "C"
