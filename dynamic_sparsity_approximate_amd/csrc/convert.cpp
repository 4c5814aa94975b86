// convert.cpp -- offline converter: fp16 W[in][out] -> the layout blob.
//
// This is the "precompute" of the method (HN thread "Show HN: Speeding up LLM
// inference 2x times (possibly)", the quoted pseudocode in the exchange with
// gcy): the stored matrix has one row per input element; each row keeps its
// weights sorted by magnitude descending (the author's reply to
// bigcat12345678), cut into P rank segments whose smallest magnitudes are the
// probes (the 16-part row split in the reply to marmaduke).  The row is further
// split by output-column group so that a GPU workgroup can own one group's
// slice of y.
//
// Options:
//  * crop c < P stores only segments 0..c-1 of every row, the largest
//    magnitudes (the post text: the data format lets one skip a share of the
//    least important weights when loading; the author's reply about running
//    Mixtral from the top ~70 % of its weights).  Probes and rowmax still come
//    from the whole row, so the cutoff is the uncropped one; per row the
//    largest magnitude left out is kept ("floor") so that a call can tell when
//    its kept set would reach into the dropped part.
//  * format r12 stores 3 bytes per entry instead of 4 (the author's reply to
//    kwikiel weighs the bits an entry spends on its position against what its
//    bucket already tells): inside a (row, group, segment) the entries are put
//    in column order -- the keep test is per entry, so the order inside a
//    segment is free -- and packed 4 to a 12-byte record: two words of fp16
//    values, then a 12-bit column and three column steps of 7, 7 and 6 bits.
//    A step that does not fit ends the record early; unused slots are pads
//    (value 0x8000, step 0).  A stored -0.0 weight becomes +0.0 so that a pad
//    is never a weight (|-0| = |+0|: the kept set and the sums are unchanged).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "effort.h"
#include "layout.hpp"

namespace effort {

namespace {

constexpr uint16_t kPad = 0x8000u;
constexpr uint32_t kStepMax[3] = {127u, 127u, 63u};

// One row in rank order: order[r] = column of rank r + 1.
void rank_row(const uint16_t* row, int64_t n, std::vector<uint64_t>& tmp, std::vector<uint32_t>& order) {
  for (int64_t j = 0; j < n; ++j)
    tmp[j] = ((uint64_t)(0x7FFFu - (row[j] & 0x7FFFu)) << 32) | (uint64_t)j;
  std::sort(tmp.begin(), tmp.begin() + n);
  for (int64_t j = 0; j < n; ++j) order[j] = (uint32_t)(tmp[j] & 0xFFFFFFFFu);
}

// Rank (1-based) that closes segment k.
inline int64_t seg_end(int64_t n, int32_t P, int32_t k) { return ((int64_t)(k + 1) * n + P - 1) / P; }

// Packs one (row, group, segment) list of in-group columns, ascending, into
// r12 records appended to out (3 words each); vals[c] = the weight bits.
void pack_records(const std::vector<uint32_t>& cols, const uint16_t* vals_row, int64_t col0,
                  std::vector<uint32_t>* out) {
  size_t e = 0;
  while (e < cols.size()) {
    uint16_t v[4] = {kPad, kPad, kPad, kPad};
    uint32_t c[4];
    c[0] = cols[e];
    uint16_t b = vals_row[col0 + c[0]];
    v[0] = b == 0x8000u ? 0u : b;
    int k = 1;
    while (k < 4 && e + k < cols.size() && cols[e + k] - cols[e + k - 1] <= kStepMax[k - 1]) {
      c[k] = cols[e + k];
      b = vals_row[col0 + c[k]];
      v[k] = b == 0x8000u ? 0u : b;
      ++k;
    }
    for (int t = k; t < 4; ++t) c[t] = c[t - 1];  // pads: step 0
    out->push_back((uint32_t)v[0] | ((uint32_t)v[1] << 16));
    out->push_back((uint32_t)v[2] | ((uint32_t)v[3] << 16));
    out->push_back(c[0] | ((c[1] - c[0]) << 12) | ((c[2] - c[1]) << 19) | ((c[3] - c[2]) << 26));
    e += (size_t)k;
  }
}

inline int64_t count_records(const std::vector<uint32_t>& cols) {
  int64_t r = 0;
  size_t e = 0;
  while (e < cols.size()) {
    int k = 1;
    while (k < 4 && e + k < cols.size() && cols[e + k] - cols[e + k - 1] <= kStepMax[k - 1]) ++k;
    e += (size_t)k;
    ++r;
  }
  return r;
}

// Per (group, segment < crop): the in-group columns of the row's entries in
// that segment (rank order; the caller sorts them for r12).
void split_row(const std::vector<uint32_t>& order, const Geometry& g,
               std::vector<std::vector<uint32_t>>& lists) {
  for (auto& l : lists) l.clear();
  int32_t k = 0;
  int64_t end = seg_end(g.n, g.P, 0);
  const int64_t stored = seg_end(g.n, g.P, g.crop - 1);
  for (int64_t r = 1; r <= stored; ++r) {
    while (r > end) end = seg_end(g.n, g.P, ++k);
    const uint32_t j = order[r - 1];
    const int32_t grp = (int32_t)(j / (uint32_t)g.TW);
    lists[(size_t)grp * g.P + k].push_back(j - (uint32_t)grp * (uint32_t)g.TW);
  }
}

// Units of the (row, group) run of each group.
int64_t run_units(const Geometry& g, std::vector<std::vector<uint32_t>>& lists, int32_t grp) {
  int64_t u = 0;
  for (int32_t k = 0; k < g.crop; ++k) {
    auto& l = lists[(size_t)grp * g.P + k];
    if (g.format == EFFORT_ENTRY_R12) {
      std::sort(l.begin(), l.end());
      u += count_records(l);
    } else {
      u += (int64_t)l.size();
    }
  }
  return u;
}

// Pass 1: the longest run over rows and groups.
void max_run_rows(const uint16_t* W, const Geometry& g, int64_t r0, int64_t r1, int64_t* out) {
  std::vector<uint64_t> tmp((size_t)g.n);
  std::vector<uint32_t> order((size_t)g.n);
  std::vector<std::vector<uint32_t>> lists((size_t)g.G * g.P);
  int64_t mx = 0;
  for (int64_t i = r0; i < r1; ++i) {
    rank_row(W + i * g.n, g.n, tmp, order);
    split_row(order, g, lists);
    for (int32_t grp = 0; grp < g.G; ++grp) mx = std::max(mx, run_units(g, lists, grp));
  }
  *out = mx;
}

// Pass 2: fill the rows' probes, counts, runs, rowmax and floor.
void convert_rows(const uint16_t* W, const Geometry& g, uint8_t* blob, int64_t r0, int64_t r1) {
  const int64_t n = g.n;
  const int32_t P = g.P, G = g.G;
  uint16_t* probes = reinterpret_cast<uint16_t*>(blob + g.off_probes);
  uint32_t* counts = reinterpret_cast<uint32_t*>(blob + g.off_counts);
  uint32_t* entries = reinterpret_cast<uint32_t*>(blob + g.off_entries);
  uint16_t* rowmax = reinterpret_cast<uint16_t*>(blob + g.off_rowmax);
  uint16_t* floor = g.off_floor ? reinterpret_cast<uint16_t*>(blob + g.off_floor) : nullptr;
  const int32_t uw = unit_words(g.format);
  std::vector<uint64_t> tmp((size_t)n);
  std::vector<uint32_t> order((size_t)n);
  std::vector<std::vector<uint32_t>> lists((size_t)G * P);
  std::vector<uint32_t> recs;
  for (int64_t i = r0; i < r1; ++i) {
    const uint16_t* row = W + i * n;
    rank_row(row, n, tmp, order);
    rowmax[i] = (uint16_t)(row[order[0]] & 0x7FFFu);
    for (int32_t k = 0; k < P; ++k) probes[i * P + k] = (uint16_t)(row[order[seg_end(n, P, k) - 1]] & 0x7FFFu);
    if (floor) {
      const int64_t stored = seg_end(n, P, g.crop - 1);
      floor[i] = stored < n ? (uint16_t)(row[order[stored]] & 0x7FFFu) : 0u;
    }
    split_row(order, g, lists);
    uint32_t* crow = counts + (size_t)i * P * g.G4;
    for (int32_t grp = 0; grp < G; ++grp) {
      uint32_t* run = entries + ((size_t)i * g.row_stride + (size_t)grp * g.gstride) * uw;
      const int64_t col0 = (int64_t)grp * g.TW;
      uint32_t acc = 0;
      for (int32_t k = 0; k < P; ++k) {
        if (k < g.crop) {
          auto& l = lists[(size_t)grp * P + k];
          if (g.format == EFFORT_ENTRY_R12) {
            std::sort(l.begin(), l.end());
            recs.clear();
            pack_records(l, row, col0, &recs);
            memcpy(run + (size_t)acc * 3, recs.data(), recs.size() * 4);
            acc += (uint32_t)(recs.size() / 3);
          } else {  // rank order: the list is already in it
            for (uint32_t c : l) run[acc++] = (uint32_t)row[col0 + c] | (c << 16);
          }
        }
        crow[(size_t)k * g.G4 + grp] = acc;  // constant past the crop
      }
    }
  }
}

int fill_desc(const Geometry& g, effort_desc* d) {
  memset(d, 0, sizeof *d);
  d->magic = EFFORT_MAGIC;
  d->version = EFFORT_VERSION;
  d->in_dim = g.m;
  d->out_dim = g.n;
  d->probes_per_row = g.P;
  d->groups = g.G;
  d->group_width = g.TW;
  d->index_bytes = g.format == EFFORT_ENTRY_U32 ? 2 : 0;
  d->row_stride = g.row_stride;
  d->group_stride = g.gstride;
  d->entry_format = g.format;
  d->crop_segments = g.crop;
  d->off_probes = g.off_probes;
  d->off_counts = g.off_counts;
  d->off_entries = g.off_entries;
  d->off_rowmax = g.off_rowmax;
  d->off_floor = g.off_floor;
  d->total_bytes = g.total;
  return EFFORT_OK;
}

unsigned thread_count(int64_t m) {
  unsigned nt = std::thread::hardware_concurrency();
  if (nt < 1) nt = 1;
  if (nt > 16) nt = 16;
  if ((int64_t)nt > m) nt = (unsigned)m;
  return nt;
}

}  // namespace

uint64_t blob_checksum(const void* blob, uint64_t total) {
  const uint64_t* w = reinterpret_cast<const uint64_t*>(static_cast<const uint8_t*>(blob) + kAlign);
  return fnv1a64_words(w, (total - kAlign) / 8);
}

// The geometry of W's layout with the given options (a pass over W when the
// runs' length depends on the data).
int plan_layout(const uint16_t* W, int64_t m, int64_t n, int32_t P, int32_t groups, int32_t format,
                int32_t crop, Geometry* g) {
  if (!W) return EFFORT_EINVAL;
  int rc = make_geometry(m, n, P, groups, g);
  if (rc) return rc;
  if (format != EFFORT_ENTRY_U32 && format != EFFORT_ENTRY_R12) return EFFORT_EINVAL;
  if (crop == 0) crop = P;
  if (crop < 1 || crop > P) return EFFORT_EINVAL;
  if (format == EFFORT_ENTRY_R12 && g->TW > 4096) return EFFORT_EUNSUPPORTED;  // 12-bit column base
  // the method is defined on finite weights
  const int64_t total = m * n;
  for (int64_t e = 0; e < total; ++e)
    if ((W[e] & 0x7C00u) == 0x7C00u) return EFFORT_EINVAL;
  g->format = format;
  g->crop = crop;
  if (format != EFFORT_ENTRY_U32 || crop < P) {
    const unsigned nt = thread_count(m);
    std::vector<int64_t> mx(nt, 0);
    std::vector<std::thread> pool;
    for (unsigned t = 0; t < nt; ++t)
      pool.emplace_back(max_run_rows, W, std::cref(*g), m * t / nt, m * (t + 1) / nt, &mx[t]);
    for (auto& th : pool) th.join();
    int64_t gs = 1;
    for (int64_t x : mx) gs = std::max(gs, x);
    g->gstride = gs;
  }
  place_regions(g);
  return EFFORT_OK;
}

int prepare_host(const uint16_t* W, int64_t m, int64_t n, int32_t P, int32_t groups, int32_t format,
                 int32_t crop, void* layout, uint64_t layout_bytes, effort_desc* desc_out) {
  if (!W || !layout || !desc_out) return EFFORT_EINVAL;
  if (reinterpret_cast<uintptr_t>(layout) % 8) return EFFORT_EINVAL;
  Geometry g;
  int rc = plan_layout(W, m, n, P, groups, format, crop, &g);
  if (rc) return rc;
  if (layout_bytes < g.total) return EFFORT_ENOSPACE;
  uint8_t* blob = static_cast<uint8_t*>(layout);
  memset(blob, 0, (size_t)g.total);
  const unsigned nt = thread_count(m);
  std::vector<std::thread> pool;
  for (unsigned t = 0; t < nt; ++t)
    pool.emplace_back(convert_rows, W, std::cref(g), blob, m * t / nt, m * (t + 1) / nt);
  for (auto& th : pool) th.join();
  effort_desc d;
  fill_desc(g, &d);
  d.checksum = blob_checksum(blob, g.total);
  d.desc_check = desc_check_of(d);
  memcpy(blob, &d, sizeof d);
  *desc_out = d;
  return EFFORT_OK;
}

}  // namespace effort
