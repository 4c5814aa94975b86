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
//    magnitudes (the post text: with this format part of the smallest-magnitude
//    weights need not be loaded; the author's reply about running
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
//  * format q8 is the bucketed Q8 form of the author's reply to kwikiel: per
//    entry 4 bits of weight, 1 sign bit and 3 bits of position, the 4 weight
//    bits spanning only the bucket's range.  The bucket of an entry is its
//    rank segment k; its range runs from lo = probe k up to hi = probe k - 1
//    (the row's largest magnitude for k = 0) in 16 levels lo + c 2^s, capped
//    at hi, s the smallest shift that reaches hi; the entry keeps its sign
//    and takes the level nearest to its magnitude key (on a tie the upper
//    one).  Since every level lies in [lo, hi] and lo itself is a level, the
//    quantized row has the same probes and largest magnitude, and the key at
//    each rank is a level of that rank's bucket.  The layout is then the one
//    of the quantized row (its own ranking decides segments, crop and floor),
//    each value written as its level code in its segment's bucket.
//    Inside a (row, group, segment) the entries are in column order, 4 to an
//    8-byte record: a header word (segment, entries - 1, the first entry's
//    8-column cell and three cell steps of 6, 6 and 5 bits) and one byte per
//    entry (sign, level, column in the cell).  A cell step that does not fit
//    ends the record early; the header's count marks the rest as unused.
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

// q8: cell steps of the header, per position 1..3 of a record
constexpr uint32_t kCellStepMax[3] = {63u, 63u, 31u};

// Whether column b may follow column a at position k (1..3) of a record.
inline bool joins(int32_t format, int k, uint32_t a, uint32_t b) {
  if (format == EFFORT_ENTRY_Q8) return (b >> 3) - (a >> 3) <= kCellStepMax[k - 1];
  return b - a <= kStepMax[k - 1];
}

inline int64_t count_records(const std::vector<uint32_t>& cols, int32_t format) {
  int64_t r = 0;
  size_t e = 0;
  while (e < cols.size()) {
    int k = 1;
    while (k < 4 && e + k < cols.size() && joins(format, k, cols[e + k - 1], cols[e + k])) ++k;
    e += (size_t)k;
    ++r;
  }
  return r;
}

// A Q8 bucket: magnitude keys lo..hi, level step 2^sh.
struct Q8Bucket {
  uint32_t lo, hi, sh;
};

Q8Bucket q8_bucket(uint32_t lo, uint32_t hi) {
  Q8Bucket b{lo, hi, 0u};
  while ((15u << b.sh) < hi - lo) ++b.sh;
  return b;
}

inline uint32_t q8_level(const Q8Bucket& b, uint32_t c) { return std::min(b.lo + (c << b.sh), b.hi); }

// The code of the level nearest to key x (a tie goes to the larger level),
// found by trying all 16.
uint32_t q8_code(const Q8Bucket& b, uint32_t x) {
  uint32_t best = 0, bl = q8_level(b, 0);
  uint32_t bd = x > bl ? x - bl : bl - x;
  for (uint32_t c = 1; c < 16; ++c) {
    const uint32_t l = q8_level(b, c);
    const uint32_t dd = x > l ? x - l : l - x;
    if (dd < bd || (dd == bd && l > bl)) {
      best = c;
      bl = l;
      bd = dd;
    }
  }
  return best;
}

// The bucket of segment k of a row (probes and rowmax already written).
inline Q8Bucket row_bucket(const uint16_t* probes_row, uint16_t rowmax, int32_t k) {
  return q8_bucket(probes_row[k], k == 0 ? rowmax : probes_row[k - 1]);
}

// The row the layout stores: W's row itself, or (q8) its quantized form in q.
const uint16_t* stored_row(const uint16_t* row, const Geometry& g, std::vector<uint64_t>& tmp,
                           std::vector<uint32_t>& order, std::vector<uint16_t>& q) {
  if (g.format != EFFORT_ENTRY_Q8) return row;
  const int64_t n = g.n;
  rank_row(row, n, tmp, order);
  int64_t r = 0;
  for (int32_t k = 0; k < g.P; ++k) {
    const int64_t end = seg_end(n, g.P, k);
    const uint32_t lo = row[order[end - 1]] & 0x7FFFu;
    const uint32_t hi = row[order[k == 0 ? 0 : seg_end(n, g.P, k - 1) - 1]] & 0x7FFFu;
    const Q8Bucket bk = q8_bucket(lo, hi);
    for (; r < end; ++r) {
      const uint16_t w = row[order[r]];
      q[order[r]] = (uint16_t)((w & 0x8000u) | q8_level(bk, q8_code(bk, w & 0x7FFFu)));
    }
  }
  return q.data();
}

// Packs one (row, group, segment k) list of in-group columns, ascending, into
// q8 records appended to out (2 words each); vals_row is the quantized row,
// whose keys are levels of the segment's bucket.
void pack_q8(const std::vector<uint32_t>& cols, const uint16_t* vals_row, int64_t col0, const Q8Bucket& bk,
             int32_t k, std::vector<uint32_t>* out) {
  size_t e = 0;
  while (e < cols.size()) {
    int cnt = 1;
    while (cnt < 4 && e + cnt < cols.size() && joins(EFFORT_ENTRY_Q8, cnt, cols[e + cnt - 1], cols[e + cnt]))
      ++cnt;
    uint32_t head = (uint32_t)k | ((uint32_t)(cnt - 1) << 4) | ((cols[e] >> 3) << 6);
    uint32_t bytes = 0;
    for (int t = 0; t < cnt; ++t) {
      const uint32_t c = cols[e + t];
      const uint16_t w = vals_row[col0 + c];
      const uint32_t code = q8_code(bk, w & 0x7FFFu);
      bytes |= (((uint32_t)(w >> 15) << 7) | (code << 3) | (c & 7u)) << (8 * t);
      if (t > 0) {
        static const int kShift[3] = {15, 21, 27};
        head |= ((c >> 3) - (cols[e + t - 1] >> 3)) << kShift[t - 1];
      }
    }
    out->push_back(head);
    out->push_back(bytes);
    e += (size_t)cnt;
  }
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
    if (g.format != EFFORT_ENTRY_U32) {
      std::sort(l.begin(), l.end());
      u += count_records(l, g.format);
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
  std::vector<uint16_t> q((size_t)g.n);
  int64_t mx = 0;
  for (int64_t i = r0; i < r1; ++i) {
    rank_row(stored_row(W + i * g.n, g, tmp, order, q), g.n, tmp, order);
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
  std::vector<uint16_t> q((size_t)n);
  for (int64_t i = r0; i < r1; ++i) {
    const uint16_t* row = stored_row(W + i * n, g, tmp, order, q);
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
          } else if (g.format == EFFORT_ENTRY_Q8) {
            std::sort(l.begin(), l.end());
            recs.clear();
            pack_q8(l, row, col0, row_bucket(probes + i * P, rowmax[i], k), k, &recs);
            memcpy(run + (size_t)acc * 2, recs.data(), recs.size() * 4);
            acc += (uint32_t)(recs.size() / 2);
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
  if (format != EFFORT_ENTRY_U32 && format != EFFORT_ENTRY_R12 && format != EFFORT_ENTRY_Q8)
    return EFFORT_EINVAL;
  if (crop == 0) crop = P;
  if (crop < 1 || crop > P) return EFFORT_EINVAL;
  // 12-bit column base (r12), 9-bit cell (q8)
  if (format != EFFORT_ENTRY_U32 && g->TW > 4096) return EFFORT_EUNSUPPORTED;
  if (format == EFFORT_ENTRY_Q8 && P > 16) return EFFORT_EUNSUPPORTED;  // 4-bit segment field
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
    // every run starts on a 128-byte line: 32 units of 4 or 12 bytes, 16 of
    // 8 (TW is a multiple of 64, so the rounded stride stays within it)
    const int64_t a = format == EFFORT_ENTRY_Q8 ? 16 : 32;
    g->gstride = std::min((gs + a - 1) / a * a, (int64_t)g->TW);
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
