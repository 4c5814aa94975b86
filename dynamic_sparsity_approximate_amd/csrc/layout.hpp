// layout.hpp -- geometry of the prepared weight layout and of the workspace.
//
// Layout blob (all offsets 256-byte aligned):
//   [0, 256)        copy of the effort_desc
//   probes          u16 [m][P]      fp16 magnitude bits at ranks ceil((k+1) n / P)
//   counts          u32 [m][P][G4]  cumulative units of group g in rank segments 0..k
//                                   (G4 = G rounded up to 4, so a (row, segment) slice
//                                   is 16-byte aligned); constant from segment crop - 1 on
//   entries         units [m][G][gstride]
//                                   per row, per group, the group's entries of the stored
//                                   segments, segment by segment.  Format u32: one unit
//                                   = one 32-bit entry, low 16 bits the fp16 value bits,
//                                   high 16 bits the column inside the group, rank order
//                                   inside a segment.  Format r12: one unit = a record of
//                                   three 32-bit words holding 4 entries of one segment
//                                   in column order; format q8: a record of 2 words,
//                                   a header and 4 one-byte Q8 entries of one segment
//                                   in column order (see the converter).
//   rowmax          u16 [m]         largest magnitude key of each row
//   floor           u16 [m]         (cropped layouts) largest magnitude key of the
//                                   entries not stored
//
// Rank order is |w| descending, ties by column ascending.  Segment k of a row is
// ranks (ceil(k n / P), ceil((k+1) n / P)]; its smallest magnitude is probe k.
// Because a group's entries are stored segment by segment in rank order, the
// entries of one row and group that can pass the keep test lie in a prefix of
// its run, and the counts table bounds that prefix by whole segments.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "effort.h"

namespace effort {

constexpr uint64_t kAlign = 256;
constexpr int32_t kTargetGroupWidth = 4096;

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

struct Geometry {
  int64_t m = 0, n = 0;
  int32_t P = 0, G = 0, G4 = 0, TW = 0;
  int32_t format = EFFORT_ENTRY_U32;  // EFFORT_ENTRY_U32 or EFFORT_ENTRY_R12
  int32_t crop = 0;                   // stored segments 0..crop-1 (crop = P: all)
  int64_t gstride = 0;                // units per (row, group) run
  int64_t row_stride = 0;             // units per row = G * gstride
  uint64_t off_probes = 0, off_counts = 0, off_entries = 0, off_rowmax = 0, off_floor = 0, total = 0;
};

// 32-bit words per unit of the entries region
inline int32_t unit_words(int32_t format) {
  return format == EFFORT_ENTRY_R12 ? 3 : format == EFFORT_ENTRY_Q8 ? 2 : 1;
}

// The smallest power of two, at least 2, whose groups hold at most
// kTargetGroupWidth columns.  A power of two divides the CU count, so the
// multiply's grid (CUs / G blocks per group) stays one block per CU; at least
// two groups halve the blocks adding into each output column (one group per
// 4096 columns measured 10-25 % slower on the Mistral shapes with 4096 or
// 1024 columns).
inline int32_t default_groups(int64_t n) {
  if (n < 1) return 1;
  int64_t g = 2;
  while ((n + g - 1) / g > kTargetGroupWidth) g *= 2;
  return (int32_t)g;
}

// Offsets of the regions from the shape, the group stride and the options.
inline void place_regions(Geometry* g) {
  g->row_stride = (int64_t)g->G * g->gstride;
  g->off_probes = kAlign;
  g->off_counts = align_up(g->off_probes + (uint64_t)g->m * g->P * 2, kAlign);
  g->off_entries = align_up(g->off_counts + (uint64_t)g->m * g->P * g->G4 * 4, kAlign);
  g->off_rowmax = align_up(g->off_entries + (uint64_t)g->m * g->row_stride * unit_words(g->format) * 4,
                           kAlign);
  const bool cropped = g->crop < g->P;
  g->off_floor = cropped ? align_up(g->off_rowmax + (uint64_t)g->m * 2, kAlign) : 0;
  g->total = align_up((cropped ? g->off_floor : g->off_rowmax) + (uint64_t)g->m * 2, kAlign);
}

// Fills g from (m, n, P, groups) for an uncropped u32 layout, whose runs hold
// every entry of their group (gstride = TW).  groups = 0 picks the default.
// The group width is ceil(n / groups) rounded up to 64 columns, and the
// effective group count is ceil(n / width), so no group is empty.  Other
// formats and cropped layouts take the same shape and a data-dependent
// gstride (the converter sets it, then calls place_regions).
inline int make_geometry(int64_t m, int64_t n, int32_t P, int32_t groups, Geometry* g) {
  if (m < 1 || n < 1 || P < 1 || (int64_t)P > n || groups < 0) return EFFORT_EINVAL;
  if (m > (1ll << 31) - 1 || n > (1ll << 31) - 1) return EFFORT_EUNSUPPORTED;
  if ((int64_t)m * P > (1ll << 31) - 1) return EFFORT_EUNSUPPORTED;  // chart size fits u32 counts
  if (groups == 0) groups = default_groups(n);
  int64_t tw = (n + groups - 1) / groups;
  tw = (int64_t)align_up((uint64_t)tw, 64);
  if (tw > EFFORT_MAX_GROUP_WIDTH) return EFFORT_EUNSUPPORTED;
  if ((int64_t)m * tw > (1ll << 32) - 1) return EFFORT_EUNSUPPORTED;  // a group's entries fit u32
  int64_t G = (n + tw - 1) / tw;
  g->m = m;
  g->n = n;
  g->P = P;
  g->G = (int32_t)G;
  g->G4 = (int32_t)((G + 3) / 4 * 4);
  g->TW = (int32_t)tw;
  g->format = EFFORT_ENTRY_U32;
  g->crop = P;
  g->gstride = tw;
  place_regions(g);
  return EFFORT_OK;
}

// Workspace of one vector (offsets in bytes from the vector's slice start).
//   result   u32[128]                 [0] cutoff bits, [1] K', [2] K, [3] candidates,
//                                     [64 + r] candidates of dispatch block r (regions)
//   hist     u32[4096]                histogram of the chart's top 12 bits
//   hist2    u32[1024]                bits 18..9 of the chart values in the cutoff's bin
//   cand     u32[ceil(m/64)*64*P]     those chart values (bit patterns)
//   runlen   u32[G][m]                per (group, row) entries to read
//   bsum     u32[ceil(m/256)][G + 1]  per 256 rows: sum of runlen per group, then
//                                     (as f32) the sum of |v_i| * rowmax_i
// result, hist and hist2 are zero on entry and left zero.  A batched call with b
// vectors uses b slices and then the union area: urunlen u32[G][m] (per
// (group, row) the largest read length over the vectors of a pass) and ubsum
// u32[ceil(m/256)][G + 1] (its per-256-row sums).
constexpr int64_t kDspRows = 256;

struct WsLayout {
  uint64_t result, hist, hist2, cand, runlen, bsum, slice;
  // batched calls: after the per-vector slices, the union read lengths
  uint64_t urunlen, ubsum, union_bytes;
};

inline WsLayout ws_layout(const Geometry& g) {
  const uint64_t nbd = ((uint64_t)g.m + kDspRows - 1) / kDspRows;
  WsLayout w;
  w.result = 0;
  w.hist = 512;
  w.hist2 = w.hist + 4096 * 4;
  w.cand = align_up(w.hist2 + 1024 * 4, kAlign);
  // the candidate capacity: m rounded up to 64 rows (a dispatch block), times P
  w.runlen = align_up(w.cand + (uint64_t)((g.m + 63) / 64 * 64) * g.P * 4, kAlign);
  w.bsum = align_up(w.runlen + (uint64_t)g.G * g.m * 4, kAlign);
  w.slice = align_up(w.bsum + nbd * (g.G + 1) * 4, kAlign);
  w.urunlen = 0;  // offsets from the end of the slices
  w.ubsum = align_up((uint64_t)g.G * g.m * 4, kAlign);
  w.union_bytes = align_up(w.ubsum + nbd * (g.G + 1) * 4, kAlign);
  return w;
}

// FNV-1a-64 over 8-byte little-endian words.
inline uint64_t fnv1a64_words(const uint64_t* p, uint64_t nwords, uint64_t h = 0xCBF29CE484222325ull) {
  for (uint64_t i = 0; i < nwords; ++i) {
    h ^= p[i];
    h *= 0x100000001B3ull;
  }
  return h;
}

inline uint64_t desc_check_of(const effort_desc& d) {
  effort_desc c = d;
  c.desc_check = 0;
  // hash every byte of the struct before desc_check (padding is zeroed by the writer)
  const uint8_t* p = reinterpret_cast<const uint8_t*>(&c);
  uint64_t h = 0xCBF29CE484222325ull;
  for (size_t i = 0; i < offsetof(effort_desc, desc_check); ++i) {
    h ^= p[i];
    h *= 0x100000001B3ull;
  }
  return h;
}

// Largest units per (row, group) run a layout of this shape may hold.
inline int64_t max_gstride(const Geometry& g) {
  // u32: one unit per entry; r12: every record holds at least one entry
  return g.TW;
}

inline bool geometry_from_desc(const effort_desc* d, Geometry* g) {
  Geometry x;
  if (make_geometry(d->in_dim, d->out_dim, d->probes_per_row, d->groups, &x) != EFFORT_OK) return false;
  if (d->entry_format != EFFORT_ENTRY_U32 && d->entry_format != EFFORT_ENTRY_R12 &&
      d->entry_format != EFFORT_ENTRY_Q8)
    return false;
  if (d->crop_segments < 1 || d->crop_segments > d->probes_per_row) return false;
  x.format = d->entry_format;
  x.crop = d->crop_segments;
  if (d->group_stride < 1 || d->group_stride > max_gstride(x)) return false;
  x.gstride = d->group_stride;
  if (x.format != EFFORT_ENTRY_U32 && x.TW > 4096) return false;  // 12-bit column / 9-bit cell
  if (x.format == EFFORT_ENTRY_Q8 && x.P > 16) return false;      // 4-bit segment field
  place_regions(&x);
  if (x.G != d->groups || x.TW != d->group_width || x.row_stride != d->row_stride ||
      x.off_probes != d->off_probes || x.off_counts != d->off_counts ||
      x.off_entries != d->off_entries || x.off_rowmax != d->off_rowmax ||
      x.off_floor != d->off_floor || x.total != d->total_bytes ||
      d->index_bytes != (x.format == EFFORT_ENTRY_U32 ? 2 : 0))
    return false;
  *g = x;
  return true;
}

}  // namespace effort
