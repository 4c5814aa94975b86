// convert.cpp -- offline converter: fp16 W[in][out] -> the layout blob.
//
// This is the "precompute" of the method (HN thread "Show HN: Speeding up LLM
// inference 2x times (possibly)", the quoted pseudocode in the exchange with
// gcy): the stored matrix has one row per input element; each row keeps all of
// its weights, sorted by magnitude descending (the author's reply to
// bigcat12345678), cut into P rank segments whose smallest magnitudes are the
// probes (the 16-part row split in the reply to marmaduke).  The row is further
// split by output-column group so that a GPU workgroup can own one group's
// slice of y; inside a group the entries keep rank order.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "effort.h"
#include "layout.hpp"

namespace effort {

static void convert_rows(const uint16_t* W, const Geometry& g, uint8_t* blob, int64_t r0, int64_t r1) {
  const int64_t n = g.n;
  const int32_t P = g.P, G = g.G, TW = g.TW;
  uint16_t* probes = reinterpret_cast<uint16_t*>(blob + g.off_probes);
  uint32_t* counts = reinterpret_cast<uint32_t*>(blob + g.off_counts);
  uint32_t* entries = reinterpret_cast<uint32_t*>(blob + g.off_entries);
  uint16_t* rowmax = reinterpret_cast<uint16_t*>(blob + g.off_rowmax);
  std::vector<uint64_t> order((size_t)n);
  std::vector<uint32_t> seg_cnt((size_t)P * G);
  std::vector<int64_t> fill((size_t)G);
  for (int64_t i = r0; i < r1; ++i) {
    const uint16_t* row = W + i * n;
    // rank order: key (|w| bits) descending, column ascending
    for (int64_t j = 0; j < n; ++j)
      order[j] = ((uint64_t)(0x7FFFu - (row[j] & 0x7FFFu)) << 32) | (uint64_t)j;
    std::sort(order.begin(), order.end());
    rowmax[i] = (uint16_t)(row[order[0] & 0xFFFFFFFFu] & 0x7FFFu);
    std::fill(seg_cnt.begin(), seg_cnt.end(), 0u);
    std::fill(fill.begin(), fill.end(), 0);
    uint32_t* row_entries = entries + i * g.row_stride;
    int32_t k = 0;
    int64_t seg_end = ((int64_t)1 * n + P - 1) / P;  // rank (1-based) that closes segment 0
    for (int64_t r = 1; r <= n; ++r) {
      while (r > seg_end) {
        ++k;
        seg_end = ((int64_t)(k + 1) * n + P - 1) / P;
      }
      const int64_t j = (int64_t)(order[r - 1] & 0xFFFFFFFFu);
      const uint16_t bits = row[j];
      const int32_t grp = (int32_t)(j / TW);
      const uint32_t local = (uint32_t)(j - (int64_t)grp * TW);
      row_entries[(int64_t)grp * TW + fill[grp]++] = (uint32_t)bits | (local << 16);
      seg_cnt[(size_t)k * G + grp] += 1;
      if (r == seg_end) probes[i * P + k] = (uint16_t)(bits & 0x7FFFu);
    }
    // cumulative counts over segments
    uint32_t* crow = counts + (size_t)i * P * g.G4;
    for (int32_t grp = 0; grp < G; ++grp) {
      uint32_t acc = 0;
      for (int32_t kk = 0; kk < P; ++kk) {
        acc += seg_cnt[(size_t)kk * G + grp];
        crow[(size_t)kk * g.G4 + grp] = acc;
      }
    }
  }
}

static int fill_desc(const Geometry& g, effort_desc* d) {
  memset(d, 0, sizeof *d);
  d->magic = EFFORT_MAGIC;
  d->version = EFFORT_VERSION;
  d->in_dim = g.m;
  d->out_dim = g.n;
  d->probes_per_row = g.P;
  d->groups = g.G;
  d->group_width = g.TW;
  d->index_bytes = 2;
  d->row_stride = g.row_stride;
  d->off_probes = g.off_probes;
  d->off_counts = g.off_counts;
  d->off_entries = g.off_entries;
  d->off_rowmax = g.off_rowmax;
  d->total_bytes = g.total;
  return EFFORT_OK;
}

uint64_t blob_checksum(const void* blob, uint64_t total) {
  const uint64_t* w = reinterpret_cast<const uint64_t*>(static_cast<const uint8_t*>(blob) + kAlign);
  return fnv1a64_words(w, (total - kAlign) / 8);
}

int prepare_host(const uint16_t* W, int64_t m, int64_t n, int32_t P, int32_t groups, void* layout,
                 uint64_t layout_bytes, effort_desc* desc_out) {
  if (!W || !layout || !desc_out) return EFFORT_EINVAL;
  if (reinterpret_cast<uintptr_t>(layout) % 8) return EFFORT_EINVAL;
  Geometry g;
  int rc = make_geometry(m, n, P, groups, &g);
  if (rc) return rc;
  if (layout_bytes < g.total) return EFFORT_ENOSPACE;
  // the method is defined on finite weights
  const int64_t total = m * n;
  for (int64_t e = 0; e < total; ++e)
    if ((W[e] & 0x7C00u) == 0x7C00u) return EFFORT_EINVAL;
  uint8_t* blob = static_cast<uint8_t*>(layout);
  memset(blob, 0, (size_t)g.total);
  unsigned nt = std::thread::hardware_concurrency();
  if (nt < 1) nt = 1;
  if (nt > 16) nt = 16;
  if ((int64_t)nt > m) nt = (unsigned)m;
  std::vector<std::thread> pool;
  for (unsigned t = 0; t < nt; ++t) {
    int64_t r0 = m * t / nt, r1 = m * (t + 1) / nt;
    pool.emplace_back(convert_rows, W, std::cref(g), blob, r0, r1);
  }
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
