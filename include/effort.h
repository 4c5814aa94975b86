/*
 * effort.h -- C ABI of the MI355X (gfx950) implementation of the "Effort"
 * approximate vector-matrix multiply ("bucketMul").
 *
 * Method (web pages, cited by title and passage):
 *  [HN] "Show HN: Speeding up LLM inference 2x times (possibly)", Hacker News
 *       thread: the quoted pseudocode precompute(W) / approxMul(v, ...) in the
 *       exchange with gcy; the sorted (index, value) row storage in the author's
 *       reply to bigcat12345678; the 16-part row split of bucketMul in the reply
 *       to marmaduke; effort as a per-call knob "in real time" in the post text.
 *  [HT] hntin item 40095016: cost O(effort*inDim*outDim) multiplications,
 *       O(inDim) dispatch, O(inDim log inDim) cutoff.
 *
 * y = v . W computed from only the products whose magnitude reaches a cutoff:
 *   W      fp16 [in_dim][out_dim], row i multiplies v_i (the stored matrix is
 *          the transposed weight, "W = W.T" in the precompute of [HN]).
 *   probes per row, P magnitudes at ranks ceil((k+1) out_dim / P) of the row
 *          sorted by |w| descending.
 *   K      min(N, max(1, ceil(effort * N))) in double, N = in_dim * P.
 *   cutoff K-th largest of fl32(|v_i| * probe_i[k]) (the pseudocode's top-K step over the chart).
 *   kept   (i, j) with fl32(|v_i| * |W_ij|) >= cutoff.
 *   y_j    sum of v_i * W_ij over kept (i, j), accumulated in fp32.
 *
 * Conventions for every function:
 *  - returns int: EFFORT_OK (0) or an error code; effort_strerror() names it.
 *  - pointers are plain host or device pointers as stated per argument; the
 *    caller owns all memory.  The library never allocates device memory; its
 *    only global state is a cache of each device's CU count and, per host
 *    thread, the last failed HIP status (effort_last_hip_error).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Device
 *    work is stream-ordered and asynchronous unless stated otherwise.
 *  - every argument is validated on the host before anything is enqueued, so
 *    EINVAL / ENOSPACE / ECORRUPT leave the stream untouched.
 *  - alignment: layouts and workspaces 256 bytes; float and int32 arrays 4
 *    bytes, 64-bit outputs 8 bytes, fp16 weights 2 bytes (16-byte aligned
 *    vectors let the multiply load them 16 bytes at a time).  A misaligned
 *    pointer is EFFORT_EINVAL.
 */
#ifndef EFFORT_H
#define EFFORT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  EFFORT_OK = 0,
  EFFORT_EINVAL = 1,      /* null / misaligned pointer, bad size, effort not in (0,1], non-finite W */
  EFFORT_ENOSPACE = 2,    /* a caller buffer (layout, workspace) is too small */
  EFFORT_EHIP = 3,        /* a HIP call or kernel launch failed */
  EFFORT_EUNSUPPORTED = 4,/* valid request this build does not handle (e.g. group too wide) */
  EFFORT_ECORRUPT = 5     /* descriptor or layout header fails its magic/version/checksum */
};

#define EFFORT_MAGIC 0x4F464645u /* "EFFO" little-endian */
#define EFFORT_VERSION 3u
#define EFFORT_MAX_GROUP_WIDTH 8192 /* output columns per group (fp32 LDS tile of 32 KiB) */
#define EFFORT_MAX_BATCH 16
#define EFFORT_MAX_MULTI 4 /* matrices of one effort_matvec_multi call */
#define EFFORT_NOALLOC_WORKSPACE_BYTES (8ull << 20) /* effort_matvec_noalloc's workspace per device */

/* Host-side descriptor of a prepared layout; filled by effort_prepare*, passed
   by pointer to the multiply.  Plain old data; a copy is stored at the start of
   the layout blob. */
/* Entry formats of a layout (effort_desc.entry_format). */
#define EFFORT_ENTRY_U32 0 /* 4 bytes per entry: fp16 value, 16-bit column in the group */
#define EFFORT_ENTRY_R12 1 /* 3 bytes per entry: records of 4 entries in 12 bytes (see
                              effort_prepare_host_opts) */
#define EFFORT_ENTRY_Q8 2  /* Q8 bucketed entries, 2 bytes per entry: records of 4 one-byte
                              entries (sign, 4-bit level, 3-bit location) and a 4-byte
                              header (see effort_prepare_host_opts); lossy: the multiply
                              runs on the quantized matrix */

typedef struct effort_desc {
  uint32_t magic, version;
  int64_t in_dim, out_dim;    /* m, n */
  int32_t probes_per_row;     /* P, 1 <= P <= n */
  int32_t groups;             /* G: output-column groups */
  int32_t group_width;        /* TW: columns per group, multiple of 64; last group may be narrower */
  int32_t index_bytes;        /* bytes of the column index of an entry: 2 (u32), 0 (r12) */
  int64_t row_stride;         /* storage units per stored row = G * group_stride */
  int64_t group_stride;       /* storage units per (row, group) run (u32: entries, r12: records) */
  int32_t entry_format;       /* EFFORT_ENTRY_U32 or EFFORT_ENTRY_R12 */
  int32_t crop_segments;      /* c: rank segments 0..c-1 of every row are stored; c = P: all */
  uint64_t off_probes;        /* byte offsets inside the layout */
  uint64_t off_counts;
  uint64_t off_entries;
  uint64_t off_rowmax;
  uint64_t off_floor;         /* cropped layouts: largest magnitude key not stored, per row (else 0) */
  uint64_t total_bytes;
  uint64_t checksum;          /* FNV-1a-64 over the blob's 8-byte words after the header */
  uint64_t desc_check;        /* FNV-1a-64 over all fields above */
} effort_desc;

/* Name of a status code (static string). */
const char* effort_strerror(int status);

/* Name of the last failed HIP status seen by a call of this library on the
   calling thread ("hipSuccess" if none); explains an EFFORT_EHIP. */
const char* effort_last_hip_error(void);

/* ---------------------------------------------------------------- sizing (host only, no HIP calls) */

/* Default number of output-column groups for out_dim columns: the smallest
   power of two, at least 2, whose groups hold at most 4096 columns. */
int32_t effort_default_groups(int64_t out_dim);

/* Bytes of the layout of an in_dim x out_dim matrix with P probes per row and
   `groups` output groups (0 = effort_default_groups(out_dim)).
   EINVAL: in_dim < 1, out_dim < 1, P not in [1, out_dim], bytes NULL.
   EUNSUPPORTED: the resulting group width exceeds EFFORT_MAX_GROUP_WIDTH. */
int effort_layout_bytes(int64_t in_dim, int64_t out_dim, int32_t P, uint64_t* bytes);
int effort_layout_bytes_ex(int64_t in_dim, int64_t out_dim, int32_t P, int32_t groups,
                           uint64_t* bytes);

/* Device workspace for one call of effort_matvec* with `batch` vectors
   (1 <= batch <= EFFORT_MAX_BATCH): one slice per vector and, for batch > 1,
   room for the union of the vectors' read lengths.  The workspace must be
   zero-filled before its first use (effort_workspace_init); every call leaves
   it ready for the next.  One workspace serves one call at a time. */
int effort_workspace_bytes(const effort_desc* desc, int32_t batch, uint64_t* bytes);

/* Zero-fill `ws_bytes` of device memory at ws_dev (stream-ordered). */
int effort_workspace_init(void* ws_dev, uint64_t ws_bytes, void* stream);

/* -------------------------------------------------- offline converter ("precompute" of [HN]) */

/* Host fp16 bits W[in_dim][out_dim] (y = v . W) -> host layout blob.
   Per row: entries sorted by |w| descending (ties: column ascending), grouped by
   output-column group; each entry is (fp16 value, 16-bit column index within
   its group); P probes (fp16 magnitudes); per (row, probe segment, group) the
   cumulative entry count; the row's largest magnitude.  layout_host: host memory of >= layout_bytes bytes,
   8-byte aligned.  desc_out: host.  EINVAL also for non-finite W. */
int effort_prepare_host(const uint16_t* w_fp16, int64_t in_dim, int64_t out_dim, int32_t P,
                        void* layout_host, uint64_t layout_bytes, effort_desc* desc_out);
int effort_prepare_host_ex(const uint16_t* w_fp16, int64_t in_dim, int64_t out_dim, int32_t P,
                           int32_t groups, void* layout_host, uint64_t layout_bytes,
                           effort_desc* desc_out);

/* Layout options (effort_prepare_host_opts):
   groups         output-column groups, 0 = effort_default_groups(out_dim).
   entry_format   EFFORT_ENTRY_U32: per entry the fp16 value and a 16-bit column
                  inside its group, rank order inside a segment.
                  EFFORT_ENTRY_R12 (group width <= 4096, else EUNSUPPORTED): inside
                  each (row, group, segment) the entries in column order, 4 to a
                  12-byte record -- two words of fp16 values, then the first
                  column (12 bits) and three column steps (7, 7, 6 bits); a step
                  that does not fit ends the record early and pads (value
                  0x8000, step 0) fill it; a -0.0 weight is stored as +0.0.
                  The position bits an entry spends against what its bucket
                  already tells is the trade-off of the author's reply to kwikiel
                  in [HN].
                  EFFORT_ENTRY_Q8 (P <= 16, group width <= 4096): the Q8 bucketed
                  form of the author's reply to kwikiel in [HN] (4 bits of weight,
                  1 sign bit, 3 location bits, the weight bits covering only its
                  bucket's range).  Buckets are the rank segments of a row: bucket
                  k spans magnitude keys from lo = probe k to hi = probe k-1 (the
                  row's largest for k = 0) in 16 levels lo + c 2^s capped at hi (s
                  the smallest shift with 15 2^s >= hi - lo); each weight moves to
                  the nearest level (ties up), sign kept.  The quantized matrix
                  has the same probes; the call computes the rule on it.  Storage:
                  per (row, group, segment) the entries in column order, 4 to an
                  8-byte record: a header word (bits 0-3 segment, 4-5 entries - 1,
                  6-14 the first entry's 8-column cell, then cell steps of 6, 6 and
                  5 bits) and a word of 4 entry bytes (bit 7 sign, bits 6-3 level,
                  bits 2-0 column in the cell).
   crop_segments  0 or P: every segment is stored.  c in [1, P): only the rank
                  segments 0..c-1 of each row (the largest magnitudes) are stored
                  ([HN] post text: with this format part of the smallest-magnitude
                  weights need not be loaded; the reply about running Mixtral from its top
                  ~70 %).  Probes and rowmax still describe the whole row, so the
                  cutoff is the uncropped one; a call keeps exactly the uncropped
                  kept set whenever none of its kept products lies in a dropped
                  segment, and otherwise keeps the stored part of it and reports
                  that (effort_matvec_debug status bit 1).
   reserved       0. */
typedef struct effort_prepare_opts {
  int32_t groups;
  int32_t entry_format;
  int32_t crop_segments;
  int32_t reserved;
} effort_prepare_opts;

/* Exact layout bytes of W with these options: a host pass over W (the length
   of a cropped or r12 run depends on the data).  EINVAL: bad options or
   non-finite W; EUNSUPPORTED as effort_layout_bytes_ex. */
int effort_layout_bytes_opts(const uint16_t* w_fp16, int64_t in_dim, int64_t out_dim, int32_t P,
                             const effort_prepare_opts* opts, uint64_t* bytes);

/* effort_prepare_host with options; layout_bytes must be at least
   effort_layout_bytes_opts of the same arguments (ENOSPACE otherwise). */
int effort_prepare_host_opts(const uint16_t* w_fp16, int64_t in_dim, int64_t out_dim, int32_t P,
                             const effort_prepare_opts* opts, void* layout_host,
                             uint64_t layout_bytes, effort_desc* desc_out);

/* Same, then copies the blob into caller-owned device memory layout_dev on
   `stream`.  Uses a temporary host buffer and synchronizes `stream` before
   returning. */
int effort_prepare(const uint16_t* w_fp16_host, int64_t in_dim, int64_t out_dim, int32_t P,
                   void* layout_dev, uint64_t layout_bytes, effort_desc* desc_out, void* stream);

/* Checks a host layout blob against its descriptor (magic, version,
   descriptor check, blob checksum).  ECORRUPT on mismatch. */
int effort_layout_check(const effort_desc* desc, const void* layout_host);

/* ---------------------------------------------------------------- hot path ("approxMul" of [HN]) */

/* y_dev[out_dim] = approximate v_dev[in_dim] . W at the given effort.
   layout_dev: device copy of the prepared blob.  v_dev: device fp32.  y_dev:
   device fp32, overwritten (zeroed by the call).  ws_dev: device workspace of
   >= effort_workspace_bytes(desc, 1) bytes.  effort in (0, 1], else EINVAL.
   v must be finite (precondition, not checked here; effort_matvec_debug
   reports a violation). */
int effort_matvec(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                  float effort, float* y_dev, void* ws_dev, uint64_t ws_bytes, void* stream);

/* effort_matvec for callers that cannot allocate device memory or pass a
   workspace (code under HIP graph capture, tight serving loops, harnesses that
   forbid allocation): the same kernels, with the workspace in a static device
   array of EFFORT_NOALLOC_WORKSPACE_BYTES that the library holds on each device
   until the process ends.  The first call on a device looks up the array's
   address and zero-fills it on `stream`; no call allocates or frees memory.
   ENOSPACE when the matrix needs a larger workspace than the array
   (effort_workspace_bytes(desc, 1) > EFFORT_NOALLOC_WORKSPACE_BYTES); other
   errors as effort_matvec.  All calls on one device share the array and leave
   it ready for the next call: calls that overlap on one device (other
   streams, other host threads) race and must be ordered by the caller. */
int effort_matvec_noalloc(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                          float effort, float* y_dev, void* stream);

/* `batch` independent vectors v_dev[batch][in_dim] -> y_dev[batch][out_dim],
   each with its own K, cutoff and kept set (the same result as `batch` calls
   of effort_matvec).  Up to 4 vectors, or any number at effort below
   0.625: launches of up to 4 vectors, one of each kernel, every vector with
   its own multiply over its own read lengths.  From 5 vectors at effort
   0.625 and above: the vectors' cutoffs and read lengths come from one
   launch each; then, per pass of up to 8 vectors (fewer for wide column
   groups: their LDS tiles must fit), every row's entries are read once up to
   the longest of the pass's read lengths and each entry is tested against
   every vector's threshold.
   ws >= effort_workspace_bytes(desc, batch). */
int effort_matvec_batched(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                          int32_t batch, float effort, float* y_dev, void* ws_dev,
                          uint64_t ws_bytes, void* stream);

/* Several independent (matrix, vector) pairs in one launch of each of the
   three kernels: ys_dev[j] = approximate vs_dev[j] . W_j at efforts[j] for
   j < count, each with its own K, cutoff and kept set -- the result of count
   calls of effort_matvec.  For matrices that share an input (a decode step
   multiplies a layer's query, key and value matrices, and its gate and up
   projections, by one activation), pass the same vector for each; efforts may
   differ per matrix ([HN], the author's reply to refulgentis: effort can be
   set layer by layer and matrix by matrix).  The pairs must not depend on
   each other's outputs.
   descs, layouts_dev, vs_dev, efforts, ys_dev: host arrays of count entries
   (the pointers in them are device pointers; vs_dev[j] holds
   descs[j].in_dim floats); 1 <= count <= EFFORT_MAX_MULTI; every effort in
   (0, 1].  ws >= effort_workspace_bytes_multi(descs, count). */
int effort_workspace_bytes_multi(const effort_desc* descs, int32_t count, uint64_t* bytes);
int effort_matvec_multi(const effort_desc* descs, const void* const* layouts_dev, int32_t count,
                        const float* const* vs_dev, const float* efforts, float* const* ys_dev,
                        void* ws_dev, uint64_t ws_bytes, void* stream);

/* effort_matvec plus parity outputs (all device pointers; each may be NULL):
   cutoff_dev[1]        cutoff value;
   K_dev[2]             K and K' = #{chart >= cutoff};
   row_kept_dev[in_dim] kept products per row;
   fingerprint_dev[1]   sum over kept (i,j) of splitmix64-output(i*out_dim+j), mod 2^64;
   kept_mask_dev        uint8 [in_dim][out_dim], 1 where kept;
   status_dev[1]        bit 0 set when v holds a NaN or an infinity (outside
                        the contract: the other outputs are then unspecified);
                        bit 1 set when the layout is cropped and the keep rule
                        keeps a product of a dropped segment (the outputs then
                        cover the stored part of the kept set).
   Same kernels as effort_matvec with the recording switched on: the keep test
   and the accumulation are the timed path's own; recording only adds the
   stores of the kept pairs.  Untimed. */
int effort_matvec_debug(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                        float effort, float* y_dev, void* ws_dev, uint64_t ws_bytes,
                        float* cutoff_dev, int64_t* K_dev, int32_t* row_kept_dev,
                        uint64_t* fingerprint_dev, uint8_t* kept_mask_dev, uint32_t* status_dev,
                        void* stream);

/* effort_matvec_batched plus the parity outputs of every vector (device
   pointers, each may be NULL): cutoff_dev[batch], K_dev[batch][2] (K, K'),
   row_kept_dev[batch][in_dim], fingerprint_dev[batch], kept_mask_dev
   [batch][in_dim][out_dim], each as in effort_matvec_debug.  The call takes
   the same route as effort_matvec_batched for the same batch and effort (the
   union pass over up to 8 vectors, or launches of up to 4 vectors with their
   own multiplies), with recording switched on in those kernels. */
int effort_matvec_batched_debug(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                                int32_t batch, float effort, float* y_dev, void* ws_dev,
                                uint64_t ws_bytes, float* cutoff_dev, int64_t* K_dev,
                                int32_t* row_kept_dev, uint64_t* fingerprint_dev,
                                uint8_t* kept_mask_dev, void* stream);

/* effort_matvec_multi plus the parity outputs of every pair (device pointers,
   each may be NULL): cutoff_dev[count], K_dev[count][2], fingerprint_dev
   [count]; row_kept_dev is a host array of count device pointers (each may be
   NULL), pair j's counts [descs[j].in_dim].  Same kernels and launches as
   effort_matvec_multi with recording switched on. */
int effort_matvec_multi_debug(const effort_desc* descs, const void* const* layouts_dev, int32_t count,
                              const float* const* vs_dev, const float* efforts, float* const* ys_dev,
                              void* ws_dev, uint64_t ws_bytes, float* cutoff_dev, int64_t* K_dev,
                              int32_t* const* row_kept_dev, uint64_t* fingerprint_dev, void* stream);

/* effort_matvec with kernel timing, for measurement.  events[0..5] are hipEvent_t
   pairs (start, stop) for the cutoff kernel, the dispatch kernel and the
   bucketMul kernel; the runtime stamps each pair with that kernel's own begin
   and end (hipExtLaunchKernelGGL).  A pair may be (NULL, NULL) to leave that
   kernel untimed; a pair with one NULL member is EINVAL.  EUNSUPPORTED while
   `stream` is being captured into a graph. */
int effort_matvec_timed(const effort_desc* desc, const void* layout_dev, const float* v_dev,
                        float effort, float* y_dev, void* ws_dev, uint64_t ws_bytes,
                        void* stream, void* const* events);

/* ---------------------------------------------------------------- comparators and glue */

/* Dense y_dev[out_dim] = v_dev[in_dim] . W, W fp16 [in_dim][out_dim] row-major on
   the device, fp32 accumulation.  The dense matvec the approximate one is
   measured against ([HN]: the author's comparison with a dense matmul). */
int dense_gemv(const uint16_t* w_dev, const float* v_dev, int64_t in_dim, int64_t out_dim,
               float* y_dev, void* stream);

/* Dense y_dev[batch][out_dim] = v_dev[batch][in_dim] . W, 1 <= batch <= EFFORT_MAX_BATCH. */
int dense_gemm_small(const uint16_t* w_dev, const float* v_dev, int32_t batch, int64_t in_dim,
                     int64_t out_dim, float* y_dev, void* stream);

/* out[i] = silu(h1[i]) * h3[i], silu(x) = x / (1 + exp(-x)): the gate of a
   gated feed-forward block between its approximate matvecs. */
int effort_silu_mul(const float* h1_dev, const float* h3_dev, int64_t n, float* out_dev,
                    void* stream);

/* out[i] = ga * a[i] + gb * b[i] (two fp32 products, one fp32 sum; out may
   alias a or b): the gated sum of two experts' outputs in a mixture-of-experts
   feed-forward block. */
int effort_axpby(const float* a_dev, float ga, const float* b_dev, float gb, int64_t n,
                 float* out_dev, void* stream);

/* ---------------------------------------------------------------- measurement helpers */

int effort_event_create(void** event_out);            /* hipEvent_t with timing */
int effort_event_record(void* event, void* stream);
int effort_event_elapsed_ms(void* start, void* end, float* ms_out); /* waits for `end` */
int effort_event_destroy(void* event);
int effort_stream_synchronize(void* stream);

#ifdef __cplusplus
}
#endif
#endif /* EFFORT_H */
