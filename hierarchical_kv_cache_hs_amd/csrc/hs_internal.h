// Internal declarations shared by the host API (hs_api.cpp) and the kernels (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hs.h"

namespace hs {

// Threads of one resolver workgroup (one workgroup per request).
constexpr int kResolveThreads = 512;
// Upper bounds the resolver's register tiling supports.
constexpr int kMaxTopK = 16 * kResolveThreads;          // 8192
constexpr int kMaxBuffer = 32 * kResolveThreads;        // 16384 slots (hit bitmap: one word per thread)
constexpr size_t kLdsLimit = 160 * 1024;                // gfx950 LDS per workgroup

// Device tables of one layer for requests 0..max_requests-1.
struct LayerTables {
  int32_t* pt;     // [n][cap]
  int32_t* rm;     // [n][B]
  int32_t* st;     // [n][B]
  int32_t* ord;    // [n][B]
  int32_t* step;   // [n]
  uint8_t* buf;    // [n][req_stride]: B rows of slot_stride bytes, then a zero row (attention padding)
  float* part;     // attention split partials (see attend.hip)
  uint32_t* fresh; // [n][B/32] bits of slots appended since the last resolve (their stamp is its step)
  uint8_t* tail;   // [n][cap][tail_bytes] device-resident row tails (HS_FLAG_RESIDENT_TAIL), else null
  int32_t* ml_tok;   // miss lists [n][k]
  int32_t* ml_slot;  // [n][k]
  int32_t* ml_cnt;   // [n]
};

struct Geometry {
  int32_t k, B, n, L, layout, heads;
  int32_t P;            // tokens per cached unit (1, or a page of P tokens); k, B and cap count units
  int32_t lgP;          // log2 P
  int64_t cap;
  int64_t entry_bytes;  // bytes of one token's row
  int64_t unit_bytes;   // bytes of one cached unit: P rows
  int64_t host_stride;  // bytes between units in the host history (unit_bytes - tail_bytes)
  int64_t tail_bytes;   // HS_FLAG_RESIDENT_TAIL: last bytes of each row kept on the device (16), else 0
  int64_t slot_stride;  // bytes between slots (= unit_bytes)
  int64_t req_stride;   // bytes per request in the slot buffer: B slot rows, then one row of zeros
  uint32_t flags;
  int32_t policy;       // hs_eviction
  uint64_t seed;        // HS_EVICT_RANDOM key
};

// Once per process, before the first launch (outside any graph capture).
void prepare_resolve();

// Dynamic LDS bytes the resolver needs for this geometry.
size_t resolve_lds_bytes(int64_t cap, int32_t k, int32_t B);

// list_only: write the miss lists instead of copying the rows (launch_fetch copies them).
hipError_t launch_resolve(const Geometry& g, const LayerTables& t, int32_t layer, const uint8_t* host_layer,
                          int32_t n_req, const int32_t* sel, int32_t* slots, int32_t* miss, int32_t* err,
                          bool list_only, hipStream_t s);

hipError_t launch_fetch(const Geometry& g, const LayerTables& t, const uint8_t* host_layer, int32_t n_req,
                        hipStream_t s);

hipError_t launch_reset(const Geometry& g, int32_t* pt, int32_t* rm, int32_t* st, int32_t* ord, int32_t* step,
                        uint32_t* fresh, int32_t first, int32_t count, hipStream_t s);

// Once per process, before the first append launch.
void prepare_append();

// Write-through append: for each request with pos[r] >= 0, the row at rows + r * row_stride
// becomes resident and is written to the host history (host_layer: device-mapped address).
hipError_t launch_append(const Geometry& g, const LayerTables& t, uint8_t* host_layer, int32_t n_req,
                         const int32_t* pos, const void* rows, int64_t row_stride, int32_t* slot_out, int32_t* err,
                         hipStream_t s);

// Page-granular write-through append: each row goes to its history position and, when its
// page is resident, into the page's slot at row offset pos mod P; no table changes.
hipError_t launch_append_pages(const Geometry& g, const LayerTables& t, uint8_t* host_layer, int32_t n_req,
                               const int32_t* pos, const void* rows, int64_t row_stride, int32_t* slot_out,
                               int32_t* err, hipStream_t s);

// Prefill offload of 16-byte-aligned rows into the pinned history (dst_mapped: device-mapped
// address of the first destination row, rows of entry_bytes - tail_bytes packed); the last
// tail_bytes of each row go to tail_dst (device, packed), when tail_bytes > 0.
hipError_t launch_offload(const void* src, int64_t src_stride, uint8_t* dst_mapped, int64_t count, int64_t entry_bytes,
                          uint8_t* tail_dst, int64_t tail_bytes, hipStream_t s);

// Once per process, before the first top-k launch.
void prepare_topk();

// Top-k selection from indexer scores: for each request, the top_k positions of largest
// score in [0, len[r]) (ties to the smaller position), ascending; -1 padding when len < k.
// hint (or null): per request, in a guess and out the exact top 12-bit digit of the k-th
// largest key (-1: none); the selection does not depend on it.
hipError_t launch_topk(const Geometry& g, int32_t n_req, const float* scores, int64_t stride, const int32_t* len,
                       int32_t* sel, int32_t* hint, int32_t* err, hipStream_t s);

// Once per process, before the first attention launch.
void prepare_attend();

// Attention: split factor and partial-buffer floats per request.
int attend_splits(const Geometry& g, int n_req);
size_t attend_partial_floats(const Geometry& g);

// Tokens attended per request: every row of the k selected units.
inline int64_t attend_tokens(const Geometry& g) { return (int64_t)g.k * g.P; }

// Dense streaming read of `bytes` (a multiple of 16, 16-byte aligned) of device memory.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);

// sel and len (both or neither): cut each request's tokens at its context length len[r],
// token o of unit i taking part iff sel[r][i] >= 0 and sel[r][i] * P + o < len[r].
hipError_t launch_attend(const Geometry& g, const LayerTables& t, int32_t n_req, const void* q, const int32_t* slots,
                         const int32_t* sel, const int32_t* len, float scale, void* out, float* lse, hipStream_t s);

// hs_attend_noalloc: the split partials live in a static device array of kNoallocPartials
// partials (one copy per GPU, up to kMaxDevices GPUs).  prepare_attend_noalloc resolves the
// array's address on `device` (current) once; launch_attend_noalloc is launch_attend with
// `heads` query heads and the partials there (hipErrorInvalidValue if the launch needs more
// than kNoallocPartials; attend_noalloc_partials gives the count, 0 for a single split).
constexpr int kNoallocPartials = 256;
constexpr int kMaxDevices = 64;
hipError_t prepare_attend_noalloc(int device);
int64_t attend_noalloc_partials(const Geometry& g, int32_t n_req, int32_t heads);
hipError_t launch_attend_noalloc(const Geometry& g, const LayerTables& t, int device, int32_t n_req, int32_t heads,
                                 const void* q, const int32_t* slots, float scale, void* out, float* lse,
                                 hipStream_t s);

// One part of a step's attention split by residency, after a list-only resolve (the miss
// lists in t): fetched == false attends the entries of `slots` outside this step's victim
// slots into split partials (it may run while launch_fetch copies the misses); fetched ==
// true, after the copy and the resident part, attends the miss list and merges every partial
// into out / lse.  len (with sel for the resident part; the fetched part takes the units from
// the miss list) cuts at the context length as in launch_attend.
hipError_t launch_attend_part(const Geometry& g, const LayerTables& t, int32_t n_req, bool fetched, const void* q,
                              const int32_t* slots, const int32_t* sel, const int32_t* len, float scale, void* out,
                              float* lse, hipStream_t s);

}  // namespace hs
