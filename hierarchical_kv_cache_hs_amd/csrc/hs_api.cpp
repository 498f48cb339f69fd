// Host side of the C ABI in include/hs.h: configuration checks, the pinned host pool,
// the device block (tables + slot buffer + attention partials) and kernel launches.
//
// Device block layout (each part 256-byte aligned), per layer l and request r:
//   err                        int32 error word
//   pt    [L][n][cap]          token -> slot
//   rm    [L][n][B]            slot -> token
//   st    [L][n][B]            slot stamp
//   ord   [L][n][B]            slots in (stamp, slot) order
//   step  [L][n]               resolves done
//   fresh [L][n][B/32]         slots appended since the last resolve (stamped with its step)
//   part  [L][n][...]          attention split partials (if num_heads > 0)
//   ml_*  [L][n][k], [L][n]    per-request miss lists (token, slot) and counts for the fetch kernel
//   buf   [L][n][B + 1][E]     KV rows of the slots, packed; row B stays zero (attention reads it
//                              for padded selection entries)
//   tail  [L][n][cap][16]      HS_FLAG_RESIDENT_TAIL: the last 16 bytes of every history row
// Host pool (pinned, mapped): [L][n][cap][host stride]: whole rows, or with
// HS_FLAG_RESIDENT_TAIL their first 640 bytes (five whole 128-byte lines per row).

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "hs_internal.h"

struct hs_handle {
  hs::Geometry g;
  int device = 0;
  uint8_t* dev_block = nullptr;
  bool own_dev = false;
  size_t dev_bytes = 0;
  uint8_t* host_pool = nullptr;      // host address
  uint8_t* host_pool_dev = nullptr;  // device address of the same memory
  size_t host_bytes = 0;
  int32_t* err = nullptr;
  int32_t* pt = nullptr;
  int32_t* rm = nullptr;
  int32_t* st = nullptr;
  int32_t* ord = nullptr;
  int32_t* step = nullptr;
  uint32_t* fresh = nullptr;
  float* part = nullptr;
  int32_t* ml_tok = nullptr;
  int32_t* ml_slot = nullptr;
  int32_t* ml_cnt = nullptr;
  uint8_t* buf = nullptr;
  uint8_t* tail = nullptr;  // HS_FLAG_RESIDENT_TAIL: row tails [L][n][cap][tail_bytes]
  size_t part_floats = 0;  // per request
  // per layer: requests whose miss lists the last resolve-side call left in the handle (a
  // list-only resolve); 0 after any other resolve, append or reset.  The copy and the attention
  // parts read those lists and refuse to run without them.
  std::vector<int32_t> lists_for;
  // per layer: requests whose resident attention part left its split partials in the handle
  // since the layer's last list-only resolve; 0 after any resolve, append, reset or whole
  // attention of the layer (which reuse the same partial space).  The fetched part merges
  // those partials and refuses to run without them.
  std::vector<int32_t> resident_for;
  // Streams this handle has enqueued work on outside graph capture, each with an event
  // recorded after the handle's latest work there: hs_get_device_error and hs_destroy wait for
  // these events only, not for the whole device.  Past kMaxStreams distinct streams the handle
  // stops tracking and waits for the whole device instead.
  struct Mark {
    hipStream_t stream;
    hipEvent_t event;
  };
  std::vector<Mark> marks;
  bool untracked = false;
  hipStream_t aux = nullptr;  // private non-blocking stream: initialisation and error-word reads
  hipError_t noalloc_ready = hipErrorNotInitialized;  // hs_attend_noalloc's scratch resolved on `device`
};

namespace {

thread_local std::string g_msg;

hs_status fail(hs_status s, const std::string& msg) {
  g_msg = msg;
  return s;
}

hs_status fail_hip(hipError_t e, const char* what) {
  g_msg = std::string(what) + ": " + hipGetErrorString(e);
  return HS_ERR_HIP;
}

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// a*b with overflow detection
bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

bool add_ok(size_t a, size_t b, size_t* out) {
  if (b > SIZE_MAX - a) return false;
  *out = a + b;
  return true;
}

struct Layout {
  size_t err, pt, rm, st, ord, step, fresh, part, ml_tok, ml_slot, ml_cnt, buf, tail, total;
  size_t host_total;
  size_t part_floats;
};

// Validates cfg and computes the geometry and both memory layouts, touching no HIP API.
hs_status plan(const hs_config* cfg, hs::Geometry* g, Layout* lay) {
  if (!cfg) return fail(HS_ERR_INVALID_ARG, "config is NULL");
  if (cfg->top_k < 1) return fail(HS_ERR_INVALID_ARG, "top_k must be >= 1");
  if (cfg->device_buffer_size < cfg->top_k)
    return fail(HS_ERR_INVALID_ARG, "device_buffer_size must be >= top_k (every selected token must fit)");
  if (cfg->host_to_device_ratio < 1) return fail(HS_ERR_INVALID_ARG, "host_to_device_ratio must be >= 1");
  if (cfg->max_requests < 1) return fail(HS_ERR_INVALID_ARG, "max_requests must be >= 1");
  if (cfg->num_layers < 1) return fail(HS_ERR_INVALID_ARG, "num_layers must be >= 1");
  if (cfg->layout != HS_KV_BF16_576 && cfg->layout != HS_KV_FP8_MLA_656)
    return fail(HS_ERR_INVALID_ARG, "unknown KV layout");
  if (cfg->num_heads < 0 || cfg->num_heads > 16) return fail(HS_ERR_INVALID_ARG, "num_heads must lie in [0, 16]");
  if (cfg->flags & ~(HS_FLAG_NO_IO | HS_FLAG_ATTN_OUT_F32 | HS_FLAG_RESIDENT_TAIL))
    return fail(HS_ERR_INVALID_ARG, "unknown flag bits");
  if (cfg->eviction != HS_EVICT_LRU && cfg->eviction != HS_EVICT_FIFO && cfg->eviction != HS_EVICT_RANDOM)
    return fail(HS_ERR_INVALID_ARG, "unknown eviction policy");
  const int32_t P = cfg->page_tokens == 0 ? 1 : cfg->page_tokens;
  if (P < 1 || P > 256 || (P & (P - 1)))
    return fail(HS_ERR_INVALID_ARG, "page_tokens must be 0, 1 or a power of two <= 256");
  const bool tail = (cfg->flags & HS_FLAG_RESIDENT_TAIL) != 0;
  if (tail && (cfg->layout != HS_KV_FP8_MLA_656 || P != 1 || (cfg->flags & HS_FLAG_NO_IO)))
    return fail(HS_ERR_INVALID_ARG,
                "HS_FLAG_RESIDENT_TAIL needs token-granular 656-byte rows and a host pool (no HS_FLAG_NO_IO)");
  if (cfg->num_heads > 0 && (int64_t)cfg->top_k * P > 65536)
    return fail(HS_ERR_UNSUPPORTED, "attention over more than 65536 tokens (top_k * page_tokens)");
  if (cfg->top_k > hs::kMaxTopK) return fail(HS_ERR_UNSUPPORTED, "top_k above 8192");
  if (cfg->device_buffer_size > hs::kMaxBuffer) return fail(HS_ERR_UNSUPPORTED, "device_buffer_size above 16384");
  const int64_t cap = (int64_t)cfg->host_to_device_ratio * (int64_t)cfg->device_buffer_size;
  if (cap * P > INT32_MAX) return fail(HS_ERR_INVALID_ARG, "capacity (ratio * B * page_tokens) exceeds 2^31-1 tokens");
  if (hs::resolve_lds_bytes(cap, cfg->top_k, cfg->device_buffer_size) > hs::kLdsLimit)
    return fail(HS_ERR_UNSUPPORTED, "capacity too large for the resolver's on-chip token bitmap");

  g->k = cfg->top_k;
  g->B = cfg->device_buffer_size;
  g->n = cfg->max_requests;
  g->L = cfg->num_layers;
  g->layout = cfg->layout;
  g->heads = cfg->num_heads;
  g->P = P;
  g->lgP = 0;
  while ((1 << g->lgP) < P) ++g->lgP;
  g->cap = cap;
  g->entry_bytes = cfg->layout == HS_KV_BF16_576 ? 1152 : 656;
  g->unit_bytes = (int64_t)P * g->entry_bytes;
  // a 656-byte row spans six 128-byte lines wherever it starts; its first 640 bytes at a
  // 640-byte stride span five
  g->tail_bytes = tail ? g->entry_bytes % 128 : 0;
  g->host_stride = g->unit_bytes - g->tail_bytes;
  g->slot_stride = g->unit_bytes;  // packed: scattered 656-byte rows gather faster packed than padded to 768
  g->req_stride = ((int64_t)g->B + 1) * g->slot_stride;
  // the attention kernel addresses a request's rows with 32-bit offsets
  if (g->req_stride > (int64_t)UINT32_MAX) return fail(HS_ERR_UNSUPPORTED, "a request's slot rows exceed 4 GiB");
  g->flags = cfg->flags;
  g->policy = cfg->eviction;
  g->seed = cfg->eviction_seed;

  const size_t LN = (size_t)g->L * (size_t)g->n;
  size_t off = 0, sz = 0, t = 0;
  auto take = [&](size_t bytes, size_t* where) -> bool {
    *where = off;
    return add_ok(off, align_up(bytes), &off);
  };
  bool ok = true;
  ok = ok && take(sizeof(int32_t), &lay->err);
  ok = ok && mul_ok(LN, (size_t)cap, &t) && mul_ok(t, 4, &sz) && take(sz, &lay->pt);
  ok = ok && mul_ok(LN, (size_t)g->B, &t) && mul_ok(t, 4, &sz) && take(sz, &lay->rm);
  ok = ok && take(sz, &lay->st) && take(sz, &lay->ord);
  ok = ok && take(LN * 4, &lay->step);
  ok = ok && mul_ok(LN, (size_t)((g->B + 31) / 32) * 4, &sz) && take(sz, &lay->fresh);
  lay->part_floats = g->heads > 0 ? hs::attend_partial_floats(*g) : 0;
  ok = ok && mul_ok(LN, lay->part_floats, &t) && mul_ok(t, 4, &sz) && take(sz, &lay->part);
  ok = ok && mul_ok(LN, (size_t)g->k, &t) && mul_ok(t, 4, &sz) && take(sz, &lay->ml_tok) && take(sz, &lay->ml_slot);
  ok = ok && take(LN * 4, &lay->ml_cnt);
  ok = ok && mul_ok(LN, (size_t)g->req_stride, &sz) && take(sz, &lay->buf);
  lay->tail = 0;
  if (tail) ok = ok && mul_ok(LN, (size_t)cap, &t) && mul_ok(t, (size_t)g->tail_bytes, &sz) && take(sz, &lay->tail);
  lay->total = off;
  // no rows ever move in no-IO mode, so no host pool is allocated
  lay->host_total = 0;
  if (!(g->flags & HS_FLAG_NO_IO)) ok = ok && mul_ok(LN, (size_t)cap, &t) && mul_ok(t, (size_t)g->host_stride, &lay->host_total);
  if (!ok) return fail(HS_ERR_INVALID_ARG, "configuration sizes overflow");
  return HS_OK;
}

hs::LayerTables layer_tables(const hs_handle* h, int32_t layer) {
  const hs::Geometry& g = h->g;
  const size_t base = (size_t)layer * (size_t)g.n;
  hs::LayerTables t;
  t.pt = h->pt + base * (size_t)g.cap;
  t.rm = h->rm + base * (size_t)g.B;
  t.st = h->st + base * (size_t)g.B;
  t.ord = h->ord + base * (size_t)g.B;
  t.step = h->step + base;
  t.fresh = h->fresh + base * (size_t)((g.B + 31) / 32);
  t.part = h->part ? h->part + base * h->part_floats : nullptr;
  t.ml_tok = h->ml_tok + base * (size_t)g.k;
  t.ml_slot = h->ml_slot + base * (size_t)g.k;
  t.ml_cnt = h->ml_cnt + base;
  t.buf = h->buf + base * (size_t)g.req_stride;
  t.tail = h->tail ? h->tail + base * (size_t)g.cap * (size_t)g.tail_bytes : nullptr;
  return t;
}

void release(hs_handle* h) {
  if (!h) return;
  for (const hs_handle::Mark& m : h->marks) (void)hipEventDestroy(m.event);
  if (h->aux) (void)hipStreamDestroy(h->aux);
  if (h->host_pool) (void)hipHostFree(h->host_pool);
  if (h->own_dev && h->dev_block) (void)hipFree(h->dev_block);
  delete h;
}

constexpr size_t kMaxStreams = 16;

// Records, after work just enqueued on `s`, an event that hs_get_device_error / hs_destroy
// wait for.  Work enqueued during graph capture runs when the graph is launched, on a stream
// the handle never sees: the caller waits for it (a failure to query the capture state makes
// the handle fall back to device-wide waits).
void note_work(hs_handle* h, void* stream) {
  if (h->untracked) return;
  hipStream_t s = (hipStream_t)stream;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    h->untracked = true;
    return;
  }
  if (cs != hipStreamCaptureStatusNone) return;
  hipEvent_t ev = nullptr;
  for (const hs_handle::Mark& m : h->marks)
    if (m.stream == s) ev = m.event;
  if (!ev) {
    // no system-scope fence: these events only tell the host that the work has finished (the
    // error word is written by device-scope atomics, and freeing memory needs no visibility),
    // and a fenced record after every launch writes back the L2 and delays the stream's next
    // kernel by several microseconds
    if (h->marks.size() >= kMaxStreams ||
        hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess) {
      (void)hipGetLastError();
      h->untracked = true;
      return;
    }
    h->marks.push_back({s, ev});
  }
  if (hipEventRecord(ev, s) != hipSuccess) {
    (void)hipGetLastError();
    h->untracked = true;
  }
}

// Waits for the work this handle enqueued (see note_work).
hipError_t wait_own_work(hs_handle* h) {
  if (h->untracked) return hipDeviceSynchronize();
  for (const hs_handle::Mark& m : h->marks) {
    hipError_t e = hipEventSynchronize(m.event);
    if (e != hipSuccess) return e;
  }
  return h->aux ? hipStreamSynchronize(h->aux) : hipSuccess;
}

}  // namespace

extern "C" {

hs_status hs_device_bytes(const hs_config* cfg, size_t* bytes) {
  hs::Geometry g;
  Layout lay;
  if (!bytes) return fail(HS_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  hs_status s = plan(cfg, &g, &lay);
  if (s != HS_OK) return s;
  *bytes = lay.total;
  return HS_OK;
}

hs_status hs_host_bytes(const hs_config* cfg, size_t* bytes) {
  hs::Geometry g;
  Layout lay;
  if (!bytes) return fail(HS_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  hs_status s = plan(cfg, &g, &lay);
  if (s != HS_OK) return s;
  *bytes = lay.host_total;
  return HS_OK;
}

hs_status hs_create(const hs_config* cfg, hs_handle** out) {
  if (!out) return fail(HS_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  hs::Geometry g;
  Layout lay;
  hs_status s = plan(cfg, &g, &lay);
  if (s != HS_OK) return s;
  if (cfg->device_mem) {
    if (cfg->device_mem_bytes < lay.total) return fail(HS_ERR_INVALID_ARG, "device_mem smaller than hs_device_bytes()");
    if (((uintptr_t)cfg->device_mem) % kAlign) return fail(HS_ERR_INVALID_ARG, "device_mem must be 256-byte aligned");
  }

  hs_handle* h = new hs_handle();
  h->g = g;
  h->part_floats = lay.part_floats;
  h->lists_for.assign((size_t)g.L, 0);
  h->resident_for.assign((size_t)g.L, 0);
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) { release(h); return fail_hip(e, "hipGetDevice"); }
  e = hipStreamCreateWithFlags(&h->aux, hipStreamNonBlocking);
  if (e != hipSuccess) { h->aux = nullptr; release(h); return fail_hip(e, "hipStreamCreateWithFlags"); }
  if (cfg->device_mem) {
    h->dev_block = (uint8_t*)cfg->device_mem;
  } else {
    e = hipMalloc((void**)&h->dev_block, lay.total);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      release(h);
      return fail(HS_ERR_OUT_OF_MEMORY, "device allocation failed");
    }
    h->own_dev = true;
  }
  h->dev_bytes = lay.total;

  const char* inject = getenv("HS_FAULT_INJECT");
  if (inject && strcmp(inject, "host_alloc") == 0) {
    release(h);
    return fail(HS_ERR_OUT_OF_MEMORY, "pinned host allocation failed (injected)");
  }
  if (lay.host_total > 0) {
    e = hipHostMalloc((void**)&h->host_pool, lay.host_total, hipHostMallocMapped | hipHostMallocPortable);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      h->host_pool = nullptr;
      release(h);
      return fail(HS_ERR_OUT_OF_MEMORY, "pinned host allocation failed");
    }
    h->host_bytes = lay.host_total;
    e = hipHostGetDevicePointer((void**)&h->host_pool_dev, h->host_pool, 0);
    if (e != hipSuccess) { release(h); return fail_hip(e, "hipHostGetDevicePointer"); }
  }

  uint8_t* b = h->dev_block;
  h->err = (int32_t*)(b + lay.err);
  h->pt = (int32_t*)(b + lay.pt);
  h->rm = (int32_t*)(b + lay.rm);
  h->st = (int32_t*)(b + lay.st);
  h->ord = (int32_t*)(b + lay.ord);
  h->step = (int32_t*)(b + lay.step);
  h->fresh = (uint32_t*)(b + lay.fresh);
  h->part = lay.part_floats ? (float*)(b + lay.part) : nullptr;
  h->ml_tok = (int32_t*)(b + lay.ml_tok);
  h->ml_slot = (int32_t*)(b + lay.ml_slot);
  h->ml_cnt = (int32_t*)(b + lay.ml_cnt);
  h->buf = b + lay.buf;
  h->tail = g.tail_bytes ? b + lay.tail : nullptr;

  hs::prepare_resolve();
  hs::prepare_attend();
  // hs_attend_noalloc's static partials: their address on this device, resolved once per device
  h->noalloc_ready = hs::prepare_attend_noalloc(h->device);
  hs::prepare_append();
  hs::prepare_topk();
  // initialisation on the handle's own stream, waited for here: no device-wide synchronisation
  e = hipMemsetAsync(h->err, 0, sizeof(int32_t), h->aux);
  if (e == hipSuccess)  // the zero row after each request's slots
    e = hipMemset2DAsync(h->buf + (size_t)g.B * (size_t)g.slot_stride, (size_t)g.req_stride, 0,
                         (size_t)g.slot_stride, (size_t)g.L * (size_t)g.n, h->aux);
  if (e != hipSuccess) { (void)hipStreamSynchronize(h->aux); release(h); return fail_hip(e, "hipMemset"); }
  e = hs::launch_reset(g, h->pt, h->rm, h->st, h->ord, h->step, h->fresh, 0, g.n, h->aux);
  hipError_t e2 = hipStreamSynchronize(h->aux);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) { release(h); return fail_hip(e, "initialising tables"); }
  *out = h;
  return HS_OK;
}

namespace {

// Device-mapped address of a layer's host rows (null without a host pool, i.e. no-IO mode).
uint8_t* host_layer_of(const hs_handle* h, int32_t layer) {
  if (!h->host_pool_dev) return nullptr;
  return h->host_pool_dev + (size_t)layer * h->g.n * (size_t)h->g.cap * (size_t)h->g.host_stride;
}

hs_status resolve_impl(hs_handle* h, int32_t layer, int32_t n_req, const int32_t* d_sel, int32_t* d_slots,
                       int32_t* d_miss, bool list_only, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  if (n_req < 0 || n_req > h->g.n) return fail(HS_ERR_INVALID_ARG, "n_req out of range");
  if (n_req == 0) return HS_OK;
  if (!d_sel || !d_slots) return fail(HS_ERR_INVALID_ARG, "selection or slot pointer is NULL");
  hs::LayerTables t = layer_tables(h, layer);
  const uint8_t* host_layer = host_layer_of(h, layer);
  hipError_t e = hs::launch_resolve(h->g, t, layer, host_layer, n_req, d_sel, d_slots, d_miss, h->err, list_only,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "resolve launch");
  h->lists_for[layer] = (list_only && !(h->g.flags & HS_FLAG_NO_IO)) ? n_req : 0;
  h->resident_for[layer] = 0;
  note_work(h, stream);
  return HS_OK;
}

}  // namespace

hs_status hs_resolve(hs_handle* h, int32_t layer, int32_t n_req, const int32_t* d_sel, int32_t* d_slots,
                     int32_t* d_miss, void* stream) {
  return resolve_impl(h, layer, n_req, d_sel, d_slots, d_miss, false, stream);
}

hs_status hs_resolve_tables(hs_handle* h, int32_t layer, int32_t n_req, const int32_t* d_sel, int32_t* d_slots,
                            int32_t* d_miss, void* stream) {
  return resolve_impl(h, layer, n_req, d_sel, d_slots, d_miss, true, stream);
}

hs_status hs_fetch_misses(hs_handle* h, int32_t layer, int32_t n_req, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  if (n_req < 0 || n_req > h->g.n) return fail(HS_ERR_INVALID_ARG, "n_req out of range");
  if (h->g.flags & HS_FLAG_NO_IO) return HS_OK;  // no rows move
  // the lists must be this step's: a fused resolve, an append or a reset since the list-only
  // resolve has changed the tables, and replaying old lists would write rows into slots the
  // page table now gives to other tokens
  if (n_req > h->lists_for[layer])
    return fail(HS_ERR_INVALID_ARG, "no miss lists for these requests: hs_resolve_tables of this layer must come first");
  if (n_req == 0) return HS_OK;
  hs::LayerTables t = layer_tables(h, layer);
  const uint8_t* host_layer = host_layer_of(h, layer);
  hipError_t e = hs::launch_fetch(h->g, t, host_layer, n_req, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "fetch launch");
  note_work(h, stream);
  return HS_OK;
}

hs_status hs_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, void* stream) {
  if (!d_src || !d_sink) return fail(HS_ERR_INVALID_ARG, "source or sink pointer is NULL");
  if (bytes % 16 != 0 || ((uintptr_t)d_src & 15u) != 0)
    return fail(HS_ERR_INVALID_ARG, "bytes must be a multiple of 16 and the source 16-byte aligned");
  if (bytes == 0) return HS_OK;
  hipError_t e = hs::launch_stream_read(d_src, bytes, d_sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "stream read launch");
  return HS_OK;
}

hs_status hs_attend(hs_handle* h, int32_t layer, int32_t n_req, const void* d_q, const int32_t* d_slots, float scale,
                    void* d_out, float* d_lse, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (h->g.heads == 0) return fail(HS_ERR_UNSUPPORTED, "handle created with num_heads = 0");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  if (n_req < 0 || n_req > h->g.n) return fail(HS_ERR_INVALID_ARG, "n_req out of range");
  if (n_req == 0) return HS_OK;
  if (!d_q || !d_slots || !d_out) return fail(HS_ERR_INVALID_ARG, "query, slot or output pointer is NULL");
  hs::LayerTables t = layer_tables(h, layer);
  hipError_t e =
      hs::launch_attend(h->g, t, n_req, d_q, d_slots, nullptr, nullptr, scale, d_out, d_lse, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "attend launch");
  h->resident_for[layer] = 0;  // a split launch reuses the layer's partial space
  note_work(h, stream);
  return HS_OK;
}

hs_status hs_attend_pages(hs_handle* h, int32_t layer, int32_t n_req, const void* d_q, const int32_t* d_slots,
                          const int32_t* d_sel, const int32_t* d_len, float scale, void* d_out, float* d_lse,
                          void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (h->g.heads == 0) return fail(HS_ERR_UNSUPPORTED, "handle created with num_heads = 0");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  if (n_req < 0 || n_req > h->g.n) return fail(HS_ERR_INVALID_ARG, "n_req out of range");
  if (n_req == 0) return HS_OK;
  if (!d_q || !d_slots || !d_out) return fail(HS_ERR_INVALID_ARG, "query, slot or output pointer is NULL");
  if (!d_sel || !d_len) return fail(HS_ERR_INVALID_ARG, "selection or length pointer is NULL");
  hs::LayerTables t = layer_tables(h, layer);
  hipError_t e =
      hs::launch_attend(h->g, t, n_req, d_q, d_slots, d_sel, d_len, scale, d_out, d_lse, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "attend launch");
  h->resident_for[layer] = 0;  // a split launch reuses the layer's partial space
  note_work(h, stream);
  return HS_OK;
}

hs_status hs_attend_noalloc(hs_handle* h, int32_t layer, int32_t n_req, int32_t num_heads, const void* d_q,
                            const int32_t* d_slots, float scale, void* d_out, float* d_lse, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  if (n_req < 0 || n_req > h->g.n) return fail(HS_ERR_INVALID_ARG, "n_req out of range");
  if (num_heads < 1 || num_heads > 16) return fail(HS_ERR_INVALID_ARG, "num_heads must lie in [1, 16]");
  if (n_req == 0) return HS_OK;
  if (!d_q || !d_slots || !d_out) return fail(HS_ERR_INVALID_ARG, "query, slot or output pointer is NULL");
  if ((int64_t)h->g.k * h->g.P > 65536)
    return fail(HS_ERR_UNSUPPORTED, "attention over more than 65536 tokens (top_k * page_tokens)");
  const int64_t need = hs::attend_noalloc_partials(h->g, n_req, num_heads);
  if (need > hs::kNoallocPartials)
    return fail(HS_ERR_UNSUPPORTED, "this launch needs " + std::to_string(need) +
                                        " split partials; the static scratch holds " +
                                        std::to_string(hs::kNoallocPartials) + " (use fewer requests or hs_attend)");
  if (h->noalloc_ready != hipSuccess) return fail_hip(h->noalloc_ready, "resolving the static scratch");
  hs::LayerTables t = layer_tables(h, layer);
  hipError_t e = hs::launch_attend_noalloc(h->g, t, h->device, n_req, num_heads, d_q, d_slots, scale, d_out, d_lse,
                                           (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "attend launch");
  note_work(h, stream);
  return HS_OK;
}

hs_status hs_attend_resident(hs_handle* h, int32_t layer, int32_t n_req, const void* d_q, const int32_t* d_slots,
                             const int32_t* d_sel, const int32_t* d_len, float scale, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (h->g.heads == 0) return fail(HS_ERR_UNSUPPORTED, "handle created with num_heads = 0");
  if (h->g.flags & HS_FLAG_NO_IO) return fail(HS_ERR_UNSUPPORTED, "no miss copy to overlap with HS_FLAG_NO_IO");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  if (n_req < 0 || n_req > h->g.n) return fail(HS_ERR_INVALID_ARG, "n_req out of range");
  if (n_req > h->lists_for[layer])
    return fail(HS_ERR_INVALID_ARG, "no miss lists for these requests: hs_resolve_tables of this layer must come first");
  if (n_req == 0) return HS_OK;
  if (!d_q || !d_slots) return fail(HS_ERR_INVALID_ARG, "query or slot pointer is NULL");
  if (!d_sel != !d_len) return fail(HS_ERR_INVALID_ARG, "selection and length pointers: give both or neither");
  hs::LayerTables t = layer_tables(h, layer);
  hipError_t e = hs::launch_attend_part(h->g, t, n_req, false, d_q, d_slots, d_sel, d_len, scale, nullptr, nullptr,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "attend launch");
  h->resident_for[layer] = n_req;
  note_work(h, stream);
  return HS_OK;
}

hs_status hs_attend_fetched(hs_handle* h, int32_t layer, int32_t n_req, const void* d_q, const int32_t* d_len,
                            float scale, void* d_out, float* d_lse, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (h->g.heads == 0) return fail(HS_ERR_UNSUPPORTED, "handle created with num_heads = 0");
  if (h->g.flags & HS_FLAG_NO_IO) return fail(HS_ERR_UNSUPPORTED, "no miss copy to overlap with HS_FLAG_NO_IO");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  if (n_req < 0 || n_req > h->g.n) return fail(HS_ERR_INVALID_ARG, "n_req out of range");
  if (n_req > h->lists_for[layer])
    return fail(HS_ERR_INVALID_ARG, "no miss lists for these requests: hs_resolve_tables of this layer must come first");
  // the partial strides depend on n_req, so the resident part must have covered exactly these requests
  if (n_req != 0 && n_req != h->resident_for[layer])
    return fail(HS_ERR_INVALID_ARG,
                "no resident partials for these requests: hs_attend_resident of this layer with the same n_req must "
                "come first");
  if (n_req == 0) return HS_OK;
  if (!d_q || !d_out) return fail(HS_ERR_INVALID_ARG, "query or output pointer is NULL");
  hs::LayerTables t = layer_tables(h, layer);
  hipError_t e = hs::launch_attend_part(h->g, t, n_req, true, d_q, nullptr, nullptr, d_len, scale, d_out, d_lse,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "attend launch");
  note_work(h, stream);
  return HS_OK;
}

hs_status hs_destroy(hs_handle* h) {
  if (!h) return HS_OK;
  hipError_t e = wait_own_work(h);
  release(h);
  if (e != hipSuccess) return fail_hip(e, "waiting for the handle's work");
  return HS_OK;
}

hs_status hs_host_kv(hs_handle* h, int32_t layer, int32_t request, void** ptr, int64_t* capacity, int64_t* row_stride) {
  if (!h || !ptr) return fail(HS_ERR_INVALID_ARG, "handle or ptr is NULL");
  if (layer < 0 || layer >= h->g.L || request < 0 || request >= h->g.n)
    return fail(HS_ERR_INVALID_ARG, "layer or request out of range");
  if (!h->host_pool) return fail(HS_ERR_UNSUPPORTED, "no host pool in no-IO mode");
  const size_t units = ((size_t)layer * h->g.n + (size_t)request) * (size_t)h->g.cap;
  *ptr = h->host_pool + units * (size_t)h->g.host_stride;
  if (capacity) *capacity = h->g.cap * h->g.P;   // token rows
  if (row_stride) *row_stride = h->g.host_stride / h->g.P;
  return HS_OK;
}

hs_status hs_device_state(hs_handle* h, int32_t layer, hs_state_view* v) {
  if (!h || !v) return fail(HS_ERR_INVALID_ARG, "handle or view is NULL");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  hs::LayerTables t = layer_tables(h, layer);
  v->page_table = t.pt;
  v->slot_owner = t.rm;
  v->slot_stamp = t.st;
  v->lru_order = t.ord;
  v->step = t.step;
  v->kv_buffer = t.buf;
  v->capacity = h->g.cap;
  v->slot_stride = h->g.slot_stride;
  v->entry_bytes = h->g.entry_bytes;
  v->request_stride = h->g.req_stride;
  v->page_tokens = h->g.P;
  v->fresh_slots = t.fresh;
  v->tail_plane = t.tail;
  v->tail_bytes = h->g.tail_bytes;
  return HS_OK;
}

hs_status hs_append(hs_handle* h, int32_t layer, int32_t n_req, const int32_t* d_pos, const void* d_rows,
                    int64_t row_stride, int32_t* d_slot_out, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  if (n_req < 0 || n_req > h->g.n) return fail(HS_ERR_INVALID_ARG, "n_req out of range");
  if (h->g.policy == HS_EVICT_RANDOM && h->g.P == 1)
    return fail(HS_ERR_UNSUPPORTED, "append needs a stamp-ordered eviction policy (LRU or FIFO)");
  if (n_req == 0) return HS_OK;
  if (!d_pos || !d_rows) return fail(HS_ERR_INVALID_ARG, "position or row pointer is NULL");
  if (row_stride < h->g.entry_bytes || row_stride % 16 || ((uintptr_t)d_rows) % 16)
    return fail(HS_ERR_INVALID_ARG, "rows must be 16-byte aligned, row_stride >= entry bytes and a multiple of 16");
  hs::LayerTables t = layer_tables(h, layer);
  uint8_t* host_layer = host_layer_of(h, layer);
  hipError_t e = h->g.P == 1 ? hs::launch_append(h->g, t, host_layer, n_req, d_pos, d_rows, row_stride, d_slot_out,
                                                 h->err, (hipStream_t)stream)
                             : hs::launch_append_pages(h->g, t, host_layer, n_req, d_pos, d_rows, row_stride,
                                                       d_slot_out, h->err, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "append launch");
  h->lists_for[layer] = 0;
  h->resident_for[layer] = 0;
  note_work(h, stream);
  return HS_OK;
}

hs_status hs_offload(hs_handle* h, int32_t layer, int32_t request, int64_t first, int64_t count,
                     const void* d_rows, int64_t row_stride, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (layer < 0 || layer >= h->g.L) return fail(HS_ERR_INVALID_ARG, "layer out of range");
  if (request < 0 || request >= h->g.n) return fail(HS_ERR_INVALID_ARG, "request out of range");
  const int64_t cap_tokens = h->g.cap * h->g.P;
  if (first < 0 || count < 0 || first > cap_tokens - count) return fail(HS_ERR_INVALID_ARG, "positions out of range");
  if (!h->host_pool) return fail(HS_ERR_UNSUPPORTED, "no host pool in no-IO mode");
  if (count == 0) return HS_OK;
  if (!d_rows) return fail(HS_ERR_INVALID_ARG, "row pointer is NULL");
  if (row_stride < h->g.entry_bytes) return fail(HS_ERR_INVALID_ARG, "row_stride below the entry size");
  const size_t E = (size_t)h->g.entry_bytes;
  const size_t T = (size_t)h->g.tail_bytes;  // bytes of each row kept in the device tail plane
  const size_t HE = E - T;                    // bytes of each row in the host pool
  const size_t row0 = ((size_t)layer * h->g.n + (size_t)request) * (size_t)cap_tokens + (size_t)first;
  const size_t off = row0 * HE;
  uint8_t* tail_dst = T ? h->tail + row0 * T : nullptr;
  // Contiguous rows go as one flat copy (the DMA engine's fast path, no compute units);
  // 16-byte-aligned padded rows, and rows split between the host pool and the tail plane,
  // through a zero-copy store kernel (a 2-D copy of small rows runs at about a third of the
  // link); anything else as 2-D copies.
  hipError_t e;
  if ((size_t)row_stride == E && T == 0)
    e = hipMemcpyAsync(h->host_pool + off, d_rows, E * (size_t)count, hipMemcpyDeviceToHost, (hipStream_t)stream);
  else if (row_stride % 16 == 0 && ((uintptr_t)d_rows) % 16 == 0)
    e = hs::launch_offload(d_rows, row_stride, h->host_pool_dev + off, count, h->g.entry_bytes, tail_dst,
                           h->g.tail_bytes, (hipStream_t)stream);
  else {
    e = hipMemcpy2DAsync(h->host_pool + off, HE, d_rows, (size_t)row_stride, HE, (size_t)count, hipMemcpyDeviceToHost,
                         (hipStream_t)stream);
    if (e == hipSuccess && T)
      e = hipMemcpy2DAsync(tail_dst, T, (const uint8_t*)d_rows + HE, (size_t)row_stride, T, (size_t)count,
                           hipMemcpyDeviceToDevice, (hipStream_t)stream);
  }
  if (e != hipSuccess) return fail_hip(e, "offload copy");
  note_work(h, stream);
  return HS_OK;
}

namespace {

hs_status topk_impl(hs_handle* h, int32_t n_req, const float* d_scores, int64_t score_stride, const int32_t* d_len,
                    int32_t* d_sel, int32_t* d_hint, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (n_req < 0 || n_req > h->g.n) return fail(HS_ERR_INVALID_ARG, "n_req out of range");
  if (n_req == 0) return HS_OK;
  if (!d_scores || !d_len || !d_sel) return fail(HS_ERR_INVALID_ARG, "score, length or output pointer is NULL");
  if (score_stride < 4 || score_stride % 4 || ((uintptr_t)d_scores) % 16)
    return fail(HS_ERR_INVALID_ARG, "scores must be 16-byte aligned with a row stride that is a multiple of 4");
  hipError_t e =
      hs::launch_topk(h->g, n_req, d_scores, score_stride, d_len, d_sel, d_hint, h->err, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "top-k launch");
  note_work(h, stream);
  return HS_OK;
}

}  // namespace

hs_status hs_topk(hs_handle* h, int32_t n_req, const float* d_scores, int64_t score_stride, const int32_t* d_len,
                  int32_t* d_sel, void* stream) {
  return topk_impl(h, n_req, d_scores, score_stride, d_len, d_sel, nullptr, stream);
}

hs_status hs_topk_hinted(hs_handle* h, int32_t n_req, const float* d_scores, int64_t score_stride,
                         const int32_t* d_len, int32_t* d_sel, int32_t* d_hint, void* stream) {
  if (h && n_req > 0 && !d_hint) return fail(HS_ERR_INVALID_ARG, "hint pointer is NULL (use hs_topk)");
  return topk_impl(h, n_req, d_scores, score_stride, d_len, d_sel, d_hint, stream);
}

hs_status hs_reset_requests(hs_handle* h, int32_t first, int32_t count, void* stream) {
  if (!h) return fail(HS_ERR_INVALID_ARG, "handle is NULL");
  if (first < 0 || count < 0 || (int64_t)first + count > h->g.n) return fail(HS_ERR_INVALID_ARG, "request range");
  if (count == 0) return HS_OK;
  hipError_t e =
      hs::launch_reset(h->g, h->pt, h->rm, h->st, h->ord, h->step, h->fresh, first, count, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "reset launch");
  h->lists_for.assign((size_t)h->g.L, 0);
  h->resident_for.assign((size_t)h->g.L, 0);
  note_work(h, stream);
  return HS_OK;
}

hs_status hs_get_device_error(hs_handle* h, int32_t* bits) {
  if (!h || !bits) return fail(HS_ERR_INVALID_ARG, "handle or bits is NULL");
  // waits for the handle's own work only (see note_work), then reads and clears the word on the
  // handle's private stream
  int32_t v = 0;
  hipError_t e = wait_own_work(h);
  if (e == hipSuccess) e = hipMemcpyAsync(&v, h->err, sizeof(int32_t), hipMemcpyDeviceToHost, h->aux);
  if (e == hipSuccess) e = hipMemsetAsync(h->err, 0, sizeof(int32_t), h->aux);
  hipError_t e2 = hipStreamSynchronize(h->aux);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) return fail_hip(e, "reading the device error word");
  *bits = v;
  return HS_OK;
}

const char* hs_status_string(hs_status s) {
  switch (s) {
    case HS_OK: return "ok";
    case HS_ERR_INVALID_ARG: return "invalid argument";
    case HS_ERR_OUT_OF_MEMORY: return "out of memory";
    case HS_ERR_UNSUPPORTED: return "unsupported";
    case HS_ERR_HIP: return "HIP runtime error";
    case HS_ERR_DEVICE: return "device reported invalid input";
  }
  return "unknown status";
}

const char* hs_last_error_message(void) { return g_msg.c_str(); }

}  // extern "C"
