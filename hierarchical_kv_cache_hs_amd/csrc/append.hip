// Write-through append of newly generated tokens (LRU and FIFO eviction; under FIFO a token
// that is already resident only has its row rewritten).
//
// What is computed (the HiSparse note's introduction: KV that is not in use is actively
// offloaded to host memory; paper abstract: each request keeps its full KV history in host
// memory): for every request r with a new token p = pos[r] (-1 = none), the token's row is
// written to position p of the request's history in the pinned host pool, and the token is
// made resident before the next resolve.  It keeps its slot if it has one; otherwise it takes
// the first slot in (stamp, slot) order -- empty slots first -- whose token leaves the page
// table.  The slot is stamped with the step the next resolve will use.
//
// The LRU order array stays sorted by (stamp, slot): the slot leaves its position and
// re-enters behind every slot that now precedes it -- all slots of smaller stamps and the
// slots of the same (newest) stamp with a smaller index.  The victim of a non-resident token
// is the array's first entry.  One workgroup per request; the array is staged in LDS for the
// shift.
//
// With pages of P tokens (paper abstract: NSA and Quest select blocks of tokens) the append
// writes through only: the row goes to the history, and into its page's slot at row offset
// p mod P when that page is resident.  No table changes -- a page that is not resident is
// fetched whole, new row included, the next time a selection names it.

#include "hs_internal.h"

namespace hs {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int AT = 256;

struct AppendArgs {
  const int32_t* pos;     // [n_req]
  const uint8_t* rows;    // [n_req] rows of entry bytes, row_stride apart (device)
  int64_t row_stride;
  int32_t* slot_out;      // [n_req] or null
  int32_t* pt;            // layer tables
  int32_t* rm;
  int32_t* st;
  int32_t* ord;
  const int32_t* step;
  uint32_t* fresh;        // [n][B/32] slots appended since the last resolve
  uint8_t* buf;
  uint8_t* host;          // the layer's host pool, device-mapped address
  uint8_t* tail;          // the layer's tail plane (HS_FLAG_RESIDENT_TAIL), else null
  int32_t* err;
  int64_t cap, host_stride, slot_stride, req_stride;
  int32_t B, chunks, io, fifo;
  int32_t body_chunks;    // chunks of a row kept in the host pool; the rest go to the tail plane
};

// Writes chunk c of token p's row into request r's history: the host pool, or for the chunks
// past the host part of a row the device-resident tail plane.
__device__ __forceinline__ void store_history(const AppendArgs& a, int r, int32_t p, int c, v4i v) {
  const int64_t row = (int64_t)r * a.cap + p;
  if (c < a.body_chunks) ((v4i*)(a.host + row * a.host_stride))[c] = v;
  else ((v4i*)(a.tail + row * (int64_t)(a.chunks - a.body_chunks) * 16))[c - a.body_chunks] = v;
}

__global__ __launch_bounds__(AT) void append_kernel(AppendArgs a) {
  extern __shared__ int32_t ord_lds[];  // [B]
  __shared__ int32_t s_pj, s_c;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int B = a.B;
  int32_t* pt = a.pt + (int64_t)r * a.cap;
  int32_t* rm = a.rm + (int64_t)r * B;
  int32_t* st = a.st + (int64_t)r * B;
  int32_t* ord = a.ord + (int64_t)r * B;
  // Round trip 1: the position, the step, this thread's 16 bytes of the row and the order
  // array -- none depends on another.  Batches of order loads are all issued before any is
  // stored (a loop of load-store pairs would wait for each load in turn).
  const int32_t p = a.pos[r];
  const int32_t t = a.step[r];
  v4i rowv = {0, 0, 0, 0};
  if (a.io && tid < a.chunks) rowv = ((const v4i*)(a.rows + (int64_t)r * a.row_stride))[tid];
  constexpr int BATCH = 16;
  for (int i0 = 0; i0 < B; i0 += AT * BATCH) {
    int32_t v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int i = i0 + u * AT + tid;
      v[u] = (i < B) ? ord[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int i = i0 + u * AT + tid;
      if (i < B) ord_lds[i] = v[u];
    }
  }
  if (p == -1) {
    if (tid == 0 && a.slot_out) a.slot_out[r] = -1;
    return;
  }
  if (p < 0 || (int64_t)p >= a.cap) {
    if (tid == 0) {
      atomicOr(a.err, (int32_t)HS_DEVERR_TOKEN_RANGE);
      if (a.slot_out) a.slot_out[r] = -1;
    }
    return;
  }
  if (tid == 0) {
    s_pj = 0;
    s_c = 0;
  }
  __syncthreads();
  // Round trip 2: the page-table entry, the first slot's owner (the victim's, if the token
  // is not resident) and the stamps of the last AT slots of the order.  Slots stamped t
  // (appended since the last resolve) form the tail of the order.
  const int32_t jr = pt[p];
  const int32_t lru = ord_lds[0];
  const int32_t lru_owner = rm[lru];
  int32_t tail_slot = -1;
  bool newest = false;
  if (tid < B) {
    tail_slot = ord_lds[B - 1 - tid];
    newest = st[tail_slot] == t;
  }
  const bool resident = jr >= 0;
  const int32_t j = resident ? jr : lru;  // least recently used: first in (stamp, slot) order
  if (a.fifo && resident) {
    // FIFO: rewriting a resident token is no refill -- its slot keeps its stamp and place
    if (tid == 0 && a.slot_out) a.slot_out[r] = j;
    if (a.io && tid < a.chunks) {
      ((v4i*)(a.buf + (int64_t)r * a.req_stride + (int64_t)j * a.slot_stride))[tid] = rowv;
      store_history(a, r, p, tid, rowv);
    }
    return;
  }
  if (resident)
    for (int i = tid; i < B; i += AT)
      if (ord_lds[i] == j) s_pj = i;
  // the slots of stamp t above j stay behind it
  int c = (newest && tail_slot > j) ? 1 : 0;
  if (__syncthreads_and(tid >= B || newest)) {
    // the tail is longer than one chunk (many appends since the last resolve): walk on
    for (int base = B - 1 - AT; base >= 0; base -= AT) {
      const int i = base - tid;
      bool nw = false;
      if (i >= 0) {
        const int32_t sl = ord_lds[i];
        nw = st[sl] == t;
        if (nw && sl > j) ++c;
      }
      if (!__syncthreads_and(i < 0 || nw)) break;
    }
  }
  if (c) atomicAdd(&s_c, c);
  __syncthreads();
  const int pj = s_pj;
  const int q = B - 1 - s_c;  // j's new position (>= pj)
  for (int i = pj + tid; i < q; i += AT) ord[i] = ord_lds[i + 1];
  if (tid == 0) {
    ord[q] = j;
    if (!resident) {
      if (lru_owner >= 0) pt[lru_owner] = -1;
      pt[p] = j;
      rm[j] = p;
    }
    st[j] = t;
    // the next resolve must treat this slot as touched: its stamp is already that step's
    atomicOr(a.fresh + (int64_t)r * ((B + 31) >> 5) + (j >> 5), 1u << (j & 31));
    if (a.slot_out) a.slot_out[r] = j;
  }
  if (a.io && tid < a.chunks) {
    ((v4i*)(a.buf + (int64_t)r * a.req_stride + (int64_t)j * a.slot_stride))[tid] = rowv;
    store_history(a, r, p, tid, rowv);
  }
}

// Prefill offload of rows that are not contiguous (a padded row stride) or that are split
// between the pinned history and the tail plane: a grid of small workgroups copies 16-byte
// chunks from the device rows, the first body_chunks of each row to the pinned history with
// zero-copy stores (rows packed), the rest to the tail plane (packed), four chunks in flight
// per thread.
constexpr int OT = 256;

__global__ __launch_bounds__(OT) void offload_kernel(const uint8_t* __restrict__ src, int64_t src_stride,
                                                     uint8_t* __restrict__ dst, int64_t count, int32_t chunks,
                                                     int32_t body_chunks, uint8_t* __restrict__ tail) {
  const int64_t total = count * chunks;
  const int64_t step = (int64_t)gridDim.x * OT;
  constexpr int U = 4;
  for (int64_t base = (int64_t)blockIdx.x * OT + threadIdx.x; base < total; base += step * U) {
    v4i v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t idx = base + u * step;
      if (idx < total) {
        const int64_t row = idx / chunks;
        v[u] = ((const v4i*)(src + row * src_stride))[idx - row * chunks];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t idx = base + u * step;
      if (idx < total) {
        const int64_t row = idx / chunks;
        const int c = (int)(idx - row * chunks);
        if (c < body_chunks) ((v4i*)dst)[row * body_chunks + c] = v[u];
        else ((v4i*)tail)[row * (chunks - body_chunks) + (c - body_chunks)] = v[u];
      }
    }
  }
}

// Page-granular write-through: one wave per request, 16 bytes per lane and step.
constexpr int PT_THREADS = 64;

__global__ __launch_bounds__(PT_THREADS) void append_pages_kernel(
    const int32_t* __restrict__ pos, const uint8_t* __restrict__ rows, int64_t row_stride,
    const int32_t* __restrict__ pt, int64_t cap, int32_t lgP, int32_t B, uint8_t* __restrict__ buf, int64_t req_stride,
    int64_t slot_stride, uint8_t* __restrict__ host, int64_t entry_bytes, int32_t* __restrict__ slot_out,
    int32_t* __restrict__ err) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t p = pos[r];
  const int64_t cap_tokens = cap << lgP;
  int32_t j = -1;
  if (p >= 0 && (int64_t)p < cap_tokens) {
    const int32_t c = p >> lgP;
    const int32_t o = p & ((1 << lgP) - 1);
    const int32_t v = pt[(int64_t)r * cap + c];
    j = (v >= 0 && v < B) ? v : -1;
    const int chunks = (int)(entry_bytes / 16);
    const v4i* src = (const v4i*)(rows + (int64_t)r * row_stride);
    v4i* hdst = host ? (v4i*)(host + ((int64_t)r * cap_tokens + p) * entry_bytes) : nullptr;
    v4i* ddst = j >= 0 ? (v4i*)(buf + (int64_t)r * req_stride + (int64_t)j * slot_stride + (int64_t)o * entry_bytes)
                       : nullptr;
    for (int i = tid; i < chunks; i += PT_THREADS) {
      const v4i x = src[i];
      if (hdst) hdst[i] = x;
      if (ddst) ddst[i] = x;
    }
  } else if (p != -1 && tid == 0) {
    atomicOr(err, HS_DEVERR_TOKEN_RANGE);
  }
  if (tid == 0 && slot_out) slot_out[r] = j;
}

}  // namespace

hipError_t launch_append_pages(const Geometry& g, const LayerTables& t, uint8_t* host_layer, int32_t n_req,
                               const int32_t* pos, const void* rows, int64_t row_stride, int32_t* slot_out,
                               int32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(append_pages_kernel, dim3(n_req), dim3(PT_THREADS), 0, s, pos, (const uint8_t*)rows, row_stride,
                     t.pt, g.cap, g.lgP, g.B, t.buf, g.req_stride, g.slot_stride,
                     (g.flags & HS_FLAG_NO_IO) ? nullptr : host_layer, g.entry_bytes, slot_out, err);
  return hipGetLastError();
}

hipError_t launch_offload(const void* src, int64_t src_stride, uint8_t* dst_mapped, int64_t count, int64_t entry_bytes,
                          uint8_t* tail_dst, int64_t tail_bytes, hipStream_t s) {
  const int32_t chunks = (int32_t)(entry_bytes / 16);
  const int32_t body_chunks = (int32_t)((entry_bytes - tail_bytes) / 16);
  const int64_t total = count * chunks;
  const int64_t blocks = (total + OT * 4 - 1) / (OT * 4);
  hipLaunchKernelGGL(offload_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(OT), 0, s,
                     (const uint8_t*)src, src_stride, dst_mapped, count, chunks, body_chunks, tail_dst);
  return hipGetLastError();
}

void prepare_append() {
  (void)hipFuncSetAttribute((const void*)append_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(kMaxBuffer * sizeof(int32_t)));
  (void)hipGetLastError();
}

hipError_t launch_append(const Geometry& g, const LayerTables& t, uint8_t* host_layer, int32_t n_req,
                         const int32_t* pos, const void* rows, int64_t row_stride, int32_t* slot_out, int32_t* err,
                         hipStream_t s) {
  AppendArgs a;
  a.pos = pos;
  a.rows = (const uint8_t*)rows;
  a.row_stride = row_stride;
  a.slot_out = slot_out;
  a.pt = t.pt;
  a.rm = t.rm;
  a.st = t.st;
  a.ord = t.ord;
  a.step = t.step;
  a.fresh = t.fresh;
  a.buf = t.buf;
  a.host = host_layer;
  a.tail = t.tail;
  a.err = err;
  a.cap = g.cap;
  a.host_stride = g.host_stride;
  a.slot_stride = g.slot_stride;
  a.req_stride = g.req_stride;
  a.B = g.B;
  a.chunks = (int32_t)(g.entry_bytes / 16);
  a.body_chunks = (int32_t)((g.entry_bytes - g.tail_bytes) / 16);
  a.io = (g.flags & HS_FLAG_NO_IO) ? 0 : 1;
  a.fifo = g.policy == HS_EVICT_FIFO ? 1 : 0;
  hipLaunchKernelGGL(append_kernel, dim3(n_req), dim3(AT), (size_t)g.B * sizeof(int32_t), s, a);
  return hipGetLastError();
}

}  // namespace hs
