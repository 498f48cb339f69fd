// Write-through append of newly generated tokens.
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
  int32_t* err;
  int64_t cap, host_stride, slot_stride, req_stride;
  int32_t B, chunks, io;
};

__global__ __launch_bounds__(AT) void append_kernel(AppendArgs a) {
  extern __shared__ int32_t ord_lds[];  // [B]
  __shared__ int32_t s_pj, s_c;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t p = a.pos[r];
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
  const int B = a.B;
  int32_t* pt = a.pt + (int64_t)r * a.cap;
  int32_t* rm = a.rm + (int64_t)r * B;
  int32_t* st = a.st + (int64_t)r * B;
  int32_t* ord = a.ord + (int64_t)r * B;
  const int32_t t = a.step[r];
  const int32_t jr = pt[p];
  const bool resident = jr >= 0;
  const int32_t j = resident ? jr : ord[0];  // least recently used: first in (stamp, slot) order

  if (tid == 0) s_c = 0;
  __syncthreads();
  // stage the order array; find j's position; count the slots of stamp t above j, which stay
  // behind it
  int c = 0;
  for (int i = tid; i < B; i += AT) {
    const int32_t s = ord[i];
    ord_lds[i] = s;
    if (s == j) s_pj = i;
    else if (s > j && st[s] == t) ++c;
  }
  if (c) atomicAdd(&s_c, c);
  __syncthreads();
  const int pj = s_pj;
  const int q = B - 1 - s_c;  // j's new position (>= pj)
  for (int i = pj + tid; i < q; i += AT) ord[i] = ord_lds[i + 1];
  if (tid == 0) {
    ord[q] = j;
    if (!resident) {
      const int32_t old = rm[j];
      if (old >= 0) pt[old] = -1;
      pt[p] = j;
      rm[j] = p;
    }
    st[j] = t;
    // the next resolve must treat this slot as touched: its stamp is already that step's
    atomicOr(a.fresh + (int64_t)r * ((B + 31) >> 5) + (j >> 5), 1u << (j & 31));
    if (a.slot_out) a.slot_out[r] = j;
  }
  if (a.io) {
    const v4i* src = (const v4i*)(a.rows + (int64_t)r * a.row_stride);
    v4i* dev = (v4i*)(a.buf + (int64_t)r * a.req_stride + (int64_t)j * a.slot_stride);
    v4i* hst = (v4i*)(a.host + ((int64_t)r * a.cap + p) * a.host_stride);
    for (int i = tid; i < a.chunks; i += AT) {
      const v4i v = src[i];
      dev[i] = v;
      hst[i] = v;
    }
  }
}

}  // namespace

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
  a.err = err;
  a.cap = g.cap;
  a.host_stride = g.host_stride;
  a.slot_stride = g.slot_stride;
  a.req_stride = g.req_stride;
  a.B = g.B;
  a.chunks = (int32_t)(g.entry_bytes / 16);
  a.io = (g.flags & HS_FLAG_NO_IO) ? 0 : 1;
  hipLaunchKernelGGL(append_kernel, dim3(n_req), dim3(AT), (size_t)g.B * sizeof(int32_t), s, a);
  return hipGetLastError();
}

}  // namespace hs
