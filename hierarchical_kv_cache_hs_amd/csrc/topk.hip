// Top-k selection from indexer scores: the step that feeds the resolver.
//
// What is computed (the HiSparse note, section 2: the serving backend's indexer decides which
// KV entries a step selects; paper abstract: the method is indexer-agnostic): for every
// request r, among positions 0 .. len[r]-1 of its score row, the k positions of largest
// score -- a tie going to the smaller position -- written in ascending position order; when
// len[r] < k every position is selected and the row is padded with -1.
//
// Design for gfx950.  One 1024-thread workgroup per request.  Scores map to 32-bit keys whose
// unsigned order is the float order (-0 folded onto +0, so equal floats give equal keys).  A
// most-significant-digit radix select finds the k-th largest key in three histogram passes
// (12, 12 and 8 bits; LDS histograms, one digit group per thread for the search) and with it
// how many of the keys equal to it are taken.  A last pass walks the positions in order; two
// block scans per tile give each tied key its rank among ties and each selected position its
// output index, so the output comes out sorted with no sort.  Four reads of the score row;
// after the first they come from the L2 / last-level cache for the row sizes here.

#include "hs_internal.h"

namespace hs {
namespace {

constexpr int TT = 1024;       // threads per workgroup
constexpr int TW = TT / 64;    // waves
constexpr int V = 4;           // positions per thread per tile (one 16-byte load)
constexpr int TILE = TT * V;
constexpr int NBIN = 4096;     // 12-bit digits
static_assert(NBIN == 4 * TT, "one group of four bins per thread");

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;  // -0 equals +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive scan of v over the workgroup; *total gets the sum.  Every thread must call.
__device__ uint32_t block_scan_incl(uint32_t v, uint32_t* wtot, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const uint32_t x = wtot[i];
    base += (i < w) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return v + base;
}

struct TopkArgs {
  const float* scores;
  int64_t stride;      // floats between request rows (multiple of 4)
  const int32_t* len;  // [n]
  int32_t* sel;        // [n][k]
  int32_t* err;
  int64_t cap;
  int32_t k;
};

__global__ __launch_bounds__(TT) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[NBIN];
  __shared__ uint32_t wtot[TW];
  __shared__ uint32_t s_digit, s_above;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = a.k;
  int32_t* out = a.sel + (int64_t)r * k;
  int64_t len = a.len[r];
  if (len < 0 || len > a.cap || len > a.stride) {
    if (tid == 0) atomicOr(a.err, (int32_t)HS_DEVERR_TOKEN_RANGE);
    for (int i = tid; i < k; i += TT) out[i] = -1;
    return;
  }
  if (len <= k) {  // every position, then padding
    for (int i = tid; i < k; i += TT) out[i] = (i < len) ? i : -1;
    return;
  }
  const float* row = a.scores + (int64_t)r * a.stride;

  // ---- radix select: digits of 12, 12 and 8 bits from the top
  uint32_t prefix = 0;  // key bits fixed so far
  uint32_t need = (uint32_t)k;  // keys still to take among those matching the prefix
  int fixed = 0;        // number of fixed bits
  for (int level = 0; level < 3; ++level) {
    const int bits = level < 2 ? 12 : 8;
    const int shift = 32 - fixed - bits;
    const uint32_t dmask = (1u << bits) - 1u;
    for (int i = tid; i < NBIN; i += TT) hist[i] = 0u;
    __syncthreads();
    for (int64_t base = 0; base < len; base += TILE) {
      const int64_t p0 = base + (int64_t)tid * V;
      if (p0 < len) {
        const f32x4 v = *(const f32x4*)(row + p0);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          if (p0 + e < len) {
            const uint32_t u = order_key(v[e]);
            const bool match = fixed == 0 || (u >> (32 - fixed)) == prefix;
            if (match) atomicAdd(&hist[(u >> shift) & dmask], 1u);
          }
        }
      }
    }
    __syncthreads();
    // thread t owns digits dtop-4t .. dtop-4t-3 (descending); counts from the top digit down
    const int dtop = (int)dmask;
    uint32_t c[4], csum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = dtop - 4 * tid - q;
      c[q] = d >= 0 ? hist[d] : 0u;
      csum += c[q];
    }
    uint32_t total;
    const uint32_t incl = block_scan_incl(csum, wtot, &total);
    uint32_t run = incl - csum;  // keys with a larger digit than this thread's first
    if (run < need && need <= incl) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (run < need && need <= run + c[q]) {
          s_digit = (uint32_t)(dtop - 4 * tid - q);
          s_above = run;
        }
        run += c[q];
      }
    }
    __syncthreads();
    prefix = (prefix << bits) | s_digit;
    need -= s_above;
    fixed += bits;
    __syncthreads();
  }
  const uint32_t thr = prefix;  // the k-th largest key; `need` of the keys equal to it are taken

  // ---- positions in order: ties ranked by position, selected positions compacted
  uint32_t eq_run = 0, sel_run = 0;
  for (int64_t base = 0; base < len; base += TILE) {
    const int64_t p0 = base + (int64_t)tid * V;
    uint32_t u[V];
    bool ok[V];
    if (p0 < len) {
      const f32x4 v = *(const f32x4*)(row + p0);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        ok[e] = p0 + e < len;
        u[e] = order_key(v[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        ok[e] = false;
        u[e] = 0u;
      }
    }
    uint32_t neq = 0;
#pragma unroll
    for (int e = 0; e < V; ++e) neq += (ok[e] && u[e] == thr) ? 1u : 0u;
    uint32_t teq;
    uint32_t tie = eq_run + block_scan_incl(neq, wtot, &teq) - neq;  // ties before this thread's
    bool take[V];
    uint32_t nsel = 0;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      take[e] = false;
      if (ok[e]) {
        if (u[e] > thr) take[e] = true;
        else if (u[e] == thr) take[e] = tie++ < need;
      }
      nsel += take[e] ? 1u : 0u;
    }
    uint32_t tsel;
    uint32_t o = sel_run + block_scan_incl(nsel, wtot, &tsel) - nsel;
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (take[e] && o < (uint32_t)k) out[o++] = (int32_t)(p0 + e);
    eq_run += teq;
    sel_run += tsel;
  }
}

}  // namespace

hipError_t launch_topk(const Geometry& g, int32_t n_req, const float* scores, int64_t stride, const int32_t* len,
                       int32_t* sel, int32_t* err, hipStream_t s) {
  TopkArgs a;
  a.scores = scores;
  a.stride = stride;
  a.len = len;
  a.sel = sel;
  a.err = err;
  a.cap = g.cap;
  a.k = g.k;
  hipLaunchKernelGGL(topk_kernel, dim3(n_req), dim3(TT), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs
