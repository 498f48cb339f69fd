// Resolver: per-layer resolution of a top-k selection against the fixed device buffer.
//
// What is computed (HiSparse paper abstract: hit detection, LRU replacement and
// host-to-device fetches of each layer's selections; "HiSparse" note, section 3:
// find the top-k misses, choose LRU eviction candidates, update the page table,
// pull the rows from host memory), with the replacement rule stated in hs.h.
//
// Design for gfx950.  One workgroup of 1024 or 512 threads (16 or 8 wave64s) per request; a
// request's tables are private, so workgroups never communicate.
//   P0  clear two LDS bitmaps (hit slots [B bits], missing tokens [capacity bits]) and
//       load this thread's contiguous chunk of the LRU order into registers.  In launches of
//       more than 96 requests whose capacity fits (up to ~40 k tokens beside the rest), the
//       owner array (slot -> token, the inverse of the page table on resident tokens) is read
//       in the same coalesced round trip and scattered into an LDS token -> slot map (16-bit
//       entries);
//   P1  look up every selected token: in the LDS map when it was built, else by a random
//       4-byte gather of its page-table entry (2048 lookups per request are ~0.5 M separate
//       cache requests per launch at 256 requests, which the map avoids); hits set their
//       slot bit, misses their token bit (LDS atomics; a bit already set flags a repeated
//       token).  Without the map, with early reads (P2) the same round trip reads the owners
//       of the first k slots in LRU order, which hold every possible victim (the m-th non-hit
//       slot lies at most k - m hits deep);
//   P2  one packed block scan gives (a) for each word of the token bitmap the number of
//       misses below it, so a miss's ascending-token rank is prefix[word] +
//       popcount(lower bits of the word), and (b) each non-hit slot's rank in LRU order; the
//       miss list (token of rank q) goes to LDS, and with few requests the fusing workgroup
//       starts reading the first rows of its misses from host memory here, so the link is
//       busy while the tables are finished (barriers from here on wait for LDS only);
//   P3  LRU: the first m non-hit slots in LRU order are the victims; the remaining non-hit
//       slots keep their order and move to position rank - m of the new order (FIFO: the
//       order is by fill step, so hits keep their places too; RANDOM: the q-th miss takes
//       the non-hit slot of rank perm(q), a keyed permutation, and no order is kept);
//   P4  the slots stamped with this step -- under LRU hits and victims, under FIFO victims,
//       and any slot appended since the last resolve (hs_append stamps it with this step) --
//       form the back of the new order in ascending slot index (a scan over their bitmap;
//       each thread then places the back-group slots of its own chunk of slot indices);
//       the stamps are written in one coalesced pass over that bitmap; the i-th miss takes
//       victim i: evict its owner from the page table, install the token and write the
//       output slot;
//   P5  the missing rows are copied from pinned host memory (zero-copy 16-byte loads over
//       PCIe, row-major over the miss list so a wave reads ~1 KiB runs) into the victim
//       slots.  hs_resolve does this inside the resolving workgroup (each request's copy
//       starts as soon as its own tables are done).  hs_resolve_tables + hs_fetch_misses
//       instead write the miss list and copy with a second kernel of 128 small workgroups,
//       so that the copy can run beside other work (an attention kernel on the compute units
//       it leaves free) instead of inside a resolving workgroup that holds its LDS for the
//       whole PCIe-bound copy.
// The new order equals the slots sorted by (stamp, slot): untouched slots keep their
// relative order, and every touched slot now has the largest stamp, so among them the
// slot index decides.  No sort is needed and a step costs O(k + B + capacity/32).

#include "hs_internal.h"
#include "hs_wave.h"

namespace hs {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int NT_MAX = 2 * kResolveThreads;  // the wide workgroup (1024 threads)
constexpr int NW_MAX = NT_MAX / 64;          // scan scratch words, sized for the wide workgroup
constexpr int32_t kPad = -2;  // entry to skip: padding, out-of-range or repeated token

struct ResolveArgs {
  const int32_t* sel;
  int32_t* slots;
  int32_t* miss;
  int32_t* pt;
  int32_t* rm;
  int32_t* st;
  int32_t* ord;
  int32_t* step;
  uint32_t* fresh;  // [n][HB] slots appended since the last resolve
  const uint8_t* host;
  const uint8_t* tail;  // device-resident row tails [n][cap][16 * (chunks - body_chunks)], or null
  uint8_t* buf;
  int32_t* err;
  int32_t* ml_tok;   // [n][k] missing tokens, ascending (mode LIST)
  int32_t* ml_slot;  // [n][k] their slots
  int32_t* ml_cnt;   // [n]
  int64_t cap;
  int64_t host_stride;
  int64_t slot_stride;
  int64_t req_stride;  // bytes per request in buf
  uint64_t seed;       // HS_EVICT_RANDOM key
  int32_t k;
  int32_t B;
  int32_t chunks;  // 16-byte chunks per row
  int32_t body_chunks;  // chunks of a row read from the host pool (the rest: tail plane)
  int32_t policy;  // hs_eviction
  int32_t layer, nlayers;
  int32_t early_reads;  // FUSED: start the host reads in P2 (see launch_resolve)
  int32_t use_map;      // build the LDS token -> slot map (capacity fits in LDS)
};

// Output number c of SplitMix64 started from state s (Steele, Lea and Flood, OOPSLA 2014).
__device__ __forceinline__ uint64_t splitmix64_at(uint64_t s, uint64_t c) {
  uint64_t z = s + (c + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// HS_EVICT_RANDOM: image of x under the keyed permutation of [0, n) -- four Feistel rounds on
// halves of h bits (4^h >= n), round i mixing the right half into the left with SplitMix64
// output (i << 32 | right) under `key`, repeated while the value lies outside [0, n) (cycle
// walking; it returns because the network permutes [0, 4^h)).
__device__ uint32_t random_rank(uint64_t key, uint32_t n, uint32_t x) {
  int h = 1;
  while ((1ull << (2 * h)) < (uint64_t)n) ++h;
  const uint32_t mask = (1u << h) - 1u;
  do {
    uint32_t lo = x & mask, hi = x >> h;
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
      const uint32_t f = (uint32_t)splitmix64_at(key, ((uint64_t)i << 32) | lo) & mask;
      const uint32_t t = hi ^ f;
      hi = lo;
      lo = t;
    }
    x = (hi << h) | lo;
  } while (x >= n);
  return x;
}

// Chunk c (16 bytes) of row s of one request's history: the host part of a row from pinned
// host memory (zero-copy, non-temporal), the chunks past it from the device-resident tail
// plane.  Without a tail plane body_chunks covers the whole row.
__device__ __forceinline__ v4i row_chunk(const uint8_t* host, int64_t host_stride, const uint8_t* tail,
                                         int body_chunks, int chunks, int64_t s, int c) {
  if (c < body_chunks) return __builtin_nontemporal_load((const v4i*)(host + s * host_stride) + c);
  return ((const v4i*)(tail + s * (int64_t)(chunks - body_chunks) * 16))[c - body_chunks];
}

// A workgroup barrier that waits for this wave's LDS operations only.  From P2 on no thread
// reads global memory another thread of the workgroup writes, so the global fence that
// __syncthreads() adds is not needed -- and it would stall on the host reads in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Exclusive block-wide prefix sum of v over NT threads; *total gets the block sum.  Every
// thread must call.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const uint32_t x = wave_scan_incl(v);
  if (lane == 63) wsum[wid] = x;
  lds_barrier();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t s = wsum[w];
    before += (w < wid) ? s : 0u;
    tot += s;
  }
  lds_barrier();
  *total = tot;
  return before + x - v;
}

// What the resolving workgroup does with the missing rows.
enum Mode : int {
  TABLES = 0,  // tables only (the no-IO measurement mode)
  FUSED = 1,   // the workgroup copies its rows itself
  LIST = 2,    // the workgroup writes its miss list; fetch_kernel copies the rows
};

// NT: threads (512 or 1024); KPT: selection entries per thread (KPT * NT >= k); OPT: LRU-order
// entries per thread (OPT * NT >= B).
template <int NT, int KPT, int OPT, int MODE>
__global__ __launch_bounds__(NT) void resolve_kernel(ResolveArgs a) {
  extern __shared__ uint32_t lds[];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int B = a.B;
  const int k = a.k;
  const int64_t cap = a.cap;
  const int W = (int)((cap + 31) >> 5);
  const int HB = (B + 31) >> 5;
  uint32_t* hitmap = lds;                       // [HB]  hit slots, then hit + victim slots
  uint32_t* missmap = hitmap + HB;              // [W]   missing tokens
  uint32_t* victims = missmap + W;              // [k]   victim slot of the i-th miss
  uint32_t* misstok = victims + k;              // [k]   token of the i-th miss (-1: none)
  uint32_t* vowner = misstok + k;               // [k]   token held by victim i before the step (-1: none)
  uint32_t* wsum = vowner + k;                  // [NW_MAX] scan scratch
  uint32_t* freshmap = wsum + NW_MAX;           // [HB]  slots appended since the last resolve
  uint32_t* backpre = freshmap + HB;            // [HB]  back-group slots below each bitmap word
  uint16_t* prefix = (uint16_t*)(backpre + HB);  // [W] misses below each bitmap word
  const bool map = a.use_map != 0;
  const int MW = (int)((cap + 1) >> 1);                        // map words (two entries each)
  int16_t* tmap = (int16_t*)((uint32_t*)prefix + ((W + 1) >> 1));  // [cap] slot of a token, -1 absent
  int32_t* rml = (int32_t*)((uint32_t*)tmap + (map ? MW : 0));     // [B] owners before the step

  int32_t* pt = a.pt + (int64_t)r * cap;
  int32_t* rm = a.rm + (int64_t)r * B;
  int32_t* st = a.st + (int64_t)r * B;
  int32_t* ord = a.ord + (int64_t)r * B;
  const int32_t* sel = a.sel + (int64_t)r * k;
  int32_t* slots = a.slots + (int64_t)r * k;
  const int32_t t = a.step[r];

  // ---- P0: every global load first (one round trip), the LDS clears while they are in flight
  static_assert(kMaxBuffer / 32 <= NT, "one word of the slot bitmaps per thread");
  uint32_t* fresh = a.fresh + (int64_t)r * HB;
  const uint32_t fw = (tid < HB) ? fresh[tid] : 0u;
  int32_t ordv[OPT];
  int32_t own[OPT];  // owners of this thread's chunk of slots (the map)
  const int o0 = tid * OPT;
#pragma unroll
  for (int x = 0; x < OPT; ++x) ordv[x] = (o0 + x < B) ? ord[o0 + x] : -1;
#pragma unroll
  for (int x = 0; x < OPT; ++x) own[x] = (map && o0 + x < B) ? rm[o0 + x] : -1;
  int32_t selv[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + j * NT;
    selv[j] = (i < k) ? sel[i] : -1;
  }
  if (tid < HB) hitmap[tid] = 0u;
  for (int w = tid; w < W; w += NT) missmap[w] = 0u;
  if (map)
    for (int e = tid; e < MW; e += NT) ((uint32_t*)tmap)[e] = 0xFFFFFFFFu;
  if (tid < HB) {
    freshmap[tid] = fw;
    if (fw) fresh[tid] = 0u;  // consumed by this resolve
  }
  __syncthreads();
  if (map) {
#pragma unroll
    for (int x = 0; x < OPT; ++x) {
      if (o0 + x >= B) continue;
      rml[o0 + x] = own[x];
      if (own[x] >= 0 && (int64_t)own[x] < cap) tmap[own[x]] = (int16_t)(o0 + x);
    }
    __syncthreads();
  }

  // ---- P1
  uint32_t err = 0;
  int32_t ptv[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int32_t s = selv[j];
    int32_t p = kPad;
    if (s != -1) {
      if (s < 0 || (int64_t)s >= cap) err |= HS_DEVERR_TOKEN_RANGE;
      else p = map ? (int32_t)tmap[s] : pt[s];
    }
    ptv[j] = p;
  }
  const int policy = a.policy;
  // A fusing workgroup under LRU or FIFO reads its first rows early (P2); it then takes the
  // victims' owners from registers, since a global load after those reads would wait for them.
  const bool early = MODE == FUSED && policy != HS_EVICT_RANDOM && a.early_reads;
  int32_t rmv[OPT];  // owners of this thread's LRU-order slots among the first k
#pragma unroll
  for (int x = 0; x < OPT; ++x) {
    const int32_t j = ordv[x];
    rmv[x] = (early && !map && o0 + x < k && j >= 0 && j < B) ? rm[j] : -1;
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int32_t p = ptv[j];
    if (p >= 0) {
      if (p >= B) {
        ptv[j] = kPad;
      } else {
        const uint32_t bit = 1u << (p & 31);
        if (atomicOr(&hitmap[p >> 5], bit) & bit) { err |= HS_DEVERR_DUPLICATE; ptv[j] = kPad; }
      }
    } else if (p == -1) {
      const int32_t s = selv[j];
      const uint32_t bit = 1u << (s & 31);
      if (atomicOr(&missmap[s >> 5], bit) & bit) { err |= HS_DEVERR_DUPLICATE; ptv[j] = kPad; }
    } else {
      ptv[j] = kPad;
    }
  }
  if (err) atomicOr(a.err, (int32_t)err);
  __syncthreads();

  // ---- P2
  const int WPT = (W + NT - 1) / NT;
  const int w0 = tid * WPT;
  const int w1 = min(W, w0 + WPT);
  uint32_t mcnt = 0;
  for (int w = w0; w < w1; ++w) mcnt += __popc(missmap[w]);
  uint32_t nhcnt = 0, nhmask = 0;
#pragma unroll
  for (int x = 0; x < OPT; ++x) {
    const int32_t j = ordv[x];
    if (j >= 0 && j < B && !((hitmap[j >> 5] >> (j & 31)) & 1u)) {
      ++nhcnt;
      nhmask |= 1u << x;
    }
  }
  uint32_t tot;
  const uint32_t pre = block_scan<NT>((mcnt << 16) | nhcnt, wsum, &tot);
  const int m = (int)(tot >> 16);
  const int nonhit = (int)(tot & 0xFFFFu);
  {
    uint32_t run = pre >> 16;
    for (int w = w0; w < w1; ++w) {
      prefix[w] = (uint16_t)run;
      run += __popc(missmap[w]);
    }
  }
  // rank q of a missing token = misses below it (ascending token order)
  auto miss_rank = [&](int32_t s) -> int {
    const int w = s >> 5;
    return (int)prefix[w] + __popc(missmap[w] & ((1u << (s & 31)) - 1u));
  };
  constexpr int U = 2048 / NT;  // 16-byte host reads in flight per thread: 32 KiB per workgroup
  const int C = a.chunks;
  const int total = m * C;
  const uint8_t* host = a.host + (int64_t)r * cap * a.host_stride;
  const uint8_t* tail = a.tail + (int64_t)r * cap * (int64_t)(C - a.body_chunks) * 16;
  const int BC = a.body_chunks;
  int qv[KPT];
  v4i v0[U];
  if (early) {
    // the miss list, then the first rows of the misses, read while the tables are finished
    // (no global load follows these reads before P5)
    lds_barrier();
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      qv[j] = -1;
      if (ptv[j] == -1) {
        qv[j] = miss_rank(selv[j]);
        if (qv[j] < k) misstok[qv[j]] = (uint32_t)selv[j];
      }
    }
    lds_barrier();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = tid + u * NT;
      if (idx < total) {
        const int q = idx / C;
        const int c = idx - q * C;
        v0[u] = row_chunk(host, a.host_stride, tail, BC, C, (int64_t)misstok[q], c);
      }
    }
  }

  // ---- P3
  if (policy == HS_EVICT_RANDOM) {
    // Candidates are the non-hit slots in slot order; the q-th miss takes candidate
    // random_rank(q), found through per-word candidate counts (one bitmap word per thread)
    // and a select within the word.  The LRU order array is not maintained.
    uint32_t* cpre = freshmap;  // no appends under RANDOM: the fresh bitmap is free
    uint32_t cand = 0;
    if (tid < HB) {
      cand = ~hitmap[tid];
      if (tid == HB - 1 && (B & 31)) cand &= (1u << (B & 31)) - 1u;
    }
    uint32_t ncand;
    const uint32_t below = block_scan<NT>((uint32_t)__popc(cand), wsum, &ncand);
    if (tid < HB) cpre[tid] = below;
    lds_barrier();
    const uint64_t key =
        splitmix64_at(a.seed, ((uint64_t)((int64_t)r * a.nlayers + a.layer) << 32) | (uint32_t)t);
    for (int q = tid; q < m && q < (int)ncand; q += NT) {
      const uint32_t x = random_rank(key, ncand, (uint32_t)q);
      int lo = 0, hi = HB - 1;  // the last word whose prefix is <= x holds candidate x
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cpre[mid] <= x) lo = mid;
        else hi = mid - 1;
      }
      uint32_t bits = ~hitmap[lo];
      if (lo == HB - 1 && (B & 31)) bits &= (1u << (B & 31)) - 1u;
      for (uint32_t z = cpre[lo]; z < x; ++z) bits &= bits - 1u;
      victims[q] = (uint32_t)(lo * 32 + __ffs(bits) - 1);
    }
  } else {
    // LRU and FIFO: the first m non-hit slots in order are the victims.  Slots stamped with
    // this step after the resolve -- victims, appended slots and, under LRU, hits -- form the
    // back of the new order (the bitmap `back`); every other slot keeps its relative order
    // and moves up past the back-group slots before it.
    uint32_t* back = (policy == HS_EVICT_FIFO) ? freshmap : hitmap;
    int rank = (int)(pre & 0xFFFFu);  // non-hit slots before this thread's entries
#pragma unroll
    for (int x = 0; x < OPT; ++x) {
      const int32_t j = ordv[x];
      if (j < 0 || j >= B) continue;
      const bool fresh_j = (freshmap[j >> 5] >> (j & 31)) & 1u;
      if (nhmask & (1u << x)) {
        if (rank < m) {
          victims[rank] = (uint32_t)j;
          if (early && !map) vowner[rank] = (uint32_t)rmv[x];
          atomicOr(&back[j >> 5], 1u << (j & 31));
        } else if (fresh_j) {
          // appended since the last resolve: its stamp is already this step's (appended
          // slots come last in the order, so no slot before them shifts)
          atomicOr(&back[j >> 5], 1u << (j & 31));
        } else {
          // LRU: hit slots all go to the back, so the untouched slots are exactly the
          // non-hit ones; FIFO: hits stay, and only the m victims before this slot leave
          ord[(policy == HS_EVICT_FIFO ? o0 + x : rank) - m] = j;
        }
        ++rank;
      } else if (policy == HS_EVICT_FIFO && !fresh_j) {
        ord[o0 + x - min(m, rank)] = j;  // a hit keeps its fill stamp and its place
      }
    }
  }
  lds_barrier();

  // ---- P4
  if (policy != HS_EVICT_RANDOM) {
    // The back group, in ascending slot order, fills the end of the new order: every thread
    // places the back-group slots of its own chunk of slot indices (a back-group slot's place
    // = the back-group slots below its word + those below it in the word), so the stores of
    // a wave land on neighbouring entries and all threads share the work.
    const uint32_t* bmap = (policy == HS_EVICT_FIFO) ? freshmap : hitmap;
    const uint32_t word = (tid < HB) ? bmap[tid] : 0u;
    uint32_t touched;
    const uint32_t below = block_scan<NT>((uint32_t)__popc(word), wsum, &touched);
    if (tid < HB) backpre[tid] = below;
    lds_barrier();
    const int base = B - (int)touched;
#pragma unroll
    for (int x = 0; x < OPT; ++x) {
      const int j = o0 + x;
      if (j < B) {
        const uint32_t wd = bmap[j >> 5];
        const uint32_t bit = (uint32_t)(j & 31);
        if ((wd >> bit) & 1u) ord[base + (int)backpre[j >> 5] + __popc(wd & ((1u << bit) - 1u))] = j;
      }
    }
  }
  // stamps, coalesced: LRU -- hits, victims and appended slots (all in the hit bitmap by
  // now); FIFO -- victims and appended slots (the fresh bitmap); RANDOM -- hits (its victims
  // are stamped below)
  {
    const uint32_t* stampmap = (policy == HS_EVICT_FIFO) ? freshmap : hitmap;
    for (int j = tid; j < B; j += NT)
      if ((stampmap[j >> 5] >> (j & 31)) & 1u) st[j] = t;
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + j * NT;
    if (i < k) {
      const int32_t p = ptv[j];
      int32_t out = -1;
      if (p >= 0) {
        out = p;
      } else if (p == -1) {
        const int32_t s = selv[j];
        const int q = early ? qv[j] : miss_rank(s);
        const int32_t v = (q < m && q < nonhit) ? (int32_t)victims[q] : -1;
        int32_t tok = -1;
        if (v >= 0 && v < B) {
          const int32_t old = map ? rml[v] : early ? (int32_t)vowner[q] : rm[v];
          if (old >= 0 && (int64_t)old < cap) pt[old] = -1;
          pt[s] = v;
          rm[v] = s;
          if (policy == HS_EVICT_RANDOM) st[v] = t;
          out = v;
          tok = s;
        }
        if (q < k) misstok[q] = (uint32_t)tok;
        if (MODE == LIST && q < k) {
          a.ml_tok[(int64_t)r * k + q] = tok;
          a.ml_slot[(int64_t)r * k + q] = v;
        }
      }
      slots[i] = out;
    }
  }
  if (tid == 0) {
    a.step[r] = t + 1;
    if (a.miss) a.miss[r] = m;
    if (MODE == LIST) a.ml_cnt[r] = m;
  }
  if (MODE != FUSED) return;
  lds_barrier();

  // ---- P5
  if (m == 0) return;
  uint8_t* buf = a.buf + (int64_t)r * a.req_stride;
  int base0 = tid;
  if (early) {  // the batch read in P2
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = tid + u * NT;
      if (idx < total) {
        const int q = idx / C;
        const int c = idx - q * C;
        if ((int32_t)misstok[q] >= 0) ((v4i*)(buf + (int64_t)victims[q] * a.slot_stride))[c] = v0[u];
      }
    }
    base0 += NT * U;
  }
  for (int base = base0; base < total; base += NT * U) {
    v4i v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * NT;
      if (idx < total) {
        const int q = idx / C;
        const int c = idx - q * C;
        const int32_t s = (int32_t)misstok[q];
        if (s >= 0) v[u] = row_chunk(host, a.host_stride, tail, BC, C, (int64_t)s, c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * NT;
      if (idx < total) {
        const int q = idx / C;
        const int c = idx - q * C;
        if ((int32_t)misstok[q] >= 0) ((v4i*)(buf + (int64_t)victims[q] * a.slot_stride))[c] = v[u];
      }
    }
  }
}

// Copies the rows of the miss lists written by resolve_kernel<..., LIST>: grid (blocks per
// request, request groups); a workgroup copies requests y, y + gridDim.y, ... in turn, its
// threads covering consecutive 16-byte chunks of the request's rows (zero-copy loads from
// pinned host memory, four in flight per thread; at most 64 VGPRs).  128 workgroups in all
// keep the link busy.  Each reserves kFetchLds bytes of LDS it never touches, so that no
// attention workgroup (a ~126 KiB ring) fits on the same compute unit: an attention workgroup
// that shares a unit with the copy's long-latency host reads proceeds at the link's pace,
// while on the other 128 units it runs at its own.  Measured, 128 requests x 8 layers of
// 656-byte rows, one graph-replayed step: 2.188 ms with no reservation, 2.155 ms with 96 KiB
// (one copy workgroup per unit; 64 KiB, two per unit: 2.186), and 2.123-2.130 ms once the
// attention of the last 2-4 layers is also split by residency (which without the reservation
// is slower than not splitting).  64 workgroups of 512 threads: 2.165-2.19 ms; 64 of 256:
// 2.21-2.29.  On 256 requests with the attention of the resident tokens alongside the whole
// step is unchanged (518 against 520 us).
constexpr int FT = 256;
constexpr int kFetchGroups = 128;         // workgroups of a launch
constexpr int kFetchLds = 96 * 1024;      // LDS reserved per workgroup (unused)

__global__ __launch_bounds__(FT, 8) void fetch_kernel(const int32_t* __restrict__ ml_tok, const int32_t* __restrict__ ml_slot,
                                                      const int32_t* __restrict__ ml_cnt, const uint8_t* __restrict__ host,
                                                      const uint8_t* __restrict__ tail, uint8_t* __restrict__ buf,
                                                      int64_t cap, int64_t host_stride, int64_t slot_stride,
                                                      int64_t req_stride, int32_t k, int32_t B, int32_t chunks,
                                                      int32_t body_chunks, int32_t n_req) {
  constexpr int U = 4;
  const int step = gridDim.x * FT;
  for (int r = blockIdx.y; r < n_req; r += gridDim.y) {
    const int m = min(ml_cnt[r], k);
    const int total = m * chunks;
    const int32_t* tok = ml_tok + (int64_t)r * k;
    const int32_t* slot = ml_slot + (int64_t)r * k;
    const uint8_t* hrow = host + (int64_t)r * cap * host_stride;
    const uint8_t* trow = tail + (int64_t)r * cap * (int64_t)(chunks - body_chunks) * 16;
    uint8_t* drow = buf + (int64_t)r * req_stride;
    for (int base = blockIdx.x * FT + threadIdx.x; base < total; base += step * U) {
      v4i v[U];
      int32_t dst[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = base + u * step;
        dst[u] = -1;
        if (idx < total) {
          const int q = idx / chunks;
          const int c = idx - q * chunks;
          const int32_t s = tok[q], j = slot[q];
          if (s >= 0 && (int64_t)s < cap && j >= 0 && j < B) {
            v[u] = row_chunk(hrow, host_stride, trow, body_chunks, chunks, (int64_t)s, c);
            dst[u] = j * chunks + c;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (dst[u] >= 0) {
          const int j = dst[u] / chunks, c = dst[u] - j * chunks;
          ((v4i*)(drow + (int64_t)j * slot_stride))[c] = v[u];
        }
      }
    }
  }
}

__global__ void reset_kernel(int32_t* pt, int32_t* rm, int32_t* st, int32_t* ord, int32_t* step, uint32_t* fresh,
                             int32_t L, int32_t n, int32_t first, int32_t count, int64_t cap, int32_t B) {
  const int64_t pairs = (int64_t)L * count;
  for (int64_t lr = blockIdx.y; lr < pairs; lr += gridDim.y) {
    const int32_t l = (int32_t)(lr / count);
    const int32_t r = first + (int32_t)(lr % count);
    const int64_t id = (int64_t)l * n + r;
    int32_t* p = pt + id * cap;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < cap; x += (int64_t)gridDim.x * blockDim.x)
      p[x] = -1;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < B; x += (int64_t)gridDim.x * blockDim.x) {
      rm[id * B + x] = -1;
      st[id * B + x] = -1;
      ord[id * B + x] = (int32_t)x;
    }
    const int HB = (B + 31) >> 5;
    for (int x = blockIdx.x * blockDim.x + threadIdx.x; x < HB; x += gridDim.x * blockDim.x) fresh[id * HB + x] = 0u;
    if (blockIdx.x == 0 && threadIdx.x == 0) step[id] = 0;
  }
}

template <int NT, int KPT, int OPT>
void allow_large_lds() {
  // Lets a workgroup take up to the whole 160 KiB of LDS; errors are left to the launch.
  (void)hipFuncSetAttribute((const void*)resolve_kernel<NT, KPT, OPT, TABLES>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
  (void)hipFuncSetAttribute((const void*)resolve_kernel<NT, KPT, OPT, FUSED>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
  (void)hipFuncSetAttribute((const void*)resolve_kernel<NT, KPT, OPT, LIST>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
  (void)hipGetLastError();
}

template <int NT, int KPT, int OPT>
hipError_t launch_one(const ResolveArgs& a, int mode, int n_req, size_t lds, hipStream_t s) {
  if (mode == FUSED)
    hipLaunchKernelGGL((resolve_kernel<NT, KPT, OPT, FUSED>), dim3(n_req), dim3(NT), lds, s, a);
  else if (mode == LIST)
    hipLaunchKernelGGL((resolve_kernel<NT, KPT, OPT, LIST>), dim3(n_req), dim3(NT), lds, s, a);
  else
    hipLaunchKernelGGL((resolve_kernel<NT, KPT, OPT, TABLES>), dim3(n_req), dim3(NT), lds, s, a);
  return hipGetLastError();
}

// Register tiling for NT threads: k up to 2048 or 8192 selections, B up to 4096 or 16384 slots.
template <int NT>
hipError_t launch_width(const ResolveArgs& a, int mode, int n_req, size_t lds, hipStream_t s) {
  constexpr int KS = 2048 / NT, KL = 8192 / NT, OS = 4096 / NT, OL = 16384 / NT;
  static_assert(KL * NT >= kMaxTopK && OL * NT >= kMaxBuffer && NT / 32 >= 1, "tiling covers the limits");
  const int kpt = (a.k + NT - 1) / NT;
  const int opt = (a.B + NT - 1) / NT;
  if (kpt <= KS)
    return opt <= OS ? launch_one<NT, KS, OS>(a, mode, n_req, lds, s) : launch_one<NT, KS, OL>(a, mode, n_req, lds, s);
  return opt <= OS ? launch_one<NT, KL, OS>(a, mode, n_req, lds, s) : launch_one<NT, KL, OL>(a, mode, n_req, lds, s);
}

}  // namespace

void prepare_resolve() {
  (void)hipFuncSetAttribute((const void*)fetch_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kFetchLds);
  (void)hipGetLastError();
  allow_large_lds<512, 4, 8>();
  allow_large_lds<512, 4, 32>();
  allow_large_lds<512, 16, 8>();
  allow_large_lds<512, 16, 32>();
  allow_large_lds<1024, 2, 4>();
  allow_large_lds<1024, 2, 16>();
  allow_large_lds<1024, 8, 4>();
  allow_large_lds<1024, 8, 16>();
}

size_t resolve_lds_bytes(int64_t cap, int32_t k, int32_t B) {
  const size_t W = (size_t)((cap + 31) >> 5);
  const size_t HB = (size_t)((B + 31) >> 5);
  size_t words = 3 * HB + W + 3 * (size_t)k + NW_MAX + (W + 1) / 2;
  return (words * 4 + 15) & ~(size_t)15;
}

// LDS of the token -> slot map and the owners' copy, when they fit beside the rest.
static size_t resolve_map_bytes(int64_t cap, int32_t k, int32_t B) {
  const size_t extra = (size_t)((cap + 1) >> 1) * 4 + (size_t)B * 4;
  return resolve_lds_bytes(cap, k, B) + extra <= kLdsLimit && B <= 32767 ? extra : 0;
}

hipError_t launch_resolve(const Geometry& g, const LayerTables& t, int32_t layer, const uint8_t* host_layer,
                          int32_t n_req, const int32_t* sel, int32_t* slots, int32_t* miss, int32_t* err,
                          bool list_only, hipStream_t s) {
  ResolveArgs a;
  a.sel = sel;
  a.slots = slots;
  a.miss = miss;
  a.pt = t.pt;
  a.rm = t.rm;
  a.st = t.st;
  a.ord = t.ord;
  a.step = t.step;
  a.fresh = t.fresh;
  a.host = host_layer;
  a.tail = t.tail;
  a.buf = t.buf;
  a.err = err;
  a.cap = g.cap;
  a.host_stride = g.host_stride;
  a.slot_stride = g.slot_stride;
  a.req_stride = g.req_stride;
  a.seed = g.seed;
  a.policy = g.policy;
  a.layer = layer;
  a.nlayers = g.L;
  a.k = g.k;
  a.B = g.B;
  a.chunks = (int32_t)(g.unit_bytes / 16);
  a.body_chunks = (int32_t)(g.host_stride / 16);
  a.ml_tok = t.ml_tok;
  a.ml_slot = t.ml_slot;
  a.ml_cnt = t.ml_cnt;
  const int mode = (g.flags & HS_FLAG_NO_IO) ? TABLES : list_only ? LIST : FUSED;
  // Early host reads pay off while the link would idle during the table phase: measured on
  // the 2048-of-4096 workloads, they save 4-6 us per launch at 32-128 requests of 656-byte
  // rows and ~4 us at 64 requests of 1152-byte rows, but cost 2-4 us from 128 requests of
  // 1152-byte rows and 192 of 656-byte rows on, where other workgroups keep the link busy.
  a.early_reads = n_req <= 96;
  // The LDS map pays once the page-table gathers of many requests crowd the caches: measured
  // no-IO, 256 requests 15.5 -> 14.6 us, but 64 requests 10.9 -> 11.8 us (the map's fill and
  // scatter cost more than a few gathers), so it is built for launches past the early-read
  // threshold only.
  const size_t map_bytes = n_req > 96 ? resolve_map_bytes(g.cap, g.k, g.B) : 0;
  a.use_map = map_bytes > 0;
  const size_t lds = resolve_lds_bytes(g.cap, g.k, g.B) + map_bytes;
  // The wide (1024-thread) workgroup finishes the tables sooner (measured 10.5 vs 12.9 us for
  // 64 requests and 15.4 vs 18.1 us for 256, no IO); with row copies from more than 128
  // requests the 512-thread one copies faster (473 vs 491 us at 256 requests of 656-byte rows).
  if (mode != FUSED || n_req <= 128) return launch_width<1024>(a, mode, n_req, lds, s);
  return launch_width<512>(a, mode, n_req, lds, s);
}

hipError_t launch_fetch(const Geometry& g, const LayerTables& t, const uint8_t* host_layer, int32_t n_req,
                        hipStream_t s) {
  if (g.flags & HS_FLAG_NO_IO) return hipSuccess;
  // kFetchGroups workgroups in all: one per request group, and with fewer requests several
  // per request (at most 16)
  const int groups = n_req < kFetchGroups ? n_req : kFetchGroups;
  int per_req = (kFetchGroups + n_req - 1) / n_req;
  if (per_req > 16) per_req = 16;
  hipLaunchKernelGGL(fetch_kernel, dim3(per_req, groups), dim3(FT), kFetchLds, s, t.ml_tok, t.ml_slot, t.ml_cnt,
                     host_layer, t.tail, t.buf, g.cap, g.host_stride, g.slot_stride, g.req_stride, g.k, g.B,
                     (int32_t)(g.unit_bytes / 16), (int32_t)(g.host_stride / 16), n_req);
  return hipGetLastError();
}

hipError_t launch_reset(const Geometry& g, int32_t* pt, int32_t* rm, int32_t* st, int32_t* ord, int32_t* step,
                        uint32_t* fresh, int32_t first, int32_t count, hipStream_t s) {
  const int64_t pairs = (int64_t)g.L * count;
  const unsigned gy = (unsigned)(pairs < 65535 ? pairs : 65535);
  hipLaunchKernelGGL(reset_kernel, dim3(16, gy), dim3(256), 0, s, pt, rm, st, ord, step, fresh, g.L, g.n, first, count,
                     g.cap, g.B);
  return hipGetLastError();
}

}  // namespace hs
