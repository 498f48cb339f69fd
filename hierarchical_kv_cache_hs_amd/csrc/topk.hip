// Top-k selection from indexer scores: the step that feeds the resolver.
//
// What is computed (the HiSparse note, section 2: the serving backend's indexer decides which
// KV entries a step selects; paper abstract: the method is indexer-agnostic): for every
// request r, among positions 0 .. len[r]-1 of its score row, the k positions of largest
// score -- a tie going to the smaller position -- written in ascending position order; when
// len[r] < k every position is selected and the row is padded with -1.
//
// Design for gfx950.  One 1024-thread workgroup per request (sixteen waves keep more loads and
// LDS atomics in flight than eight: 13 % faster at 128 x 65536); rows of up to 2^18 positions.
// Scores map to 32-bit keys whose unsigned order is the float order (-0 folded onto +0, so
// equal floats give equal keys).  A most-significant-digit radix select, reading the row
// twice:
//   pass A   histogram of the top 12 key bits (two copies interleaved by lane parity, summed)
//            -> the digit d holding the k-th largest key;
//   pass B   positions whose top digit exceeds d are set in an LDS selection bitmap; those
//            whose top digit equals d (for scores like these, a percent or so of the row)
//            are appended to an LDS candidate list (key, position), one wave scan and one
//            LDS atomic per wave and batch;
//   list     the next 12 and the last 8 key bits are resolved by histograms over the list,
//            giving the k-th largest key exactly and how many keys equal to it are taken;
//            candidates above it join the selection bitmap, those equal to it a tie bitmap;
//   output   one block scan of (selected, tied) bit counts over the bitmap words decides which
//            ties are taken (the first ones in position order) and how many selected
//            positions lie below each word; output i is then the (i - below)-th set bit of the
//            last word whose count below is <= i, found by a binary search, so consecutive
//            threads write consecutive outputs, with no sort.
// If the candidate list would overflow (many equal scores), the last two digits are resolved
// with re-reads of the row instead.
// With a hint (hs_topk_hinted: per request a guess g of the top digit, as returned for the same
// request and layer at the previous decode step), one pass sets the positions whose top digit
// exceeds g + 1 in the selection bitmap, counts them, and lists the keys of digits g - 1 .. g + 1.
// If the count shows the k-th largest key among them (and the list did not overflow), pass A is
// skipped and two 11-bit levels over the listed keys' offsets from the bracket's lowest key
// (less than 3 * 2^20) find the k-th largest; otherwise the bitmap is cleared and the two passes
// run as above.  The digit found is written back.  Reads are batched: eight 16-byte loads per thread are in
// flight before any is used, and batches that lie wholly inside the row skip the per-key
// bounds checks (the passes over the row are bound by VALU work per key and the histogram's
// LDS atomics, not by the reads).

#include "hs_internal.h"
#include "hs_wave.h"

namespace hs {
namespace {

constexpr int TT = 1024;                  // threads per workgroup
constexpr int TW = TT / 64;               // waves
constexpr int V = 4;                      // positions per thread per tile (one 16-byte load)
constexpr int TILE = TT * V;
constexpr int U = 8;                      // tiles per batch
constexpr int NBIN = 4096;                // 12-bit digits
constexpr int BPT = NBIN / TT;            // digits per thread in the search
constexpr int MAXLEN = 1 << 18;           // positions per row
constexpr int MAXW = MAXLEN / 32;         // bitmap words
constexpr int CMAX = 8192;                // candidate list entries
static_assert(2 * NBIN <= CMAX, "pass A's two histogram copies fit in the candidate list");
static_assert(NBIN % TT == 0, "whole groups of digits per thread");

constexpr size_t topk_lds_bytes() {
  return (NBIN + 2 * MAXW + 2 * CMAX) * sizeof(uint32_t);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// key of a float given by its bits: negative floats are complemented, the others get the sign
// bit set, so unsigned order is float order; -0 (complemented to 0x7FFFFFFF) moves up one to
// +0's key 0x80000000
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  const uint32_t k = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
  return k + (b == 0x80000000u ? 1u : 0u);
}

// Inclusive scan of v over the workgroup; *total gets the sum.  Every thread must call.
// In-wave inclusive scan: 32-bit values on DPP; 64-bit values here are two independent 32-bit
// counts packed (hi, lo) whose sums stay below 2^32, so each half is scanned on its own.
__device__ __forceinline__ uint32_t wave_incl(uint32_t v) { return wave_scan_incl(v); }
__device__ __forceinline__ uint64_t wave_incl(uint64_t v) {
  return ((uint64_t)wave_scan_incl((uint32_t)(v >> 32)) << 32) | wave_scan_incl((uint32_t)v);
}

template <typename T>
__device__ T block_scan_incl(T v, T* wtot, T* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  v = wave_incl(v);
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const T x = wtot[i];
    base += (i < w) ? x : (T)0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return v + base;
}

// Calls batch(key, b0) for every batch of UU tiles of the row, the loads of a batch all issued
// first; this thread's key[j][e] is that of position b0 + j * TILE + 4 tid + e.  With KEYS the
// scores are mapped to their keys and positions past the row get key 0, below every score's
// key (-inf maps to 0x007FFFFF); without, key[j][e] holds the score's bits and positions past
// the row hold a quiet NaN, which no comparison passes.
template <int UU, bool KEYS = true, typename F>
__device__ __forceinline__ void for_each_batch(const uint32_t* row, int n, F batch) {
  const int tid = threadIdx.x;
  constexpr uint32_t PAD = KEYS ? 0u : 0x7FC00000u;
  for (int b0 = 0; b0 < n; b0 += TILE * UU) {
    u32x4 key[UU];
    if (b0 + TILE * UU <= n) {  // the whole batch lies in the row: no per-key checks
#pragma unroll
      for (int j = 0; j < UU; ++j) key[j] = *(const u32x4*)(row + b0 + j * TILE + 4 * tid);
      if (KEYS) {
#pragma unroll
        for (int j = 0; j < UU; ++j)
#pragma unroll
          for (int e = 0; e < V; ++e) key[j][e] = order_key(key[j][e]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < UU; ++j) {  // in bounds: p < n <= stride, p and stride multiples of 4
        const int p = b0 + j * TILE + 4 * tid;
        key[j] = p < n ? *(const u32x4*)(row + p) : (u32x4){PAD, PAD, PAD, PAD};
      }
#pragma unroll
      for (int j = 0; j < UU; ++j) {
        const int p = b0 + j * TILE + 4 * tid;
#pragma unroll
        for (int e = 0; e < V; ++e) key[j][e] = (p + e < n) ? (KEYS ? order_key(key[j][e]) : key[j][e]) : PAD;
      }
    }
    batch(key, b0);
  }
}

// The score whose key is kk (the inverse of order_key for keys of non-NaN floats).
__device__ __forceinline__ float key_float(uint32_t kk) {
  return __uint_as_float((kk & 0x80000000u) ? (kk ^ 0x80000000u) : ~kk);
}

// A bound b with "score >= b" exactly when "key >= d << 20", for every score (no NaN) and top
// digit d in 0 .. 4096: edges at or below -inf's key (digits 0 .. 7; below -inf lie only NaN
// patterns) hold every score, the edge 2^32 (d = 4096) none, and edges past +inf's key (their
// float is a NaN) none as well.
__device__ __forceinline__ float digit_edge(uint32_t d) {
  if (d >= (uint32_t)NBIN) return __uint_as_float(0x7FC00000u);
  const uint32_t kk = d << 20;
  return kk <= 0x007FFFFFu ? -INFINITY : key_float(kk);
}

// for_each_batch, one key at a time: f(key, position)
template <int UU, typename F>
__device__ __forceinline__ void for_each_key(const uint32_t* row, int n, F f) {
  const int tid = threadIdx.x;
  for_each_batch<UU>(row, n, [&](u32x4 (&key)[UU], int b0) {
#pragma unroll
    for (int j = 0; j < UU; ++j)
#pragma unroll
      for (int e = 0; e < V; ++e) f(key[j][e], b0 + j * TILE + 4 * tid + e);
  });
}

// The digit of histogram h holding the need-th largest key (counting from the top) and the
// number of keys above that digit.  Every thread must call.
__device__ __forceinline__ void find_digit(const uint32_t* h, int dtop, uint32_t need, uint32_t* wtot,
                                           uint32_t* s_digit, uint32_t* s_above) {
  const int tid = threadIdx.x;
  uint32_t cnt[BPT], csum = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int d = dtop - BPT * tid - q;  // this thread's digits, descending
    cnt[q] = d >= 0 ? h[d] : 0u;
    csum += cnt[q];
  }
  uint32_t total;
  const uint32_t incl = block_scan_incl<uint32_t>(csum, wtot, &total);
  uint32_t run = incl - csum;
  if (run < need && need <= incl) {
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (run < need && need <= run + cnt[q]) {
        *s_digit = (uint32_t)(dtop - BPT * tid - q);
        *s_above = run;
      }
      run += cnt[q];
    }
  }
  __syncthreads();
}

struct TopkArgs {
  const float* scores;
  int64_t stride;      // floats between request rows (multiple of 4)
  const int32_t* len;  // [n]
  int32_t* sel;        // [n][k]
  int32_t* err;
  int32_t* hint;       // [n] in/out: top digit of the k-th largest key (guess in, exact out), or null
  int64_t cap;
  int32_t k;
};

__global__ __launch_bounds__(TT) void topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t lds[];
  uint32_t* hist = lds;                  // [NBIN]
  uint32_t* selmap = hist + NBIN;        // [MAXW] positions taken for sure
  uint32_t* tiemap = selmap + MAXW;      // [MAXW] positions holding the k-th largest key
  uint32_t* ckey = tiemap + MAXW;        // [CMAX] candidates: keys
  uint32_t* cpos = ckey + CMAX;          //        and positions
  __shared__ uint32_t wtot[TW];
  __shared__ uint64_t wtot64[TW];
  __shared__ uint32_t s_digit, s_above, s_ncand, s_nabove;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int k = a.k;
  int32_t* out = a.sel + (int64_t)r * k;
  const int64_t len = a.len[r];
  if (len < 0 || len > a.cap || len > a.stride || len > MAXLEN) {
    if (tid == 0) {
      atomicOr(a.err, (int32_t)HS_DEVERR_TOKEN_RANGE);
      if (a.hint) a.hint[r] = -1;
    }
    for (int i = tid; i < k; i += TT) out[i] = -1;
    return;
  }
  if (len <= k) {  // every position, then padding
    if (tid == 0 && a.hint) a.hint[r] = -1;
    for (int i = tid; i < k; i += TT) out[i] = (i < len) ? i : -1;
    return;
  }
  const int n = (int)len;
  const int nw = (n + 31) >> 5;
  const uint32_t* row = (const uint32_t*)(a.scores + (int64_t)r * a.stride);

  // ---- pass B, for the top digits dlo .. dhi: keys above dhi -> selection bitmap (and counted
  // in s_nabove), keys inside -> candidate list.  Key order is float order (scores hold no NaN),
  // so the pass compares the scores themselves against the floats at the range's two edges,
  // with no key per score (at 128 x 65536: the plain launch 26.4 -> 24.1 us; the hinted bracket
  // pass 9.2 -> 7.2 us on cached rows, little on rows read from HBM).  A thread masks its
  // candidates in a batch; one wave scan and one LDS atomic per wave place them.
  auto classify = [&](uint32_t dlo, uint32_t dhi) {
    const float lo_f = digit_edge(dlo), hi_f = digit_edge(dhi + 1u);
    uint32_t nabove = 0;
    for_each_batch<U, false>(row, n, [&](u32x4 (&raw)[U], int b0) {
      uint32_t cmask = 0;
#pragma unroll
      for (int j = 0; j < U; ++j) {
        // a thread's four positions of a tile share one bitmap word: one atomic per tile
        const int p = b0 + j * TILE + 4 * tid;
        uint32_t nib = 0;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float x = __uint_as_float(raw[j][e]);
          const bool above = x >= hi_f;
          nib |= (above ? 1u : 0u) << e;
          cmask |= (x >= lo_f && !above ? 1u : 0u) << (j * V + e);
        }
        if (nib) {
          atomicOr(&selmap[p >> 5], nib << (p & 31));
          nabove += __popc(nib);
        }
      }
      const uint32_t c = __popc(cmask);
      const uint32_t incl = wave_scan_incl(c);
      uint32_t base = 0;
      if (lane == 63 && incl) base = atomicAdd(&s_ncand, incl);
      uint32_t idx = __shfl(base, 63) + incl - c;
      // candidates are rare: walk the set bits and take each score again (an L2 hit) rather
      // than branching over every slot of the batch
      while (cmask) {
        const int sb = __ffs(cmask) - 1;
        cmask &= cmask - 1u;
        const int p = b0 + (sb / V) * TILE + 4 * tid + (sb % V);
        if (idx < (uint32_t)CMAX) {
          ckey[idx] = order_key(row[p]);
          cpos[idx] = (uint32_t)p;
        }
        ++idx;
      }
    });
    const uint32_t total = wave_scan_incl(nabove);
    if (lane == 63 && total) atomicAdd(&s_nabove, total);
  };

  for (int i = tid; i < nw; i += TT) {
    selmap[i] = 0u;
    tiemap[i] = 0u;
  }
  if (tid == 0) {
    s_ncand = 0;
    s_nabove = 0;
  }
  const int32_t h_in = a.hint ? a.hint[r] : -1;
  bool hinted = h_in >= 0 && h_in < NBIN;  // the same in every thread
  __syncthreads();
  uint32_t d1 = 0, need = 0, prefix = 0;
  int fixed = 0;
  bool all_taken = false;
  if (hinted) {
    // ---- with a guess of the top digit (as from the previous decode step, whose scores moved
    // little): one pass collects the keys of the digit and its two neighbours; when the k-th
    // largest key is among them the histogram pass is not needed
    const uint32_t dlo = h_in > 0 ? (uint32_t)h_in - 1u : 0u;
    const uint32_t dhi = h_in < NBIN - 1 ? (uint32_t)h_in + 1u : (uint32_t)(NBIN - 1);
    classify(dlo, dhi);
    __syncthreads();
    const uint32_t above = s_nabove, nc = s_ncand;
    hinted = nc <= (uint32_t)CMAX && above < (uint32_t)k && (uint32_t)k <= above + nc;
    need = (uint32_t)k - above;
    __syncthreads();  // every thread has read the counts
    if (!hinted) {    // the guess missed: start over on the exact path
      for (int i = tid; i < nw; i += TT) selmap[i] = 0u;
      if (tid == 0) {
        s_ncand = 0;
        s_nabove = 0;
      }
    }
  }
  if (!hinted) {
    // ---- pass A: top digit
    // Two interleaved copies of the histogram, chosen by lane parity, in the candidate list
    // (pass B rebuilds it): lanes of a wave that hit one digit split over two adjacent words in
    // different banks, which halves the same-address serialisation of the LDS atomics (the
    // scores crowd into a few dozen digits); pass A 7.8 -> 7.2 us at 128 x 65536 (four copies: 7.6)
    uint32_t* hist2 = ckey;  // [2 NBIN] <= CMAX
    for (int i = tid; i < 2 * NBIN; i += TT) hist2[i] = 0u;
    __syncthreads();
    {
      // padding (key 0) lands in digit 0, which the search never reaches since len > k
      const uint32_t c = (uint32_t)(tid & 1);
      for_each_key<U>(row, n, [&](uint32_t u, int) { atomicAdd(&hist2[((u >> 20) << 1) | c], 1u); });
    }
    __syncthreads();
    for (int i = tid; i < NBIN; i += TT) hist[i] = hist2[2 * i] + hist2[2 * i + 1];
    __syncthreads();
    find_digit(hist, NBIN - 1, (uint32_t)k, wtot, &s_digit, &s_above);
    d1 = s_digit;
    const uint32_t in_d1 = hist[d1];  // keys with top digit d1
    need = (uint32_t)k - s_above;     // keys to take among those with top digit d1
    classify(d1, d1);
    __syncthreads();
    prefix = d1;
    fixed = 12;
    all_taken = in_d1 == need;
  }
  const uint32_t ncand = s_ncand;
  const bool overflow = ncand > (uint32_t)CMAX;  // only on the exact path (a guess is refused)

  uint32_t thr;
  if (hinted) {
    // ---- after the guessed bracket: the listed keys lie within three consecutive top digits,
    // i.e. within 3 * 2^20 of the bracket's base, so two 11-bit levels over key - base find
    // the k-th largest key (the top digit falls out of the first)
    const uint32_t base = (uint32_t)(h_in > 0 ? h_in - 1 : 0) << 20;
    const uint32_t end = (uint32_t)(h_in < NBIN - 1 ? h_in + 2 : NBIN) << 20;  // 0 for the last digit (2^32)
    const int topA = (int)((end - base - 1u) >> 11);                          // <= 1535
    for (int i = tid; i <= topA; i += TT) hist[i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < ncand; i += TT) {
      const uint32_t o = (ckey[i] - base) >> 11;  // <= topA for every listed key
      if (o <= (uint32_t)topA) atomicAdd(&hist[o], 1u);
    }
    __syncthreads();
    find_digit(hist, topA, need, wtot, &s_digit, &s_above);
    const uint32_t dA = s_digit, in_a = hist[dA];
    need -= s_above;
    d1 = (base + (dA << 11)) >> 20;
    __syncthreads();
    if (in_a == need) {  // every key of the bin is taken
      thr = base + (dA << 11) - 1u;
      need = 0u;
    } else {
      for (int i = tid; i < 2048; i += TT) hist[i] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < ncand; i += TT) {
        const uint32_t o = ckey[i] - base;
        if ((o >> 11) == dA) atomicAdd(&hist[o & 0x7FFu], 1u);
      }
      __syncthreads();
      find_digit(hist, 2047, need, wtot, &s_digit, &s_above);
      const uint32_t in_b = hist[s_digit];
      need -= s_above;
      thr = base + (dA << 11) + s_digit;
      if (in_b == need) {  // every key equal to it is taken: no tie left
        thr -= 1u;
        need = 0u;
      }
      __syncthreads();
    }
  } else {
    // ---- the next 12 bits, then the last 8: over the list, or over the row on overflow.  When
    // every key of the digit just chosen is taken (its count equals `need`), no tie is left to
    // resolve and the remaining levels are skipped: the threshold drops to just below that
    // digit's range and nothing is taken at it.
    for (int level = 0; level < 2 && !all_taken; ++level) {
      const int bits = level == 0 ? 12 : 8;
      const int shift = 32 - fixed - bits;
      const uint32_t dmask = (1u << bits) - 1u;
      for (int i = tid; i < NBIN; i += TT) hist[i] = 0u;
      __syncthreads();
      if (!overflow) {
        for (uint32_t i = tid; i < ncand; i += TT) {
          const uint32_t u = ckey[i];
          if ((u >> (32 - fixed)) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
        }
      } else {
        for_each_key<U>(row, n, [&](uint32_t u, int) {
          if (u != 0u && (u >> (32 - fixed)) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
        });
      }
      __syncthreads();
      find_digit(hist, (int)dmask, need, wtot, &s_digit, &s_above);
      const uint32_t in_d = hist[s_digit];
      prefix = (prefix << bits) | s_digit;
      need -= s_above;
      fixed += bits;
      all_taken = in_d == need;  // the same in every thread
      __syncthreads();
    }
    // the k-th largest key, `need` of the keys equal to it taken; or, with all_taken, one below
    // the lowest key of the chosen digit's range (keys > 0: the smallest, -inf's, is 0x007FFFFF)
    thr = prefix;
    if (all_taken) {
      thr = (prefix << (32 - fixed)) - 1u;
      need = 0u;
    }
  }

  // ---- candidates above thr are taken; those equal to it are ties
  if (!overflow) {
    for (uint32_t i = tid; i < ncand; i += TT) {
      const uint32_t u = ckey[i], p = cpos[i];
      if (u > thr) atomicOr(&selmap[p >> 5], 1u << (p & 31));
      else if (u == thr) atomicOr(&tiemap[p >> 5], 1u << (p & 31));
    }
  } else {
    for_each_key<U>(row, n, [&](uint32_t u, int p) {
      if ((u >> 20) == d1 && u > thr) atomicOr(&selmap[p >> 5], 1u << (p & 31));
      else if (u == thr) atomicOr(&tiemap[p >> 5], 1u << (p & 31));
    });
  }
  __syncthreads();

  // ---- output.  Each thread takes consecutive bitmap words (ceil(words / threads) each) and
  // one block scan of their (selected, tied) bit counts gives it the ties before them, hence
  // which of its ties are taken (the first `need` ties in position order); it writes each
  // word's final mask over the selection bitmap and the number of selected positions below
  // the word over the tie bitmap.  Then output i is found by thread i mod 1024: the last word
  // whose count below is <= i (a binary search), and in it the (i - count)-th set bit.
  const int wpt = (nw + TT - 1) / TT;
  const int w0 = tid * wpt;
  const int w1 = min(nw, w0 + wpt);
  uint32_t ns = 0, nt = 0;
  for (int w = w0; w < w1; ++w) {
    ns += __popc(selmap[w]);
    nt += __popc(tiemap[w]);
  }
  const uint64_t mine = ((uint64_t)ns << 32) | nt;
  uint64_t tot;
  const uint64_t excl = block_scan_incl<uint64_t>(mine, wtot64, &tot) - mine;
  uint32_t tie_before = (uint32_t)excl;
  uint32_t o = (uint32_t)(excl >> 32) + min(tie_before, need);
  uint32_t* below = tiemap;  // [nw] selected positions below each word
  for (int w = w0; w < w1; ++w) {
    uint32_t t = tiemap[w];
    // ties are taken in position order while fewer than `need` came before
    const uint32_t room = need > tie_before ? need - tie_before : 0u;
    const uint32_t nt_w = __popc(t);
    tie_before += nt_w;
    if (nt_w > room) {  // keep the first `room` set bits of t
      uint32_t keep = 0;
      for (uint32_t q = 0; q < room; ++q) {
        keep |= t & (~t + 1u);  // lowest set bit
        t &= t - 1u;
      }
      t = keep;
    }
    const uint32_t m = selmap[w] | t;
    selmap[w] = m;
    below[w] = o;
    o += __popc(m);
  }
  __syncthreads();
  for (int i = tid; i < k; i += TT) {
    // the last word with below[w] <= i; below[0] = 0 <= i, and the word holds bit i - below[w]
    int lo = 0, hi = nw - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (below[mid] <= (uint32_t)i) lo = mid;
      else hi = mid - 1;
    }
    uint32_t m = selmap[lo], j = (uint32_t)i - below[lo], pos = 0;
    // the j-th set bit of m: halve the window five times
#pragma unroll
    for (int h = 16; h >= 1; h >>= 1) {
      const uint32_t c = __popc(m & ((1u << h) - 1u));
      if (j >= c) {
        j -= c;
        m >>= h;
        pos += (uint32_t)h;
      }
    }
    out[i] = (int32_t)(lo * 32 + (int)pos);
  }
  if (tid == 0 && a.hint) a.hint[r] = (int32_t)d1;  // exact: the next call's guess
}

}  // namespace

void prepare_topk() {
  (void)hipFuncSetAttribute((const void*)topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)topk_lds_bytes());
  (void)hipGetLastError();
}

hipError_t launch_topk(const Geometry& g, int32_t n_req, const float* scores, int64_t stride, const int32_t* len,
                       int32_t* sel, int32_t* hint, int32_t* err, hipStream_t s) {
  TopkArgs a;
  a.hint = hint;
  a.scores = scores;
  a.stride = stride;
  a.len = len;
  a.sel = sel;
  a.err = err;
  a.cap = g.cap;
  a.k = g.k;
  hipLaunchKernelGGL(topk_kernel, dim3(n_req), dim3(TT), topk_lds_bytes(), s, a);
  return hipGetLastError();
}

}  // namespace hs
