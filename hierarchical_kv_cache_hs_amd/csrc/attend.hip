// Sparse MLA decode attention over resolved slots.
//
// What is computed (HiSparse paper abstract: each decode step reads only the selected
// KV entries; only KV placement changes, so the result is exact attention over the
// selected tokens): for every request r and query head h,
//   s_j = scale * <q_h, K_j>,  out_h = sum_j softmax(s)_j V_j,  lse_h = log sum_j exp(s_j),
// over the valid slots j of the request (slot -1 skipped), with K_j the 576 decoded values
// of the slot's entry (512 latent + 64 rope) and V_j its first 512 values (MLA form).
// FP8 entries decode as e4m3 code * fp32 block scale (one scale per 128 latent values).
// With pages of P tokens (paper abstract: NSA and Quest select blocks of tokens), a slot holds
// P rows and the attended tokens are the rows of the valid slots, optionally cut at each
// request's context length; the slot list is expanded to rows once, in the prologue.
//
// Design for gfx950.  The kernel is bound by HBM (about 1.3 MB of rows per request at
// k = 2048 against 71 MFLOP), so the design is about keeping rows in flight:
//  * grid (splits, requests); a workgroup of 8 wave64s walks its chunk of the selection in
//    64-token tiles.  Rows of a tile are gathered global -> LDS with 16-byte LDS-DMA loads
//    (global_load_lds_dwordx4), up to NBUF - 1 tiles ahead of the one being computed, so
//    the bytes in flight do not occupy registers; one barrier per tile both publishes the
//    tile and frees the buffer the next DMA refills;
//  * a tile's 64 tokens form four 16-token groups; each group is taken by a pair of waves
//    that split the 576 values: wave half 0 owns latent values 0..255 and rope 0..31, half 1
//    latent 256..511 and rope 32..63.  A wave converts only its half, computes its partial
//    scores, and the pair exchanges the partials through LDS; both then hold the full scores
//    and the same softmax state, and each accumulates P V for its own 256 output columns;
//  * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_bf16 with the
//    K values as the A operand (a lane holds 8 consecutive values of one token).  In S^T's
//    accumulator layout a lane holds one head and four consecutive tokens -- exactly the
//    A-operand layout of v_mfma_f32_16x16x16bf16_1k -- so P needs no data movement;
//  * V must reach the P V MFMA as four consecutive tokens of one column per lane, the
//    transpose of how rows are held.  gfx950's LDS transpose reads produce that layout
//    straight from the ring: per 32 value columns, one ds_read_b64_tr_b8 gives a lane the
//    fp8 codes of its four tokens in two columns (converted exactly to bf16), or two
//    ds_read_b64_tr_b16 give the bf16 values; they are read with the tile's K operands, so
//    the ring slot is freed at the same point as before (the reads are one asm block with its
//    own wait, see read_v_transposed);
//  * FP8 codes decode with v_cvt_scalef32_pk_bf16_fp8 (exact); block scales are applied per
//    token to the partial scores of each 128-value block and folded into P for the P V
//    product of that block;
//  * four token groups merge through LDS at the end; with splits > 1 each workgroup writes
//    an unnormalised partial (max, sum, 16 x 512 values) and a second kernel combines them in
//    split order;
//  * a step whose misses are still being copied (hs_fetch_misses) can attend in two parts:
//    the resident part skips the step's victim slots (an LDS bitmap of the miss list, built
//    in the prologue inside the then idle ring) and may run while the copy writes those
//    slots; the fetched part walks the compact miss list once the rows have landed.  The
//    resident part writes split partials; a fetched part of one workgroup per request merges
//    them in its epilogue (they were written by an earlier kernel on the stream, so no fence
//    is needed), a fetched part of several leaves the merge to the combine kernel;
//  * fp32-output mode: P enters the P V product as a sum of three bf16 terms (hi, mid, lo:
//    each the round-to-nearest-even of what the previous ones leave), which carries P to 2^-27
//    relative -- below fp32 rounding -- so the output is fp32 attention; it costs two more
//    MFMAs per P V block.  (A last-arriving-workgroup combine needs a device-scope fence in every
//    workgroup; on this chip each such fence writes back an XCD's L2, and they serialize.)

#include <math.h>

#include <mutex>

#include "hs_internal.h"

namespace hs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVES = 8;
constexpr int NT = WAVES * 64;
constexpr int GROUPS = 4;                   // 16-token groups per tile
constexpr int HMAX = 16;                    // heads per workgroup (one MFMA tile)
constexpr int DQK = 576;                    // q.K length
constexpr int DV = 512;                     // value length
constexpr int KB_HALF = 9;                  // reduction blocks of 32 values per half
constexpr int PART = 2 * HMAX + HMAX * DV;  // floats of one split partial
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttendArgs {
  const uint8_t* buf;     // layer's rows [n][B][stride]
  const int32_t* slots;   // [n_req][k >> lgP] slots of the selected units
  const int32_t* sel;     // [n_req][k >> lgP] the selection, or null (no length cut)
  const int32_t* len;     // [n_req] context length in tokens (with sel)
  const uint16_t* q;      // [n_req][heads][576] bf16
  void* out;              // [n_req][heads][512] bf16, or fp32 in fp32-output mode
  float* lse;             // [n_req][heads] or null
  float* part;            // [n][part_stride][PART]
  const int32_t* ml_slot; // [n_req][k >> lgP] this step's victim slots, miss list order (parts)
  const int32_t* ml_tok;  // [n_req][k >> lgP] the units fetched into them
  const int32_t* ml_cnt;  // [n_req] misses of this step
  int64_t stride;         // bytes between token rows
  int64_t rstride;        // bytes between requests: B token rows, then zero rows
  int32_t k, B, heads, chunk, splits;   // k and B count token rows (units times P)
  int32_t lgP;            // log2 of the rows per slot
  int32_t part_mode;      // ATT_ALL, ATT_RESIDENT or ATT_FETCHED
  int32_t part_stride;    // partials per request in `part`
  int32_t part0;          // this launch's first partial
  int32_t to_part;        // write partials even with one split
  int32_t merge_prev;     // one split: also merge partials 0 .. part0-1 and write out / lse
  float scale_log2;       // softmax scale * log2(e)
};

// Which entries a launch attends.
enum PartMode : int {
  ATT_ALL = 0,       // every valid entry of the slot list
  ATT_RESIDENT = 1,  // the entries whose slot is not one of this step's victims
  ATT_FETCHED = 2,   // the miss list: the rows just copied into the victim slots
};

__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Eight E4M3FN codes -> eight bf16, exact (E4M3 values, subnormals included, are bf16
// values): v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two codes per instruction.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 v;
  v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return v;
}

// Four E4M3FN codes (bytes of w, in order) -> four bf16, exact.
__device__ __forceinline__ s16x4 e4m3x4_to_bf16x4(uint32_t w) {
  u32x2 v;
  v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return __builtin_bit_cast(s16x4, v);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Four fp32 -> packed bf16, round to nearest even (two v_cvt_pk_bf16_f32).
__device__ __forceinline__ s16x4 pack4_rne(float a, float b, float c, float d) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  u32x2 v;
  v[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  v[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){c, d}, bf16x2));
  return __builtin_bit_cast(s16x4, v);
}

// x[j] -> three packed bf16 terms with hi + mid + lo = x to 2^-27 relative: each term is the
// round-to-nearest-even of the remainder the previous terms leave (subtractions exact in fp32).
__device__ __forceinline__ void split3(const float (&x)[4], s16x4& hi, s16x4& mid, s16x4& lo) {
  hi = pack4_rne(x[0], x[1], x[2], x[3]);
  const u32x2 h = __builtin_bit_cast(u32x2, hi);
  float r[4] = {x[0] - bf16_lo_to_f32(h[0]), x[1] - bf16_hi_to_f32(h[0]), x[2] - bf16_lo_to_f32(h[1]),
                x[3] - bf16_hi_to_f32(h[1])};
  mid = pack4_rne(r[0], r[1], r[2], r[3]);
  const u32x2 m = __builtin_bit_cast(u32x2, mid);
  lo = pack4_rne(r[0] - bf16_lo_to_f32(m[0]), r[1] - bf16_hi_to_f32(m[0]), r[2] - bf16_lo_to_f32(m[1]),
                 r[3] - bf16_hi_to_f32(m[1]));
}

// Value offset (within the 576) of reduction block kb (0..17) for lane group g: latent
// blocks kb = 4b + i hold d = 128b + 32g + 8i + [0, 8); rope blocks kb = 16 + i hold
// d = 512 + 16g + 8i + [0, 8).  Half hf owns latent kb 8hf..8hf+7 and rope kb 16 + hf.
__device__ __forceinline__ int kb_offset(int kb, int g) {
  return kb < 16 ? 128 * (kb >> 2) + 32 * g + 8 * (kb & 3) : 512 + 16 * g + 8 * (kb - 16);
}

// Output column of accumulator tile tau (= 16 value half + 2 block + sigma) at tile column n:
// block i of half hf covers columns 256 hf + 32 i .. + 31, sigma its 16-column halves.
__device__ __forceinline__ int out_col(int tau, int n) { return 16 * tau + n; }

// Reductions across the four 16-lane rows of a wave with gfx950's row-swap moves (plain VALU,
// no LDS round trip).  v_permlane16_swap(x, x) leaves every lane holding its own value and
// that of the lane 16 away (rows 0<->1, 2<->3); v_permlane32_swap(x, x) likewise for the lane
// 32 away.  Both operands combine in the same order in both lanes, so every lane of the wave
// ends with the bitwise same result.
__device__ __forceinline__ float rows_max(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ float rows_sum(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A workgroup barrier without the fence __syncthreads() implies: that fence would wait for
// every LDS-DMA load in flight, which is exactly what the ring must not do.  LDS writes made
// before it must be waited for explicitly (lgkmcnt) by the caller.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void lds_done_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 32-bit LDS address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// A tile's transposed V operands for this lane (see voff): fp8, 8 reads of 8 codes at columns
// 32 i; bf16, 16 reads of 4 values at columns 16 i.  The reads are written out in one asm
// block that ends by waiting for them: the compiler's own transpose-read builtins are treated
// as possibly aliasing the ring's in-flight LDS-DMA loads and get a wait for all of them
// (every tile prefetched behind this one), which serialises the ring.  The tile read here
// has landed: its DMA completed before the barrier that published it.
template <int LAYOUT>
__device__ __forceinline__ void read_v_transposed(uint32_t a, i32x2 (&vr)[LAYOUT == 0 ? 16 : 8]) {
  if constexpr (LAYOUT == 1) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8\n\t"
        "ds_read_b64_tr_b8 %1, %8 offset:32\n\t"
        "ds_read_b64_tr_b8 %2, %8 offset:64\n\t"
        "ds_read_b64_tr_b8 %3, %8 offset:96\n\t"
        "ds_read_b64_tr_b8 %4, %8 offset:128\n\t"
        "ds_read_b64_tr_b8 %5, %8 offset:160\n\t"
        "ds_read_b64_tr_b8 %6, %8 offset:192\n\t"
        "ds_read_b64_tr_b8 %7, %8 offset:224\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]),
          "=&v"(vr[7])
        : "v"(a)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:32\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %16 offset:96\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:128\n\t"
        "ds_read_b64_tr_b16 %5, %16 offset:160\n\t"
        "ds_read_b64_tr_b16 %6, %16 offset:192\n\t"
        "ds_read_b64_tr_b16 %7, %16 offset:224\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:256\n\t"
        "ds_read_b64_tr_b16 %9, %16 offset:288\n\t"
        "ds_read_b64_tr_b16 %10, %16 offset:320\n\t"
        "ds_read_b64_tr_b16 %11, %16 offset:352\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:384\n\t"
        "ds_read_b64_tr_b16 %13, %16 offset:416\n\t"
        "ds_read_b64_tr_b16 %14, %16 offset:448\n\t"
        "ds_read_b64_tr_b16 %15, %16 offset:480\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]),
          "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]), "=&v"(vr[12]), "=&v"(vr[13]),
          "=&v"(vr[14]), "=&v"(vr[15])
        : "v"(a)
        : "memory");
  }
}

template <int LAYOUT>
struct TileGeo {
  static constexpr int E = LAYOUT == 0 ? 1152 : 656;      // bytes per row
  static constexpr int VR = LAYOUT == 0 ? 16 : 8;         // 8-byte transposed V reads per wave and tile
  static constexpr int C = E / 16;                        // 16-byte chunks per row
  static constexpr int NBUF = LAYOUT == 0 ? 2 : 3;        // ring depth
  static constexpr int T = 16 * GROUPS;                   // tokens per tile
  static constexpr int TILE = T * E;                      // bytes per tile
  static constexpr int CHUNKS = T * C;
  static constexpr int L0 = (CHUNKS + NT - 1) / NT;       // DMA instructions per tile, wave 0
  static constexpr int MAXCHUNK = LAYOUT == 0 ? 1024 : 2048;  // tokens per workgroup
  // Score exchange slots.  With two, one barrier per tile suffices (a slot is rewritten only
  // two tiles later, after a barrier its reader has passed); the bf16 ring leaves room for one
  // only, and a second barrier per tile guards its reuse.
  static constexpr int XCH = LAYOUT == 0 ? 1 : 2;
  static_assert(CHUNKS % 64 == 0, "tile chunks must fill whole waves");
};

// DMA instructions wave w issues per tile: j with j * NT + 64 w < CHUNKS (wave-uniform).
template <int LAYOUT>
__device__ __forceinline__ int dma_per_tile(int w) {
  return (TileGeo<LAYOUT>::CHUNKS - 64 * w + NT - 1) / NT;
}

// Wait until at most `pending` (0 .. NBUF - 1) later tiles of this wave's DMA are outstanding;
// `per` is the wave's DMA instruction count per tile (the counter counts instructions).
template <int LAYOUT>
__device__ __forceinline__ void wait_tiles(int pending, int per) {
  if (LAYOUT == 0) {
    static_assert(TileGeo<0>::NBUF == 2 && TileGeo<0>::CHUNKS % NT == 0, "wait table");
    if (pending == 0) wait_vmcnt<0>();
    else wait_vmcnt<TileGeo<0>::L0>();
  } else {
    static_assert(TileGeo<1>::NBUF == 3 && TileGeo<1>::L0 == 6, "wait table");
    if (pending == 0) wait_vmcnt<0>();
    else if (pending == 1) { if (per == 6) wait_vmcnt<6>(); else wait_vmcnt<5>(); }
    else { if (per == 6) wait_vmcnt<12>(); else wait_vmcnt<10>(); }
  }
}

template <int LAYOUT>
constexpr size_t ring_bytes() { return (size_t)TileGeo<LAYOUT>::NBUF * TileGeo<LAYOUT>::TILE; }


template <int LAYOUT>
constexpr size_t attend_lds_bytes() {
  return ring_bytes<LAYOUT>() + TileGeo<LAYOUT>::MAXCHUNK * sizeof(int32_t) +
         TileGeo<LAYOUT>::XCH * WAVES * 64 * sizeof(f32x4);
}

constexpr int MAXPREV = 16;  // earlier partials a workgroup can merge (the resident part's splits)
constexpr size_t kStaticLds = (3 * GROUPS + 1 + MAXPREV) * HMAX * sizeof(float);  // wm, wl, fac, inv_l, pfac
constexpr size_t kParkBytes = (size_t)GROUPS * 2 * 16 * 64 * sizeof(f32x4);   // parked accumulators
static_assert(attend_lds_bytes<0>() + kStaticLds <= kLdsLimit, "bf16 LDS budget");
static_assert(attend_lds_bytes<1>() + kStaticLds <= kLdsLimit, "fp8 LDS budget");
static_assert(kParkBytes <= attend_lds_bytes<0>() && kParkBytes <= attend_lds_bytes<1>(), "parking fits");

template <int LAYOUT, bool F32>
__global__ __launch_bounds__(NT, 1) void attend_kernel(AttendArgs a) {
  using G = TileGeo<LAYOUT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* ring = smem;                                              // [NBUF][TILE]
  int32_t* slot_lds = (int32_t*)(smem + ring_bytes<LAYOUT>());       // [MAXCHUNK]
  f32x4* xch = (f32x4*)(smem + ring_bytes<LAYOUT>() + G::MAXCHUNK * sizeof(int32_t));  // [WAVES][64]
  f32x4* o_park = (f32x4*)smem;  // after the loop: [GROUPS][2][16][64] accumulators
  __shared__ float wm[GROUPS][HMAX];
  __shared__ float wl[GROUPS][HMAX];
  __shared__ float fac[GROUPS][HMAX];
  __shared__ float inv_l[HMAX];
  __shared__ float pfac[MAXPREV][HMAX];  // merge_prev: factors of the earlier partials
  __shared__ int wlast[WAVES];

  const int s = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int tg = w & 3;          // token group within a tile
  const int hf = w >> 2;         // value half
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int heads = a.heads;

  const int tok0 = s * a.chunk;
  const int tok1 = min(a.k, tok0 + a.chunk);
  const int ntok = tok1 > tok0 ? tok1 - tok0 : 0;
  const int ntiles_all = (ntok + G::T - 1) / G::T;
  const uint8_t* rbase = a.buf + (int64_t)r * a.rstride;

  // ---- this workgroup's row list (invalid, cut or missing -> -1) and this wave's Q operands
  {
    const int lg = a.lgP;
    const int ku = a.k >> lg, bu = a.B >> lg;
    const int mode = a.part_mode;
    const int32_t* su = (mode == ATT_FETCHED ? a.ml_slot : a.slots) + (int64_t)r * ku;
    const int32_t* cu = nullptr;  // the units, where the context length cuts
    if (a.len) cu = (mode == ATT_FETCHED ? a.ml_tok : a.sel) + (int64_t)r * ku;
    const int64_t len = a.len ? (int64_t)a.len[r] : 0;
    int units = ku;  // entries of the list
    uint32_t* vbits = (uint32_t*)ring;  // ATT_RESIDENT: this step's victim slots (prologue only)
    if (mode != ATT_ALL) {
      const int m = a.ml_cnt[r];
      units = m < 0 ? 0 : (m < ku ? m : ku);
    }
    if (mode == ATT_RESIDENT) {
      for (int x = tid; x < (bu + 31) >> 5; x += NT) vbits[x] = 0u;
      __syncthreads();
      const int32_t* vs = a.ml_slot + (int64_t)r * ku;
      for (int q = tid; q < units; q += NT) {
        const int32_t j = vs[q];
        if (j >= 0 && j < bu) atomicOr(&vbits[j >> 5], 1u << (j & 31));
      }
      __syncthreads();
      units = ku;
    }
    // A thread's entries are i = tid + e * NT, e < PER (the chunk, rounded up to whole tiles,
    // is at most MAXCHUNK): all their slot and unit loads are issued before any is used, so the
    // list costs one global round trip, not one per entry.
    constexpr int PER = G::MAXCHUNK / NT;
    static_assert(G::MAXCHUNK % NT == 0, "whole entries per thread");
    int32_t jv[PER], cv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = tid + e * NT;
      const int u = (tok0 + i) >> lg;
      const bool in = i < ntok && u < units;
      jv[e] = in ? su[u] : -1;
      cv[e] = (in && cu) ? cu[u] : 0;
    }
    int last = 0;  // one past this thread's last valid entry
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = tid + e * NT;
      if (i >= ntiles_all * G::T) break;
      const int o = (tok0 + i) & ((1 << lg) - 1);
      const int32_t j = jv[e];
      int32_t v = -1;
      if (j >= 0 && j < bu && !(mode == ATT_RESIDENT && ((vbits[j >> 5] >> (j & 31)) & 1u))) {
        v = (j << lg) + o;
        if (cu && (cv[e] < 0 || ((int64_t)cv[e] << lg) + o >= len)) v = -1;
      }
      slot_lds[i] = v;
      if (v >= 0) last = i + 1;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o));
    if (lane == 0) wlast[w] = last;
  }
  u32x4 qreg[KB_HALF];
#pragma unroll
  for (int i = 0; i < KB_HALF; ++i) {
    const int kb = (i < 8) ? 8 * hf + i : 16 + hf;
    qreg[i] = (c16 < heads) ? load16(a.q + ((int64_t)r * heads + c16) * DQK + kb_offset(kb, g))
                            : (u32x4){0u, 0u, 0u, 0u};
  }
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0);
  // tiles past the last valid entry (trailing padding: short contexts, cut pages) are skipped
  int nvalid = 0;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) nvalid = max(nvalid, wlast[v]);
  const int ntiles = (nvalid + G::T - 1) / G::T;

  const int wu = __builtin_amdgcn_readfirstlane(w) & (WAVES - 1);  // the wave index, scalar and known < WAVES
  const int per = dma_per_tile<LAYOUT>(wu);
  // The row and 16-byte column of each of this lane's DMA chunks are the same in every tile.
  int drow[G::L0], dcol[G::L0];
#pragma unroll
  for (int j = 0; j < G::L0; ++j) {
    const int c = j * NT + 64 * wu + lane;
    drow[j] = c / G::C;
    dcol[j] = 16 * (c - drow[j] * G::C);
  }
  const uint32_t stride32 = (uint32_t)a.stride;  // a request's rows span less than 4 GiB
  const int32_t zero_slot = a.B;                 // the zero row after the request's slots
  auto issue = [&](int u) {
    uint8_t* dst = ring + (u % G::NBUF) * G::TILE;
    const int32_t* su = slot_lds + u * G::T;
    // All slots first, then the loads: the compiler keeps an LDS read that follows an
    // LDS-DMA load behind it, so interleaving them costs one LDS round trip per load.
    int32_t sl[G::L0];
#pragma unroll
    for (int j = 0; j < G::L0; ++j) sl[j] = (j * NT + 64 * wu < G::CHUNKS) ? su[drow[j]] : 0;
#pragma unroll
    for (int j = 0; j < G::L0; ++j) {
      const int base = j * NT + 64 * wu;
      if (base < G::CHUNKS) {
        // padding reads the zero row, so its operands are finite and contribute nothing
        const uint32_t off = (uint32_t)(sl[j] < 0 ? zero_slot : sl[j]) * stride32 + (uint32_t)dcol[j];
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(rbase + off),
                                         (void __attribute__((address_space(3)))*)(dst + base * 16), 16, 0, 0);
      }
    }
  };

  // This lane's address (bytes into a tile) of its transposed V reads, for block 0 of its half:
  // fp8 -- source lane s = c16 of lane group g reads the 8 codes at row 4 g + (s/2 mod 4) of
  // the wave's token group, column 16 (s/8) + 8 (s mod 2); the transpose hands lane (g, n)
  // tokens 4g..4g+3 of columns n and 16 + n.  bf16 -- source lane s reads the 4 values at
  // row 4 g + s/4, column 4 (s mod 4) (+16 for the second read); lane (g, n) receives tokens
  // 4g..4g+3 of column n.  Block i adds 32 i columns.
  const int voff = (LAYOUT == 1)
                       ? (16 * tg + 4 * g + ((c16 >> 1) & 3)) * G::E + 256 * hf + 16 * (c16 >> 3) + 8 * (c16 & 1)
                       : (16 * tg + 4 * g + (c16 >> 2)) * G::E + 2 * (256 * hf + 4 * (c16 & 3));

  f32x4 O[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) O[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // This wave's K operands (its half of the 576 values of tokens 16 tg .. 16 tg + 15 of
  // tile t, converted to bf16), block scales of tokens 4g + j, and the slots of tokens
  // 4g .. 4g + 3 (-1 = padding).
  auto load_tile = [&](int t, u32x4 (&kr)[KB_HALF], float (&scl)[4][2], u32x4& vqr, i32x2 (&vr)[G::VR]) {
    const uint8_t* tile = ring + (t % G::NBUF) * G::TILE;
    const uint8_t* row = tile + (16 * tg + c16) * G::E;  // this lane's token (A-operand row)
    vqr = *(const u32x4*)(slot_lds + t * G::T + 16 * tg + 4 * g);
    read_v_transposed<LAYOUT>(lds_addr(tile + voff), vr);
    if (LAYOUT == 0) {
#pragma unroll
      for (int i = 0; i < KB_HALF; ++i) {
        const int kb = (i < 8) ? 8 * hf + i : 16 + hf;
        kr[i] = *(const u32x4*)(row + 2 * kb_offset(kb, g));
      }
    } else {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int b = 2 * hf + bb;
        const u32x4 lo = *(const u32x4*)(row + 128 * b + 32 * g);
        const u32x4 hi = *(const u32x4*)(row + 128 * b + 32 * g + 16);
        kr[4 * bb + 0] = e4m3x8_to_bf16x8(lo[0], lo[1]);
        kr[4 * bb + 1] = e4m3x8_to_bf16x8(lo[2], lo[3]);
        kr[4 * bb + 2] = e4m3x8_to_bf16x8(hi[0], hi[1]);
        kr[4 * bb + 3] = e4m3x8_to_bf16x8(hi[2], hi[3]);
      }
      kr[8] = *(const u32x4*)(row + 528 + 32 * g + 16 * hf);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 sv = *(const u32x2*)(tile + (16 * tg + 4 * g + j) * G::E + 512 + 8 * hf);
        scl[j][0] = __uint_as_float(sv[0]);
        scl[j][1] = __uint_as_float(sv[1]);
      }
    }
  };

  // Partial S^T[tok][h] over this wave's half of the values.
  auto qk = [&](const u32x4 (&kr)[KB_HALF], const float (&scl)[4][2]) -> f32x4 {
    f32x4 part;
    if (LAYOUT == 0) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KB_HALF; i += 2)
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[i]),
                                                       __builtin_bit_cast(bf16x8, qreg[i]), acc0, 0, 0, 0);
#pragma unroll
      for (int i = 1; i < KB_HALF; i += 2)
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[i]),
                                                       __builtin_bit_cast(bf16x8, qreg[i]), acc1, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) part[j] = acc0[j] + acc1[j];
    } else {
      f32x4 accb[2], accr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        accb[bb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          accb[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[4 * bb + i]),
                                                             __builtin_bit_cast(bf16x8, qreg[4 * bb + i]),
                                                             accb[bb], 0, 0, 0);
      }
      accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[8]),
                                                     __builtin_bit_cast(bf16x8, qreg[8]), accr, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) part[j] = accr[j] + scl[j][0] * accb[0][j] + scl[j][1] * accb[1][j];
    }
    return part;
  };

  // Pair exchange of tile t's partial scores.  One barrier publishes them together with this
  // wave's share of tile t + 1, and frees tile t's buffer (every wave holds its K values in
  // registers by then), which takes tile t + NBUF.
  auto publish = [&](int t, const f32x4& part) {
    f32x4* xs = xch + (t % G::XCH) * (WAVES * 64);
    if (G::XCH == 1) lds_done_barrier();  // the partner has read the previous tile's scores
    xs[w * 64 + lane] = part;
    wait_tiles<LAYOUT>(max(0, min(G::NBUF - 2, ntiles - 2 - t)), per);
    lds_done_barrier();
    if (t + G::NBUF < ntiles) issue(t + G::NBUF);
  };

  // A tile's buffer is refilled as soon as every wave holds the tile's K values in
  // registers, so all NBUF buffers start in flight.
  for (int u = 0; u < G::NBUF && u < ntiles; ++u) issue(u);

  float sccur[4][2];
  u32x4 vqcur;
  f32x4 partcur;
  i32x2 vcur[G::VR];  // tile t's V operands (transposed reads)
  if (ntiles > 0) {
    u32x4 k0[KB_HALF];
    wait_tiles<LAYOUT>(min(G::NBUF - 1, ntiles - 1), per);  // this wave's share of tile 0
    barrier_only();
    load_tile(0, k0, sccur, vqcur, vcur);
    partcur = qk(k0, sccur);
    publish(0, partcur);
  }

  // Software pipelined: while the P V products of tile t run on the matrix cores, the
  // operands of tile t + 1 are read, converted and multiplied by Q in the same block.
  for (int t = 0; t < ntiles; ++t) {
    const f32x4 other = xch[(t % G::XCH) * (WAVES * 64) + (w ^ 4) * 64 + lane];
    float s2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sj = partcur[j] + other[j];
      s2[j] = (vqcur[j] != 0xFFFFFFFFu) ? sj * a.scale_log2 : -INFINITY;
    }

    // ---- online softmax for head c16 over tokens 4g + j of this group
    const float mx = rows_max(fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3])));
    // The reference maximum moves only when a score exceeds it by more than 2^8 (lazy
    // rescaling): P = 2^(s - m) then stays below 256, well inside fp32 and bf16 range, and the
    // accumulator rescale below runs only on the rare tiles that move some head's reference.
    const float m_new = (mx > m_run + 8.f) ? mx : m_run;
    float alpha = 1.f, p[4] = {0.f, 0.f, 0.f, 0.f};
    if (m_new != -INFINITY) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(s2[j] - m_new);
    }
    const float rs = rows_sum((p[0] + p[1]) + (p[2] + p[3]));
    l_run = l_run * alpha + rs;
    m_run = m_new;

    // rescale the accumulator rows (heads 4g + j) only when some head's maximum moved
    if (__any(alpha != 1.f)) {
      float aj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) aj[j] = __shfl(alpha, 4 * g + j);
#pragma unroll
      for (int tau = 0; tau < 16; ++tau)
#pragma unroll
        for (int j = 0; j < 4; ++j) O[tau][j] *= aj[j];
    }

    s16x4 pa[2], pm[2], pl[2];  // P (fp32-output mode: its hi, mid and lo bf16 terms)
    if (LAYOUT == 0) {
      if (F32) split3(p, pa[0], pm[0], pl[0]);
      else pa[0] = pack4_rne(p[0], p[1], p[2], p[3]);
      pa[1] = pa[0];
      pm[1] = pm[0];
      pl[1] = pl[0];
    } else {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const float x[4] = {p[0] * sccur[0][bb], p[1] * sccur[1][bb], p[2] * sccur[2][bb], p[3] * sccur[3][bb]};
        if (F32) split3(x, pa[bb], pm[bb], pl[bb]);
        else pa[bb] = pack4_rne(x[0], x[1], x[2], x[3]);
      }
    }

    // ---- tile t + 1's operands (its bytes landed before the last barrier); the last
    // iteration re-reads tile t, which keeps this block free of branches
    u32x4 knext[KB_HALF];
    float scnext[4][2];
    u32x4 vqnext;
    i32x2 vnext[G::VR];
    load_tile(min(t + 1, ntiles - 1), knext, scnext, vqnext, vnext);

    // ---- O += P V over this half's 256 columns (block i: columns 256 hf + 32 i .. + 31)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const s16x4 P = pa[i >> 2];
      s16x4 v0, v1;
      if (LAYOUT == 1) {
        v0 = e4m3x4_to_bf16x4((uint32_t)vcur[i][0]);
        v1 = e4m3x4_to_bf16x4((uint32_t)vcur[i][1]);
      } else {
        v0 = __builtin_bit_cast(s16x4, vcur[2 * i]);
        v1 = __builtin_bit_cast(s16x4, vcur[2 * i + 1]);
      }
      if (F32) {  // smallest terms first
        O[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl[i >> 2], v0, O[2 * i], 0, 0, 0);
        O[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl[i >> 2], v1, O[2 * i + 1], 0, 0, 0);
        O[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pm[i >> 2], v0, O[2 * i], 0, 0, 0);
        O[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pm[i >> 2], v1, O[2 * i + 1], 0, 0, 0);
      }
      O[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(P, v0, O[2 * i], 0, 0, 0);
      O[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(P, v1, O[2 * i + 1], 0, 0, 0);
    }

    const f32x4 partnext = qk(knext, scnext);
#pragma unroll
    for (int i = 0; i < G::VR; ++i) vcur[i] = vnext[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sccur[j][0] = scnext[j][0];
      sccur[j][1] = scnext[j][1];
    }
    vqcur = vqnext;
    partcur = partnext;
    if (t + 1 < ntiles) publish(t + 1, partcur);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- merge the four token groups (fixed order).  Each wave parks its accumulators in
  // the now idle ring, in their register layout (lane-contiguous 16-byte rows, no bank
  // conflicts); 16 threads work out each head's merge factors once; then every thread
  // combines float4s of 4 heads x 1 column.
  if (hf == 0 && g == 0) {
    wm[tg][c16] = m_run;
    wl[tg][c16] = l_run;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) o_park[((tg * 2 + hf) * 16 + i) * 64 + lane] = O[i];
  __syncthreads();
  // direct: write out / lse (one split, or one split that also merges the earlier partials of
  // its request, which a kernel earlier on the stream wrote); else a partial for the combine
  const bool prev = a.merge_prev != 0;
  const bool direct = a.splits == 1 && (!a.to_part || prev);
  float* mypart = a.part + ((int64_t)r * a.part_stride + a.part0 + s) * PART;
  const float* prevpart = a.part + (int64_t)r * a.part_stride * PART;  // prev: partials 0 .. part0-1
  if (tid < HMAX) {
    const int h = tid;
    float M = wm[0][h];
#pragma unroll
    for (int v = 1; v < GROUPS; ++v) M = fmaxf(M, wm[v][h]);
    if (prev)
      for (int v = 0; v < a.part0; ++v) M = fmaxf(M, prevpart[v * PART + h]);
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < GROUPS; ++v) {
      const float f = (M == -INFINITY) ? 0.f : exp2f(wm[v][h] - M);
      fac[v][h] = f;
      L += f * wl[v][h];
    }
    if (prev)
      for (int v = 0; v < a.part0; ++v) {
        const float f = (M == -INFINITY) ? 0.f : exp2f(prevpart[v * PART + h] - M);
        pfac[v][h] = f;
        L += f * prevpart[v * PART + HMAX + h];
      }
    if (direct) {
      inv_l[h] = L > 0.f ? 1.f / L : 0.f;
      if (a.lse && h < heads) a.lse[(int64_t)r * heads + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    } else {
      inv_l[h] = 1.f;
      mypart[h] = M;
      mypart[HMAX + h] = L;
    }
  }
  __syncthreads();
  // slot e = (value half, accumulator tile, lane): heads 4 (lane / 16) + j, one column
  for (int e = tid; e < 2 * 16 * 64; e += NT) {
    const int he = e >> 10, tau = (e >> 6) & 15, ln = e & 63;
    const int h0 = 4 * (ln >> 4);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < GROUPS; ++v) {
      const f32x4 o = o_park[((v * 2 + he) * 16 + tau) * 64 + ln];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += fac[v][h0 + j] * o[j];
    }
    const int col = out_col(16 * he + tau, ln & 15);
    if (prev)
      for (int v = 0; v < a.part0; ++v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += pfac[v][h0 + j] * prevpart[v * PART + 2 * HMAX + (h0 + j) * DV + col];
      }
    if (direct) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (h0 + j < heads) {
          const int64_t o = ((int64_t)r * heads + h0 + j) * DV + col;
          if (F32) ((float*)a.out)[o] = acc[j] * inv_l[h0 + j];
          else ((uint16_t*)a.out)[o] = (uint16_t)bf16_rne(acc[j] * inv_l[h0 + j]);
        }
    } else {
      // an unnormalised partial (per-head max and sum, 16 x 512 values); the combine kernel
      // that follows on the stream merges the splits (the kernel boundary makes these stores
      // visible, so no device-scope fence is needed)
#pragma unroll
      for (int j = 0; j < 4; ++j) mypart[2 * HMAX + (h0 + j) * DV + col] = acc[j];
    }
  }
}

// Merges the splits of every request in split order: with M the largest split maximum,
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s  and  lse = (M + log2 L) ln 2.
// Grid (HMAX * DV / 4 / 256, requests): each thread owns four consecutive outputs of one head
// and issues its splits' loads independently.
constexpr int COMBINE_THREADS = 256;
constexpr int COMBINE_BLOCKS = HMAX * DV / 4 / COMBINE_THREADS;

template <bool F32>
__global__ __launch_bounds__(COMBINE_THREADS) void combine_kernel(const float* __restrict__ part, int splits, int heads,
                                                                  void* __restrict__ out, float* __restrict__ lse) {
  const int r = blockIdx.y;
  const int i4 = blockIdx.x * COMBINE_THREADS + threadIdx.x;   // float4 index within 16 x 512
  const int h = (4 * i4) / DV;
  if (h >= heads) return;
  const float* prow = part + (int64_t)r * splits * PART;
  float M = -INFINITY;
  for (int v = 0; v < splits; ++v) M = fmaxf(M, prow[v * PART + h]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    for (int v = 0; v < splits; ++v) {
      const float fv = exp2f(prow[v * PART + h] - M);
      const f32x4 o = *(const f32x4*)(prow + v * PART + 2 * HMAX + 4 * i4);
      L += fv * prow[v * PART + HMAX + h];
      acc += fv * o;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int64_t o = ((int64_t)r * heads + h) * DV + (4 * i4) % DV;
  if (F32) {
    *(f32x4*)((float*)out + o) = acc * inv;
  } else {
    uint2 packed;
    packed.x = bf16_rne(acc[0] * inv) | (bf16_rne(acc[1] * inv) << 16);
    packed.y = bf16_rne(acc[2] * inv) | (bf16_rne(acc[3] * inv) << 16);
    *(uint2*)((uint16_t*)out + o) = packed;
  }
  if ((4 * i4) % DV == 0 && lse) lse[(int64_t)r * heads + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

int max_chunk(const Geometry& g) {
  return g.layout == HS_KV_BF16_576 ? TileGeo<0>::MAXCHUNK : TileGeo<1>::MAXCHUNK;
}

}  // namespace

int attend_splits(const Geometry& g, int n_req) {
  // A workgroup's ring fills most of a compute unit's LDS, so one runs per CU: the splits keep
  // n_req * splits within the 256 CUs (one round -- a second, partial round costs more than the
  // idle CUs of a floor), with at most MAXCHUNK tokens and at least one 64-token tile each.
  const int tokens = (int)attend_tokens(g);
  int s = 256 / (n_req > 0 ? n_req : 1);
  const int by_len = (tokens + 63) / 64;
  const int need = (tokens + max_chunk(g) - 1) / max_chunk(g);
  if (s > by_len) s = by_len;
  if (s > 16) s = 16;
  if (s < need) s = need;
  return s < 1 ? 1 : s;
}

// Splits of the fetched part: the whole miss list may fill the selection, MAXCHUNK tokens each.
int fetched_splits(const Geometry& g) {
  const int tokens = (int)attend_tokens(g);
  return (tokens + max_chunk(g) - 1) / max_chunk(g);
}

size_t attend_partial_floats(const Geometry& g) {
  // per request slot: room for the largest n * (partials per request) over the launch sizes the
  // handle allows -- a split launch, or a resident part and a fetched part
  int64_t most = 0;
  const int sf = fetched_splits(g);
  for (int n = 1; n <= g.n; ++n) {
    const int s = attend_splits(g, n) + sf;
    if ((int64_t)n * s > most) most = (int64_t)n * s;
  }
  return (size_t)((most + g.n - 1) / g.n) * PART;
}

void prepare_attend() {
  (void)hipFuncSetAttribute((const void*)attend_kernel<0, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)attend_lds_bytes<0>());
  (void)hipFuncSetAttribute((const void*)attend_kernel<1, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)attend_lds_bytes<1>());
  (void)hipFuncSetAttribute((const void*)attend_kernel<0, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)attend_lds_bytes<0>());
  (void)hipFuncSetAttribute((const void*)attend_kernel<1, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)attend_lds_bytes<1>());
  (void)hipGetLastError();
}

namespace {

hipError_t launch_combine(const Geometry& g, const LayerTables& t, int32_t n_req, int parts, void* out, float* lse,
                          hipStream_t st) {
  if (g.flags & HS_FLAG_ATTN_OUT_F32)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(COMBINE_BLOCKS, n_req), dim3(COMBINE_THREADS), 0, st, t.part, parts,
                       g.heads, out, lse);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(COMBINE_BLOCKS, n_req), dim3(COMBINE_THREADS), 0, st, t.part,
                       parts, g.heads, out, lse);
  return hipGetLastError();
}

void launch_kernel(const Geometry& g, const AttendArgs& a, int32_t n_req, hipStream_t st) {
  dim3 grid(a.splits, n_req);
  const bool f32 = (g.flags & HS_FLAG_ATTN_OUT_F32) != 0;
  if (g.layout == HS_KV_BF16_576) {
    if (f32) hipLaunchKernelGGL((attend_kernel<0, true>), grid, dim3(NT), attend_lds_bytes<0>(), st, a);
    else hipLaunchKernelGGL((attend_kernel<0, false>), grid, dim3(NT), attend_lds_bytes<0>(), st, a);
  } else {
    if (f32) hipLaunchKernelGGL((attend_kernel<1, true>), grid, dim3(NT), attend_lds_bytes<1>(), st, a);
    else hipLaunchKernelGGL((attend_kernel<1, false>), grid, dim3(NT), attend_lds_bytes<1>(), st, a);
  }
}

}  // namespace

hipError_t launch_attend(const Geometry& g, const LayerTables& t, int32_t n_req, const void* q, const int32_t* slots,
                         const int32_t* sel, const int32_t* len, float scale, void* out, float* lse, hipStream_t st) {
  AttendArgs a;
  a.ml_slot = a.ml_tok = a.ml_cnt = nullptr;
  a.part_mode = ATT_ALL;
  a.part0 = 0;
  a.to_part = 0;
  a.merge_prev = 0;
  a.buf = t.buf;
  a.slots = slots;
  a.sel = sel;
  a.len = len;
  a.q = (const uint16_t*)q;
  a.out = out;
  a.lse = lse;
  a.part = t.part;
  a.stride = g.entry_bytes;
  a.rstride = g.req_stride;
  a.k = (int32_t)attend_tokens(g);
  a.B = g.B * g.P;
  a.lgP = g.lgP;
  a.heads = g.heads;
  a.splits = attend_splits(g, n_req);
  a.part_stride = a.splits;
  const int per = (a.k + a.splits - 1) / a.splits;
  a.chunk = (per + 15) / 16 * 16;
  a.scale_log2 = scale * kLog2e;
  if (a.splits > 1 && !a.part) return hipErrorInvalidValue;
  if (a.chunk > max_chunk(g)) return hipErrorInvalidValue;
  launch_kernel(g, a, n_req, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_combine(g, t, n_req, a.splits, out, lse, st);
}

// Split partials of hs_attend_noalloc: a file-scope device array, one copy on every GPU the
// library runs on (held until the process ends), so that the call allocates nothing.
static __device__ __align__(256) float scratch[(size_t)kNoallocPartials * PART];

namespace {
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each GPU, once resolved
}  // namespace

hipError_t prepare_attend_noalloc(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  // the array's host-side name is only a stand-in: its address on this device comes from here
  float* p = nullptr;
  hipError_t e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[device] = p;
  return hipSuccess;
}

int64_t attend_noalloc_partials(const Geometry& g, int32_t n_req, int32_t heads) {
  Geometry g2 = g;
  g2.heads = heads;
  const int splits = attend_splits(g2, n_req);
  return splits > 1 ? (int64_t)n_req * splits : 0;
}

hipError_t launch_attend_noalloc(const Geometry& g, const LayerTables& t, int device, int32_t n_req, int32_t heads,
                                 const void* q, const int32_t* slots, float scale, void* out, float* lse,
                                 hipStream_t st) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  float* p;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[device];
  }
  if (!p) return hipErrorNotInitialized;
  if (attend_noalloc_partials(g, n_req, heads) > kNoallocPartials) return hipErrorInvalidValue;
  Geometry g2 = g;
  g2.heads = heads;
  LayerTables t2 = t;
  t2.part = p;  // the handle's own partial space (if any) is left untouched
  return launch_attend(g2, t2, n_req, q, slots, nullptr, nullptr, scale, out, lse, st);
}

hipError_t launch_attend_part(const Geometry& g, const LayerTables& t, int32_t n_req, bool fetched, const void* q,
                              const int32_t* slots, const int32_t* sel, const int32_t* len, float scale, void* out,
                              float* lse, hipStream_t st) {
  AttendArgs a;
  a.buf = t.buf;
  a.slots = slots;
  a.sel = sel;
  a.len = len;
  a.q = (const uint16_t*)q;
  a.out = out;
  a.lse = lse;
  a.part = t.part;
  a.ml_slot = t.ml_slot;
  a.ml_tok = t.ml_tok;
  a.ml_cnt = t.ml_cnt;
  a.stride = g.entry_bytes;
  a.rstride = g.req_stride;
  a.k = (int32_t)attend_tokens(g);
  a.B = g.B * g.P;
  a.lgP = g.lgP;
  a.heads = g.heads;
  a.scale_log2 = scale * kLog2e;
  a.to_part = 1;
  const int sr = attend_splits(g, n_req), sf = fetched_splits(g);
  // a single fetched split merges the resident partials itself (no combine launch)
  a.merge_prev = fetched && sf == 1 && sr <= MAXPREV;
  a.part_stride = sr + sf;
  a.part_mode = fetched ? ATT_FETCHED : ATT_RESIDENT;
  a.splits = fetched ? sf : sr;
  a.part0 = fetched ? sr : 0;
  const int per = (a.k + a.splits - 1) / a.splits;
  a.chunk = (per + 15) / 16 * 16;
  if (!a.part || a.chunk > max_chunk(g)) return hipErrorInvalidValue;
  launch_kernel(g, a, n_req, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !fetched || a.merge_prev) return e;
  return launch_combine(g, t, n_req, a.part_stride, out, lse, st);
}

}  // namespace hs
