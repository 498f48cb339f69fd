// Sparse MLA decode attention over resolved slots.
//
// What is computed (HiSparse paper abstract: each decode step reads only the selected
// KV entries; only KV placement changes, so the result is exact attention over the
// selected tokens): for every request r and query head h,
//   s_j = scale * <q_h, K_j>,  out_h = sum_j softmax(s)_j V_j,  lse_h = log sum_j exp(s_j),
// over the valid slots j of the request (slot -1 skipped), with K_j the 576 decoded values
// of the slot's entry (512 latent + 64 rope) and V_j its first 512 values (MLA form).
// FP8 entries decode as e4m3 code * fp32 block scale (one scale per 128 latent values).
//
// Design for gfx950 (HBM-bound: ~1.3 MB of rows per request at k = 2048 against 71 MFLOP):
//  * grid (splits, requests); a workgroup of 4 wave64s takes a contiguous chunk of the
//    selection; each wave walks 16-token subtiles of it with its own online softmax and
//    its own 16 x 512 fp32 output accumulator;
//  * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_bf16: a lane loads
//    16-byte pieces of one token's row straight into the A operand (no LDS for K); Q sits in
//    LDS and is read as the B operand.  The reduction index of the MFMA is mapped onto the
//    576 values so that each lane's pieces of a 128-value block are contiguous in memory;
//  * in S^T's accumulator layout a lane holds one head and four consecutive tokens, which is
//    exactly the A-operand layout of v_mfma_f32_16x16x16bf16_1k, so P needs no shuffle;
//  * V must arrive with four consecutive tokens per lane and a fixed column, the transpose of
//    how rows are read.  One MFMA against a 0/1 selector matrix (exact: one product per
//    output) turns the K registers into that layout, so V is never re-read or staged;
//  * FP8 scales: per 128-value block, partial scores are scaled per token before they are
//    summed; for P V the token's block scale is folded into P;
//  * the four waves merge through LDS; with splits > 1 every workgroup writes an
//    unnormalised partial (max, sum, 16 x 512 values) and the last one to arrive (atomic
//    counter, reset by that workgroup) combines them in split order, so results do not
//    depend on arrival order.

#include <math.h>

#include "hs_internal.h"

namespace hs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVES = 4;
constexpr int NT = WAVES * 64;
constexpr int HMAX = 16;        // heads per workgroup (one MFMA tile)
constexpr int DQK = 576;        // q.K length
constexpr int DV = 512;         // value length
constexpr int QS = DQK + 8;     // padded LDS row of Q (bf16 elements)
constexpr int PART = 2 * HMAX + HMAX * DV;  // floats of one split partial
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttendArgs {
  const uint8_t* buf;     // layer's slot rows [n][B][stride]
  const int32_t* slots;   // [n_req][k]
  const uint16_t* q;      // [n_req][heads][576] bf16
  uint16_t* out;          // [n_req][heads][512] bf16
  float* lse;             // [n_req][heads] or null
  float* part;            // [n][splits][PART]
  uint32_t* cnt;          // [n]
  int64_t stride;
  int32_t k, B, heads, chunk, splits;
  float scale_log2;       // softmax scale * log2(e)
};

__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ s16x4 pack4(float a, float b, float c, float d) {
  s16x4 v;
  v[0] = (short)bf16_rne(a);
  v[1] = (short)bf16_rne(b);
  v[2] = (short)bf16_rne(c);
  v[3] = (short)bf16_rne(d);
  return v;
}

// Two E4M3FN codes (low 16 bits) -> two bf16 (exact).  The 7 magnitude bits shifted to
// bit 20 form an fp32 whose exponent field is the code's exponent: scaling by 2^120
// re-biases normals (bias 7 -> 127) and turns subnormal codes, which land in fp32's
// subnormal range, into m * 2^-9.  The result has at most 4 significant bits, so its
// top 16 bits are the bf16 value.
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t two) {
  const uint32_t c0 = two & 0xFFu, c1 = (two >> 8) & 0xFFu;
  const float f0 = __uint_as_float((c0 & 0x7Fu) << 20) * 0x1p120f;
  const float f1 = __uint_as_float((c1 & 0x7Fu) << 20) * 0x1p120f;
  const uint32_t b0 = (__float_as_uint(f0) >> 16) | ((c0 & 0x80u) << 8);
  const uint32_t b1 = (__float_as_uint(f1) >> 16) | ((c1 & 0x80u) << 8);
  return b0 | (b1 << 16);
}

__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 v;
  v[0] = e4m3x2_to_bf16x2(lo);
  v[1] = e4m3x2_to_bf16x2(lo >> 16);
  v[2] = e4m3x2_to_bf16x2(hi);
  v[3] = e4m3x2_to_bf16x2(hi >> 16);
  return v;
}

// Element offset in a 576-value row of reduction block kb for lane group g:
// latent blocks kb = 4b + i cover d = 128b + 32g + 8i + [0, 8); rope kb = 16 + i covers
// d = 512 + 16g + 8i + [0, 8).
__device__ __forceinline__ int kb_offset(int kb, int g) {
  return kb < 16 ? 128 * (kb >> 2) + 32 * g + 8 * (kb & 3) : 512 + 16 * g + 8 * (kb - 16);
}

// Output column held by accumulator tile tau = 2 kb + sigma, column n of the tile.
__device__ __forceinline__ int out_col(int tau, int n) {
  const int kb = tau >> 1, sigma = tau & 1;
  const int kappa = 16 * sigma + n;
  return 128 * (kb >> 2) + 32 * (kappa >> 3) + 8 * (kb & 3) + (kappa & 7);
}

template <int LAYOUT>
__global__ __launch_bounds__(NT) void attend_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[HMAX * QS];
  __shared__ float wm[WAVES][HMAX];
  __shared__ float wl[WAVES][HMAX];
  __shared__ float o_acc[HMAX * DV];
  __shared__ int last_flag;

  const int s = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int heads = a.heads;

  // ---- Q to LDS (rows >= heads are zero)
  for (int c = tid; c < HMAX * (DQK / 8); c += NT) {
    const int h = c / (DQK / 8), part = c - h * (DQK / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (h < heads) v = load16(a.q + ((int64_t)r * heads + h) * DQK + part * 8);
    *(u32x4*)(q_lds + h * QS + part * 8) = v;
  }
  __syncthreads();

  // selector B operands: lane (g, n=c16) holds reduction rows 8g..8g+7 of column n;
  // sigma = 0 picks reduction row n, sigma = 1 picks row 16 + n.
  bf16x8 sel0, sel1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int kappa = 8 * g + e;
    sel0[e] = (kappa == c16) ? (__bf16)1.0f : (__bf16)0.0f;
    sel1[e] = (kappa == 16 + c16) ? (__bf16)1.0f : (__bf16)0.0f;
  }

  f32x4 O[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) O[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int tok0 = s * a.chunk;
  const int tok1 = min(a.k, tok0 + a.chunk);
  const int nsub = tok1 > tok0 ? (tok1 - tok0 + 15) / 16 : 0;
  const int32_t* slots = a.slots + (int64_t)r * a.k;
  const uint8_t* rbase = a.buf + (int64_t)r * a.B * a.stride;

  for (int sub = w; sub < nsub; sub += WAVES) {
    const int t = tok0 + sub * 16 + c16;
    const int32_t slot = (t < tok1) ? slots[t] : -1;
    const bool valid = slot >= 0 && slot < a.B;
    const uint8_t* row = rbase + (int64_t)(valid ? slot : 0) * a.stride;

    u32x4 kreg[18];
    float sc[4] = {1.f, 1.f, 1.f, 1.f};
    if (LAYOUT == 0) {
#pragma unroll
      for (int kb = 0; kb < 18; ++kb)
        kreg[kb] = valid ? load16(row + 2 * kb_offset(kb, g)) : (u32x4){0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        u32x4 lo = valid ? load16(row + 128 * b + 32 * g) : (u32x4){0u, 0u, 0u, 0u};
        u32x4 hi = valid ? load16(row + 128 * b + 32 * g + 16) : (u32x4){0u, 0u, 0u, 0u};
        kreg[4 * b + 0] = e4m3x8_to_bf16x8(lo[0], lo[1]);
        kreg[4 * b + 1] = e4m3x8_to_bf16x8(lo[2], lo[3]);
        kreg[4 * b + 2] = e4m3x8_to_bf16x8(hi[0], hi[1]);
        kreg[4 * b + 3] = e4m3x8_to_bf16x8(hi[2], hi[3]);
      }
      kreg[16] = valid ? load16(row + 528 + 32 * g) : (u32x4){0u, 0u, 0u, 0u};
      kreg[17] = valid ? load16(row + 528 + 32 * g + 16) : (u32x4){0u, 0u, 0u, 0u};
      if (valid) {
        const u32x4 sv = load16(row + 512);
#pragma unroll
        for (int b = 0; b < 4; ++b) sc[b] = __uint_as_float(sv[b]);
      }
    }

    // ---- S^T[tok][h] = K Q^T
    float sv4[4];
    const uint16_t* qrow = q_lds + c16 * QS;
    if (LAYOUT == 0) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 18; ++kb) {
        const bf16x8 qb = *(const bf16x8*)(qrow + kb_offset(kb, g));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[kb]), qb, acc, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sv4[j] = acc[j];
    } else {
      f32x4 accb[4], accr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        accb[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kb = 4 * b + i;
          const bf16x8 qb = *(const bf16x8*)(qrow + kb_offset(kb, g));
          accb[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[kb]), qb, accb[b], 0, 0, 0);
        }
      }
#pragma unroll
      for (int kb = 16; kb < 18; ++kb) {
        const bf16x8 qb = *(const bf16x8*)(qrow + kb_offset(kb, g));
        accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[kb]), qb, accr, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = accr[j];
#pragma unroll
        for (int b = 0; b < 4; ++b) v += __shfl(sc[b], 4 * g + j) * accb[b][j];
        sv4[j] = v;
      }
    }

    // ---- online softmax for head c16 over tokens 4g + j of this subtile
    float s2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vj = __shfl((int)valid, 4 * g + j);
      s2[j] = vj ? sv4[j] * a.scale_log2 : -INFINITY;
    }
    float mx = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.f, p[4] = {0.f, 0.f, 0.f, 0.f};
    if (m_new != -INFINITY) {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = exp2f(s2[j] - m_new);
    }
    float rs = (p[0] + p[1]) + (p[2] + p[3]);
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;

    // rescale the accumulator rows (heads 4g + j)
    float aj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) aj[j] = __shfl(alpha, 4 * g + j);
#pragma unroll
    for (int tau = 0; tau < 32; ++tau)
#pragma unroll
      for (int j = 0; j < 4; ++j) O[tau][j] *= aj[j];

    // ---- O += P V
    s16x4 pa[4];
    if (LAYOUT == 0) {
      pa[0] = pack4(p[0], p[1], p[2], p[3]);
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float t4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) t4[j] = p[j] * __shfl(sc[b], 4 * g + j);
        pa[b] = pack4(t4[0], t4[1], t4[2], t4[3]);
      }
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, kreg[kb]);
      const s16x4 P = (LAYOUT == 0) ? pa[0] : pa[kb >> 2];
      const f32x4 t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, sel0, zero, 0, 0, 0);
      const f32x4 t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, sel1, zero, 0, 0, 0);
      O[2 * kb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(P, pack4(t0[0], t0[1], t0[2], t0[3]), O[2 * kb], 0, 0, 0);
      O[2 * kb + 1] =
          __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(P, pack4(t1[0], t1[1], t1[2], t1[3]), O[2 * kb + 1], 0, 0, 0);
    }
  }

  // ---- merge the four waves (fixed order)
  if (g == 0) {
    wm[w][c16] = m_run;
    wl[w][c16] = l_run;
  }
  __syncthreads();
  float f[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * g + j;
    float M = wm[0][h];
#pragma unroll
    for (int v = 1; v < WAVES; ++v) M = fmaxf(M, wm[v][h]);
    f[j] = (M == -INFINITY) ? 0.f : exp2f(wm[w][h] - M);
  }
  for (int v = 0; v < WAVES; ++v) {
    if (w == v) {
#pragma unroll
      for (int tau = 0; tau < 32; ++tau) {
        const int col = out_col(tau, c16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int idx = (4 * g + j) * DV + col;
          const float val = O[tau][j] * f[j];
          o_acc[idx] = (v == 0) ? val : o_acc[idx] + val;
        }
      }
    }
    __syncthreads();
  }

  // per-head max and sum of the workgroup
  float Mh[1], Lh[1];
  (void)Mh;
  (void)Lh;
  const int splits = a.splits;
  if (splits == 1) {
    for (int idx = tid; idx < heads * DV; idx += NT) {
      const int h = idx / DV;
      float M = wm[0][h];
      for (int v = 1; v < WAVES; ++v) M = fmaxf(M, wm[v][h]);
      float L = 0.f;
      if (M != -INFINITY)
        for (int v = 0; v < WAVES; ++v) L += exp2f(wm[v][h] - M) * wl[v][h];
      const float val = L > 0.f ? o_acc[idx] / L : 0.f;
      a.out[(int64_t)r * heads * DV + idx] = (uint16_t)bf16_rne(val);
      if ((idx % DV) == 0 && a.lse) a.lse[(int64_t)r * heads + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
    return;
  }

  float* mypart = a.part + ((int64_t)r * splits + s) * PART;
  if (tid < HMAX) {
    const int h = tid;
    float M = wm[0][h];
    for (int v = 1; v < WAVES; ++v) M = fmaxf(M, wm[v][h]);
    float L = 0.f;
    if (M != -INFINITY)
      for (int v = 0; v < WAVES; ++v) L += exp2f(wm[v][h] - M) * wl[v][h];
    mypart[h] = M;
    mypart[HMAX + h] = L;
  }
  for (int idx = tid; idx < HMAX * DV; idx += NT) mypart[2 * HMAX + idx] = o_acc[idx];
  __threadfence();
  __syncthreads();
  if (tid == 0) last_flag = (atomicAdd(&a.cnt[r], 1u) == (uint32_t)(splits - 1)) ? 1 : 0;
  __syncthreads();
  if (!last_flag) return;
  __threadfence();

  const float* prow = a.part + (int64_t)r * splits * PART;
  for (int idx = tid; idx < heads * DV; idx += NT) {
    const int h = idx / DV;
    float M = -INFINITY;
    for (int v = 0; v < splits; ++v) M = fmaxf(M, prow[v * PART + h]);
    float L = 0.f, acc = 0.f;
    if (M != -INFINITY) {
      for (int v = 0; v < splits; ++v) {
        const float fv = exp2f(prow[v * PART + h] - M);
        L += fv * prow[v * PART + HMAX + h];
        acc += fv * prow[v * PART + 2 * HMAX + idx];
      }
    }
    a.out[(int64_t)r * heads * DV + idx] = (uint16_t)bf16_rne(L > 0.f ? acc / L : 0.f);
    if ((idx % DV) == 0 && a.lse) a.lse[(int64_t)r * heads + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  if (tid == 0) a.cnt[r] = 0u;
}

}  // namespace

int attend_splits(const Geometry& g) {
  // enough workgroups for two per compute unit at full batch, at least 64 tokens each
  const int by_batch = (2 * 256 + g.n - 1) / g.n;
  const int by_len = (g.k + 63) / 64;
  int s = by_batch < by_len ? by_batch : by_len;
  if (s > 16) s = 16;
  return s < 1 ? 1 : s;
}

size_t attend_partial_floats(const Geometry& g) {
  const int s = attend_splits(g);
  return s > 1 ? (size_t)s * PART : 0;
}

hipError_t launch_attend(const Geometry& g, const LayerTables& t, int32_t n_req, const void* q, const int32_t* slots,
                         float scale, void* out, float* lse, hipStream_t st) {
  AttendArgs a;
  a.buf = t.buf;
  a.slots = slots;
  a.q = (const uint16_t*)q;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.part = t.part;
  a.cnt = t.cnt;
  a.stride = g.slot_stride;
  a.k = g.k;
  a.B = g.B;
  a.heads = g.heads;
  a.splits = attend_splits(g);
  const int per = (g.k + a.splits - 1) / a.splits;
  a.chunk = (per + 15) / 16 * 16;
  a.scale_log2 = scale * kLog2e;
  if (a.splits > 1 && !a.part) return hipErrorInvalidValue;
  dim3 grid(a.splits, n_req);
  if (g.layout == HS_KV_BF16_576)
    hipLaunchKernelGGL(attend_kernel<0>, grid, dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL(attend_kernel<1>, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs
