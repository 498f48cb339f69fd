/*
 * Seeded synthetic KV rows for the host pool (input generator only).
 *
 * This file holds no step of the cache method: it writes the bytes that a
 * model's attention layer would have offloaded to host memory.  Both the
 * device library's tests and the CPU oracle receive these bytes as input.
 *
 * Element randomness is a counter-based hash (SplitMix64's output mixer, Steele,
 * Lea & Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014)
 * keyed by (seed, request, layer, position, element group).  Each 64-bit hash
 * feeds four 16-bit indices into a 65536-entry table of standard-normal
 * quantiles supplied by the caller (synth/kv.py builds it), so every element
 * is an inverse-CDF N(0,1) draw.
 *
 * Layouts:
 *   0  bf16 entry, 576 bf16 values (512 latent + 64 rope)           = 1152 B
 *   1  fp8 entry: 512 E4M3FN latent codes, 4 fp32 block scales (one per 128
 *      latent values, scale = amax/448), 64 bf16 rope values         =  656 B
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t row_key(uint64_t seed, int64_t r, int64_t l, int64_t pos) {
  return mix64(mix64(mix64(mix64(seed) ^ (uint64_t)r) ^ (uint64_t)l) ^ (uint64_t)pos);
}

static inline unsigned idx16(uint64_t key, int e) {
  uint64_t u = mix64(key + (uint64_t)(e >> 2));
  return (unsigned)((u >> (16 * (e & 3))) & 0xFFFFu);
}

/* Round-to-nearest-even, saturating fp32 -> OCP E4M3FN byte (max finite 448). */
static uint8_t e4m3_encode(float v) {
  uint32_t bits;
  memcpy(&bits, &v, 4);
  uint8_t sign = (uint8_t)((bits >> 24) & 0x80u);
  if (isnan(v)) return (uint8_t)(sign | 0x7F);
  float a = fabsf(v);
  if (a >= 448.0f) return (uint8_t)(sign | 0x7E);
  if (a == 0.0f) return sign;
  int e2;
  frexpf(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
  int E = e2 - 1;          /* unbiased exponent */
  if (E < -6) E = -6;      /* subnormal binade: spacing 2^-9 */
  float q = rintf(ldexpf(a, 3 - E)); /* exact scaling by a power of two, then RNE */
  int code;
  if (E == -6 && q < 8.0f) {
    code = (int)q;
  } else {
    if (q >= 16.0f) { q = 8.0f; E += 1; }
    code = ((E + 7) << 3) | ((int)q - 8);
  }
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

static void make_row(uint64_t seed, int64_t r, int64_t l, int64_t pos, int layout,
                     const uint16_t* tb, const float* tf, uint8_t* dst) {
  uint64_t key = row_key(seed, r, l, pos);
  if (layout == 0) {
    uint16_t* o = (uint16_t*)dst;
    for (int e = 0; e < 576; ++e) o[e] = tb[idx16(key, e)];
    return;
  }
  float x[512];
  for (int e = 0; e < 512; ++e) x[e] = tf[idx16(key, e)];
  float scales[4];
  for (int b = 0; b < 4; ++b) {
    float amax = 0.0f;
    for (int e = 0; e < 128; ++e) {
      float a = fabsf(x[b * 128 + e]);
      if (a > amax) amax = a;
    }
    float s = amax / 448.0f;
    scales[b] = s;
    for (int e = 0; e < 128; ++e) dst[b * 128 + e] = e4m3_encode(x[b * 128 + e] / s);
  }
  memcpy(dst + 512, scales, 16);
  uint16_t* rope = (uint16_t*)(dst + 528);
  for (int e = 0; e < 64; ++e) rope[e] = tb[idx16(key, 512 + e)];
}

typedef struct {
  uint64_t seed;
  int64_t r, l;
  const int64_t* pos; /* NULL: contiguous from pos0 */
  int64_t pos0, begin, end;
  int layout;
  const uint16_t* tb;
  const float* tf;
  uint8_t* dst;
  int64_t stride;
  int64_t body;      /* split rows: bytes of each row written at dst (0: whole rows) */
  uint8_t* tail;     /* split rows: the rest of each row, at tail + i * tail_stride */
  int64_t tail_stride;
} job_t;

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  const int64_t E = j->layout == 0 ? 1152 : 656;
  uint8_t row[1152];
  for (int64_t i = j->begin; i < j->end; ++i) {
    int64_t pos = j->pos ? j->pos[i] : j->pos0 + i;
    if (!j->body) {
      make_row(j->seed, j->r, j->l, pos, j->layout, j->tb, j->tf, j->dst + i * j->stride);
      continue;
    }
    make_row(j->seed, j->r, j->l, pos, j->layout, j->tb, j->tf, row);
    memcpy(j->dst + i * j->stride, row, (size_t)j->body);
    memcpy(j->tail + i * j->tail_stride, row + j->body, (size_t)(E - j->body));
  }
  return NULL;
}

static void run_split(uint64_t seed, int64_t r, int64_t l, const int64_t* pos, int64_t pos0, int64_t count,
                      int layout, const uint16_t* tb, const float* tf, uint8_t* dst, int64_t stride,
                      int64_t body, uint8_t* tail, int64_t tail_stride, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (count < 4096) nthreads = 1;
  pthread_t th[256];
  job_t jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (job_t){seed, r, l, pos, pos0, count * t / nthreads, count * (t + 1) / nthreads,
                      layout, tb, tf, dst, stride, body, tail, tail_stride};
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run_job, &jobs[t]);
  run_job(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

static void run(uint64_t seed, int64_t r, int64_t l, const int64_t* pos, int64_t pos0, int64_t count,
                int layout, const uint16_t* tb, const float* tf, uint8_t* dst, int64_t stride, int nthreads) {
  run_split(seed, r, l, pos, pos0, count, layout, tb, tf, dst, stride, 0, NULL, 0, nthreads);
}

/* Rows for positions pos0 .. pos0+count-1 of (request r, layer l), written at dst + i*stride. */
void synth_fill_rows(uint64_t seed, int64_t r, int64_t l, int64_t pos0, int64_t count, int layout,
                     const uint16_t* tbl_bf16, const float* tbl_f32, uint8_t* dst, int64_t stride,
                     int nthreads) {
  run(seed, r, l, NULL, pos0, count, layout, tbl_bf16, tbl_f32, dst, stride, nthreads);
}

/* Rows for an explicit list of positions. */
void synth_rows_at(uint64_t seed, int64_t r, int64_t l, const int64_t* pos, int64_t count, int layout,
                   const uint16_t* tbl_bf16, const float* tbl_f32, uint8_t* dst, int64_t stride,
                   int nthreads) {
  run(seed, r, l, pos, 0, count, layout, tbl_bf16, tbl_f32, dst, stride, nthreads);
}

/* Exposed for the generator's own tests. */
uint8_t synth_e4m3_encode(float v) { return e4m3_encode(v); }
uint64_t synth_mix64(uint64_t z) { return mix64(z); }

/* The same rows split in two: the first `body` bytes of row i at dst + i*stride, the rest at
   tail + i*tail_stride (0 < body < entry bytes). */
void synth_fill_rows_split(uint64_t seed, int64_t r, int64_t l, int64_t pos0, int64_t count, int layout,
                           const uint16_t* tbl_bf16, const float* tbl_f32, uint8_t* dst, int64_t stride,
                           int64_t body, uint8_t* tail, int64_t tail_stride, int nthreads) {
  run_split(seed, r, l, NULL, pos0, count, layout, tbl_bf16, tbl_f32, dst, stride, body, tail, tail_stride,
            nthreads);
}
