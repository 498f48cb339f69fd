/*
 * CPU oracle for the HiSparse hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header or table with the device
 * library and is deliberately plain: sorts via qsort, one request at a time,
 * fp64 arithmetic for attention.
 *
 * What it computes (HiSparse paper abstract; "HiSparse" note, sections 2 and 3):
 * each request keeps its whole KV history in host memory and a fixed number B of
 * device slots.  Per layer and step, a top-k selection S is resolved:
 *   hit detection  -- a token t is resident iff its page-table entry PT[t] >= 0;
 *   LRU replacement -- each missing token takes a slot that is not holding a hit,
 *                      least recently used first;
 *   page-table update and host-to-device fetch of the missing rows.
 * The tie rules the pages leave open are fixed as follows:
 *   - a slot's recency stamp is the step at which it was last selected (hits
 *     and fills alike); an empty slot has stamp -1;
 *   - candidate slots are ordered by (stamp, slot index) ascending;
 *   - misses are handled in ascending token order, the i-th miss taking the
 *     i-th candidate.
 * Sparse decode attention over the resolved slots is exact softmax attention
 * over the selected tokens (MLA form: K = all 576 values, V = the 512 latent
 * values), since only the placement of KV changes (paper abstract).
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_TOKEN -1
#define ORC_DUPLICATE -2
#define ORC_NO_ROOM -3
#define ORC_NOMEM -4
#define ORC_BAD_POLICY -5

/* Eviction policies (the note, section 3: the miss-count experiment compares buffer sizes
 * and eviction policies; LRU is steadier than a policy that does not exploit locality). */
#define ORC_LRU 0     /* candidates by (last-selection stamp, slot)                        */
#define ORC_FIFO 1    /* candidates by (fill stamp, slot): a hit does not refresh a slot    */
#define ORC_RANDOM 2  /* candidates in slot order, taken through a keyed random permutation */

/* ------------------------------------------------------------------ resolve */

/* The c-th output of SplitMix64 seeded with s (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): state s + (c + 1) * golden gamma, then the
 * generator's output mix. */
static uint64_t splitmix64_at(uint64_t s, uint64_t c) {
  uint64_t z = s + (c + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* The RANDOM policy's permutation of [0, N) for one (request-layer rl, step t): a balanced
 * 4-round Feistel network on 2h-bit values, 4^h the smallest power of four >= N, whose round
 * function i maps the right half R to the low h bits of splitmix64_at(key, i * 2^32 + R)
 * with key = splitmix64_at(seed, rl * 2^32 + t); values that land outside [0, N) are
 * encrypted again (cycle walking, Black and Rogaway, "Ciphers with arbitrary finite
 * domains", CT-RSA 2002) until they land inside. */
uint32_t orc_random_perm(uint64_t seed, int64_t rl, int64_t t, uint32_t N, uint32_t x) {
  const uint64_t key = splitmix64_at(seed, ((uint64_t)rl << 32) | (uint32_t)t);
  int h = 1;
  while (((uint64_t)1 << (2 * h)) < N) ++h;
  const uint32_t mask = (1u << h) - 1u;
  do {
    uint32_t L = x >> h, R = x & mask;
    for (uint32_t i = 0; i < 4; ++i) {
      const uint32_t F = (uint32_t)splitmix64_at(key, ((uint64_t)i << 32) | R) & mask;
      const uint32_t nl = R;
      R = L ^ F;
      L = nl;
    }
    x = (L << h) | R;
  } while (x >= N);
  return x;
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

typedef struct { int64_t stamp; int32_t slot; } cand_t;

static int cmp_cand(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->stamp != y->stamp) return (x->stamp > y->stamp) - (x->stamp < y->stamp);
  return (x->slot > y->slot) - (x->slot < y->slot);
}

/*
 * Resolve one selection S[k] (entries in [0, cap) or -1 for padding) against
 * the state of one (request, layer) under eviction policy `policy` (ORC_LRU
 * unless a policy study asks otherwise; rl = request * layers + layer and seed
 * key the RANDOM permutation):
 *   PT[cap]  token -> slot, -1 = not resident
 *   RM[B]    slot -> token, -1 = empty
 *   ST[B]    slot recency stamp, -1 = never used
 *   t        this resolve's step number (strictly increasing per state)
 * Writes slots[i] = slot now holding S[i] (-1 for padding) and *miss = number
 * of missing tokens.  When DEV and HOST are both non-NULL, the missing rows are
 * copied: DEV[slot] <- HOST[token], E bytes each.
 * Returns ORC_OK, or a negative code with the state untouched when S is invalid.
 */
int orc_resolve(int64_t B, int64_t cap, int64_t k, int32_t* PT, int32_t* RM, int64_t* ST, int64_t t,
                const int32_t* S, int32_t* slots, int64_t* miss, uint8_t* DEV, const uint8_t* HOST,
                int64_t E, int policy, uint64_t seed, int64_t rl) {
  if (policy != ORC_LRU && policy != ORC_FIFO && policy != ORC_RANDOM) return ORC_BAD_POLICY;
  int32_t* sorted = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
  int32_t* M = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
  unsigned char* is_hit = (unsigned char*)calloc((size_t)B, 1);
  cand_t* C = (cand_t*)malloc(sizeof(cand_t) * (size_t)B);
  if (!sorted || !M || !is_hit || !C) {
    free(sorted); free(M); free(is_hit); free(C);
    return ORC_NOMEM;
  }
  int rc = ORC_OK;

  /* 1. validate: every non-padding entry in range, no token twice */
  int64_t nv = 0;
  for (int64_t i = 0; i < k; ++i) {
    int32_t s = S[i];
    if (s == -1) continue;
    if (s < 0 || s >= cap) { rc = ORC_BAD_TOKEN; goto done; }
    sorted[nv++] = s;
  }
  qsort(sorted, (size_t)nv, sizeof(int32_t), cmp_i32);
  for (int64_t i = 1; i < nv; ++i)
    if (sorted[i] == sorted[i - 1]) { rc = ORC_DUPLICATE; goto done; }

  /* 2. classify: hits through the page table; misses collected in ascending token order */
  int64_t m = 0;
  for (int64_t i = 0; i < nv; ++i) {
    int32_t s = sorted[i];
    if (PT[s] >= 0) is_hit[PT[s]] = 1;
    else M[m++] = s;
  }

  /* 3. candidates: every slot not holding a hit, ordered by (stamp, slot) -- LRU and FIFO
   *    (their stamps differ) -- or, for RANDOM, left in slot order */
  int64_t nc = 0;
  for (int64_t j = 0; j < B; ++j)
    if (!is_hit[j]) { C[nc].stamp = ST[j]; C[nc].slot = (int32_t)j; ++nc; }
  if (nc < m) { rc = ORC_NO_ROOM; goto done; }
  if (policy != ORC_RANDOM) qsort(C, (size_t)nc, sizeof(cand_t), cmp_cand);

  /* 4. assign the i-th miss to the i-th candidate (RANDOM: candidate perm(i)): evict,
   *    update both maps, fetch; a filled slot is stamped with this step */
  for (int64_t i = 0; i < m; ++i) {
    int32_t j = policy == ORC_RANDOM ? C[orc_random_perm(seed, rl, t, (uint32_t)nc, (uint32_t)i)].slot : C[i].slot;
    ST[j] = t;
    if (RM[j] >= 0) PT[RM[j]] = -1;
    PT[M[i]] = j;
    RM[j] = M[i];
    if (DEV && HOST) memcpy(DEV + (size_t)j * (size_t)E, HOST + (size_t)M[i] * (size_t)E, (size_t)E);
  }

  /* 5. LRU and RANDOM: stamp every selected token's slot with this step (FIFO: fills only) */
  if (policy != ORC_FIFO)
    for (int64_t i = 0; i < nv; ++i) ST[PT[sorted[i]]] = t;

  /* 6. outputs in selection order */
  for (int64_t i = 0; i < k; ++i) slots[i] = (S[i] == -1) ? -1 : PT[S[i]];
  *miss = m;

done:
  free(sorted); free(M); free(is_hit); free(C);
  return rc;
}

/* Batch over n independent request states laid out back to back. */
typedef struct {
  int64_t B, cap, k, E;
  int policy; uint64_t seed; int64_t L, l;
  int32_t* PT; int32_t* RM; int64_t* ST; const int64_t* t;
  const int32_t* S; int32_t* slots; int64_t* miss;
  uint8_t* DEV; const uint8_t* HOST;
  int64_t r0, r1;
  int rc;
} rjob_t;

static void* rjob_run(void* p) {
  rjob_t* j = (rjob_t*)p;
  j->rc = ORC_OK;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    int rc = orc_resolve(j->B, j->cap, j->k, j->PT + r * j->cap, j->RM + r * j->B, j->ST + r * j->B, j->t[r],
                         j->S + r * j->k, j->slots + r * j->k, j->miss + r,
                         j->DEV ? j->DEV + r * j->B * j->E : NULL,
                         j->HOST ? j->HOST + r * j->cap * j->E : NULL, j->E, j->policy, j->seed,
                         r * j->L + j->l);
    if (rc != ORC_OK && j->rc == ORC_OK) j->rc = rc;
  }
  return NULL;
}

int orc_resolve_batch(int64_t n, int64_t B, int64_t cap, int64_t k, int32_t* PT, int32_t* RM, int64_t* ST,
                      const int64_t* t, const int32_t* S, int32_t* slots, int64_t* miss, uint8_t* DEV,
                      const uint8_t* HOST, int64_t E, int nthreads, int policy, uint64_t seed, int64_t L,
                      int64_t l) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  pthread_t th[256];
  rjob_t jobs[256];
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (rjob_t){B, cap, k, E, policy, seed, L, l, PT, RM, ST, t, S, slots, miss, DEV, HOST,
                       n * i / nthreads, n * (i + 1) / nthreads, ORC_OK};
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, rjob_run, &jobs[i]);
  rjob_run(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  for (int i = 0; i < nthreads; ++i)
    if (jobs[i].rc != ORC_OK) return jobs[i].rc;
  return ORC_OK;
}

/* ------------------------------------------------------------------- append */

/*
 * Write-through append of one newly generated token p (the note's introduction:
 * inactive KV is actively offloaded to host memory; paper abstract: each request's
 * full history lives in host memory).  Its row R (E bytes) is written to HOST[p]
 * and the token is made resident before the next resolve:
 *   - a resident token keeps its slot;
 *   - otherwise it takes the first slot in (stamp, slot) order over all slots --
 *     empty slots first -- evicting that slot's token from the page table;
 * the slot's stamp becomes t, the step number the next resolve will use (under
 * FIFO only when the token is placed), and with DEV non-NULL the slot's bytes
 * become R.  *slot_out gets the slot.  Returns ORC_OK, ORC_BAD_TOKEN (state
 * untouched) when p is not in [0, cap), or ORC_BAD_POLICY for RANDOM, whose
 * candidate order exists only within a resolve.
 */
int orc_append(int64_t B, int64_t cap, int32_t* PT, int32_t* RM, int64_t* ST, int64_t t, int32_t p,
               const uint8_t* R, uint8_t* DEV, uint8_t* HOST, int64_t E, int32_t* slot_out, int policy) {
  if (policy != ORC_LRU && policy != ORC_FIFO) return ORC_BAD_POLICY;
  if (p < 0 || p >= cap) return ORC_BAD_TOKEN;
  int32_t j = PT[p];
  if (j < 0) {
    j = 0;
    for (int64_t i = 1; i < B; ++i)
      if (ST[i] < ST[j]) j = (int32_t)i;   /* strict: the lowest slot wins ties */
    if (RM[j] >= 0) PT[RM[j]] = -1;
    PT[p] = j;
    RM[j] = p;
    ST[j] = t;
  } else if (policy == ORC_LRU) {
    ST[j] = t;  /* FIFO: rewriting a resident token is a use, which does not refresh its slot */
  }
  if (DEV) memcpy(DEV + (size_t)j * (size_t)E, R, (size_t)E);
  if (HOST) memcpy(HOST + (size_t)p * (size_t)E, R, (size_t)E);
  *slot_out = j;
  return ORC_OK;
}

/* ---------------------------------------------------------------- attention */

/* OCP FP8 E4M3FN: bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN. */
double orc_e4m3_decode(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

static double bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* K row (576 values) of one entry; layout 0 = 576 bf16, 1 = 512 e4m3 + 4 fp32 scales + 64 bf16. */
static void decode_row(const uint8_t* row, int layout, double* K) {
  if (layout == 0) {
    for (int d = 0; d < 576; ++d) {
      uint16_t b;
      memcpy(&b, row + 2 * d, 2);
      K[d] = bf16_decode(b);
    }
    return;
  }
  float sc[4];
  memcpy(sc, row + 512, 16);
  for (int d = 0; d < 512; ++d) K[d] = orc_e4m3_decode(row[d]) * (double)sc[d / 128];
  for (int d = 0; d < 64; ++d) {
    uint16_t b;
    memcpy(&b, row + 528 + 2 * d, 2);
    K[512 + d] = bf16_decode(b);
  }
}

/*
 * Sparse decode attention of H query heads over the k entries idx[i] >= 0 of
 * the row table base[.][stride] (idx[i] = -1 is skipped):
 *   s_i = scale * <q_h, K_i>,  p = softmax(s),  out_h = sum_i p_i V_i,  lse_h = log sum_i exp(s_i)
 * with K_i the 576 decoded values and V_i = K_i[0:512]; fp64 throughout, entries
 * in selection order.  With no valid entry, out = 0 and lse = -inf.
 */
int orc_attend(int64_t k, int layout, int64_t H, const uint16_t* q, const int32_t* idx, const uint8_t* base,
               int64_t stride, double scale, double* out, double* lse) {
  double* K = (double*)malloc(sizeof(double) * 576 * (size_t)(k > 0 ? k : 1));
  double* s = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  double* qd = (double*)malloc(sizeof(double) * 576);
  if (!K || !s || !qd) { free(K); free(s); free(qd); return ORC_NOMEM; }
  int64_t nv = 0;
  for (int64_t i = 0; i < k; ++i) {
    if (idx[i] < 0) continue;
    decode_row(base + (size_t)idx[i] * (size_t)stride, layout, K + 576 * nv);
    ++nv;
  }
  for (int64_t h = 0; h < H; ++h) {
    double* o = out + 512 * h;
    for (int d = 0; d < 512; ++d) o[d] = 0.0;
    if (nv == 0) { lse[h] = -INFINITY; continue; }
    for (int d = 0; d < 576; ++d) qd[d] = bf16_decode(q[576 * h + d]);
    double mx = -INFINITY;
    for (int64_t j = 0; j < nv; ++j) {
      double acc = 0.0;
      for (int d = 0; d < 576; ++d) acc += qd[d] * K[576 * j + d];
      s[j] = scale * acc;
      if (s[j] > mx) mx = s[j];
    }
    double den = 0.0;
    for (int64_t j = 0; j < nv; ++j) {
      double p = exp(s[j] - mx);
      den += p;
      for (int d = 0; d < 512; ++d) o[d] += p * K[576 * j + d];
    }
    for (int d = 0; d < 512; ++d) o[d] /= den;
    lse[h] = mx + log(den);
  }
  free(K); free(s); free(qd);
  return ORC_OK;
}

typedef struct {
  int64_t k, H, stride, base_step;
  int layout;
  const uint16_t* q; const int32_t* idx; const uint8_t* base;
  double scale; double* out; double* lse;
  int64_t r0, r1;
  int rc;
} ajob_t;

static void* ajob_run(void* p) {
  ajob_t* j = (ajob_t*)p;
  j->rc = ORC_OK;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    int rc = orc_attend(j->k, j->layout, j->H, j->q + r * j->H * 576, j->idx + r * j->k,
                        j->base + r * j->base_step, j->stride, j->scale, j->out + r * j->H * 512, j->lse + r * j->H);
    if (rc != ORC_OK) j->rc = rc;
  }
  return NULL;
}

/* n requests; request r's rows start at base + r*base_step. */
int orc_attend_batch(int64_t n, int64_t k, int layout, int64_t H, const uint16_t* q, const int32_t* idx,
                     const uint8_t* base, int64_t base_step, int64_t stride, double scale, double* out, double* lse,
                     int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  pthread_t th[256];
  ajob_t jobs[256];
  for (int i = 0; i < nthreads; ++i)
    jobs[i] = (ajob_t){k, H, stride, base_step, layout, q, idx, base, scale, out, lse,
                       n * i / nthreads, n * (i + 1) / nthreads, ORC_OK};
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, ajob_run, &jobs[i]);
  ajob_run(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  for (int i = 0; i < nthreads; ++i)
    if (jobs[i].rc != ORC_OK) return jobs[i].rc;
  return ORC_OK;
}
