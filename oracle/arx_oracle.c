/*
 * Oracle for the one-shot W-way bf16 reduction (test infrastructure only).
 *
 * This file is the plain, slow, obviously correct CPU statement of what the
 * reduction step computes. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product library never links or calls it,
 * and it shares no code, header or constant with the HIP path.
 *
 * What is computed (page "arx.cu", the reduction loop of arx_kernel and the
 * protocol comment at the top of the file):
 *   for every element i in [0, n):
 *     acc = -0.0f                       additive identity of IEEE binary32
 *     for src = 0 .. W-1:               ascending rank order, so every rank
 *       acc = acc + widen(x_src[i])     gets the same bits; binary32 adds,
 *                                        round to nearest even, subnormals kept
 *     out[i] = bf16 round-to-nearest-even of acc, any NaN -> 0x7FC0
 *   out[i] for i >= n is never written.
 *
 * Readings where the page is silent (listed with the others in the design
 * notes): the page starts the accumulator at +0.0f; -0.0f gives the same bits
 * except in columns where every addend is -0, and keeps x + (-0) = x exact for
 * every x. NaN results are canonicalised to the positive quiet NaN 0x7FC0.
 *
 * Build: gcc -O2 -fPIC -shared -fno-fast-math -ffp-contract=off. On x86-64 the
 * binary32 adds are SSE adds, IEEE round-to-nearest-even with subnormals kept
 * (MXCSR FTZ/DAZ are off by default and nothing here sets them).
 */
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* bf16 -> binary32 is exact: the bf16 bits are the upper half of the float. */
static float widen(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* binary32 -> bf16, round to nearest, ties to even (IEEE 754 roundTiesToEven
 * applied at the bf16 precision of 8 significand bits). The 16 discarded bits
 * are compared against one half of the last kept bit; on an exact tie the
 * result is the neighbour whose last kept bit is 0. Carrying out of the
 * significand moves to the next binade, and out of the largest binade to
 * +-Inf, which is what round-to-nearest does on overflow. NaN -> 0x7FC0. */
static uint16_t round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) return 0x7FC0u;
  uint32_t kept = u >> 16;        /* sign, exponent and 7 fraction bits */
  uint32_t dropped = u & 0xFFFFu; /* the discarded part, in units of 2^-16 ulp */
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
  return (uint16_t)kept;
}

/* Rounds n binary32 bit patterns to bf16 (the conversion alone, for pins). */
void oracle_round_bf16(const uint32_t* f32_bits, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    float f;
    memcpy(&f, &f32_bits[i], sizeof f);
    out[i] = round_bf16(f);
  }
}

/* Widens n bf16 patterns to binary32 bit patterns (for pins). */
void oracle_widen_bf16(const uint16_t* in, uint32_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    float f = widen(in[i]);
    memcpy(&out[i], &f, sizeof f);
  }
}

/* The reduction over elements [lo, hi). parts[src] points at partial src. */
static void reduce_range(const uint16_t* const* parts, int W, size_t lo, size_t hi, uint16_t* out) {
  for (size_t i = lo; i < hi; ++i) {
    float acc = -0.0f;
    for (int src = 0; src < W; ++src) acc = acc + widen(parts[src][i]);
    out[i] = round_bf16(acc);
  }
}

/* out[i] = rank-ordered W-way sum, i in [0, n). W >= 1; out may alias a part
 * only if it is the same array position by position (each element is read in
 * full before it is written). */
void oracle_reduce(const uint16_t* const* parts, int W, size_t n, uint16_t* out) {
  reduce_range(parts, W, 0, n, out);
}

typedef struct {
  const uint16_t* const* parts;
  int W;
  size_t lo, hi;
  uint16_t* out;
} range_job;

static void* run_range(void* p) {
  range_job* j = (range_job*)p;
  reduce_range(j->parts, j->W, j->lo, j->hi, j->out);
  return NULL;
}

/* Same result as oracle_reduce, split into `threads` contiguous index ranges.
 * Every element is computed by the same per-element formula, so the bits do
 * not depend on the thread count. Returns 0, or -1 if a thread failed to
 * start (the remaining ranges are then computed on the calling thread). */
int oracle_reduce_threads(const uint16_t* const* parts, int W, size_t n, uint16_t* out, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  pthread_t tid[256];
  range_job job[256];
  int started[256];
  int rc = 0;
  for (int t = 0; t < threads; ++t) {
    job[t].parts = parts;
    job[t].W = W;
    job[t].lo = n * (size_t)t / (size_t)threads;
    job[t].hi = n * (size_t)(t + 1) / (size_t)threads;
    job[t].out = out;
    started[t] = pthread_create(&tid[t], NULL, run_range, &job[t]) == 0;
    if (!started[t]) {
      rc = -1;
      run_range(&job[t]);
    }
  }
  for (int t = 0; t < threads; ++t)
    if (started[t]) pthread_join(tid[t], NULL);
  return rc;
}
