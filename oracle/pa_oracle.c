/*
 * pa_oracle.c -- CPU oracle for decode-time paged attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.  Built with
 * gcc -O2 -ffp-contract=off (no fast-math, no fused multiply-add), so each
 * operation rounds exactly once, in the precision of its instantiation.
 *
 * ORACLE_MUTATION (default 0) plants one known mistake for the tests that
 * prove the pins can fail; the shipped build has none:
 *   1 window one key short          6 merge weight without l_j
 *   2 interleaved GQA head map      7 softmax scale dropped
 *   3 slot mirrored inside a page   8 MLA value row shifted by d_rope
 *   4 W_UK read as [j][d]           9 MLA rope term dropped
 *   5 lse without the max          10 split partitions counted from key 0
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "pa_oracle.h"

#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif

/* bf16 -> float is exact: the 16 stored bits are the top half of an IEEE
 * binary32 pattern. */
static float bf16_to_float(uint16_t u) {
  uint32_t w = (uint32_t)u << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return f;
}

#define REAL double
#define EXPR exp
#define LOGR log
#define NAME(x) x##_f64
#define BF(x) ((REAL)bf16_to_float(x))
#include "pa_oracle_body.h"
#undef REAL
#undef EXPR
#undef LOGR
#undef NAME
#undef BF

#define REAL float
#define EXPR expf
#define LOGR logf
#define NAME(x) x##_f32
#define BF(x) ((REAL)bf16_to_float(x))
#include "pa_oracle_body.h"
#undef REAL
#undef EXPR
#undef LOGR
#undef NAME
#undef BF

void oracle_set_num_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t oracle_max_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

int32_t oracle_mutation(void) { return ORACLE_MUTATION; }
