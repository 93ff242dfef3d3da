/*
 * canon_oracle.c — CPU oracle for canonical reduction and canonical inclusive
 * scan.
 *
 * TEST INFRASTRUCTURE.  This file is the slow, literal statement of what the
 * GPU library must compute, used to check it.  Only the tests, the package's
 * smoke check and the benchmark's CPU-baseline leg may load it.  The GPU path
 * neither includes, links nor calls anything here, and nothing here comes
 * from the GPU path.
 *
 * What it computes (sources are the canonical-reduce README, sections
 * "P4016R0 — Canonical Parallel Reduction" and "P4229R0 — Canonical Parallel
 * Scan"):
 *   - PW(s), the iterative pairwise tree over a sequence;
 *   - reduce(x, n, L, init) = init + PW(PW(lane 0), ..., PW(lane m-1)),
 *     lane j = (x_j, x_{j+L}, ...), m = min(n, L);  init alone when n = 0;
 *   - inclusive scans that return the value of a named expression on every
 *     prefix: pairwise, iterated_pairwise<L>, block_dyadic<B>;
 *   - scans with an initial value (inclusive, exclusive, include_initial):
 *     every output is init + the policy's expression over the prefix it
 *     observes, init alone for the empty prefix;
 *   - row-batched versions of all of these.
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (x86-64 SSE2
 * arithmetic: every float operation is one IEEE-754 operation in its own
 * type, round to nearest even, no flush of subnormals).
 *
 * Readings of points the pages leave open are listed in the design notes:
 * adjacent pairing with an odd carry for PW; lanes without an element take no
 * part; init on the left; block_dyadic's prefix split into whole blocks and
 * the open block.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* The operators (the expression is defined for any binary operator:        */
/* P4016R0 "Summary").  min and max are IEEE 754-2019 minimum / maximum: a   */
/* NaN operand gives NaN, and -0.0 is below +0.0; both are then associative  */
/* and commutative, so every parenthesisation gives the same value.          */
static double min_f64(double a, double b)
{
    if (isnan(a) || isnan(b)) return a + b;
    if (a < b) return a;
    if (b < a) return b;
    return signbit(a) ? a : b;
}
static double max_f64(double a, double b)
{
    if (isnan(a) || isnan(b)) return a + b;
    if (a > b) return a;
    if (b > a) return b;
    return signbit(a) ? b : a;
}
static float min_f32(float a, float b)
{
    if (isnan(a) || isnan(b)) return a + b;
    if (a < b) return a;
    if (b < a) return b;
    return signbit(a) ? a : b;
}
static float max_f32(float a, float b)
{
    if (isnan(a) || isnan(b)) return a + b;
    if (a > b) return a;
    if (b > a) return b;
    return signbit(a) ? b : a;
}

/* A skewed operator for tests of operand order and parenthesisation:
 * a (+) b = (a + b) + ((a * 0.25) * b) * b, neither commutative nor
 * associative; -0.0 is a two-sided identity for finite operands. */
static double skew_f64(double a, double b)
{
    const double s = a + b;
    const double q = (a * 0.25) * b;
    return s + q * b;
}
static float skew_f32(float a, float b)
{
    const float s = a + b;
    const float q = (a * 0.25f) * b;
    return s + q * b;
}

#define T double
#define SFX f64
#define OP(a, b) ((a) + (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP
#define SFX f64_mul
#define OP(a, b) ((a) * (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP
#define SFX f64_min
#define OP(a, b) min_f64((a), (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP
#define SFX f64_max
#define OP(a, b) max_f64((a), (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP

#define SFX f64_skew
#define OP(a, b) skew_f64((a), (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP
#undef T

#define T float
#define SFX f32
#define OP(a, b) ((a) + (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP
#define SFX f32_mul
#define OP(a, b) ((a) * (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP
#define SFX f32_min
#define OP(a, b) min_f32((a), (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP
#define SFX f32_max
#define OP(a, b) max_f32((a), (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP

#define SFX f32_skew
#define OP(a, b) skew_f32((a), (b))
#include "canon_oracle_body.h"
#undef SFX
#undef OP
#undef T

int oracle_abi_version(void) { return 1; }
