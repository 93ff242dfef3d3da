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
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define T double
#define SFX f64
#include "canon_oracle_body.h"
#undef T
#undef SFX

#define T float
#define SFX f32
#include "canon_oracle_body.h"
#undef T
#undef SFX

int oracle_abi_version(void) { return 1; }
