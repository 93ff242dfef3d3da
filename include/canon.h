/*
 * canon.h — canonical (reproducible) parallel reduction and inclusive scan on
 * AMD MI355X (gfx950).  C ABI of libcanon.
 *
 * What is computed (canonical-reduce README: "P4016R0 — Canonical Parallel
 * Reduction" > "Key Design Points"; "P4229R0 — Canonical Parallel Scan" >
 * "Summary" and "Key Design Points"):
 *
 *   PW(s)            the iterative pairwise tree over a sequence s: pair
 *                    neighbours (s0+s1)(s2+s3)..., carry an odd trailing
 *                    element up unchanged, repeat until one value is left.
 *   CR_L(x[0..n))    element i goes to lane i mod L; each lane is reduced by
 *                    PW in index order; the lane values are combined by PW in
 *                    lane order.  Lanes that hold no element (n < L) take no
 *                    part.
 *   reduce           init + CR_L(x): init is combined once, on the left, after
 *                    the tree; the result is init itself when n == 0.
 *   scan<E>(x)[i]    the value of expression E over the prefix x[0..i]:
 *                      CANON_PAIRWISE           E = PW
 *                      CANON_ITERATED_PAIRWISE  E = CR_L, L = param
 *                      CANON_BLOCK_DYADIC       E(n) = PW(PW(block 0), ...,
 *                                               PW(block q-1)) + PW(tail),
 *                                               n = qB + t, 0 <= t < B,
 *                                               B = param (a power of two);
 *                                               an empty part is left out.
 *                    Hence scan<E>(x)[n-1] == reduce<E>(x[0..n)) bit for bit.
 *
 * The results are bit-identical for every input of a given (n, L) or
 * (policy, param), whatever the launch shape, GPU or run: the library
 * evaluates exactly the expression above (IEEE-754 binary64 / binary32
 * additions, round to nearest even, no contraction into FMA, subnormals
 * kept).  Only NaN payloads are not specified.
 *
 * Conventions for every entry point:
 *   - Array arguments (x, y, out, ws) are DEVICE pointers on the current HIP
 *     device.  `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Work is enqueued on `stream` and the call returns at once.
 *   - Elements are contiguous (the row functions take a row pitch `ld` in
 *     elements).  Any element alignment is accepted; 16-byte aligned data
 *     with a 16-byte aligned row pitch takes the fastest path.
 *   - The caller owns every buffer.  `ws` is scratch device memory of at
 *     least the size returned by the matching *_workspace_bytes function
 *     (which may be 0; ws may then be NULL).  It must be 256-byte aligned.
 *     Its contents on entry are ignored and on exit unspecified; calls that
 *     may run concurrently must not share a workspace.
 *   - Argument errors are detected before anything is enqueued and return
 *     CANON_EINVAL (bad pointer / size / parameter), CANON_EUNSUPPORTED
 *     (parameter beyond the supported range) or CANON_EWORKSPACE (workspace
 *     too small or misaligned).  A failed launch returns CANON_EHIP and
 *     keeps the HIP error code for canon_last_hip_error().  Device faults
 *     surface at the caller's next synchronisation.  The library never
 *     prints and holds no device memory between calls.
 */
#ifndef CANON_H
#define CANON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CANON_ABI_VERSION 4 /* 2: scans with an initial value; 3: operators;
                               4: tile geometry queries, schedule override */

/* Largest lane count L for reduce and iterated_pairwise, and largest block
 * size B for block_dyadic.  Larger values return CANON_EUNSUPPORTED. */
#define CANON_MAX_L 65536u
#define CANON_MAX_B 65536u
/* Largest lane count L of the iterated_pairwise scan. */
#define CANON_MAX_IP_L 65536u

typedef enum {
    CANON_OK = 0,
    CANON_EINVAL = 1,
    CANON_EUNSUPPORTED = 2,
    CANON_EWORKSPACE = 3,
    CANON_EHIP = 4
} canon_status_t;

typedef enum {
    CANON_PAIRWISE = 0,          /* param must be 0 or 1 */
    CANON_ITERATED_PAIRWISE = 1, /* param = L, 1 <= L <= CANON_MAX_IP_L */
    CANON_BLOCK_DYADIC = 2       /* param = B, power of two, 1 <= B <= CANON_MAX_B */
} canon_policy_t;

/* The binary operator the expression is evaluated with (P4016R0 "Summary":
 * the canonical expression is defined for any operator).  Absent values
 * (lanes without an element, padding) take the operator's exact identity:
 * -0.0, 1.0, +inf, -inf.  MIN and MAX are IEEE 754-2019 minimum and maximum:
 * NaN if either operand is NaN, -0.0 below +0.0.  Other operators
 * (non-commutative ones included) are compiled into the caller's own library
 * through canon_user_op.hpp. */
typedef enum {
    CANON_OP_ADD = 0,
    CANON_OP_MUL = 1,
    CANON_OP_MIN = 2,
    CANON_OP_MAX = 3
} canon_op_t;

/* Which prefix each output of a scan with an initial value observes. */
typedef enum {
    CANON_SCAN_INCLUSIVE = 0,      /* output i observes x[0..i]             */
    CANON_SCAN_EXCLUSIVE = 1,      /* output i observes x[0..i-1]           */
    CANON_SCAN_INCLUDE_INITIAL = 2 /* as exclusive, with n + 1 outputs      */
} canon_scan_kind_t;

/* ABI version of the loaded library (CANON_ABI_VERSION). */
int canon_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* canon_status_str(int status);

/* HIP error code of the last CANON_EHIP returned on this thread (0 if none). */
int canon_last_hip_error(void);

/* ---------------------------------------------------------------- reduce */
/* out[0] = init + CR_L(x[0..n)), or init when n == 0.
 *   x     device, n elements (may be NULL when n == 0)
 *   L     lane count, 1 <= L <= CANON_MAX_L
 *   out   device, one element; written on `stream`
 *   ws    device, canon_reduce_workspace_bytes(n, L, elem_size) bytes
 *         (none when that is 0), 256-byte aligned; its contents on entry do
 *         not matter (each call tags what it writes with an id of its own);
 *         calls that may overlap in time must not share a workspace.
 * One kernel: the last workgroup finishes (canon_workspace_error reports a
 * finish that gave up waiting for the others).
 * Source: P4016R0 "Key Design Points" (lanes i mod L, pairwise tree per lane,
 * lanes combined by the same rule, op(init, R)). */
size_t canon_reduce_workspace_bytes(size_t n, uint32_t L, size_t elem_size);
canon_status_t canon_reduce_f64(const double* x, size_t n, uint32_t L, double init, double* out,
                                void* ws, size_t ws_bytes, void* stream);
canon_status_t canon_reduce_f32(const float* x, size_t n, uint32_t L, float init, float* out,
                                void* ws, size_t ws_bytes, void* stream);

/* Row-batched reduce: row r is the sequence x[r*ldx + 0 .. r*ldx + cols);
 * out[r] = init + CR_L(row r) (init when cols == 0).
 *   x     device, rows x ldx elements (ldx >= cols)
 *   out   device, `rows` elements */
size_t canon_reduce_rows_workspace_bytes(size_t rows, size_t cols, uint32_t L, size_t elem_size);
canon_status_t canon_reduce_rows_f64(const double* x, size_t rows, size_t cols, size_t ldx,
                                     uint32_t L, double init, double* out, void* ws,
                                     size_t ws_bytes, void* stream);
canon_status_t canon_reduce_rows_f32(const float* x, size_t rows, size_t cols, size_t ldx,
                                     uint32_t L, float init, float* out, void* ws,
                                     size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ scan */
/* y[i] = value of the policy's expression over x[0..i], for i < n.
 * Source: P4229R0 "Summary" (policies) and "Key Design Points" (reduce
 * observes the root, scan observes the prefixes).
 *   x, y  device, n elements each; y == x (in place) is allowed, any other
 *         overlap is undefined. */
size_t canon_scan_workspace_bytes(size_t n, int policy, uint32_t param, size_t elem_size);
canon_status_t canon_scan_f64(const double* x, double* y, size_t n, int policy, uint32_t param,
                              void* ws, size_t ws_bytes, void* stream);
canon_status_t canon_scan_f32(const float* x, float* y, size_t n, int policy, uint32_t param,
                              void* ws, size_t ws_bytes, void* stream);

/* Row-batched scan: every row is an independent sequence of `cols` elements;
 * y[r*ldy + i] = scan<E>(row r)[i].  ldx, ldy >= cols; y == x with ldy == ldx
 * is allowed. */
size_t canon_scan_rows_workspace_bytes(size_t rows, size_t cols, int policy, uint32_t param,
                                       size_t elem_size);
canon_status_t canon_scan_rows_f64(const double* x, size_t ldx, double* y, size_t ldy,
                                   size_t rows, size_t cols, int policy, uint32_t param,
                                   void* ws, size_t ws_bytes, void* stream);
canon_status_t canon_scan_rows_f32(const float* x, size_t ldx, float* y, size_t ldy,
                                   size_t rows, size_t cols, int policy, uint32_t param,
                                   void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------- scan with an initial value */
/* Every output is init + E(prefix it observes), and init itself for the
 * empty prefix: init is combined once, on the left, after the policy's whole
 * expression, as the reduction places it (P4016R0 "Key Design Points", init
 * placement), so an inclusive output equals the reduction with init of the
 * same prefix.  With S_i = scan<E>(x)[i] (and S_{-1} the empty prefix):
 *   CANON_SCAN_INCLUSIVE        y[i] = init + S_i,      i < n   (n outputs)
 *   CANON_SCAN_EXCLUSIVE        y[i] = init + S_{i-1},  i < n   (n outputs)
 *   CANON_SCAN_INCLUDE_INITIAL  y[i] = init + S_{i-1},  i <= n  (n + 1)
 * so y[0] = init for the last two.  The inclusive/exclusive duality and
 * include_initial are those of the array API's cumulative_sum (gt4py
 * scan-redesign research page, B.2 "Array API standard / NumPy").
 *   x     device, n elements (may be NULL when n == 0)
 *   y     device, n outputs (n + 1 for include_initial); y == x (in place)
 *         is allowed, any other overlap is undefined
 *   kind  a canon_scan_kind_t; anything else returns CANON_EINVAL
 * The workspace is the plain scan's (canon_scan_workspace_bytes).  With init
 * = -0.0 and CANON_SCAN_INCLUSIVE the result is bit-identical to
 * canon_scan_*: -0.0 is the exact identity of IEEE addition. */
canon_status_t canon_scan_with_init_f64(const double* x, double* y, size_t n, int policy,
                                       uint32_t param, int kind, double init, void* ws,
                                       size_t ws_bytes, void* stream);
canon_status_t canon_scan_with_init_f32(const float* x, float* y, size_t n, int policy,
                                       uint32_t param, int kind, float init, void* ws,
                                       size_t ws_bytes, void* stream);

/* Row-batched scan with an initial value: row r of y (pitch ldy) is
 * canon_scan_with_init of row r of x.  ldx >= cols; ldy >= cols, or cols + 1
 * for include_initial.  y == x with ldy == ldx is allowed.  Workspace:
 * canon_scan_rows_workspace_bytes. */
canon_status_t canon_scan_rows_with_init_f64(const double* x, size_t ldx, double* y, size_t ldy,
                                            size_t rows, size_t cols, int policy, uint32_t param,
                                            int kind, double init, void* ws, size_t ws_bytes,
                                            void* stream);
canon_status_t canon_scan_rows_with_init_f32(const float* x, size_t ldx, float* y, size_t ldy,
                                            size_t rows, size_t cols, int policy, uint32_t param,
                                            int kind, float init, void* ws, size_t ws_bytes,
                                            void* stream);

/* ------------------------------------------------------------- operators */
/* The same expressions with `op` (a canon_op_t; anything else returns
 * CANON_EINVAL) in place of every addition, op(init, R) in place of
 * init + R, and the operator's identity as the absent value.  Arguments,
 * layouts, workspaces (the *_workspace_bytes functions above, which do not
 * depend on the operator) and errors are those of the functions above;
 * canon_scan_op_* and canon_scan_rows_op_* take kind and init as the scans
 * with an initial value do (kind CANON_SCAN_INCLUSIVE with init = the
 * identity is the plain scan).  CANON_OP_ADD gives exactly the results of
 * the functions above.  The other operators run the reduce kernels of
 * addition (the register streaming kernel for a power-of-two L and 16-byte
 * aligned input, the general streaming kernel otherwise) and the scan
 * kernels with an output stage; CANON_OP_MIN and CANON_OP_MAX, associative
 * and commutative, run one scan kernel whatever the policy. */
canon_status_t canon_reduce_op_f64(const double* x, size_t n, uint32_t L, int op, double init,
                                   double* out, void* ws, size_t ws_bytes, void* stream);
canon_status_t canon_reduce_op_f32(const float* x, size_t n, uint32_t L, int op, float init,
                                   float* out, void* ws, size_t ws_bytes, void* stream);
canon_status_t canon_reduce_rows_op_f64(const double* x, size_t rows, size_t cols, size_t ldx,
                                        uint32_t L, int op, double init, double* out, void* ws,
                                        size_t ws_bytes, void* stream);
canon_status_t canon_reduce_rows_op_f32(const float* x, size_t rows, size_t cols, size_t ldx,
                                        uint32_t L, int op, float init, float* out, void* ws,
                                        size_t ws_bytes, void* stream);
canon_status_t canon_scan_op_f64(const double* x, double* y, size_t n, int policy, uint32_t param,
                                 int op, int kind, double init, void* ws, size_t ws_bytes,
                                 void* stream);
canon_status_t canon_scan_op_f32(const float* x, float* y, size_t n, int policy, uint32_t param,
                                 int op, int kind, float init, void* ws, size_t ws_bytes,
                                 void* stream);
canon_status_t canon_scan_rows_op_f64(const double* x, size_t ldx, double* y, size_t ldy,
                                      size_t rows, size_t cols, int policy, uint32_t param,
                                      int op, int kind, double init, void* ws, size_t ws_bytes,
                                      void* stream);
canon_status_t canon_scan_rows_op_f32(const float* x, size_t ldx, float* y, size_t ldy,
                                      size_t rows, size_t cols, int policy, uint32_t param,
                                      int op, int kind, float init, void* ws, size_t ws_bytes,
                                      void* stream);

/* -------------------------------------------------------------- checking */
/* Every scan workspace, and every reduce workspace, begins with a 32-bit
 * error word, which every scan or reduce call given a workspace of nonzero
 * size sets.  The single-pass scans wait on values published by earlier
 * workgroups, and the reduce's finishing workgroup on the other workgroups'
 * partial values, with a bounded spin; if a bound is ever exceeded the
 * kernel stops waiting, records a nonzero error word and finishes (the
 * output is then invalid).  This call copies the word to *err_out and
 * synchronises `stream`.  0 means no error. */
canon_status_t canon_workspace_error(const void* ws, uint32_t* err_out, void* stream);

/* -------------------------------------------------------------- geometry */
/* Elements per tile, the unit one workgroup step of a scan covers: for the
 * 1-D scans (canon_scan_*) and for the row scans (canon_scan_rows_*, tiles
 * within a row), given the policy, its param and elem_size (4 or 8), for
 * 16-byte aligned data.  Results never depend on it; it tells a caller (a
 * test) where sizes cross tile and tile-group edges.  0 for an invalid
 * policy, param or element size. */
size_t canon_scan_tile_elems(int policy, uint32_t param, size_t elem_size);
size_t canon_scan_rows_tile_elems(int policy, uint32_t param, size_t elem_size);

/* ------------------------------------------------------- no allocation */
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the plain
 * scan canon_scan_f64 with its workspace in a static device array of the
 * library, CANON_NOALLOC_SCRATCH_BYTES (8 MiB) per device, held from the
 * first call on a device until the process ends.  Nothing is allocated by
 * the call.  Same arguments (minus ws / ws_bytes), results (bit for bit) and
 * errors as canon_scan_f64, plus CANON_EUNSUPPORTED when the scan needs more
 * than the array, i.e. canon_scan_workspace_bytes(n, policy, param, 8) >
 * CANON_NOALLOC_SCRATCH_BYTES (pairwise and block_dyadic up to about 8.3e9
 * elements, iterated_pairwise<128> up to about 3.3e7, iterated_pairwise<16>
 * up to about 2.6e8).  Every call on one
 * device shares the array, which keeps the last call's contents: calls that
 * may overlap on one device (other streams, other host threads) race, and
 * the error word of canon_workspace_error is not available. */
#define CANON_NOALLOC_SCRATCH_BYTES (8u << 20)
canon_status_t canon_scan_noalloc_f64(const double* x, double* y, size_t n, int policy,
                                      uint32_t param, void* stream);

/* ------------------------------------------------------ schedule override */
/* Process-wide override of how work is spread over workgroups, for tests
 * that show the results do not depend on the schedule (P4016R0 "Summary":
 * an implementation may schedule freely as long as the value is the
 * canonical one).  value 0 restores the default.
 *   CANON_SCHED_GRID             at most `value` workgroups for every
 *                                persistent (ticket-driven) or grid-stride
 *                                kernel: single-pass scans, the pipelined
 *                                iterated_pairwise pass, the three-kernel
 *                                iterated_pairwise path, row reduces and row
 *                                scans (kernels with one workgroup per tile
 *                                keep their grid)
 *   CANON_SCHED_REDUCE_PARTIALS  workgroups (row ranges, hence partials) the
 *                                streaming reduce aims for; the reduce
 *                                workspace size follows it
 *   CANON_SCHED_SPIN_LIMIT       polls of every bounded wait (single-pass
 *                                scans, the reduce's finish) before it gives
 *                                up and records the error word (the scans'
 *                                waits check it every 64 polls); for tests of
 *                                that path only: a small value makes waits
 *                                give up, and the output is then invalid
 *                                (default 2^20)
 * Returns CANON_EINVAL for an unknown knob.  Not synchronised with calls in
 * flight on other host threads: set it between calls. */
#define CANON_SCHED_GRID 0
#define CANON_SCHED_REDUCE_PARTIALS 1
#define CANON_SCHED_SPIN_LIMIT 2
canon_status_t canon_set_schedule(int knob, uint64_t value);
uint64_t canon_get_schedule(int knob);

#ifdef __cplusplus
}
#endif

#endif /* CANON_H */
