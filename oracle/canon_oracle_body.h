/*
 * Body of the CPU oracle, instantiated once per floating-point type and
 * operator by canon_oracle.c (T = double / float; SFX = f64 / f32 for +,
 * f64_mul, f64_min, ... for the others; OP(a, b) the operator).
 *
 * TEST INFRASTRUCTURE ONLY — see the header of canon_oracle.c.
 *
 * Every OP below is one IEEE-754 operation in type T, rounded to nearest
 * even; the file is built with -ffp-contract=off and without fast-math, so
 * the compiler may neither fuse nor reassociate.  The left operand of every
 * OP always covers the lower input indices.  (The comments write OP as "+".)
 */

#define CAT2(a, b) a##b
#define CAT(a, b) CAT2(a, b)
#define FN(name) CAT(name, CAT(_, SFX))

/* The operator itself, one application (for evaluations from scratch).    */
T FN(oracle_apply)(T a, T b)
{
    return OP(a, b);
}

/* ------------------------------------------------------------------------ */
/* PW(s): the iterative pairwise tree (canonical-reduce README, P4016R0,    */
/* "Key Design Points", first bullet).  Literal bottom-up evaluation: pair   */
/* (s0+s1), (s2+s3), ...; an odd trailing element is carried unchanged to    */
/* the next level; repeat until one value is left.  Returns 0 ("absent")     */
/* for an empty sequence, 1 otherwise.                                       */
/* ------------------------------------------------------------------------ */
static int FN(pw_strided)(const T* s, size_t n, size_t stride, T* out)
{
    if (n == 0) return 0;
    T* buf = (T*)malloc(n * sizeof(T));
    if (!buf) abort();
    for (size_t i = 0; i < n; ++i) buf[i] = s[i * stride];
    size_t m = n;
    while (m > 1) {
        size_t k = 0;
        for (size_t i = 0; i + 1 < m; i += 2) buf[k++] = OP(buf[i], buf[i + 1]);
        if (m & 1) buf[k++] = buf[m - 1];
        m = k;
    }
    *out = buf[0];
    free(buf);
    return 1;
}

int FN(oracle_pw)(const T* s, size_t n, T* out)
{
    return FN(pw_strided)(s, n, 1, out);
}

/* Per-lane values of the two-stage reduction (P4016R0, "Key Design Points": */
/* element i goes to lane i mod L; each lane is reduced by PW in increasing  */
/* index order).  lanes[j] receives PW(lane j) for j < min(n, L); the return */
/* value is that count m (lanes j >= m hold no element).                     */
size_t FN(oracle_lane_values)(const T* x, size_t n, uint32_t L, T* lanes)
{
    if (L == 0) return 0;
    size_t m = n < (size_t)L ? n : (size_t)L;
    for (size_t j = 0; j < m; ++j) {
        size_t len = (n - j + L - 1) / L;
        FN(pw_strided)(x + j, len, L, &lanes[j]);
    }
    return m;
}

/* CR_L(x[0..n)): the lane results combined "by the same tree rule", i.e.    */
/* PW over lanes 0..m-1 in lane order (P4016R0, "Key Design Points").        */
int FN(oracle_cr)(const T* x, size_t n, uint32_t L, T* out)
{
    if (n == 0 || L == 0) return 0;
    size_t m = n < (size_t)L ? n : (size_t)L;
    T* lanes = (T*)malloc(m * sizeof(T));
    if (!lanes) abort();
    FN(oracle_lane_values)(x, n, L, lanes);
    int r = FN(pw_strided)(lanes, m, 1, out);
    free(lanes);
    return r;
}

/* reduce(x, n, L, init) = op(init, R) with R = CR_L(x): init is combined     */
/* once, on the left, after the tree (P4016R0, "Key Design Points", init     */
/* placement bullet).  With no element the result is init itself.           */
T FN(oracle_reduce)(const T* x, size_t n, uint32_t L, T init)
{
    T r;
    if (!FN(oracle_cr)(x, n, L, &r)) return init;
    return OP(init, r);
}

/* ------------------------------------------------------------------------ */
/* Scan policies (P4229R0, "Summary" and "Key Design Points"): the scan     */
/* returns, for every i, the value of the policy's expression over the      */
/* prefix x[0..i].                                                           */
/*   policy 0  pairwise              E = PW                                  */
/*   policy 1  iterated_pairwise<L>  E = CR_L  (param = L)                   */
/*   policy 2  block_dyadic<B>       E(n) = PW(PW(block 0..q-1)) + PW(tail), */
/*                                   n = qB + t, 0 <= t < B (param = B);     */
/*                                   an empty part is left out.              */
/* ------------------------------------------------------------------------ */

/* One prefix, evaluated literally from scratch: O(i) work.  Returns 0 on a  */
/* bad argument, 1 otherwise.                                                */
int FN(oracle_scan_prefix)(const T* x, size_t i, int policy, uint32_t param, T* out)
{
    size_t n = i + 1;
    if (policy == 0) {
        return FN(pw_strided)(x, n, 1, out);
    }
    if (policy == 1) {
        if (param == 0) return 0;
        return FN(oracle_cr)(x, n, param, out);
    }
    if (policy == 2) {
        if (param == 0) return 0;
        size_t B = param, q = n / B, t = n % B;
        T H = 0, Tl = 0;
        int hasH = 0, hasT = 0;
        if (q > 0) {
            T* blocks = (T*)malloc(q * sizeof(T));
            if (!blocks) abort();
            for (size_t k = 0; k < q; ++k) FN(pw_strided)(x + k * B, B, 1, &blocks[k]);
            hasH = FN(pw_strided)(blocks, q, 1, &H);
            free(blocks);
        }
        if (t > 0) hasT = FN(pw_strided)(x + q * B, t, 1, &Tl);
        if (hasH && hasT) *out = OP(H, Tl);
        else if (hasH) *out = H;
        else *out = Tl;
        return 1;
    }
    return 0;
}

/* ---- streaming form: every prefix in one pass --------------------------- */
/* The "shift-reduce" reading of the pairwise tree (P4016R0, "Key Design     */
/* Points"): push each element as a level-0 subtree; while the two topmost   */
/* subtrees have the same level, replace them by (lower + upper).  The       */
/* stack then holds complete subtrees over consecutive ranges, largest       */
/* first; the prefix value is their right-to-left collapse                   */
/* s0 + (s1 + (... + s_top)).  The tests check this against the literal      */
/* bottom-up PW above on every prefix of small inputs.                       */
typedef struct {
    T val[72];
    int lvl[72];
    int top;
} FN(stack_t);

static void FN(st_push)(FN(stack_t)* s, T v)
{
    s->val[s->top] = v;
    s->lvl[s->top] = 0;
    s->top++;
    while (s->top >= 2 && s->lvl[s->top - 1] == s->lvl[s->top - 2]) {
        s->val[s->top - 2] = OP(s->val[s->top - 2], s->val[s->top - 1]);
        s->lvl[s->top - 2] += 1;
        s->top--;
    }
}

static int FN(st_collapse)(const FN(stack_t)* s, T* out)
{
    if (s->top == 0) return 0;
    T acc = s->val[s->top - 1];
    for (int k = s->top - 2; k >= 0; --k) acc = OP(s->val[k], acc);
    *out = acc;
    return 1;
}

/* All prefixes of x[0..n) under a policy.  y may equal x.  Returns 0 on a   */
/* bad argument, 1 otherwise.                                                */
int FN(oracle_scan)(const T* x, T* y, size_t n, int policy, uint32_t param)
{
    if (policy == 0) {
        FN(stack_t) st;
        st.top = 0;
        for (size_t i = 0; i < n; ++i) {
            FN(st_push)(&st, x[i]);
            FN(st_collapse)(&st, &y[i]);
        }
        return 1;
    }
    if (policy == 2) {
        if (param == 0) return 0;
        size_t B = param;
        /* blocks: shift-reduce over completed block values PW(block k);   */
        /* tail:   shift-reduce over the elements of the open block.       */
        FN(stack_t) blocks, tail;
        blocks.top = 0;
        tail.top = 0;
        for (size_t i = 0; i < n; ++i) {
            FN(st_push)(&tail, x[i]);
            if ((i + 1) % B == 0) {
                T bv = 0;
                FN(st_collapse)(&tail, &bv); /* PW of the whole block */
                FN(st_push)(&blocks, bv);
                tail.top = 0;
            }
            T H = 0, Tl = 0;
            int hasH = FN(st_collapse)(&blocks, &H);
            int hasT = FN(st_collapse)(&tail, &Tl);
            if (hasH && hasT) y[i] = OP(H, Tl);
            else if (hasH) y[i] = H;
            else y[i] = Tl;
        }
        return 1;
    }
    if (policy == 1) {
        if (param == 0) return 0;
        size_t L = param;
        /* lane j: shift-reduce stack over its elements, and the collapse   */
        /* of that stack (the PW prefix of lane j) kept up to date.         */
        FN(stack_t)* st = (FN(stack_t)*)malloc(L * sizeof(FN(stack_t)));
        T* cur = (T*)malloc(L * sizeof(T));
        T* buf = (T*)malloc(L * sizeof(T));
        if (!st || !cur || !buf) abort();
        for (size_t j = 0; j < L; ++j) st[j].top = 0;
        for (size_t i = 0; i < n; ++i) {
            size_t j = i % L;
            FN(st_push)(&st[j], x[i]);
            FN(st_collapse)(&st[j], &cur[j]);
            size_t m = (i + 1) < L ? (i + 1) : L; /* lanes holding an element */
            for (size_t k = 0; k < m; ++k) buf[k] = cur[k];
            FN(pw_strided)(buf, m, 1, &y[i]); /* PW over lanes 0..m-1 */
        }
        free(st);
        free(cur);
        free(buf);
        return 1;
    }
    return 0;
}

/* ---- scan with an initial value ------------------------------------------ */
/* Every output observes one prefix x[0..m) of the input and takes the value  */
/* init + E(x[0..m)): init is combined once, on the left, after the policy's  */
/* whole expression, exactly as the reduction places it (P4016R0 "Key Design  */
/* Points", init placement); the empty prefix (m = 0) observes init alone.    */
/* Which prefix output k observes follows the inclusive/exclusive duality of  */
/* the gt4py scan-redesign research page, B.2 "Array API standard / NumPy":   */
/*   kind 0  inclusive          m = k + 1,  k < n   (n outputs)              */
/*   kind 1  exclusive          m = k,      k < n   (n outputs)              */
/*   kind 2  include_initial    m = k,      k <= n  (n + 1 outputs)          */
/* y may equal x.  Returns 0 on a bad argument, 1 otherwise.                 */
int FN(oracle_scan_with_init)(const T* x, T* y, size_t n, int policy, uint32_t param, int kind,
                              T init)
{
    if (kind < 0 || kind > 2) return 0;
    T* s = (T*)malloc((n ? n : 1) * sizeof(T));
    if (!s) abort();
    if (!FN(oracle_scan)(x, s, n, policy, param)) {
        free(s);
        return 0;
    }
    const size_t nout = kind == 2 ? n + 1 : n;
    for (size_t k = 0; k < nout; ++k) {
        const size_t m = kind == 0 ? k + 1 : k;
        y[k] = m == 0 ? init : OP(init, s[m - 1]);
    }
    free(s);
    return 1;
}

/* ---- left fold (contrast only) --------------------------------------------- */
/* The sequential fold ((init + x0) + x1) + ... of std::accumulate, which the */
/* canonical expression replaces (P4016R0 "Summary": deterministic but       */
/* sequential); every prefix of it for the scan form (std::partial_sum with  */
/* init in front).  y may equal x.  Used to contrast, never to check the GPU.*/
T FN(oracle_left_fold)(const T* x, size_t n, T init)
{
    T acc = init;
    for (size_t i = 0; i < n; ++i) acc = OP(acc, x[i]);
    return acc;
}

void FN(oracle_left_fold_scan)(const T* x, T* y, size_t n, T init)
{
    T acc = init;
    for (size_t i = 0; i < n; ++i) {
        acc = OP(acc, x[i]);
        y[i] = acc;
    }
}

/* ---- batched rows: every row is an independent sequence ----------------- */
void FN(oracle_reduce_rows)(const T* x, size_t rows, size_t cols, size_t ldx, uint32_t L,
                            T init, T* out)
{
    for (size_t r = 0; r < rows; ++r) out[r] = FN(oracle_reduce)(x + r * ldx, cols, L, init);
}

int FN(oracle_scan_rows)(const T* x, size_t ldx, T* y, size_t ldy, size_t rows, size_t cols,
                         int policy, uint32_t param)
{
    for (size_t r = 0; r < rows; ++r)
        if (!FN(oracle_scan)(x + r * ldx, y + r * ldy, cols, policy, param)) return 0;
    return 1;
}

/* Row r of y (pitch ldy) is oracle_scan_with_init of row r of x; an        */
/* include_initial row has cols + 1 outputs (ldy >= cols + 1).               */
int FN(oracle_scan_rows_with_init)(const T* x, size_t ldx, T* y, size_t ldy, size_t rows,
                                   size_t cols, int policy, uint32_t param, int kind, T init)
{
    for (size_t r = 0; r < rows; ++r)
        if (!FN(oracle_scan_with_init)(x + r * ldx, y + r * ldy, cols, policy, param, kind, init))
            return 0;
    return 1;
}

#undef FN
#undef CAT
#undef CAT2
