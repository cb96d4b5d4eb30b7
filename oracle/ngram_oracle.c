/*
 * CPU oracle of the hashed bigram + trigram embedding path.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or constant generator with the HIP library: everything
 * here is written out again from the method's description.  It is slow and
 * plain on purpose: fp64 wherever the GPU accumulates, one loop per
 * definition, a library sort where grouping is needed.
 *
 * What the method is (sources: modded-nanogpt README, technique list; the
 * @classiclarryd post quoted on the airebao.com item on the 39.9 s record;
 * agentic-affairs "NanoGPT Training Record", ablation and architecture
 * sections; amund.blog "My 2nd modded-nanogpt world record attempt",
 * "The four improvements", item 4):
 *   - every position looks up one row of a hashed bigram table and one row of
 *     a hashed trigram table, each with a +/-1 sign, and the two signed rows
 *     are summed (the "sign trick");
 *   - n-gram context never crosses a document start: batches are aligned so a
 *     document opens with the EoS token;
 *   - the table is trained with Adam with beta1 = 0 and a single second-moment
 *     float per 768-wide row; only rows touched by the batch are updated, the
 *     beta2 decay a row missed is applied when the row is next touched, and the
 *     update runs once every 4 steps on the summed gradients.
 *
 * The pages give no hash function, seeds, dtypes or formulas.  The readings
 * taken here (each is also what the HIP path implements):
 *   hash   : SplitMix64 finaliser (Steele, Lea & Flood 2014, with Stafford's
 *            "Mix13" multipliers) of (key XOR seed) + golden gamma; the row is
 *            Lemire's multiply-shift of the upper 32 bits; the sign is bit 0.
 *   keys   : bigram (p1, t) and trigram (p2, p1, t) packed in base V+1, with
 *            V (one past the last id) standing for "no token".
 *   context: p1 = token i-1 unless i == 0 or token i is EoS; p2 = token i-2
 *            unless i < 2 or token i or token i-1 is EoS.
 *   forward: y = fp32(s_b*W_b[r_b] + s_t*W_t[r_t]), then rounded once to the
 *            table dtype (bf16: round to nearest, ties to even).
 *   grad   : G[r] = sum over the window, in (micro-step, position) order, of
 *            s*dY, in fp64, rounded once to fp32.
 *   step t : k = t - t_last; v' = fp32(beta2^k v + (1-beta2) mean(G^2));
 *            W' = round(W - lr G / (sqrt(v') + eps)); t_last = t.  No bias
 *            correction, eps outside the square root, t counts optimizer steps.
 */
#include <math.h>
#include <fenv.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

/* ---------------------------------------------------------------- hashing */

/* SplitMix64 output function applied to (key ^ seed) advanced by one gamma
 * step.  With seed 0 and key n*gamma this is the (n+1)-th SplitMix64 output of
 * state 0, which is how the tests pin it. */
uint64_t orc_hash64(uint64_t key, uint64_t seed)
{
    uint64_t z = (key ^ seed) + UINT64_C(0x9E3779B97F4A7C15);
    z = (z ^ (z >> 30)) * UINT64_C(0xBF58476D1CE4E5B9);
    z = (z ^ (z >> 27)) * UINT64_C(0x94D049BB133111EB);
    return z ^ (z >> 31);
}

/* Lemire's multiply-shift: maps the upper 32 bits of z onto [0, R). */
int64_t orc_row_of(uint64_t z, int64_t R)
{
    uint64_t hi = z >> 32;
    return (int64_t)((hi * (uint64_t)R) >> 32);
}

/* n-gram context of one micro-step: p1[i], p2[i] in [0, V], V = "none". */
void orc_context(const int32_t *tok, int64_t T, int64_t vocab, int32_t eos,
                 int64_t *p1, int64_t *p2)
{
    const int64_t none = vocab;
    for (int64_t i = 0; i < T; ++i) {
        int opens_doc = (tok[i] == eos);
        p1[i] = (i >= 1 && !opens_doc) ? (int64_t)(uint32_t)tok[i - 1] : none;
        p2[i] = (i >= 2 && !opens_doc && tok[i - 1] != eos)
                    ? (int64_t)(uint32_t)tok[i - 2] : none;
    }
}

/* The two 64-bit n-gram keys of a position. */
void orc_keys(int64_t vocab, int64_t p2, int64_t p1, int32_t t,
              uint64_t *kb, uint64_t *kt)
{
    uint64_t B = (uint64_t)vocab + 1u;
    uint64_t tt = (uint64_t)(uint32_t)t;
    *kb = (uint64_t)p1 * B + tt;
    *kt = ((uint64_t)p2 * B + (uint64_t)p1) * B + tt;
}

/* Rows and signs of both channels for one micro-step.  neg = 1 means the row
 * enters with sign -1.  Returns the number of ids outside [0, vocab). */
int64_t orc_ngram_rows(int64_t vocab, int32_t eos, const int64_t rows[2],
                       const uint64_t seeds[2], const int32_t *tok, int64_t T,
                       int64_t *row_b, uint8_t *neg_b, int64_t *row_t,
                       uint8_t *neg_t)
{
    int64_t bad = 0;
    int64_t *p1 = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
    int64_t *p2 = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
    orc_context(tok, T, vocab, eos, p1, p2);
    for (int64_t i = 0; i < T; ++i) {
        if (tok[i] < 0 || tok[i] >= vocab)
            ++bad;
        uint64_t kb, kt;
        orc_keys(vocab, p2[i], p1[i], tok[i], &kb, &kt);
        uint64_t zb = orc_hash64(kb, seeds[0]);
        uint64_t zt = orc_hash64(kt, seeds[1]);
        row_b[i] = orc_row_of(zb, rows[0]);
        neg_b[i] = (uint8_t)(zb & 1u);
        row_t[i] = orc_row_of(zt, rows[1]);
        neg_t[i] = (uint8_t)(zt & 1u);
    }
    free(p1);
    free(p2);
    return bad;
}

/* ------------------------------------------------------------- bf16 values */

double orc_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to the nearest bfloat16 (8 significant bits, fp32 exponent
 * range, subnormal quantum 2^-133), ties to even, by scaling to an integer
 * significand and using the C library's round-to-nearest-even.  NaN becomes
 * the canonical quiet NaN 0x7FC0; values past the largest finite bf16 after
 * rounding become infinity. */
uint16_t orc_double_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    if (isinf(x))
        return x > 0 ? 0x7F80 : 0xFF80;
    if (x == 0.0)
        return signbit(x) ? 0x8000 : 0x0000;
    int e;
    (void)frexp(x, &e);              /* x = m 2^e, 0.5 <= |m| < 1 */
    int q = e - 8;                   /* exponent of the last kept bit */
    if (q < -133)
        q = -133;
    double r = nearbyint(ldexp(x, -q));   /* default mode: ties to even */
    double y = ldexp(r, q);
    if (fabs(y) >= ldexp(1.0, 128))
        return x > 0 ? 0x7F80 : 0xFF80;
    float f = (float)y;              /* exact: y has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    if (y == 0.0)
        return signbit(x) ? 0x8000 : 0x0000;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------- table views */

/* A table as the oracle sees it: dense (ids == NULL, row r at r*dim) or a
 * snapshot of some rows (ids ascending, row ids[j] at j*dim). */
typedef struct {
    int32_t dtype;        /* ORC_F32 or ORC_BF16 */
    int32_t pad;
    int64_t n_ids;
    const int64_t *ids;
    const void *data;
} orc_table;

static int64_t orc_find(const orc_table *t, int64_t r)
{
    if (!t->ids)
        return r;
    int64_t lo = 0, hi = t->n_ids - 1;
    while (lo <= hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (t->ids[mid] == r)
            return mid;
        if (t->ids[mid] < r)
            lo = mid + 1;
        else
            hi = mid - 1;
    }
    return -1;
}

static double orc_get(const orc_table *t, int64_t j, int64_t dim, int64_t d)
{
    if (t->dtype == ORC_F32)
        return (double)((const float *)t->data)[j * dim + d];
    return orc_bf16_to_double(((const uint16_t *)t->data)[j * dim + d]);
}

/* ----------------------------------------------------------------- forward */

/* out[i] = s_b W_b[r_b(i)] + s_t W_t[r_t(i)], rounded to fp32, then to the
 * output dtype.  The fp32 sum is taken as (float)(double a + double b): for
 * addition, rounding through double (53 >= 2*24 + 2 bits) and then to float
 * gives the correctly rounded float sum.  Returns -1 if a row is missing from
 * a snapshot view, else 0. */
int orc_forward(const orc_table *Wb, const orc_table *Wt, int64_t dim,
                const int64_t *row_b, const uint8_t *neg_b,
                const int64_t *row_t, const uint8_t *neg_t, int64_t T,
                void *out, int32_t out_dtype)
{
    int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int64_t i = 0; i < T; ++i) {
        int64_t jb = orc_find(Wb, row_b[i]);
        int64_t jt = orc_find(Wt, row_t[i]);
        if (jb < 0 || jt < 0) {
            err = 1;
            continue;
        }
        for (int64_t d = 0; d < dim; ++d) {
            double a = orc_get(Wb, jb, dim, d);
            double b = orc_get(Wt, jt, dim, d);
            if (neg_b[i])
                a = -a;
            if (neg_t[i])
                b = -b;
            float y = (float)(a + b);
            if (out_dtype == ORC_F32)
                ((float *)out)[i * dim + d] = y;
            else
                ((uint16_t *)out)[i * dim + d] = orc_double_to_bf16((double)y);
        }
    }
    return err ? -1 : 0;
}

/* -------------------------------------------------------- window gradient */

typedef struct {
    int64_t row;
    int64_t pos;          /* index in the concatenated window stream */
} orc_entry;

static int orc_entry_cmp(const void *a, const void *b)
{
    const orc_entry *x = (const orc_entry *)a, *y = (const orc_entry *)b;
    if (x->row != y->row)
        return x->row < y->row ? -1 : 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

/* Gradient of one channel summed over a whole accumulation window.
 *
 * The window's micro-steps are given concatenated in order: entry e (0 <= e <
 * N) has row[e], neg[e] and the upstream gradient row dY[e*dim ..].  For every
 * row that occurs, G[row] = sum over its entries in stream order of s*dY, in
 * fp64, rounded once to fp32.  Writes the touched rows in ascending order to
 * touched[0..U) and their gradients to G[U][dim]; returns U. */
int64_t orc_window_grad(int64_t dim, int64_t N, const int64_t *row,
                        const uint8_t *neg, const float *dY, int64_t *touched,
                        float *G)
{
    if (N <= 0)
        return 0;
    orc_entry *e = (orc_entry *)malloc(sizeof(orc_entry) * (size_t)N);
    for (int64_t i = 0; i < N; ++i) {
        e[i].row = row[i];
        e[i].pos = i;
    }
    qsort(e, (size_t)N, sizeof(orc_entry), orc_entry_cmp);
    /* group starts */
    int64_t U = 0;
    int64_t *start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + 1));
    for (int64_t i = 0; i < N; ++i)
        if (i == 0 || e[i].row != e[i - 1].row)
            start[U++] = i;
    start[U] = N;
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)dim);
#pragma omp for schedule(dynamic, 64)
        for (int64_t u = 0; u < U; ++u) {
            for (int64_t d = 0; d < dim; ++d)
                acc[d] = 0.0;
            for (int64_t k = start[u]; k < start[u + 1]; ++k) {
                const float *g = dY + e[k].pos * dim;
                double s = neg[e[k].pos] ? -1.0 : 1.0;
                for (int64_t d = 0; d < dim; ++d)
                    acc[d] += s * (double)g[d];
            }
            touched[u] = e[start[u]].row;
            for (int64_t d = 0; d < dim; ++d)
                G[u * dim + d] = (float)acc[d];
        }
        free(acc);
    }
    free(start);
    free(e);
    return U;
}

/* ------------------------------------------------------- sparse row step */

/* beta2^k by the C library's pow in fp64. */
static double orc_decay(double beta2, int64_t k)
{
    return pow(beta2, (double)k);
}

/* Lazy row-wise Adam(beta1 = 0) step number t on the U touched rows of one
 * channel.  W[U][dim] (dtype w_dtype), v[U], t_last[U] hold the rows' state
 * and are updated in place; G[U][dim] is the window gradient. */
void orc_sparse_step(int64_t dim, int64_t U, const float *G, int32_t w_dtype,
                     void *W, float *v, int32_t *t_last, int32_t t, float lr,
                     float beta2, float eps)
{
#pragma omp parallel for schedule(static)
    for (int64_t u = 0; u < U; ++u) {
        const float *g = G + u * dim;
        int64_t k = (int64_t)t - (int64_t)t_last[u];
        double m = 0.0;
        for (int64_t d = 0; d < dim; ++d)
            m += (double)g[d] * (double)g[d];
        m /= (double)dim;
        double vn = orc_decay((double)beta2, k) * (double)v[u]
                    + (1.0 - (double)beta2) * m;
        float v32 = (float)vn;
        double denom = sqrt((double)v32) + (double)eps;
        for (int64_t d = 0; d < dim; ++d) {
            double w;
            if (w_dtype == ORC_F32)
                w = (double)((float *)W)[u * dim + d];
            else
                w = orc_bf16_to_double(((uint16_t *)W)[u * dim + d]);
            double wn = w - (double)lr * (double)g[d] / denom;
            if (w_dtype == ORC_F32)
                ((float *)W)[u * dim + d] = (float)wn;
            else
                ((uint16_t *)W)[u * dim + d] = orc_double_to_bf16(wn);
        }
        v[u] = v32;
        t_last[u] = t;
    }
}

/* Threads the OpenMP loops above use (1 when built without OpenMP). */
int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads of the OpenMP loops (n <= 0: all processors). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
#else
    (void)n;
#endif
}

int orc_rounding_is_nearest(void) { return fegetround() == FE_TONEAREST; }
