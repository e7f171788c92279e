/*
 * hs_oracle.c -- plain, slow, double-precision CPU oracle for batched HLG tone-curve +
 * Gumbel-max token sampling.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this file;
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg use it. It shares
 * no code, header, table or constant generator with the HIP library.
 *
 * Sources (cited by title and section):
 *   [HLG]  "HLG sampling -- a piecewise tone curve on the logits", mlx-bun design document
 *          docs/design/hlg-sampling.md (mlx-bun 0.0.4).
 *   [GMX]  "Softmax-free GPU sampling: Gumbel-max categorical sampling kernel", lablup/mlxcel
 *          issue #900.
 *   [P123] J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As
 *          Easy as 1, 2, 3", SC'11 -- the published definition of Philox4x32-10.
 *
 * Every step is written the way the sources state it, in double precision, with no blocking,
 * fusion or reordering. Readings taken where the sources are silent:
 *   - Philox counter/key for "(seed, row, i, offset)" [GMX, Task 1]: key = (seed mod 2^32,
 *     seed >> 32); counter = (i >> 2, row, off mod 2^32, off >> 32); element i takes output
 *     word (i & 3). Draw k of a row uses off = offset_row + k (mod 2^64).
 *   - word -> uniform: u = (r + 1/2) * 2^-32, which is exact in double and never 0 or 1.
 *   - temperature with the curve: score = g(z) / T + G; greedy when T == 0 [HLG, Greedy is
 *     untouched; GMX, Task 3]; T < 0, T not finite, or T subnormal (0 < T < FLT_MIN, where
 *     1/T overflows single precision) gives -2.
 *   - ties go to the lowest index; a row with no finite logit gives -1.
 *   - logits must be finite or -inf; NaN or +inf makes the call fail (-1 return).
 *   - top-k / top-p on the Gumbel path (the follow-on the Gumbel-max issue names, without an
 *     algorithm): with the curve off, temperature first, then top-k, then top-p on the
 *     tempered probabilities of the tokens top-k keeps; each filter is a threshold on the
 *     logit and every token at or above it is kept (ties included). See or_filter_tau.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (never -ffast-math: it would break -inf masking).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------------------------
 * Philox4x32-10 [P123]: 4x32-bit counter, 2x32-bit key, 10 rounds. Each round multiplies
 * counter words 0 and 2 by the two round multipliers into 64-bit products, rebuilds the
 * counter from the high halves xor'd with the other counter words and the round key, and
 * keeps the low halves; the key is advanced by the two Weyl constants between rounds.
 * ------------------------------------------------------------------------------------- */
#define OR_PHILOX_M0 0xD2511F53u
#define OR_PHILOX_M1 0xCD9E8D57u
#define OR_PHILOX_W0 0x9E3779B9u
#define OR_PHILOX_W1 0xBB67AE85u

void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += OR_PHILOX_W0;
            k1 += OR_PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)OR_PHILOX_M0 * (uint64_t)c[0];
        uint64_t p1 = (uint64_t)OR_PHILOX_M1 * (uint64_t)c[2];
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c[1] ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c[3] ^ k1;
        uint32_t n3 = lo0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* Batch form for tests: n independent (counter, key) pairs. */
void or_philox4x32_10_n(int64_t n, const uint32_t *ctr, const uint32_t *key, uint32_t *out)
{
    for (int64_t j = 0; j < n; ++j)
        or_philox4x32_10(ctr + 4 * j, key + 2 * j, out + 4 * j);
}

/* The 32-bit random word of element i in draw stream (seed, row, off) [GMX, Task 1]. */
uint32_t or_element_word(uint64_t seed, uint64_t row, uint64_t off, uint64_t i)
{
    uint32_t ctr[4], key[2], out[4];
    ctr[0] = (uint32_t)(i >> 2);
    ctr[1] = (uint32_t)row;
    ctr[2] = (uint32_t)off;
    ctr[3] = (uint32_t)(off >> 32);
    key[0] = (uint32_t)seed;
    key[1] = (uint32_t)(seed >> 32);
    or_philox4x32_10(ctr, key, out);
    return out[i & 3];
}

/* The screened layout of the same stream: element i = 8q + e takes the high 16 bits of its
 * word from the 16-bit half e of the 128-bit output of the call at counter word 2q, and the
 * low 16 bits from the half e of the call at 2q + 1 (half e of an output: word e >> 1, bits
 * 16 (e & 1) .. 16 (e & 1) + 15). The other counter and key words are those of the plain
 * layout. It draws on the same calls as the plain layout (calls 2q and 2q + 1 cover elements
 * 8q .. 8q + 7 there) and only hands their bits out differently, so that one call gives the
 * leading 16 bits of eight elements. */
static uint32_t or_half16(const uint32_t out[4], unsigned e)
{
    return (out[e >> 1] >> (16u * (e & 1u))) & 0xFFFFu;
}

uint32_t or_element_word_screened(uint64_t seed, uint64_t row, uint64_t off, uint64_t i)
{
    uint32_t ctr[4], key[2], hi[4], lo[4];
    const uint64_t q = i >> 3;
    const unsigned e = (unsigned)(i & 7u);
    key[0] = (uint32_t)seed;
    key[1] = (uint32_t)(seed >> 32);
    ctr[1] = (uint32_t)row;
    ctr[2] = (uint32_t)off;
    ctr[3] = (uint32_t)(off >> 32);
    ctr[0] = (uint32_t)(2 * q);
    or_philox4x32_10(ctr, key, hi);
    ctr[0] = (uint32_t)(2 * q + 1);
    or_philox4x32_10(ctr, key, lo);
    return (or_half16(hi, e) << 16) | or_half16(lo, e);
}

/* Word of element i in the given layout: 0 plain, 1 screened. */
uint32_t or_element_word_layout(uint64_t seed, uint64_t row, uint64_t off, uint64_t i,
                                int layout)
{
    return layout == 1 ? or_element_word_screened(seed, row, off, i)
                       : or_element_word(seed, row, off, i);
}

/* Gumbel noise from a word [GMX, Background]: g = -log(-log(u)), u = (r + 1/2) 2^-32. */
double or_gumbel(uint32_t r)
{
    double u = ((double)r + 0.5) * 0x1p-32;
    return -log(-log(u));
}

/* ---------------------------------------------------------------------------------------
 * The HLG transfer function [HLG, The transfer function, eq. g]: toe for z < -w, linear
 * mid for |z| <= w, log shoulder for z > w. ln(1 + t) is evaluated as log1p(t).
 * -inf lands in the toe and maps to -inf [HLG, Properties that matter]. With w = +inf the
 * mid branch covers everything, including -inf (m * -inf = -inf).
 * ------------------------------------------------------------------------------------- */
double or_hlg_g(double z, double m, double w, double beta_t, double beta_h)
{
    if (z < -w)
        return -m * w - m * beta_t * log1p((-z - w) / beta_t);
    if (fabs(z) <= w)
        return m * z;
    return m * w + m * beta_h * log1p((z - w) / beta_h);
}

/* A usable temperature: 0 (greedy) or a normal positive single-precision value. T is read as
 * float, so FLT_MIN bounds the subnormals from above. */
static int or_temp_ok(double t)
{
    return t == 0.0 || (t >= (double)FLT_MIN && isfinite(t));
}

/* Validation shared by the row routines: curve knobs in nats [HLG, Knobs]. */
static int or_params_ok(double m, double w, double bt, double bh)
{
    if (!(m > 0.0) || !isfinite(m)) return 0;
    if (!(w >= 0.0)) return 0;                 /* +inf allowed: rolloff off */
    if (!(bt > 0.0) || !isfinite(bt)) return 0;
    if (!(bh > 0.0) || !isfinite(bh)) return 0;
    return 1;
}

static int or_row_ok(const double *x, int64_t V)
{
    for (int64_t i = 0; i < V; ++i)
        if (isnan(x[i]) || x[i] == INFINITY) return 0;
    return 1;
}

/* log-sum-exp of one row over its finite entries [HLG, The transfer function: log-prob
 * space]: LSE = M + log(sum_i exp(x_i - M)) with M the largest finite entry. The sum is
 * compensated (Neumaier's variant of Kahan summation: the rounding error of every addition is
 * carried in a second accumulator), so its error does not grow with the row length. Returns
 * -inf for a row with no finite entry. */
double or_row_logsumexp(const double *x, int64_t V)
{
    double M = -INFINITY;
    for (int64_t i = 0; i < V; ++i)
        if (x[i] > M) M = x[i];
    if (M == -INFINITY) return -INFINITY;
    double s = 0.0, comp = 0.0;
    for (int64_t i = 0; i < V; ++i) {
        if (!(x[i] > -INFINITY)) continue;
        double term = exp(x[i] - M);
        double t = s + term;
        if (fabs(s) >= fabs(term))
            comp += (s - t) + term;
        else
            comp += (term - t) + s;
        s = t;
    }
    return M + log(s + comp);
}

/* lse[r] for n rows of length V with row stride ld (elements). Returns 0, or -1 on a NaN /
 * +inf logit. */
int or_logsumexp(const double *x, int64_t n, int64_t V, int64_t ld, double *lse)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n; ++r) {
        const double *xr = x + r * ld;
        if (!or_row_ok(xr, V)) { bad |= 1; continue; }
        lse[r] = or_row_logsumexp(xr, V);
    }
    return bad ? -1 : 0;
}

double or_filter_tau_row(const double *x, int64_t V, double t, int32_t k, double p, int *amb);

/* The pivot mu of one row [HLG, The pivot], in log-prob nats, computed from the full
 * normalised log-prob vector l_i = x_i - LSE over the finite entries:
 *   mode 0 (given):   mu = mu_in;
 *   mode 1 (top):     mu = l_max - c, the curve centred c nats below the most probable token;
 *   mode 2 (entropy): mu = sum_i p_i l_i with p_i = exp(l_i), i.e. minus the entropy;
 *   mode 3 (median):  mu = the log-prob at which the probability mass, summed from the most
 *                     probable token down over groups of equal logits, first reaches one half
 *                     (the top-p boundary at p = 0.5 and T = 1: or_filter_tau_row).
 * lse is the row's log-sum-exp (finite: the row has a finite entry). */
double or_row_pivot(const double *x, int64_t V, double lse, int mode, double c, double mu_in)
{
    if (mode == 3) {
        int amb = 0;
        return or_filter_tau_row(x, V, 1.0, 0, 0.5, &amb) - lse;
    }
    if (mode == 1) {
        double lmax = -INFINITY;
        for (int64_t i = 0; i < V; ++i) {
            if (!(x[i] > -INFINITY)) continue;
            double ell = x[i] - lse;
            if (ell > lmax) lmax = ell;
        }
        return lmax - c;
    }
    if (mode == 2) {
        double acc = 0.0;
        for (int64_t i = 0; i < V; ++i) {
            if (!(x[i] > -INFINITY)) continue;
            double ell = x[i] - lse;
            acc += exp(ell) * ell;
        }
        return acc;
    }
    return mu_in;
}

/* Pivot of n rows (row stride ld): mu_out[r], NAN for a row with no finite entry. mu_in may
 * be NULL unless mode == 0. Returns 0, -1 on a NaN / +inf logit, -2 on a bad mode / offset. */
int or_pivot(const double *x, int64_t n, int64_t V, int64_t ld, int mode, double c,
             const float *mu_in, double *mu_out)
{
    if (mode < 0 || mode > 3 || (mode == 1 && !isfinite(c))) return -2;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n; ++r) {
        const double *xr = x + r * ld;
        if (!or_row_ok(xr, V)) { bad |= 1; continue; }
        double lse = or_row_logsumexp(xr, V);
        mu_out[r] = (lse > -INFINITY) ? or_row_pivot(xr, V, lse, mode, c,
                                                      mu_in ? (double)mu_in[r] : 0.0)
                                      : NAN;
    }
    return bad ? -1 : 0;
}

/* l'[r, i] = g(l_i - mu_r) with l_i = x_i - LSE_r, the log-prob [HLG, The transfer function,
 * eq. z and eq. g]. The +mu shift is dropped because it cancels under softmax [HLG, same
 * section]. Masked entries stay -inf. The pivot mu_r comes from or_row_pivot (mode pivot,
 * offset c); a given mu is read as float and widened. */
int or_hlg_transform(const double *x, int64_t n, int64_t V, int64_t ld, const float *mu,
                     float m, float w, float bt, float bh, int pivot, float c, double *out,
                     int64_t ldo)
{
    if (!or_params_ok(m, w, bt, bh)) return -2;
    if (pivot < 0 || pivot > 3 || (pivot == 1 && !isfinite(c))) return -2;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n; ++r) {
        const double *xr = x + r * ld;
        double *orow = out + r * ldo;
        if (!or_row_ok(xr, V)) { bad |= 1; continue; }
        double lse = or_row_logsumexp(xr, V);
        double mur = (lse > -INFINITY) ? or_row_pivot(xr, V, lse, pivot, (double)c,
                                                       pivot == 0 ? (double)mu[r] : 0.0)
                                       : 0.0;
        for (int64_t i = 0; i < V; ++i) {
            if (xr[i] == -INFINITY) { orow[i] = -INFINITY; continue; }
            double ell = xr[i] - lse;          /* log-prob */
            double z = ell - mur;              /* centred coordinate */
            orow[i] = or_hlg_g(z, m, w, bt, bh);
        }
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------------------------
 * Sampling [GMX, Background; Task 1]: for every draw k the score of element i is
 * s_i = l'_i / T + g_i with g_i Gumbel noise from the element's Philox word, and the token is
 * argmax_i s_i (lowest index on ties). l' = x with the curve off, the transformed log-prob
 * with it on. T == 0 is greedy: argmax of x, the curve being monotone [HLG, Greedy is
 * untouched]. Masked (-inf) tokens are never chosen [GMX, Regression guard].
 *
 * Inputs per row r of the n given rows: x (double, n x ld), row_id[r] (the global row index
 * that keys the counter), T[r], mu[r] (only with the curve on and pivot mode 0), seed[r],
 * offset[r]; pivot and c select the pivot mode (or_row_pivot).
 * Outputs: out[r*K + k] token index, or -1 (no finite logit) / -2 (bad T, or bad given mu);
 * best[r*K+k] and second[r*K+k] (may be NULL) the two largest scores of that draw
 * (-inf when absent). With hlg == 0 the curve parameters are ignored. layout selects the
 * stream's word layout (0 plain, 1 screened: or_element_word_layout).
 * Returns 0, -1 on a NaN/+inf logit, -2 on bad curve parameters or layout.
 * ------------------------------------------------------------------------------------- */
int or_sample(const double *x, int64_t n, int64_t V, int64_t ld, const int64_t *row_id,
              const float *T, const float *mu, int hlg, float m, float w, float bt, float bh,
              int pivot, float c, const uint64_t *seed, const uint64_t *offset, int32_t K,
              int32_t *out, double *best, double *second, int layout)
{
    if (layout != 0 && layout != 1) return -2;
    if (hlg && !or_params_ok(m, w, bt, bh)) return -2;
    if (hlg && (pivot < 0 || pivot > 3 || (pivot == 1 && !isfinite(c)))) return -2;
    int bad = 0;
    for (int64_t r = 0; r < n; ++r)
        if (!or_row_ok(x + r * ld, V)) bad = 1;
    if (bad) return -1;
    /* every (row, draw) pair is independent; the row's log-sum-exp is recomputed per pair
     * so each pair follows the definition on its own */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t rk = 0; rk < n * (int64_t)K; ++rk) {
        int64_t r = rk / K;
        int32_t k = (int32_t)(rk % K);
        const double *xr = x + r * ld;
        int32_t *o = out + rk;
        double *b1 = best ? best + rk : NULL;
        double *b2 = second ? second + rk : NULL;
        *o = -1;
        if (b1) *b1 = -INFINITY;
        if (b2) *b2 = -INFINITY;
        int64_t nfinite = 0;
        for (int64_t i = 0; i < V; ++i) nfinite += (xr[i] > -INFINITY);
        if (nfinite == 0) continue;                                   /* -1 */
        double t = (double)T[r];
        if (!or_temp_ok(t) || (hlg && pivot == 0 && !isfinite((double)mu[r]))) {
            *o = -2;
            continue;
        }
        int64_t j = -1;
        double s1 = -INFINITY, s2 = -INFINITY;
        if (t == 0.0) {                                               /* greedy on x */
            for (int64_t i = 0; i < V; ++i) {
                if (!(xr[i] > -INFINITY)) continue;
                if (j < 0 || xr[i] > s1) { s2 = s1; s1 = xr[i]; j = i; }
                else if (xr[i] > s2) s2 = xr[i];
            }
        } else {
            double lse = hlg ? or_row_logsumexp(xr, V) : 0.0;
            double mur = hlg ? or_row_pivot(xr, V, lse, pivot, (double)c,
                                            pivot == 0 ? (double)mu[r] : 0.0)
                             : 0.0;
            uint64_t off = offset[r] + (uint64_t)k;                   /* mod 2^64 */
            for (int64_t i = 0; i < V; ++i) {
                if (!(xr[i] > -INFINITY)) continue;
                double lp = hlg ? or_hlg_g((xr[i] - lse) - mur, m, w, bt, bh) : xr[i];
                uint32_t word = or_element_word_layout(seed[r], (uint64_t)row_id[r], off,
                                                       (uint64_t)i, layout);
                double s = lp / t + or_gumbel(word);
                if (j < 0 || s > s1) { s2 = s1; s1 = s; j = i; }
                else if (s > s2) s2 = s;
            }
        }
        *o = (int32_t)j;
        if (b1) *b1 = s1;
        if (b2) *b2 = s2;
    }
    return 0;
}

/* The Philox words of one draw stream, for bit-exact comparison: words[i] for i < V. */
void or_stream_words(uint64_t seed, uint64_t row, uint64_t off, int64_t V, uint32_t *words)
{
    for (int64_t i = 0; i < V; ++i)
        words[i] = or_element_word(seed, row, off, (uint64_t)i);
}

/* The same in a given layout (0 plain, 1 screened). */
void or_stream_words_layout(uint64_t seed, uint64_t row, uint64_t off, int64_t V, int layout,
                            uint32_t *words)
{
    for (int64_t i = 0; i < V; ++i)
        words[i] = or_element_word_layout(seed, row, off, (uint64_t)i, layout);
}

/* Element-wise batch forms for tests. */
void or_gumbel_n(int64_t n, const uint32_t *r, double *g)
{
    for (int64_t j = 0; j < n; ++j) g[j] = or_gumbel(r[j]);
}

void or_hlg_g_n(int64_t n, const double *z, double m, double w, double bt, double bh, double *out)
{
    for (int64_t j = 0; j < n; ++j) out[j] = or_hlg_g(z[j], m, w, bt, bh);
}


/* ---------------------------------------------------------------------------------------
 * Top-k / top-p filters on the Gumbel path (curve off). Reading: the draw is the Gumbel-max
 * of the tempered logits restricted to the kept tokens, i.e. an exact sample of softmax(x/T)
 * renormalised over them [GMX, Background: argmax of x/T + G is a sample of softmax(x/T); the
 * same holds on any subset]. The kept set, in the usual order of the two filters:
 *   - top-k (k > 0): the tokens whose logit is at least the k-th largest finite logit;
 *     k <= 0 or k >= the number of finite logits keeps every finite token;
 *   - top-p (0 < p < 1): among the tokens top-k keeps, sorted by logit, the shortest prefix
 *     whose tempered probability mass exp((x - x_max)/T) / S reaches p, where S is the mass of
 *     the tokens top-k keeps; every token whose logit equals the last one's is kept too.
 *     p >= 1 keeps every token; p <= 0 or NaN is invalid (-2 for the row).
 * The combined kept set is {i : x_i >= tau}. tau = -inf when nothing is filtered (and for
 * greedy rows, whose argmax is always kept).
 * ------------------------------------------------------------------------------------- */
static int or_cmp_desc(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

/* tau of one row; *amb = 1 when the top-p crossing lies within 1e-5 * S of p * S on either
 * side, so that an fp32 computation may take a neighbouring boundary. */
double or_filter_tau_row(const double *x, int64_t V, double t, int32_t k, double p, int *amb)
{
    *amb = 0;
    if (t == 0.0) return -INFINITY;
    double *v = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
    int64_t n = 0;
    for (int64_t i = 0; i < V; ++i)
        if (x[i] > -INFINITY) v[n++] = x[i];
    double tau = -INFINITY;
    if (n == 0) { free(v); return tau; }
    qsort(v, (size_t)n, sizeof(double), or_cmp_desc);
    int64_t nk = n;                                  /* tokens top-k keeps: v[0 .. nk) */
    if (k > 0 && (int64_t)k < n) {
        tau = v[k - 1];
        nk = k;
        while (nk < n && v[nk] == tau) ++nk;         /* ties with the k-th are kept */
    }
    if (p < 1.0) {
        double S = 0.0;
        for (int64_t i = 0; i < nk; ++i) S += exp((v[i] - v[0]) / t);
        double P = p * S, cum = 0.0;
        int64_t i = 0;
        while (i < nk) {
            int64_t j = i;                           /* the group of logits equal to v[i] */
            double wsum = 0.0;
            while (j < nk && v[j] == v[i]) { wsum += exp((v[j] - v[0]) / t); ++j; }
            double before = cum;
            cum += wsum;
            if (cum >= P) {
                if (v[i] > tau) tau = v[i];
                *amb = (P - before < 1e-5 * S) || (cum - P < 1e-5 * S);
                break;
            }
            i = j;
        }
    }
    free(v);
    return tau;
}

/* tau[r] and amb[r] of n rows; returns 0, -1 on a NaN/+inf logit. Rows with an invalid T or
 * p get tau = NaN. */
int or_filter_tau(const double *x, int64_t n, int64_t V, int64_t ld, const float *T,
                  const int32_t *top_k, const float *top_p, double *tau, int32_t *amb)
{
    int bad = 0;
    for (int64_t r = 0; r < n; ++r)
        if (!or_row_ok(x + r * ld, V)) bad = 1;
    if (bad) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        double t = (double)T[r];
        double p = top_p ? (double)top_p[r] : 1.0;
        int a = 0;
        if (!or_temp_ok(t) || !(p > 0.0)) {
            tau[r] = NAN;
        } else {
            tau[r] = or_filter_tau_row(x + r * ld, V, t, top_k ? top_k[r] : 0, p, &a);
        }
        if (amb) amb[r] = a;
    }
    return 0;
}

/* or_sample with the curve off and the kept set {x >= tau[r]} of or_filter_tau: tokens below
 * the threshold are treated as masked. Outputs and layout as or_sample; -2 also for an invalid
 * p. */
int or_sample_filtered(const double *x, int64_t n, int64_t V, int64_t ld,
                       const int64_t *row_id, const float *T, const int32_t *top_k,
                       const float *top_p, const uint64_t *seed, const uint64_t *offset,
                       int32_t K, int32_t *out, double *best, double *second, double *tau,
                       int32_t *amb, int layout)
{
    if (layout != 0 && layout != 1) return -2;
    int rc = or_filter_tau(x, n, V, ld, T, top_k, top_p, tau, amb);
    if (rc) return rc;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t rk = 0; rk < n * (int64_t)K; ++rk) {
        int64_t r = rk / K;
        int32_t k = (int32_t)(rk % K);
        const double *xr = x + r * ld;
        double *b1 = best ? best + rk : NULL;
        double *b2 = second ? second + rk : NULL;
        out[rk] = -1;
        if (b1) *b1 = -INFINITY;
        if (b2) *b2 = -INFINITY;
        int64_t nfinite = 0;
        for (int64_t i = 0; i < V; ++i) nfinite += (xr[i] > -INFINITY);
        if (nfinite == 0) continue;                                   /* -1 */
        double t = (double)T[r];
        if (isnan(tau[r])) { out[rk] = -2; continue; }                /* bad T or p */
        int64_t j = -1;
        double s1 = -INFINITY, s2 = -INFINITY;
        uint64_t off = offset[r] + (uint64_t)k;
        for (int64_t i = 0; i < V; ++i) {
            if (!(xr[i] > -INFINITY) || xr[i] < tau[r]) continue;
            double s = (t == 0.0) ? xr[i]
                                  : xr[i] / t + or_gumbel(or_element_word_layout(
                                                    seed[r], (uint64_t)row_id[r], off,
                                                    (uint64_t)i, layout));
            if (j < 0 || s > s1) { s2 = s1; s1 = s; j = i; }
            else if (s > s2) s2 = s;
        }
        out[rk] = (int32_t)j;
        if (b1) *b1 = s1;
        if (b2) *b2 = s2;
    }
    return 0;
}
