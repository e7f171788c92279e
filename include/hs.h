/*
 * hs.h -- C ABI of libhs: batched HLG tone-curve + Gumbel-max token sampling on MI355X.
 *
 * Sources for every operation below (cited by page title and section):
 *   [HLG] "HLG sampling -- a piecewise tone curve on the logits", mlx-bun design document
 *         docs/design/hlg-sampling.md.
 *   [GMX] "Softmax-free GPU sampling: Gumbel-max categorical sampling kernel", lablup/mlxcel
 *         issue #900.
 *   [P123] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11
 *         (Philox4x32-10).
 *
 * Conventions shared by every call
 *   - Array arguments are DEVICE pointers owned by the caller (the library allocates nothing
 *     and keeps no state between calls). `hs_logits*` and `hs_hlg_params*` are HOST pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls only enqueue
 *     work on it and return at once; nothing synchronises.
 *   - The return value reports host-checkable errors only (hs_status). On any error no work
 *     is enqueued. Device-side per-row conditions are written into the output instead.
 *   - Logits are row-major [B, ld] with ld >= V elements; values must be finite or -inf
 *     (NaN / +inf are a precondition violation with undefined result). 16-byte aligned rows
 *     (data pointer and ld * element size both multiples of 16) take the vector load path;
 *     other layouts are accepted and read element by element.
 *   - Results do not depend on the grid the library picks: random numbers are a function of
 *     (seed, row, element, offset) only [GMX, Background].
 */
#ifndef HS_H
#define HS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HS_OK = 0,
    HS_ERR_INVALID_ARG = -1,  /* null pointer, B/V/K <= 0, ld < V, bad curve parameter ...  */
    HS_ERR_DTYPE = -2,        /* unknown hs_dtype                                          */
    HS_ERR_WORKSPACE = -3,    /* workspace missing or smaller than hs_workspace_bytes()     */
    HS_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed                 */
    HS_ERR_UNSUPPORTED = -5   /* size outside the supported range (V >= 2^31, ...)         */
} hs_status;

typedef enum { HS_F32 = 0, HS_BF16 = 1, HS_F16 = 2 } hs_dtype;

/* Logits [B, V] of one of the three input types of [GMX, Task 1] ("f32 or bf16/f16
 * upcast"); bf16 and f16 are widened to fp32 exactly. */
typedef struct {
    const void *data;   /* device pointer, row-major, row stride ld elements */
    int32_t dtype;      /* hs_dtype */
    int64_t B;          /* rows (batch) */
    int64_t V;          /* vocabulary size, 1 <= V < 2^31 and V * element size < 2^32 bytes
                           (fp32 rows below 2^30 elements); larger rows: HS_ERR_UNSUPPORTED */
    int64_t ld;         /* row stride in elements, ld >= V */
} hs_logits;

/* Where the curve's pivot mu comes from [HLG, The pivot]. */
typedef enum {
    HS_PIVOT_GIVEN = 0,   /* mu[b] passed in by the caller (log-prob nats)                 */
    HS_PIVOT_TOP = 1,     /* top-anchored: mu = l_max - pivot_offset, so z = x - (x_max - c) */
    HS_PIVOT_ENTROPY = 2, /* entropy-anchored: mu = sum_i p_i l_i (minus the entropy), so
                             z = x - E_p[x], p = softmax(x)                                 */
    HS_PIVOT_MEDIAN = 3   /* mass median: mu = the log-prob at which the mass of softmax(x),
                             summed from the top over groups of equal logits, first reaches
                             one half, so z = x - x_med (a first kernel finds x_med: the top-p
                             boundary at p = 0.5, T = 1)                                  */
} hs_pivot;

/* The curve knobs of [HLG, Knobs]: mid gain m > 0 (finite), mid half-width w >= 0 (+inf
 * turns the rolloff off), toe and shoulder rolloff constants beta_t, beta_h > 0 (finite),
 * all in nats; the pivot mode (hs_pivot) and, for HS_PIVOT_TOP, the offset c (finite; it is
 * ignored by the other modes). A zero-filled tail (pivot 0) keeps the caller-given pivot. */
typedef struct {
    float m;
    float w;
    float beta_t;
    float beta_h;
    int32_t pivot;
    float pivot_offset;
} hs_hlg_params;

/* lse[b] = log(sum_i exp(x[b,i])) over the finite entries of row b, -inf for a row with no
 * finite entry [HLG, The transfer function: the log-prob space l = x - LSE(x)].
 * lse: device float[B]. */
int hs_logsumexp(const hs_logits *x, float *lse, void *stream);

/* out[b*ldo + i] = g(z) with z = (x[b,i] - LSE_b) - mu[b] and g the toe / mid / shoulder
 * transfer function of [HLG, The transfer function, eq. z and eq. g]; -inf stays -inf.
 * This is l' before any temperature. mu: device float[B] (pivot, log-prob nats), read
 * only for HS_PIVOT_GIVEN; the other pivot modes compute mu[b] in the kernel (hs_hlg_pivot
 * gives its value); p: host pointer; out: device float[B*ldo], ldo >= V. A row with no finite entry is
 * written as all -inf. */
int hs_hlg_transform(const hs_logits *x, const float *mu, const hs_hlg_params *p, float *out,
                     int64_t ldo, void *stream);

/* mu_out[b] = the pivot the curve uses for row b in p's pivot mode, in log-prob nats
 * [HLG, The pivot]: mu[b] (HS_PIVOT_GIVEN), (x_max - LSE) - c (HS_PIVOT_TOP),
 * sum_i p_i (x_i - LSE) (HS_PIVOT_ENTROPY), or x_med - LSE (HS_PIVOT_MEDIAN); NaN for a row
 * with no finite entry.
 * mu: device float[B], read only for HS_PIVOT_GIVEN (may be NULL otherwise);
 * mu_out: device float[B]; p: host pointer. */
int hs_hlg_pivot(const hs_logits *x, const float *mu, const hs_hlg_params *p, float *mu_out,
                 void *stream);

/* Gumbel-max draws without the curve [GMX, Task 1]:
 *   out[b*K + k] = argmax_i ( x[b,i] / T[b] + G(word(seed[b], b, i, offset[b] + k)) ),
 * G(r) = -log(-log(u)), u = (r + 1/2) 2^-32, word = Philox4x32-10 [P123] with
 * key = (seed lo, seed hi), counter = (i >> 2, b, off lo, off hi), output word i & 3.
 * Ties go to the lowest index; -inf entries are never chosen [GMX, Regression guard].
 * Per-row results: -1 if the row has no finite entry, -2 if T[b] is negative, NaN,
 * infinite or subnormal (0 < T[b] < 2^-126, where 1/T overflows fp32). T[b] == 0 is greedy:
 * argmax of x, the same index for all K draws. Scores x/T (l'/T with the curve) must stay
 * inside the fp32 range; a row where they overflow has an undefined result.
 * T: device float[B]; seed, offset: device uint64[B]; out: device int32[B*K].
 * ws / ws_bytes: device workspace of at least hs_workspace_bytes(B, V, K, dtype, 0) bytes,
 * zero-filled before its first use (hs_workspace_init); every successful call leaves its
 * counters, keys and exchange slots zero-filled again (the split pre-pass's partials, and the
 * per-row filter thresholds and row marks of hs_sample_filtered, are left as written: each call
 * writes them before it reads them). Those regions' offsets depend on B and K, so a workspace
 * reused for a call with another B or K must be zero-filled again first (hs_workspace_init).
 * Calls that may run concurrently need separate workspaces. ws may be
 * NULL with ws_bytes 0, in which case only single-block-per-row kernels are used. */
int hs_gumbel_argmax(const hs_logits *x, const float *T, const uint64_t *seed,
                     const uint64_t *offset, int32_t K, int32_t *out, void *ws,
                     size_t ws_bytes, void *stream);

/* The full sampling step: the optional curve feeds the Gumbel-max draw [HLG, The transfer
 * function; GMX, Background]:
 *   l'_i = g((x_i - LSE_b) - mu[b])   when hlg != NULL,   l'_i = x_i   when hlg == NULL,
 *   out[b*K + k] = argmax_i ( l'_i / T[b] + G(word(seed[b], b, i, offset[b] + k)) ).
 * With the curve on and hlg->pivot == HS_PIVOT_GIVEN, mu must be a device float[B] and a
 * row with a non-finite mu gives -2; the other pivot modes derive mu[b] from the row in the
 * kernel (hs_hlg_pivot) and ignore mu. HS_PIVOT_MEDIAN needs the workspace (ws NULL gives
 * HS_ERR_WORKSPACE): a first kernel finds every row's mass median, the top-p boundary at
 * p = 0.5 and T = 1 (as hs_filter_threshold).
 * T[b] == 0 is greedy on x (the curve is monotone, so it cannot change the argmax
 * [HLG, Greedy is untouched]). Everything else as hs_gumbel_argmax; the workspace size is
 * hs_workspace_bytes(B, V, K, dtype, hlg != NULL). */
int hs_sample(const hs_logits *x, const float *T, const float *mu, const hs_hlg_params *hlg,
              const uint64_t *seed, const uint64_t *offset, int32_t K, int32_t *out,
              void *ws, size_t ws_bytes, void *stream);

/* Per-row curve settings for hs_sample_rows, one per row in device memory (32 bytes):
 * the knobs and pivot of hs_hlg_params, and whether the curve is on for the row
 * [HLG, The pivot; Knobs: one setting per request]. */
typedef struct {
    float m;
    float w;
    float beta_t;
    float beta_h;
    int32_t pivot;        /* hs_pivot (HS_PIVOT_MEDIAN needs the workspace)              */
    float pivot_offset;   /* c of HS_PIVOT_TOP */
    int32_t enabled;      /* 0: curve off for this row (l' = x) */
    int32_t reserved;     /* must be 0 */
} hs_hlg_row;

/* Workspace bytes the multi-block-per-row kernels of hs_sample / hs_gumbel_argmax need for
 * this shape (0 on invalid arguments). */
size_t hs_workspace_bytes(int64_t B, int64_t V, int32_t K, int32_t dtype, int32_t hlg_on);

/* Zero-fills a workspace on `stream` with a fill kernel (graph-capture safe). */
int hs_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Word layouts of the random stream (seed, row, i, offset) [GMX, Background: counter-based
 * Philox keyed on seed and offset]. Both hand out the bits of the same Philox4x32-10 calls
 * (counter (c, row, off lo, off hi), key (seed lo, seed hi)):
 *   HS_LAYOUT_PLAIN:    element i takes output word i & 3 of the call at c = i >> 2;
 *   HS_LAYOUT_SCREENED: element i = 8q + e takes the 16-bit half e (word e >> 1, low bits
 *                       for even e) of the call at c = 2q as the high half of its word and
 *                       the half e of the call at c = 2q + 1 as the low half.
 * Every element's word is uniform on 32 bits either way, so both give exact samples. The
 * screened layout lets the samplers draw one call per eight elements for most of the row: the
 * leading 16 bits bound each element's Gumbel value, and only the few elements those bounds
 * cannot rule out need the second call. */
typedef enum { HS_LAYOUT_PLAIN = 0, HS_LAYOUT_SCREENED = 1 } hs_layout;

/* Tuning / test control for hs_sample_ex. Zero-initialised = automatic choices and the plain
 * word layout. */
typedef struct {
    int32_t variant;     /* 0 automatic, 1 one block per row, 2 split the row over blocks */
    int32_t nchunk;      /* blocks per row when split (0 = automatic)                      */
    int32_t no_screen;   /* 1 = evaluate every element exactly (no candidate screening)    */
    int32_t draw_groups; /* blocks sharing one row's K draws (0 = automatic)               */
    int32_t split_lse;   /* split rows with the curve on: 0 automatic, 1 log-sum-exp
                            pre-pass, 2 exchange the chunks' partials inside the sampling
                            kernel (one draw group per row). Automatic: the exchange, either
                            with one block per (row, chunk) when they are all resident at
                            once, or (aligned rows, chunks of 12 or 16 vectors per thread)
                            with a resident grid whose blocks take the (row, chunk) items
                            from a counter in the workspace (so a row's chunks still run
                            together); the pre-pass when neither applies                    */
    int32_t exchange_wait; /* polls for the other chunks' partials before a block works
                              them out itself: 0 default, -1 none (test control), > 0 that
                              many                                                         */
    int32_t median_rows;   /* hs_sample_rows only: 1 = some row may ask for the mass-median
                              pivot, so a first kernel works out those rows' shifts (it needs
                              the workspace); 0 = no row does, nothing runs before the
                              sampler, and a row that asks for it anyway gives -2           */
    int32_t layout;        /* word layout of the random stream (hs_layout); the ids differ
                              between layouts, each an exact sample                         */
} hs_sample_opts;

/* hs_sample with explicit kernel choices. best (device float[B*K] or NULL) receives the
 * winning score of each draw (l'/T + G in fp32; the logit for greedy rows; -inf for rows
 * with a -1/-2 result). Results are identical for every choice of opts up to fp32 rounding
 * of the row's LSE. */
int hs_sample_ex(const hs_logits *x, const float *T, const float *mu,
                 const hs_hlg_params *hlg, const uint64_t *seed, const uint64_t *offset,
                 int32_t K, int32_t *out, float *best, void *ws, size_t ws_bytes,
                 const hs_sample_opts *opts, void *stream);

/* The launch plan hs_sample_ex would use for this shape (introspection; nothing is launched):
 * plan[0] blocks per row (chunks), [1] 16-byte vectors per chunk, [2] threads per block,
 * [3] vector slots per thread, [4] blocks sharing a row's draws, [5] draws per such block,
 * [6] grid size, [7] the CU count the plan assumed (256 when no device is visible).
 * have_ws: whether a workspace would be given (split rows need one). plan: host int64[8]. */
int hs_sample_plan(const hs_logits *x, int32_t K, int32_t hlg_on, int32_t have_ws,
                   const hs_sample_opts *opts, int64_t *plan);

/* hs_sample_ex with the curve set per row: row b is sampled as hs_sample_ex would sample it
 * alone with hlg = NULL (rows[b].enabled == 0) or with the curve of rows[b] (otherwise), in one
 * launch [HLG, The transfer function; The pivot; GMX, Background]. Per-row parameters are
 * validated in the kernel: a row whose enabled curve has an invalid knob (the rules of
 * hs_hlg_params), an unknown pivot, a non-finite top offset or a non-zero reserved field gives
 * -2, as does a given-pivot row whose mu is not finite or whose mu array is NULL, and a
 * median-pivot row unless opts->median_rows is 1 and ws is given (the rows' median shifts are
 * worked out into the workspace by a first kernel, which skips every other row). mu: device
 * float[B] or NULL (read only for enabled rows with HS_PIVOT_GIVEN); rows: device
 * hs_hlg_row[B]. Ids and scores of a row are bit-identical to hs_sample_ex's for that row's
 * setting. The workspace size is hs_workspace_bytes(B, V, K, dtype, 1). best and opts as
 * hs_sample_ex (NULL allowed). */
int hs_sample_rows(const hs_logits *x, const float *T, const float *mu, const hs_hlg_row *rows,
                   const uint64_t *seed, const uint64_t *offset, int32_t K, int32_t *out,
                   float *best, void *ws, size_t ws_bytes, const hs_sample_opts *opts,
                   void *stream);

/* hs_sample_ex without a workspace argument, for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the workspace
 * comes from a static device array of hs_sample_noalloc_max_workspace() bytes (4 MiB) that the
 * library holds on every GPU it runs on until the process ends. A shape whose workspace
 * (hs_workspace_bytes) exceeds it gives HS_ERR_UNSUPPORTED. The first call on a device
 * zero-fills the array on `stream`, and so does (over the span of both shapes' workspaces) a
 * call whose B or K differs from the previous call's on that device; a run of calls of one
 * shape adds no launch. All calls on one
 * GPU share its array: calls that overlap in time on one GPU (concurrent streams, or
 * unsynchronised host threads) race and their results are undefined. No hipMalloc, hipFree
 * or allocating library routine is called. Ids and scores equal hs_sample_ex's. */
int hs_sample_noalloc(const hs_logits *x, const float *T, const float *mu,
                      const hs_hlg_params *hlg, const uint64_t *seed, const uint64_t *offset,
                      int32_t K, int32_t *out, float *best, const hs_sample_opts *opts,
                      void *stream);

/* Size in bytes of hs_sample_noalloc's static workspace. */
size_t hs_sample_noalloc_max_workspace(void);

/* Top-k / top-p filters on the Gumbel path, curve off (the follow-on [GMX] names without an
 * algorithm; the reading taken): temperature first, then top-k, then top-p on the tempered
 * probabilities of the tokens top-k keeps. Row b keeps every token with x >= tau[b]:
 *   - top-k (top_k[b] > 0): tau_k = the top_k[b]-th largest finite logit (ties with it are
 *     kept); top_k[b] <= 0, or at least the number of finite logits, keeps every token;
 *   - top-p (0 < top_p[b] < 1): among the tokens top-k keeps, sorted by logit, the logit at
 *     which the mass exp((x - x_max) / T[b]), summed from the top, first reaches top_p[b]
 *     times their total (every token with that logit is kept); top_p[b] >= 1 keeps every
 *     token; top_p[b] <= 0 or NaN is invalid;
 *   - tau[b] = max(tau_k, tau_p); -inf when nothing is filtered or T[b] == 0 (greedy); NaN
 *     for an invalid T[b] or top_p[b].
 * The top-p boundary is found with fp64 sums of fp32 terms. top_k: device int32[B] or NULL;
 * top_p: device float[B] or NULL; tau: device float[B]. */
int hs_filter_threshold(const hs_logits *x, const float *T, const int32_t *top_k,
                        const float *top_p, float *tau, void *stream);

/* hs_gumbel_argmax over the tokens the filters keep (hs_filter_threshold): the Gumbel-max of
 * x / T over {i : x_i >= tau[b]}, an exact sample of softmax(x / T) renormalised over them
 * [GMX, Background]. A row with an invalid T or top_p gives -2; greedy rows (T == 0) are the
 * argmax of x. A workspace of hs_workspace_bytes(B, V, K, dtype, 0) bytes is required (the
 * thresholds live in it). best and opts as hs_sample_ex (NULL allowed). With the automatic
 * plan (opts NULL or variant 0), a row known to keep at most 2048 tokens (16-bit logits: the
 * kept count; fp32: the tokens at or above the top-k threshold, or the finite count without
 * top-k), with K <= 2048 and that count times K <= 65536, is drawn by the threshold kernel
 * itself, which scores only the kept tokens; an explicit variant runs the sampling kernel on
 * every row. Both give the same ids and scores. */
int hs_sample_filtered(const hs_logits *x, const float *T, const int32_t *top_k,
                       const float *top_p, const uint64_t *seed, const uint64_t *offset,
                       int32_t K, int32_t *out, float *best, void *ws, size_t ws_bytes,
                       const hs_sample_opts *opts, void *stream);

/* Philox4x32-10 [P123] on n (counter, key) pairs: ctr device uint32[4n], key device
 * uint32[2n], out device uint32[4n]. Uses the same device routine as the samplers. */
int hs_philox4x32_10(const uint32_t *ctr, const uint32_t *key, uint32_t *out, int64_t n,
                     void *stream);

/* The random words the samplers use for draw k: out[b*V + i] = word(seed[b], b,
 * i, offset[b] + k) (layout as in hs_gumbel_argmax). out: device uint32[B*V]. */
int hs_stream_words(const uint64_t *seed, const uint64_t *offset, int64_t B, int64_t V,
                    int32_t k, uint32_t *out, void *stream);

/* The same in a given word layout (hs_layout). */
int hs_stream_words_ex(const uint64_t *seed, const uint64_t *offset, int64_t B, int64_t V,
                       int32_t k, int32_t layout, uint32_t *out, void *stream);

/* The samplers' fp32 Gumbel map on n words: g[j] = G(words[j]). */
int hs_gumbel_f32(const uint32_t *words, float *g, int64_t n, void *stream);

/* Human-readable name of an hs_status value. */
const char *hs_status_str(int status);

/* Library version string. */
const char *hs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HS_H */
