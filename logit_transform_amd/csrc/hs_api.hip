// hs_api.hip -- host side of libhs: argument validation, kernel choice and launches behind
// the C ABI declared in include/hs.h. Every check here runs before any HIP call, so a bad
// argument never enqueues work.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/hs.h"
#include "hs_internal.hpp"

// The workspace of hs_sample_noalloc, for callers that cannot allocate: a file-scope device
// array (each GPU the library runs on holds its own copy until the process ends). Host code
// never passes the array's name to a kernel: it takes each device's address from
// hipGetSymbolAddress once (scratch_for_device) and uses only that.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using hs::SampleArgs;

// Register-resident vectors per thread that kernels are generated for (blocks of up to 1024
// threads, 128 registers per lane).
constexpr int kNvBuckets[] = {1, 2, 4, 6, 8, 12, 16, 19};
constexpr int64_t kBlockCapacity = 19 * 1024;   // vectors one block can hold

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

inline int epv_of(int dt) { return dt == HS_F32 ? 4 : 8; }
inline int esize_of(int dt) { return dt == HS_F32 ? 4 : 2; }

int check_logits(const hs_logits *x) {
    if (!x || !x->data) return HS_ERR_INVALID_ARG;
    if (x->dtype != HS_F32 && x->dtype != HS_BF16 && x->dtype != HS_F16) return HS_ERR_DTYPE;
    if (x->B < 1 || x->V < 1 || x->ld < x->V) return HS_ERR_INVALID_ARG;
    if (x->V >= ((int64_t)1 << 31) || x->B >= ((int64_t)1 << 31)) return HS_ERR_UNSUPPORTED;
    // the kernels form byte offsets within a row in 32 bits: a row must stay below 4 GiB
    if ((uint64_t)x->V * (uint64_t)esize_of(x->dtype) >= ((uint64_t)1 << 32))
        return HS_ERR_UNSUPPORTED;
    return HS_OK;
}

int check_curve(const hs_hlg_params *p) {
    if (!p) return HS_ERR_INVALID_ARG;
    if (!(p->m > 0.0f) || !isfinite(p->m)) return HS_ERR_INVALID_ARG;
    if (!(p->w >= 0.0f)) return HS_ERR_INVALID_ARG;   // +inf allowed (rolloff off)
    if (!(p->beta_t > 0.0f) || !isfinite(p->beta_t)) return HS_ERR_INVALID_ARG;
    if (!(p->beta_h > 0.0f) || !isfinite(p->beta_h)) return HS_ERR_INVALID_ARG;
    if (p->pivot != HS_PIVOT_GIVEN && p->pivot != HS_PIVOT_TOP &&
        p->pivot != HS_PIVOT_ENTROPY && p->pivot != HS_PIVOT_MEDIAN)
        return HS_ERR_INVALID_ARG;
    if (p->pivot == HS_PIVOT_TOP && !isfinite(p->pivot_offset)) return HS_ERR_INVALID_ARG;
    return HS_OK;
}

hs::Curve make_curve(const hs_hlg_params *p) {
    hs::Curve c;
    c.m = p->m;
    c.w = p->w;
    c.mw = p->m * p->w;
    c.mbt = p->m * p->beta_t;
    c.mbh = p->m * p->beta_h;
    c.ibt = 1.0f / p->beta_t;
    c.ibh = 1.0f / p->beta_h;
    return c;
}

bool rows_aligned(const hs_logits *x) {
    const size_t es = (size_t)esize_of(x->dtype);
    return ((uintptr_t)x->data % 16 == 0) && (((size_t)x->ld * es) % 16 == 0);
}

int num_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cache[dev] = n;
    return n;
}

struct WsLayout {
    size_t counters, keys, partials, xslots, tau, done, queue, total;
};

WsLayout ws_layout(int64_t B, int32_t K) {
    WsLayout L;
    L.counters = 0;
    L.keys = align256((size_t)B * (size_t)K * 4);   // counters: one per (row, draw group)
    L.partials = L.keys + align256((size_t)B * (size_t)K * 8);
    L.xslots = L.partials + align256((size_t)B * hs::kMaxChunks * sizeof(float4));
    L.tau = L.xslots + align256((size_t)B * hs::kMaxChunks * 16);   // exchange slots
    L.done = L.tau + align256((size_t)B * 4);    // top-k / top-p thresholds
    L.queue = L.done + align256((size_t)B * 4);  // rows the threshold kernel drew
    L.total = L.queue + 256;                     // the resident grid's work counters
    return L;
}

struct Plan {
    int nchunk, nv, bs, nkg, kpg;
    int64_t nvec, cv;
    int64_t grid;
};

// Block size and vectors per thread for a chunk of cv vectors.
bool pick_block(int64_t cv, int *bs, int *nv) {
    int b = 1024;
    if (cv <= 256 * 4) b = 256;
    else if (cv <= 512 * 8) b = 512;
    const int64_t per = (cv + b - 1) / b;
    for (int x : kNvBuckets)
        if (per <= x) { *bs = b; *nv = x; return true; }
    return false;
}

// Kernel shape for a call. A row's draws are spread over blocks first ("draw groups": blocks
// that share a chunk of the row but not its draws need no cross-block combine), up to about one
// block per CU. Only if that leaves more than half of the CUs idle are rows split into chunks
// (of at least 256 vectors), aiming at one block per CU with the curve on (at most 16 chunks:
// they exchange log-sum-exp partials) and at one per two CUs without it (at most 32; each
// chunk then adds only its share of the cross-block combine); the chunks' maxima meet in the
// workspace. Rows longer than one block holds (kBlockCapacity vectors) are always split.
int make_plan(const hs_logits *x, int32_t K, bool hlg, bool ws_ok, const hs_sample_opts *o,
              Plan *P) {
    const int64_t B = x->B;
    const int64_t nvec = (x->V + epv_of(x->dtype) - 1) / epv_of(x->dtype);
    const int64_t cap = kBlockCapacity;
    const int64_t nchunk_min = (nvec + cap - 1) / cap;
    const int64_t cus = (int64_t)num_cus();
    const int variant = o ? o->variant : 0;
    const int64_t groups_given = (o && o->draw_groups > 0) ? o->draw_groups : 0;
    auto groups_for = [&](int64_t nchunk) -> int64_t {
        if (groups_given) return groups_given;
        int64_t g = (cus + B * nchunk - 1) / (B * nchunk);
        if (g > K) g = K;
        return g < 1 ? 1 : g;
    };
    int64_t nchunk = nchunk_min;
    if (variant == 1) {
        if (nchunk_min > 1) return HS_ERR_UNSUPPORTED;
        nchunk = 1;
    } else if (variant == 2 && o->nchunk > 0) {
        nchunk = o->nchunk;
    } else {
        const int64_t g = groups_for(nchunk_min);
        if (variant == 2 || (ws_ok && 2 * B * nchunk_min * g < cus)) {
            const int64_t target = hlg ? cus : cus / 2;
            int64_t want = (target + B * g - 1) / (B * g);
            int64_t lim = nvec / 256;
            // with the curve, a row's chunks exchange their log-sum-exp partials: past about
            // 16 chunks the exchange costs more than the shorter pass saves
            const int64_t cap = hlg ? 16 : 32;
            if (lim > cap) lim = cap;
            if (lim < 1) lim = 1;
            nchunk = want < lim ? want : lim;
            if (nchunk < nchunk_min) nchunk = nchunk_min;
            if (variant == 2 && nchunk < 2 && nvec >= 2) nchunk = 2;
        }
    }
    if (nchunk > hs::kMaxChunks) nchunk = hs::kMaxChunks;
    if (nchunk > nvec) nchunk = nvec;
    if (nchunk < nchunk_min) return HS_ERR_UNSUPPORTED;
    if (nchunk < 1) nchunk = 1;
    int64_t cv = (nvec + nchunk - 1) / nchunk;
    // fp32 chunks hold an even number of vectors: in the screened word layout the two lanes
    // whose vectors make up one eight-element group share its Philox call
    if (epv_of(x->dtype) == 4 && nchunk > 1 && (cv & 1)) ++cv;
    nchunk = (nvec + cv - 1) / cv;
    if (nchunk > 1 && !ws_ok) return HS_ERR_WORKSPACE;
    int bs = 0, nv = 0;
    if (!pick_block(cv, &bs, &nv)) return HS_ERR_UNSUPPORTED;
    int64_t nkg = groups_for(nchunk);
    if (nkg > K) nkg = K;
    int64_t kpg = (K + nkg - 1) / nkg;
    nkg = (K + kpg - 1) / kpg;
    const int64_t grid = B * nchunk * nkg;
    if (grid >= ((int64_t)1 << 31)) return HS_ERR_UNSUPPORTED;
    P->nchunk = (int)nchunk;
    P->nv = nv;
    P->bs = bs;
    P->nkg = (int)nkg;
    P->kpg = (int)kpg;
    P->nvec = nvec;
    P->cv = cv;
    P->grid = grid;
    return HS_OK;
}

bool opts_valid(const hs_sample_opts *o) {
    return !o || !(o->layout < 0 || o->layout > 1 || o->variant < 0 || o->variant > 2 || o->nchunk < 0 ||
                   o->nchunk > hs::kMaxChunks || o->draw_groups < 0 || o->split_lse < 0 ||
                   o->split_lse > 2 || o->exchange_wait < -1 || o->median_rows < 0 ||
                   o->median_rows > 1);
}

// Top-k / top-p parameters of a filtered call (device arrays, either may be null).
struct Filter {
    const int32_t *top_k;
    const float *top_p;
};

// rows: per-row curve settings (device), or NULL for the per-call curve hlg (or none);
// filt: top-k / top-p filters (curve off), or NULL.
int sample_impl(const hs_logits *x, const float *T, const float *mu, const hs_hlg_params *hlg,
                const hs_hlg_row *rows, const uint64_t *seed, const uint64_t *offset, int32_t K,
                int32_t *out, float *best, void *ws, size_t ws_bytes,
                const hs_sample_opts *opts, void *stream, const Filter *filt = nullptr) {
    int rc = check_logits(x);
    if (rc) return rc;
    if (!T || !seed || !offset || !out || K < 1) return HS_ERR_INVALID_ARG;
    if (hlg) {
        rc = check_curve(hlg);
        if (rc) return rc;
        if (hlg->pivot == HS_PIVOT_GIVEN && !mu) return HS_ERR_INVALID_ARG;
    }
    if (rows && hlg) return HS_ERR_INVALID_ARG;
    if (filt && (hlg || rows)) return HS_ERR_INVALID_ARG;
    const bool curve_on = hlg != nullptr || rows != nullptr;
    if ((size_t)x->B * (size_t)K >= ((size_t)1 << 31)) return HS_ERR_UNSUPPORTED;
    const WsLayout L = ws_layout(x->B, K);
    const bool ws_ok = ws && ws_bytes >= L.total && ((uintptr_t)ws % 256 == 0);
    if (ws && !ws_ok && ws_bytes > 0) {
        // a workspace was given but is unusable: report it rather than silently ignore it
        if (ws_bytes < L.total) return HS_ERR_WORKSPACE;
        return HS_ERR_INVALID_ARG;
    }
    const bool filtering = filt && (filt->top_k || filt->top_p);
    if (filtering && !ws_ok) return HS_ERR_WORKSPACE;   // the thresholds live in it
    Plan P;
    rc = make_plan(x, K, curve_on, ws_ok, opts, &P);
    if (rc) return rc;

    SampleArgs a{};
    a.data = x->data;
    a.ld = x->ld;
    a.V = x->V;
    a.nvec = P.nvec;
    a.cv = P.cv;
    a.nchunk = P.nchunk;
    a.nkg = P.nkg;
    a.kpg = P.kpg;
    a.K = K;
    a.aligned = rows_aligned(x) ? 1 : 0;
    a.no_screen = (opts && opts->no_screen) ? 1 : 0;
    a.layout = opts ? opts->layout : HS_LAYOUT_PLAIN;
    a.T = T;
    // internal pivot codes: 0 given, 1 top, 2 entropy, 3 per row, 4 mass median
    const int piv = rows ? 3 : !hlg ? 0 : hlg->pivot == HS_PIVOT_MEDIAN ? 4 : hlg->pivot;
    a.mu = (piv == HS_PIVOT_GIVEN || piv == 3) ? mu : nullptr;
    a.row_curves = reinterpret_cast<const hs::RowCurve *>(rows);
    a.seed = seed;
    a.offset = offset;
    a.out = out;
    a.best_out = best;
    if (hlg) {
        a.curve = make_curve(hlg);
        a.pivot_offset = hlg->pivot == HS_PIVOT_TOP ? hlg->pivot_offset : 0.0f;
    }
    if (P.nchunk > 1) {
        char *w = reinterpret_cast<char *>(ws);
        a.counters = reinterpret_cast<uint32_t *>(w + L.counters);
        a.keys = reinterpret_cast<uint64_t *>(w + L.keys);
        a.partials = reinterpret_cast<float4 *>(w + L.partials);
        a.part_stride = hs::kMaxChunks;
        a.xslots = reinterpret_cast<uint32_t *>(w + L.xslots);
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (filtering) {
        hs::FilterArgs f{};
        f.data = x->data;
        f.ld = x->ld;
        f.V = x->V;
        f.aligned = a.aligned;
        f.T = T;
        f.top_k = filt->top_k;
        f.top_p = filt->top_p;
        f.tau = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.tau);
        // With the automatic plan, rows that keep few tokens are drawn by the threshold kernel
        // and skipped by the sampler; an explicit kernel choice runs the sampler on every row.
        if (!opts || opts->variant == 0) {
            f.done = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) + L.done);
            f.out = out;
            f.best_out = best;
            f.seed = seed;
            f.offset = offset;
            f.K = K;
            f.layout = a.layout;
            a.done = f.done;
        }
        if (hs::launch_filter_tau(x->dtype, f, (int)x->B, s) != hipSuccess) return HS_ERR_HIP;
        a.tau = f.tau;
    }
    // Split rows with the curve on: the chunks' log-sum-exp partials are exchanged inside the
    // sampling kernel (one draw group per row) when every block of the grid is resident at
    // once, or on a resident work-queue grid (chunks of 12 or 16 slots); otherwise a pre-pass
    // computes them.
    // The mass median: the threshold kernel's top-p selection at p = 0.5, T = 1 gives every
    // row's shift c before the sampling kernel runs (which then needs no log-sum-exp).
    // Per-row settings: the same for the rows whose record asks for the median (the others
    // return at once), when the caller says some row may (opts->median_rows); otherwise, or
    // without a workspace, such rows give -2.
    if (piv == 4 || (piv == 3 && ws_ok && opts && opts->median_rows)) {
        if (!ws_ok) return HS_ERR_WORKSPACE;   // the shifts live in it
        hs::FilterArgs f{};
        f.data = x->data;
        f.ld = x->ld;
        f.V = x->V;
        f.aligned = a.aligned;
        f.median = 1;
        f.row_curves = piv == 3 ? a.row_curves : nullptr;
        f.tau = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.tau);
        if (hs::launch_filter_tau(x->dtype, f, (int)x->B, s) != hipSuccess) return HS_ERR_HIP;
        a.shift = f.tau;
    }
    int64_t grid = P.grid;
    a.items = (int32_t)P.grid;
    if (curve_on && P.nchunk > 1 && P.nkg == 1 && piv != 4) {
        const int mode = opts ? opts->split_lse : 0;
        int per_cu = 0;
        if (mode != 1 &&
            hs::launch_sample(x->dtype, true, piv, a, P.nv, P.bs, 0, s, &per_cu) != hipSuccess)
            per_cu = 0;
        const int64_t resident = (int64_t)per_cu * num_cus();
        if (mode == 2 || (mode == 0 && per_cu > 0 && P.grid <= resident)) {
            a.exchange = 1;
        } else if (mode == 0 && hs::queue_nv(P.nv) && a.aligned && a.V >= epv_of(x->dtype)) {
            // more blocks than fit at once (aligned rows, the chunk sizes that have a
            // work-queue kernel): a resident grid takes the (row, chunk) items from a counter,
            // so a row's chunks still run together and exchange their partials
            a.queue = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) + L.queue);
            int per_cu_q = 0;
            if (hs::launch_sample(x->dtype, true, piv, a, P.nv, P.bs, 0, s, &per_cu_q) ==
                    hipSuccess && per_cu_q > 0 && (int64_t)per_cu_q * num_cus() >= P.nchunk) {
                a.exchange = 1;
                grid = (int64_t)per_cu_q * num_cus();
            } else {
                a.queue = nullptr;
            }
        }
        const int wait = opts ? opts->exchange_wait : 0;
        a.spins = wait < 0 ? 0 : wait > 0 ? wait : hs::kExchangeSpins;
    }
    if (curve_on && P.nchunk > 1 && !a.exchange && piv != 4) {
        const int bs = P.cv >= 4096 ? 1024 : 256;
        if (hs::launch_lse_partial(x->dtype, piv, a, bs, (int)(x->B * P.nchunk), s) != hipSuccess)
            return HS_ERR_HIP;
    }
    if (hs::launch_sample(x->dtype, curve_on, piv, a, P.nv, P.bs, (int)grid, s) != hipSuccess)
        return HS_ERR_HIP;
    return HS_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];
int64_t g_scratch_B[kMaxDevices], g_scratch_K[kMaxDevices];   // the last call's shape

// The current device's scratch address, for a call of B rows and K draws. On a device's first
// use: the symbol's address on that device (the device is current), and a zero fill of the
// whole array on the caller's stream, since the workspace must start zero-filled. Every
// successful call leaves the regions that must start zero (counters, keys, exchange slots,
// queue counters) zero again, but the region offsets depend on B and K, and the regions a call
// leaves as written (pre-pass partials, filter thresholds, row marks) can lie where a call of
// another shape needs zeros: so when B or K differs from the previous call's, the span of
// both layouts is zero-filled first (a fill kernel, never hipMemsetAsync, since the call may
// be captured into a graph).
int scratch_for_device(hipStream_t s, int64_t B, int64_t K, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HS_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return HS_ERR_HIP;
        if (hs::launch_fill_zero(p, (int64_t)(kScratchBytes / 4), s) != hipSuccess)
            return HS_ERR_HIP;
        g_scratch[dev] = p;
    } else if (g_scratch_B[dev] != B || g_scratch_K[dev] != K) {
        const size_t prev = ws_layout(g_scratch_B[dev], (int32_t)g_scratch_K[dev]).total;
        const size_t cur = ws_layout(B, (int32_t)K).total;
        const size_t span = prev > cur ? prev : cur;
        if (hs::launch_fill_zero(g_scratch[dev], (int64_t)(span / 4), s) != hipSuccess)
            return HS_ERR_HIP;
    }
    g_scratch_B[dev] = B;
    g_scratch_K[dev] = K;
    *out = g_scratch[dev];
    return HS_OK;
}

}  // namespace

// The mass median of every row (the threshold kernel's top-p selection at p = 0.5, T = 1)
// into dst[b * stride]: the shift c of the median pivot [HLG, The pivot].
hipError_t launch_median_shift(const hs_logits *x, float *dst, int64_t stride, hipStream_t s) {
    hs::FilterArgs f{};
    f.data = x->data;
    f.ld = x->ld;
    f.V = x->V;
    f.aligned = rows_aligned(x) ? 1 : 0;
    f.median = 1;
    f.tau = dst;
    f.tau_stride = stride;
    return hs::launch_filter_tau(x->dtype, f, (int)x->B, s);
}

extern "C" {

int hs_logsumexp(const hs_logits *x, float *lse, void *stream) {
    int rc = check_logits(x);
    if (rc) return rc;
    if (!lse) return HS_ERR_INVALID_ARG;
    hs::RowOpArgs a{};
    a.data = x->data;
    a.ld = x->ld;
    a.V = x->V;
    a.aligned = rows_aligned(x) ? 1 : 0;
    a.lse = lse;
    return hs::launch_row_lse(x->dtype, 0, 0, a, (int)x->B, reinterpret_cast<hipStream_t>(stream))
                   == hipSuccess ? HS_OK : HS_ERR_HIP;
}

int hs_hlg_transform(const hs_logits *x, const float *mu, const hs_hlg_params *p, float *out,
                     int64_t ldo, void *stream) {
    int rc = check_logits(x);
    if (rc) return rc;
    rc = check_curve(p);
    if (rc) return rc;
    if ((p->pivot == HS_PIVOT_GIVEN && !mu) || !out || ldo < x->V) return HS_ERR_INVALID_ARG;
    hs::RowOpArgs a{};
    a.data = x->data;
    a.ld = x->ld;
    a.V = x->V;
    a.aligned = rows_aligned(x) ? 1 : 0;
    a.mu = p->pivot == HS_PIVOT_GIVEN ? mu : nullptr;
    a.out = out;
    a.ldo = ldo;
    a.curve = make_curve(p);
    a.pivot_offset = p->pivot == HS_PIVOT_TOP ? p->pivot_offset : 0.0f;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int piv = p->pivot;
    if (piv == HS_PIVOT_MEDIAN) {
        // each row's shift goes to the first element of its output row, which the transform
        // reads before it writes the row
        if (launch_median_shift(x, out, ldo, s) != hipSuccess) return HS_ERR_HIP;
        a.shift = out;
        a.shift_stride = ldo;
        piv = 4;
    }
    return hs::launch_row_lse(x->dtype, 1, piv, a, (int)x->B, s) == hipSuccess ? HS_OK
                                                                              : HS_ERR_HIP;
}

int hs_hlg_pivot(const hs_logits *x, const float *mu, const hs_hlg_params *p, float *mu_out,
                 void *stream) {
    int rc = check_logits(x);
    if (rc) return rc;
    rc = check_curve(p);
    if (rc) return rc;
    if ((p->pivot == HS_PIVOT_GIVEN && !mu) || !mu_out) return HS_ERR_INVALID_ARG;
    hs::RowOpArgs a{};
    a.data = x->data;
    a.ld = x->ld;
    a.V = x->V;
    a.aligned = rows_aligned(x) ? 1 : 0;
    a.mu = p->pivot == HS_PIVOT_GIVEN ? mu : nullptr;
    a.mu_out = mu_out;
    a.pivot_offset = p->pivot == HS_PIVOT_TOP ? p->pivot_offset : 0.0f;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int piv = p->pivot;
    if (piv == HS_PIVOT_MEDIAN) {
        // each row's shift goes to mu_out[b], which the pivot kernel reads before it writes
        // mu = c - LSE there
        if (launch_median_shift(x, mu_out, 1, s) != hipSuccess) return HS_ERR_HIP;
        a.shift = mu_out;
        a.shift_stride = 1;
        piv = 4;
    }
    return hs::launch_row_lse(x->dtype, 2, piv, a, (int)x->B, s) == hipSuccess ? HS_OK
                                                                              : HS_ERR_HIP;
}

int hs_gumbel_argmax(const hs_logits *x, const float *T, const uint64_t *seed,
                     const uint64_t *offset, int32_t K, int32_t *out, void *ws, size_t ws_bytes,
                     void *stream) {
    return sample_impl(x, T, nullptr, nullptr, nullptr, seed, offset, K, out, nullptr, ws,
                       ws_bytes, nullptr, stream);
}

int hs_sample(const hs_logits *x, const float *T, const float *mu, const hs_hlg_params *hlg,
              const uint64_t *seed, const uint64_t *offset, int32_t K, int32_t *out, void *ws,
              size_t ws_bytes, void *stream) {
    return sample_impl(x, T, mu, hlg, nullptr, seed, offset, K, out, nullptr, ws, ws_bytes, nullptr,
                       stream);
}

int hs_sample_ex(const hs_logits *x, const float *T, const float *mu, const hs_hlg_params *hlg,
                 const uint64_t *seed, const uint64_t *offset, int32_t K, int32_t *out,
                 float *best, void *ws, size_t ws_bytes, const hs_sample_opts *opts,
                 void *stream) {
    if (!opts_valid(opts)) return HS_ERR_INVALID_ARG;
    return sample_impl(x, T, mu, hlg, nullptr, seed, offset, K, out, best, ws, ws_bytes, opts,
                       stream);
}

int hs_sample_noalloc(const hs_logits *x, const float *T, const float *mu,
                      const hs_hlg_params *hlg, const uint64_t *seed, const uint64_t *offset,
                      int32_t K, int32_t *out, float *best, const hs_sample_opts *opts,
                      void *stream) {
    // every host-checkable argument first, so that a bad call touches no device
    if (!opts_valid(opts)) return HS_ERR_INVALID_ARG;
    int rc = check_logits(x);
    if (rc) return rc;
    if (!T || !seed || !offset || !out || K < 1) return HS_ERR_INVALID_ARG;
    if (hlg) {
        rc = check_curve(hlg);
        if (rc) return rc;
        if (hlg->pivot == HS_PIVOT_GIVEN && !mu) return HS_ERR_INVALID_ARG;
    }
    if ((size_t)x->B * (size_t)K >= ((size_t)1 << 31)) return HS_ERR_UNSUPPORTED;
    const size_t need = ws_layout(x->B, K).total;
    if (need > kScratchBytes) return HS_ERR_UNSUPPORTED;
    void *ws = nullptr;
    rc = scratch_for_device(reinterpret_cast<hipStream_t>(stream), x->B, K, &ws);
    if (rc) return rc;
    return sample_impl(x, T, mu, hlg, nullptr, seed, offset, K, out, best, ws, need, opts,
                       stream);
}

size_t hs_sample_noalloc_max_workspace(void) { return kScratchBytes; }

int hs_filter_threshold(const hs_logits *x, const float *T, const int32_t *top_k,
                        const float *top_p, float *tau, void *stream) {
    int rc = check_logits(x);
    if (rc) return rc;
    if (!T || !tau) return HS_ERR_INVALID_ARG;
    hs::FilterArgs f{};
    f.data = x->data;
    f.ld = x->ld;
    f.V = x->V;
    f.aligned = rows_aligned(x) ? 1 : 0;
    f.T = T;
    f.top_k = top_k;
    f.top_p = top_p;
    f.tau = tau;
    return hs::launch_filter_tau(x->dtype, f, (int)x->B, reinterpret_cast<hipStream_t>(stream))
                   == hipSuccess ? HS_OK : HS_ERR_HIP;
}

int hs_sample_filtered(const hs_logits *x, const float *T, const int32_t *top_k,
                       const float *top_p, const uint64_t *seed, const uint64_t *offset,
                       int32_t K, int32_t *out, float *best, void *ws, size_t ws_bytes,
                       const hs_sample_opts *opts, void *stream) {
    if (!opts_valid(opts)) return HS_ERR_INVALID_ARG;
    const Filter f{top_k, top_p};
    return sample_impl(x, T, nullptr, nullptr, nullptr, seed, offset, K, out, best, ws,
                       ws_bytes, opts, stream, &f);
}

int hs_sample_rows(const hs_logits *x, const float *T, const float *mu, const hs_hlg_row *rows,
                   const uint64_t *seed, const uint64_t *offset, int32_t K, int32_t *out,
                   float *best, void *ws, size_t ws_bytes, const hs_sample_opts *opts,
                   void *stream) {
    if (!rows || !opts_valid(opts)) return HS_ERR_INVALID_ARG;
    return sample_impl(x, T, mu, nullptr, rows, seed, offset, K, out, best, ws, ws_bytes, opts,
                       stream);
}

size_t hs_workspace_bytes(int64_t B, int64_t V, int32_t K, int32_t dtype, int32_t hlg_on) {
    (void)hlg_on;
    if (B < 1 || V < 1 || K < 1) return 0;
    if (dtype != HS_F32 && dtype != HS_BF16 && dtype != HS_F16) return 0;
    return ws_layout(B, K).total;
}

int hs_sample_plan(const hs_logits *x, int32_t K, int32_t hlg_on, int32_t have_ws,
                   const hs_sample_opts *opts, int64_t *plan) {
    int rc = check_logits(x);
    if (rc) return rc;
    if (!plan || K < 1 || !opts_valid(opts)) return HS_ERR_INVALID_ARG;
    if ((size_t)x->B * (size_t)K >= ((size_t)1 << 31)) return HS_ERR_UNSUPPORTED;
    Plan P;
    rc = make_plan(x, K, hlg_on != 0, have_ws != 0, opts, &P);
    if (rc) return rc;
    plan[0] = P.nchunk;
    plan[1] = P.cv;
    plan[2] = P.bs;
    plan[3] = P.nv;
    plan[4] = P.nkg;
    plan[5] = P.kpg;
    plan[6] = P.grid;
    plan[7] = num_cus();
    return HS_OK;
}

int hs_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws || ws_bytes % 4 != 0) return HS_ERR_INVALID_ARG;
    if (ws_bytes == 0) return HS_OK;
    return hs::launch_fill_zero(ws, (int64_t)(ws_bytes / 4), reinterpret_cast<hipStream_t>(stream))
                   == hipSuccess ? HS_OK : HS_ERR_HIP;
}

int hs_philox4x32_10(const uint32_t *ctr, const uint32_t *key, uint32_t *out, int64_t n,
                     void *stream) {
    if (!ctr || !key || !out || n < 0) return HS_ERR_INVALID_ARG;
    if (n == 0) return HS_OK;
    if (n >= ((int64_t)1 << 38)) return HS_ERR_UNSUPPORTED;
    return hs::launch_philox(ctr, key, out, n, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
                   ? HS_OK : HS_ERR_HIP;
}

int hs_stream_words_ex(const uint64_t *seed, const uint64_t *offset, int64_t B, int64_t V,
                       int32_t k, int32_t layout, uint32_t *out, void *stream) {
    if (!seed || !offset || !out || B < 1 || V < 1 || k < 0) return HS_ERR_INVALID_ARG;
    if (layout != HS_LAYOUT_PLAIN && layout != HS_LAYOUT_SCREENED) return HS_ERR_INVALID_ARG;
    if (V >= ((int64_t)1 << 31) || B > 65535) return HS_ERR_UNSUPPORTED;
    return hs::launch_stream_words(seed, offset, B, V, k, layout, out,
                                   reinterpret_cast<hipStream_t>(stream)) == hipSuccess
                   ? HS_OK : HS_ERR_HIP;
}

int hs_stream_words(const uint64_t *seed, const uint64_t *offset, int64_t B, int64_t V,
                    int32_t k, uint32_t *out, void *stream) {
    return hs_stream_words_ex(seed, offset, B, V, k, HS_LAYOUT_PLAIN, out, stream);
}

int hs_gumbel_f32(const uint32_t *words, float *g, int64_t n, void *stream) {
    if (!words || !g || n < 0) return HS_ERR_INVALID_ARG;
    if (n == 0) return HS_OK;
    if (n >= ((int64_t)1 << 40)) return HS_ERR_UNSUPPORTED;
    return hs::launch_gumbel(words, g, n, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
                   ? HS_OK : HS_ERR_HIP;
}

const char *hs_status_str(int status) {
    switch (status) {
        case HS_OK: return "HS_OK";
        case HS_ERR_INVALID_ARG: return "HS_ERR_INVALID_ARG: invalid argument";
        case HS_ERR_DTYPE: return "HS_ERR_DTYPE: unknown logits dtype";
        case HS_ERR_WORKSPACE: return "HS_ERR_WORKSPACE: workspace missing or too small";
        case HS_ERR_HIP: return "HS_ERR_HIP: HIP runtime or launch failure";
        case HS_ERR_UNSUPPORTED: return "HS_ERR_UNSUPPORTED: size outside the supported range";
    }
    return "unknown hs_status";
}

const char *hs_version(void) { return "libhs 0.2.0 (gfx950)"; }

}  // extern "C"
