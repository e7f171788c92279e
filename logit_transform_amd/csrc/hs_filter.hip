// hs_filter.hip -- the per-row logit threshold of the top-k / top-p filters on the Gumbel path
// (curve off). The Gumbel-max issue names rejection-based top-k / top-p as its follow-on
// without an algorithm ("Softmax-free GPU sampling", the follow-on list). Reading taken:
// temperature first, then top-k, then top-p on the tempered probabilities of the tokens top-k
// keeps; each filter keeps every token whose logit is at or above a threshold tau (ties
// included), and the sampler draws the Gumbel-max of x / T over the kept tokens, an exact
// sample of the renormalised softmax [GMX, Background].
//
// One block per row finds tau. For 16-bit logits (k_filter_tau16) one pass counts every
// distinct value of the row in an LDS histogram of all 65536 bit patterns, and the thresholds
// come from scans over that histogram (see the section below). For fp32 logits, and for a
// 16-bit row where more than 65535 elements share a value, a radix selection over an
// order-preserving integer key of the logit is used: each level a pass over the row (which
// stays in the caches after the first) that histograms one digit of the keys sharing the
// digits selected so far: 11 + 11 + 10 bits for fp32, 11 + 5 for 16-bit logits (a wide first
// digit spreads the bulk of a row over many bins, so the LDS atomics seldom collide).
// Top-k selects the k-th largest finite key by counts (its first pass also finds the row's
// maximum and finite count); top-p selects, among the keys top-k keeps, the key at which the
// tempered mass exp((x - x_max) / T), summed from the top, reaches p times the total, by fp64
// sums of fp32 terms. Wave 0 picks each level's bin with a parallel scan over the bins.
//
// The same kernels serve two more uses. In median mode (T = 1, top-p 0.5, no top-k) tau is
// the mass median of the row, the shift of the curve's median pivot [HLG, The pivot]. And when
// the caller asks for it, a row known to keep few tokens is drawn here as well (draw_kept): a
// second pass gathers the kept tokens and every (token, draw) pair is scored exactly, so the
// sampling kernel can skip the row.
#include <hip/hip_runtime.h>

#include "hs_device.hpp"
#include "hs_internal.hpp"

namespace hs {
namespace {

// Order-preserving keys (-0 folded onto +0); -inf keys sort below every finite key and
// every finite key is > 0.
__device__ __forceinline__ uint32_t key16(uint32_t h) {
    if (h == 0x8000u) h = 0u;
    return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}
__device__ __forceinline__ uint32_t key32(uint32_t u) {
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int DT>
__device__ __forceinline__ uint32_t elem_key(const uint4 &v, int e) {
    if constexpr (DT == DT_F32) {
        const uint32_t w = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
        return key32(w);
    } else {
        const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
        return key16((e & 1) ? (w >> 16) : (w & 0xFFFFu));
    }
}

template <int DT>
__device__ __forceinline__ float key_value(uint32_t key) {
    if constexpr (DT == DT_F32) {
        return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
    } else {
        const uint32_t h = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
        if constexpr (DT == DT_BF16) return __uint_as_float(h << 16);
        return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    }
}

// (wave 0) The bin, scanning the NB bins from the top, at which the running total first
// reaches target, and the total of the bins above it. A total that falls short by rounding
// takes the lowest non-empty bin. Lane l holds the bins NB-1-l*CPL ... NB-CPL-l*CPL.
template <typename Cnt, int NB>
__device__ __forceinline__ void select_bin(const Cnt *hist, Cnt target, int lane, int *bin,
                                           Cnt *above) {
    constexpr int CPL = NB >= 64 ? NB / 64 : 1;
    Cnt c[CPL];
    Cnt own = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int r = lane * CPL + j;   // rank from the top
        c[j] = r < NB ? hist[NB - 1 - r] : (Cnt)0;
        own += c[j];
    }
    Cnt incl = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const Cnt o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    const Cnt excl = incl - own;
    const uint64_t hit = __ballot(incl >= target);
    const uint64_t nonempty = __ballot(own > 0);
    const int src = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(nonempty | 1ull);
    int b = -1;
    Cnt ab = excl;
    if (lane == src) {
        Cnt run = excl;
        int last = -1;
        Cnt last_above = excl;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            if (c[j] > 0) {
                last = j;
                last_above = run;
            }
            if (b < 0 && hit && run + c[j] >= target) {
                b = j;
                ab = run;
            }
            run += c[j];
        }
        if (b < 0) {
            b = last < 0 ? 0 : last;
            ab = last < 0 ? excl : last_above;
        }
        b = NB - 1 - (lane * CPL + b);
    }
    *bin = __shfl(b, src, 64);
    *above = __shfl(ab, src, 64);
}

// The digits of a key, most significant first: widths and shifts per level.
template <int DT> struct Digits;
template <> struct Digits<DT_F32> {
    static constexpr int n = 3;
    static constexpr int bits[3] = {11, 11, 10};
    static constexpr int shift[3] = {21, 10, 0};
};
template <> struct Digits<DT_BF16> {
    static constexpr int n = 2;
    static constexpr int bits[2] = {11, 5};
    static constexpr int shift[2] = {5, 0};
};
template <> struct Digits<DT_F16> : Digits<DT_BF16> {};

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t *red) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if (lane == 0) red[wid] = v;
    __syncthreads();
    uint32_t t = lane < nw ? red[lane] : 0u;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
    __syncthreads();
    return t;
}

// f(v) on every 16-byte vector of the row, four loads in flight per lane: whole vectors of
// aligned rows are read directly, four per step; the rest (and misaligned rows) one at a time.
template <int DT, typename F>
__device__ __forceinline__ void for_each_vec(const char *rowp, int64_t nvec, int64_t V,
                                             int32_t aligned, F f) {
    const int BS = blockDim.x;
    int64_t gv = threadIdx.x;
    if (aligned) {
        const int64_t nfull = V / dtype_traits<DT>::epv;
        const uint4 *p = reinterpret_cast<const uint4 *>(rowp);
        for (; gv + 3 * BS < nfull; gv += 4 * BS) {
            const uint4 v0 = p[gv], v1 = p[gv + BS], v2 = p[gv + 2 * BS], v3 = p[gv + 3 * BS];
            f(v0, gv);
            f(v1, gv + BS);
            f(v2, gv + 2 * BS);
            f(v3, gv + 3 * BS);
        }
    }
    for (; gv < nvec; gv += BS) f(load_vec<DT>(rowp, gv, V, aligned), gv);
}

// One level of the selection: the histogram (counts, or masses w(x)) of digit `lev` over the
// finite keys >= kmin whose higher digits equal prefix, then the bin where the total from the
// top reaches target (wave 0). Returns the new prefix; *tgt (wave 0) becomes what is left to
// reach inside the bin.
template <int DT, int LEV, typename Cnt, typename W>
__device__ __forceinline__ uint32_t select_level(const char *rowp, int64_t nvec, int64_t V,
                                                 int32_t aligned, uint32_t prefix, uint32_t kmin,
                                                 Cnt *hist, Cnt *tgt, W weight, int lane,
                                                 int wid) {
    using D = Digits<DT>;
    constexpr int EPV = dtype_traits<DT>::epv;
    constexpr int NB = 1 << D::bits[LEV];
    constexpr int SH = D::shift[LEV];
    for (int j = threadIdx.x; j < NB; j += blockDim.x) hist[j] = (Cnt)0;
    __syncthreads();
    // the keys of the selected bin (and >= kmin) span a range of values [lo, hi]: elements
    // outside it are rejected with two compares before their key is formed
    // (keys beyond those of -inf and +inf decode to NaN: such a bound is loosened to -inf or
    // +inf; kmin, when set, is the key of a finite logit)
    float lo = kmin > 0u ? key_value<DT>(kmin) : -__builtin_inff(), hi = __builtin_inff();
    if constexpr (LEV > 0) {
        constexpr int LOWB = SH + D::bits[LEV];   // bits below the selected prefix
        const uint32_t k0 = prefix << LOWB;
        const uint32_t k1 = k0 | ((1u << LOWB) - 1u);
        const float v0 = key_value<DT>(k0), v1 = key_value<DT>(k1);
        if (v0 == v0) lo = fmaxf(lo, v0);
        if (v1 == v1) hi = v1;
    }
    for_each_vec<DT>(rowp, nvec, V, aligned, [&](const uint4 &v, int64_t) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float x = elem<DT>(v, e);
            if (x >= lo && x <= hi && x > -__builtin_inff()) {
                const uint32_t key = elem_key<DT>(v, e);
                bool in = key >= kmin;
                if constexpr (LEV > 0) in = in && (key >> (SH + D::bits[LEV])) == prefix;
                if (in) atomicAdd(&hist[(key >> SH) & (uint32_t)(NB - 1)], weight(x));
            }
        }
    });
    __syncthreads();
    __shared__ uint32_t s_new;
    if (wid == 0) {
        int bin;
        Cnt above;
        select_bin<Cnt, NB>(hist, *tgt, lane, &bin, &above);
        *tgt -= above;
        if (lane == 0) s_new = (prefix << D::bits[LEV]) | (uint32_t)bin;
    }
    __syncthreads();
    return s_new;
}

// A row's filter settings; false (with tau written) when they decide tau without the logits:
// NaN for an invalid temperature or p (the sampler turns it into -2 for the row), -inf when
// nothing is filtered (greedy rows, k <= 0 or k >= V with p >= 1).
struct RowFilter {
    float T, p;
    int32_t k;
};

__device__ __forceinline__ bool row_filter(const FilterArgs &a, int64_t b, RowFilter *f) {
    if (a.median) {   // the mass median [HLG, The pivot]: the top-p boundary at p = 0.5, T = 1
        if (a.row_curves != nullptr) {
            const RowCurve r = a.row_curves[b];
            if (!(r.enabled != 0 && r.pivot == 3)) return false;   // not a median row
        }
        f->T = 1.0f;
        f->k = 0;
        f->p = 0.5f;
        return true;
    }
    f->T = a.T[b];
    f->k = a.top_k ? a.top_k[b] : 0;
    if ((int64_t)f->k >= a.V) f->k = 0;   // a k of at least V keeps every token
    f->p = a.top_p ? a.top_p[b] : 1.0f;
    float tau;
    if (!temp_valid(f->T) || !(f->p > 0.0f)) {
        tau = __builtin_nanf("");
    } else if (f->T == 0.0f || (f->k <= 0 && !(f->p < 1.0f))) {
        tau = -__builtin_inff();
    } else {
        return true;
    }
    if (threadIdx.x == 0) a.tau[b * (a.tau_stride ? a.tau_stride : 1)] = tau;
    return false;
}

// The radix selection of tau (every dtype) with the LDS histograms hc [2048] and hm [2048].
// tau, and an upper bound on the tokens at or above it (the count at or above the top-k
// threshold, ties included, or the finite count); the same in every thread.
struct TauKept {
    float tau;
    uint32_t kept;
};
template <int DT>
__device__ __forceinline__ TauKept tau_radix(const FilterArgs &a, int64_t b, const RowFilter &f,
                                             uint32_t *hc, double *hm, float *red_f,
                                             uint32_t *red_n) {
    uint32_t kept_v = 0u;
    uint32_t *kept = &kept_v;
    using tr = dtype_traits<DT>;
    using D = Digits<DT>;
    constexpr int EPV = tr::epv;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const float T = f.T, p = f.p;
    const int32_t k = f.k;
    const char *rowp = reinterpret_cast<const char *>(a.data) + b * a.ld * tr::esize;
    const int64_t nvec = (a.V + EPV - 1) / EPV;

    // the row's maximum and finite count (with top-k on, its first level counts them too)
    float M = -__builtin_inff();
    uint32_t NF = 0u;
    uint32_t keyk = 0u;   // 0: every finite key passes
    float tau = -__builtin_inff();
    if (k > 0) {
        uint32_t tgt = (uint32_t)k;   // (wave 0) rank still to go inside the selected bin
        float mx = -__builtin_inff();
        auto one = [&](float x) {
            mx = fmaxf(mx, x);
            return 1u;
        };
        uint32_t prefix = select_level<DT, 0>(rowp, nvec, a.V, a.aligned, 0u, 0u, hc, &tgt, one,
                                              lane, wid);
        M = block_max(mx, red_f);
        // the level's bins hold every finite key: their total is the finite count
        uint32_t part = 0u;
        for (int j = tid; j < (1 << D::bits[0]); j += blockDim.x) part += hc[j];
        NF = block_sum_u32(part, red_n);
        if ((uint32_t)k < NF) {
            prefix = select_level<DT, 1>(rowp, nvec, a.V, a.aligned, prefix, 0u, hc, &tgt,
                                         [](float) { return 1u; }, lane, wid);
            if constexpr (D::n == 3)
                prefix = select_level<DT, 2>(rowp, nvec, a.V, a.aligned, prefix, 0u, hc, &tgt,
                                             [](float) { return 1u; }, lane, wid);
            keyk = prefix;
            tau = key_value<DT>(keyk);
            // keys above tau's (k less the rank left inside its bin) plus tau's own count
            __shared__ uint32_t s_kept_r;
            if (tid == 0) {
                constexpr int NBL = 1 << D::bits[D::n - 1];
                s_kept_r = (uint32_t)k - tgt + hc[prefix & (uint32_t)(NBL - 1)];
            }
            __syncthreads();
            *kept = s_kept_r;
        } else {
            *kept = NF;
        }
    } else {
        uint32_t nf = 0u;
        float mx = -__builtin_inff();
        for_each_vec<DT>(rowp, nvec, a.V, a.aligned, [&](const uint4 &v, int64_t) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float x = elem<DT>(v, e);
                nf += x > -__builtin_inff() ? 1u : 0u;
                mx = fmaxf(mx, x);
            }
        });
        M = block_max(mx, red_f);
        NF = block_sum_u32(nf, red_n);
        *kept = NF;
    }
    if (NF == 0u) return TauKept{-__builtin_inff(), 0u};

    // top-p over the tokens top-k keeps: the key at which the tempered mass from the top
    // reaches p times their total
    if (p < 1.0f) {
        const float c1 = kLog2e / T;
        auto mass = [=](float x) { return (double)__builtin_amdgcn_exp2f((x - M) * c1); };
        // the target needs the kept tokens' total mass: wave 0 sums the first level's bins
        // before selecting (a target of +inf selects nothing; it is set below)
        double tgt = 0.0;
        for (int j = tid; j < (1 << D::bits[0]); j += blockDim.x) hm[j] = 0.0;
        __syncthreads();
        const float lo = keyk > 0u ? tau : -__builtin_inff();   // tau = the value of keyk
        for_each_vec<DT>(rowp, nvec, a.V, a.aligned, [&](const uint4 &v, int64_t) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float x = elem<DT>(v, e);
                if (x >= lo && x > -__builtin_inff())
                    atomicAdd(&hm[elem_key<DT>(v, e) >> D::shift[0]], mass(x));
            }
        });
        __syncthreads();
        __shared__ uint32_t s_p0;
        if (wid == 0) {
            constexpr int NB = 1 << D::bits[0];
            double t = 0.0;
            for (int j = lane; j < NB; j += 64) t += hm[j];
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
            tgt = (double)p * t;
            int bin;
            double above;
            select_bin<double, NB>(hm, tgt, lane, &bin, &above);
            tgt -= above;
            if (lane == 0) s_p0 = (uint32_t)bin;
        }
        __syncthreads();
        uint32_t prefix = s_p0;
        prefix = select_level<DT, 1>(rowp, nvec, a.V, a.aligned, prefix, keyk, hm, &tgt, mass,
                                     lane, wid);
        if constexpr (D::n == 3)
            prefix = select_level<DT, 2>(rowp, nvec, a.V, a.aligned, prefix, keyk, hm, &tgt,
                                         mass, lane, wid);
        tau = fmaxf(tau, key_value<DT>(prefix));
    }
    return TauKept{tau, kept_v};
}


// ---- 16-bit logits: one exact-value histogram per row ---------------------------------------
// A 16-bit logit takes one of 65536 bit patterns, so one pass can count every distinct value
// of the row: two 16-bit counters per LDS word (pattern h in word h >> 1, half h & 1), 128 KiB.
// Counts, the row's maximum, the k-th largest value and the tempered masses then come from
// that histogram alone: the row is read once, and an element costs one LDS atomic instead of
// one per selection level (with an exponential and an fp64 atomic for top-p). A counter
// overflows only when more than 65535 elements share one value; the sum of all counters then
// falls short of the finite count, and the block runs the radix selection instead.
//
// Ranks order the patterns by value from the top: ranks 0 .. 32767 are the non-negative
// patterns 0x7FFF down to 0x0000, ranks 32768 .. 65535 the negative ones 0x8000 up to 0xFFFF.
// NaN and -inf patterns never hold a count, and -0 is merged into +0 before any selection.
// Thread t owns ranks 64t .. 64t + 63, i.e. 32 consecutive words.
__device__ __forceinline__ uint32_t rank_bits(uint32_t r) {
    return r < 32768u ? 32767u - r : r;
}
__device__ __forceinline__ uint32_t bits_rank(uint32_t h) {
    return h < 32768u ? 32767u - h : h;
}
__device__ __forceinline__ int owned_words(int t) {
    return t < 512 ? 16352 - 32 * t : 32 * t;
}
__device__ __forceinline__ uint32_t hist_count(const uint32_t *hist, uint32_t h) {
    return (hist[h >> 1] >> ((h & 1u) << 4)) & 0xFFFFu;
}
template <int DT>
__device__ __forceinline__ float bits_value(uint32_t h) {
    if constexpr (DT == DT_BF16) return __uint_as_float(h << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Inclusive and exclusive block scan over threads in index order (1024 threads), and the
// total. incl of a thread equals excl of the next one exactly, also in floating point.
template <typename T>
__device__ __forceinline__ void block_scan(T v, T *red, T *excl, T *incl, T *total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    T in = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const T o = __shfl_up(in, d, 64);
        if (lane >= d) in += o;
    }
    T ex = __shfl_up(in, 1, 64);
    if (lane == 0) ex = (T)0;
    if (lane == 63) red[wid] = in;
    __syncthreads();
    T base = (T)0, run = (T)0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        if (w == wid) base = run;
        run = run + red[w];
    }
    __syncthreads();
    *excl = lane == 0 ? base : base + ex;
    *incl = base + in;
    *total = run;
}

// (wave 0) Among the 64 ranks of thread t, the first at which the running total of weight()
// from `above` reaches target; the last rank of non-zero weight when it never does (a total
// that rounding left short of the target).
template <typename Tw, typename W>
__device__ __forceinline__ uint32_t resolve_rank(int t, Tw above, Tw target, int lane, W weight,
                                                 Tw *cum) {
    t = min(max(t, 0), 1023);
    const uint32_t r = 64u * (uint32_t)t + (uint32_t)lane;
    const Tw w = weight(r);
    Tw in = w;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const Tw o = __shfl_up(in, d, 64);
        if (lane >= d) in += o;
    }
    const uint64_t hit = __ballot(above + in >= target);
    const uint64_t nz = __ballot(w > (Tw)0);
    const int l = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(nz | 1ull);
    *cum = __shfl(above + in, l, 64);
    return 64u * (uint32_t)t + (uint32_t)l;
}

// (wave) The sum of v over lanes 0 .. l.
__device__ __forceinline__ uint32_t wave_prefix_at(uint32_t v, int lane, int l) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return __shfl(v, l, 64);
}

// The draw of a row that keeps few tokens, in the threshold kernel: when at most kSparseKept
// tokens are kept (nk, an upper bound), with K <= kSparseKept and nk * K <= kSparsePairs, a
// second pass over the row gathers the kept tokens (x >= tau) into LDS, and every (token, draw)
// pair is scored exactly, x / T + G(word) [GMX, Background], with the sampling kernel's Philox
// words, arithmetic and keys; an LDS atomic maximum per draw picks the winner. Returns whether
// the row was drawn (then out / best_out hold its draws). lds: 8192 words, 8-byte aligned,
// free for this use.
template <int DT>
__device__ __forceinline__ bool draw_kept(const FilterArgs &a, int64_t b, float T, float tau,
                                          uint32_t nk, const char *rowp, int64_t nvec,
                                          uint32_t *lds) {
    constexpr int EPV = dtype_traits<DT>::epv;
    const int tid = threadIdx.x;
    const int K = a.K;
    if (!(nk <= (uint32_t)kSparseKept && K <= kSparseKept && (int64_t)nk * K <= kSparsePairs))
        return false;
    __syncthreads();   // lds may still be read by the selection
    uint32_t *l_idx = lds;                                                  // [kSparseKept]
    float *l_x = reinterpret_cast<float *>(lds + kSparseKept);              // [kSparseKept]
    uint64_t *l_key = reinterpret_cast<uint64_t *>(lds + 2 * kSparseKept);  // [kSparseKept]
    __shared__ uint32_t s_n;
    if (tid == 0) s_n = 0u;
    for (int j = tid; j < K; j += 1024) l_key[j] = 0ull;
    __syncthreads();
    for_each_vec<DT>(rowp, nvec, a.V, a.aligned, [&](const uint4 &v, int64_t gv) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float x = elem<DT>(v, e);
            if (x >= tau && x > -__builtin_inff()) {
                const uint32_t pos = atomicAdd(&s_n, 1u);
                if (pos < (uint32_t)kSparseKept) {
                    l_idx[pos] = (uint32_t)(gv * EPV + e);
                    l_x[pos] = x;
                }
            }
        }
    });
    __syncthreads();
    const uint32_t n = min(s_n, (uint32_t)kSparseKept);
    const uint64_t seed = a.seed[b];
    const uint64_t off0 = a.offset[b];
    const float invT = 1.0f / T;
    const uint32_t npairs = n * (uint32_t)K;
    for (uint32_t q = (uint32_t)tid; q < npairs; q += 1024u) {
        const uint32_t k = q / n, e = q - k * n;
        const uint32_t i = l_idx[e];
        const uint64_t off = off0 + (uint64_t)k;
        Stream st;
        st.row = (uint32_t)b;
        st.off_lo = (uint32_t)off;
        st.off_hi = (uint32_t)(off >> 32);
        st.key0 = (uint32_t)seed;
        st.key1 = (uint32_t)(seed >> 32);
        const uint32_t r = a.layout == LAY_SCREENED ? element_word<LAY_SCREENED>(st, i)
                                                    : element_word<LAY_PLAIN>(st, i);
        const float sc = l_x[e] * invT + gumbel32(r);
        atomicMax(reinterpret_cast<unsigned long long *>(&l_key[k]),
                  (unsigned long long)make_key(sc, i));
    }
    __syncthreads();
    for (int k = tid; k < K; k += 1024) {
        const uint64_t kk = l_key[k];
        a.out[b * K + k] = key_index(kk);
        if (a.best_out) a.best_out[b * K + k] = key_score(kk);
    }
    return true;
}

template <int DT>
__global__ __launch_bounds__(1024) void k_filter_tau(FilterArgs a) {
    __shared__ uint32_t hc[2048];
    __shared__ double hm[2048];
    __shared__ float red_f[16];
    __shared__ uint32_t red_n[16];
    __shared__ uint4 s_draw[2048];   // the draw of a small kept set
    const int64_t b = blockIdx.x;
    if (a.done != nullptr && threadIdx.x == 0) a.done[b] = 0u;   // set below if drawn here
    RowFilter f;
    if (!row_filter(a, b, &f)) return;
    const TauKept r = tau_radix<DT>(a, b, f, hc, hm, red_f, red_n);
    const float tau = r.tau;
    const uint32_t kept = r.kept;
    if (threadIdx.x == 0) a.tau[b * (a.tau_stride ? a.tau_stride : 1)] = tau;
    if (a.done == nullptr) return;
    constexpr int EPV = dtype_traits<DT>::epv;
    const char *rowp = reinterpret_cast<const char *>(a.data) + b * a.ld * dtype_traits<DT>::esize;
    if (draw_kept<DT>(a, b, f.T, tau, kept, rowp, (a.V + EPV - 1) / EPV,
                      reinterpret_cast<uint32_t *>(s_draw))) {
        if (threadIdx.x == 0) a.done[b] = 1u;
    }
}

template <int DT>
__global__ __launch_bounds__(1024) void k_filter_tau16(FilterArgs a) {
    using tr = dtype_traits<DT>;
    constexpr int EPV = tr::epv;
    __shared__ uint4 s_hist[8192];
    __shared__ uint32_t red_u[16];
    __shared__ double red_d[16];
    __shared__ float red_f[16];
    __shared__ int s_thr[3];
    __shared__ uint32_t s_above[2];
    __shared__ double s_above_m;
    __shared__ uint32_t s_rank[3];
    __shared__ uint32_t s_above_c, s_kept;   // count above the top-p crossing; kept tokens
    uint32_t *hist = reinterpret_cast<uint32_t *>(s_hist);

    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    if (a.done != nullptr && tid == 0) a.done[b] = 0u;   // set below if the row is drawn here
    RowFilter f;
    if (!row_filter(a, b, &f)) return;
    const char *rowp = reinterpret_cast<const char *>(a.data) + b * a.ld * tr::esize;
    const int64_t nvec = (a.V + EPV - 1) / EPV;

#pragma unroll
    for (int j = 0; j < 8; ++j) s_hist[tid + 1024 * j] = make_uint4(0u, 0u, 0u, 0u);
    if (tid < 3) s_thr[tid] = -1;
    __syncthreads();
    uint32_t nf = 0u;
    for_each_vec<DT>(rowp, nvec, a.V, a.aligned, [&](const uint4 &v, int64_t) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
            const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
            if (elem<DT>(v, e) > -__builtin_inff()) {   // NaN and -inf are not counted
                atomicAdd(&hist[h >> 1], (h & 1u) ? 0x10000u : 1u);
                ++nf;
            }
        }
    });
    __syncthreads();
    if (tid == 0) {   // -0 (pattern 0x8000, word 0x4000 low half) joins +0 (word 0 low half)
        const uint32_t neg0 = hist[0x4000] & 0xFFFFu;
        hist[0x4000] -= neg0;
        hist[0] += neg0;
    }
    const uint32_t NF = block_sum_u32(nf, red_u);

    // per-thread counts over the owned words (read in a lane-rotated order: no bank conflicts)
    const int base = owned_words(tid);
    uint32_t own = 0u;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
        const uint32_t w = hist[base + ((j + lane) & 31)];
        own += (w & 0xFFFFu) + (w >> 16);
    }
    uint32_t ex, in, total;
    block_scan(own, red_u, &ex, &in, &total);
    if (total != NF) {   // a counter overflowed: select by radix levels (LDS reused)
        const TauKept r = tau_radix<DT>(a, b, f, hist, reinterpret_cast<double *>(hist + 2048),
                                        red_f, red_u);
        const float tau = r.tau;
        const uint32_t kept = r.kept;
        if (tid == 0) a.tau[b * (a.tau_stride ? a.tau_stride : 1)] = tau;
        if (a.done != nullptr && draw_kept<DT>(a, b, f.T, tau, kept, rowp, nvec, hist)) {
            if (tid == 0) a.done[b] = 1u;
        }
        return;
    }
    if (NF == 0u) {
        if (tid == 0) a.tau[b * (a.tau_stride ? a.tau_stride : 1)] = -__builtin_inff();
        return;
    }
    const bool topk = f.k > 0 && (uint32_t)f.k < NF;
    if (ex < 1u && in >= 1u) s_thr[0] = tid;   // holds the largest logit
    if (topk && ex < (uint32_t)f.k && in >= (uint32_t)f.k) {
        s_thr[1] = tid;
        s_above[1] = ex;
    }
    __syncthreads();
    if (wid == 0) {
        auto cnt = [&](uint32_t r) { return hist_count(hist, rank_bits(r)); };
        uint32_t c1, kept = NF;
        const uint32_t rmax = resolve_rank<uint32_t>(s_thr[0], 0u, 1u, lane, cnt, &c1);
        const uint32_t rk = topk ? resolve_rank<uint32_t>(s_thr[1], s_above[1], (uint32_t)f.k,
                                                          lane, cnt, &kept)
                                 : 65535u;
        if (lane == 0) {
            s_rank[0] = rmax;
            s_rank[1] = rk;
            s_kept = kept;   // tokens at or above the top-k threshold
        }
    }
    __syncthreads();
    const float M = bits_value<DT>(rank_bits(s_rank[0]));
    const uint32_t rk = s_rank[1];
    float tau = topk ? bits_value<DT>(rank_bits(rk)) : -__builtin_inff();

    // top-p over the values top-k keeps (ranks <= rk): tempered mass count * 2^((x - M) c1),
    // fp32 terms summed in fp64
    if (f.p < 1.0f) {
        const float c1 = kLog2e / f.T;
        auto mass = [&](uint32_t r, uint32_t c) -> double {
            return (c > 0u && r <= rk)
                       ? (double)c * (double)__builtin_amdgcn_exp2f(
                                         (bits_value<DT>(rank_bits(r)) - M) * c1)
                       : 0.0;
        };
        const uint32_t rmax = s_rank[0];
        if (rk - rmax < 256u) {
            // every kept value lies fewer than 256 ranks below the largest (top-k keeps few
            // tokens): wave 0 alone scans ranks rmax .. rk, four consecutive ranks per lane
            if (wid == 0) {
                const uint32_t r0 = rmax + 4u * (uint32_t)lane;
                uint32_t c[4];
                double m[4];
                double own = 0.0;
                uint32_t ownc = 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t r = r0 + (uint32_t)j;
                    c[j] = r <= rk ? hist_count(hist, rank_bits(r)) : 0u;
                    m[j] = mass(r, c[j]);
                    own += m[j];
                    ownc += c[j];
                }
                double in = own;
                uint32_t inc = ownc;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const double o = __shfl_up(in, d, 64);
                    const uint32_t oc = __shfl_up(inc, d, 64);
                    if (lane >= d) {
                        in += o;
                        inc += oc;
                    }
                }
                double exm = __shfl_up(in, 1, 64);
                uint32_t exc = __shfl_up(inc, 1, 64);
                if (lane == 0) {
                    exm = 0.0;
                    exc = 0u;
                }
                const double P = (double)f.p * __shfl(in, 63, 64);
                // the crossing lane, or (a total that rounding left short) the last with mass
                const uint64_t hit = __ballot(in >= P);
                const uint64_t nz = __ballot(own > 0.0);
                const int l = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(nz | 1ull);
                if (lane == l) {
                    int jj = -1, last = 0;
                    double run = exm;
                    uint32_t cnt = exc, cnt_at = exc;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        run += m[j];
                        cnt += c[j];
                        if (m[j] > 0.0) last = j;
                        if (jj < 0 && hit && run >= P) {
                            jj = j;
                            cnt_at = cnt;
                        }
                    }
                    if (jj < 0) {
                        jj = last;
                        cnt_at = exc;
#pragma unroll
                        for (int j = 0; j < 4; ++j) cnt_at += j <= jj ? c[j] : 0u;
                    }
                    s_rank[2] = r0 + (uint32_t)jj;
                    s_kept = cnt_at;
                }
            }
            __syncthreads();
        } else {
            double own_m = 0.0;
            if (64u * (uint32_t)tid <= rk) {
                for (int j = 0; j < 32; ++j) {
                    const int wd = base + ((j + lane) & 31);
                    const uint32_t w = hist[wd];
                    if (w) {
                        own_m += mass(bits_rank(2u * (uint32_t)wd), w & 0xFFFFu);
                        own_m += mass(bits_rank(2u * (uint32_t)wd + 1u), w >> 16);
                    }
                }
            }
            double exm, inm, S;
            block_scan(own_m, red_d, &exm, &inm, &S);
            const double P = (double)f.p * S;
            if (exm < P && inm >= P) {
                s_thr[2] = tid;
                s_above_m = exm;
                s_above_c = ex;
            }
            __syncthreads();
            int tp = s_thr[2];
            double above = s_above_m;
            if (tp < 0) {   // rounding left the total short of P: the last thread with kept mass
                const uint64_t m = __ballot(own_m > 0.0);
                if (lane == 0) red_u[wid] = m ? (uint32_t)(64 * wid + 63 - __builtin_clzll(m)) : 0u;
                __syncthreads();
                tp = 0;
                for (int w = 0; w < 16; ++w) tp = max(tp, (int)red_u[w]);
                above = 0.0;
            }
            if (wid == 0) {
                double cm;
                const uint32_t rp = resolve_rank<double>(tp, above, P, lane, [&](uint32_t r) {
                    return mass(r, hist_count(hist, rank_bits(r)));
                }, &cm);
                // tokens at or above the top-p threshold (rp <= rk: masses stop at rk); unknown
                // when rounding left the total short
                const uint32_t base_r = rp & ~63u;
                const uint32_t kp = wave_prefix_at(hist_count(hist, rank_bits(base_r + lane)), lane,
                                                   (int)(rp - base_r));
                if (lane == 0) {
                    s_rank[2] = rp;
                    s_kept = s_thr[2] >= 0 ? s_above_c + kp : 0xFFFFFFFFu;
                }
            }
            __syncthreads();
        }
        tau = fmaxf(tau, bits_value<DT>(rank_bits(s_rank[2])));
    }
    if (tid == 0) a.tau[b * (a.tau_stride ? a.tau_stride : 1)] = tau;
    if (a.done == nullptr) return;

    // ---- a row that keeps few tokens is drawn here (its kept count comes from the selection
    // scans: the count down to tau's rank) ----
    if (draw_kept<DT>(a, b, f.T, tau, s_kept, rowp, nvec, hist)) {
        if (tid == 0) a.done[b] = 1u;
    }
}

}  // namespace

hipError_t launch_filter_tau(int dt, const FilterArgs &a, int grid, hipStream_t s) {
    switch (dt) {
        case DT_F32: hipLaunchKernelGGL(k_filter_tau<DT_F32>, dim3(grid), dim3(1024), 0, s, a); break;
        case DT_BF16: hipLaunchKernelGGL(k_filter_tau16<DT_BF16>, dim3(grid), dim3(1024), 0, s, a); break;
        case DT_F16: hipLaunchKernelGGL(k_filter_tau16<DT_F16>, dim3(grid), dim3(1024), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hs
