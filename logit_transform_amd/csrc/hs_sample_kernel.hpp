// hs_sample_kernel.hpp -- the sampling kernel of libhs (gfx950): batched HLG tone curve +
// Gumbel-max draws, its split-row pre-pass, and their launchers. Included by the translation
// units that instantiate them (hs_kernels.hip: given pivot and curve off; hs_kernels_pivot.hip:
// top- and entropy-anchored pivots; hs_kernels_rows.hip: the curve set per row).
//
// Sources, cited by page title and section:
//   [HLG]  "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document).
//   [GMX]  "Softmax-free GPU sampling: Gumbel-max categorical sampling kernel" (mlxcel #900).
//
// Work decomposition. A block owns one contiguous chunk of one row (the whole row when it
// fits) and one group of the row's draws. Lane t owns the 16-byte vectors t, t+BS, t+2BS, ...
// ("slots"), so every wave load is one contiguous 1 KiB. One streaming pass reads the chunk
// once: the first draw's random words run a few slots ahead of the logits, and per slot the
// pass keeps only summaries in LDS (the vector's largest logit as a bf16-grid upper bound, the
// top 16 bits of its largest word), the lane's running maximum and log-sum-exp, and the
// lane's "champion" vector (the one holding its largest word) in registers (chunks of at most
// 6 slots keep every slot's vector there). Rows split over
// several blocks combine their chunks' log-sum-exp partials either from a pre-pass or, when
// a row's blocks run together (the whole grid resident, or a resident grid taking items from
// a work queue), by exchanging them inside this kernel; the chunks' winning keys
// meet in a 64-bit atomic max, and the last block of each (row, draw group) writes the token
// ids and zeroes its workspace slots again.
//
// Screening. A draw's winner is the exact argmax over all elements, but the expensive part
// of an element's score (curve branches, two logarithms) is evaluated only when an upper
// bound on that score reaches a lower bound on the draw's winning score, less a slack:
//   score = l'/T + G(r) <= U(x) + (n(r) + 1) ln 2,
// where U(x) = (m/T) * max(x - c, -w) bounds g(x - c)/T (g lies below its mid line past the
// shoulder knot and below -m*w in the toe; a tangent of the shoulder tightens it near the
// top) and n(r), the leading ones of the word, bounds G (G(r) <= -log(1 - u) <= (n + 1) ln 2).
// A vector whose largest logit and largest word cannot reach the bound is skipped whole; the
// champion is scored from registers and the few other vectors that can are taken from the
// kept slots or read again, drawn again and tested element by element. The lower bound is the
// best exact score of the bootstrap candidates, each the element holding a champion's largest
// word: every lane's, ranked within its wave, or (chunks of 8 or more slots) one champion per
// 16 lanes, all drawn and scored by wave 0. The
// bounds are rigorous up to fp32 rounding, which the slack covers many times over, so the
// screened result equals the exhaustive one bit for bit (a test checks this).
#pragma once

#include <hip/hip_runtime.h>

#include "hs_device.hpp"
#include "hs_internal.hpp"

namespace hs {

__device__ __forceinline__ float screen_slack(float s) {
    return 1e-3f + 1e-5f * (fabsf(s) + 32.0f);
}

// A block-uniform float moved to a scalar register.
__device__ __forceinline__ float uniform(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Per-row constants of one block.
struct RowConst {
    float invT;      // 1 / T
    float c;         // LSE + mu (curve on)
    float mt;        // m / T
    float mtc;       // (m / T) * c
    float mtw;       // (m / T) * w
    Curve curve;
};

// The exact fp32 score of one finite element: l'/T + G(r) [GMX, Background], with
// l' = g(x - (LSE + mu)) when the curve is on [HLG, The transfer function]. Every kernel
// variant scores elements through this one function.
template <bool HLG>
__device__ __forceinline__ float exact_score_inl(float x, uint32_t word, const RowConst &rc) {
    float a;
    if constexpr (HLG) {
        a = hlg32(x - rc.c, rc.curve) * rc.invT;
    } else {
        a = x * rc.invT;
    }
    return a + gumbel32(word);
}

// The same function kept out of line for the rare candidate path, so that its code is not
// repeated at every vector of the unrolled screen.
template <bool HLG>
__device__ __noinline__ float exact_score(float x, uint32_t word, RowConst rc) {
    return exact_score_inl<HLG>(x, word, rc);
}


template <int DT>
__device__ __forceinline__ uint64_t greedy_vec(uint4 raw, uint32_t i0, uint64_t best) {
    constexpr int EPV = dtype_traits<DT>::epv;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
        const float x = elem<DT>(raw, e);
        if (x > -__builtin_inff()) best = umax64(best, make_key(x, i0 + (uint32_t)e));
    }
    return best;
}

// Largest of the EPV logits of a vector.
template <int EPV>
__device__ __forceinline__ float vec_max(const float (&x)[EPV]) {
    if constexpr (EPV == 8) {
        const float t = max3f(x[0], x[1], x[2]);
        const float u = max3f(x[3], x[4], x[5]);
        return max2f(max3f(x[6], x[7], t), u);
    } else {
        return max2f(max3f(x[0], x[1], x[2]), x[3]);
    }
}

// (all threads of a block) One chunk's (max, sum exp(x - max), sum exp(x - max) (x - max)),
// for rows split over several blocks, in natural units, written by thread 0 to *dst: each
// thread keeps a running maximum in base 2 and rescales its sums when it moves; the block
// combines them. The top anchor needs only the maximum, only the entropy anchor the third sum.
// The same code gives the split pre-pass and the in-kernel exchange, so a chunk's partial does
// not depend on which block computes it.
// (wave 0) A chunk's log-sum-exp partial from its waves' (reference, sum, u) in base 2 and
// their largest logits: (reference in nats, sum of 2^(x log2(e) - reference), u in nats, the
// chunk's largest logit); (-inf, 0, 0, max) when the chunk has no finite logit.
template <int PIV>
__device__ __forceinline__ float4 waves_to_partial(const float *red_m, const float *red_s,
                                                   const float *red_u, const float *red_x,
                                                   int lane, int nw) {
    constexpr bool ENT = PIV == 2 || PIV == 3;
    const float xb = wave_max(lane < nw ? red_x[lane] : -__builtin_inff());
    if constexpr (PIV == 1) {
        return make_float4(-__builtin_inff(), 0.0f, 0.0f, xb);
    } else {
        const float pm = lane < nw ? red_m[lane] : -3.402823466e38f;
        const float mb = wave_max(pm);
        const float sb_ = lane < nw ? __builtin_amdgcn_exp2f(pm - mb) : 0.0f;
        const float S = wave_sum(lane < nw ? red_s[lane] * sb_ : 0.0f);
        const float U = ENT ? wave_sum(lane < nw && red_s[lane] > 0.0f
                                           ? __builtin_fmaf(red_s[lane], pm - mb, red_u[lane]) * sb_
                                           : 0.0f)
                            : 0.0f;
        const bool fin = S > 0.0f;
        return make_float4(fin ? mb * kLn2 : -__builtin_inff(), fin ? S : 0.0f,
                           fin ? U * kLn2 : 0.0f, xb);
    }
}

template <int DT, int PIV>
__device__ __forceinline__ void chunk_partial(const SampleArgs &a, int64_t b, int chunk,
                                              float *red_m, float *red_s, float *red_u,
                                              float *red_x, float4 *dst) {
    using tr = dtype_traits<DT>;
    constexpr int EPV = tr::epv;
    constexpr bool ENT = PIV == 2 || PIV == 3;   // the entropy anchor's sum is needed
    const int64_t v0 = (int64_t)chunk * a.cv;
    const int64_t vend = min(a.nvec, v0 + a.cv);
    const char *rowp = reinterpret_cast<const char *>(a.data) + b * a.ld * tr::esize;
    float m = -3.402823466e38f, s = 0.0f, u = 0.0f;   // base 2: m a maximum of x log2(e)
    float mx = -__builtin_inff();                       // the chunk's largest logit
    for (int64_t gv = v0 + threadIdx.x; gv < vend; gv += blockDim.x) {
        const uint4 v = load_vec<DT>(rowp, gv, a.V, a.aligned);
        float xv[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) xv[e] = elem<DT>(v, e);
        mx = fmaxf(mx, vec_max<EPV>(xv));
        const float mv = vec_max<EPV>(xv) * kLog2e;
        if constexpr (PIV == 1) {
            m = fmaxf(m, mv);
        } else {
            if (mv > m) {
                const float sc = __builtin_amdgcn_exp2f(m - mv);
                if constexpr (ENT) u = __builtin_fmaf(s, m - mv, u) * sc;
                s *= sc;
                m = mv;
            }
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                float t = __builtin_fmaf(xv[e], kLog2e, -m);
                if constexpr (ENT) t = max2f(t, kExpFloor);
                const float p = __builtin_amdgcn_exp2f(t);
                s += p;
                if constexpr (ENT) u = __builtin_fmaf(p, t, u);
            }
        }
    }
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    const float mw = wave_max(m);
    const float sc = __builtin_amdgcn_exp2f(m - mw);
    const float sw = wave_sum(s * sc);
    const float uw = ENT ? wave_sum(s > 0.0f ? __builtin_fmaf(s, m - mw, u) * sc : 0.0f) : 0.0f;
    const float xw = wave_max(mx);
    if (lane == 0) {
        red_m[wid] = mw;
        red_s[wid] = sw;
        red_u[wid] = uw;
        red_x[wid] = xw;
    }
    __syncthreads();
    if (wid == 0) {
        const float4 r = waves_to_partial<PIV>(red_m, red_s, red_u, red_x, lane, nw);
        if (lane == 0) *dst = r;
    }
}

// PIV selects the curve's pivot [HLG, The pivot] (curve on only): 0 given per row,
// 1 top-anchored (mu = l_max - c: z = x - (x_max - c), no log-sum-exp needed),
// 2 entropy-anchored (mu = sum p l: z = x - E_p[x], one more accumulator),
// 3 set per row with the rest of the curve (a.row_curves): both sums are accumulated and each
// row picks its shift; a row with its curve off runs the curve as the identity (m = 1, no
// rolloff, c = 0), which scores x / T exactly as the curve-off kernel does.
// LAY selects the word layout of the random stream (LAY_PLAIN or LAY_SCREENED, see
// element_word): the pass draws only what the screen needs, the largest leading 16 bits of
// each vector's words, and the few vectors scored exactly draw their whole words.
// One work item: one chunk of one row and one group of its draws (item = (row * nkg + group)
// * nchunk + chunk). Every thread of the block calls it with the same item.
template <int DT, int NV, bool HLG, int PIV, int MAXBS, bool ALIGNED, int LAY>
__device__ __forceinline__ void sample_item(const SampleArgs &a, int item) {
    static_assert(HLG || PIV == 0, "a pivot needs the curve");
    constexpr bool LSE = HLG && PIV != 1 && PIV != 4;   // the exponential sum is needed
    constexpr bool ENT = PIV == 2 || PIV == 3;   // and the entropy anchor's sum
    using tr = dtype_traits<DT>;
    constexpr int EPV = tr::epv;
    constexpr int NG = EPV / 4;                // Philox calls per vector
    // loads in flight per lane, and slots of random words ahead of the logits (measured on
    // MI355X: more loads in flight than 6 lengthen the pass, the words gain from a long lead)
    constexpr int D = NV < 6 ? NV : 6;
    constexpr int LAG = NV < 11 ? NV - 1 : 10;
    // Chunks of few slots keep every slot's vector in registers from the pass on, so that the
    // vectors that pass the screen (and later draws' champions) need no second read: a read
    // after the pass costs a whole memory round trip on the block's critical path.
    constexpr bool KEEP = NV <= 6;
    // The first draw's bootstrap candidates: chunks of many slots (1024-thread blocks whose
    // post-pass is bound by instruction issue) post their champions for wave 0 to draw and
    // score; small chunks (latency-bound) draw and rank them in every wave instead, which
    // keeps wave 0's serial work short.
    constexpr bool BOOT0 = NV >= 8;
    // The same for the later draws of a block, where it adds a barrier and wave 0's serial
    // work to every draw: only chunks of 12 or more slots gain (1024 x 262144 fp32 with 16
    // draws: -1.2%; 1 x 32768 fp32 with 4 draws per block, 8 slots: +4%).
    constexpr bool BOOTK = NV >= 12;
    // Dynamic LDS, one dword per lane and slot: the vector's largest logit as a bf16-grid upper
    // bound in the low half (draw-invariant) and the high 16 bits of its largest random word of
    // the current draw in the high half. Each lane's entries are contiguous (odd stride: lanes
    // hit distinct banks), so every access is one base register plus an immediate offset.
    extern __shared__ uint32_t s_vec[];
    __shared__ float red_m[16], red_s[16], red_u[16], red_x[16];
    // the first draw's bootstrap candidates: with BOOT0 one per group of 16 lanes (the champion
    // vector, its key (0: none) and the thread that holds it), else one per wave (its key, 0:
    // none, logit and the Gumbel value of its word)
    __shared__ uint4 s_cv[64];
    __shared__ uint32_t s_ck[64];
    __shared__ int32_t s_ct[64];
    __shared__ uint64_t red_ck[16];
    __shared__ float red_cx[16];
    __shared__ float red_cg[16];
    __shared__ __align__(16) float row_bc[13];   // row constants from wave 0
    // per wave, the best exact candidate score of a later draw; two buffers, alternating
    // between draws (a wave may post draw k + 1's before a slower one has read draw k's)
    __shared__ float red_sb[2][16];
    // the block's best key of each draw of a batch of up to 64, by LDS atomic maxima; wave 0
    // writes a batch out after one barrier
    __shared__ uint64_t s_best[64];
    // split rows with the partials exchanged in the kernel: every chunk's partial, and the
    // chunks whose partial did not arrive in time
    __shared__ float4 s_part[kMaxChunks];
    __shared__ float red_xp[16];       // per wave: largest logit of a replayed chunk
    __shared__ uint64_t s_miss;
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int BS = blockDim.x;
    constexpr int SC = NV | 1;
    uint16_t *s_vec16 = reinterpret_cast<uint16_t *>(s_vec);
    int lane_lds = tid * SC;
    if (tid < 64) s_best[tid] = 0ull;   // visible to every wave after the combine's barrier
    // item coordinates in scalar registers (the divisions would otherwise run per lane)
    int bid = item;
    const int chunk = __builtin_amdgcn_readfirstlane(bid % a.nchunk);
    bid /= a.nchunk;
    const int kg = __builtin_amdgcn_readfirstlane(bid % a.nkg);
    const int64_t b = __builtin_amdgcn_readfirstlane(bid / a.nkg);
    const int k0 = kg * a.kpg;
    const int k1 = min(a.K, k0 + a.kpg);
    // a filtered row whose few kept tokens the threshold kernel has drawn already
    if (a.done != nullptr && a.done[b] != 0u) return;

    // ---- row parameters (wave-uniform) ----
    const float T = a.T[b];
    float mu = 0.0f;
    bool bad = !temp_valid(T);
    Curve cv = a.curve;
    float poff = a.pivot_offset;
    int rpiv = PIV;   // this row's pivot mode; -1: curve off
    if constexpr (HLG && PIV == 0) {
        mu = a.mu[b];
        bad = bad || !(fabsf(mu) < __builtin_inff());
    }
    if constexpr (PIV == 3) {
        const RowCurve r = a.row_curves[b];
        const bool fin_m = r.m > 0.0f && r.m < __builtin_inff();
        const bool fin_t = r.beta_t > 0.0f && r.beta_t < __builtin_inff();
        const bool fin_h = r.beta_h > 0.0f && r.beta_h < __builtin_inff();
        // (a median row needs the shifts worked out before this kernel: a.shift)
        const bool valid = fin_m && r.w >= 0.0f && fin_t && fin_h && r.pivot >= 0 &&
                           r.pivot <= 3 && (r.pivot != 1 || fabsf(r.pivot_offset) < __builtin_inff()) &&
                           (r.pivot != 3 || a.shift != nullptr) && r.reserved == 0;
        const bool on = r.enabled != 0 && valid;
        if (r.enabled != 0 && !valid) bad = true;
        if (on) {
            // the same constants the host derives for a per-call curve (IEEE division)
            cv.m = r.m;
            cv.w = r.w;
            cv.mw = r.m * r.w;
            cv.mbt = r.m * r.beta_t;
            cv.mbh = r.m * r.beta_h;
            cv.ibt = 1.0f / r.beta_t;
            cv.ibh = 1.0f / r.beta_h;
            rpiv = r.pivot == 3 ? 4 : r.pivot;   // 4: the shift read per row (mass median)
            poff = r.pivot_offset;
            if (rpiv == 0) {
                mu = a.mu ? a.mu[b] : __builtin_nanf("");
                bad = bad || !(fabsf(mu) < __builtin_inff());
            }
        } else {
            cv.m = 1.0f;
            cv.w = __builtin_inff();
            cv.mw = __builtin_inff();
            cv.mbt = cv.mbh = cv.ibt = cv.ibh = 1.0f;
            rpiv = -1;
        }
    }
    // top-k / top-p (curve off): tokens below the row's threshold are not candidates; a NaN
    // threshold marks an invalid filter parameter
    float tau_row = -__builtin_inff();
    if constexpr (!HLG) {
        if (a.tau) {
            tau_row = a.tau[b];
            bad = bad || !(tau_row == tau_row);
        }
    }
    const bool greedy = (T == 0.0f);

    // ---- this block's chunk of the row: lane t owns vectors v0 + t + n*BS, n < NV ----
    const int v0 = chunk * (int)a.cv;
    const int vend = (int)min(a.nvec, (int64_t)v0 + a.cv);
    const int nfull = (int)(a.V / EPV);   // vectors with all EPV elements inside the row
    const int vlim = min(vend, nfull);    // vectors below this one load whole
    const char *rowp = reinterpret_cast<const char *>(a.data) + b * a.ld * tr::esize;
    int lane_v = v0 + tid;
    // the last vector index of this wave at slot 0 (wave-uniform)
    const int wave_last = __builtin_amdgcn_readfirstlane(v0 + (tid | 63));
    const uint4 ninf4 = make_uint4(tr::neg_inf_word, tr::neg_inf_word, tr::neg_inf_word,
                                   tr::neg_inf_word);

    // Vector gv of the chunk; -inf past the chunk or the row.
    auto fetch = [&](int gv) -> uint4 {
        if (gv >= vend) return ninf4;
        return load_vec<DT>(rowp, gv, a.V, ALIGNED);
    };
    // ALIGNED: slot n's load carries no branch (a lane past the chunk's whole vectors reads
    // zeros, see issue_load) and is patched when its data is used, with selects only: a load
    // inside the pipelined pass would make the compiler wait for every load in flight. The
    // row's partial last vector (V not a multiple of EPV) is read element by element up front
    // by every lane, with clamped addresses (one cache line, no branch); only waves that reach
    // past vlim at slot n test per lane.
    uint4 rag = ninf4;
    if constexpr (ALIGNED) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = tr::neg_inf_word;
        const int64_t i0 = (int64_t)nfull * EPV;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const int64_t i = min(i0 + e, a.V - 1);
            uint32_t h;
            if constexpr (DT == DT_F32) {
                h = reinterpret_cast<const uint32_t *>(rowp)[i];
            } else {
                h = reinterpret_cast<const uint16_t *>(rowp)[i];
            }
            if (i0 + e < a.V) {
                if constexpr (DT == DT_F32) {
                    w[e] = h;
                } else {
                    const int j = e >> 1;
                    w[j] = (e & 1) ? ((w[j] & 0x0000FFFFu) | (h << 16))
                                   : ((w[j] & 0xFFFF0000u) | h);
                }
            }
        }
        rag = make_uint4(w[0], w[1], w[2], w[3]);
    }
    // The streaming pass reads every vector once: its loads carry the non-temporal hint (on
    // MI355X a row-per-block read of the 256 x 151936 bf16 shape runs at ~75% of the HBM peak
    // with it, ~65% without). They are buffer loads through one resource that spans the
    // chunk's whole vectors: a lane past them reads zeros without touching memory (its vector
    // is patched before use), so no lane clamps its offset.
    const uint32_t lane16 = (uint32_t)tid * 16u;
    const __amdgpu_buffer_rsrc_t chunk_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(rowp + (uint32_t)min(v0, vlim) * 16u), (short)0,
        max(0, vlim - v0) * 16, kBufferWord3);
    auto issue_load = [&](int n) -> uint4 {
        if constexpr (ALIGNED) {
            typedef unsigned int u4v __attribute__((ext_vector_type(4)));
            const u4v t = __builtin_amdgcn_raw_buffer_load_b128(
                chunk_rsrc, lane16 + (uint32_t)(n * BS) * 16u, 0, kCachePolicyNT);
            return make_uint4(t.x, t.y, t.z, t.w);
        } else {
            return fetch(lane_v + n * BS);
        }
    };
    auto patch = [&](int n, uint4 v) -> uint4 {
        if constexpr (ALIGNED) {
            if (wave_last + n * BS >= vlim) {
                const int gv = lane_v + n * BS;
                const bool past = gv >= vend;
                const bool part = gv >= nfull;
                v.x = past ? ninf4.x : part ? rag.x : v.x;
                v.y = past ? ninf4.y : part ? rag.y : v.y;
                v.z = past ? ninf4.z : part ? rag.z : v.z;
                v.w = past ? ninf4.w : part ? rag.w : v.w;
            }
        }
        return v;
    };

    const uint64_t seed = a.seed[b];
    const uint64_t off0 = a.offset[b];
    Stream st;
    st.row = (uint32_t)b;
    st.key0 = (uint32_t)seed;
    st.key1 = (uint32_t)(seed >> 32);
    auto stream_k = [&](int k) {
        const uint64_t off = off0 + (uint64_t)k;
        Stream sk = st;
        sk.off_lo = (uint32_t)off;
        sk.off_hi = (uint32_t)(off >> 32);
        return sk;
    };

    // Random words of slot n for draw stream sk: the largest leading 16 bits of the vector's
    // words go to the slot's LDS dword (high half); returns the slot's key for the lane's
    // champion: those bits (and, in the plain layout, the next 11) over the slot index. Slots
    // past the chunk are drawn too (their words are never used).
    // Screened layout: one call (counter word 2q of the vector's group q) holds the leading
    // halves of the group's eight elements; an fp32 vector is half a group (elements 4h ..
    // 4h + 3, h = gv & 1, the same for every slot of a lane since BS is even).
    auto draw_vec = [&](const Stream &sk, int n) -> uint32_t {
        uint32_t code, key;
        if constexpr (LAY == LAY_PLAIN) {
            // counter word (lane_v + n BS) NG: the lane's part, and the slot's (uniform) part
            uint32_t ql = (uint32_t)lane_v * NG;
            asm volatile("" : "+v"(ql));
            const uint32_t dq = (uint32_t)(n * BS * NG);
            uint32_t mw;
            const Words4 w = philox4x32_10_lane(ql, dq, sk.row, sk.off_lo, sk.off_hi, sk.key0,
                                                sk.key1);
            mw = max(max3u(w.w[0], w.w[1], w.w[2]), w.w[3]);
            if constexpr (NG == 2) {
                const Words4 u = philox4x32_10_lane(ql, dq + 1u, sk.row, sk.off_lo, sk.off_hi,
                                                    sk.key0, sk.key1);
                mw = max3u(max3u(w.w[0], w.w[1], w.w[2]), max3u(w.w[3], u.w[0], u.w[1]),
                           max(u.w[2], u.w[3]));
            }
            code = mw >> 16;
            key = (mw & ~31u) | (uint32_t)n;
        } else {
            // counter word 2q of the group q of vector gv = lane_v + n BS: 2 gv for eight
            // elements per vector, gv rounded down to even for four (BS is even, so the
            // rounding is the lane's own: lane_v & ~1, plus the slot's n BS)
            uint32_t ql = EPV == 8 ? (uint32_t)lane_v << 1 : (uint32_t)lane_v & ~1u;
            asm volatile("" : "+v"(ql));
            const uint32_t dq = EPV == 8 ? (uint32_t)(2 * n * BS) : (uint32_t)(n * BS);
            const Words4 w = philox4x32_10_lane(ql, dq, sk.row, sk.off_lo, sk.off_hi, sk.key0,
                                                sk.key1);
            if constexpr (EPV == 8) {
                code = max_half16(max_half16_pk(w.w[0], w.w[1]), max_half16_pk(w.w[2], w.w[3]));
            } else {
                const bool h = ((uint32_t)lane_v & 1u) != 0u;
                code = max_half16(h ? w.w[2] : w.w[0], h ? w.w[3] : w.w[1]);
            }
            key = (code << 16) | (uint32_t)n;
        }
        s_vec16[2 * (lane_lds + n) + 1] = (uint16_t)code;
        return key;
    };
    // Whole words of the vector gv for stream sk (the bootstrap candidate and the vectors
    // scored exactly): element e's word into w[e].
    auto vec_words = [&](const Stream &sk, int gvi, uint32_t (&w)[EPV]) {
        if constexpr (LAY == LAY_PLAIN) {
            uint32_t q = (uint32_t)gvi * NG;
            asm volatile("" : "+v"(q));
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const Words4 ww = philox4x32_10_uk(q + g, sk.row, sk.off_lo, sk.off_hi, sk.key0,
                                                   sk.key1);
#pragma unroll
                for (int e = 0; e < 4; ++e) w[4 * g + e] = ww.w[e];
            }
        } else {
            const uint32_t gv = (uint32_t)gvi;
            uint32_t q2 = EPV == 8 ? gv << 1 : gv & ~1u;
            asm volatile("" : "+v"(q2));
            const Words4 hi = philox4x32_10_uk(q2, sk.row, sk.off_lo, sk.off_hi, sk.key0, sk.key1);
            const Words4 lo = philox4x32_10_uk(q2 | 1u, sk.row, sk.off_lo, sk.off_hi, sk.key0,
                                               sk.key1);
            if constexpr (EPV == 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = (half16(hi, e) << 16) | half16(lo, e);
            } else {
                const bool h = (gv & 1u) != 0u;
                const uint32_t h0 = h ? hi.w[2] : hi.w[0], h1 = h ? hi.w[3] : hi.w[1];
                const uint32_t l0 = h ? lo.w[2] : lo.w[0], l1 = h ? lo.w[3] : lo.w[1];
                w[0] = (h0 << 16) | (l0 & 0xFFFFu);
                w[1] = (h0 & 0xFFFF0000u) | (l0 >> 16);
                w[2] = (h1 << 16) | (l1 & 0xFFFFu);
                w[3] = (h1 & 0xFFFF0000u) | (l1 >> 16);
            }
        }
    };
    // the bits of a word that the champion key holds: (w ^ key) <= kMatch when they agree
    constexpr uint32_t kMatch = LAY == LAY_PLAIN ? 31u : 0xFFFFu;
    // Screened layout with four elements per vector: the two lanes whose vectors make up a group
    // (lanes 2j and 2j + 1: a chunk starts at an even vector and BS is even) take turns, so each
    // lane makes one call per two slots. For the slot pair (n, n + 1) the even lane draws the
    // group of its slot n and the odd lane that of its slot n + 1; each keeps the half of the
    // call that is its own and passes the other half's largest code to its neighbour (one DPP
    // swap). Returns the keys of slots n and n + 1 (the second unused past the last slot).
    constexpr bool PAIR = LAY == LAY_SCREENED && EPV == 4;
    auto draw_pair = [&](const Stream &sk, int n, uint32_t &key0, uint32_t &key1) {
        const uint32_t p = (uint32_t)lane_v & 1u;
        uint32_t ql = ((uint32_t)lane_v & ~1u) + p * (uint32_t)BS;
        asm volatile("" : "+v"(ql));
        const Words4 w = philox4x32_10_lane(ql, (uint32_t)(n * BS), sk.row, sk.off_lo,
                                            sk.off_hi, sk.key0, sk.key1);
        const uint32_t mlo = max_half16(w.w[0], w.w[1]);   // elements 0..3: the even vector
        const uint32_t mhi = max_half16(w.w[2], w.w[3]);   // elements 4..7: the odd vector
        const uint32_t keep = p ? mhi : mlo;
        const uint32_t recv = dpp_u32<kDppQuad1032>(p ? mlo : mhi);
        const uint32_t c0 = p ? recv : keep;   // slot n
        const uint32_t c1 = p ? keep : recv;   // slot n + 1
        s_vec16[2 * (lane_lds + n) + 1] = (uint16_t)c0;
        if (n + 1 < NV) s_vec16[2 * (lane_lds + n + 1) + 1] = (uint16_t)c1;
        key0 = (c0 << 16) | (uint32_t)n;
        key1 = (c1 << 16) | (uint32_t)(n + 1);
    };
    // The lane's champion key over a whole draw (draws without the logits at hand).
    auto draw_all = [&](const Stream &sk) -> uint32_t {
        uint32_t champ = 0;
        if constexpr (PAIR) {
#pragma unroll
            for (int n = 0; n < NV; n += 2) {
                uint32_t ka, kb;
                draw_pair(sk, n, ka, kb);
                champ = n + 1 < NV ? max3u(champ, ka, kb) : max(champ, ka);
                asm volatile("" : "+v"(champ));
            }
        } else {
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                champ = max(champ, draw_vec(sk, n));
                // one running maximum: otherwise the compiler regroups the chain of maxima and
                // keeps every slot's word alive until the end of the pass
                asm volatile("" : "+v"(champ));
            }
        }
        return champ;
    };

    // Slot n's logits: the vector's largest logit (rounded up to the bf16 grid for f32/f16
    // input, so it stays an upper bound) into the low half of its LDS dword, the lane's largest
    // logit, and with the curve on the log-sum-exp of the row [HLG, The transfer function:
    // l = x - LSE(x)], streamed per lane in base 2 against a fixed reference r, the scaled
    // maximum of the lane's first vector: s = sum 2^(x log2(e) - r). Lanes whose largest logit
    // ends up far from r (where the sum could overflow or lose its terms) sum again against
    // their own maximum after the pass.
    // With the entropy anchor also u = sum 2^t t, t = x log2(e) - r, for E_p[x].
    float xmax_lane = -__builtin_inff();
    float lse_r = 0.0f, lse_s = 0.0f, lse_u = 0.0f;
    auto data_vec = [&](int n, uint4 v) {
        // Keep the slots in order: otherwise the scheduler issues the exponentials of many
        // vectors first and holds all their results at once.
        asm volatile("" : "+v"(lse_s), "+v"(xmax_lane), "+v"(lse_u));
        float xv[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) xv[e] = elem<DT>(v, e);
        const float m = vec_max<EPV>(xv);
        xmax_lane = max2f(xmax_lane, m);
        uint32_t mb = __float_as_uint(m);
        if constexpr (DT != DT_BF16) {
            // toward +inf on the bf16 grid: positive values round up, negative ones truncate
            mb = ((int32_t)mb >= 0) ? mb + 0xFFFFu : mb;
        }
        s_vec16[2 * (lane_lds + n)] = (uint16_t)(mb >> 16);
        if constexpr (LSE) {
            if (n == 0) lse_r = (m > -__builtin_inff()) ? m * kLog2e : 0.0f;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                float t = __builtin_fmaf(xv[e], kLog2e, -lse_r);
                if constexpr (ENT) t = max2f(t, kExpFloor);
                const float p = __builtin_amdgcn_exp2f(t);
                lse_s += p;
                if constexpr (ENT) lse_u = __builtin_fmaf(p, t, lse_u);
            }
        }
    };

    const bool sampled = !bad && !greedy;
    const bool screen = sampled && !a.no_screen;
    const float invT = 1.0f / T;
    // Linear part of the score used to rank bootstrap candidates before c = LSE + mu is known:
    // (m/T) x with the curve on (the mid line of g, up to the common shift -(m/T) c), x/T
    // without it.
    const float lin = HLG ? cv.m * invT : invT;
    // Bootstrap candidate of a lane for draw stream sk: the element holding the largest word of
    // its champion vector v (nearly the largest Gumbel value among the lane's elements; in the
    // screened layout the largest leading half, the first element of a tie). The vector's whole
    // words are drawn again into cw and kept for the screen: in the screened layout its two
    // calls are independent, so they overlap, and a champion that passes the screen needs no
    // further call. Returns the candidate's rank key (lin x - log(1 - u) -- a monotone
    // stand-in for the Gumbel value, close to it where u is near 1 -- and the lane) and its
    // logit and word.
    struct Cand {
        uint64_t key;
        float x;
        uint32_t w;
    };
    // (have_words: cw holds the champion's words already)
    auto candidate = [&](const Stream &sk, uint32_t champ, const uint4 &v, uint32_t (&cw)[EPV],
                         bool have_words = false) -> Cand {
        Cand c{0ull, -__builtin_inff(), 0u};
        if (!have_words) vec_words(sk, lane_v + (int)(champ & 31u) * BS, cw);
#pragma unroll
        for (int e = EPV - 1; e >= 0; --e) {
            if ((cw[e] ^ champ) <= kMatch) {
                c.w = cw[e];
                c.x = elem<DT>(v, e);
            }
        }
        const float nlv = __builtin_amdgcn_logf(__builtin_fmaf((float)(~c.w), 0x1p-32f, 0x1p-33f));
        const bool ok = c.x > -__builtin_inff() && (HLG || c.x >= tau_row) &&
                        lane_v + (int)(champ & 31u) * BS < vend;
        c.key = ok ? make_key(__builtin_fmaf(c.x, lin, -nlv * kLn2), (uint32_t)tid) : 0ull;
        return c;
    };

    // ---- one pass over the chunk: the first draw's random words (which need no logit) run
    // LAG slots ahead of the logits, so the first loads land while they are computed; D loads
    // stay in flight. The lane's champion (its slot with the largest word) follows from the
    // draws alone; its vector stays in registers (long chunks) or is taken from the kept slots
    // (short ones), and its words are drawn again: after the pass, or in short chunks as soon
    // as the last slot is drawn, while the loads are in flight. The pass is the same
    // for every row (greedy and invalid rows draw words they never use):
    // without row-dependent branches the scheduler interleaves the integer Philox chains with
    // the float work freely. ----
    uint32_t champ0 = 0;
    uint4 craw0 = ninf4;
    uint32_t cw0[EPV];   // the champion vector's words
    uint4 keep[KEEP ? NV : 1];
    // Slot n's vector again (n lane-varying): selected from the kept registers, or read.
    auto slot_vec = [&](int n) -> uint4 {
        if constexpr (KEEP) {
            uint4 v = keep[0];
#pragma unroll
            for (int j = 1; j < NV; ++j) {
                const bool h = n == j;
                v.x = h ? keep[j].x : v.x;
                v.y = h ? keep[j].y : v.y;
                v.z = h ? keep[j].z : v.z;
                v.w = h ? keep[j].w : v.w;
            }
            return v;
        } else {
            return fetch(lane_v + n * BS);
        }
    };
    {
        const Stream sk = stream_k(k0);
        uint4 buf[D];   // loads in flight
        // long chunks: slot keys between a slot's draw and its logits, and the champion's
        // vector selected as the logits come in; short chunks take it from the kept slots
        // after the pass, so their champion is just the largest key (it needs no logit)
        constexpr int RING = KEEP ? 1 : LAG + 2;
        uint32_t ring[RING];
#pragma unroll
        for (int n = 0; n < D; ++n) buf[n] = issue_load(n);
#pragma unroll
        for (int n = 0; n < NV + LAG; ++n) {
            if constexpr (PAIR) {
                if (n < NV && (n & 1) == 0) {
                    if constexpr (KEEP) {
                        uint32_t ka, kb;
                        draw_pair(sk, n, ka, kb);
                        champ0 = n + 1 < NV ? max3u(champ0, ka, kb) : max(champ0, ka);
                        asm volatile("" : "+v"(champ0));
                    } else {
                        draw_pair(sk, n, ring[n % RING], ring[(n + 1) % RING]);
                    }
                }
            } else {
                if (n < NV) {
                    if constexpr (KEEP) {
                        champ0 = max(champ0, draw_vec(sk, n));
                        asm volatile("" : "+v"(champ0));
                    } else {
                        ring[n % RING] = draw_vec(sk, n);
                    }
                }
            }
            if constexpr (KEEP) {
                if (n == NV - 1) vec_words(sk, lane_v + (int)(champ0 & 31u) * BS, cw0);
            }
            const int j = n - LAG;
            if (j >= 0 && j < NV) {
                const uint4 v = patch(j, buf[j % D]);
                data_vec(j, v);
                if constexpr (KEEP) {
                    keep[j] = v;
                } else {
                    // the champion's vector stays in registers (no second read: reading it
                    // again once the last slot is drawn costs more than these selects)
                    const uint32_t kj = ring[j % RING];
                    if (kj > champ0) {
                        champ0 = kj;
                        craw0 = v;
                    }
                }
                if (j + D < NV) buf[j % D] = issue_load(j + D);
            }
        }
        if constexpr (KEEP) craw0 = slot_vec((int)(champ0 & 31u));
    }
    if constexpr (LSE) {
        // A lane whose largest logit lies more than 100 binary orders above or below its
        // reference (never for logits of ordinary range) sums again against that maximum.
        const float tm = xmax_lane * kLog2e;
        if (xmax_lane > -__builtin_inff() && !(fabsf(tm - lse_r) <= 100.0f)) {
            lse_r = tm;
            lse_s = 0.0f;
            lse_u = 0.0f;
            for (int n = 0; n < NV; ++n) {
                const uint4 v = fetch(lane_v + n * BS);
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    float t = __builtin_fmaf(elem<DT>(v, e), kLog2e, -lse_r);
                    if constexpr (ENT) t = max2f(t, kExpFloor);
                    const float p = __builtin_amdgcn_exp2f(t);
                    lse_s += p;
                    if constexpr (ENT) lse_u = __builtin_fmaf(p, t, lse_u);
                }
            }
        }
    }

    // ---- block combine: log-sum-exp (curve on), the largest logit, and the first draw's
    // bootstrap candidate; wave 0 turns them into the row's constants, which reach every wave
    // through LDS ----
    RowConst rc;
    rc.invT = invT;
    rc.c = 0.0f;
    rc.mt = rc.mtc = rc.mtw = 0.0f;
    rc.curve = cv;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    int wid = threadIdx.x >> 6;
    asm volatile("" : "+v"(wid));
    const int nw = (BS + 63) >> 6;
    // The first draw's bootstrap with BOOT0, without drawing words in every wave: each group of
    // 16 lanes posts the champion of its best-ranked lane, ranked by lin xm - log(1 - u) with
    // xm the champion vector's largest logit (its LDS summary) and u the middle of the interval
    // its code leaves for the largest word. Wave 0 then draws the posted vectors' words, one
    // candidate per lane, and scores them (at the latency of one).
    auto post_champion = [&](uint32_t champ, const uint4 &cvec) {
        uint64_t rk = 0ull;
        if (champ != 0u) {
            const uint32_t d = s_vec[lane_lds + (int)(champ & 31u)];
            const float xm = __uint_as_float(d << 16);
            const float v1u = __builtin_fmaf((float)(0xFFFFu - (d >> 16)), 0x1p-16f, 0x1p-17f);
            const float r = __builtin_fmaf(xm, lin, -__builtin_amdgcn_logf(v1u) * kLn2);
            if (xm > -__builtin_inff() && (HLG || xm >= tau_row)) rk = make_key(r, (uint32_t)tid);
        }
        const uint64_t gk = row_max_u64(rk);
        const int j = (wid << 2) | (lane >> 4);
        if (gk != 0ull && rk == gk) {
            s_cv[j] = cvec;
            s_ck[j] = champ;
            s_ct[j] = tid;
        } else if (gk == 0ull && (lane & 15) == 0) {
            s_ck[j] = 0u;
        }
    };
    // Without BOOT0: each wave's best candidate by its exact rank key, with the logit and the
    // Gumbel value of its word (which needs no row constant, so each wave works it out before
    // the block combine).
    // (Every lane's Gumbel value is formed before the reduction, so the two overlap.)
    auto post_candidate = [&](const Cand &c) {
        const float g = gumbel32(c.w);
        const uint64_t wk = wave_max_u64(c.key);
        if (lane == 0) red_ck[wid] = wk;
        if (wk != 0 && c.key == wk) {
            red_cx[wid] = c.x;
            red_cg[wid] = g;
        }
    };
    // (wave 0, BOOT0) Lane j's candidate from group j: the element of the posted vector whose
    // word the champion key matches, its logit and the Gumbel value of its word (no row
    // constant needed, so this overlaps the block combine).
    float cand_x = -__builtin_inff(), cand_g = 0.0f;
    auto take_candidate = [&](const Stream &sk) {
        cand_x = -__builtin_inff();
        cand_g = 0.0f;
        const uint32_t ck = lane < 4 * nw ? s_ck[lane] : 0u;
        if (ck != 0u) {
            const uint4 v = s_cv[lane];
            const int gv = v0 + s_ct[lane] + (int)(ck & 31u) * BS;
            uint32_t w[EPV];
            vec_words(sk, gv, w);
            float x = -__builtin_inff();
            uint32_t we = 0u;
#pragma unroll
            for (int e = EPV - 1; e >= 0; --e) {
                if ((w[e] ^ ck) <= kMatch) {
                    we = w[e];
                    x = elem<DT>(v, e);
                }
            }
            if (x > -__builtin_inff() && (HLG || x >= tau_row) && gv < vend) {
                cand_x = x;
                cand_g = gumbel32(we);
            }
        }
    };
    // (wave 0) The best score among the bootstrap candidates, l'/T + G as exact_score_inl
    // forms it (without BOOT0 lane w scores wave w's).
    auto candidate_score = [&]() -> float {
        if constexpr (!BOOT0) {
            if (lane < nw && red_ck[lane] != 0ull) {
                cand_x = red_cx[lane];
                cand_g = red_cg[lane];
            }
        }
        float cs = -__builtin_inff();
        if (cand_x > -__builtin_inff()) {
            float a;
            if constexpr (HLG) {
                a = hlg32(cand_x - rc.c, rc.curve) * rc.invT;
            } else {
                a = cand_x * rc.invT;
            }
            cs = a + cand_g;
        }
        return uniform(wave_max(cs));
    };
    // Rows whose scores come near the fp32 range (a temperature of ~1e-38) can overflow the
    // screen's constants: then the screen is switched off for the row (every vector passes
    // and every element is scored exactly), which is always correct.
    auto screen_guard = [](float &sa_, float &sb_, float &sc_, float &ta_, float &tb_) {
        const float lim = 1.0e38f;
        if (fabsf(sa_) < lim && fabsf(sb_) < lim && fabsf(ta_) < lim && fabsf(tb_) < lim &&
            !(sc_ != sc_))
            return;
        sa_ = ta_ = 0.0f;
        sb_ = tb_ = -3.0e38f;
        sc_ = __builtin_inff();
    };
    // (wave 0) The screen's constants from a lower bound bs on the draw's winning score:
    // threshold thr = (bs - slack) / ln 2 - 1 in units of ln 2, and the coefficients with which
    //   need(x) = min(max(x sa + sb, x ta + tb), sc)
    // is the smallest word code n (leading ones) that lets a logit x reach it:
    // thr - U(x) / ln 2, U(x) an upper bound on l'(x)/T. With the curve on,
    //   U(x) = max(min(mid(x), tan(x)), -(m/T) w),
    // where mid(x) = (m/T)(x - c) is the mid line (above the shoulder), tan the tangent of the
    // concave shoulder at the chunk's largest logit (above the shoulder, and above the mid line
    // left of the knot), and -(m/T) w the top of the toe; without the curve U(x) = x/T.
    // No bound (no screening): every vector passes.
    auto screen_consts = [&](float bs, float xtop, float *o) {
        // (a bound that overflowed to +inf screens nothing out)
        float thr = -3.0e38f;
        if (bs > -__builtin_inff() && bs < __builtin_inff())
            thr = (bs - screen_slack(bs)) * kInvLn2 - 1.0f;
        o[0] = thr;
        if constexpr (HLG) {
            o[1] = -rc.mt * kInvLn2;
            o[2] = __builtin_fmaf(rc.mtc, kInvLn2, thr);
            o[3] = __builtin_fmaf(rc.mtw, kInvLn2, thr);
            o[4] = o[1];
            o[5] = o[2];
            o[6] = 0.0f;
            o[7] = 0.0f;
            o[8] = 0.0f;
            const float z0 = xtop - rc.c;
            const float d = z0 - rc.curve.w;
            const float bh = 1.0f / rc.curve.ibh;
            // the tangent lies below the mid line at the top by m (d - b log(1 + d/b)) >=
            // m d^2 / (2 (b + d)); it is only set up when that can pass 1.5 (units of ln 2)
            if (d > 0.0f && rc.curve.w < __builtin_inff() &&
                rc.curve.m * d * d * rc.invT * kInvLn2 > 3.0f * (bh + d)) {
                const float g0 = rc.curve.mw + rc.curve.mbh * log1p_acc(d * rc.curve.ibh);
                const float s0 = rc.curve.mbh / (bh + d);   // m b / (b + d)
                // tan(x) = (s0 x + g0 - s0 (z0 + c)) / T
                const float ti = __builtin_fmaf(-s0, xtop, g0) * rc.invT;
                o[4] = -s0 * rc.invT * kInvLn2;
                o[5] = __builtin_fmaf(ti, -kInvLn2, thr);
                o[7] = 1.0f;   // the tangent is set up; its intercept before thr:
                o[8] = ti;
                // the vector screen pays two instructions per slot for the tangent: worth it
                // when it lies well below the mid line at the top (in units of ln 2)
                o[6] = ((rc.curve.m * z0 - g0) * rc.invT * kInvLn2 > 1.5f) ? 1.0f : 0.0f;
            }
        } else {
            o[1] = -rc.invT * kInvLn2;
            o[2] = thr;
            o[3] = __builtin_inff();
            o[4] = o[1];
            o[5] = o[2];
            o[6] = 0.0f;
            o[7] = 0.0f;
            o[8] = 0.0f;
        }
        screen_guard(o[1], o[2], o[3], o[4], o[5]);
        if (!(o[1] == 0.0f && o[4] == 0.0f && o[2] < -1.0e38f)) return;
        o[0] = -3.0e38f;   // the screen is off for the row: no tangent either
        o[6] = o[7] = o[8] = 0.0f;
    };

    // Per wave: the lanes' largest logit into rx, and (curve on) their log-sum-exp sums.
    auto waves_combine = [&](float xm, float r, float s_, float u, float *rx) {
        const float xw = wave_max(xm);
        float mw = 0.0f, sw = 0.0f, uw = 0.0f;
        if constexpr (LSE) {
            // each lane's sums moved to the wave's reference mw: s 2^(r - mw), and for the
            // entropy anchor (u + s (r - mw)) 2^(r - mw)
            mw = wave_max(r);
            const float sc = __builtin_amdgcn_exp2f(r - mw);
            sw = wave_sum(s_ * sc);
            if constexpr (ENT)
                uw = wave_sum(s_ > 0.0f ? __builtin_fmaf(s_, r - mw, u) * sc : 0.0f);
        }
        if (lane == 0) {
            rx[wid] = xw;
            if constexpr (LSE) {
                red_m[wid] = mw;
                red_s[wid] = sw;
                red_u[wid] = uw;
            }
        }
    };
    if (screen) {
        if constexpr (BOOT0) {
            post_champion(champ0, craw0);
        } else {
            post_candidate(candidate(stream_k(k0), champ0, craw0, cw0, KEEP));
        }
    }
    waves_combine(xmax_lane, lse_r, lse_s, lse_u, red_x);
    __syncthreads();
    // Split rows without the pre-pass (the host chooses this only when a row's chunks run at
    // once: every block of the grid resident, or a resident grid taking items from a work
    // queue): each block publishes its own chunk's partial, combined from the streaming pass's
    // sums; wave 0 collects the row's other partials, waiting a bounded time for each; any
    // still missing then is worked out here by replaying that chunk's pass (the same slots,
    // order and arithmetic per lane), so the combined shift is the same whoever computes a
    // partial. The exchange slots are only touched by agent-scope atomics.
    const float4 *parts = a.partials + b * a.part_stride;
    if constexpr (HLG) {
        if (a.nchunk > 1 && a.exchange) {
            // chunk j's per-lane pass sums, replayed (see the streaming pass and its re-sum)
            auto replay_partial = [&](int j) {
                const int v0j = j * (int)a.cv;
                const int vendj = (int)min(a.nvec, (int64_t)v0j + a.cv);
                const int lvj = v0j + tid;
                auto fetch_j = [&](int gv) -> uint4 {
                    if (gv >= vendj) return ninf4;
                    return load_vec<DT>(rowp, gv, a.V, ALIGNED);
                };
                float xm = -__builtin_inff(), r = 0.0f, s_ = 0.0f, u = 0.0f;
#pragma unroll 1
                for (int n = 0; n < NV; ++n) {
                    const uint4 v = fetch_j(lvj + n * BS);
                    float xv[EPV];
#pragma unroll
                    for (int e = 0; e < EPV; ++e) xv[e] = elem<DT>(v, e);
                    const float m = vec_max<EPV>(xv);
                    xm = max2f(xm, m);
                    if constexpr (LSE) {
                        if (n == 0) r = (m > -__builtin_inff()) ? m * kLog2e : 0.0f;
#pragma unroll
                        for (int e = 0; e < EPV; ++e) {
                            const float t = __builtin_fmaf(xv[e], kLog2e, -r);
                            const float pe = __builtin_amdgcn_exp2f(t);
                            s_ += pe;
                            if constexpr (ENT) u = (pe > 0.0f) ? __builtin_fmaf(pe, t, u) : u;
                        }
                    }
                }
                if constexpr (LSE) {
                    const float tm = xm * kLog2e;
                    if (xm > -__builtin_inff() && !(fabsf(tm - r) <= 100.0f)) {
                        r = tm;
                        s_ = 0.0f;
                        u = 0.0f;
#pragma unroll 1
                        for (int n = 0; n < NV; ++n) {
                            const uint4 v = fetch_j(lvj + n * BS);
#pragma unroll
                            for (int e = 0; e < EPV; ++e) {
                                const float t = __builtin_fmaf(elem<DT>(v, e), kLog2e, -r);
                                const float pe = __builtin_amdgcn_exp2f(t);
                                s_ += pe;
                                if constexpr (ENT)
                                    u = (pe > 0.0f) ? __builtin_fmaf(pe, t, u) : u;
                            }
                        }
                    }
                }
                waves_combine(xm, r, s_, u, red_xp);
                __syncthreads();
                if (wid == 0) {
                    const float4 pr = waves_to_partial<PIV>(red_m, red_s, red_u, red_xp, lane, nw);
                    if (lane == 0) s_part[j] = pr;
                }
                __syncthreads();
            };
            if (wid == 0) {
                const float4 pr = waves_to_partial<PIV>(red_m, red_s, red_u, red_x, lane, nw);
                if (lane == 0) s_part[chunk] = pr;
            }
            __syncthreads();
            // A partial's four words carry their own presence: each is stored inverted, so a
            // zero word is one not yet written (the slots start zero-filled and the row's last
            // block fills them with zeros again); the one word whose inverse is zero (all bits
            // set: a NaN) is stored as another NaN. Every word is written once per call, so a
            // reader that sees all four nonzero has the final partial: no flag and no wait for
            // the stores to complete.
            uint32_t *slots = a.xslots + (size_t)b * a.part_stride * 4;
            if (tid == 0) {
                const float4 mine = s_part[chunk];
                const float mv[4] = {mine.x, mine.y, mine.z, mine.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t u = __float_as_uint(mv[q]);
                    __hip_atomic_store(slots + 4 * chunk + q, ~(u == 0xFFFFFFFFu ? 0x7FC00000u : u),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            if (wid == 0) {
                bool have = lane >= a.nchunk || lane == chunk;
                uint32_t pw[4] = {0u, 0u, 0u, 0u};
                for (int it = 0; it < a.spins; ++it) {
                    if (!have) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (pw[q] == 0u)
                                pw[q] = __hip_atomic_load(slots + 4 * lane + q, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                        have = pw[0] != 0u && pw[1] != 0u && pw[2] != 0u && pw[3] != 0u;
                    }
                    if (__ballot(!have) == 0ull) break;
                    __builtin_amdgcn_s_sleep(1);
                }
                if (have && lane < a.nchunk && lane != chunk)
                    s_part[lane] = make_float4(__uint_as_float(~pw[0]), __uint_as_float(~pw[1]),
                                               __uint_as_float(~pw[2]), __uint_as_float(~pw[3]));
                const uint64_t miss = __ballot(!have);
                if (lane == 0) s_miss = miss;
            }
            __syncthreads();
            uint64_t miss = s_miss;
            while (miss) {
                const int j = __builtin_ctzll(miss);
                miss &= miss - 1ull;
                replay_partial(j);
            }
            parts = s_part;
        }
    }
    if (wid == 0) {
        if (BOOT0 && screen) take_candidate(stream_k(k0));
        const float xmb = wave_max(lane < nw ? red_x[lane] : -__builtin_inff());
        float c = 0.0f;
        bool ok = xmb > -__builtin_inff();   // the chunk has a finite logit
        if constexpr (HLG) {
            // the shift c of z = x - c: LSE + mu (given pivot), x_max - offset (top anchor),
            // E_p[x] (entropy anchor), from this block's waves or the chunks' pre-pass
            // (the row's own mode when the curve is set per row: runtime, but wave-uniform)
            const int mode = PIV == 3 ? rpiv : PIV;
            if (mode == 1) {
                c = (a.nchunk == 1 ? xmb
                                   : wave_max(lane < a.nchunk ? parts[lane].w
                                                              : -__builtin_inff())) - poff;
                ok = c > -__builtin_inff();
            } else if (mode < 0) {
                c = 0.0f;   // curve off for this row: identity curve, no shift
            } else if (mode == 4) {
                // the mass median, worked out per row before this kernel (NaN or -inf for a
                // row with no finite logit)
                c = a.shift[b];
                ok = c > -__builtin_inff() && c < __builtin_inff();
            } else if constexpr (LSE) {
                if (a.nchunk == 1) {
                    const float pm = lane < nw ? red_m[lane] : -3.402823466e38f;
                    const float mb = wave_max(pm);
                    const float sc = lane < nw ? __builtin_amdgcn_exp2f(pm - mb) : 0.0f;
                    const float sb = wave_sum(lane < nw ? red_s[lane] * sc : 0.0f);
                    ok = sb > 0.0f;
                    if (mode == 0) {
                        c = (mb + __builtin_amdgcn_logf(sb)) * kLn2 + mu;
                    } else if constexpr (ENT) {
                        const float ub = wave_sum(
                            lane < nw && red_s[lane] > 0.0f
                                ? __builtin_fmaf(red_s[lane], pm - mb, red_u[lane]) * sc : 0.0f);
                        c = (mb + ub / sb) * kLn2;
                    }
                } else {
                    // the chunks' (max, sum, u), from the pre-pass or the exchange, one per
                    // lane (nchunk <= 64), all read at once; natural units
                    const float4 pj = lane < a.nchunk
                                          ? parts[lane]
                                          : make_float4(-__builtin_inff(), 0.0f, 0.0f, 0.0f);
                    const float Mb = wave_max(pj.x);
                    ok = Mb > -__builtin_inff();
                    const float e = pj.x > -__builtin_inff()
                                        ? __builtin_amdgcn_exp2f((pj.x - Mb) * kLog2e) : 0.0f;
                    const float Sb = wave_sum(pj.y * e);
                    if (mode == 0) {
                        c = Mb + logf(Sb) + mu;
                    } else if constexpr (ENT) {
                        const float Ub = wave_sum(pj.x > -__builtin_inff()
                                                      ? __builtin_fmaf(pj.y, pj.x - Mb, pj.z) * e
                                                      : 0.0f);
                        c = Mb + Ub / Sb;
                    }
                }
            }
            ok = ok && xmb > -__builtin_inff();
            c = uniform(c);
            rc.c = c;
            rc.mt = uniform(rc.curve.m * rc.invT);
            rc.mtc = uniform(rc.mt * rc.c);
            rc.mtw = uniform(rc.mt * rc.curve.w);
        }
        // The row's largest logit, for the lower bounds below: of split rows with the
        // chunks' partials (the curve on), every chunk's; otherwise the chunk's own.
        float xrow = xmb;
        if constexpr (HLG && PIV != 4) {
            if (a.nchunk > 1)
                xrow = uniform(fmaxf(wave_max(lane < a.nchunk ? parts[lane].w
                                                              : -__builtin_inff()), xmb));
        }
        float o[9] = {xmb, 0.0f, 0.0f, __builtin_inff(), 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if (ok && screen) {
            // lower bounds on the first draw's winning score: the best candidate's exact
            // score, and from the row's largest logit (its curve value is at least
            // (m/T) min(x - c, w) -- the toe lies above its mid line, the shoulder above m w --
            // and every Gumbel value is at least G(0) > -3.14)
            float lbx;
            if constexpr (HLG) {
                lbx = fminf(xrow - rc.c, rc.curve.w) * rc.mt - 3.14f;
            } else {
                lbx = xrow * rc.invT - 3.14f;
            }
            screen_consts(uniform(fmaxf(candidate_score(), lbx)), xmb, o);
        } else if (ok && sampled) {
            screen_consts(-__builtin_inff(), xmb, o);
        }
        if (lane == 0) {
            row_bc[0] = xmb;
            row_bc[1] = c;
            row_bc[2] = ok ? 1.0f : 0.0f;
            row_bc[3] = o[0];
            row_bc[4] = o[1];
            row_bc[5] = o[2];
            row_bc[6] = o[3];
            row_bc[7] = o[4];
            row_bc[8] = o[5];
            row_bc[9] = o[6];
            row_bc[10] = o[7];
            row_bc[11] = o[8];
            row_bc[12] = xrow;
        }
    }
    __syncthreads();
    // the row constants, read at once (three 16-byte LDS reads and one more behind one wait)
    float rb[13];
    {
        const float4 *q = reinterpret_cast<const float4 *>(row_bc);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const float4 t = q[i];
            rb[4 * i] = t.x;
            rb[4 * i + 1] = t.y;
            rb[4 * i + 2] = t.z;
            rb[4 * i + 3] = t.w;
        }
        rb[12] = row_bc[12];
    }
    const float xmax_blk = uniform(rb[0]);
    const bool skip = bad | !(uniform(rb[2]) > 0.0f);
    if constexpr (HLG) {
        rc.c = uniform(rb[1]);
        rc.mt = uniform(rc.curve.m * rc.invT);
        rc.mtc = uniform(rc.mt * rc.c);
        rc.mtw = uniform(rc.mt * rc.curve.w);
    }
    float sa = uniform(rb[4]), sb = uniform(rb[5]), sc = uniform(rb[6]);
    float ta = uniform(rb[7]), tb = uniform(rb[8]);
    bool tan_on = uniform(rb[9]) > 0.0f;
    // whether the first draw's screen is on (its constants were finite)
    const bool scr_on = !(sa == 0.0f && ta == 0.0f && sb < -1.0e38f);
    // for later draws: whether the shoulder tangent is set up, its intercept before the
    // threshold, and the lower bound from the chunk's largest logit (the first draw's)
    const bool tan_set = uniform(rb[10]) > 0.0f;
    const float tan_i = uniform(rb[11]);
    const float xmax_row = uniform(rb[12]);
    float lbx_row;
    if constexpr (HLG) {
        lbx_row = uniform(fminf(xmax_row - rc.c, rc.curve.w) * rc.mt - 3.14f);
    } else {
        lbx_row = uniform(xmax_row * rc.invT - 3.14f);
    }
    auto code_needed = [&](float x) -> float {
        return fminf(fmaxf(__builtin_fmaf(x, sa, sb), __builtin_fmaf(x, ta, tb)), sc);
    };
    // Exact scores of the elements of slot n (vector v, words w) that pass their own bound,
    // folded into the draw's best key.
    // The elements that pass are marked first and then scored one at a time, so a wave makes
    // as many exact scores as its busiest lane has passing elements (usually one), however
    // the lanes' elements differ.
    auto score_words = [&](int n, const uint4 &v, const uint32_t (&w)[EPV],
                           uint64_t best) -> uint64_t {
        const int gv = lane_v + n * BS;
        uint32_t pm = 0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float x = elem<DT>(v, e);
            const float cf = (float)__clz(~w[e]);
            const bool pass = x > -__builtin_inff() && (HLG || x >= tau_row) &&
                              cf >= code_needed(x);
            pm |= (pass ? 1u : 0u) << e;
        }
        while (pm) {
            const int e = __builtin_ctz(pm);
            pm &= pm - 1u;
            float x = 0.0f;
            uint32_t we = 0u;
#pragma unroll
            for (int q = 0; q < EPV; ++q) {
                x = q == e ? elem<DT>(v, q) : x;
                we = q == e ? w[q] : we;
            }
            const uint32_t i = (uint32_t)gv * EPV + (uint32_t)e;
            best = umax64(best, make_key(exact_score<HLG>(x, we, rc), i));
        }
        return best;
    };
    // The same for a vector read again: its words are drawn again; greedy rows compare logits.
    auto score_vec = [&](const Stream &sk, int n, const uint4 &v, uint64_t best) -> uint64_t {
        const int gv = lane_v + n * BS;
        if (greedy) return greedy_vec<DT>(v, (uint32_t)gv * EPV, best);
        uint32_t w[EPV];
        vec_words(sk, gv, w);
        return score_words(n, v, w, best);
    };

    for (int k = k0; k < k1; ++k) {
        asm volatile("" : "+v"(lane_lds));
        asm volatile("" : "+v"(lane_v));
        const Stream sk = stream_k(k);
        uint32_t champ = champ0;
        if (k > k0 && !skip && screen) {
            // this draw's words and champions, and the block's best bootstrap score (c is
            // known by now) as the lower bound for the screen: with BOOTK wave 0 draws and
            // scores one champion per 16 lanes between two barriers, as for the first draw;
            // otherwise every lane scores its own and one barrier combines the waves'
            champ = draw_all(sk);
            craw0 = slot_vec((int)(champ & 31u));
            float *sbp = red_sb[(k - k0) & 1];
            float bsw;
            if constexpr (BOOTK) {
                post_champion(champ, craw0);
                __syncthreads();
                if (wid == 0) {
                    take_candidate(sk);
                    const float cs = candidate_score();
                    if (lane == 0) sbp[0] = cs;
                }
                __syncthreads();
                bsw = sbp[0];
            } else {
                const Cand cd = candidate(sk, champ, craw0, cw0);
                const float cs =
                    cd.key != 0ull ? exact_score<HLG>(cd.x, cd.w, rc) : -__builtin_inff();
                const float csw = wave_max(cs);
                if (lane == 0) sbp[wid] = csw;
                __syncthreads();
                bsw = wave_max(lane < nw ? sbp[lane] : -__builtin_inff());
            }
            const float bs = uniform(fmaxf(bsw, lbx_row));
            // the same arithmetic as the first draw's constants, from the new bound
            const float thr = bs < __builtin_inff() ? (bs - screen_slack(bs)) * kInvLn2 - 1.0f
                                                    : -3.0e38f;
            if (scr_on) {
                if constexpr (HLG) {
                    sb = __builtin_fmaf(rc.mtc, kInvLn2, thr);
                    sc = __builtin_fmaf(rc.mtw, kInvLn2, thr);
                    tb = tan_set ? __builtin_fmaf(tan_i, -kInvLn2, thr) : sb;
                } else {
                    sb = thr;
                    tb = thr;
                }
                screen_guard(sa, sb, sc, ta, tb);
            }
        }
        // The least code any vector of the chunk needs: need falls as x grows, so it is the
        // need at the chunk's largest logit (rounded up to the bf16 grid as the vectors'
        // maxima are).
        float need_min;
        {
            uint32_t xb = __float_as_uint(xmax_blk);
            if constexpr (DT != DT_BF16) xb = ((int32_t)xb >= 0) ? xb + 0xFFFFu : xb;
            const float xt = __uint_as_float(xb & 0xFFFF0000u);
            need_min = uniform(tan_on ? code_needed(xt) : fminf(__builtin_fmaf(xt, sa, sb), sc));
            if (!(xmax_blk > -__builtin_inff())) need_min = 0.0f;
        }
        uint64_t best = 0;
        if (!skip) {
            // Screen: a vector can hold a winner only if U(its largest logit) + (n + 1) ln 2
            // reaches the bound less the slack, where n counts the leading ones of its largest
            // word's high 16 bits (n = 16 leaves the word unbounded); for greedy rows, only if
            // its largest logit reaches the chunk's. The champion vector and its words are at
            // hand from the bootstrap; the other vectors that pass (rare) come from the kept
            // registers (chunks of few slots) or are read again two at a time, so their loads
            // overlap.
            uint32_t bits = 0;   // bit n: slot n passes
            if (greedy) {
#pragma unroll
                for (int n = NV - 1; n >= 0; --n) {
                    const float xm = __uint_as_float(s_vec[lane_lds + n] << 16);
                    bits = (bits << 1) | (xm >= xmax_blk ? 1u : 0u);
                }
            } else if (need_min >= 8.0f) {
                // Even the chunk's largest logit needs a code with nb >= 8 leading ones, so no
                // vector whose code has fewer can pass: a first sweep keeps the others (about
                // 8 2^-nb of the vectors), and only those are tested in full.
                const int nb = (int)fminf(need_min, 16.0f);
                const uint32_t lim = (0xFFFFu << (16 - nb)) << 16;   // nb leading ones
                uint32_t cand = 0;
#pragma unroll
                for (int n = NV - 1; n >= 0; --n)
                    cand = (cand << 1) | (s_vec[lane_lds + n] >= lim ? 1u : 0u);
                while (cand) {
                    const int n = __builtin_ctz(cand);
                    cand &= cand - 1u;
                    const uint32_t d = s_vec[lane_lds + n];
                    const float xm = __uint_as_float(d << 16);
                    float need = fminf(tan_on ? code_needed(xm)
                                              : fminf(__builtin_fmaf(xm, sa, sb), sc), 16.0f);
                    if constexpr (!HLG) need = xm >= tau_row ? need : 17.0f;
                    bits |= ((float)lead_ones_hi16(d) >= need ? 1u : 0u) << n;
                }
            } else if (tan_on) {
#pragma unroll
                for (int n = NV - 1; n >= 0; --n) {
                    const uint32_t d = s_vec[lane_lds + n];
                    const float xm = __uint_as_float(d << 16);
                    // a needed code above 16 is met only by n = 16, which stands for any word
                    // (so the cap keeps such vectors)
                    const float need = fminf(code_needed(xm), 16.0f);
                    bits = (bits << 1) | ((float)lead_ones_hi16(d) >= need ? 1u : 0u);
                }
            } else {
                // the same with the mid line alone (also an upper bound)
#pragma unroll
                for (int n = NV - 1; n >= 0; --n) {
                    const uint32_t d = s_vec[lane_lds + n];
                    const float xm = __uint_as_float(d << 16);
                    float need = fminf(fminf(__builtin_fmaf(xm, sa, sb), sc), 16.0f);
                    // (curve off) a vector whose largest logit is below the filter threshold
                    // holds no candidate: a code no word reaches
                    if constexpr (!HLG) need = xm >= tau_row ? need : 17.0f;
                    bits = (bits << 1) | ((float)lead_ones_hi16(d) >= need ? 1u : 0u);
                }
            }
            if (screen) {   // champ and craw0 belong to this draw
                const uint32_t cbit = 1u << (champ & 31u);
                if (bits & cbit) {
                    bits &= ~cbit;
                    // (the per-lane bootstrap drew the champion's words already)
                    if (k == k0 ? BOOT0 : BOOTK)
                        vec_words(sk, lane_v + (int)(champ & 31u) * BS, cw0);
                    best = score_words((int)(champ & 31u), craw0, cw0, best);
                }
            }
            while (bits) {
                const int n1 = __builtin_ctz(bits);
                bits &= bits - 1u;
                const bool two = bits != 0u;
                const int n2 = two ? __builtin_ctz(bits) : n1;
                if (two) bits &= bits - 1u;
                const uint4 v1 = slot_vec(n1);
                const uint4 v2 = two ? slot_vec(n2) : ninf4;
                best = score_vec(sk, n1, v1, best);
                if (two) best = score_vec(sk, n2, v2, best);
            }
        }
        // block maximum of the draw's key: each wave's maximum goes into the draw's LDS entry
        // by an atomic maximum, with no barrier; a batch of up to 64 draws (or the last) is
        // written out by wave 0 after one barrier. Wave 0 alone issues the global atomics of
        // split rows, so its thread 0 can wait for all of them before counting the block in.
        {
            const int d = (k - k0) & 63;
            const uint64_t wk = wave_max_u64(best);
            if (lane == 0 && wk != 0ull)
                __hip_atomic_fetch_max(&s_best[d], wk, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            if (d == 63 || k == k1 - 1) {
                __syncthreads();
                if (wid == 0 && lane <= d) {
                    const uint64_t kb = s_best[lane];
                    s_best[lane] = 0ull;
                    const int64_t o = b * a.K + (k - d + lane);
                    if (a.nchunk == 1) {
                        a.out[o] = bad ? -2 : key_index(kb);
                        if (a.best_out) a.best_out[o] = bad ? -__builtin_inff() : key_score(kb);
                    } else if (kb != 0ull) {
                        __hip_atomic_fetch_max(a.keys + o, kb, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                if (k < k1 - 1) __syncthreads();   // the entries are reused
            }
        }
    }

    // ---- split rows: of the blocks that share this row's draws k0..k1-1 (one per chunk), the
    // last to finish writes their ids and re-zeroes their slots ----
    if (a.nchunk > 1) {
        // The keys and counters of split rows are only ever touched by agent-scope atomics, so
        // no fence is needed: an agent-scope fence writes back and invalidates the whole L2,
        // which stalls every load in flight on the device. Thread 0, which made this block's
        // maxima, waits for them to complete before it counts the block in; the block that
        // counts last reads the keys after that, with atomic loads.
        if (tid == 0) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const unsigned prev = __hip_atomic_fetch_add(a.counters + b * a.nkg + kg, 1u,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == (unsigned)(a.nchunk - 1));
        }
        __syncthreads();
        if (s_last) {
            for (int k = k0 + tid; k < k1; k += BS) {
                const int64_t o = b * a.K + k;
                const uint64_t kk = __hip_atomic_load(a.keys + o, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
                a.out[o] = bad ? -2 : key_index(kk);
                if (a.best_out) a.best_out[o] = bad ? -__builtin_inff() : key_score(kk);
                __hip_atomic_store(a.keys + o, (uint64_t)0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            if (tid == 0) {
                __hip_atomic_store(a.counters + b * a.nkg + kg, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            // the exchange's slots (one draw group per row: every block of the row is past
            // its wait once it has counted in, and thread 0 of each, which published its
            // partial, saw those stores complete before it counted in)
            if (a.exchange && tid < 4 * a.nchunk)
                __hip_atomic_store(a.xslots + (size_t)b * a.part_stride * 4 + tid, 0u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The sampling kernel: one work item per block.
template <int DT, int NV, bool HLG, int PIV, int MAXBS, bool ALIGNED, int LAY>
__global__ __launch_bounds__(MAXBS) void k_sample(SampleArgs a) {
    sample_item<DT, NV, HLG, PIV, MAXBS, ALIGNED, LAY>(a, blockIdx.x);
}

// The same on a resident grid whose blocks take items from a counter in the workspace
// (a.queue) until none is left. Consecutive items are the chunks of one row, so a row's chunks
// go to blocks that ask at about the same time and, all blocks being resident, run together:
// their log-sum-exp partials meet in the in-kernel exchange with no pre-pass. Every block
// leaves once the counter passes the last item; the last block out sets both counters back to
// zero for the next call. (A kernel of its own: the loop around the item costs registers.)
template <int DT, int NV, bool HLG, int PIV, int MAXBS, bool ALIGNED, int LAY>
__global__ __launch_bounds__(MAXBS) void k_sample_q(SampleArgs a) {
    __shared__ int s_item;
    for (;;) {
        if (threadIdx.x == 0)
            s_item = (int)__hip_atomic_fetch_add(a.queue, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int item = __builtin_amdgcn_readfirstlane(s_item);
        if (item >= a.items) break;
        sample_item<DT, NV, HLG, PIV, MAXBS, ALIGNED, LAY>(a, item);
        __syncthreads();   // the block's LDS serves its next item
    }
    if (threadIdx.x == 0) {
        // every other block has taken its last item (and seen the counter past the end)
        // before it counts itself out here
        const unsigned out = __hip_atomic_fetch_add(a.queue + 1, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (out == gridDim.x - 1) {
            __hip_atomic_store(a.queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.queue + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The instantiations that have a work-queue kernel: the curve on (the exchange of log-sum-exp
// partials is what the queue makes possible), aligned rows, and the chunk sizes queue_nv admits.
template <bool HLG, int PIV, bool AL, int NV>
constexpr bool kHasQueueKernel = HLG && PIV != 4 && AL && queue_nv(NV);

// The split pre-pass: one block per (row, chunk).
template <int DT, int PIV>
__global__ __launch_bounds__(1024) void k_lse_partial(SampleArgs a) {
    __shared__ float red_m[16], red_s[16], red_u[16], red_x[16];
    const int chunk = blockIdx.x % a.nchunk;
    const int64_t b = blockIdx.x / a.nchunk;
    chunk_partial<DT, PIV>(a, b, chunk, red_m, red_s, red_u, red_x,
                           &a.partials[b * a.part_stride + chunk]);
}

// ------------------------------------------------------------------------------------------
// Launchers, instantiated by the translation units that include this header.
// ------------------------------------------------------------------------------------------
// occ: when not null, the resident blocks per CU of the kernel this call would launch are
// written there instead of launching it.
template <int DT, bool HLG, int PIV, bool AL, int LAY>
hipError_t launch_sample_nv(const SampleArgs &a, int nv, int bs, int grid, hipStream_t s,
                            int *occ) {
    // blocks of up to 1024 threads, nv slots of 16-byte vectors per thread; the dynamic LDS
    // holds one dword per lane and slot
#define HS_CASE(N, MB)                                                                     \
    case N:                                                                                \
        if (bs > MB) return hipErrorInvalidValue;                                          \
        if (a.queue) {                                                                     \
            if constexpr (kHasQueueKernel<HLG, PIV, AL, N>) {                              \
                if (occ)                                                                   \
                    return hipOccupancyMaxActiveBlocksPerMultiprocessor(                   \
                        occ,                                                               \
                        reinterpret_cast<const void *>(&k_sample_q<DT, N, HLG, PIV, MB, AL, LAY>), \
                        bs, (size_t)(N | 1) * bs * 4);                                    \
                hipLaunchKernelGGL((k_sample_q<DT, N, HLG, PIV, MB, AL, LAY>), dim3(grid),  \
                                   dim3(bs), (size_t)(N | 1) * bs * 4, s, a);             \
                break;                                                                     \
            } else {                                                                       \
                return hipErrorInvalidValue;                                               \
            }                                                                              \
        }                                                                                  \
        if (occ)                                                                           \
            return hipOccupancyMaxActiveBlocksPerMultiprocessor(                           \
                occ, reinterpret_cast<const void *>(&k_sample<DT, N, HLG, PIV, MB, AL, LAY>), \
                bs, (size_t)(N | 1) * bs * 4);                                            \
        hipLaunchKernelGGL((k_sample<DT, N, HLG, PIV, MB, AL, LAY>), dim3(grid), dim3(bs), \
                           (size_t)(N | 1) * bs * 4, s, a);                               \
        break;
    switch (nv) {
        HS_CASE(1, 1024) HS_CASE(2, 1024) HS_CASE(4, 1024) HS_CASE(6, 1024) HS_CASE(8, 1024)
        HS_CASE(12, 1024) HS_CASE(16, 1024) HS_CASE(19, 1024)
        default: return hipErrorInvalidValue;
    }
#undef HS_CASE
    return hipGetLastError();
}

template <int DT, bool HLG, int PIV, int LAY>
hipError_t launch_sample_al(const SampleArgs &a, int nv, int bs, int grid, hipStream_t s,
                            int *occ) {
    // the branch-free load path needs 16-byte aligned rows holding at least one full vector
    if (a.aligned && a.V >= dtype_traits<DT>::epv)
        return launch_sample_nv<DT, HLG, PIV, true, LAY>(a, nv, bs, grid, s, occ);
    return launch_sample_nv<DT, HLG, PIV, false, LAY>(a, nv, bs, grid, s, occ);
}

// The sampling kernel of one word layout for each family of pivots: curve off or pivot given
// (PIV 0), anchored pivots (1 top, 2 entropy, 4 the mass median's shift), curve set per row
// (3). Each family and layout is instantiated in a translation unit of its own.
template <int LAY>
hipError_t launch_sample_given(int dt, bool hlg, const SampleArgs &a, int nv, int bs, int grid,
                               hipStream_t s, int *occ) {
    switch (dt) {
        case DT_F32: return hlg ? launch_sample_al<DT_F32, true, 0, LAY>(a, nv, bs, grid, s, occ)
                                : launch_sample_al<DT_F32, false, 0, LAY>(a, nv, bs, grid, s, occ);
        case DT_BF16: return hlg ? launch_sample_al<DT_BF16, true, 0, LAY>(a, nv, bs, grid, s, occ)
                                 : launch_sample_al<DT_BF16, false, 0, LAY>(a, nv, bs, grid, s, occ);
        case DT_F16: return hlg ? launch_sample_al<DT_F16, true, 0, LAY>(a, nv, bs, grid, s, occ)
                                : launch_sample_al<DT_F16, false, 0, LAY>(a, nv, bs, grid, s, occ);
    }
    return hipErrorInvalidValue;
}

template <int LAY>
hipError_t launch_sample_pivot(int dt, int piv, const SampleArgs &a, int nv, int bs, int grid,
                               hipStream_t s, int *occ) {
    switch (dt) {
        case DT_F32:
            return piv == 1 ? launch_sample_al<DT_F32, true, 1, LAY>(a, nv, bs, grid, s, occ)
                 : piv == 4 ? launch_sample_al<DT_F32, true, 4, LAY>(a, nv, bs, grid, s, occ)
                            : launch_sample_al<DT_F32, true, 2, LAY>(a, nv, bs, grid, s, occ);
        case DT_BF16:
            return piv == 1 ? launch_sample_al<DT_BF16, true, 1, LAY>(a, nv, bs, grid, s, occ)
                 : piv == 4 ? launch_sample_al<DT_BF16, true, 4, LAY>(a, nv, bs, grid, s, occ)
                            : launch_sample_al<DT_BF16, true, 2, LAY>(a, nv, bs, grid, s, occ);
        case DT_F16:
            return piv == 1 ? launch_sample_al<DT_F16, true, 1, LAY>(a, nv, bs, grid, s, occ)
                 : piv == 4 ? launch_sample_al<DT_F16, true, 4, LAY>(a, nv, bs, grid, s, occ)
                            : launch_sample_al<DT_F16, true, 2, LAY>(a, nv, bs, grid, s, occ);
    }
    return hipErrorInvalidValue;
}

template <int LAY>
hipError_t launch_sample_rows(int dt, const SampleArgs &a, int nv, int bs, int grid,
                              hipStream_t s, int *occ) {
    switch (dt) {
        case DT_F32: return launch_sample_al<DT_F32, true, 3, LAY>(a, nv, bs, grid, s, occ);
        case DT_BF16: return launch_sample_al<DT_BF16, true, 3, LAY>(a, nv, bs, grid, s, occ);
        case DT_F16: return launch_sample_al<DT_F16, true, 3, LAY>(a, nv, bs, grid, s, occ);
    }
    return hipErrorInvalidValue;
}

// Each family and layout is instantiated explicitly in its own translation unit; no other
// unit instantiates them implicitly.
extern template hipError_t launch_sample_given<LAY_PLAIN>(int, bool, const SampleArgs &, int,
                                                          int, int, hipStream_t, int *);
extern template hipError_t launch_sample_given<LAY_SCREENED>(int, bool, const SampleArgs &, int,
                                                             int, int, hipStream_t, int *);
extern template hipError_t launch_sample_pivot<LAY_PLAIN>(int, int, const SampleArgs &, int,
                                                          int, int, hipStream_t, int *);
extern template hipError_t launch_sample_pivot<LAY_SCREENED>(int, int, const SampleArgs &, int,
                                                             int, int, hipStream_t, int *);
extern template hipError_t launch_sample_rows<LAY_PLAIN>(int, const SampleArgs &, int, int, int,
                                                         hipStream_t, int *);
extern template hipError_t launch_sample_rows<LAY_SCREENED>(int, const SampleArgs &, int, int,
                                                            int, hipStream_t, int *);

template <int PIV>
hipError_t launch_lse_partial_t(int dt, const SampleArgs &a, int bs, int grid, hipStream_t s) {
    switch (dt) {
        case DT_F32: hipLaunchKernelGGL((k_lse_partial<DT_F32, PIV>), dim3(grid), dim3(bs), 0, s, a); break;
        case DT_BF16: hipLaunchKernelGGL((k_lse_partial<DT_BF16, PIV>), dim3(grid), dim3(bs), 0, s, a); break;
        case DT_F16: hipLaunchKernelGGL((k_lse_partial<DT_F16, PIV>), dim3(grid), dim3(bs), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hs
