// hs_kernels.hip -- gfx950 kernels of libhs: batched HLG tone curve + Gumbel-max sampling.
//
// Sources, cited by page title and section:
//   [HLG]  "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document).
//   [GMX]  "Softmax-free GPU sampling: Gumbel-max categorical sampling kernel" (mlxcel #900).
//
// Work decomposition. A block owns one contiguous chunk of one row and keeps it in VGPRs as
// raw 16-byte vectors (thread t holds vectors t, t+BS, t+2BS, ...: consecutive lanes read
// consecutive 16 B, so every wave load is one contiguous 1 KiB). The row is read from HBM
// once; every pass after the load (max, sum of exponentials, and each draw) runs on the
// register copy. With one chunk per row the row's log-sum-exp is reduced inside the block
// (single read). With several chunks per row a pre-pass leaves per-chunk (max, sum) pairs in
// the workspace, every block of the row folds them in the same fixed order, and the chunks'
// winning keys meet in a 64-bit atomic max; the last block of the row to finish writes the
// token ids and zeroes its workspace slots again.
//
// Screening. A draw's winner is the exact argmax over all elements, but the expensive part
// of an element's score (curve branches, two logarithms) is evaluated only when an upper
// bound on that score reaches the best score already found in the block minus a slack:
//   score = l'/T + G(r) <= U(x) + (clz(~r) + 1) ln 2,
// where U(x) = (m/T) * max(x - c, -w) bounds g(x - c)/T (g lies below its mid line past the
// shoulder knot and below -m*w in the toe) and clz(~r) bounds G from the word's leading
// ones. The bound is rigorous up to fp32 rounding, which the slack covers many times over,
// so the screened result equals the exhaustive one bit for bit (a test checks this).
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

// Element e (run-time index) of a register-held vector.
template <int DT>
__device__ __forceinline__ float elem_dyn(const uint4 &v, uint32_t e) {
    const uint32_t j = (DT == DT_F32) ? e : (e >> 1);
    const uint32_t w = j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
    if constexpr (DT == DT_F32) {
        return __uint_as_float(w);
    } else if constexpr (DT == DT_BF16) {
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else {
        const uint16_t h = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
        return (float)__builtin_bit_cast(_Float16, h);
    }
}

__device__ __forceinline__ uint32_t word_dyn(const Words4 &q, uint32_t j) {
    return j == 0 ? q.w[0] : j == 1 ? q.w[1] : j == 2 ? q.w[2] : q.w[3];
}

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

// Which of the 8 codes in cw (4 bits each) are >= t (0..15). Bytes serve as 8-bit lanes (no
// carry crosses a nibble): code 2j is tested in byte j of the low half, code 2j+1 in byte j
// of the high half. Bit 8j of the result flags code 2j, bit 8j+1 code 2j+1.
__device__ __forceinline__ uint32_t codes_ge(uint32_t cw, uint32_t t) {
    const uint32_t add = (16u - t) * 0x01010101u;
    const uint32_t lo = ((cw & 0x0F0F0F0Fu) + add) & 0x10101010u;
    const uint32_t hi = (((cw >> 4) & 0x0F0F0F0Fu) + add) & 0x10101010u;
    return (lo >> 4) | (hi >> 3);
}

// Element index of a set bit position of codes_ge's result.
__device__ __forceinline__ uint32_t codes_bit_elem(uint32_t p) { return ((p >> 3) << 1) | (p & 1u); }

template <int DT, int NV, bool HLG, int MAXBS, bool ALIGNED>
__global__ __launch_bounds__(MAXBS) void k_sample(SampleArgs a) {
    using tr = dtype_traits<DT>;
    constexpr int EPV = tr::epv;
    // Dynamic LDS, per lane and vector: the word codes of the current draw (EPV nibbles) in
    // s_codes; in s_vmax the vector's largest logit as a bf16-grid upper bound (high half,
    // draw-invariant) and the largest of its codes (low half). Each lane's entries are
    // contiguous, so every access is one base register plus an immediate offset.
    extern __shared__ uint32_t s_dyn[];
    __shared__ float2 red_lse[16];
    __shared__ float red_boot[16];
    __shared__ uint64_t red_draw[16];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int BS = blockDim.x;
    constexpr int SC = NV | 1;   // per-lane stride (odd: lanes hit distinct banks)
    uint32_t *s_codes = s_dyn;
    uint32_t *s_vmax = s_dyn + SC * BS;
    int lane_lds = tid * SC;   // re-made opaque per draw: no per-vector address hoisting
    // block coordinates in scalar registers (the divisions would otherwise run per lane)
    int bid = blockIdx.x;
    const int chunk = __builtin_amdgcn_readfirstlane(bid % a.nchunk);
    bid /= a.nchunk;
    const int kg = __builtin_amdgcn_readfirstlane(bid % a.nkg);
    const int64_t b = __builtin_amdgcn_readfirstlane(bid / a.nkg);
    const int k0 = kg * a.kpg;
    const int k1 = min(a.K, k0 + a.kpg);

    // ---- row parameters (wave-uniform) ----
    const float T = a.T[b];
    float mu = 0.0f;
    bool bad = !(T >= 0.0f) || !(T < __builtin_inff());
    if constexpr (HLG) {
        mu = a.mu[b];
        bad = bad || !(fabsf(mu) < __builtin_inff());
    }
    const bool greedy = (T == 0.0f);
    const bool sampled = !bad && !greedy;

    // ---- issue the loads of this chunk (registers) ----
    const int v0 = chunk * (int)a.cv;
    const int vend = (int)min(a.nvec, (int64_t)v0 + a.cv);
    const int nfull = (int)(a.V / EPV);   // vectors with all EPV elements inside the row
    const char *rowp = reinterpret_cast<const char *>(a.data) + b * a.ld * tr::esize;
    uint4 raw[NV];
    // ALIGNED: a vector outside the chunk or past the last full vector reads an in-row full
    // vector instead (clamped index) and is patched after the Philox phase, when waiting for
    // it costs nothing. The loads carry no branch: a branch would merge the loaded registers
    // into copies, and every copy waits for its load.
    const int gmax = min(vend, nfull) - 1;   // >= 0 when ALIGNED: the caller ensures V >= epv
    auto issue_load = [&](int n) {
        if constexpr (ALIGNED) {
            const int gv = min(v0 + tid + n * BS, gmax);
            raw[n] = *reinterpret_cast<const uint4 *>(rowp + (size_t)gv * 16);
        } else {
            const int gv = v0 + tid + n * BS;
            if (gv < vend) {
                raw[n] = load_vec<DT>(rowp, gv, a.V, false);
            } else {
                raw[n] = make_uint4(tr::neg_inf_word, tr::neg_inf_word, tr::neg_inf_word,
                                    tr::neg_inf_word);
            }
        }
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
    // Per lane and vector, s_vmax holds the vector's largest logit in its high half (exact
    // for bf16 input, rounded toward +inf to the bf16 grid otherwise, so it stays an upper
    // bound) and the vector's largest word code of the current draw in its low half.
    uint16_t *s_vmax16 = reinterpret_cast<uint16_t *>(s_vmax);

    // Word codes of one vector for draw stream sk: EPV 4-bit codes into s_codes, their
    // maximum into s_vmax. Vectors past the chunk are coded too (their words are never
    // used). Returns the lane's champion key after this vector: max code << 5 | vector.
    auto codes_vec = [&](const Stream &sk, int lane_v, int n, uint32_t champ) -> uint32_t {
        uint32_t q = ((uint32_t)(lane_v + n * BS) * EPV) >> 2;
        asm volatile("" : "+v"(q));
        uint32_t cw = 0, vm = 0;
#pragma unroll
        for (int g = 0; g < EPV / 4; ++g) {
            const Words4 qw = philox4x32_10_uk(q + g, sk.row, sk.off_lo, sk.off_hi, sk.key0,
                                               sk.key1);
            uint32_t c[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                c[e] = word_code(qw.w[e]);
                cw |= c[e] << (4 * (4 * g + e));
            }
            vm = max(vm, max(max(c[0], c[1]), max(c[2], c[3])));
        }
        s_codes[lane_lds + n] = cw;
        s_vmax16[2 * (lane_lds + n)] = (uint16_t)vm;
        return max(champ, (vm << 5) | (uint32_t)n);
    };

    // Patch the vectors the branch-free loads could not take whole (ragged row end, vectors
    // outside the chunk); waits for that vector's load.
    auto patch_vec = [&](int n) {
        if constexpr (ALIGNED) {
            const int gv = v0 + tid + n * BS;
            if (gv >= vend || gv >= nfull)
                raw[n] = (gv < vend) ? load_vec<DT>(rowp, gv, a.V, false)
                                     : make_uint4(tr::neg_inf_word, tr::neg_inf_word,
                                                  tr::neg_inf_word, tr::neg_inf_word);
        }
    };

    // Per vector once its load has landed: its largest logit into s_vmax and, with the curve
    // on, the log-sum-exp of the row [HLG, The transfer function: l = x - LSE(x)] streamed per
    // lane in base 2, with a running maximum mL of x log2(e) (floor -FLT_MAX: no inf - inf).
    float lse_m = -3.402823466e38f, lse_s = 0.0f;
    auto vec_pass = [&](int n) {
        patch_vec(n);
        // Tie this vector to the running sum: otherwise the scheduler issues every
        // exponential of the row first and holds all results at once.
        asm volatile("" : "+v"(lse_s), "+v"(raw[n].x), "+v"(raw[n].y), "+v"(raw[n].z),
                     "+v"(raw[n].w));
        float xv[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) xv[e] = elem<DT>(raw[n], e);
        float m;
        if constexpr (EPV == 8) {
            m = fmaxf(fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3])),
                      fmaxf(fmaxf(xv[4], xv[5]), fmaxf(xv[6], xv[7])));
        } else {
            m = fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3]));
        }
        uint32_t mb = __float_as_uint(m);
        if constexpr (DT != DT_BF16) {
            // toward +inf on the bf16 grid: positive values round up, negative ones truncate
            mb = ((int32_t)mb >= 0) ? mb + 0xFFFFu : mb;
        }
        s_vmax16[2 * (lane_lds + n) + 1] = (uint16_t)(mb >> 16);
        if constexpr (HLG) {
            const float mn = fmaxf(lse_m, m * kLog2e);
            float t = 0.0f;
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                t += __builtin_amdgcn_exp2f(__builtin_fmaf(xv[e], kLog2e, -mn));
            lse_s = __builtin_fmaf(lse_s, __builtin_amdgcn_exp2f(lse_m - mn), t);
            lse_m = mn;
        }
    };

    // Element (within its vector) of the lane's champion: the first one whose code equals the
    // champion's code.
    auto champion_elem = [&](uint32_t champ) -> uint32_t {
        const uint32_t bits = codes_ge(s_codes[lane_lds + (champ & 31u)], champ >> 5);
        return codes_bit_elem((uint32_t)__builtin_ctz(bits));
    };
    auto champion_logit = [&](uint32_t champ, int lane_v) -> float {
        const int gv = lane_v + (int)(champ & 31u) * BS;
        const int64_t i = (int64_t)gv * EPV + champion_elem(champ);
        if (gv >= vend || i >= a.V) return -__builtin_inff();
        if constexpr (DT == DT_F32) {
            return reinterpret_cast<const float *>(rowp)[i];
        } else {
            const uint16_t h = reinterpret_cast<const uint16_t *>(rowp)[i];
            if constexpr (DT == DT_BF16) return __uint_as_float((uint32_t)h << 16);
            else return (float)__builtin_bit_cast(_Float16, h);
        }
    };

    // Prologue, first draw. Loads go out a group of LG vectors at a time between the first
    // draw's Philox work (which needs no logit), starting after the first vector's codes so
    // that no wave begins by stalling on the memory queue; each vector's pass over its logits
    // follows its codes LAG vectors later, when its load has landed, so float work mixes with
    // the integer Philox chains. The logit pass runs for every row (greedy and invalid rows
    // included): keeping it free of row-dependent branches keeps the register allocator from
    // duplicating the row copy.
    constexpr int LG = 4;
    constexpr int LAG = 8;
    uint32_t champ0 = 0;
    float champ_x0 = -__builtin_inff();
    {
        const Stream sk = stream_k(k0);
        int lane_v = v0 + tid;
        asm volatile("" : "+v"(lane_v));
        const bool do_codes = sampled && k0 < k1;
        auto load_group = [&](int n) {
            if (n == 0) {
#pragma unroll
                for (int j = 0; j < 2 * LG && j < NV; ++j) issue_load(j);
            } else if (n % LG == 0) {
#pragma unroll
                for (int j = n + LG; j < n + 2 * LG && j < NV; ++j) issue_load(j);
            }
        };
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            if (do_codes) champ0 = codes_vec(sk, lane_v, n, champ0);
            load_group(n);
            if (n >= LAG) vec_pass(n - LAG);
        }
        // The champion's logit, for the bootstrap after the log-sum-exp: read once more (a
        // cache hit) rather than picked out of the register copy by a run-time index.
        if (do_codes) champ_x0 = champion_logit(champ0, lane_v);
#pragma unroll
        for (int n = (NV > LAG ? NV - LAG : 0); n < NV; ++n) vec_pass(n);
    }

    RowConst rc;
    rc.invT = 1.0f / T;
    rc.c = 0.0f;
    rc.mt = rc.mtc = rc.mtw = 0.0f;
    rc.curve = a.curve;
    bool skip = bad;

    if constexpr (HLG) {
        float lse;
        if (a.nchunk == 1) {
            const MaxSum ms = block_maxsum_log2(lse_m, lse_s, red_lse);
            lse = (ms.s > 0.0f) ? (ms.m + __builtin_amdgcn_logf(ms.s)) * kLn2 : -__builtin_inff();
        } else {
            const float2 *part = a.partials + b * a.part_stride;
            float Mb = -__builtin_inff();
            for (int j = 0; j < a.nchunk; ++j) Mb = fmaxf(Mb, part[j].x);
            float Sb = 0.0f;
            if (Mb > -__builtin_inff())
                for (int j = 0; j < a.nchunk; ++j)
                    if (part[j].x > -__builtin_inff())
                        Sb += part[j].y * __builtin_amdgcn_exp2f((part[j].x - Mb) * kLog2e);
            lse = (Mb > -__builtin_inff()) ? Mb + logf(Sb) : -__builtin_inff();
        }
        lse = uniform(lse);
        if (!(lse > -__builtin_inff())) skip = true;   // no finite logit in the row
        rc.c = uniform(lse + mu);
        rc.mt = uniform(a.curve.m * rc.invT);
        rc.mtc = uniform(rc.mt * rc.c);
        rc.mtw = uniform(rc.mt * a.curve.w);
    }

    for (int k = k0; k < k1; ++k) {
        asm volatile("" : "+v"(lane_lds));
        uint32_t champ = champ0;
        float champ_x = champ_x0;
        int lane_v = v0 + tid;
        asm volatile("" : "+v"(lane_v));
        if (k > k0 && sampled) {
            const Stream sk = stream_k(k);
            champ = 0;
#pragma unroll
            for (int n = 0; n < NV; ++n) champ = codes_vec(sk, lane_v, n, champ);
            // the champion's logit, picked out of the register copy
            const uint32_t cs = champ & 31u;
            const uint32_t e = champion_elem(champ);
            uint4 cv4 = raw[0];
#pragma unroll
            for (int n = 1; n < NV; ++n) {
                if (cs == (uint32_t)n) cv4 = raw[n];
            }
            champ_x = (lane_v + (int)cs * BS < vend) ? elem_dyn<DT>(cv4, e) : -__builtin_inff();
        }
        // Keep per-element work inside the draw loop: without this the compiler hoists the
        // draw-invariant part of the screen (one value per element) out of the loop and runs
        // out of registers. Likewise for everything derived from the element indices.
#pragma unroll
        for (int n = 0; n < NV; ++n)
            asm volatile("" : "+v"(raw[n].x), "+v"(raw[n].y), "+v"(raw[n].z), "+v"(raw[n].w));
        uint64_t best = 0;
        if (!skip && greedy) {
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                const int gv = lane_v + n * BS;
                if (gv < vend) best = greedy_vec<DT>(raw[n], (uint32_t)(gv * EPV), best);
            }
        } else if (!skip) {
            const Stream sk = stream_k(k);

            // Bootstrap: each lane bounds from below the score of its champion (an element
            // with the lane's largest code, hence nearly the largest Gumbel value among the
            // lane's elements); the block maximum of these bounds is at most the draw's
            // winning score. Lower bounds used: g(z) >= m min(z, w) (the toe lies above its
            // mid line, the shoulder above m w), and for code n >= 1 the word has
            // clz(~r) >= n, so u >= 1 - 2^-n and G >= n ln 2 + ln(1 - 2^-n); code 0 only
            // gives G >= -3.14.
            float thr_s = -3.0e38f;   // (best known - slack) / ln 2 - 1
            if (!a.no_screen) {
                const uint32_t cn = champ >> 5;
                float lb = -__builtin_inff();
                if (champ_x > -__builtin_inff()) {
                    float alo;
                    if constexpr (HLG) {
                        alo = fminf(champ_x - rc.c, rc.curve.w) * rc.mt;
                    } else {
                        alo = champ_x * rc.invT;
                    }
                    const float glo = cn == 0u ? -3.14f
                                    : cn == 1u ? 0.0f
                                    : cn == 2u ? 1.0986f
                                    : cn == 3u ? 1.9459f
                                    : __builtin_fmaf((float)cn, kLn2, -0.0646f);
                    lb = alo + glo;
                }
                const float bs = block_max(lb, red_boot);
                if (bs > -__builtin_inff())
                    thr_s = uniform((bs - screen_slack(bs)) * kInvLn2 - 1.0f);
            }

            // Screen, one vector at a time: a vector can hold a winner only if
            // U(max x of the vector) + (max code + 1) ln 2 >= best - slack; its elements are
            // then tested one by one with their own code and U(x) before the exact score.
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                const int gv = lane_v + n * BS;
                const uint32_t sv = s_vmax[lane_lds + n];
                const float xm = __uint_as_float(sv & 0xFFFF0000u);
                float Uv;
                if constexpr (HLG) {
                    Uv = fmaxf(__builtin_fmaf(xm, rc.mt, -rc.mtc), -rc.mtw);
                } else {
                    Uv = xm * rc.invT;
                }
                // smallest code that can pass; code 15 stands for "15 or more"
                const float tf = fminf(__builtin_fmaf(Uv, -kInvLn2, thr_s), 15.0f);
                const float cmax = (float)(sv & 0xFFu);
                if (gv < vend && cmax >= tf) {
                    const uint32_t cw = s_codes[lane_lds + n];
                    const uint32_t t = (uint32_t)fmaxf(ceilf(tf), 0.0f);
                    uint32_t bits = codes_ge(cw, t);
                    if constexpr (EPV == 4) bits &= 0x0303u;
                    while (bits) {
                        const uint32_t e = codes_bit_elem((uint32_t)__builtin_ctz(bits));
                        bits &= bits - 1u;
                        const float x = elem_dyn<DT>(raw[n], e);
                        float U;
                        if constexpr (HLG) {
                            U = fmaxf(__builtin_fmaf(x, rc.mt, -rc.mtc), -rc.mtw);
                        } else {
                            U = x * rc.invT;
                        }
                        const uint32_t ce = (cw >> (4 * e)) & 15u;
                        const float cf = (ce == 15u) ? 32.0f : (float)ce;
                        if (x > -__builtin_inff() && cf >= __builtin_fmaf(U, -kInvLn2, thr_s)) {
                            const uint32_t i = (uint32_t)gv * EPV + e;
                            const Words4 q = stream_group_in_loop(sk, i >> 2);
                            best = umax64(best, make_key(exact_score<HLG>(x, word_dyn(q, i & 3u), rc), i));
                        }
                    }
                }
            }
        }
        // block reduction of the draw's key
        const uint64_t kb = block_max_u64(best, red_draw);
        if (tid == 0) {
            const int64_t o = b * a.K + k;
            if (a.nchunk == 1) {
                a.out[o] = bad ? -2 : key_index(kb);
                if (a.best_out) a.best_out[o] = bad ? -__builtin_inff() : key_score(kb);
            } else if (kb != 0) {
                atomicMax(reinterpret_cast<unsigned long long *>(a.keys + o),
                          (unsigned long long)kb);
            }
        }
    }

    // ---- split rows: the last block of the row writes the ids and re-zeroes its slots ----
    if (a.nchunk > 1) {
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const unsigned prev = atomicAdd(a.counters + b, 1u);
            s_last = (prev == (unsigned)(a.nchunk * a.nkg - 1));
        }
        __syncthreads();
        if (s_last) {
            __threadfence();
            for (int k = tid; k < a.K; k += BS) {
                const int64_t o = b * a.K + k;
                const uint64_t kk = __hip_atomic_load(a.keys + o, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
                a.out[o] = bad ? -2 : key_index(kk);
                if (a.best_out) a.best_out[o] = bad ? -__builtin_inff() : key_score(kk);
                __hip_atomic_store(a.keys + o, (uint64_t)0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            if (tid == 0)
                __hip_atomic_store(a.counters + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Per-chunk (max, sum exp(x - max)) pairs for rows split over several blocks.
template <int DT>
__global__ __launch_bounds__(1024) void k_lse_partial(SampleArgs a) {
    using tr = dtype_traits<DT>;
    constexpr int EPV = tr::epv;
    __shared__ float red_m[16], red_s[16];
    const int chunk = blockIdx.x % a.nchunk;
    const int64_t b = blockIdx.x / a.nchunk;
    const int64_t v0 = (int64_t)chunk * a.cv;
    const int64_t vend = min(a.nvec, v0 + a.cv);
    const char *rowp = reinterpret_cast<const char *>(a.data) + b * a.ld * tr::esize;
    float mx = -__builtin_inff();
    for (int64_t gv = v0 + threadIdx.x; gv < vend; gv += blockDim.x) {
        const uint4 v = load_vec<DT>(rowp, gv, a.V, a.aligned);
#pragma unroll
        for (int e = 0; e < EPV; ++e) mx = fmaxf(mx, elem<DT>(v, e));
    }
    const float M = block_max(mx, red_m);
    float s = 0.0f;
    if (M > -__builtin_inff()) {
        const float mb = M * kLog2e;
        for (int64_t gv = v0 + threadIdx.x; gv < vend; gv += blockDim.x) {
            const uint4 v = load_vec<DT>(rowp, gv, a.V, a.aligned);
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                s += __builtin_amdgcn_exp2f(elem<DT>(v, e) * kLog2e - mb);
        }
    }
    const float S = block_sum(s, red_s);
    if (threadIdx.x == 0) a.partials[b * a.part_stride + chunk] = make_float2(M, S);
}

// One block per row: log-sum-exp of the row, and (transform) l' = g(x - LSE - mu).
template <int DT, bool TRANSFORM>
__global__ __launch_bounds__(1024) void k_row_lse(RowOpArgs a) {
    using tr = dtype_traits<DT>;
    constexpr int EPV = tr::epv;
    __shared__ float red_m[16], red_s[16];
    const int64_t b = blockIdx.x;
    const int64_t nvec = (a.V + EPV - 1) / EPV;
    const char *rowp = reinterpret_cast<const char *>(a.data) + b * a.ld * tr::esize;
    float mx = -__builtin_inff();
    for (int64_t gv = threadIdx.x; gv < nvec; gv += blockDim.x) {
        const uint4 v = load_vec<DT>(rowp, gv, a.V, a.aligned);
#pragma unroll
        for (int e = 0; e < EPV; ++e) mx = fmaxf(mx, elem<DT>(v, e));
    }
    const float M = block_max(mx, red_m);
    float s = 0.0f;
    if (M > -__builtin_inff()) {
        const float mb = M * kLog2e;
        for (int64_t gv = threadIdx.x; gv < nvec; gv += blockDim.x) {
            const uint4 v = load_vec<DT>(rowp, gv, a.V, a.aligned);
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                s += __builtin_amdgcn_exp2f(elem<DT>(v, e) * kLog2e - mb);
        }
    }
    const float S = block_sum(s, red_s);
    const float lse = (M > -__builtin_inff()) ? M + logf(S) : -__builtin_inff();
    if constexpr (!TRANSFORM) {
        if (threadIdx.x == 0) a.lse[b] = lse;
    } else {
        const float c = lse + a.mu[b];
        float *orow = a.out + b * a.ldo;
        for (int64_t gv = threadIdx.x; gv < nvec; gv += blockDim.x) {
            const uint4 v = load_vec<DT>(rowp, gv, a.V, a.aligned);
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int64_t i = gv * EPV + e;
                if (i < a.V) {
                    const float x = elem<DT>(v, e);
                    orow[i] = (x > -__builtin_inff()) ? hlg32(x - c, a.curve) : -__builtin_inff();
                }
            }
        }
    }
}

__global__ void k_philox(const uint32_t *__restrict__ ctr, const uint32_t *__restrict__ key,
                         uint32_t *__restrict__ out, int64_t n) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    const Words4 o = philox4x32_10(ctr[4 * j], ctr[4 * j + 1], ctr[4 * j + 2], ctr[4 * j + 3],
                                   key[2 * j], key[2 * j + 1]);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * j + e] = o.w[e];
}

// One block row (blockIdx.y) per sampled row, so that the row's key is wave-uniform as in
// the sampling kernels, which share stream_group with this export.
__global__ void k_stream_words(const uint64_t *__restrict__ seed,
                               const uint64_t *__restrict__ offset, int64_t B, int64_t V,
                               int32_t k, uint32_t *__restrict__ out) {
    const int64_t ng = (V + 3) / 4;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = blockIdx.y;
    const uint64_t off = offset[b] + (uint64_t)k;
    Stream st;
    st.row = (uint32_t)b;
    st.off_lo = (uint32_t)off;
    st.off_hi = (uint32_t)(off >> 32);
    st.key0 = (uint32_t)seed[b];
    st.key1 = (uint32_t)(seed[b] >> 32);
    if (q >= ng) return;
    const Words4 o = stream_group(st, (uint32_t)q);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = q * 4 + e;
        if (i < V) out[b * V + i] = o.w[e];
    }
}

__global__ void k_gumbel(const uint32_t *__restrict__ w, float *__restrict__ g, int64_t n) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < n) g[j] = gumbel32(w[j]);
}

__global__ void k_fill_zero(uint32_t *__restrict__ p, int64_t n) {
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n;
         j += (int64_t)gridDim.x * blockDim.x)
        p[j] = 0u;
}

// ------------------------------------------------------------------------------------------
// Host-side launchers (called from hs_api.hip).
// ------------------------------------------------------------------------------------------
template <int DT, bool HLG, bool AL>
static hipError_t launch_sample_nv(const SampleArgs &a, int nv, int bs, int grid, hipStream_t s) {
    // Blocks of up to 1024 threads hold up to 19 vectors per thread in registers (128 per
    // lane at 16 waves per CU); the dynamic LDS holds each lane's codes and vector maxima.
#define HS_CASE(N, MB)                                                                     \
    case N:                                                                                \
        if (bs > MB) return hipErrorInvalidValue;                                          \
        hipLaunchKernelGGL((k_sample<DT, N, HLG, MB, AL>), dim3(grid), dim3(bs),          \
                           (size_t)(N | 1) * bs * 4 * 2, s, a);                               \
        break;
    switch (nv) {
        HS_CASE(1, 1024) HS_CASE(2, 1024) HS_CASE(4, 1024) HS_CASE(6, 1024) HS_CASE(8, 1024)
        HS_CASE(12, 1024) HS_CASE(16, 1024) HS_CASE(19, 1024)
        default: return hipErrorInvalidValue;
    }
#undef HS_CASE
    return hipGetLastError();
}

template <int DT, bool HLG>
static hipError_t launch_sample_al(const SampleArgs &a, int nv, int bs, int grid, hipStream_t s) {
    // the branch-free load path needs 16-byte aligned rows holding at least one full vector
    if (a.aligned && a.V >= dtype_traits<DT>::epv)
        return launch_sample_nv<DT, HLG, true>(a, nv, bs, grid, s);
    return launch_sample_nv<DT, HLG, false>(a, nv, bs, grid, s);
}

hipError_t launch_sample(int dt, bool hlg, const SampleArgs &a, int nv, int bs, int grid,
                         hipStream_t s) {
    switch (dt) {
        case DT_F32: return hlg ? launch_sample_al<DT_F32, true>(a, nv, bs, grid, s)
                                : launch_sample_al<DT_F32, false>(a, nv, bs, grid, s);
        case DT_BF16: return hlg ? launch_sample_al<DT_BF16, true>(a, nv, bs, grid, s)
                                 : launch_sample_al<DT_BF16, false>(a, nv, bs, grid, s);
        case DT_F16: return hlg ? launch_sample_al<DT_F16, true>(a, nv, bs, grid, s)
                                : launch_sample_al<DT_F16, false>(a, nv, bs, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_lse_partial(int dt, const SampleArgs &a, int bs, int grid, hipStream_t s) {
    switch (dt) {
        case DT_F32: hipLaunchKernelGGL((k_lse_partial<DT_F32>), dim3(grid), dim3(bs), 0, s, a); break;
        case DT_BF16: hipLaunchKernelGGL((k_lse_partial<DT_BF16>), dim3(grid), dim3(bs), 0, s, a); break;
        case DT_F16: hipLaunchKernelGGL((k_lse_partial<DT_F16>), dim3(grid), dim3(bs), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_row_lse(int dt, bool transform, const RowOpArgs &a, int grid, hipStream_t s) {
    const int bs = 1024;
#define HS_ROW(D)                                                                              \
    if (transform) hipLaunchKernelGGL((k_row_lse<D, true>), dim3(grid), dim3(bs), 0, s, a);  \
    else hipLaunchKernelGGL((k_row_lse<D, false>), dim3(grid), dim3(bs), 0, s, a);
    switch (dt) {
        case DT_F32: HS_ROW(DT_F32) break;
        case DT_BF16: HS_ROW(DT_BF16) break;
        case DT_F16: HS_ROW(DT_F16) break;
        default: return hipErrorInvalidValue;
    }
#undef HS_ROW
    return hipGetLastError();
}

hipError_t launch_philox(const uint32_t *ctr, const uint32_t *key, uint32_t *out, int64_t n,
                         hipStream_t s) {
    const int bs = 256;
    const int64_t grid = (n + bs - 1) / bs;
    hipLaunchKernelGGL(k_philox, dim3((unsigned)grid), dim3(bs), 0, s, ctr, key, out, n);
    return hipGetLastError();
}

hipError_t launch_stream_words(const uint64_t *seed, const uint64_t *offset, int64_t B,
                               int64_t V, int32_t k, uint32_t *out, hipStream_t s) {
    const int bs = 256;
    const int64_t ng = (V + 3) / 4;
    const int64_t gx = (ng + bs - 1) / bs;
    if (B > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_stream_words, dim3((unsigned)gx, (unsigned)B), dim3(bs), 0, s, seed,
                       offset, B, V, k, out);
    return hipGetLastError();
}

hipError_t launch_gumbel(const uint32_t *w, float *g, int64_t n, hipStream_t s) {
    const int bs = 256;
    const int64_t grid = (n + bs - 1) / bs;
    hipLaunchKernelGGL(k_gumbel, dim3((unsigned)grid), dim3(bs), 0, s, w, g, n);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, int64_t nwords, hipStream_t s) {
    const int bs = 256;
    int64_t grid = (nwords + bs - 1) / bs;
    if (grid > 4096) grid = 4096;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)grid), dim3(bs), 0, s,
                       reinterpret_cast<uint32_t *>(p), nwords);
    return hipGetLastError();
}

}  // namespace hs
