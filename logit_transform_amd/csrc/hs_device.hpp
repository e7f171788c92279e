// hs_device.hpp -- device-side building blocks of libhs (gfx950, wave64).
//
// Sources, cited by page title and section:
//   [HLG]  "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document).
//   [GMX]  "Softmax-free GPU sampling: Gumbel-max categorical sampling kernel" (mlxcel #900).
//   [P123] Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11.
//
// Every kernel variant evaluates the per-element arithmetic through the functions in this
// file, compiled with -ffp-contract=off, so that all variants round identically.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

template <int DT> struct dtype_traits;
template <> struct dtype_traits<DT_F32> {
    static constexpr int esize = 4, epv = 4;          // elements per 16-byte vector
    static constexpr uint32_t neg_inf_word = 0xFF800000u;
};
template <> struct dtype_traits<DT_BF16> {
    static constexpr int esize = 2, epv = 8;
    static constexpr uint32_t neg_inf_word = 0xFF80FF80u;
};
template <> struct dtype_traits<DT_F16> {
    static constexpr int esize = 2, epv = 8;
    static constexpr uint32_t neg_inf_word = 0xFC00FC00u;
};

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kInvLn2 = 1.44269504088896341f;
constexpr float kLog2e = 1.44269504088896341f;

// ------------------------------------------------------------------------------------------
// Philox4x32-10 [P123]. Counter words 0 and 2 are multiplied by the two round multipliers
// into 64-bit products (one v_mad_u64_u32 each); the new counter is (hi1^c1^k0, lo1,
// hi0^c3^k1, lo0) and the key advances by the Weyl constants between rounds. When some
// counter or key words are wave-uniform the compiler moves their part of the early rounds
// to the scalar unit.
// ------------------------------------------------------------------------------------------
struct Words4 {
    uint32_t w[4];
};

__device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    Words4 o;
    o.w[0] = c0;
    o.w[1] = c1;
    o.w[2] = c2;
    o.w[3] = c3;
    return o;
}

// The same function for a wave-uniform key (k0, k1 in scalar registers), as the sampling
// kernels have it. From the third round on, both counter words that enter the xors are
// per-lane, and the compiler emits two v_xor_b32 per word; gfx950's three-input bitwise
// v_bitop3_b32 with truth table 0x96 (a ^ b ^ c) and the round key as its scalar operand
// does the same work in one. The first two rounds keep plain code: there one operand of each
// xor is itself uniform and folds into the scalar unit.
__device__ __forceinline__ uint32_t xor3_sk(uint32_t a, uint32_t b, uint32_t k) {
    return __builtin_amdgcn_bitop3_b32(a, b, k, 0x96);
}

// The rounds of a call whose counter word 0 alone is per lane (c0 = cl + delta: the lane's part
// and a wave-uniform part, cl + delta < 2^32); counter words 1..3 and the key are wave-uniform.
// Which words are uniform after each round: round 0 leaves c0, c1 uniform; round 1 leaves c3
// uniform, so round 2's second xor takes the scalar c3 ^ k1 in one instruction; from round 3 on
// every word is per lane and each xor pair is one v_bitop3_b32. (A vector multiply-add reads
// one scalar operand, the multiplier, so delta cannot ride in the first multiply's addend.)
__device__ __forceinline__ Words4 philox4x32_10_lane(uint32_t cl, uint32_t delta, uint32_t c1,
                                                     uint32_t c2, uint32_t c3, uint32_t k0,
                                                     uint32_t k1) {
    uint32_t c0 = 0;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)(r == 0 ? cl + delta : c0) * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
        uint32_t n0, n2;
        if (r < 2) {
            n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
            n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        } else if (r == 2) {
            n0 = xor3_sk((uint32_t)(p1 >> 32), c1, k0);
            n2 = (uint32_t)(p0 >> 32) ^ (c3 ^ k1);
        } else {
            n0 = xor3_sk((uint32_t)(p1 >> 32), c1, k0);
            n2 = xor3_sk((uint32_t)(p0 >> 32), c3, k1);
        }
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    Words4 o;
    o.w[0] = c0;
    o.w[1] = c1;
    o.w[2] = c2;
    o.w[3] = c3;
    return o;
}

__device__ __forceinline__ Words4 philox4x32_10_uk(uint32_t c0, uint32_t c1, uint32_t c2,
                                                   uint32_t c3, uint32_t k0, uint32_t k1) {
    return philox4x32_10_lane(c0, 0u, c1, c2, c3, k0, k1);
}

// Random words of the element group q (elements 4q..4q+3) of draw stream (seed, row, off)
// [GMX, Task 1: "philox(seed, row, i, offset)"]: counter (q, row, off lo, off hi),
// key (seed lo, seed hi); element i takes word i & 3.
struct Stream {
    uint32_t row, off_lo, off_hi, key0, key1;
};

// The stream's row, offset and key must be wave-uniform (one row per block).
__device__ __forceinline__ Words4 stream_group(const Stream &s, uint32_t q) {
    return philox4x32_10_uk(q, s.row, s.off_lo, s.off_hi, s.key0, s.key1);
}

// Word layouts of a stream. Plain: element i takes word i & 3 of the call at counter word
// i >> 2. Screened: element i = 8q + e takes the 16-bit half e of the call at counter word 2q
// as the high half of its word and that of the call at 2q + 1 as the low half (half e of an
// output: word e >> 1, low bits for even e). The two layouts use the same calls; the screened
// one puts the leading 16 bits of eight elements into one call, so a pass that only needs
// those bits (to bound each element's Gumbel value) makes half the calls.
enum : int { LAY_PLAIN = 0, LAY_SCREENED = 1 };

__device__ __forceinline__ uint32_t half16(const Words4 &w, uint32_t e) {
    const uint32_t d = (e >> 1) == 0 ? w.w[0] : (e >> 1) == 1 ? w.w[1] : (e >> 1) == 2 ? w.w[2] : w.w[3];
    return (e & 1u) ? (d >> 16) : (d & 0xFFFFu);
}

// The word of element i of stream s in layout LAY (one element per lane; exports and the few
// elements a threshold kernel draws).
template <int LAY>
__device__ __forceinline__ uint32_t element_word(const Stream &s, uint32_t i) {
    if constexpr (LAY == LAY_PLAIN) {
        const Words4 w = stream_group(s, i >> 2);
        return (i & 2u) ? ((i & 1u) ? w.w[3] : w.w[2]) : ((i & 1u) ? w.w[1] : w.w[0]);
    } else {
        const uint32_t q2 = (i >> 3) << 1;
        const Words4 hi = stream_group(s, q2);
        const Words4 lo = stream_group(s, q2 | 1u);
        return (half16(hi, i & 7u) << 16) | half16(lo, i & 7u);
    }
}

// Packed 16-bit integer maxima of two words (low halves, high halves), and the largest of the
// four 16-bit halves of two words.
__device__ __forceinline__ uint32_t max_half16_pk(uint32_t a, uint32_t b) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t max_half16(uint32_t a, uint32_t b) {
    const uint32_t m = max_half16_pk(a, b);
    return max(m & 0xFFFFu, m >> 16);
}

// A row's temperature is usable when it is 0 (greedy) or a normal positive float below +inf:
// then 1/T is finite in fp32. Negative, NaN, infinite and subnormal temperatures (where 1/T
// overflows) make the row invalid (-2).
__device__ __forceinline__ bool temp_valid(float T) {
    return T == 0.0f || (T >= 0x1p-126f && T < __builtin_inff());
}

// ------------------------------------------------------------------------------------------
// Accurate fp32 log1p(t) for t > -1 by the log(1+t) * t / ((1+t) - 1) correction (Goldberg,
// "What every computer scientist should know about floating-point arithmetic", 1991): the
// rounding of 1 + t is compensated exactly, leaving a few ulps from logf.
// The helpers below run without branches: every case is computed and the result selected, so
// a wave whose lanes fall in different cases runs one short sequence, and independent parts
// (the curve's logarithm and the Gumbel value's) can overlap.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float log1p_acc(float t) {
    const float u = 1.0f + t;
    // t / (u - 1) = 1 + (t - d) / d with d = u - 1 exact and t - d the exact rounding error of
    // 1 + t: the quotient is within an ulp of 1, so a hardware reciprocal (no IEEE divide
    // sequence) keeps it to about half an ulp.
    const float d = u - 1.0f;
    const float corr = __builtin_fmaf(t - d, __builtin_amdgcn_rcpf(d), 1.0f);
    float r = logf(u) * corr;
    r = (u == __builtin_inff()) ? __builtin_inff() : r;
    return (u == 1.0f) ? t : r;   // (1 + t rounds to 1: log1p(t) = t to fp32 precision)
}

// Gumbel noise of one word [GMX, Background: g = -log(-log(u))], u = (r + 1/2) 2^-32.
// E = -log(u) is formed from u on the lower half and from v = 1 - u = (~r + 1/2) 2^-32 by
// log1p on the upper half, so E keeps full relative precision where u is close to 1 -- the
// words that win draws. Both halves share one conversion and one logarithm (of u, or of the
// rounded 1 - v that log1p_acc corrects).
__device__ __forceinline__ float gumbel32(uint32_t r) {
    const bool lower = r < 0x80000000u;
    const float f = __builtin_fmaf((float)(lower ? r : ~r), 0x1p-32f, 0x1p-33f);   // u or v
    const float t = -f;
    const float u1 = 1.0f + t;
    const float L = logf(lower ? f : u1);
    const float d = u1 - 1.0f;
    const float corr = __builtin_fmaf(t - d, __builtin_amdgcn_rcpf(d), 1.0f);
    const float l1p = (u1 == 1.0f) ? t : L * corr;   // log1p(-v) (1 - v never overflows)
    const float E = lower ? -L : -l1p;
    return -logf(E);
}

// Leading ones of the high 16 bits of d, 0..16, in two instructions: gfx950's v_bitop3_b32 forms
// ~d | 0xFFFF (truth table 0xCF = ~S0 | S1) and v_ffbh_u32 counts its leading zeros; the low
// 16 bits, all set, cap the count at 16 (so the operand is never zero).
__device__ __forceinline__ uint32_t lead_ones_hi16(uint32_t d) {
    return __builtin_clz(__builtin_amdgcn_bitop3_b32(d, 0xFFFFu, 0xFFFFu, 0xCF));
}

// Maxima of fp32 values that are never NaN (finite logits or -inf): the hardware max
// instructions directly, without the quieting steps the compiler adds to fmaxf for inputs it
// cannot prove canonical.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ uint32_t max3u(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_max3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Exponents at or below this give 2^t = 0 in fp32 (far below the smallest subnormal). The
// entropy sums clamp t there before 2^t: a -inf logit then adds 0 * (-200) = 0 instead of
// 0 * (-inf) = NaN, with no select, and every other term is the one the unclamped sum adds.
constexpr float kExpFloor = -200.0f;

// ------------------------------------------------------------------------------------------
// The HLG transfer function [HLG, The transfer function, eq. g]: toe / mid / shoulder
// selected on z vs +-w: both logarithmic branches share one log1p_acc, whose argument and
// result are selected (a value the other branch would have produced, NaN included, is
// discarded). ln(1 + t) by log1p_acc.
// ------------------------------------------------------------------------------------------
struct Curve {
    float m, w;          // mid gain, mid half-width (w may be +inf)
    float mw;            // m * w
    float mbt, mbh;      // m * beta_t, m * beta_h
    float ibt, ibh;      // 1 / beta_t, 1 / beta_h
};

__device__ __forceinline__ float hlg32(float z, const Curve &c) {
    const bool toe = z < -c.w;
    const bool shoulder = z > c.w;
    const float L = log1p_acc(toe ? (-z - c.w) * c.ibt : (z - c.w) * c.ibh);
    const float r = toe ? -c.mw - c.mbt * L : c.mw + c.mbh * L;
    return (toe || shoulder) ? r : c.m * z;
}

// ------------------------------------------------------------------------------------------
// Index-carrying max [GMX, Background: "one index-carrying max-reduction pass"]: a 64-bit
// key whose high word orders the fp32 score (-0 folded onto +0) and whose low word is
// 0xFFFFFFFF - i, so the unsigned maximum is the largest score with the lowest index.
// Key 0 means "no finite element".
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_bits(float s) {
    uint32_t b = __float_as_uint(s);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float order_bits_to_float(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t i) {
    return ((uint64_t)order_bits(s) << 32) | (uint64_t)(0xFFFFFFFFu - i);
}

__device__ __forceinline__ int32_t key_index(uint64_t k) {
    return k == 0 ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)k);
}

__device__ __forceinline__ float key_score(uint64_t k) {
    return k == 0 ? -__builtin_inff() : order_bits_to_float((uint32_t)(k >> 32));
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Buffer resources (gfx950): the fourth word of a raw byte buffer, and the cache-policy bits
// of a load that streams data read once (non-temporal).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kCachePolicyNT = 2;

// ------------------------------------------------------------------------------------------
// Loads: 16-byte vectors of 4 fp32 or 8 bf16/f16 logits, upcast exactly to fp32 on use.
// ------------------------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float elem(const uint4 &v, int e) {
    const uint32_t w = (e >> (DT == DT_F32 ? 0 : 1)) == 0 ? v.x
                     : (e >> (DT == DT_F32 ? 0 : 1)) == 1 ? v.y
                     : (e >> (DT == DT_F32 ? 0 : 1)) == 2 ? v.z : v.w;
    if constexpr (DT == DT_F32) {
        return __uint_as_float(w);
    } else if constexpr (DT == DT_BF16) {
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else {
        const uint16_t h = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
        return (float)__builtin_bit_cast(_Float16, h);
    }
}

// Vector gv of a row (elements gv*epv .. gv*epv+epv-1); elements at or past V read as -inf.
template <int DT>
__device__ __forceinline__ uint4 load_vec(const char *__restrict__ rowp, int64_t gv, int64_t V,
                                          bool aligned) {
    using tr = dtype_traits<DT>;
    const int64_t i0 = gv * tr::epv;
    if (aligned && i0 + tr::epv <= V)
        return *reinterpret_cast<const uint4 *>(rowp + i0 * tr::esize);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = tr::neg_inf_word;
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (i0 + e < V) w[e] = reinterpret_cast<const uint32_t *>(rowp)[i0 + e];
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (i0 + e < V) {
                const uint32_t h = reinterpret_cast<const uint16_t *>(rowp)[i0 + e];
                const int j = e >> 1;
                w[j] = (e & 1) ? ((w[j] & 0x0000FFFFu) | (h << 16)) : ((w[j] & 0xFFFF0000u) | h);
            }
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------------------------------------------------
// Wave64 and block reductions. Within each row of 16 lanes four DPP steps (quad permutes,
// half-row and row mirrors) leave the row's result in every lane; the four rows are then
// combined from v_readlane into scalar registers. No LDS traffic inside a wave. The combine
// order is fixed, so every result is a deterministic function of the inputs. All lanes of
// the wave must be active.
// ------------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuad1032 = 0xB1, kDppQuad2301 = 0x4E, kDppRowHalfMirror = 0x141,
              kDppRowMirror = 0x140;

__device__ __forceinline__ float rl_f32(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Order-preserving map of non-NaN fp32 values onto unsigned integers, and its inverse: the
// maximum of the images is the image of the maximum (-0 ranks just below +0).
__device__ __forceinline__ uint32_t f2ord(float f) {
    const uint32_t b = __float_as_uint(f);
    return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o) {
    return __uint_as_float(o ^ ((uint32_t)((int32_t)~o >> 31) | 0x80000000u));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppQuad1032>(v));
    v = max(v, dpp_u32<kDppQuad2301>(v));
    v = max(v, dpp_u32<kDppRowHalfMirror>(v));
    v = max(v, dpp_u32<kDppRowMirror>(v));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}

// Maximum over the wave of values that are never NaN (integer maxima of their order images:
// one DPP-fused instruction per step).
__device__ __forceinline__ float wave_max(float v) { return ord2f(wave_max_u32(f2ord(v))); }

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f32<kDppQuad1032>(v);
    v += dpp_f32<kDppQuad2301>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    v += dpp_f32<kDppRowMirror>(v);
    return (rl_f32(v, 0) + rl_f32(v, 16)) + (rl_f32(v, 32) + rl_f32(v, 48));
}

__device__ __forceinline__ uint64_t umax64_pair(uint64_t a, uint32_t hi, uint32_t lo) {
    const uint64_t b = ((uint64_t)hi << 32) | lo;
    return b > a ? b : a;
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
    return umax64_pair(v, dpp_u32<CTRL>((uint32_t)(v >> 32)), dpp_u32<CTRL>((uint32_t)v));
}

__device__ __forceinline__ uint64_t rl_u64(uint64_t v, int lane) {
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    return ((uint64_t)hi << 32) | lo;
}

// Maximum over each row of 16 lanes, left in every lane of the row.
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
    v = dpp_max_u64<kDppQuad1032>(v);
    v = dpp_max_u64<kDppQuad2301>(v);
    v = dpp_max_u64<kDppRowHalfMirror>(v);
    return dpp_max_u64<kDppRowMirror>(v);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = row_max_u64(v);
    const uint64_t a = umax64(rl_u64(v, 0), rl_u64(v, 16));
    const uint64_t b = umax64(rl_u64(v, 32), rl_u64(v, 48));
    return umax64(a, b);
}

// Block-wide reductions (up to 16 waves) through a caller-owned LDS buffer `red` of 16
// entries. One barrier each: a call site must not reuse its buffer before a later barrier
// that all waves pass after reading it. Every thread returns the result.
__device__ __forceinline__ float block_max(float v, float *red) {
    // lane and wave index recomputed at each call, not held in registers across a caller's loop
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    int wid = threadIdx.x >> 6;
    asm volatile("" : "+v"(wid));
    const int nw = (blockDim.x + 63) >> 6;
    v = wave_max(v);
    if (lane == 0) red[wid] = v;
    __syncthreads();
    return wave_max(lane < nw ? red[lane] : -__builtin_inff());
}

__device__ __forceinline__ float block_sum(float v, float *red) {
    // lane and wave index recomputed at each call, not held in registers across a caller's loop
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    int wid = threadIdx.x >> 6;
    asm volatile("" : "+v"(wid));
    const int nw = (blockDim.x + 63) >> 6;
    v = wave_sum(v);
    if (lane == 0) red[wid] = v;
    __syncthreads();
    return wave_sum(lane < nw ? red[lane] : 0.0f);
}

}  // namespace hs
