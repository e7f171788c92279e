// hs_kernels.hip -- gfx950 kernels of libhs and their host-side launchers: the sampling kernel
// with the curve off or with a given pivot (the pivot anchors are instantiated in
// hs_kernels_pivot.hip), the row log-sum-exp / curve transform / pivot, and the exports of
// the random-number steps.
//
// Sources, cited by page title and section:
//   [HLG]  "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document).
//   [GMX]  "Softmax-free GPU sampling: Gumbel-max categorical sampling kernel" (mlxcel #900).
#include <hip/hip_runtime.h>

#include "hs_device.hpp"
#include "hs_internal.hpp"
#include "hs_sample_kernel.hpp"

namespace hs {

// One block per row: the row's log-sum-exp (OP 0), its transformed logits
// l' = g((x - LSE) - mu) (OP 1) [HLG, The transfer function, eq. z and eq. g], or its pivot mu
// (OP 2) [HLG, The pivot], with the pivot given (PIV 0), top-anchored (1: mu = l_max - c) or
// entropy-anchored (2: mu = sum p l). Two passes over the row, which stays in the caches:
// the maximum M, then sum exp(x - M) and sum exp(x - M) (x - M).
template <int DT, int OP, int PIV>
__global__ __launch_bounds__(1024) void k_row_lse(RowOpArgs a) {
    using tr = dtype_traits<DT>;
    constexpr int EPV = tr::epv;
    __shared__ float red_m[16], red_s[16], red_u[16];
    const int64_t b = blockIdx.x;
    const int64_t nvec = (a.V + EPV - 1) / EPV;
    const char *rowp = reinterpret_cast<const char *>(a.data) + b * a.ld * tr::esize;
    // the mass median's shift, read before the first barrier (no output is written before it)
    float c4 = 0.0f;
    if constexpr (PIV == 4) c4 = a.shift[b * a.shift_stride];
    float mx = -__builtin_inff();
    for (int64_t gv = threadIdx.x; gv < nvec; gv += blockDim.x) {
        const uint4 v = load_vec<DT>(rowp, gv, a.V, a.aligned);
#pragma unroll
        for (int e = 0; e < EPV; ++e) mx = fmaxf(mx, elem<DT>(v, e));
    }
    const float M = block_max(mx, red_m);
    float s = 0.0f, u = 0.0f;
    if (M > -__builtin_inff()) {
        const float mb = M * kLog2e;
        for (int64_t gv = threadIdx.x; gv < nvec; gv += blockDim.x) {
            const uint4 v = load_vec<DT>(rowp, gv, a.V, a.aligned);
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                float t = elem<DT>(v, e) * kLog2e - mb;
                if constexpr (PIV == 2) t = max2f(t, kExpFloor);
                const float p = __builtin_amdgcn_exp2f(t);
                s += p;
                if constexpr (PIV == 2) u = __builtin_fmaf(p, t, u);
            }
        }
    }
    const float S = block_sum(s, red_s);
    const float lse = (M > -__builtin_inff()) ? M + logf(S) : -__builtin_inff();
    if constexpr (OP == 0) {
        if (threadIdx.x == 0) a.lse[b] = lse;
    } else {
        // c = LSE + mu: the shift of z = x - c
        float c;
        if constexpr (PIV == 0) {
            c = lse + a.mu[b];
        } else if constexpr (PIV == 1) {
            c = M - a.pivot_offset;
        } else if constexpr (PIV == 4) {
            c = c4;
        } else {
            const float U = block_sum(u, red_u);
            c = M + U * kLn2 / S;
        }
        if constexpr (OP == 2) {
            if (threadIdx.x == 0)
                a.mu_out[b] = (M > -__builtin_inff()) ? (PIV == 0 ? a.mu[b] : c - lse)
                                                      : __builtin_nanf("");
        } else {
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
// the sampling kernels, which share stream_group with this export; one element per thread.
template <int LAY>
__global__ void k_stream_words(const uint64_t *__restrict__ seed,
                               const uint64_t *__restrict__ offset, int64_t B, int64_t V,
                               int32_t k, uint32_t *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = blockIdx.y;
    const uint64_t off = offset[b] + (uint64_t)k;
    Stream st;
    st.row = (uint32_t)b;
    st.off_lo = (uint32_t)off;
    st.off_hi = (uint32_t)(off >> 32);
    st.key0 = (uint32_t)seed[b];
    st.key1 = (uint32_t)(seed[b] >> 32);
    if (i >= V) return;
    out[b * V + i] = element_word<LAY>(st, (uint32_t)i);
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
template hipError_t launch_sample_given<LAY_PLAIN>(int, bool, const SampleArgs &, int, int,
                                                   int, hipStream_t, int *);

hipError_t launch_sample(int dt, bool hlg, int piv, const SampleArgs &a, int nv, int bs,
                         int grid, hipStream_t s, int *occ) {
    const bool scr = a.layout == LAY_SCREENED;
    if (hlg && piv == 3)
        return scr ? launch_sample_rows<LAY_SCREENED>(dt, a, nv, bs, grid, s, occ)
                   : launch_sample_rows<LAY_PLAIN>(dt, a, nv, bs, grid, s, occ);
    if (hlg && piv != 0)
        return scr ? launch_sample_pivot<LAY_SCREENED>(dt, piv, a, nv, bs, grid, s, occ)
                   : launch_sample_pivot<LAY_PLAIN>(dt, piv, a, nv, bs, grid, s, occ);
    return scr ? launch_sample_given<LAY_SCREENED>(dt, hlg, a, nv, bs, grid, s, occ)
               : launch_sample_given<LAY_PLAIN>(dt, hlg, a, nv, bs, grid, s, occ);
}

hipError_t launch_lse_partial(int dt, int piv, const SampleArgs &a, int bs, int grid,
                              hipStream_t s) {
    if (piv == 3) return launch_lse_partial_rows(dt, a, bs, grid, s);
    if (piv != 0) return launch_lse_partial_pivot(dt, piv, a, bs, grid, s);
    return launch_lse_partial_t<0>(dt, a, bs, grid, s);
}

template <int OP, int PIV>
static hipError_t launch_row_op(int dt, const RowOpArgs &a, int grid, hipStream_t s) {
    const int bs = 1024;
    switch (dt) {
        case DT_F32: hipLaunchKernelGGL((k_row_lse<DT_F32, OP, PIV>), dim3(grid), dim3(bs), 0, s, a); break;
        case DT_BF16: hipLaunchKernelGGL((k_row_lse<DT_BF16, OP, PIV>), dim3(grid), dim3(bs), 0, s, a); break;
        case DT_F16: hipLaunchKernelGGL((k_row_lse<DT_F16, OP, PIV>), dim3(grid), dim3(bs), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_row_lse(int dt, int op, int piv, const RowOpArgs &a, int grid, hipStream_t s) {
    if (op == 0) return launch_row_op<0, 0>(dt, a, grid, s);
    if (op == 1) {
        if (piv == 1) return launch_row_op<1, 1>(dt, a, grid, s);
        if (piv == 2) return launch_row_op<1, 2>(dt, a, grid, s);
        if (piv == 4) return launch_row_op<1, 4>(dt, a, grid, s);
        return launch_row_op<1, 0>(dt, a, grid, s);
    }
    if (piv == 1) return launch_row_op<2, 1>(dt, a, grid, s);
    if (piv == 2) return launch_row_op<2, 2>(dt, a, grid, s);
    if (piv == 4) return launch_row_op<2, 4>(dt, a, grid, s);
    return launch_row_op<2, 0>(dt, a, grid, s);
}

hipError_t launch_philox(const uint32_t *ctr, const uint32_t *key, uint32_t *out, int64_t n,
                         hipStream_t s) {
    const int bs = 256;
    const int64_t grid = (n + bs - 1) / bs;
    hipLaunchKernelGGL(k_philox, dim3((unsigned)grid), dim3(bs), 0, s, ctr, key, out, n);
    return hipGetLastError();
}

hipError_t launch_stream_words(const uint64_t *seed, const uint64_t *offset, int64_t B,
                               int64_t V, int32_t k, int32_t layout, uint32_t *out,
                               hipStream_t s) {
    const int bs = 256;
    const int64_t gx = (V + bs - 1) / bs;
    if (B > 65535) return hipErrorInvalidValue;
    if (layout == LAY_SCREENED)
        hipLaunchKernelGGL(k_stream_words<LAY_SCREENED>, dim3((unsigned)gx, (unsigned)B),
                           dim3(bs), 0, s, seed, offset, B, V, k, out);
    else
        hipLaunchKernelGGL(k_stream_words<LAY_PLAIN>, dim3((unsigned)gx, (unsigned)B),
                           dim3(bs), 0, s, seed, offset, B, V, k, out);
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
