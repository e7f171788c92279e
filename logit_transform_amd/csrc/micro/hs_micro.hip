// hs_micro.hip -- ceilings the sampling kernel is measured against on the same shape: a plain
// streaming read of the logits with the sampler's access pattern (each block reads one row,
// 16-byte loads, eight in flight per lane, and reduces it to its maximum), the same read with
// non-temporal loads (four in flight), and the Philox4x32-10
// word rate with the sampler's counter layout and no memory traffic. Benchmark infrastructure,
// built as a library of its own; the sampling library does not depend on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs_device.hpp"

namespace {

using namespace hs;

typedef unsigned int u4v __attribute__((ext_vector_type(4)));

// Row maximum of [B, V] logits (V a multiple of the vector width, rows 16-byte aligned).
// D loads in flight per lane; NT: loads carry the non-temporal (streaming) cache hint.
template <int DT, int D, bool NT>
__global__ __launch_bounds__(1024) void k_stream_max(const char *x, int64_t ld_bytes,
                                                     int64_t nvec, float *out) {
    constexpr int EPV = dtype_traits<DT>::epv;
    __shared__ float red[16];
    const char *row = x + (int64_t)blockIdx.x * ld_bytes;
    const uint4 *p = reinterpret_cast<const uint4 *>(row);
    float m = -__builtin_inff();
    int64_t v = threadIdx.x;
    for (; v + (D - 1) * 1024 < nvec; v += D * 1024) {
        uint4 buf[D];
#pragma unroll
        for (int j = 0; j < D; ++j) {
            if constexpr (NT) {
                const u4v t = __builtin_nontemporal_load(
                    reinterpret_cast<const u4v *>(p + v + j * 1024));
                buf[j] = make_uint4(t.x, t.y, t.z, t.w);
            } else {
                buf[j] = p[v + j * 1024];
            }
        }
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) m = fmaxf(m, elem<DT>(buf[j], e));
    }
    for (; v < nvec; v += 1024) {
        const uint4 q = p[v];
#pragma unroll
        for (int e = 0; e < EPV; ++e) m = fmaxf(m, elem<DT>(q, e));
    }
    const float bm = block_max(m, red);
    if (threadIdx.x == 0) out[blockIdx.x] = bm;
}

// For every element of a [B, V] row-major layout and draw offsets 0..K-1: the word
// Philox4x32-10 gives it with the sampler's layout (counter (i >> 2, row, offset lo, offset
// hi), key = seed of the row). Block (row, g) of B * groups takes the offsets g, g + groups, ...;
// each lane keeps the maximum of its words, so only the words are computed.
__global__ __launch_bounds__(1024) void k_philox_max(const uint64_t *seed, int64_t ncall,
                                                     int32_t K, int32_t groups, uint32_t *out) {
    const int row = blockIdx.x / groups, g = blockIdx.x % groups;
    const uint64_t s = seed[row];
    const uint32_t k0 = (uint32_t)s, k1 = (uint32_t)(s >> 32);
    uint32_t m = 0;
    for (int k = g; k < K; k += groups) {
        for (int64_t q = threadIdx.x; q < ncall; q += 1024) {
            const Words4 w = philox4x32_10_uk((uint32_t)q, (uint32_t)row, (uint32_t)k, 0u, k0, k1);
            m = max(m, max(max(w.w[0], w.w[1]), max(w.w[2], w.w[3])));
        }
    }
    out[(int64_t)blockIdx.x * 1024 + threadIdx.x] = m;
}

template <int D, bool NT>
int stream_max(const void *x, int32_t dtype, int64_t B, int64_t V, int64_t ld, float *out,
               void *stream) {
    const int es = dtype == 0 ? 4 : 2;
    if (!x || !out || B < 1 || V < 1 || (V * es) % 16 != 0 || ((uintptr_t)x % 16) != 0 ||
        (ld * es) % 16 != 0)
        return -1;
    const int64_t nvec = V * es / 16;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const char *p = reinterpret_cast<const char *>(x);
    switch (dtype) {
        case 0: hipLaunchKernelGGL((k_stream_max<DT_F32, D, NT>), dim3(B), dim3(1024), 0, s, p, ld * es, nvec, out); break;
        case 1: hipLaunchKernelGGL((k_stream_max<DT_BF16, D, NT>), dim3(B), dim3(1024), 0, s, p, ld * es, nvec, out); break;
        case 2: hipLaunchKernelGGL((k_stream_max<DT_F16, D, NT>), dim3(B), dim3(1024), 0, s, p, ld * es, nvec, out); break;
        default: return -1;
    }
    return (int)hipGetLastError();
}

}  // namespace

extern "C" {

// out: device float[B]; x: device [B, ld] logits of dtype (0 f32, 1 bf16, 2 f16), rows
// 16-byte aligned, V a multiple of 16 / element size. Returns 0 or a HIP error code.
int hs_micro_stream_max(const void *x, int32_t dtype, int64_t B, int64_t V, int64_t ld,
                        float *out, void *stream) {
    return stream_max<8, false>(x, dtype, B, V, ld, out, stream);
}

// The same read with the non-temporal cache hint on every load and four loads in flight per
// lane (the fastest plain read of a row per block measured on MI355X).
int hs_micro_stream_max_nt(const void *x, int32_t dtype, int64_t B, int64_t V, int64_t ld,
                           float *out, void *stream) {
    return stream_max<4, true>(x, dtype, B, V, ld, out, stream);
}

// Words for B rows of V elements (V a multiple of 4) and K draws, over B * groups blocks;
// out: device uint32[B * groups * 1024].
int hs_micro_philox_max(const uint64_t *seed, int64_t B, int64_t V, int32_t K, int32_t groups,
                        uint32_t *out, void *stream) {
    if (!seed || !out || B < 1 || V < 4 || V % 4 != 0 || K < 1 || groups < 1 || groups > K ||
        B * groups >= ((int64_t)1 << 31))
        return -1;
    hipLaunchKernelGGL(k_philox_max, dim3(B * groups), dim3(1024), 0,
                       reinterpret_cast<hipStream_t>(stream), seed, V / 4, K, groups, out);
    return (int)hipGetLastError();
}

}  // extern "C"
