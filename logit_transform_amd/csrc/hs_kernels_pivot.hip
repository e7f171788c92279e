// hs_kernels_pivot.hip -- the sampling kernel and its split-row pre-pass with the curve's
// pivot anchored in the kernel [HLG, The pivot]: top-anchored (mu = l_max - c) and
// entropy-anchored (mu = sum p l). A translation unit of its own, so that the library's
// instantiations compile in parallel.
//
// Source: "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document).
#include <hip/hip_runtime.h>

#include "hs_device.hpp"
#include "hs_internal.hpp"
#include "hs_sample_kernel.hpp"

namespace hs {

hipError_t launch_sample_pivot(int dt, int piv, const SampleArgs &a, int nv, int bs, int grid,
                               hipStream_t s, int *occ) {
    switch (dt) {
        case DT_F32:
            return piv == 1 ? launch_sample_al<DT_F32, true, 1>(a, nv, bs, grid, s, occ)
                 : piv == 4 ? launch_sample_al<DT_F32, true, 4>(a, nv, bs, grid, s, occ)
                            : launch_sample_al<DT_F32, true, 2>(a, nv, bs, grid, s, occ);
        case DT_BF16:
            return piv == 1 ? launch_sample_al<DT_BF16, true, 1>(a, nv, bs, grid, s, occ)
                 : piv == 4 ? launch_sample_al<DT_BF16, true, 4>(a, nv, bs, grid, s, occ)
                            : launch_sample_al<DT_BF16, true, 2>(a, nv, bs, grid, s, occ);
        case DT_F16:
            return piv == 1 ? launch_sample_al<DT_F16, true, 1>(a, nv, bs, grid, s, occ)
                 : piv == 4 ? launch_sample_al<DT_F16, true, 4>(a, nv, bs, grid, s, occ)
                            : launch_sample_al<DT_F16, true, 2>(a, nv, bs, grid, s, occ);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_lse_partial_pivot(int dt, int piv, const SampleArgs &a, int bs, int grid,
                                    hipStream_t s) {
    return piv == 1 ? launch_lse_partial_t<1>(dt, a, bs, grid, s)
                    : launch_lse_partial_t<2>(dt, a, bs, grid, s);
}

}  // namespace hs
