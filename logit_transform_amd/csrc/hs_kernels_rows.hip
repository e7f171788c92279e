// hs_kernels_rows.hip -- the sampling kernel and its split-row pre-pass with the curve set per
// row: each row carries its own knobs, pivot mode and on/off switch ([HLG, Knobs; The pivot]:
// settings arrive per request, and one batch mixes requests). A translation unit of its own,
// so that the library's instantiations compile in parallel.
//
// Source: "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document).
#include <hip/hip_runtime.h>

#include "hs_device.hpp"
#include "hs_internal.hpp"
#include "hs_sample_kernel.hpp"

namespace hs {

hipError_t launch_sample_rows(int dt, const SampleArgs &a, int nv, int bs, int grid,
                              hipStream_t s, int *occ) {
    switch (dt) {
        case DT_F32: return launch_sample_al<DT_F32, true, 3>(a, nv, bs, grid, s, occ);
        case DT_BF16: return launch_sample_al<DT_BF16, true, 3>(a, nv, bs, grid, s, occ);
        case DT_F16: return launch_sample_al<DT_F16, true, 3>(a, nv, bs, grid, s, occ);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_lse_partial_rows(int dt, const SampleArgs &a, int bs, int grid,
                                   hipStream_t s) {
    return launch_lse_partial_t<3>(dt, a, bs, grid, s);
}

}  // namespace hs
