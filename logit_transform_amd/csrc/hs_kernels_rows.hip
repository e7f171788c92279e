// hs_kernels_rows.hip -- the sampling kernel and its split-row pre-pass with the curve set per
// row: each row carries its own knobs, pivot mode and on/off switch ([HLG, Knobs; The pivot]:
// settings arrive per request, and one batch mixes requests), in the plain word layout. A
// translation unit of its own, so that the library's instantiations compile in parallel.
//
// Source: "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document).
#include <hip/hip_runtime.h>

#include "hs_device.hpp"
#include "hs_internal.hpp"
#include "hs_sample_kernel.hpp"

namespace hs {

template hipError_t launch_sample_rows<LAY_PLAIN>(int, const SampleArgs &, int, int, int,
                                                  hipStream_t, int *);

hipError_t launch_lse_partial_rows(int dt, const SampleArgs &a, int bs, int grid,
                                   hipStream_t s) {
    return launch_lse_partial_t<3>(dt, a, bs, grid, s);
}

}  // namespace hs
