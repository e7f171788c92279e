// hs_kernels_pivot.hip -- the sampling kernel and its split-row pre-pass with the curve's
// pivot anchored in the kernel [HLG, The pivot]: top-anchored (mu = l_max - c) and
// entropy-anchored (mu = sum p l), and the mass median's shift, in the plain word layout. A
// translation unit of its own, so that the library's instantiations compile in parallel.
//
// Source: "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document).
#include <hip/hip_runtime.h>

#include "hs_device.hpp"
#include "hs_internal.hpp"
#include "hs_sample_kernel.hpp"

namespace hs {

template hipError_t launch_sample_pivot<LAY_PLAIN>(int, int, const SampleArgs &, int, int,
                                                   int, hipStream_t, int *);

hipError_t launch_lse_partial_pivot(int dt, int piv, const SampleArgs &a, int bs, int grid,
                                    hipStream_t s) {
    return piv == 1 ? launch_lse_partial_t<1>(dt, a, bs, grid, s)
                    : launch_lse_partial_t<2>(dt, a, bs, grid, s);
}

}  // namespace hs
