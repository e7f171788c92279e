// hs_kernels_scr.hip -- the sampling kernel with the curve off or with a given pivot in the screened word layout (element_word):
// a translation unit of its own, so that the library's instantiations compile in parallel.
//
// Sources, cited by page title and section:
//   [HLG]  "HLG sampling -- a piecewise tone curve on the logits" (mlx-bun design document).
//   [GMX]  "Softmax-free GPU sampling: Gumbel-max categorical sampling kernel" (mlxcel #900).
#include <hip/hip_runtime.h>

#include "hs_device.hpp"
#include "hs_internal.hpp"
#include "hs_sample_kernel.hpp"

namespace hs {

template hipError_t launch_sample_given<LAY_SCREENED>(int, bool, const SampleArgs &, int, int,
                                                      int, hipStream_t, int *);

}  // namespace hs
