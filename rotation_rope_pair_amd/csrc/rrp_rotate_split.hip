// rrp_rotate_split.hip -- the rotate + quantise kernel for small batches
// (fewer than 4096 tokens, e.g. one decode step): each token's row passes are
// split over several waves.  Compiled on its own so the two kernel families
// build in parallel.
#include "rrp_rotate_kernel.hpp"

namespace rrp {

hipError_t launch_rotate_quantize_split(const RotateArgs& a, int dtype, int head_dim, int layout, hipStream_t st) {
    return dispatch<true>(a, dtype, head_dim, layout, st);
}

}  // namespace rrp
