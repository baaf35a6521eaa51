// rrp_sweep_f32.hip -- the support sweep's kernels for fp32 K rows.
#include "rrp_sweep.hpp"

namespace rrp {

hipError_t launch_sweep_f32(const StatsArgs& a, int n_blocks, int head_dim, int layout, hipStream_t st) {
    return launch_sweep_e<float>(a, n_blocks, head_dim, layout, st);
}

}  // namespace rrp
