// rrp_sweep_bf16.hip -- the support sweep's kernels for bf16 K rows.
#include "rrp_sweep.hpp"

namespace rrp {

hipError_t launch_sweep_bf16(const StatsArgs& a, int n_blocks, int head_dim, int layout, hipStream_t st) {
    return launch_sweep_e<bf16_tag>(a, n_blocks, head_dim, layout, st);
}

}  // namespace rrp
