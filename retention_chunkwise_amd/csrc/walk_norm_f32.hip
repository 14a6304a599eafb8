// walk_norm_f32.hip -- instantiations of the chunk-walk kernel (see walk_kernel.h)
// for fp32 retention with the row-sum floor (mode 2) and the floor plus
// GroupNorm (mode 3).
#include "walk_kernel.h"

namespace ret {

hipError_t launch_walk_norm_f32(const WalkArgs& a, int chunk, int dk, int nt, bool group, hipStream_t stream) {
    return group ? walk::launch_variant<false, 3>(a, chunk, dk, nt, stream)
                 : walk::launch_variant<false, 2>(a, chunk, dk, nt, stream);
}

}  // namespace ret
