// walk_ret_f32.hip -- instantiations of the chunk-walk kernel (see walk_kernel.h).
#include "walk_kernel.h"

namespace ret {

hipError_t launch_walk_ret_f32(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream) {
    return walk::launch_variant<false, false>(a, chunk, dk, nt, stream);
}

bool walk_fits_ret_f32(int chunk, int dk, int nt) { return walk::variant_fits<false, false>(chunk, dk, nt); }

}  // namespace ret
