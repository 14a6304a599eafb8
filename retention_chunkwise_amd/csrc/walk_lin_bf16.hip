// walk_lin_bf16.hip -- instantiations of the chunk-walk kernel (see walk_kernel.h).
#include "walk_kernel.h"

namespace ret {

hipError_t launch_walk_lin_bf16(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream) {
    return walk::launch_variant<true, true>(a, chunk, dk, nt, stream);
}

bool walk_fits_lin_bf16(int chunk, int dk, int nt) { return walk::variant_fits<true, true>(chunk, dk, nt); }

}  // namespace ret
