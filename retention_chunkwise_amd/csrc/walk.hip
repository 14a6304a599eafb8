// walk.hip -- dispatch of the chunk-walk kernel variants (see walk_kernel.h).
#include "internal.h"

namespace ret {

int choose_walk_nt(long long bh, int dv, int target_groups, bool bf16, int chunk, int dk) {
    // widest value slice (fewer recomputed Q K^T tiles) that still yields
    // enough workgroups to occupy every compute unit; the bf16 variant with
    // chunk 128, dk 128 and 32-column slices does not fit in LDS
    if (bf16 && chunk == 128 && dk == 128) return 1;
    int best = 1;
    if (dv % 32 == 0 && bh * (dv / 32) >= target_groups) best = 2;
    return best;
}

hipError_t launch_walk(const WalkArgs& a, bool bf16, int chunk, int dk, int nt, bool linattn,
                       hipStream_t stream) {
    if (bf16) {
        return linattn ? launch_walk_lin_bf16(a, chunk, dk, nt, stream)
                       : launch_walk_ret_bf16(a, chunk, dk, nt, stream);
    }
    return linattn ? launch_walk_lin_f32(a, chunk, dk, nt, stream)
                   : launch_walk_ret_f32(a, chunk, dk, nt, stream);
}

}  // namespace ret
