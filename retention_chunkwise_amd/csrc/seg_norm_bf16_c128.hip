// seg_norm_bf16_c128.hip -- segment-split retention with the row-sum floor
// (and optionally GroupNorm) fused into the output, bf16, chunk 128.
#include "seg_kernel.h"

namespace ret {

hipError_t launch_seg_norm_c128(const SegArgs& a, int dk, int dv, bool group, hipStream_t stream) {
    return group ? seg::launch_chunk<128, seg::kModeGroup>(a, dk, dv, stream)
                 : seg::launch_chunk<128, seg::kModeNorm>(a, dk, dv, stream);
}

}  // namespace ret
