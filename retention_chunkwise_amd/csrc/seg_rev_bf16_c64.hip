// seg_rev_bf16_c64.hip -- time-reversed segment-split retention walk, bf16,
// chunk 64 (the key and value gradients of the backward pass).
#include "seg_kernel.h"

namespace ret {

hipError_t launch_seg_rev_c64(const SegArgs& a, int dk, int dv, hipStream_t stream) {
    return seg::launch_chunk<64, seg::kModeRet, true>(a, dk, dv, stream);
}

}  // namespace ret
