// seg_ret_bf16_c64.hip -- segment-split retention forward, bf16, chunk 64.
#include "seg_kernel.h"

namespace ret {

hipError_t launch_seg_c64(const SegArgs& a, int dk, int dv, hipStream_t stream) {
    return seg::launch_chunk<64, seg::kModeRet>(a, dk, dv, stream);
}

}  // namespace ret
