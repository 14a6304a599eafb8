// seg_ret_bf16_c128.hip -- segment-split retention forward, bf16, chunk 128.
#include "seg_kernel.h"

namespace ret {

hipError_t launch_seg_c128(const SegArgs& a, int dk, int dv, hipStream_t stream) {
    return seg::launch_chunk<128, seg::kModeRet>(a, dk, dv, stream);
}

}  // namespace ret
