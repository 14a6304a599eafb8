// seg_lin_bf16_c128.hip -- segment-split elu+1 linear attention, bf16, chunk 128.
#include "seg_kernel.h"

namespace ret {

hipError_t launch_seg_lin_c128(const SegArgs& a, int dk, int dv, hipStream_t stream) {
    return seg::launch_chunk<128, seg::kModeLin>(a, dk, dv, stream);
}

}  // namespace ret
