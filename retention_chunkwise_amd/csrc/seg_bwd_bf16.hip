// seg_bwd_bf16.hip -- fused reverse walk of the backward pass (dk and dv), bf16, chunk 64.
#include "seg_bwd.h"

namespace ret {

hipError_t launch_seg_bwd_kv(const SegArgs& a, int dk, int dv, hipStream_t stream) {
    if (dk == 64 && dv == 64) return seg::launch_bwd_kv_t<64, 64>(a, stream);
    if (dk == 64 && dv == 128) return seg::launch_bwd_kv_t<64, 128>(a, stream);
    if (dk == 128 && dv == 64) return seg::launch_bwd_kv_t<128, 64>(a, stream);
    if (dk == 128 && dv == 128) return seg::launch_bwd_kv_t<128, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace ret
