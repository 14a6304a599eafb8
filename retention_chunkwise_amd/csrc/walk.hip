// walk.hip -- dispatch of the chunk-walk kernel variants (walk_kernel.h) and of
// the segment-split forward (seg_kernel.h).
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

bool walk_variant_fits(bool bf16, bool linattn, int chunk, int dk, int nt) {
    if (bf16) return linattn ? walk_fits_lin_bf16(chunk, dk, nt) : walk_fits_ret_bf16(chunk, dk, nt);
    return linattn ? walk_fits_lin_f32(chunk, dk, nt) : walk_fits_ret_f32(chunk, dk, nt);
}

int choose_walk_nt_wide(int dv, bool bf16, int chunk, int dk, bool linattn) {
    // the fp32 128-token walk with dk = 128 runs out of registers beyond one tile per slice
    if (!bf16 && chunk == 128 && dk == 128) return 1;
    for (int nt = dv / 16; nt > 1; nt /= 2)
        if (walk_variant_fits(bf16, linattn, chunk, dk, nt)) return nt;
    return 1;
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

hipError_t launch_seg_norm(const SegArgs& a, int chunk, int dk, int dv, bool group, hipStream_t stream) {
    if (chunk == 64) return launch_seg_norm_c64(a, dk, dv, group, stream);
    if (chunk == 128) return launch_seg_norm_c128(a, dk, dv, group, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_seg(const SegArgs& a, int chunk, int dk, int dv, bool linattn, hipStream_t stream) {
    if (linattn) {
        if (chunk == 64) return launch_seg_lin_c64(a, dk, dv, stream);
        if (chunk == 128) return launch_seg_lin_c128(a, dk, dv, stream);
        return hipErrorInvalidValue;
    }
    if (chunk == 64) return launch_seg_c64(a, dk, dv, stream);
    if (chunk == 128) return launch_seg_c128(a, dk, dv, stream);
    return hipErrorInvalidValue;
}

int choose_segments(long long bh, int nch, int target_groups, int min_cps, int max_g, int* cps) {
    long long g = (bh > 0) ? (target_groups + bh - 1) / bh : 1;
    const long long by_len = (min_cps > 0) ? nch / min_cps : nch;
    if (g > by_len) g = by_len;
    if (g > max_g) g = max_g;
    if (g < 1) g = 1;
    int c = static_cast<int>((nch + g - 1) / g);
    if (c < 1) c = 1;
    *cps = c;
    const int G = (nch + c - 1) / c;
    return G < 1 ? 1 : G;
}

}  // namespace ret
