// rownorm.hip -- GroupNorm over each output row in place (fp32), for the
// normalised forwards whose rows span several value slices of the walk.
//
// Each row of dv values (one head's features at one token) becomes
// (x - mean) / sqrt(var + eps), population variance, no gain or bias: the
// reading of the RetNet layer's optional GroupNorm with one group per head.
// One wave per row, grid-stride; dv / 64 values per lane, reductions by
// cross-lane shuffles.  Statistics in fp32, as in the fused walks; the row is
// in registers, so the variance takes two passes (mean, then squared
// deviations), exact for rows whose mean is large against their spread.
#include "internal.h"

namespace ret {
namespace {

constexpr int kRowThreads = 256;

template <int DV>
__global__ void __launch_bounds__(kRowThreads) group_norm_rows_kernel(float* out, long long rows, float eps) {
    constexpr int PER = DV / 64;
    const int lane = threadIdx.x & 63;
    const long long wave = (static_cast<long long>(blockIdx.x) * kRowThreads + threadIdx.x) >> 6;
    const long long waves = (static_cast<long long>(gridDim.x) * kRowThreads) >> 6;
    for (long long r = wave; r < rows; r += waves) {
        float* row = out + r * DV;
        float x[PER];
        float s1 = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            x[i] = row[lane + 64 * i];
            s1 += x[i];
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) s1 += __shfl_xor(s1, o);
        const float mu = s1 * (1.f / DV);
        float s2 = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) s2 += (x[i] - mu) * (x[i] - mu);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) s2 += __shfl_xor(s2, o);
        const float rstd = 1.f / sqrtf(s2 * (1.f / DV) + eps);
#pragma unroll
        for (int i = 0; i < PER; ++i) row[lane + 64 * i] = (x[i] - mu) * rstd;
    }
}

}  // namespace

hipError_t launch_group_norm_rows_f32(float* out, long long rows, int dv, float eps, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const long long waves_needed = rows;
    long long blocks = (waves_needed + (kRowThreads / 64) - 1) / (kRowThreads / 64);
    if (blocks > 8192) blocks = 8192;  // grid-stride beyond this
    if (dv == 64) {
        hipLaunchKernelGGL((group_norm_rows_kernel<64>), dim3(static_cast<unsigned>(blocks)), dim3(kRowThreads), 0,
                           stream, out, rows, eps);
    } else if (dv == 128) {
        hipLaunchKernelGGL((group_norm_rows_kernel<128>), dim3(static_cast<unsigned>(blocks)), dim3(kRowThreads), 0,
                           stream, out, rows, eps);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ret
