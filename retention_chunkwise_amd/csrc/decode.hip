// decode.hip -- recurrent decode steps on gfx950.
//
// Retention, for every (sequence, head): S <- gamma S + k v^T, then o = q S,
// reading the output from the updated state ("RetNet", "Recurrent
// Representation"; "Efficient and Sparse Transformers", section 6, recurrent
// form and its minimal recurrent step).  S is fp32, dk x dv, updated in place.
//
// Linear attention with phi = elu+1 ("Linear attention", the decode-step
// exercise): S <- S + phi(k) v^T, z <- z + phi(k), then
// o = S^T phi(q) / (z^T phi(q) + eps) from the updated pair; S and z are fp32
// and updated in place.  The same kernel runs it with gamma = 1, phi applied
// to q and k as they are staged, and the denominator reduced by wave 0.
//
// The step is bound by HBM: each state element is read once and written once
// and takes two FMAs.  One workgroup streams one state tile.  Thread t owns
// four adjacent value columns (one 16-byte vector) of every 8th (dv = 128) row,
// so each wave reads two whole 512-byte rows per load instruction.  All loads
// of a thread are issued before any arithmetic; loads and stores bypass the
// caches' retention policy (non-temporal), since the state is far larger than
// the L2 and is not re-read within the step.  The column sums of q_k S[k][:]
// are reduced across row phases through LDS.
#include "internal.h"

namespace ret {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, long long i) {
    if constexpr (BF16) {
        const unsigned short b = static_cast<const unsigned short*>(p)[i];
        return __uint_as_float(static_cast<unsigned>(b) << 16);
    } else {
        return static_cast<const float*>(p)[i];
    }
}

// elu(x) + 1: x + 1 for x > 0, e^x otherwise
__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : expf(x); }

template <bool BF16, int DK, int DV, bool LIN>
__global__ void __launch_bounds__(kThreads) decode_kernel(const DecodeArgs a) {
    constexpr int CG = DV / 4;          // 16-byte column groups per row
    constexpr int RP = kThreads / CG;   // row phases
    constexpr int RPT = DK / RP;        // rows per thread
    static_assert(RPT * RP == DK, "rows must split evenly");

    __shared__ float qs[DK];
    __shared__ float ks[DK];
    __shared__ float vs[DV];
    __shared__ __attribute__((aligned(16))) float red[RP][DV];
    __shared__ float den_s;  // linear attention: z^T phi(q) + eps

    const int tid = threadIdx.x;
    const long long nh = blockIdx.x;
    const float gam = LIN ? 1.f : a.gamma[nh % a.H];
    const int cg = tid % CG, rp = tid / CG;
    float* S = a.state + nh * DK * DV;

    // stream this thread's part of the state in first
    f32x4 sv[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rp + m * RP;
        sv[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + row * DV + 4 * cg));
    }
    constexpr int ZPT = LIN ? DK / 64 : 1;  // normaliser entries per wave-0 lane
    float zr[ZPT];
    if constexpr (LIN) {
        if (tid < 64) {
#pragma unroll
            for (int u = 0; u < ZPT; ++u) zr[u] = a.z[nh * DK + tid + 64 * u];
        }
    }
    for (int i = tid; i < 2 * DK + DV; i += kThreads) {
        if (i < DK) {
            const float x = load_elem<BF16>(a.q, nh * DK + i);
            qs[i] = LIN ? phi_elu1(x) : x;
        } else if (i < 2 * DK) {
            const float x = load_elem<BF16>(a.k, nh * DK + (i - DK));
            ks[i - DK] = LIN ? phi_elu1(x) : x;
        } else {
            vs[i - 2 * DK] = load_elem<BF16>(a.v, nh * DV + (i - 2 * DK));
        }
    }
    __syncthreads();

    if constexpr (LIN) {
        // z <- z + phi(k); denominator z^T phi(q) + eps, reduced across wave 0
        if (tid < 64) {
            float part = 0.f;
#pragma unroll
            for (int u = 0; u < ZPT; ++u) {
                const int i = tid + 64 * u;
                const float zn = zr[u] + ks[i];
                a.z[nh * DK + i] = zn;
                part = fmaf(zn, qs[i], part);
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
            if (tid == 0) den_s = part + a.eps;
        }
    }

    const f32x4 vv = *reinterpret_cast<const f32x4*>(&vs[4 * cg]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rp + m * RP;
        const float kk = ks[row], qq = qs[row];
        f32x4 s;
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = fmaf(gam, sv[m][e], kk * vv[e]);
        __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(S + row * DV + 4 * cg));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(qq, s[e], acc[e]);
    }
    *reinterpret_cast<f32x4*>(&red[rp][4 * cg]) = acc;
    __syncthreads();
    for (int n = tid; n < DV; n += kThreads) {
        float o = 0.f;
#pragma unroll
        for (int r = 0; r < RP; ++r) o += red[r][n];
        if constexpr (LIN) o /= den_s;
        if constexpr (BF16) {
            static_cast<unsigned short*>(a.out)[nh * DV + n] =
                __builtin_bit_cast(unsigned short, static_cast<__bf16>(o));
        } else {
            static_cast<float*>(a.out)[nh * DV + n] = o;
        }
    }
}

template <bool BF16, int DK, int DV, bool LIN>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    const long long groups = static_cast<long long>(a.N) * a.H;
    if (groups <= 0) return hipSuccess;
    if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_kernel<BF16, DK, DV, LIN>), dim3(static_cast<unsigned>(groups)),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <bool BF16, bool LIN>
hipError_t launch_b(const DecodeArgs& a, int dk, int dv, hipStream_t stream) {
    if (dk == 64 && dv == 64) return launch_t<BF16, 64, 64, LIN>(a, stream);
    if (dk == 64 && dv == 128) return launch_t<BF16, 64, 128, LIN>(a, stream);
    if (dk == 128 && dv == 64) return launch_t<BF16, 128, 64, LIN>(a, stream);
    if (dk == 128 && dv == 128) return launch_t<BF16, 128, 128, LIN>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t stream) {
    return bf16 ? launch_b<true, false>(a, dk, dv, stream) : launch_b<false, false>(a, dk, dv, stream);
}

hipError_t launch_decode_lin(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t stream) {
    return bf16 ? launch_b<true, true>(a, dk, dv, stream) : launch_b<false, true>(a, dk, dv, stream);
}

}  // namespace ret
