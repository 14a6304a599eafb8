// gla.hip -- chunkwise gated linear attention (per-token, per-key-channel
// gates), fp32, gfx950.
//
// What is computed ("Efficient and Sparse Transformers", section "Gated
// Linear Attention: Toward Input-Dependent Forgetting": the fixed decay of
// RetNet becomes a data-dependent gate applied element-wise to the state; here
// one gate per key channel, alpha_t = exp(lg_t)):
//   S_t[c][n] = alpha_t[c] S_{t-1}[c][n] + k_t[c] v_t[n],   o_t = q_t S_t.
// Chunk form.  With b_i[c] the log-gates summed over the chunk up to and
// including its token i, and S the state before the chunk:
//   o_i   = sum_{j<=i} sum_c q_i[c] k_j[c] e^{b_i[c] - b_j[c]} v_j + sum_c q_i[c] e^{b_i[c]} S[c][:]
//   S_new = diag(e^{b_last}) S + sum_j diag(e^{b_last - b_j}) k_j v_j^T
// Every exponent used is <= 0, so nothing overflows:
//  - key tile J before query tile I: with e_J the last token of tile J,
//    e^{b_i - b_j} = e^{b_i - b_{e_J}} e^{b_{e_J} - b_j}, both factors <= 1,
//    folded into the Q and K operands of an fp32 MFMA;
//  - the diagonal tiles (i, j in one 16-token tile) are summed directly, one
//    exponent per term;
//  - the inter-chunk and state products scale Q by e^{b_i} and K by
//    e^{b_last - b_j}.
// A gate of 0 (lg = -inf) closes a channel exactly.
//
// Mapping.  One workgroup (4 waves) per (b, h, slice of 16 NT value columns)
// walks all chunks of 64 tokens; wave W owns query tile W and state tiles
// {W, W + 4, ...} of the slice.  The chunk's q, k, cumulative gates and the
// value slice are staged in LDS (padded fp32 rows); S^T is copied to LDS for
// the next chunk's inter-chunk product.  This first version walks whole
// sequences (no segment split) and does not overlap loads with compute.
#include "internal.h"
#include "kcommon.h"

namespace ret {
namespace gla {
namespace {

using namespace ::ret::kc;

constexpr int kThreads = 256;
constexpr int C = 64;

template <int DK, int NT>
struct Cfg {
    static constexpr int KSTR = DK + 4;    // padded row stride of q, k, gates
    static constexpr int DVS = 16 * NT;    // value columns per workgroup
    static constexpr int VSTR = DVS + 4;   // padded row stride of the value slice
    static constexpr int KT = DK / 16;
    static constexpr int SPW = NT * KT / 4;  // state tiles per wave
    static_assert(NT * KT % 4 == 0, "state tiles split over 4 waves");
};

template <int DK, int NT>
struct Smem {
    using Cf = Cfg<DK, NT>;
    alignas(16) float q[C * Cf::KSTR];
    alignas(16) float k[C * Cf::KSTR];
    alignas(16) float b[C * Cf::KSTR];     // log-gates, then their running sums over the chunk
    alignas(16) float v[C * Cf::VSTR];
    alignas(16) float st[Cf::DVS * Cf::KSTR];  // S^T copy: st[n][c] = S[c][nbase + n]
};

template <int DK, int NT>
constexpr bool fits() { return sizeof(Smem<DK, NT>) <= 160 * 1024; }

template <int DK, int NT, int W>
__device__ __forceinline__ void body(const GlaArgs& a, Smem<DK, NT>& sm, int bh, int nbase) {
    using Cf = Cfg<DK, NT>;
    constexpr int KSTR = Cf::KSTR, VSTR = Cf::VSTR, KT = Cf::KT, SPW = Cf::SPW, DVS = Cf::DVS;
    const int T = a.T, DV = a.dv;
    const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, g = l >> 4;
    const float* qh = a.q + static_cast<long long>(bh) * T * DK;
    const float* kh = a.k + static_cast<long long>(bh) * T * DK;
    const float* gh = a.lg + static_cast<long long>(bh) * T * DK;
    const float* vh = a.v + static_cast<long long>(bh) * T * DV + nbase;
    float* oh = a.out + static_cast<long long>(bh) * T * DV + nbase;
    constexpr int I = W;  // query tile

    f32x4 sacc[SPW];  // S[16 kt + l16][nbase + 16 nt + 4g + r], tile W + 4m = (nt, kt)
#pragma unroll
    for (int m = 0; m < SPW; ++m) sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nch = (T + C - 1) / C;
    for (int c = 0; c < nch; ++c) {
        const long long t0 = static_cast<long long>(c) * C;
        const int clen = (T - t0 < C) ? static_cast<int>(T - t0) : C;
        __syncthreads();  // the previous chunk's reads of q, k, b, v are done

        // ---- stage the chunk (rows past the end: zeros, gate 1)
        for (int u = tid; u < C * DK / 4; u += kThreads) {
            const int r = u / (DK / 4), c4 = 4 * (u % (DK / 4));
            f32x4 xq = {0.f, 0.f, 0.f, 0.f}, xk = xq, xg = xq;
            if (r < clen) {
                const long long o = (t0 + r) * DK + c4;
                xq = *reinterpret_cast<const f32x4*>(qh + o);
                xk = *reinterpret_cast<const f32x4*>(kh + o);
                xg = *reinterpret_cast<const f32x4*>(gh + o);
            }
            *reinterpret_cast<f32x4*>(&sm.q[r * KSTR + c4]) = xq;
            *reinterpret_cast<f32x4*>(&sm.k[r * KSTR + c4]) = xk;
            *reinterpret_cast<f32x4*>(&sm.b[r * KSTR + c4]) = xg;
        }
        for (int u = tid; u < C * DVS / 4; u += kThreads) {
            const int r = u / (DVS / 4), c4 = 4 * (u % (DVS / 4));
            f32x4 xv = {0.f, 0.f, 0.f, 0.f};
            if (r < clen) xv = *reinterpret_cast<const f32x4*>(vh + (t0 + r) * DV + c4);
            *reinterpret_cast<f32x4*>(&sm.v[r * VSTR + c4]) = xv;
        }
        __syncthreads();
        // ---- running sums of the log-gates down each key channel
        if (tid < DK) {
            float acc = 0.f;
            for (int r = 0; r < C; ++r) {
                acc += sm.b[r * KSTR + tid];
                sm.b[r * KSTR + tid] = acc;
            }
        }
        __syncthreads();

        const int qi = 16 * I + l16;  // this lane's query row
        // ---- scores S^T[j][i] for key tiles J <= I: lane holds keys 16J + 4g + r of query qi
        f32x4 pacc[I + 1];
#pragma unroll
        for (int J = 0; J < I; ++J) {
            pacc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int eJ = 16 * J + 15, kj = 16 * J + l16;
#pragma unroll 4
            for (int s = 0; s < DK / 4; ++s) {
                const int ch = 4 * s + g;
                const float be = sm.b[eJ * KSTR + ch];
                const float ka = sm.k[kj * KSTR + ch] * __expf(be - sm.b[kj * KSTR + ch]);
                const float qb = sm.q[qi * KSTR + ch] * __expf(sm.b[qi * KSTR + ch] - be);
                pacc[J] = mfma_f32(ka, qb, pacc[J]);
            }
        }
        {
            // diagonal tile: one exponent per term, keys after the query masked
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * I + 4 * g + r;
                if (j <= qi) {
                    float acc = 0.f;
                    for (int ch = 0; ch < DK; ++ch)
                        acc += sm.q[qi * KSTR + ch] * sm.k[j * KSTR + ch] *
                               __expf(sm.b[qi * KSTR + ch] - sm.b[j * KSTR + ch]);
                    d[r] = acc;
                }
            }
            pacc[I] = d;
        }

        // ---- O^T = S_prev^T (Q e^{b})^T + V^T P^T, 16-byte stores of rows qi
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int s = 0; s < DK / 4; ++s) {
                const int ch = 4 * s + g;
                const float sa = sm.st[(16 * nt + l16) * KSTR + ch];
                const float qb = sm.q[qi * KSTR + ch] * __expf(sm.b[qi * KSTR + ch]);
                o = mfma_f32(sa, qb, o);
            }
#pragma unroll
            for (int J = 0; J <= I; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o = mfma_f32(sm.v[(16 * J + 4 * g + r) * VSTR + 16 * nt + l16], pacc[J][r], o);
            if (qi < clen) *reinterpret_cast<f32x4*>(oh + (t0 + qi) * DV + 16 * nt + 4 * g) = o;
        }

        // ---- S = diag(e^{b_last}) S + sum_j diag(e^{b_last - b_j}) k_j v_j^T
        const int last = clen - 1;
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = W + 4 * m, nt = qt / KT, kt = qt % KT;
            const int ch = 16 * kt + l16;
            const float bl = sm.b[last * KSTR + ch];
            sacc[m] *= __expf(bl);
#pragma unroll
            for (int J = 0; J < C / 16; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * J + 4 * g + r;
                    const float kb = sm.k[j * KSTR + ch] * __expf(bl - sm.b[j * KSTR + ch]);
                    sacc[m] = mfma_f32(sm.v[j * VSTR + 16 * nt + l16], kb, sacc[m]);
                }
        }
        __syncthreads();  // every wave is done reading the old state copy
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = W + 4 * m, nt = qt / KT, kt = qt % KT;
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.st[(16 * nt + 4 * g + r) * KSTR + 16 * kt + l16] = sacc[m][r];
        }
    }

    if (a.final_state) {
        float* fs = a.final_state + static_cast<long long>(bh) * DK * DV + nbase;
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = W + 4 * m, nt = qt / KT, kt = qt % KT;
            *reinterpret_cast<f32x4*>(fs + (16 * kt + l16) * DV + 16 * nt + 4 * g) = sacc[m];
        }
    }
}

template <int DK, int NT>
__global__ void __launch_bounds__(kThreads, 1) gla_kernel(const GlaArgs a) {
    __shared__ Smem<DK, NT> sm;
    const int bh = blockIdx.x / a.nslices;
    const int nbase = (blockIdx.x % a.nslices) * Cfg<DK, NT>::DVS;
    for (int m = threadIdx.x; m < Cfg<DK, NT>::DVS * Cfg<DK, NT>::KSTR; m += kThreads) sm.st[m] = 0.f;
    // (the first barrier of the chunk loop orders this before any read)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    switch (wave) {
        case 0: body<DK, NT, 0>(a, sm, bh, nbase); break;
        case 1: body<DK, NT, 1>(a, sm, bh, nbase); break;
        case 2: body<DK, NT, 2>(a, sm, bh, nbase); break;
        default: body<DK, NT, 3>(a, sm, bh, nbase); break;
    }
}

template <int DK, int NT>
hipError_t launch_t(const GlaArgs& a, hipStream_t stream) {
    if constexpr (!fits<DK, NT>()) {
        return hipErrorInvalidConfiguration;
    } else {
        const long long groups = static_cast<long long>(a.B) * a.H * a.nslices;
        if (groups <= 0) return hipSuccess;
        if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gla_kernel<DK, NT>), dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    }
}

}  // namespace
}  // namespace gla

int gla_choose_nt(long long bh, int dv) {
    // wide slices (fewer recomputed scores) while there are enough workgroups
    if (dv % 64 == 0 && bh * (dv / 64) >= 256) return 4;
    if (dv % 32 == 0 && bh * (dv / 32) >= 256) return 2;
    return 1;
}

hipError_t launch_gla(const GlaArgs& a, int dk, int nt, hipStream_t stream) {
    if (dk == 64 && nt == 1) return gla::launch_t<64, 1>(a, stream);
    if (dk == 64 && nt == 2) return gla::launch_t<64, 2>(a, stream);
    if (dk == 64 && nt == 4) return gla::launch_t<64, 4>(a, stream);
    if (dk == 128 && nt == 1) return gla::launch_t<128, 1>(a, stream);
    if (dk == 128 && nt == 2) return gla::launch_t<128, 2>(a, stream);
    if (dk == 128 && nt == 4) return gla::launch_t<128, 4>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace ret
