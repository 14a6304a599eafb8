// walk.hip -- chunkwise causal retention / elu+1 linear attention on gfx950.
//
// What is computed ("RetNet", single-head definition O = (Q K^T (.) D) V,
// D_nm = gamma^(n-m) for n >= m, and "Chunked Recurrent Representation";
// "Efficient and Sparse Transformers" section 6, "Chunkwise form"):
// the sequence is cut into chunks of C tokens.  With S the fp32 dk x dv state
// before a chunk, local indices i, j in [0, c) and c <= C the chunk length,
//   O_i   = sum_{j<=i} gamma^(i-j) (q_i . k_j) v_j  +  gamma^(i+1) q_i S
//   S_new = gamma^c S + sum_j gamma^(c-1-j) k_j v_j^T
// (obtained by unrolling S_t = gamma S_{t-1} + k_t v_t^T inside the chunk).
// Linear attention ("Linear attention", box "Causal linear attention,
// recurrent form") is the same walk with gamma = 1, phi = elu+1 applied to q
// and k, and the normaliser z carried beside S:
//   O_i = (intra_i + phi(q_i) S) / (rowsum_i + phi(q_i) . z + eps),
//   z_new = z + sum_j phi(k_j).
//
// Mapping onto the chip.  One workgroup (4 waves, 256 threads) owns one
// (batch, head) pair and one slice of 16*NT value columns, and walks every
// chunk of the sequence in order, keeping its slice of S in registers (fp32).
// Value columns of S and O are independent, so slices need no communication;
// each slice recomputes Q K^T for its chunk.  Slices of one (b, h) are placed
// on the same XCD so their shared Q / K reads hit that XCD's L2.
//
// Per chunk, wave w owns query tiles {w, C/16-1-w} (16 rows each; one tile
// when C = 64), which balances the causal triangle across waves.  All
// contractions run on MFMA (bf16: v_mfma_f32_16x16x32_bf16, fp32:
// v_mfma_f32_16x16x4f32) with fp32 accumulation:
//   S^T_tile = K Q^T      A = K rows (LDS), B = Q rows (registers)
//   P^T      = S^T (.) D  decay factors from a per-head LDS table, masked
//   O^T     += S_prev^T (xi Q)^T   A = state copy (LDS), B = Q (registers)
//   O^T     += V^T P^T    A = V slice packed 4 tokens deep (LDS), B = P^T
//   S^T      = gamma^c S^T + (zeta V)^T K
// Computing the transposed products lets the output of the Q K^T MFMA feed the
// P V MFMA directly from registers (each lane holds 4 consecutive keys of one
// query), so P never goes through LDS.  The next chunk's K, V and Q are loaded
// from HBM into registers while the current chunk computes.
#include "internal.h"

namespace ret {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ float bf2f(unsigned short b) {
    return __uint_as_float(static_cast<unsigned>(b) << 16);
}

__device__ __forceinline__ unsigned short f2bf(float f) {
    return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

// phi(x) = elu(x) + 1: x + 1 for x > 0, e^x otherwise.
__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : expf(x); }

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 cat_bf16(const u16x4& lo, const u16x4& hi) {
    u16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ u16x4 cvt4_bf16(const f32x4& x) {
    return __builtin_bit_cast(u16x4, __builtin_convertvector(x, bf16x4));
}

__device__ __forceinline__ float sum_over_groups(float x) {
    // lanes l, l^16, l^32, l^48 hold the four 4-row groups of one column
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

template <bool BF16, int C, int DK, int NT, bool LIN>
struct WalkCfg {
    static constexpr int NI = C / 16;                 // 16-token tiles per chunk
    static constexpr int NS = (NI == 8) ? 2 : 1;      // query tiles per wave
    static constexpr int DVS = 16 * NT;               // value columns per workgroup
    static constexpr int ESZ = BF16 ? 2 : 4;          // element bytes
    static constexpr int KPAD = 16 / ESZ;             // 16-byte row padding
    static constexpr int KSTR = DK + KPAD;            // row stride of K / state copy
    static constexpr int KT = DK / 16;                // 16-wide key tiles
    static constexpr int SPW = NT * KT / 4;           // state tiles per wave
    static constexpr int KU = C * DK * ESZ / 16 / kThreads;  // 16-B K units per thread
    static constexpr int RU = DK * ESZ / 16;          // 16-B units per K row
    static constexpr int VCOLS = 16 / ESZ;            // value columns per 16-B load
    static constexpr int VU = (C / 4) * (DVS / VCOLS);  // V staging units (<= 256)
    static constexpr int QU = DK * ESZ / 64;          // 16-B Q units per lane per tile
    static constexpr int DEC = C + 32;                // decay table entries
    static_assert(NI == 4 || NI == 8, "chunk must be 64 or 128");
    static_assert(DK == 64 || DK == 128, "dk must be 64 or 128");
    static_assert(NT * KT % 4 == 0, "state tiles must split over 4 waves");
    static_assert(C * DK * ESZ / 16 % kThreads == 0, "K staging split");
    static_assert(VU <= kThreads, "V staging split");
};

template <bool BF16, int C, int DK, int NT, bool LIN>
__global__ void __launch_bounds__(kThreads, 1) walk_kernel(const WalkArgs a) {
    using Cfg = WalkCfg<BF16, C, DK, NT, LIN>;
    constexpr int NI = Cfg::NI, NS = Cfg::NS, DVS = Cfg::DVS, KSTR = Cfg::KSTR;
    constexpr int KT = Cfg::KT, SPW = Cfg::SPW, KU = Cfg::KU, RU = Cfg::RU;
    constexpr int VCOLS = Cfg::VCOLS, VU = Cfg::VU, QU = Cfg::QU, DEC = Cfg::DEC;
    typedef typename std::conditional<BF16, unsigned short, float>::type E;

    __shared__ __attribute__((aligned(16))) E Ks[C * KSTR];          // K (or phi(K)) rows
    __shared__ __attribute__((aligned(16))) E V4s[C * DVS];          // V slice, [j/4][n][4]
    __shared__ __attribute__((aligned(16))) E V4z[C * DVS];          // zeta-scaled copy
    __shared__ __attribute__((aligned(16))) E Sts[2][DVS * KSTR];    // S^T copy, [n][k]
    __shared__ __attribute__((aligned(16))) float dec[DEC];          // [16 + m] = gamma^m
    __shared__ __attribute__((aligned(16))) float zs[2][LIN ? DK : 4];

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;

    // workgroup -> (b*H + h, value slice); slices of one (b, h) share an XCD
    int L = blockIdx.x;
    if (a.xcd_remap) {
        const int per = gridDim.x >> 3;
        L = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    }
    const int bh = L / a.nslices;
    const int nbase = (L % a.nslices) * DVS;
    const int h = bh % a.H;
    const int T = a.T, DV = a.dv;
    const long long qk_base = static_cast<long long>(bh) * T * DK;
    const long long v_base = static_cast<long long>(bh) * T * DV;
    const E* __restrict__ qg = static_cast<const E*>(a.q) + qk_base;
    const E* __restrict__ kg = static_cast<const E*>(a.k) + qk_base;
    const E* __restrict__ vg = static_cast<const E*>(a.v) + v_base;
    E* __restrict__ og = static_cast<E*>(a.out) + v_base;

    // per-head decay table: dec[16 + m] = gamma^m (m >= 0), dec[0..15] = 0
    const float lg = LIN ? 0.f : a.log2g[h];
    for (int m = tid; m < DEC; m += kThreads)
        dec[m] = (m < 16) ? 0.f : exp2f(static_cast<float>(m - 16) * lg);
    for (int m = tid; m < DVS * KSTR; m += kThreads) Sts[0][m] = E(0);
    if (LIN)
        for (int m = tid; m < DK; m += kThreads) zs[0][m] = 0.f;

    int its[NS];
    its[0] = (NS == 2) ? w : w;
    if (NS == 2) its[NS - 1] = NI - 1 - w;
    const int itmax = its[NS - 1];

    f32x4 sacc[SPW];
#pragma unroll
    for (int m = 0; m < SPW; ++m) sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---------------- prefetch registers
    uint4 kpre[KU];
    uint4 vpre[4];
    uint4 qnext[NS][QU];
    uint4 qcur[NS][QU];

    auto load_chunk = [&](int c) {
        const int t0 = c * C;
#pragma unroll
        for (int m = 0; m < KU; ++m) {
            const int u = tid + m * kThreads;
            const int row = u / RU, col = u % RU;
            const int t = t0 + row;
            kpre[m] = (t < T) ? *reinterpret_cast<const uint4*>(kg + static_cast<long long>(t) * DK + col * (16 / sizeof(E)))
                              : uint4{0, 0, 0, 0};
        }
        if (tid < VU) {
            const int jq = tid / (DVS / VCOLS), cg = tid % (DVS / VCOLS);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + 4 * jq + r;
                vpre[r] = (t < T) ? *reinterpret_cast<const uint4*>(vg + static_cast<long long>(t) * DV + nbase + cg * VCOLS)
                                  : uint4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int t = t0 + its[s] * 16 + l16;
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                // bf16: unit u covers k = 32u + 8g .. +7 ; fp32: k = (DK/4) g + 4u .. +3
                const int k0 = BF16 ? (32 * u + 8 * g) : ((DK / 4) * g + 4 * u);
                qnext[s][u] = (t < T) ? *reinterpret_cast<const uint4*>(qg + static_cast<long long>(t) * DK + k0)
                                      : uint4{0, 0, 0, 0};
            }
        }
    };

    auto apply_phi16 = [&](uint4 x) -> uint4 {
        if constexpr (BF16) {
            u16x8 e = __builtin_bit_cast(u16x8, x);
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = f2bf(phi_elu1(bf2f(e[i])));
            return __builtin_bit_cast(uint4, e);
        } else {
            f32x4 e = __builtin_bit_cast(f32x4, x);
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = phi_elu1(e[i]);
            return __builtin_bit_cast(uint4, e);
        }
    };

    const int nch = (T + C - 1) / C;
    if (nch > 0) load_chunk(0);

    for (int c = 0; c < nch; ++c) {
        const int t0 = c * C;
        const int clen = (T - t0 < C) ? (T - t0) : C;
        const int cur = c & 1, nxt = cur ^ 1;

        __syncthreads();  // previous chunk's LDS reads are done
        // ---- stage K rows
#pragma unroll
        for (int m = 0; m < KU; ++m) {
            const int u = tid + m * kThreads;
            const int row = u / RU, col = u % RU;
            uint4 x = kpre[m];
            if (LIN) x = apply_phi16(x);
            *reinterpret_cast<uint4*>(&Ks[row * KSTR + col * (16 / sizeof(E))]) = x;
        }
        // ---- stage the V slice, packed 4 tokens deep, plain and zeta-scaled
        if (tid < VU) {
            const int jq = tid / (DVS / VCOLS), cg = tid % (DVS / VCOLS);
            float zeta[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = 16 + clen - 1 - (4 * jq + r);  // gamma^(c-1-j), 0 past the end
                zeta[r] = dec[e < 0 ? 0 : e];
            }
            E* dst = &V4s[(jq * DVS + cg * VCOLS) * 4];
            E* dstz = &V4z[(jq * DVS + cg * VCOLS) * 4];
            if constexpr (BF16) {
                u16x8 rows[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) rows[r] = __builtin_bit_cast(u16x8, vpre[r]);
#pragma unroll
                for (int p = 0; p < 2; ++p) {  // 4 columns (= 32 bytes) per half
                    u16x8 o0, o1, z0, z1;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        o0[r] = rows[r][4 * p + 0];
                        o0[4 + r] = rows[r][4 * p + 1];
                        o1[r] = rows[r][4 * p + 2];
                        o1[4 + r] = rows[r][4 * p + 3];
                        z0[r] = f2bf(bf2f(rows[r][4 * p + 0]) * zeta[r]);
                        z0[4 + r] = f2bf(bf2f(rows[r][4 * p + 1]) * zeta[r]);
                        z1[r] = f2bf(bf2f(rows[r][4 * p + 2]) * zeta[r]);
                        z1[4 + r] = f2bf(bf2f(rows[r][4 * p + 3]) * zeta[r]);
                    }
                    *reinterpret_cast<u16x8*>(dst + 16 * p) = o0;
                    *reinterpret_cast<u16x8*>(dst + 16 * p + 8) = o1;
                    *reinterpret_cast<u16x8*>(dstz + 16 * p) = z0;
                    *reinterpret_cast<u16x8*>(dstz + 16 * p + 8) = z1;
                }
            } else {
                f32x4 rows[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) rows[r] = __builtin_bit_cast(f32x4, vpre[r]);
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    f32x4 o, z;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        o[r] = rows[r][cc];
                        z[r] = rows[r][cc] * zeta[r];
                    }
                    *reinterpret_cast<f32x4*>(dst + 4 * cc) = o;
                    *reinterpret_cast<f32x4*>(dstz + 4 * cc) = z;
                }
            }
        }
        // ---- this chunk's Q (feature-mapped for linear attention)
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int u = 0; u < QU; ++u) qcur[s][u] = LIN ? apply_phi16(qnext[s][u]) : qnext[s][u];
        __syncthreads();

        if (c + 1 < nch) load_chunk(c + 1);

        // ---------------- S^T tiles = K Q^T for key tiles jt <= query tile
        f32x4 pacc[NS][NI];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int jt = 0; jt < NI; ++jt) pacc[s][jt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int jt = 0; jt < NI; ++jt) {
            if (jt <= itmax) {
                const E* krow = &Ks[(jt * 16 + l16) * KSTR];
                if constexpr (BF16) {
#pragma unroll
                    for (int ks = 0; ks < DK / 32; ++ks) {
                        const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 32 * ks + 8 * g));
#pragma unroll
                        for (int s = 0; s < NS; ++s)
                            if (jt <= its[s]) pacc[s][jt] = mfma_bf16(av, as_bf16x8(qcur[s][ks]), pacc[s][jt]);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < QU; ++u) {
                        const f32x4 a4 = *reinterpret_cast<const f32x4*>(krow + (DK / 4) * g + 4 * u);
#pragma unroll
                        for (int s = 0; s < NS; ++s) {
                            if (jt <= its[s]) {
                                const f32x4 q4 = __builtin_bit_cast(f32x4, qcur[s][u]);
#pragma unroll
                                for (int e = 0; e < 4; ++e) pacc[s][jt] = mfma_f32(a4[e], q4[e], pacc[s][jt]);
                            }
                        }
                    }
                }
            }
        }

        // ---------------- decay mask: P^T[j][i] = S^T[j][i] * gamma^(i-j), 0 for j > i
        float rsum[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            rsum[s] = 0.f;
#pragma unroll
            for (int jt = 0; jt < NI; ++jt) {
                if (jt <= its[s]) {
                    const int base = 16 * (its[s] - jt) + l16 - 4 * g + 16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) pacc[s][jt][r] *= dec[base - r];
                }
            }
        }

        // bf16 copies of P^T, two key tiles per MFMA operand
        bf16x8 pb[NS][NI / 2];
        if constexpr (BF16) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
#pragma unroll
                for (int p = 0; p < NI / 2; ++p) {
                    if (2 * p <= its[s]) {
                        const u16x4 lo = cvt4_bf16(pacc[s][2 * p]);
                        const u16x4 hi = (2 * p + 1 <= its[s]) ? cvt4_bf16(pacc[s][2 * p + 1]) : u16x4{0, 0, 0, 0};
                        pb[s][p] = cat_bf16(lo, hi);
                        if (LIN) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) rsum[s] += bf2f(lo[r]) + bf2f(hi[r]);
                        }
                    }
                }
            }
        } else if (LIN) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int jt = 0; jt < NI; ++jt)
                    if (jt <= its[s])
#pragma unroll
                        for (int r = 0; r < 4; ++r) rsum[s] += pacc[s][jt][r];
        }

        // ---------------- O^T = S_prev^T (xi Q)^T + V^T P^T
        f32x4 oacc[NS][NT];
        const E* st = Sts[cur];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int s = 0; s < NS; ++s) oacc[s][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const E* srow = st + (nt * 16 + l16) * KSTR;
            if constexpr (BF16) {
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(srow + 32 * ks + 8 * g));
#pragma unroll
                    for (int s = 0; s < NS; ++s) oacc[s][nt] = mfma_bf16(av, as_bf16x8(qcur[s][ks]), oacc[s][nt]);
                }
            } else {
#pragma unroll
                for (int u = 0; u < QU; ++u) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(srow + (DK / 4) * g + 4 * u);
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        const f32x4 q4 = __builtin_bit_cast(f32x4, qcur[s][u]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) oacc[s][nt] = mfma_f32(a4[e], q4[e], oacc[s][nt]);
                    }
                }
            }
            if (!LIN) {
#pragma unroll
                for (int s = 0; s < NS; ++s) oacc[s][nt] *= dec[16 + its[s] * 16 + l16 + 1];  // gamma^(i+1)
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if constexpr (BF16) {
#pragma unroll
                for (int p = 0; p < NI / 2; ++p) {
                    if (2 * p <= itmax) {
                        const E* v0 = &V4s[((8 * p + g) * DVS + nt * 16 + l16) * 4];
                        const E* v1 = &V4s[((8 * p + 4 + g) * DVS + nt * 16 + l16) * 4];
                        const bf16x8 av = cat_bf16(*reinterpret_cast<const u16x4*>(v0),
                                                   *reinterpret_cast<const u16x4*>(v1));
#pragma unroll
                        for (int s = 0; s < NS; ++s)
                            if (2 * p <= its[s]) oacc[s][nt] = mfma_bf16(av, pb[s][p], oacc[s][nt]);
                    }
                }
            } else {
#pragma unroll
                for (int jt = 0; jt < NI; ++jt) {
                    if (jt <= itmax) {
                        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&V4s[((4 * jt + g) * DVS + nt * 16 + l16) * 4]);
#pragma unroll
                        for (int s = 0; s < NS; ++s)
                            if (jt <= its[s])
#pragma unroll
                                for (int r = 0; r < 4; ++r) oacc[s][nt] = mfma_f32(a4[r], pacc[s][jt][r], oacc[s][nt]);
                    }
                }
            }
        }

        // ---------------- normalise (linear attention) and store O
        float rden[NS];
        if (LIN) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                // phi(q_i) . z over this lane's key slots
                float dq = 0.f;
                const float* zc = zs[cur];
#pragma unroll
                for (int u = 0; u < QU; ++u) {
                    if constexpr (BF16) {
                        const u16x8 e = __builtin_bit_cast(u16x8, qcur[s][u]);
#pragma unroll
                        for (int i = 0; i < 8; ++i) dq += bf2f(e[i]) * zc[32 * u + 8 * g + i];
                    } else {
                        const f32x4 e = __builtin_bit_cast(f32x4, qcur[s][u]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) dq += e[i] * zc[(DK / 4) * g + 4 * u + i];
                    }
                }
                const float den = sum_over_groups(rsum[s] + dq) + a.eps;
                rden[s] = 1.f / den;
            }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int row = its[s] * 16 + l16;
            if (row < clen) {
                E* orow = og + static_cast<long long>(t0 + row) * DV + nbase + 4 * g;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4 o = oacc[s][nt];
                    if (LIN) o *= rden[s];
                    if constexpr (BF16) {
                        *reinterpret_cast<u16x4*>(orow + nt * 16) = cvt4_bf16(o);
                    } else {
                        *reinterpret_cast<f32x4*>(orow + nt * 16) = o;
                    }
                }
            }
        }

        // ---------------- state: S^T <- gamma^c S^T + (zeta V)^T K   (and z += sum phi(k))
        const float gc = dec[16 + clen];
        E* stn = Sts[nxt];
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = w + 4 * m;
            const int nt = qt / KT, kt = qt % KT;
            f32x4 acc = sacc[m] * gc;
            float zsum = 0.f;
            const int kcol = kt * 16 + l16;
            if constexpr (BF16) {
#pragma unroll
                for (int js = 0; js < C / 32; ++js) {
                    const E* v0 = &V4z[((8 * js + g) * DVS + nt * 16 + l16) * 4];
                    const E* v1 = &V4z[((8 * js + 4 + g) * DVS + nt * 16 + l16) * 4];
                    const bf16x8 av = cat_bf16(*reinterpret_cast<const u16x4*>(v0),
                                               *reinterpret_cast<const u16x4*>(v1));
                    u16x4 blo, bhi;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        blo[r] = Ks[(js * 32 + 4 * g + r) * KSTR + kcol];
                        bhi[r] = Ks[(js * 32 + 16 + 4 * g + r) * KSTR + kcol];
                    }
                    acc = mfma_bf16(av, cat_bf16(blo, bhi), acc);
                    if (LIN && nt == 0) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) zsum += bf2f(blo[r]) + bf2f(bhi[r]);
                    }
                }
            } else {
#pragma unroll
                for (int jt = 0; jt < NI; ++jt) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(&V4z[((4 * jt + g) * DVS + nt * 16 + l16) * 4]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float b = Ks[(jt * 16 + 4 * g + r) * KSTR + kcol];
                        acc = mfma_f32(a4[r], b, acc);
                        if (LIN && nt == 0) zsum += b;
                    }
                }
            }
            sacc[m] = acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (BF16) stn[(nt * 16 + 4 * g + r) * KSTR + kcol] = f2bf(acc[r]);
                else stn[(nt * 16 + 4 * g + r) * KSTR + kcol] = acc[r];
            }
            if (LIN && nt == 0) {
                zsum = sum_over_groups(zsum);
                if (g == 0) zs[nxt][kcol] = zs[cur][kcol] + zsum;
            }
        }
    }

    // ---------------- final state [dk][dv] fp32
    if (a.final_state) {
        float* fs = a.final_state + static_cast<long long>(bh) * DK * DV;
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = w + 4 * m;
            const int nt = qt / KT, kt = qt % KT;
            *reinterpret_cast<f32x4*>(fs + static_cast<long long>(kt * 16 + l16) * DV + nbase + nt * 16 + 4 * g) = sacc[m];
        }
    }
}

template <bool BF16, int C, int DK, int NT, bool LIN>
hipError_t launch_t(const WalkArgs& a, hipStream_t stream) {
    const long long groups = static_cast<long long>(a.B) * a.H * a.nslices;
    if (groups <= 0) return hipSuccess;
    if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
    WalkArgs args = a;
    args.xcd_remap = (groups % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((walk_kernel<BF16, C, DK, NT, LIN>), dim3(static_cast<unsigned>(groups)),
                       dim3(kThreads), 0, stream, args);
    return hipGetLastError();
}

template <bool BF16, int C, bool LIN>
hipError_t launch_dk(const WalkArgs& a, int dk, int nt, hipStream_t stream) {
    if (dk == 64) {
        if (nt == 1) return launch_t<BF16, C, 64, 1, LIN>(a, stream);
        if (nt == 2) return launch_t<BF16, C, 64, 2, LIN>(a, stream);
    } else if (dk == 128) {
        if (nt == 1) return launch_t<BF16, C, 128, 1, LIN>(a, stream);
        if (nt == 2) return launch_t<BF16, C, 128, 2, LIN>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <bool BF16, bool LIN>
hipError_t launch_c(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream) {
    if (chunk == 64) return launch_dk<BF16, 64, LIN>(a, dk, nt, stream);
    if (chunk == 128) return launch_dk<BF16, 128, LIN>(a, dk, nt, stream);
    return hipErrorInvalidValue;
}

}  // namespace

int choose_walk_nt(long long bh, int dv, int target_groups) {
    int best = 1;
    for (int nt = 2; nt <= 2; nt *= 2) {
        if (dv % (16 * nt) != 0) break;
        if (bh * (dv / (16 * nt)) >= target_groups) best = nt;
    }
    return best;
}

hipError_t launch_walk(const WalkArgs& a, bool bf16, int chunk, int dk, int nt, bool linattn,
                       hipStream_t stream) {
    if (bf16) {
        return linattn ? launch_c<true, true>(a, chunk, dk, nt, stream)
                       : launch_c<true, false>(a, chunk, dk, nt, stream);
    }
    return linattn ? launch_c<false, true>(a, chunk, dk, nt, stream)
                   : launch_c<false, false>(a, chunk, dk, nt, stream);
}

}  // namespace ret
