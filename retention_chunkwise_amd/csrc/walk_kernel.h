// walk_kernel.h -- chunkwise causal retention / elu+1 linear attention on gfx950.
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
// (batch, head) pair, one segment of G consecutive runs of whole chunks and
// one slice of 16*NT value columns, and walks the chunks of its segment in
// order, keeping its slice of S in registers (fp32).  Value columns of S and
// O are independent, so slices need no communication; each slice recomputes
// Q K^T for its chunk.  Slices of one (b, h, segment) are placed on the same
// XCD so their shared Q / K reads hit that XCD's L2.  The recurrence is
// linear, so the state entering segment g is
//   S_in(g) = gamma^(g L) S_0 + sum_{j<g} gamma^(L (g-1-j)) dS_j,
// with L the segment length and dS_j = sum_{t in segment j}
// gamma^(end_j - 1 - t) k_t v_t^T computed beforehand by slice_state_kernel.
//
// Per chunk, wave W owns query tiles {W, C/16-1-W} (16 rows each; one tile
// when C = 64), which balances the causal triangle across waves.  The wave
// index is a template parameter, so every tile loop is unrolled at compile
// time with no divergent branches.  All contractions run on MFMA (bf16:
// v_mfma_f32_16x16x32_bf16, fp32: v_mfma_f32_16x16x4f32), fp32 accumulate:
//   S^T_tile = K Q^T      A = K rows (LDS), B = Q rows (registers)
//   P^T      = S^T (.) D  decay factors precomputed per lane, in registers
//   O^T     += S_prev^T (xi Q)^T   A = state copy (LDS), B = Q (registers)
//   O^T     += V^T P^T    A = V slice packed 4 tokens deep (LDS), B = P^T
//   S^T      = gamma^c S^T + (zeta V)^T K
// Computing the transposed products lets the output of the Q K^T MFMA feed the
// P V MFMA directly from registers (each lane holds 4 consecutive keys of one
// query), so P never goes through LDS.  The next chunk's K, V and Q are loaded
// from HBM into registers while the current chunk computes.
#pragma once

#include <type_traits>

#include "internal.h"
#include "kcommon.h"

namespace ret {
namespace walk {

constexpr int kThreads = 256;
using namespace ::ret::kc;

template <bool BF16, int C, int DK, int NT, int MODE>
struct Cfg {
    typedef typename std::conditional<BF16, unsigned short, float>::type E;
    static constexpr int NI = C / 16;                 // 16-token tiles per chunk
    static constexpr int NS = (NI == 8) ? 2 : 1;      // query tiles per wave
    static constexpr int DVS = 16 * NT;               // value columns per workgroup
    static constexpr int ESZ = BF16 ? 2 : 4;          // element bytes
    static constexpr int EPV = 16 / ESZ;              // elements per 16-byte vector
    static constexpr int KSTR = DK + EPV;             // padded row stride (fp32 K, state copy)
    static constexpr int VSTR = DVS;                  // row stride of the V slice copies
    static constexpr int KT = DK / 16;                // 16-wide key tiles
    static constexpr int NTILE = NT * KT;             // 16x16 state tiles of a slice
    static constexpr int KU = C * DK * ESZ / 16 / kThreads;  // 16-B units of a Q / K chunk per thread
    static constexpr int RU = DK * ESZ / 16;          // 16-B units (slots) per Q / K row
    static constexpr int RB = DK * ESZ;               // bytes per Q / K row
    static constexpr int VRU = DVS * ESZ / 16;        // 16-B units per V-slice row
    static constexpr int VUT = C * VRU;               // V-slice units per chunk
    static constexpr int VPT = (VUT + kThreads - 1) / kThreads;
    // bf16: Q and K go HBM -> LDS by DMA into double-buffered, unpadded,
    // slot-swizzled tiles; fp32: K staged through registers into padded rows,
    // Q kept in registers by the wave that uses it.
    static constexpr bool DMA = BF16;
    static constexpr int QU = DK * ESZ / 64;          // 16-B Q units per lane per tile
    static constexpr int KI = C * DK * ESZ / 1024;    // 1-KB DMA instructions per Q / K chunk
    static constexpr int VI = C * DVS * ESZ / 1024;   // 1-KB DMA instructions per V slice chunk
    static constexpr int DEC = C + 32;                // decay table entries
    static_assert(NI == 4 || NI == 8, "chunk must be 64 or 128");
    static_assert(DK == 64 || DK == 128, "dk must be 64 or 128");
    static_assert(NT * KT % 4 == 0, "state tiles must split over 4 waves");
    static_assert(C * DK * ESZ / 16 % kThreads == 0, "Q/K staging split");
    static_assert(!DMA || RU == 8 || RU == 16, "swizzle assumes 8 or 16 slots per row");
};

// Split of the NT * KT state tiles over the 4 waves.  Wave W's query tiles
// cost it (tiles of Q K^T) + (tiles of P V) + (inter-chunk tiles); with
// 64-token chunks wave W owns query tile W alone, so that work grows with W,
// and the state tiles (C contraction steps each) go greedily to the least
// loaded wave until the loads even out (7/5/3/1 tiles for dk = dv = 64).
// Each wave's tiles are a contiguous run in (value tile, key tile) order.
template <int C, int DK, int NT>
struct StateSplit {
    static constexpr int NI = C / 16, KT = DK / 16;
    static constexpr int qtiles(int w) { return (NI == 8) ? (w + 1) + (NI - w) : (w + 1); }  // key tiles seen
    static constexpr int load(int w) {
        return qtiles(w) * DK + NT * qtiles(w) * 16 + ((NI == 8) ? 2 : 1) * NT * DK;
    }
    static constexpr int count(int w) {
        int ld[4] = {load(0), load(1), load(2), load(3)};
        int cnt[4] = {0, 0, 0, 0};
        for (int t = 0; t < NT * KT; ++t) {
            int b = 0;
            for (int i = 1; i < 4; ++i)
                if (ld[i] < ld[b]) b = i;
            ld[b] += C;
            ++cnt[b];
        }
        return cnt[w];
    }
    static constexpr int start(int w) {
        int s = 0;
        for (int i = 0; i < w; ++i) s += count(i);
        return s;
    }
};

// Byte offset of 16-byte slot `col16` of row `r` in a swizzled Q / K tile.
// Rows are unpadded; slots are XOR-permuted so that 16 consecutive rows read
// at one column hit 16 different bank groups.
template <int RU>
__device__ __forceinline__ int swz_off(int r, int col16) {
    const int x = (RU == 16) ? (r & 15) : ((r >> 1) & 7);
    return r * (RU * 16) + ((col16 ^ x) << 4);
}

template <bool BF16, int C, int DK, int NT, int MODE>
struct Smem {
    using Cf = Cfg<BF16, C, DK, NT, MODE>;
    using E = typename Cf::E;
    static constexpr bool DMA = Cf::DMA;
    alignas(16) float dec[Cf::DEC];                   // [16 + m] = gamma^m, [0..15] = 0
    alignas(16) float zs[2][MODE != 0 ? DK : 4];      // normaliser z (linear attention, row-sum floor)
    alignas(16) E Sts[2][Cf::DVS * Cf::KSTR];         // S^T copy, [n][k], double-buffered
    alignas(16) E Vs[Cf::DMA ? 8 : C * Cf::VSTR];     // V slice, row-major (fp32 path)
    alignas(16) E Vz[C * Cf::VSTR];                   // zeta-scaled V slice
    alignas(16) E Ks[DMA ? 8 : C * Cf::KSTR];         // K rows, padded (fp32)
};

// The double-buffered Q / K chunk tiles of the DMA path.  Each buffer is its
// own __shared__ array, so the compiler can tell that a DMA into one buffer
// does not touch the other and need not wait for it before reading.
template <typename E>
struct QKTiles {
    E* q[2];
    E* k[2];
    E* v[2];  // the V slice, row-major
};

template <bool BF16, int C, int DK, int NT, int MODE, int W>
__device__ __forceinline__ void walk_body(const WalkArgs& a, Smem<BF16, C, DK, NT, MODE>& sm,
                                          const QKTiles<typename Cfg<BF16, C, DK, NT, MODE>::E>& qk,
                                          const int bh, const int nbase, const int seg, const float lg) {
    using Cf = Cfg<BF16, C, DK, NT, MODE>;
    using E = typename Cf::E;
    // MODE: 0 retention, 1 elu+1 linear attention, 2 retention with the row-sum
    // floor, 3 the floor plus GroupNorm (the numbering of the segment kernels)
    constexpr bool LIN = MODE == 1, ZN = MODE != 0, NRM = MODE >= 2, GRP = MODE == 3;
    static_assert(!(BF16 && NRM), "the normalised value-slice walks are fp32 only");
    constexpr int NI = Cf::NI, NS = Cf::NS, KSTR = Cf::KSTR, EPV = Cf::EPV;
    constexpr int VSTR = Cf::VSTR, KT = Cf::KT, KU = Cf::KU, RU = Cf::RU;
    constexpr int SPW = StateSplit<C, DK, NT>::count(W);  // state tiles of this wave
    constexpr int TS = StateSplit<C, DK, NT>::start(W);   // its first tile
    static_assert(StateSplit<C, DK, NT>::start(3) + StateSplit<C, DK, NT>::count(3) == Cf::NTILE,
                  "every state tile has one owner");
    constexpr int VRU = Cf::VRU, VUT = Cf::VUT, VPT = Cf::VPT, QU = Cf::QU, ESZ = Cf::ESZ;
    constexpr bool DMA = Cf::DMA;
    constexpr int IT0 = W;                                // query tiles of this wave
    constexpr int IT1 = (NS == 2) ? NI - 1 - W : W;
    constexpr int ITMAX = IT1;                            // IT1 >= IT0
    // vector-memory ops a thread issues after a chunk's Q/K (and V) loads:
    // the V loads and the output stores of the chunk being computed
    constexpr int STORES = NS * NT;

    const int tid = threadIdx.x;
    const int l = tid & 63, l16 = l & 15, g = l >> 4;
    const int lq = l16 >> 2, lr = l16 & 3;                // transpose-read lane roles
    const int T = a.T, DV = a.dv;
    const E* __restrict__ qh = static_cast<const E*>(a.q) + static_cast<long long>(bh) * T * DK;
    const E* __restrict__ kh = static_cast<const E*>(a.k) + static_cast<long long>(bh) * T * DK;
    const E* __restrict__ vh = static_cast<const E*>(a.v) + static_cast<long long>(bh) * T * DV + nbase;
    E* __restrict__ oh = static_cast<E*>(a.out) + static_cast<long long>(bh) * T * DV + nbase;

    auto its = [](int s) constexpr { return s == 0 ? IT0 : IT1; };

    // decay factors of this lane for the tiles this wave owns:
    // dfac[dt][r] = gamma^(16 dt + l16 - 4g - r) for a non-negative exponent, else 0
    float dfac[ITMAX + 1][4];
#pragma unroll
    for (int dt = 0; dt <= ITMAX; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = 16 * dt + l16 - 4 * g - r;
            dfac[dt][r] = (e < 0) ? 0.f : exp2f(static_cast<float>(e) * lg);
        }
    float xi[NS];  // gamma^(i+1) for this lane's query row in each owned tile
#pragma unroll
    for (int s = 0; s < NS; ++s) xi[s] = exp2f(static_cast<float>(its(s) * 16 + l16 + 1) * lg);

    // ---- state entering the segment: S[16 kt + l16][nbase + 16 nt + 4g + r] of this wave's tiles
    f32x4 sacc[SPW > 0 ? SPW : 1];
#pragma unroll
    for (int m = 0; m < SPW; ++m) sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float lseg = static_cast<float>(a.seg_len) * lg;  // log2 of gamma^L
    if constexpr (!BF16) {
        // fp32: every thread of the workgroup forms EPT consecutive columns of one
        // row of S_in = sum_{j<seg} gamma^(L (seg-1-j)) dS_j (+ the decayed initial
        // state), up to SB segments' values in flight, straight into the first
        // chunk's operand copy Sts[0][j][i] = S[i][nbase + j]; each wave then takes
        // its tiles from there
        constexpr int DVS = Cf::DVS;
        constexpr int TPR = kThreads / DK;          // threads per state row
        constexpr int EPT = DVS / TPR;              // columns per thread (>= 4)
        constexpr int V4 = EPT / 4;
        constexpr int SB = (32 / EPT) > 0 ? 32 / EPT : 1;  // segments' values in flight
        static_assert(EPT % 4 == 0, "16-byte column groups");
        const int row = tid / TPR, col0 = (tid % TPR) * EPT;
        f32x4 acc[V4];
#pragma unroll
        for (int v4 = 0; v4 < V4; ++v4) acc[v4] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (seg > 0) {
            constexpr int ZW = ZN ? DK : 0;  // normaliser floats after each state slot
            const long long slot = static_cast<long long>(DK) * DV + ZW;
            const float* wsb = a.ws + static_cast<long long>(bh) * (a.G - 1) * slot;
            const bool tr = !ZN && a.ws_tr;
            for (int j0 = 0; j0 < seg; j0 += SB) {
                f32x4 x[SB][V4];
#pragma unroll
                for (int b = 0; b < SB; ++b) {
                    const int j = j0 + b;
                    const float* sj = wsb + static_cast<long long>(j < seg ? j : 0) * slot;
#pragma unroll
                    for (int v4 = 0; v4 < V4; ++v4) {
                        if (j >= seg) {
                            x[b][v4] = f32x4{0.f, 0.f, 0.f, 0.f};
                        } else if (tr) {
                            // S[i][nbase + c] is element (nbase + c) * DK + i of the transposed (DV x DK) state
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                x[b][v4][e] = sj[static_cast<long long>(nbase + col0 + 4 * v4 + e) * DK + row];
                        } else {
                            x[b][v4] = *reinterpret_cast<const f32x4*>(sj + static_cast<long long>(row) * DV + nbase +
                                                                        col0 + 4 * v4);
                        }
                    }
                }
#pragma unroll
                for (int b = 0; b < SB; ++b) {
                    const int j = j0 + b;
                    const float wj = (j < seg) ? exp2f(lseg * static_cast<float>(seg - 1 - j)) : 0.f;
#pragma unroll
                    for (int v4 = 0; v4 < V4; ++v4) acc[v4] += wj * x[b][v4];
                }
            }
        }
        if (a.init_state) {
            const float w0 = exp2f(lseg * static_cast<float>(seg));
            const float* si = a.init_state + static_cast<long long>(bh) * DK * DV + static_cast<long long>(row) * DV +
                              nbase + col0;
#pragma unroll
            for (int v4 = 0; v4 < V4; ++v4) acc[v4] += w0 * *reinterpret_cast<const f32x4*>(si + 4 * v4);
        }
        E* st0 = sm.Sts[0];
#pragma unroll
        for (int e = 0; e < EPT; ++e) st0[(col0 + e) * KSTR + row] = acc[e / 4][e % 4];
        __syncthreads();
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = TS + m;
            const int nt = qt / KT, kt = qt % KT;
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[m][r] = st0[(nt * 16 + 4 * g + r) * KSTR + kt * 16 + l16];
        }
    } else {
        if (seg > 0) {
            constexpr int ZW = ZN ? DK : 0;  // normaliser floats after each state slot
            const long long slot = static_cast<long long>(DK) * DV + ZW;
            const float* wsb = a.ws + static_cast<long long>(bh) * (a.G - 1) * slot + nbase;
            for (int j = 0; j < seg; ++j) {
                const float wj = exp2f(lseg * static_cast<float>(seg - 1 - j));
                if (!ZN && a.ws_tr) {
                    // S[i][nbase + c] is element (nbase + c) * DK + i of the transposed (DV x DK) state
                    const float* sj = a.ws + (static_cast<long long>(bh) * (a.G - 1) + j) * slot;
#pragma unroll
                    for (int m = 0; m < SPW; ++m) {
                        const int qt = TS + m;
                        const int nt = qt / KT, kt = qt % KT;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            sacc[m][r] += wj * sj[static_cast<long long>(nbase + nt * 16 + 4 * g + r) * DK + kt * 16 + l16];
                    }
                    continue;
                }
#pragma unroll
                for (int m = 0; m < SPW; ++m) {
                    const int qt = TS + m;
                    const int nt = qt / KT, kt = qt % KT;
                    sacc[m] += wj * *reinterpret_cast<const f32x4*>(wsb + j * slot + (kt * 16 + l16) * DV + nt * 16 + 4 * g);
                }
            }
        }
        if (a.init_state) {
            const float w0 = exp2f(lseg * static_cast<float>(seg));
            const float* si = a.init_state + static_cast<long long>(bh) * DK * DV + nbase;
#pragma unroll
            for (int m = 0; m < SPW; ++m) {
                const int qt = TS + m;
                const int nt = qt / KT, kt = qt % KT;
                sacc[m] += w0 * *reinterpret_cast<const f32x4*>(si + (kt * 16 + l16) * DV + nt * 16 + 4 * g);
            }
        }
        {
            // operand copy for the first chunk: Sts[0][j][i] = S[i][nbase + j] (the
            // first barrier of the first step orders these writes before any read)
            E* st0 = sm.Sts[0];
#pragma unroll
            for (int m = 0; m < SPW; ++m) {
                const int qt = TS + m;
                const int nt = qt / KT, kt = qt % KT;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (BF16) st0[(nt * 16 + 4 * g + r) * KSTR + kt * 16 + l16] = f2bf(sacc[m][r]);
                    else st0[(nt * 16 + 4 * g + r) * KSTR + kt * 16 + l16] = sacc[m][r];
                }
            }
        }
    }

    // DMA path: 1-KB instruction i of a chunk is issued by wave i % 4 and fills
    // LDS bytes [1024 i, +1024) of its tile; lane l's 16 bytes land at +16 l.
    // The per-lane source offsets inside a chunk are loop invariant.
    constexpr int KIW = DMA ? Cf::KI / 4 : 1;                        // Q/K instructions per wave
    constexpr int VIW = DMA ? (Cf::VI > W ? (Cf::VI - W + 3) / 4 : 0) : 0;  // V instructions per wave
    int goff[KIW];
    int gvoff[VIW > 0 ? VIW : 1];
    if constexpr (DMA) {
#pragma unroll
        for (int m = 0; m < KIW; ++m) {
            const int b = (W + 4 * m) * 1024 + l * 16;
            const int r = b / (RU * 16), slot = (b % (RU * 16)) >> 4;
            const int x = (RU == 16) ? (r & 15) : ((r >> 1) & 7);
            goff[m] = r * (RU * 16) + ((slot ^ x) << 4);
        }
#pragma unroll
        for (int m = 0; m < VIW; ++m) {
            const int b = (W + 4 * m) * 1024 + l * 16;
            const int r = b / (VRU * 16), unit = (b % (VRU * 16)) >> 4;
            gvoff[m] = r * DV * ESZ + unit * 16;
        }
    }

    uint4 kpre[DMA ? 1 : KU];
    uint4 vpre[DMA ? 1 : VPT];
    uint4 qnext[NS][DMA ? 1 : QU];
    uint4 qcur[NS][DMA ? 1 : QU];

    // Time-reversed walks (fp32 only) read and write chunk row r of a chunk of
    // cl rows starting at token t0 at memory row T - 1 - (t0 + r): the chunk's
    // memory rows start at T - t0 - cl and run backwards.
    const bool rev = !DMA && a.reverse;
    auto mem_row0 = [&](int t0, int cl) -> long long { return rev ? T - t0 - cl : t0; };
    auto row_in = [&](int r, int cl) -> int { return rev ? cl - 1 - r : r; };

    // Issue the loads of chunk c (into LDS buffer `buf` on the DMA path) through
    // range-checked buffer resources: rows past the end of the sequence read as
    // zeros.  No instruction consumes these values in the step that issues them.
    auto load_chunk = [&](int c, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const int t0 = c * C;
        const int cl = (T - t0 < C) ? (T - t0) : C;
        const long long mrow = mem_row0(t0, cl);
        const auto rk = make_rsrc(kh + mrow * DK, cl * DK * ESZ);
        const auto rq = make_rsrc(qh + mrow * DK, cl * DK * ESZ);
        const auto rv = make_rsrc(vh + mrow * DV, cl * DV * ESZ);
        if constexpr (DMA) {
            const u32x4 wk = rsrc_words(kh + static_cast<long long>(t0) * DK, cl * DK * ESZ);
            const u32x4 wq = rsrc_words(qh + static_cast<long long>(t0) * DK, cl * DK * ESZ);
            const u32x4 wv = rsrc_words(vh + static_cast<long long>(t0) * DV, cl * DV * ESZ);
            const unsigned kbase = __builtin_amdgcn_readfirstlane(lds_addr_of(qk.k[buf]));
            const unsigned qbase = __builtin_amdgcn_readfirstlane(lds_addr_of(qk.q[buf]));
            const unsigned vbase = __builtin_amdgcn_readfirstlane(lds_addr_of(qk.v[buf]));
#pragma unroll
            for (int m = 0; m < KIW; ++m) {
                const unsigned o = (W + 4 * m) * 1024;  // LDS bytes this instruction fills
                dma16(wk, kbase + o, static_cast<unsigned>(goff[m]));
                dma16(wq, qbase + o, static_cast<unsigned>(goff[m]));
            }
#pragma unroll
            for (int m = 0; m < VIW; ++m)
                dma16(wv, vbase + (W + 4 * m) * 1024, static_cast<unsigned>(gvoff[m]));
        } else {
#pragma unroll
            for (int m = 0; m < KU; ++m) {
                const int u = tid + m * kThreads;
                const int row = row_in(u / RU, cl), col = u % RU;
                kpre[m] = bload16(rk, static_cast<unsigned>((row * DK + col * EPV) * ESZ));
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int row = row_in(its(s) * 16 + l16, cl);
#pragma unroll
                for (int u = 0; u < QU; ++u)  // k = (DK/4) g + 4u .. +3
                    qnext[s][u] = bload16(rq, static_cast<unsigned>((row * DK + (DK / 4) * g + 4 * u) * ESZ));
            }
        }
        if constexpr (!DMA) {
#pragma unroll
            for (int m = 0; m < VPT; ++m) {
                const int u = tid + m * kThreads;
                if (VUT % kThreads == 0 || u < VUT) {
                    const int row = row_in(u / VRU, cl), col = u % VRU;
                    vpre[m] = bload16(rv, static_cast<unsigned>((row * DV + col * EPV) * ESZ));
                }
            }
        }
    };

    auto apply_phi16 = [](uint4 x) -> uint4 {
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

    // Operand reads of Q / K tiles (A or B operand of the Q K^T MFMA): row r,
    // 16-byte unit u of the k-slots this lane owns.
    auto k_unit = [&](auto bufc, int r, int u) -> uint4 {
        constexpr int buf = decltype(bufc)::value;
        if constexpr (DMA)
            return *reinterpret_cast<const uint4*>(&qk.k[buf][swz_off<RU>(r, u) / ESZ]);
        else
            return *reinterpret_cast<const uint4*>(&sm.Ks[r * KSTR + u * EPV]);
    };

    const int nch = (T + C - 1) / C;
    const int c_begin = seg * a.cps;
    const int c_end = (c_begin + a.cps < nch) ? c_begin + a.cps : nch;

    // One chunk.  B is the LDS buffer holding this chunk's Q / K (DMA path)
    // and the state-copy buffer the chunk reads; chunk c + 1 goes to 1 - B.
    auto step = [&](int c, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        constexpr int NB = 1 - B;
        const int t0 = c * C;
        const int clen = (T - t0 < C) ? (T - t0) : C;
        const bool tail = clen < C;  // uniform: only the last chunk can be short

        // This chunk's loads were issued one step ago, and the only vector-memory
        // ops issued after them are the previous step's output stores (vector
        // memory ops complete in issue order).  Before the first step nothing
        // else is in flight, so wait for everything.
        if (c == c_begin) wait_vmcnt<0>();
        else wait_vmcnt<STORES>();
        __syncthreads();  // loads landed everywhere; previous chunk's LDS reads done

        // ---- stage: K rows (fp32), the V slice (plain and zeta-scaled), feature maps
        if constexpr (!DMA) {
#pragma unroll
            for (int m = 0; m < KU; ++m) {
                const int u = tid + m * kThreads;
                const int row = u / RU, col = u % RU;
                uint4 x = kpre[m];
                if constexpr (LIN) x = apply_phi16(x);
                if (LIN && tail && row >= clen) x = uint4{0, 0, 0, 0};
                *reinterpret_cast<uint4*>(&sm.Ks[row * KSTR + col * EPV]) = x;
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bool pad = LIN && tail && (its(s) * 16 + l16 >= clen);
#pragma unroll
                for (int u = 0; u < QU; ++u) {
                    uint4 x = qnext[s][u];
                    if constexpr (LIN) x = apply_phi16(x);
                    qcur[s][u] = pad ? uint4{0, 0, 0, 0} : x;
                }
            }
        } else if constexpr (LIN) {
            // phi on this thread's DMA units of Q and K, in place; rows past the
            // end (loaded as zeros) must stay zero, not phi(0) = 1
#pragma unroll
            for (int m = 0; m < KU; ++m) {
                const int b = (W * KU + m) * 1024 + l * 16;
                const int r = b / (RU * 16);
                uint4* pk = reinterpret_cast<uint4*>(&qk.k[B][b / ESZ]);
                uint4* pq = reinterpret_cast<uint4*>(&qk.q[B][b / ESZ]);
                const unsigned keep = (tail && r >= clen) ? 0u : ~0u;  // bit mask, not a select
                uint4 xk = apply_phi16(*pk);
                uint4 xq = apply_phi16(*pq);
                xk.x &= keep; xk.y &= keep; xk.z &= keep; xk.w &= keep;
                xq.x &= keep; xq.y &= keep; xq.z &= keep; xq.w &= keep;
                *pk = xk;
                *pq = xq;
            }
        }
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
            const int u = tid + m * kThreads;
            if (VUT % kThreads == 0 || u < VUT) {
                const int row = u / VRU, col = u % VRU;
                const int ez = 16 + clen - 1 - row;  // gamma^(c-1-j); 0 past the end
                const float zeta = sm.dec[ez < 0 ? 0 : ez];
                uint4 x;
                if constexpr (DMA) x = *reinterpret_cast<const uint4*>(&qk.v[B][row * VSTR + col * EPV]);
                else x = vpre[m];
                uint4 xz;
                if constexpr (BF16) {
                    const u16x8 e = __builtin_bit_cast(u16x8, x);
                    u16x8 z;
#pragma unroll
                    for (int i = 0; i < 8; ++i) z[i] = f2bf(bf2f(e[i]) * zeta);
                    xz = __builtin_bit_cast(uint4, z);
                } else {
                    xz = __builtin_bit_cast(uint4, __builtin_bit_cast(f32x4, x) * zeta);
                }
                if constexpr (!DMA) *reinterpret_cast<uint4*>(&sm.Vs[row * VSTR + col * EPV]) = x;
                *reinterpret_cast<uint4*>(&sm.Vz[row * VSTR + col * EPV]) = xz;
            }
        }
        __syncthreads();

        if (c + 1 < c_end) load_chunk(c + 1, std::integral_constant<int, NB>{});

        // ---------------- Q operands of this wave's query tiles
        uint4 qb[NS][QU];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                if constexpr (DMA)
                    qb[s][u] = *reinterpret_cast<const uint4*>(&qk.q[B][swz_off<RU>(its(s) * 16 + l16, 4 * u + g) / ESZ]);
                else
                    qb[s][u] = qcur[s][u];
            }

        // ---------------- S^T tiles = K Q^T for key tiles jt <= query tile
        f32x4 pacc[NS][NI];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int jt = 0; jt < NI; ++jt) pacc[s][jt] = f32x4{0.f, 0.f, 0.f, 0.f};

        if constexpr (BF16) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                bf16x8 ka[ITMAX + 1];
#pragma unroll
                for (int jt = 0; jt <= ITMAX; ++jt) ka[jt] = as_bf16x8(k_unit(bufc, jt * 16 + l16, 4 * ks + g));
#pragma unroll
                for (int jt = 0; jt <= ITMAX; ++jt)
#pragma unroll
                    for (int s = 0; s < NS; ++s)
                        if (jt <= its(s)) pacc[s][jt] = mfma_bf16(ka[jt], as_bf16x8(qb[s][ks]), pacc[s][jt]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                f32x4 ka[ITMAX + 1];
#pragma unroll
                for (int jt = 0; jt <= ITMAX; ++jt)
                    ka[jt] = *reinterpret_cast<const f32x4*>(&sm.Ks[(jt * 16 + l16) * KSTR + (DK / 4) * g + 4 * u]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int jt = 0; jt <= ITMAX; ++jt)
#pragma unroll
                        for (int s = 0; s < NS; ++s)
                            if (jt <= its(s)) {
                                const f32x4 q4 = __builtin_bit_cast(f32x4, qb[s][u]);
                                pacc[s][jt] = mfma_f32(ka[jt][e], q4[e], pacc[s][jt]);
                            }
            }
        }

        // ---------------- state: S^T <- gamma^c S^T + (zeta V)^T K   (and z += sum phi(k))
        // Independent of the Q K^T tiles, so it is issued here, where its MFMAs
        // overlap the decay arithmetic below.  The per-tile accumulation chains
        // are interleaved (token blocks outer, tiles inner).
        f32x4 snew[SPW > 0 ? SPW : 1];
        float zsum[SPW > 0 ? SPW : 1];
        {
            const float gc = sm.dec[16 + clen];
#pragma unroll
            for (int m = 0; m < SPW; ++m) {
                snew[m] = sacc[m] * gc;
                zsum[m] = 0.f;
            }
            if constexpr (BF16) {
#pragma unroll
                for (int js = 0; js < C / 32; ++js) {
#pragma unroll
                    for (int m = 0; m < SPW; ++m) {
                        const int qt = TS + m;
                        const int nt = qt / KT, kt = qt % KT;
                        // A = (zeta V)^T, B = K: tokens 32js + 4g + {0..3}, 32js + 16 + 4g + {0..3}
                        const E* v0 = &sm.Vz[(32 * js + 4 * g + lq) * VSTR + nt * 16 + 4 * lr];
                        const bf16x8 av = cat_bf16(lds_tr4(v0), lds_tr4(v0 + 16 * VSTR));
                        const int r0 = 32 * js + 4 * g + lq;
                        const int c16 = 2 * kt + (lr >> 1), half = (lr & 1) * 8;
                        const u16x4 blo = lds_tr4(&qk.k[B][(swz_off<RU>(r0, c16) + half) / ESZ]);
                        const u16x4 bhi = lds_tr4(&qk.k[B][(swz_off<RU>(r0 + 16, c16) + half) / ESZ]);
                        snew[m] = mfma_bf16(av, cat_bf16(blo, bhi), snew[m]);
                        if (LIN && nt == 0) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) zsum[m] += bf2f(blo[r]) + bf2f(bhi[r]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int jt = 0; jt < NI; ++jt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
#pragma unroll
                        for (int m = 0; m < SPW; ++m) {
                            const int qt = TS + m;
                            const int nt = qt / KT, kt = qt % KT;
                            const float av = sm.Vz[(jt * 16 + 4 * g + r) * VSTR + nt * 16 + l16];
                            const float b = sm.Ks[(jt * 16 + 4 * g + r) * KSTR + kt * 16 + l16];
                            snew[m] = mfma_f32(av, b, snew[m]);
                            if (ZN && nt == 0) {
                                if constexpr (NRM) {
                                    // decayed key sums: zeta_j = gamma^(c-1-j), 0 past the end
                                    const int ez = 16 + clen - 1 - (jt * 16 + 4 * g + r);
                                    zsum[m] += b * sm.dec[ez < 0 ? 0 : ez];
                                } else {
                                    zsum[m] += b;
                                }
                            }
                        }
                    }
                }
            }
        }

        // ---------------- decay mask: P^T[j][i] = S^T[j][i] * gamma^(i-j), 0 for j > i
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int jt = 0; jt <= ITMAX; ++jt)
                if (jt <= its(s))
#pragma unroll
                    for (int r = 0; r < 4; ++r) pacc[s][jt][r] *= dfac[its(s) - jt][r];

        // bf16 copies of P^T, two key tiles per MFMA operand; row sums for the normaliser
        float rsum[NS];
        bf16x8 pb[NS][NI / 2];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            rsum[s] = 0.f;
            if constexpr (BF16) {
#pragma unroll
                for (int p = 0; p < NI / 2; ++p) {
                    if (2 * p <= its(s)) {
                        const u16x4 lo = cvt4_bf16(pacc[s][2 * p]);
                        const u16x4 hi = (2 * p + 1 <= its(s)) ? cvt4_bf16(pacc[s][2 * p + 1]) : u16x4{0, 0, 0, 0};
                        pb[s][p] = cat_bf16(lo, hi);
                        if constexpr (LIN) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) rsum[s] += bf2f(lo[r]) + bf2f(hi[r]);
                        }
                    }
                }
            } else if constexpr (ZN) {
#pragma unroll
                for (int jt = 0; jt <= ITMAX; ++jt)
                    if (jt <= its(s))
#pragma unroll
                        for (int r = 0; r < 4; ++r) rsum[s] += pacc[s][jt][r];
            }
        }

        // ---------------- O^T = S_prev^T (xi Q)^T + V^T P^T
        f32x4 oacc[NS][NT];
        const E* st = sm.Sts[B];
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
                    for (int s = 0; s < NS; ++s) oacc[s][nt] = mfma_bf16(av, as_bf16x8(qb[s][ks]), oacc[s][nt]);
                }
            } else {
#pragma unroll
                for (int u = 0; u < QU; ++u) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(srow + (DK / 4) * g + 4 * u);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int s = 0; s < NS; ++s) {
                            const f32x4 q4 = __builtin_bit_cast(f32x4, qb[s][u]);
                            oacc[s][nt] = mfma_f32(a4[e], q4[e], oacc[s][nt]);
                        }
                }
            }
            if constexpr (!LIN) {
#pragma unroll
                for (int s = 0; s < NS; ++s) oacc[s][nt] *= xi[s];
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if constexpr (BF16) {
#pragma unroll
                for (int p = 0; 2 * p <= ITMAX; ++p) {
                    // A = V^T: tokens 32p + 4g + {0..3} and 32p + 16 + 4g + {0..3} of column l16
                    const E* v0 = &qk.v[B][(32 * p + 4 * g + lq) * VSTR + nt * 16 + 4 * lr];
                    const bf16x8 av = cat_bf16(lds_tr4(v0), lds_tr4(v0 + 16 * VSTR));
#pragma unroll
                    for (int s = 0; s < NS; ++s)
                        if (2 * p <= its(s)) oacc[s][nt] = mfma_bf16(av, pb[s][p], oacc[s][nt]);
                }
            } else {
#pragma unroll
                for (int jt = 0; jt <= ITMAX; ++jt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float av = sm.Vs[(jt * 16 + 4 * g + r) * VSTR + nt * 16 + l16];
#pragma unroll
                        for (int s = 0; s < NS; ++s)
                            if (jt <= its(s)) oacc[s][nt] = mfma_f32(av, pacc[s][jt][r], oacc[s][nt]);
                    }
                }
            }
        }

        // ---------------- normalise (linear attention, row-sum floor) and store O
        float rden[NS];
        if constexpr (ZN) {
            const float* zc = sm.zs[B];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                float dq = 0.f;  // phi(q_i) . z over this lane's key slots
#pragma unroll
                for (int u = 0; u < QU; ++u) {
                    if constexpr (BF16) {
                        const u16x8 e = __builtin_bit_cast(u16x8, qb[s][u]);
#pragma unroll
                        for (int i = 0; i < 8; ++i) dq += bf2f(e[i]) * zc[32 * u + 8 * g + i];
                    } else {
                        const f32x4 e = __builtin_bit_cast(f32x4, qb[s][u]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) dq += e[i] * zc[(DK / 4) * g + 4 * u + i];
                    }
                }
                if constexpr (LIN) {
                    rden[s] = 1.f / (sum_over_groups(rsum[s] + dq) + a.eps);
                } else {
                    // retention: the earlier tokens' share is decayed by xi like the read-out
                    rden[s] = 1.f / fmaxf(fabsf(sum_over_groups(rsum[s] + xi[s] * dq)), 1.f);
                }
            }
        }
        // GroupNorm over each output row (the slice holds whole rows): lanes
        // l, l^16, l^32, l^48 hold the row's four column groups.  The row is
        // in registers, so the variance takes two passes (mean, then squared
        // deviations), which stays exact for rows whose mean dwarfs their spread.
        float mu[NS], rstd[NS];
        if constexpr (GRP) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                float s1 = 0.f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const f32x4 o = oacc[s][nt] * rden[s];
#pragma unroll
                    for (int r = 0; r < 4; ++r) s1 += o[r];
                }
                mu[s] = sum_over_groups(s1) * (1.f / Cf::DVS);
                float s2 = 0.f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const f32x4 o = oacc[s][nt] * rden[s] - mu[s];
#pragma unroll
                    for (int r = 0; r < 4; ++r) s2 += o[r] * o[r];
                }
                rstd[s] = 1.f / sqrtf(sum_over_groups(s2) * (1.f / Cf::DVS) + a.gn_eps);
            }
        }
        {
            const auto ro = make_rsrc(oh + mem_row0(t0, clen) * DV, clen * DV * ESZ);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int row = row_in(its(s) * 16 + l16, clen);  // rows past the end are dropped by the resource
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4 o = oacc[s][nt];
                    if constexpr (ZN) o *= rden[s];
                    if constexpr (GRP) o = (o - mu[s]) * rstd[s];
                    const unsigned off = static_cast<unsigned>((row * DV + nt * 16 + 4 * g) * ESZ);
                    if constexpr (BF16) bstore8(ro, off, cvt4_bf16(o));
                    else bstore16(ro, off, o);
                }
            }
        }

        // ---------------- commit the new state: fp32 master in registers, operand copy in LDS
        {
            E* stn = sm.Sts[NB];
#pragma unroll
            for (int m = 0; m < SPW; ++m) {
                const int qt = TS + m;
                const int nt = qt / KT, kt = qt % KT;
                const int kcol = kt * 16 + l16;
                sacc[m] = snew[m];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (BF16) stn[(nt * 16 + 4 * g + r) * KSTR + kcol] = f2bf(snew[m][r]);
                    else stn[(nt * 16 + 4 * g + r) * KSTR + kcol] = snew[m][r];
                }
                if (ZN && nt == 0) {
                    const float zt = sum_over_groups(zsum[m]);
                    // the row-sum floor's normaliser decays like the state: z = gamma^c z + sum zeta k
                    const float zd = NRM ? sm.dec[16 + clen] : 1.f;
                    if (g == 0) sm.zs[NB][kcol] = zd * sm.zs[B][kcol] + zt;
                }
            }
        }
    };

    if (c_begin < c_end) load_chunk(c_begin, std::integral_constant<int, 0>{});
    for (int c = c_begin; c < c_end; c += 2) {
        step(c, std::integral_constant<int, 0>{});
        if (c + 1 < c_end) step(c + 1, std::integral_constant<int, 1>{});
    }

    // ---------------- final state [dk][dv] fp32 (the last segment ends the sequence)
    if (a.final_state && seg == a.G - 1) {
        float* fs = a.final_state + static_cast<long long>(bh) * DK * DV + nbase;
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = TS + m;
            const int nt = qt / KT, kt = qt % KT;
            *reinterpret_cast<f32x4*>(fs + (kt * 16 + l16) * DV + nt * 16 + 4 * g) = sacc[m];
        }
    }
}

template <bool BF16, int C, int DK, int NT, int MODE>
__global__ void __launch_bounds__(kThreads, 1) walk_kernel(const WalkArgs a) {
    using Cf = Cfg<BF16, C, DK, NT, MODE>;
    using E = typename Cf::E;
    constexpr bool LIN = MODE == 1, ZN = MODE != 0;
    __shared__ Smem<BF16, C, DK, NT, MODE> sm;
    constexpr int QKN = Cf::DMA ? C * DK : 8;
    __shared__ __attribute__((aligned(16))) E sq0[QKN];
    __shared__ __attribute__((aligned(16))) E sq1[QKN];
    __shared__ __attribute__((aligned(16))) E sk0[QKN];
    __shared__ __attribute__((aligned(16))) E sk1[QKN];
    constexpr int VN = Cf::DMA ? C * Cf::VSTR : 8;
    __shared__ __attribute__((aligned(16))) E sv0[VN];
    __shared__ __attribute__((aligned(16))) E sv1[VN];
    const QKTiles<E> qk{{sq0, sq1}, {sk0, sk1}, {sv0, sv1}};

    // workgroup -> ((b*H + h) * G + segment, value slice); the slices of one
    // (b, h, segment) share an XCD
    int L = blockIdx.x;
    if (a.xcd_remap) {
        const int per = gridDim.x >> 3;
        L = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    }
    const int bhs = L / a.nslices;
    const int bh = bhs / a.G, seg = bhs % a.G;
    const int nbase = (L % a.nslices) * Cf::DVS;
    const int h = bh % a.H;
    const float lg = LIN ? 0.f : a.log2g[h];

    const int tid = threadIdx.x;
    for (int m = tid; m < Cf::DEC; m += kThreads)
        sm.dec[m] = (m < 16) ? 0.f : exp2f(static_cast<float>(m - 16) * lg);
    if constexpr (ZN) {
        // normaliser entering the segment: z_0 + the earlier segments' sums, each decayed
        // over the segments after it like the state (gamma = 1 for linear attention)
        const long long slot = static_cast<long long>(DK) * a.dv + DK;
        const float* zw = a.ws + static_cast<long long>(bh) * (a.G - 1) * slot + static_cast<long long>(DK) * a.dv;
        const float lseg = static_cast<float>(a.seg_len) * lg;
        for (int m = tid; m < DK; m += kThreads) {
            float z = (LIN && a.init_z) ? a.init_z[static_cast<long long>(bh) * DK + m] : 0.f;
            for (int j = 0; j < seg; ++j) z += exp2f(lseg * static_cast<float>(seg - 1 - j)) * zw[j * slot + m];
            sm.zs[0][m] = z;
        }
    }
    // (the first barrier inside walk_body orders these writes, and the state
    // copy walk_body writes, before any read)

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    switch (wave) {
        case 0: walk_body<BF16, C, DK, NT, MODE, 0>(a, sm, qk, bh, nbase, seg, lg); break;
        case 1: walk_body<BF16, C, DK, NT, MODE, 1>(a, sm, qk, bh, nbase, seg, lg); break;
        case 2: walk_body<BF16, C, DK, NT, MODE, 2>(a, sm, qk, bh, nbase, seg, lg); break;
        default: walk_body<BF16, C, DK, NT, MODE, 3>(a, sm, qk, bh, nbase, seg, lg); break;
    }
    if constexpr (LIN) {
        // the normaliser after the segment's last chunk sits in zs[chunks % 2];
        // every slice holds the same z, slice 0 of the last segment writes it
        if (a.final_z && nbase == 0 && seg == a.G - 1) {
            __syncthreads();
            const int nch = (a.T + C - 1) / C;
            const int c_begin = seg * a.cps;
            const int n = (c_begin < nch) ? nch - c_begin : 0;
            for (int m = tid; m < DK; m += kThreads) a.final_z[static_cast<long long>(bh) * DK + m] = sm.zs[n & 1][m];
        }
    }
}

// Segment contributions for the segmented walk.  Workgroup (b*H + h, j), for
// each full segment j < G - 1, writes
//   dS_j = sum_{t in segment j} gamma^(end_j - 1 - t) k_t v_t^T
// row-major [dk][dv] to workspace slot (b*H + h, j); for linear attention k_t
// is phi(k_t), gamma = 1, and z_j = sum phi(k_t) follows the state.  Wave w
// owns key-feature tiles {w, w + 4} and every value tile; each fp32 MFMA
// (16x16x4) contracts over 4 consecutive tokens: A = zeta K^T, B = V, both
// read straight from HBM / L2 (one 4- or 2-byte element per lane per tile).
template <bool BF16, int DK, int DV, int MODE>
__global__ void __launch_bounds__(kThreads) slice_state_kernel(const WalkArgs a) {
    using E = typename std::conditional<BF16, unsigned short, float>::type;
    constexpr bool LIN = MODE == 1, ZN = MODE != 0;
    constexpr int KT = DK / 16, NV = DV / 16, MW = KT / 4, ESZ = sizeof(E);
    static_assert(KT % 4 == 0, "every wave owns KT / 4 key-feature tiles");
    // token quads per batch (64 or 32 tokens); the next batch's loads stay in flight
    constexpr int U = (MW + NV <= 5) ? 16 : 8;
    const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x / (a.G - 1), seg = blockIdx.x % (a.G - 1);
    const float lg = LIN ? 0.f : a.log2g[bh % a.H];
    const long long t0 = static_cast<long long>(seg) * a.seg_len;
    // range-checked resources over exactly this segment: the prefetch past its
    // last batch reads zeros, so every load is unconditional.  A time-reversed
    // walk reads segment token t at row T - 1 - (t0 + t).
    const bool rev = a.reverse != 0;
    const long long mrow = rev ? a.T - t0 - a.seg_len : t0;
    const auto rk = make_rsrc(static_cast<const E*>(a.k) + (static_cast<long long>(bh) * a.T + mrow) * DK,
                              a.seg_len * DK * ESZ);
    const auto rv = make_rsrc(static_cast<const E*>(a.v) + (static_cast<long long>(bh) * a.T + mrow) * DV,
                              a.seg_len * DV * ESZ);
    auto ld = [](__amdgpu_buffer_rsrc_t r, int elem) -> float {
        if constexpr (BF16) {
            const unsigned short b = __builtin_amdgcn_raw_buffer_load_b16(r, elem * 2, 0, 0);
            return __uint_as_float(static_cast<unsigned>(b) << 16);
        } else {
            return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, elem * 4, 0, 0));
        }
    };
    // this lane's elements of the 64-token batch starting at token tb:
    // token tb + 4u + g, key features 16 (w + 4 mi) + l16, value features 16 n + l16
    float ka[2][U][MW], vb[2][U][NV];
    auto load = [&](int tb, auto bufc) {
        constexpr int b = decltype(bufc)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = tb + 4 * u + g;
            const int tr = rev ? a.seg_len - 1 - t : t;  // memory row within the segment
#pragma unroll
            for (int mi = 0; mi < MW; ++mi)
                ka[b][u][mi] = ld(rk, tr * DK + 16 * (w + 4 * mi) + l16);
#pragma unroll
            for (int n = 0; n < NV; ++n) vb[b][u][n] = ld(rv, tr * DV + 16 * n + l16);
        }
    };

    f32x4 acc[MW][NV];
    float zs[MW];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
        zs[mi] = 0.f;
#pragma unroll
        for (int n = 0; n < NV; ++n) acc[mi][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // A batch past the segment (at most one, when the batch count is odd) holds
    // zeros and gets zero weights: it adds nothing, phi(0) included.
    auto compute = [&](int tb, auto bufc) {
        constexpr int b = decltype(bufc)::value;
        const bool valid = tb < a.seg_len;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = tb + 4 * u + g;
            const float zeta = valid ? (LIN ? 1.f : exp2f(static_cast<float>(a.seg_len - 1 - t) * lg)) : 0.f;
#pragma unroll
            for (int mi = 0; mi < MW; ++mi) {
                const float x = (LIN ? phi_elu1(ka[b][u][mi]) : ka[b][u][mi]) * zeta;
                if constexpr (ZN) zs[mi] += x;  // phi(k), or zeta k for the row-sum floor
#pragma unroll
                for (int n = 0; n < NV; ++n) acc[mi][n] = mfma_f32(x, vb[b][u][n], acc[mi][n]);
            }
        }
    };
    // every full segment is a whole number of 64-token chunks, so of batches
    // (the empty asm statements keep the scheduler from sinking a prefetch
    // below the MFMAs it is meant to overlap)
    load(0, std::integral_constant<int, 0>{});
    for (int tb = 0; tb < a.seg_len; tb += 8 * U) {
        load(tb + 4 * U, std::integral_constant<int, 1>{});
        asm volatile("" ::: "memory");
        compute(tb, std::integral_constant<int, 0>{});
        load(tb + 8 * U, std::integral_constant<int, 0>{});
        asm volatile("" ::: "memory");
        compute(tb + 4 * U, std::integral_constant<int, 1>{});
    }
    const long long slot = static_cast<long long>(DK) * DV + (ZN ? DK : 0);
    float* out = a.ws + (static_cast<long long>(bh) * (a.G - 1) + seg) * slot;
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
        const int m = w + 4 * mi;
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[(16 * m + 4 * g + r) * DV + 16 * n + l16] = acc[mi][n][r];
        if constexpr (ZN) {
            const float z = sum_over_groups(zs[mi]);
            if (g == 0) out[DK * DV + 16 * m + l16] = z;
        }
    }
}

// LDS available to one workgroup on gfx950.
constexpr size_t kLdsBytes = 160 * 1024;

template <bool BF16, int C, int DK, int NT, int MODE>
constexpr bool fits() {
    using Cf = Cfg<BF16, C, DK, NT, MODE>;
    return sizeof(Smem<BF16, C, DK, NT, MODE>) + 4 * sizeof(typename Cf::E) * (Cf::DMA ? C * DK : 8) +
               2 * sizeof(typename Cf::E) * (Cf::DMA ? C * Cf::VSTR : 8) <= kLdsBytes;
}

template <bool BF16, int C, int DK, int NT, int MODE>
hipError_t launch_t(const WalkArgs& a, hipStream_t stream) {
    if constexpr (!fits<BF16, C, DK, NT, MODE>()) {
        return hipErrorInvalidConfiguration;
    } else {
    const long long groups = static_cast<long long>(a.B) * a.H * a.nslices * a.G;
    if (groups <= 0) return hipSuccess;
    if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
    WalkArgs args = a;
    args.xcd_remap = (groups % 8 == 0) ? 1 : 0;
    args.seg_len = a.cps * C;
    if (a.G > 1 && !a.ws_tr) {
        const long long sgroups = static_cast<long long>(a.B) * a.H * (a.G - 1);
        const int dv = a.dv;
#define RET_SLICE_STATE(DV_)                                                                             \
        if (dv == DV_) hipLaunchKernelGGL((slice_state_kernel<BF16, DK, DV_, MODE>),                      \
                                          dim3(static_cast<unsigned>(sgroups)), dim3(kThreads), 0, stream, args);
        RET_SLICE_STATE(64)
        RET_SLICE_STATE(128)
#undef RET_SLICE_STATE
        if (dv != 64 && dv != 128) return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((walk_kernel<BF16, C, DK, NT, MODE>), dim3(static_cast<unsigned>(groups)),
                       dim3(kThreads), 0, stream, args);
    return hipGetLastError();
    }
}

// Instantiates every (chunk, dk, NT) variant for one (dtype, operator) pair.
template <bool BF16, int MODE>
hipError_t launch_variant(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream) {
#define RET_WALK_CASE(C_, DK_, NT_) \
    if (chunk == C_ && dk == DK_ && nt == NT_) return launch_t<BF16, C_, DK_, NT_, MODE>(a, stream);
    RET_WALK_CASE(64, 64, 1)
    RET_WALK_CASE(64, 64, 2)
    RET_WALK_CASE(64, 128, 1)
    RET_WALK_CASE(64, 128, 2)
    RET_WALK_CASE(128, 64, 1)
    RET_WALK_CASE(128, 64, 2)
    RET_WALK_CASE(128, 128, 1)
    RET_WALK_CASE(128, 128, 2)
    if constexpr (!BF16) {
        RET_WALK_CASE(64, 64, 4)
        RET_WALK_CASE(64, 64, 8)
        RET_WALK_CASE(64, 128, 4)
        RET_WALK_CASE(64, 128, 8)
        RET_WALK_CASE(128, 64, 4)
        RET_WALK_CASE(128, 128, 4)
    }
#undef RET_WALK_CASE
    return hipErrorInvalidValue;
}

// Whether the (chunk, dk, NT) variant fits in LDS (and is instantiated).
template <bool BF16, int MODE>
bool variant_fits(int chunk, int dk, int nt) {
#define RET_WALK_FITS(C_, DK_, NT_) \
    if (chunk == C_ && dk == DK_ && nt == NT_) return fits<BF16, C_, DK_, NT_, MODE>();
    RET_WALK_FITS(64, 64, 1)
    RET_WALK_FITS(64, 64, 2)
    RET_WALK_FITS(64, 128, 1)
    RET_WALK_FITS(64, 128, 2)
    RET_WALK_FITS(128, 64, 1)
    RET_WALK_FITS(128, 64, 2)
    RET_WALK_FITS(128, 128, 1)
    RET_WALK_FITS(128, 128, 2)
    if constexpr (!BF16) {
        RET_WALK_FITS(64, 64, 4)
        RET_WALK_FITS(64, 64, 8)
        RET_WALK_FITS(64, 128, 4)
        RET_WALK_FITS(64, 128, 8)
        RET_WALK_FITS(128, 64, 4)
        RET_WALK_FITS(128, 128, 4)
    }
#undef RET_WALK_FITS
    return false;
}

}  // namespace walk
}  // namespace ret
