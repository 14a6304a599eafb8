// gla.hip -- chunkwise gated linear attention (per-token, per-key-channel
// gates), fp32 arithmetic, fp32 or bf16 q/k/v/out, gfx950.
//
// What is computed ("Efficient and Sparse Transformers", section "Gated
// Linear Attention: Toward Input-Dependent Forgetting": the fixed decay of
// RetNet becomes a data-dependent gate applied element-wise to the state; here
// one gate per key channel, alpha_t = exp(lg_t)):
//   S_t[c][n] = alpha_t[c] S_{t-1}[c][n] + k_t[c] v_t[n],   o_t = q_t S_t.
// Chunk form.  With b_i[c] the log-gates summed over the chunk up to and
// including its token i (non-increasing in i), b_L its value at the chunk's
// last token, and S the state before the chunk:
//   o_i   = sum_{j<=i} sum_c q_i[c] k_j[c] e^{b_i[c] - b_j[c]} v_j + sum_c q_i[c] e^{b_i[c]} S[c][:]
//   S_new = diag(e^{b_L}) S + sum_j diag(e^{b_L - b_j}) k_j v_j^T
//
// Tile-relative factors.  The chunk's 64 tokens form four 16-token tiles.  For
// token i of tile I let cum_i be the gate sum from the tile's start to i, t_I
// the tile's total and B_I = t_0 + ... + t_I (B_{-1} = 0), so b_i = B_{I-1} +
// cum_i.  Every operand is folded once per chunk and stays bounded:
//   Q^ = q e^{cum_i}             (<= |q|)    queries, relative to their tile's start
//   K^ = k e^{t_J - cum_j}       (<= |k|)    keys, relative to their tile's end
//   K' = k e^{b_L - b_j}         (<= |k|)    keys for the state update
// and the scores of query tile I against key tile J <= I are
//   P^T = K^ (Q^ (.) F_IJ)^T,  F_IJ = e^{B_{I-1} - B_J} (<= 1) for J < I,
//                              F_II = e^{-t_I}          (>= 1) on the diagonal,
// with F_{I,I-1} = 1; the inter-chunk read takes Q^ (.) e^{B_{I-1}} (<= |q|).
// Only F_II grows, as e^{-t_I}: it stays finite while every 16-token tile's
// gate sum is above -80 in every channel.  A chunk with a stronger tile (a
// gate below e^-5 per token on average over 16 tokens) forms its scores term
// by term instead (exact path), one exponent e^{b_i - b_j} <= 1 per term.  The
// masked upper triangle of the diagonal tile is discarded by a select.
//
// Segments.  Each (b, h) sequence is cut into G segments of whole chunks.  A
// state-only pass (SO) walks every segment but the last and writes its
// contribution dS_j (the state it would end with from zero) and its per-channel
// log-gate total L_j; the walk of segment g starts from
//   S_in(g) = sum_{j<g} diag(exp(L_{j+1} + ... + L_{g-1})) dS_j,
// all exponents <= 0.
//
// Mapping.  One workgroup of 8 waves per (b, h, segment, 64-column value
// slice) walks the segment's 64-token chunks, so Q K^T is formed once per
// chunk for the whole slice (the only slice when dv = 64).
//  - Folding: lane l of wave w covers tokens 4 (l % 16) .. + 3 (in tile
//    (l % 16) / 4) of the 4 channels 16 (w % 4) + 4 (l / 16) .. + 3 (+ 64 for
//    dk = 128), loaded as 16-byte (bf16: 8-byte) runs.  Waves 4-7 fold the
//    keys.  At dk = 64 they also fold the queries and stage the same 4 value
//    columns of their channel slice over the same tokens, sharing one set of
//    gate sums, and waves 0-3 do nothing but products; at dk = 128 wave w
//    folds query slice w and stages value slice w.  Running sums: a sum over the lane's 4
//    tokens, a DPP prefix scan over the 16 lanes of a row, and shuffles for
//    the tile totals.  The next chunk's raw q or k, gates and values are
//    loaded straight into registers (range-checked buffer loads: rows past
//    the end read as zeros) while the current chunk is computed.
//  - LDS layouts: Q^, K^ and the S^T copy row-major by token / value column
//    with channels in order; K' and V transposed ([channel][key],
//    [column][key]).  In every product a lane of group g contracts over a run
//    of 4 consecutive channels or keys, so each MFMA operand pair comes from
//    16-byte reads and the folded keys and values go in with 16-byte writes.
//  - Products: waves 0-3 (O-waves) own query tile W: scores, then O^T = S^T
//    Q~^T + V^T P^T over the slice.  Waves 4-7 (S-waves) own state tiles,
//    split so that each SIMD (O-wave W and S-wave W + 4) issues the same
//    number of MFMAs.  The state-only pass splits the state tiles over all 8.
//  - Two barriers per chunk: after the folded operands are written, and after
//    the products (then the S-waves refresh the LDS copy of S^T).  Whether a
//    chunk needs the exact path is voted on by the key waves between those two
//    barriers of the step before the one that folds it (at dk = 64; right
//    after its products at dk = 128), once its gates have arrived.
//  - On gfx950 fp32 MFMAs and VALU instructions of the two waves of a SIMD do
//    not overlap (each SIMD's time is its VALU plus its MFMA time), so the
//    fold is written for few VALU instructions: gate sums in log2 units,
//    summed once per lane, one v_exp_f32 per factor.
#include "internal.h"
#include "kcommon.h"

namespace ret {
namespace gla {
namespace {

using namespace ::ret::kc;

constexpr int kThreads = 512;
constexpr int C = 64;
constexpr float kLog2e = 1.4426950408889634f;
// Gate sums are kept in log2 units (log-gate times log2 e), so every factor is
// one v_exp_f32.  F_II = 2^{-t_I} <= 2^{80 log2 e} = e^{80} = 5.5e34.
constexpr float kTileBound = -80.f * kLog2e;

template <int DK, int NT>
struct Cfg {
    static constexpr int KT = DK / 16;              // channel tiles
    static constexpr int DVS = 16 * NT;             // value columns per workgroup
    static constexpr int QS = DK + 4;               // row stride (floats) of Q^, K^ and the S^T copy
    static constexpr int CS = C + 4;                // row stride of the transposed K' and V
    static constexpr int NTILE = KT * NT;           // 16 x 16 state tiles
    static constexpr int CPT = DK / 64;             // channels folded per thread
    static_assert(DVS == 64, "the O-side waves stage 64 value columns");
    static_assert(NTILE % 8 == 0, "state tiles split over 8 waves in the state-only pass");
};

// Rows of the factor table (each DK floats, channels in order):
//   0..3   F_II = e^{-t_I}
//   4, 5   F_20, F_30 = e^{B_1 - B_0}, e^{B_2 - B_0}
//   6      F_31 = e^{B_2 - B_1}
//   7..9   E_I = e^{B_{I-1}} for I = 1..3 (inter-chunk read)
constexpr int kFRows = 10;
constexpr int frow(int I, int J) { return I == J ? I : (I == 2 && J == 0) ? 4 : (I == 3 && J == 0) ? 5 : 6; }

// Buffer sets of folded operands: two at dk = 64, so that the next chunk is
// folded while the current one's products run; one at dk = 128 (LDS).
template <int DK>
constexpr int nbuf() { return DK == 64 ? 2 : 1; }

template <int DK, int NT>
struct OpBuf {
    using Cf = Cfg<DK, NT>;
    alignas(16) float qb[C * Cf::QS];        // Q^ [token][channel]; exact path: raw q
    alignas(16) float kb[C * Cf::QS];        // K^ [key][channel]; exact path: raw k
    alignas(16) float gt[DK * Cf::CS];       // K'^T [channel][key]; exact path: b^T
    alignas(16) float vt[Cf::DVS * Cf::CS];  // V^T [column][key]
    alignas(16) float fb[kFRows * DK];       // factor table
    alignas(16) float bl[DK];                // e^{b_L} per channel
};

template <int DK, int NT>
struct Smem {
    using Cf = Cfg<DK, NT>;
    OpBuf<DK, NT> op[nbuf<DK>()];
    alignas(16) float sc[Cf::DVS * Cf::QS];  // S^T copy: sc[n][c] = S[c][nbase + n]
    int flag[2][4];                          // [chunk parity][key wave]: a tile past the bound (exact path)
};

template <int DK, int NT>
constexpr bool fits() { return sizeof(Smem<DK, NT>) <= 160 * 1024; }
static_assert(sizeof(Smem<64, 4>) <= 160 * 1024 && sizeof(Smem<128, 4>) <= 160 * 1024, "LDS");

// State tiles of each S-wave in the walk.  O-wave W issues (W+1) DK/4 score,
// 4 NT (W+1) intra-chunk and NT DK/4 inter-chunk MFMAs per chunk; a state
// tile costs 16 (64 keys / 4).  S-wave W + 4 takes the tiles that bring its
// SIMD to the mean.
struct Split {
    int first[4];
    int cnt[4];
};

template <int DK, int NT>
constexpr Split make_split() {
    constexpr int NTILE = (DK / 16) * NT;
    int work[4] = {};
    int total = 16 * NTILE;
    for (int w = 0; w < 4; ++w) {
        work[w] = (w + 1) * (DK / 4) + 4 * NT * (w + 1) + NT * (DK / 4);
        total += work[w];
    }
    Split s{};
    int sum = 0;
    for (int w = 0; w < 4; ++w) {
        int c = (total / 4 - work[w] + 8) / 16;
        if (c < 0) c = 0;
        s.cnt[w] = c;
        sum += c;
    }
    while (sum != NTILE) {  // even out rounding: adjust the most / least loaded SIMD
        int best = 0;
        for (int w = 1; w < 4; ++w) {
            const int lw = work[w] + 16 * s.cnt[w], lb = work[best] + 16 * s.cnt[best];
            if (sum > NTILE ? (lw > lb && s.cnt[w] > 0) || s.cnt[best] == 0 : lw < lb) best = w;
        }
        s.cnt[best] += (sum > NTILE) ? -1 : 1;
        sum += (sum > NTILE) ? -1 : 1;
    }
    int f = 0;
    for (int w = 0; w < 4; ++w) {
        s.first[w] = f;
        f += s.cnt[w];
    }
    return s;
}

// 4 consecutive q, k or v elements: fp32 (16 bytes) or bf16 (8 bytes), kept
// raw in registers until they are folded (widening them at load time would
// make the compiler wait for the load there).
template <bool BF>
struct Quad;
template <>
struct Quad<false> {
    u32x4 x;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        x = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
    }
    __device__ __forceinline__ f32x4 f() const { return __builtin_bit_cast(f32x4, x); }
};
template <>
struct Quad<true> {
    u32x2 x;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        x = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, 0);
    }
    __device__ __forceinline__ f32x4 f() const {
        const u16x4 e = __builtin_bit_cast(u16x4, x);
        return f32x4{bf2f(e[0]), bf2f(e[1]), bf2f(e[2]), bf2f(e[3])};
    }
};

// Inclusive prefix sum over the 16 lanes of a DPP row (lanes shifted in from
// outside the row read as zero).
__device__ __forceinline__ float row_scan16(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true));
    return x;
}

// 4 output values at byte offset off of a chunk's range-checked output
// resource: rows past the chunk's end are dropped without a branch.
template <bool BF>
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, unsigned off, const f32x4& o) {
    if constexpr (BF) bstore8(r, off, cvt4_bf16(o));
    else bstore16(r, off, o);
}

__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// The lane's index, hidden from loop-invariant code motion: re-issued in every
// chunk step, it keeps the compiler from hoisting each LDS address of the
// products out of the chunk loop (one register each for the whole walk); the
// addresses then share a base register per array and immediate offsets.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ void sts4(float* p, const f32x4& x) { *reinterpret_cast<f32x4*>(p) = x; }

// 2^x on v_exp_f32 (about 1 ulp), x a gate sum in log2 units.  Results below
// the normal range flush to zero: every factor here is a decay or a product
// with one, and a factor under 1e-38 contributes nothing at fp32 precision.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool BF, int DK, int NT, int W8, bool SO>
__device__ __forceinline__ void body(const GlaArgs& a, Smem<DK, NT>& sm, int bh, int seg, int nbase) {
    using Cf = Cfg<DK, NT>;
    using Buf = OpBuf<DK, NT>;
    constexpr int QS = Cf::QS, CS = Cf::CS, KT = Cf::KT, NTILE = Cf::NTILE;
    constexpr int CPT = Cf::CPT, NQ = DK / 4, NB = nbuf<DK>();
    constexpr int ESZ = BF ? 2 : 4;
    constexpr bool QW = W8 < 4;         // waves 0-3
    constexpr bool OW = !SO && QW;      // output wave: query tile W8
    constexpr Split SP = make_split<DK, NT>();
    constexpr int TF = SO ? W8 * (NTILE / 8) : (OW ? 0 : SP.first[W8 - 4]);
    constexpr int TN = SO ? NTILE / 8 : (OW ? 0 : SP.cnt[W8 - 4]);
    constexpr int W = W8 & 3;
    // Fold roles in the walk: at dk = 64 S-wave W + 4 folds the channel /
    // value-column slice W of q, k and v, sharing one set of gate sums, and
    // the O-waves do nothing but products (fp32 MFMAs do not overlap VALU work
    // on the same SIMD, so every gate scan done twice costs its full time).
    // At dk = 128 (twice the raw registers per fold) O-wave W folds q slice W.
    // The state-only pass: waves 0-3 stage v, waves 4-7 fold k.
    constexpr bool LQ = !SO && (DK == 64 ? !QW : QW);  // folds q
    constexpr bool LK = !QW;                           // folds k
    constexpr bool LV = SO ? QW : LQ;                  // stages v
    constexpr bool LG = LQ || LK;                      // loads gates
    const int T = a.T, DV = a.dv;
    const int l = threadIdx.x & 63, l16 = l & 15, g = l >> 4;
    const char* qh = static_cast<const char*>(a.q) + static_cast<long long>(bh) * T * DK * ESZ;
    const char* kh = static_cast<const char*>(a.k) + static_cast<long long>(bh) * T * DK * ESZ;
    const float* gh = a.lg + static_cast<long long>(bh) * T * DK;
    const char* vh = static_cast<const char*>(a.v) + (static_cast<long long>(bh) * T * DV + nbase) * ESZ;
    char* oh = static_cast<char*>(a.out) + (static_cast<long long>(bh) * T * DV + nbase) * ESZ;

    // ---- state tiles of this wave: tile t = (m = t % KT channel tile, n = t / KT value tile);
    // lane holds S[16 m + 4 g + r][nbase + 16 n + l16]
    f32x4 sacc[TN > 0 ? TN : 1];
#pragma unroll
    for (int t = 0; t < TN; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const long long slot = static_cast<long long>(DK) * DV + DK;  // workspace floats per (b, h, segment)
    // S^T copy: the lane's 4 values are 4 consecutive channels of value column 16 n + l16
    auto write_state_copy = [&]() {
        if constexpr (!SO && !OW) {
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                const int m = (TF + t) % KT, n = (TF + t) / KT;
                sts4(&sm.sc[(16 * n + l16) * QS + 16 * m + 4 * g], sacc[t]);
            }
        }
    };
    // Run after the first chunk's loads are issued, so that their latency and
    // the prologue's overlap.
    auto prologue = [&]() {
        if constexpr (SO) return;
        // ---- the state entering the segment, by every thread of the workgroup:
        //   S_in = sum_{j<seg} diag(exp(L_{j+1} + ... + L_{seg-1})) dS_j
        // (all exponents <= 0), newest segment first.  Thread t takes EPT
        // consecutive columns of one row of the slice and keeps up to SB
        // segments' values in flight; the sums go to the state copy, from
        // which the key waves take their tiles after the first barrier.
        constexpr int EPT = DK * Cf::DVS / kThreads;  // 8 (dk = 64) or 16 (dk = 128)
        constexpr int V4 = EPT / 4;
        constexpr int SB = (DK == 64) ? 8 : 4;       // segments' values in flight per thread
        const int tid = threadIdx.x;
        const int row = tid / (Cf::DVS / EPT), col0 = (tid % (Cf::DVS / EPT)) * EPT;
        f32x4 acc[V4];
#pragma unroll
        for (int v4 = 0; v4 < V4; ++v4) acc[v4] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (seg > 0) {
            const float* wsb = a.ws + static_cast<long long>(bh) * (a.G - 1) * slot;
            float esum = 0.f;  // log-gate total of the segments already added
            for (int j0 = seg - 1; j0 >= 0; j0 -= SB) {
                f32x4 x[SB][V4];
                float L[SB];
#pragma unroll
                for (int b = 0; b < SB; ++b) {
                    const int j = j0 - b;
                    const float* sj = wsb + static_cast<long long>(j < 0 ? 0 : j) * slot;
#pragma unroll
                    for (int v4 = 0; v4 < V4; ++v4)
                        x[b][v4] = (j >= 0) ? *reinterpret_cast<const f32x4*>(sj + row * DV + nbase + col0 + 4 * v4)
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
                    L[b] = (j >= 0) ? sj[DK * DV + row] : 0.f;
                }
#pragma unroll
                for (int b = 0; b < SB; ++b) {
                    const float wgt = fexp2(esum);
#pragma unroll
                    for (int v4 = 0; v4 < V4; ++v4) acc[v4] += wgt * x[b][v4];
                    esum += L[b];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) sm.sc[(col0 + i) * QS + row] = acc[i / 4][i % 4];
    };

    // ---- raw chunk registers.  Lane l of wave W8 covers token group tg = l % 16
    // (tokens 4 tg .. 4 tg + 3, tile TT = tg / 4) of channel group cg = l / 16:
    // channels c0(u) = 16 W + 4 cg + 64 u .. + 3 (q, k and the gates, as the
    // wave's roles say) and value columns 16 W + 4 cg .. + 3.  A channel
    // group's 16 token groups fill one DPP row, so running sums over the chunk
    // are row scans.
    const int tg = l & 15, cg = l >> 4, TT = tg >> 2;
    Quad<BF> rq[CPT][4], rk[CPT][4], rv[4];
    f32x4 rgt[CPT][4];
    const int nch = (T + C - 1) / C;
    const int c_begin = seg * a.cps;
    const int c_end = (c_begin + a.cps < nch) ? c_begin + a.cps : nch;
    auto chunk_len = [&](int c) {
        const long long t0 = static_cast<long long>(c) * C;
        return (T - t0 < C) ? static_cast<int>(T - t0) : C;
    };
    // Issued for every step (a chunk past the segment gets a zero-length
    // range and reads zeros), so the compiler's waits see one shape.
    auto load_chunk = [&](int c) {
        const int tg = opaque(l & 15), cg = opaque(l >> 4);
        const long long t0 = static_cast<long long>(c) * C;
        const int cl = (c < c_end) ? chunk_len(c) : 0;
        if constexpr (LG) {
            const auto rsq = make_rsrc(qh + t0 * DK * ESZ, cl * DK * ESZ);
            const auto rsk = make_rsrc(kh + t0 * DK * ESZ, cl * DK * ESZ);
            const auto rsg = make_rsrc(gh + t0 * DK, cl * DK * 4);
#pragma unroll
            for (int u = 0; u < CPT; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned e = static_cast<unsigned>((4 * tg + i) * DK + 16 * W + 4 * cg + 64 * u);
                    if constexpr (LQ) rq[u][i].load(rsq, e * ESZ);
                    if constexpr (LK) rk[u][i].load(rsk, e * ESZ);
                    rgt[u][i] = __builtin_bit_cast(f32x4, bload16(rsg, e * 4));
                }
        }
        if constexpr (LV) {
            const auto rsv = make_rsrc(vh + t0 * DV * ESZ, cl * DV * ESZ);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rv[i].load(rsv, static_cast<unsigned>(((4 * tg + i) * DV + 16 * W + 4 * cg) * ESZ));
        }
    };
    // The log-gates of this lane's 4 channels, taken as 0 above 0 (NaN kept)
    // and scaled to log2 units, summed over the lane's 4 tokens in place:
    // rgt[u][i] becomes the sum up to and including token i.  The key waves do
    // it when they vote on the chunk, the other folding waves in gate_sums.
    constexpr bool PRESUM = !SO && !QW;
    auto lane_sums = [&](int u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = rgt[u][i][e];
                run = __builtin_fmaf((x > 0.f) ? 0.f : x, kLog2e, run);
                rgt[u][i][e] = run;
            }
        }
    };
    // Gate sums of this lane's 4 channels over the chunk: b[i] at its tokens
    // and the tile boundary sums B[0..3] (B[3] = b_L).
    auto gate_sums = [&](int u, f32x4 (&b)[4], f32x4 (&B)[4]) {
        if constexpr (!PRESUM) lane_sums(u);
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = rgt[u][i];
        const f32x4 run = rgt[u][3];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float incl = row_scan16(run[e]);
            const float ex = incl - run[e];
#pragma unroll
            for (int i = 0; i < 4; ++i) b[i][e] += ex;
#pragma unroll
            for (int j = 0; j < 4; ++j) B[j][e] = __shfl(incl, 16 * cg + 4 * j + 3);
        }
    };
    // Exact-path vote for the chunk now in the registers (key waves only): a
    // 16-token tile whose gate sum in some channel is below the bound, or NaN.
    auto vote = [&](int c) {
        if constexpr (PRESUM) {
            bool bad = false;
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                lane_sums(u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float run = rgt[u][3][e];
                    // the tile's sum: this lane and the next three token groups
                    float tile = run;
                    tile += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, run), 0x101, 0xf, 0xf, true));
                    tile += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, run), 0x102, 0xf, 0xf, true));
                    tile += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, run), 0x103, 0xf, 0xf, true));
                    bad = bad || ((tg & 3) == 0 && !(tile >= kTileBound));
                }
            }
            const bool wbad = __any(bad);
            if (l == 0) sm.flag[c & 1][W] = wbad ? 1 : 0;
        }
    };
    // Wave-uniform (a scalar), so the fold and the products branch on it
    // instead of computing both paths and selecting.
    auto exact_of = [&](int c) {
        if constexpr (SO) return false;
        const int f = sm.flag[c & 1][0] | sm.flag[c & 1][1] | sm.flag[c & 1][2] | sm.flag[c & 1][3];
        return __builtin_amdgcn_readfirstlane(f) != 0;
    };

    f32x4 ltot[CPT];  // state-only pass: log-gate totals of this lane's channels over the segment
#pragma unroll
    for (int u = 0; u < CPT; ++u) ltot[u] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- fold the chunk in the registers into a buffer set
    auto fold = [&](Buf& bf, bool exact) {
        const int tg = opaque(l & 15), cg = opaque(l >> 4), TT = tg >> 2;
        if constexpr (LG) {
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int c0 = 16 * W + 4 * cg + 64 * u;
                f32x4 b[4], B[4];
                gate_sums(u, b, B);
                // B[TT - 1] and B[TT] by selects (TT varies across lanes; no indexed registers)
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 boff = (TT == 0) ? zero : (TT == 1) ? B[0] : (TT == 2) ? B[1] : B[2];
                const f32x4 bI = (TT == 0) ? B[0] : (TT == 1) ? B[1] : (TT == 2) ? B[2] : B[3];
                const f32x4 tI = bI - boff;
                const f32x4 bL = B[3];
                if constexpr (LQ) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const f32x4 x = rq[u][i].f();
                        f32x4 y;
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = exact ? x[e] : x[e] * fexp2(b[i][e] - boff[e]);
                        sts4(&bf.qb[(4 * tg + i) * QS + c0], y);
                    }
                    if (TT > 0 && (tg & 3) == 0)
                        sts4(&bf.fb[(6 + TT) * DK + c0], f32x4{fexp2(boff[0]), fexp2(boff[1]), fexp2(boff[2]), fexp2(boff[3])});
                }
                if constexpr (LK) {
                    f32x4 xk[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) xk[i] = rk[u][i].f();
                    if (exact) {
                        // raw k and b^T: the products form every factor on the spot
#pragma unroll
                        for (int i = 0; i < 4; ++i) sts4(&bf.kb[(4 * tg + i) * QS + c0], xk[i]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sts4(&bf.gt[(c0 + e) * CS + 4 * tg], f32x4{b[0][e], b[1][e], b[2][e], b[3][e]});
                    } else {
                        // K^ = k e^{t_I - cum_j}, and K' = k e^{b_L - b_j} = K^ e^{b_L - B_I}
                        // (b_L - B_I: the gates of the tiles after token j's, <= 0; when it
                        // underflows, K' is below 1e-38 |k| and nothing is lost)
                        f32x4 kh[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int e = 0; e < 4; ++e) kh[i][e] = xk[i][e] * fexp2(tI[e] - (b[i][e] - boff[e]));
                        if constexpr (!SO) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) sts4(&bf.kb[(4 * tg + i) * QS + c0], kh[i]);
                        }
                        f32x4 after;
#pragma unroll
                        for (int e = 0; e < 4; ++e) after[e] = fexp2(bL[e] - bI[e]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sts4(&bf.gt[(c0 + e) * CS + 4 * tg],
                                 f32x4{kh[0][e] * after[e], kh[1][e] * after[e], kh[2][e] * after[e], kh[3][e] * after[e]});
                    }
                    if ((tg & 3) == 0) {
                        if constexpr (SO) {
                            if (TT == 0) ltot[u] += bL;
                        } else {
                            if (!exact)
                                sts4(&bf.fb[TT * DK + c0], f32x4{fexp2(-tI[0]), fexp2(-tI[1]), fexp2(-tI[2]), fexp2(-tI[3])});
                            if (TT == 0) {
                                const f32x4 d1 = B[1] - B[0], d2 = B[2] - B[0];
                                sts4(&bf.fb[4 * DK + c0], f32x4{fexp2(d1[0]), fexp2(d1[1]), fexp2(d1[2]), fexp2(d1[3])});
                                sts4(&bf.fb[5 * DK + c0], f32x4{fexp2(d2[0]), fexp2(d2[1]), fexp2(d2[2]), fexp2(d2[3])});
                            } else if (TT == 1) {
                                const f32x4 d3 = B[2] - B[1];
                                sts4(&bf.fb[6 * DK + c0], f32x4{fexp2(d3[0]), fexp2(d3[1]), fexp2(d3[2]), fexp2(d3[3])});
                            }
                        }
                        if (TT == 0) sts4(&bf.bl[c0], f32x4{fexp2(bL[0]), fexp2(bL[1]), fexp2(bL[2]), fexp2(bL[3])});
                    }
                }
            }
        }
        if constexpr (LV) {
            // values: columns 16 W + 4 cg + e of the slice, keys 4 tg .. 4 tg + 3, stored transposed
            f32x4 xv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = rv[i].f();
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sts4(&bf.vt[(16 * W + 4 * cg + e) * CS + 4 * tg], f32x4{xv[0][e], xv[1][e], xv[2][e], xv[3][e]});
        }
    };

    // ---- products of a chunk from buffer set X
    // Products.  Each runs as one unrolled sequence of groups of 4 MFMAs that
    // share one 16-byte LDS operand read; every group's operands are read RA
    // groups ahead (a ring of RA + 1 register sets), so the MFMAs do not wait
    // on fresh LDS reads.  A scheduling barrier after each group keeps the
    // compiler from hoisting the whole sequence's reads (and their registers).
    constexpr int RA = 2;
    auto products = [&](const Buf& bf, long long t0, int clen, bool exact) {
        const int l16 = opaque(l & 15), g = opaque(l >> 4);
        if constexpr (OW) {
            constexpr int SG = NQ / 4;  // groups per contraction over the channels
            const int qrow = 16 * W + l16;
            float qo[NQ];  // Q^ of query row qrow, channels NQ g + s (exact path: raw q)
#pragma unroll
            for (int s4 = 0; s4 < SG; ++s4) {
                const f32x4 x = lds4(&bf.qb[qrow * QS + NQ * g + 4 * s4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) qo[4 * s4 + e] = x[e];
            }
            f32x4 pacc[W + 1];
            if (!exact) {
                // scores P^T[key 16 J + 4 g + r][query] = K^ (Q^ (.) F_WJ)^T: group (J, s4)
                // contracts channels NQ g + 4 s4 .. + 3 of key tile J (F_{W,W-1} = 1 is not read)
                constexpr int NG = (W + 1) * SG;
                auto k_at = [&](int gi) { return lds4(&bf.kb[(16 * (gi / SG) + l16) * QS + NQ * g + 4 * (gi % SG)]); };
                auto f_at = [&](int gi) {
                    const int J = gi / SG;
                    return (J == W - 1) ? f32x4{1.f, 1.f, 1.f, 1.f}
                                        : lds4(&bf.fb[frow(W, J) * DK + NQ * g + 4 * (gi % SG)]);
                };
                f32x4 kr[RA + 1], fr[RA + 1];
#pragma unroll
                for (int i = 0; i < RA; ++i) {
                    kr[i] = k_at(i);
                    fr[i] = f_at(i);
                }
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    if (gi + RA < NG) {
                        kr[(gi + RA) % (RA + 1)] = k_at(gi + RA);
                        fr[(gi + RA) % (RA + 1)] = f_at(gi + RA);
                    }
                    const int J = gi / SG, s4 = gi % SG, x = gi % (RA + 1);
                    if (s4 == 0) pacc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int e = 0; e < 4; ++e) pacc[J] = mfma_f32(kr[x][e], qo[4 * s4 + e] * fr[x][e], pacc[J]);
                    __builtin_amdgcn_sched_barrier(0);  // keep the read-ahead distance (and the registers it needs)
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) pacc[W][r] = (4 * g + r > l16) ? 0.f : pacc[W][r];
                if constexpr (W > 0) {  // the inter-chunk read takes Q^ (.) E_W, E_W = e^{B_{W-1}}
#pragma unroll
                    for (int s4 = 0; s4 < SG; ++s4) {
                        const f32x4 ex = lds4(&bf.fb[(6 + W) * DK + NQ * g + 4 * s4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) qo[4 * s4 + e] *= ex[e];
                    }
                }
            } else {
                // exact path: scores term by term, e^{b_i - b_j} <= 1; then q e^{b_i} for the inter-chunk read
#pragma unroll
                for (int J = 0; J <= W; ++J)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * J + 4 * g + r;
                        float acc = 0.f;
                        if (j <= qrow) {
                            for (int cc = 0; cc < DK; ++cc)
                                acc += bf.qb[qrow * QS + cc] * bf.kb[j * QS + cc] *
                                       fexp2(bf.gt[cc * CS + qrow] - bf.gt[cc * CS + j]);
                        }
                        pacc[J][r] = acc;
                    }
#pragma unroll
                for (int s = 0; s < NQ; ++s) qo[s] *= fexp2(bf.gt[(NQ * g + s) * CS + qrow]);
            }
            // ---- O^T = S^T Q~^T + V^T P^T per 16-column value tile nt: SG groups from the
            // state copy, then W + 1 from V^T; rows past the chunk's end are dropped
            constexpr int GPN = SG + W + 1;
            constexpr int NGO = NT * GPN;
            auto o_at = [&](int gi) {
                const int nt = gi / GPN, k = gi % GPN;
                return (k < SG) ? lds4(&sm.sc[(16 * nt + l16) * QS + NQ * g + 4 * k])
                                : lds4(&bf.vt[(16 * nt + l16) * CS + 16 * (k - SG) + 4 * g]);
            };
            const auto rso = make_rsrc(oh + t0 * DV * ESZ, (clen * DV - nbase) * ESZ);
            f32x4 ar[RA + 1], o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < RA; ++i) ar[i] = o_at(i);
#pragma unroll
            for (int gi = 0; gi < NGO; ++gi) {
                if (gi + RA < NGO) ar[(gi + RA) % (RA + 1)] = o_at(gi + RA);
                const int nt = gi / GPN, k = gi % GPN, x = gi % (RA + 1);
                if (k == 0) o = f32x4{0.f, 0.f, 0.f, 0.f};
                if (k < SG) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) o = mfma_f32(ar[x][e], qo[4 * k + e], o);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) o = mfma_f32(ar[x][r], pacc[k - SG][r], o);
                }
                if (k == GPN - 1)
                    bstore4<BF>(rso, static_cast<unsigned>((qrow * DV + 16 * nt + 4 * g) * ESZ), o);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // ---- S = diag(e^{b_L}) S + K'^T V for this wave's tiles; lane group g contracts keys 16 g ..
            if (!exact) {
                if constexpr (TN > 0) {
                    // group (t, s4): keys 16 g + 4 s4 .. + 3 of state tile t
                    constexpr int NG = 4 * TN;
                    auto kp_at = [&](int gi) {
                        const int m = (TF + gi / 4) % KT;
                        return lds4(&bf.gt[(16 * m + l16) * CS + 16 * g + 4 * (gi % 4)]);
                    };
                    auto v_at = [&](int gi) {
                        const int n = (TF + gi / 4) / KT;
                        return lds4(&bf.vt[(16 * n + l16) * CS + 16 * g + 4 * (gi % 4)]);
                    };
#pragma unroll
                    for (int t = 0; t < TN; ++t) sacc[t] *= lds4(&bf.bl[16 * ((TF + t) % KT) + 4 * g]);
                    f32x4 xr[RA + 1], yr[RA + 1];
#pragma unroll
                    for (int i = 0; i < RA; ++i) {
                        xr[i] = kp_at(i);
                        yr[i] = v_at(i);
                    }
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi) {
                        if (gi + RA < NG) {
                            xr[(gi + RA) % (RA + 1)] = kp_at(gi + RA);
                            yr[(gi + RA) % (RA + 1)] = v_at(gi + RA);
                        }
                        const int t = gi / 4, x = gi % (RA + 1);
#pragma unroll
                        for (int e = 0; e < 4; ++e) sacc[t] = mfma_f32(xr[x][e], yr[x][e], sacc[t]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < TN; ++t) {
                    const int m = (TF + t) % KT, n = (TF + t) / KT;
                    // exact path: K' = k e^{b_L - b_j} and e^{b_L} from raw k and b^T
                    const int ch = 16 * m + l16;
                    const float bLc = bf.gt[ch * CS + C - 1];
#pragma unroll
                    for (int r = 0; r < 4; ++r) sacc[t][r] *= fexp2(bf.gt[(16 * m + 4 * g + r) * CS + C - 1]);
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const f32x4 vx = lds4(&bf.vt[(16 * n + l16) * CS + 16 * g + 4 * s4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int key = 16 * g + 4 * s4 + e;
                            const float kp = bf.kb[key * QS + ch] * fexp2(bLc - bf.gt[ch * CS + key]);
                            sacc[t] = mfma_f32(kp, vx[e], sacc[t]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);  // one tile's exponentials in flight at a time
                }
            }
        }
    };

    // ---- the walk.  Chunk c uses buffer set (c - c_begin) % NB; its exact-path
    // flag is read once the vote is published and then kept in a register.
    if (c_begin < c_end) load_chunk(c_begin);
    prologue();
    if (c_begin < c_end) vote(c_begin);
    lds_barrier();  // the first vote and the state copy
    if constexpr (!SO && !OW) {
        // this wave's state tiles, from the copy the whole workgroup wrote
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const int m = (TF + t) % KT, n = (TF + t) / KT;
            sacc[t] = lds4(&sm.sc[(16 * n + l16) * QS + 16 * m + 4 * g]);
        }
    }
    bool ex_cur = (c_begin < c_end) && exact_of(c_begin);
    if (c_begin < c_end) {
        fold(sm.op[0], ex_cur);
        load_chunk(c_begin + 1);
        if constexpr (NB == 2) vote(c_begin + 1);
    }
    lds_barrier();  // the first chunk's operands and the second chunk's vote

    auto step = [&](int c, auto xc) {
        constexpr int X = decltype(xc)::value;
        const long long t0 = static_cast<long long>(c) * C;
        const int clen = chunk_len(c);
        if constexpr (NB == 2) {
            // fold the next chunk into the other buffer set while this chunk's products run
            const bool ex_next = (c + 1 < c_end) && exact_of(c + 1);
            if (c + 1 < c_end) fold(sm.op[1 - X], ex_next);
            load_chunk(c + 2);
            products(sm.op[X], t0, clen, ex_cur);
            lds_barrier();     // operands of c + 1 written; every read of c's operands and of the state copy done
#ifdef RET_DEBUG
            lds_poison(&sm.op[X], sizeof(Buf));  // dead until chunk c + 2 is folded into it
#endif
            write_state_copy();
            // The gates of chunk c + 2 were loaded before the products, which
            // have hidden their latency; its flag slot was last read in the
            // previous step, and the next barrier publishes the vote.
            vote(c + 2);
            lds_barrier();
            ex_cur = ex_next;
        } else {
            products(sm.op[0], t0, clen, ex_cur);
            vote(c + 1);       // the gates of chunk c + 1 have arrived by now
            lds_barrier();     // every read of c's operands and of the state copy done
#ifdef RET_DEBUG
            lds_poison(&sm.op[0], sizeof(Buf));  // dead until chunk c + 1 is folded into it
            lds_barrier();
#endif
            write_state_copy();
            const bool ex_next = (c + 1 < c_end) && exact_of(c + 1);
            if (c + 1 < c_end) fold(sm.op[0], ex_next);
            load_chunk(c + 2);
            lds_barrier();
            ex_cur = ex_next;
        }
    };
    for (int c = c_begin; c < c_end; c += NB) {
        step(c, std::integral_constant<int, 0>{});
        if constexpr (NB == 2) {
            if (c + 1 < c_end) step(c + 1, std::integral_constant<int, 1>{});
        }
    }

    if constexpr (SO) {
        // this segment's contribution (its end state from zero) and log-gate totals
        float* out = a.ws + (static_cast<long long>(bh) * (a.G - 1) + seg) * slot;
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const int m = (TF + t) % KT, n = (TF + t) / KT;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[(16 * m + 4 * g + r) * DV + nbase + 16 * n + l16] = sacc[t][r];
        }
        if constexpr (!QW) {
            if (nbase == 0 && tg == 0) {
#pragma unroll
                for (int u = 0; u < CPT; ++u) *reinterpret_cast<f32x4*>(out + DK * DV + 16 * W + 4 * cg + 64 * u) = ltot[u];
            }
        }
    } else if constexpr (!OW) {
        if (a.final_state && seg == a.G - 1) {
            float* fs = a.final_state + static_cast<long long>(bh) * DK * DV + nbase;
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                const int m = (TF + t) % KT, n = (TF + t) / KT;
#pragma unroll
                for (int r = 0; r < 4; ++r) fs[(16 * m + 4 * g + r) * DV + 16 * n + l16] = sacc[t][r];
            }
        }
    }
}

template <bool BF, int DK, int NT, bool SO>
__global__ void __launch_bounds__(kThreads, 1) gla_kernel(const GlaArgs a) {
    __shared__ Smem<DK, NT> sm;
    const int nseg = SO ? a.G - 1 : a.G;
    const int bhs = blockIdx.x / a.nslices;
    const int bh = bhs / nseg, seg = bhs % nseg;
    const int nbase = (blockIdx.x % a.nslices) * Cfg<DK, NT>::DVS;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    switch (wave) {
        case 0: body<BF, DK, NT, 0, SO>(a, sm, bh, seg, nbase); break;
        case 1: body<BF, DK, NT, 1, SO>(a, sm, bh, seg, nbase); break;
        case 2: body<BF, DK, NT, 2, SO>(a, sm, bh, seg, nbase); break;
        case 3: body<BF, DK, NT, 3, SO>(a, sm, bh, seg, nbase); break;
        case 4: body<BF, DK, NT, 4, SO>(a, sm, bh, seg, nbase); break;
        case 5: body<BF, DK, NT, 5, SO>(a, sm, bh, seg, nbase); break;
        case 6: body<BF, DK, NT, 6, SO>(a, sm, bh, seg, nbase); break;
        default: body<BF, DK, NT, 7, SO>(a, sm, bh, seg, nbase); break;
    }
}

template <bool BF, int DK, int NT>
hipError_t launch_t(const GlaArgs& a, hipStream_t stream) {
    static_assert(fits<DK, NT>(), "LDS");
    const long long groups = static_cast<long long>(a.B) * a.H * a.nslices * a.G;
    if (groups <= 0) return hipSuccess;
    if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.G > 1) {
        const long long sgroups = static_cast<long long>(a.B) * a.H * a.nslices * (a.G - 1);
        hipLaunchKernelGGL((gla_kernel<BF, DK, NT, true>), dim3(static_cast<unsigned>(sgroups)), dim3(kThreads), 0,
                           stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gla_kernel<BF, DK, NT, false>), dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace
}  // namespace gla

// Value slices of 64 columns: the whole value width when dv = 64, two slices
// (each forming Q K^T) when dv = 128.
int gla_choose_nt(long long bh, int dk, int dv) {
    (void)bh;
    (void)dk;
    return dv >= 64 ? 4 : dv / 16;
}

int gla_target_groups(int dk, int nt) {
    (void)dk;
    (void)nt;
    return 256;  // one 8-wave workgroup per CU
}

hipError_t launch_gla(const GlaArgs& a, bool bf16, int dk, int nt, hipStream_t stream) {
    if (nt != 4) return hipErrorInvalidValue;
    if (dk == 64) return bf16 ? gla::launch_t<true, 64, 4>(a, stream) : gla::launch_t<false, 64, 4>(a, stream);
    if (dk == 128) return bf16 ? gla::launch_t<true, 128, 4>(a, stream) : gla::launch_t<false, 128, 4>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace ret
