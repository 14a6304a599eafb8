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
// Fast path.  One pre-scaled key array serves every product:
// K^[j][c] = k_j[c] e^{b_{e_J}[c] - b_j[c]} (<= |k|).  Scores of key tile J
// <= I take Q operands q_i e^{b_i - b_{e_I}} (>= 1 in size, bounded by
// e^{span of one tile}) times e^{b_{e_I} - b_{e_J}} (<= 1); the diagonal tile
// is that product masked.  The state update takes K^ times e^{b_last -
// b_{e_J}} (<= 1).  It is used when every channel's log-gate sum over the
// chunk stays above -80, so that no factor can overflow; a chunk with
// stronger gates takes the exact path above (diagonal tiles summed term by
// term, every exponent formed on the spot).
//
// Segments.  Each (b, h) sequence is cut into G segments of whole chunks.  A
// state-only pass (SO) walks every segment but the last and writes its
// contribution dS_j (the state it would end with from zero) and its per-channel
// log-gate total L_j; the walk of segment g then starts from
//   S_in(g) = sum_{j<g} diag(exp(L_{j+1} + ... + L_{g-1})) dS_j,
// all exponents <= 0.
//
// Mapping.  One workgroup (4 waves) per (b, h, segment, slice of 16 NT value
// columns) walks the segment's chunks of 64 tokens; wave W owns query tile W
// and state tiles {W, W + 4, ...} of the slice.  The chunk's q, k, cumulative
// gates and the value slice are staged in LDS (padded fp32 rows); S^T is
// copied to LDS for the next chunk's inter-chunk product.
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
    int unsafe[4];                             // per wave: this chunk's gates are too strong for the fast path
};

template <int DK, int NT>
constexpr bool fits() { return sizeof(Smem<DK, NT>) <= 160 * 1024; }

template <int DK, int NT, int W, bool SO>
__device__ __forceinline__ void body(const GlaArgs& a, Smem<DK, NT>& sm, int bh, int seg, int nbase) {
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
    const long long slot = static_cast<long long>(DK) * DV + DK;  // workspace floats per (b, h, segment)
    if (!SO && seg > 0) {
        // S_in = sum_{j<seg} diag(exp(L_{j+1} + ... + L_{seg-1})) dS_j
        const float* wsb = a.ws + static_cast<long long>(bh) * (a.G - 1) * slot;
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = W + 4 * m, nt = qt / KT, kt = qt % KT, ch = 16 * kt + l16;
            float dsum = 0.f;
            for (int j = seg - 1; j >= 0; --j) {
                const float* sj = wsb + j * slot;
                sacc[m] += __expf(dsum) * *reinterpret_cast<const f32x4*>(sj + ch * DV + nbase + 16 * nt + 4 * g);
                dsum += sj[DK * DV + ch];
            }
        }
    }
#pragma unroll
    for (int m = 0; m < SPW; ++m) {  // state copy for the first chunk (ordered by the loop's first barrier)
        const int qt = W + 4 * m, nt = qt / KT, kt = qt % KT;
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.st[(16 * nt + 4 * g + r) * KSTR + 16 * kt + l16] = sacc[m][r];
    }
    // Staging.  q and the value slice load as 16-byte rows; keys and log-gates
    // in a column layout: lane (c16, rq) of wave W holds key channels
    // 16 W + c16 + 64 u (u < DK / 64) of rows 16 rq .. 16 rq + 15, i.e. one
    // 16-token tile per channel, so the running gate sums, the tile totals and
    // the pre-scaled keys K^ come out of registers.  The next chunk's loads
    // are issued before the current chunk's products.
    constexpr int NU = C * DK / 4 / kThreads;
    constexpr int NV = (C * DVS / 4 + kThreads - 1) / kThreads;
    constexpr int CPW = DK / 64;
    static_assert(NU * kThreads * 4 == C * DK, "q staging split");
    const int c16 = l & 15, rq = l >> 4;
    f32x4 pq[SO ? 1 : NU], pv[NV];
    float pk[CPW][16], pg[CPW][16];
    float ltot[CPW];  // state-only pass: log-gate totals of this lane's channels over the segment
#pragma unroll
    for (int u = 0; u < CPW; ++u) ltot[u] = 0.f;

    const int nch = (T + C - 1) / C;
    const int c_begin = seg * a.cps;
    const int c_end = (c_begin + a.cps < nch) ? c_begin + a.cps : nch;
    auto chunk_len = [&](int c) {
        const long long t0 = static_cast<long long>(c) * C;
        return (T - t0 < C) ? static_cast<int>(T - t0) : C;
    };
    // rows past the end read row 0 of the chunk (always valid); they are zeroed when stored
    auto load_qv = [&](int c) {
        const long long t0 = static_cast<long long>(c) * C;
        const int clen = chunk_len(c);
        if constexpr (!SO) {
#pragma unroll
            for (int m = 0; m < NU; ++m) {
                const int u = tid + m * kThreads, r = u / (DK / 4), c4 = 4 * (u % (DK / 4));
                pq[m] = *reinterpret_cast<const f32x4*>(qh + (t0 + (r < clen ? r : 0)) * DK + c4);
            }
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int u = tid + m * kThreads, r = u / (DVS / 4), c4 = 4 * (u % (DVS / 4));
            if (u < C * DVS / 4) pv[m] = *reinterpret_cast<const f32x4*>(vh + (t0 + (r < clen ? r : 0)) * DV + c4);
        }
    };
    auto load_kg = [&](int c) {
        const long long t0 = static_cast<long long>(c) * C;
        const int clen = chunk_len(c);
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
            const int ch = 16 * W + c16 + 64 * u;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * rq + i;
                const long long o = (t0 + (r < clen ? r : 0)) * DK + ch;
                pk[u][i] = kh[o];
                pg[u][i] = gh[o];
            }
        }
    };
    // With dk = 128 the registers do not hold the next chunk's keys and gates
    // beside the products, so each chunk loads its own at the top of its step.
    constexpr bool KG_EARLY = DK == 64;
    if (c_begin < c_end) {
        load_qv(c_begin);
        if constexpr (KG_EARLY) load_kg(c_begin);
    }

    for (int c = c_begin; c < c_end; ++c) {
        const long long t0 = static_cast<long long>(c) * C;
        const int clen = chunk_len(c);
        if constexpr (!KG_EARLY) load_kg(c);
        __syncthreads();  // the previous chunk's reads of q, k, b, v and the flags are done

        // ---- store the chunk (rows past the end: zeros, log-gate 0)
        {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            if constexpr (!SO) {
#pragma unroll
                for (int m = 0; m < NU; ++m) {
                    const int u = tid + m * kThreads, r = u / (DK / 4), c4 = 4 * (u % (DK / 4));
                    *reinterpret_cast<f32x4*>(&sm.q[r * KSTR + c4]) = (r < clen) ? pq[m] : zero;
                }
            }
#pragma unroll
            for (int m = 0; m < NV; ++m) {
                const int u = tid + m * kThreads, r = u / (DVS / 4), c4 = 4 * (u % (DVS / 4));
                if (u < C * DVS / 4) *reinterpret_cast<f32x4*>(&sm.v[r * VSTR + c4]) = (r < clen) ? pv[m] : zero;
            }
            int bad = 0;
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                const int ch = 16 * W + c16 + 64 * u;
                float cum[16];
                float run = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    run += (16 * rq + i < clen) ? pg[u][i] : 0.f;
                    cum[i] = run;
                }
                // tile totals of the four row quarters of this channel (lanes c16 + 16 q)
                const float t0s = __shfl(run, c16), t1s = __shfl(run, c16 + 16);
                const float t2s = __shfl(run, c16 + 32), t3s = __shfl(run, c16 + 48);
                const float off = (rq > 0 ? t0s : 0.f) + (rq > 1 ? t1s : 0.f) + (rq > 2 ? t2s : 0.f);
                const float tot = t0s + t1s + t2s + t3s;
                if (!(tot >= -80.f)) bad = 1;
                ltot[u] += tot;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = 16 * rq + i;
                    sm.b[r * KSTR + ch] = off + cum[i];
                    // K^ = k e^{b_{e_J} - b_j}: the tile's total minus the running sum
                    sm.k[r * KSTR + ch] = ((r < clen) ? pk[u][i] : 0.f) * __expf(run - cum[i]);
                }
            }
            const bool wbad = __any(bad);
            if (l == 0) sm.unsafe[W] = wbad ? 1 : 0;
        }
        __syncthreads();
        const bool unsafe = (sm.unsafe[0] | sm.unsafe[1] | sm.unsafe[2] | sm.unsafe[3]) != 0;
        if (unsafe) {
            // the exact path works from the raw keys
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                const int ch = 16 * W + c16 + 64 * u;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = 16 * rq + i;
                    sm.k[r * KSTR + ch] = (r < clen) ? pk[u][i] : 0.f;
                }
            }
            __syncthreads();
        }
        if (c + 1 < c_end) {
            load_qv(c + 1);
            if constexpr (KG_EARLY) load_kg(c + 1);
        }

        const int qi = 16 * I + l16;  // this lane's query row
        const int last = clen - 1;
        if (!unsafe) {
            // ---- fast path (see the header): Q factors in registers, K^ in place of k
            constexpr int NQ = DK / 4;
            const int eI = 16 * I + 15;
            float qd[NQ], qx[NQ];  // q_i e^{b_i - b_{e_I}} and q_i e^{b_i} for channels 4s + g
#pragma unroll
            for (int s = 0; s < (SO ? 0 : NQ); ++s) {
                const int ch = 4 * s + g;
                const float qv = sm.q[qi * KSTR + ch], bq = sm.b[qi * KSTR + ch];
                qd[s] = qv * __expf(bq - sm.b[eI * KSTR + ch]);
                qx[s] = qv * __expf(bq);
            }

            f32x4 pacc[I + 1];
#pragma unroll
            for (int J = 0; J <= (SO ? -1 : I); ++J) {
                pacc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int eJ = 16 * J + 15, kj = 16 * J + l16;
#pragma unroll 4
                for (int s = 0; s < NQ; ++s) {
                    const int ch = 4 * s + g;
                    const float f = (J == I) ? 1.f : __expf(sm.b[eI * KSTR + ch] - sm.b[eJ * KSTR + ch]);
                    pacc[J] = mfma_f32(sm.k[kj * KSTR + ch], qd[s] * f, pacc[J]);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)  // causal mask of the diagonal tile
                if (16 * I + 4 * g + r > qi) pacc[I][r] = 0.f;

#pragma unroll
            for (int nt = 0; nt < (SO ? 0 : NT); ++nt) {
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
                for (int s = 0; s < NQ; ++s) o = mfma_f32(sm.st[(16 * nt + l16) * KSTR + 4 * s + g], qx[s], o);
#pragma unroll
                for (int J = 0; J <= I; ++J)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        o = mfma_f32(sm.v[(16 * J + 4 * g + r) * VSTR + 16 * nt + l16], pacc[J][r], o);
                if (qi < clen) *reinterpret_cast<f32x4*>(oh + (t0 + qi) * DV + 16 * nt + 4 * g) = o;
            }

#pragma unroll
            for (int m = 0; m < SPW; ++m) {
                const int qt = W + 4 * m, nt = qt / KT, kt = qt % KT;
                const int ch = 16 * kt + l16;
                const float bl = sm.b[last * KSTR + ch];
                sacc[m] *= __expf(bl);
#pragma unroll
                for (int J = 0; J < C / 16; ++J) {
                    const float f = __expf(bl - sm.b[(16 * J + 15) * KSTR + ch]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * J + 4 * g + r;
                        sacc[m] = mfma_f32(sm.v[j * VSTR + 16 * nt + l16], sm.k[j * KSTR + ch] * f, sacc[m]);
                    }
                }
            }
            __syncthreads();  // every wave is done reading the old state copy
#pragma unroll
            for (int m = 0; m < SPW; ++m) {
                const int qt = W + 4 * m, nt = qt / KT, kt = qt % KT;
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.st[(16 * nt + 4 * g + r) * KSTR + 16 * kt + l16] = sacc[m][r];
            }
            continue;
        }

        // ---- exact path for chunks with strong gates
        if constexpr (!SO) {
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
        }  // !SO

        // ---- S = diag(e^{b_last}) S + sum_j diag(e^{b_last - b_j}) k_j v_j^T
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

    if constexpr (SO) {
        // this segment's contribution (its end state from zero) and log-gate totals
        float* out = a.ws + (static_cast<long long>(bh) * (a.G - 1) + seg) * slot;
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = W + 4 * m, nt = qt / KT, kt = qt % KT;
            *reinterpret_cast<f32x4*>(out + (16 * kt + l16) * DV + nbase + 16 * nt + 4 * g) = sacc[m];
        }
        if (nbase == 0 && rq == 0) {
#pragma unroll
            for (int u = 0; u < CPW; ++u) out[DK * DV + 16 * W + c16 + 64 * u] = ltot[u];
        }
        return;
    }
    if (a.final_state && seg == a.G - 1) {
        float* fs = a.final_state + static_cast<long long>(bh) * DK * DV + nbase;
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int qt = W + 4 * m, nt = qt / KT, kt = qt % KT;
            *reinterpret_cast<f32x4*>(fs + (16 * kt + l16) * DV + 16 * nt + 4 * g) = sacc[m];
        }
    }
}

// SO: the state-only pass over segments 0 .. G-2.  The 32-column slices at
// dk = 64 are held to 256 registers (they need 254), so that two workgroups
// share a CU and hide each other's latencies; the other variants use more.
template <int DK, int NT>
constexpr int gla_min_blocks() { return (DK == 64 && NT == 2) ? 2 : 1; }

template <int DK, int NT, bool SO>
__global__ void __launch_bounds__(kThreads, (gla_min_blocks<DK, NT>())) gla_kernel(const GlaArgs a) {
    __shared__ Smem<DK, NT> sm;
    const int nseg = SO ? a.G - 1 : a.G;
    const int bhs = blockIdx.x / a.nslices;
    const int bh = bhs / nseg, seg = bhs % nseg;
    const int nbase = (blockIdx.x % a.nslices) * Cfg<DK, NT>::DVS;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    switch (wave) {
        case 0: body<DK, NT, 0, SO>(a, sm, bh, seg, nbase); break;
        case 1: body<DK, NT, 1, SO>(a, sm, bh, seg, nbase); break;
        case 2: body<DK, NT, 2, SO>(a, sm, bh, seg, nbase); break;
        default: body<DK, NT, 3, SO>(a, sm, bh, seg, nbase); break;
    }
}

template <int DK, int NT>
hipError_t launch_t(const GlaArgs& a, hipStream_t stream) {
    if constexpr (!fits<DK, NT>()) {
        return hipErrorInvalidConfiguration;
    } else {
        const long long groups = static_cast<long long>(a.B) * a.H * a.nslices * a.G;
        if (groups <= 0) return hipSuccess;
        if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
        if (a.G > 1) {
            const long long sgroups = static_cast<long long>(a.B) * a.H * a.nslices * (a.G - 1);
            hipLaunchKernelGGL((gla_kernel<DK, NT, true>), dim3(static_cast<unsigned>(sgroups)), dim3(kThreads), 0,
                               stream, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL((gla_kernel<DK, NT, false>), dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0, stream,
                           a);
        return hipGetLastError();
    }
}

}  // namespace
}  // namespace gla

int gla_choose_nt(long long bh, int dk, int dv) {
    // dk = dv = 64: 32-column slices, two workgroups per CU (measured on [4, 8, 2048, 64]: 65 us against
    // 69 us for 64-column slices at one per CU, bit-identical results); otherwise the widest slice
    // that fits, 64 columns at most (the segments supply the parallelism)
    (void)bh;
    if (dk == 64 && dv == 64) return 2;
    return dv >= 64 ? 4 : dv / 16;
}

int gla_target_groups(int dk, int nt) { return (dk == 64 && nt == 2) ? 512 : 256; }

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
