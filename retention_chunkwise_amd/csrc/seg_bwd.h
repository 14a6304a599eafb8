// seg_bwd.h -- the key and value gradients of chunkwise retention from one
// walk over the time-reversed sequence (bf16 in, fp32 accumulate, gfx950).
//
// What is computed.  The gradients of retention are cumulative sums, the
// keys' and values' running backwards in time ("Linear attention",
// "Decoding, training, and what each costs"; the operator of "RetNet",
// single-head definition).  With the reversed state
//   U_s = sum_{t >= s} gamma^(t-s) q_t dout_t^T        (dk x dv)
// the gradients are
//   dv_s = U_s^T k_s = sum_{t>=s} gamma^(t-s) (k_s . q_t) dout_t
//   dk_s = U_s v_s   = sum_{t>=s} gamma^(t-s) (v_s . dout_t) q_t
// Over the time-reversed sequence both are causal chunkwise forwards that
// share one state: dv is the forward of (queries k, keys q, values dout) and
// dk that of (queries v, keys dout, values q), whose state is U^T.  One walk
// reads q, k, v and dout once and writes dk and dv once, where two separate
// walks read six tensors.
//
// Chunk form (64-token chunks, local indices i, j in reversed time, U the
// state after the chunk's later tokens, i.e. before it in the walk):
//   A_ij = gamma^(i-j) (k_i . q_j),  B_ij = gamma^(i-j) (v_i . dout_j)   (j <= i)
//   dv_i = sum_j A_ij dout_j + gamma^(i+1) U^T k_i
//   dk_i = sum_j B_ij q_j    + gamma^(i+1) U v_i
//   U   <- gamma^c U + sum_j gamma^(c-1-j) q_j dout_j^T
//
// Layout and roles follow the forward segment walk (seg_kernel.h): the
// sequence is cut into segments (the reversed-time state kernel sums their
// contributions), q and dout go HBM -> LDS by DMA into double-buffered
// swizzled tiles, k and v go into the O-waves' registers, all one chunk
// ahead.  O-wave P owns query tile P of the chunk:
//   A^T = Q_tile k^T, B^T = Dout_tile v^T      (row reads of the q / dout tiles)
//   dv^T = xi U^T k^T + Dout^T A^T             (U^T copy rows; dout transpose reads)
//   dk^T = xi U v^T   + Q^T B^T                (U^T copy and q transpose reads)
// The S-waves carry U in fp32 registers and refresh the bf16 U^T copy after
// each chunk, exactly as the forward walk carries its state.  The U^T copy
// keeps its rows (value columns) in the forward's permuted order, which both
// the row reads (dv) and the transpose reads (dk: rows are the contraction
// index there) take as they are: a transpose read of rows 32 b + slot_key(g,
// e) of that order meets value channel 32 b + 8 g + e, the channel a plain
// 16-byte load of v puts in the same operand slot.
#pragma once

#include "seg_kernel.h"

namespace ret {
namespace seg {

template <int DK, int DV, int P, bool OW>
__device__ __forceinline__ void bwd_kv_body(const SegArgs& a, const STiles& tl, int bh, int seg, float lg) {
    constexpr int C = 64;
    using Cf = SCfg<C, DK, DV, kModeRet>;
    constexpr int NI = Cf::NI, NB = Cf::NB, NVT = Cf::NVT, SKT = Cf::SKT;
    constexpr int KRU = Cf::KRU, VRU = Cf::VRU, KIW = Cf::KIW, VIW = Cf::VIW;
    constexpr int KRB = KRU * 16, VRB = VRU * 16;
    constexpr int QFK = DK / 32, QFV = DV / 32;  // operand blocks of k (and q) rows, of v (and dout) rows
    constexpr int NPV = DV / 32, NPK = DK / 32;  // output tile pairs of dv, of dk
    constexpr int IT = P;                        // this O-wave's query tile
    // vector-memory ops a thread issues after a chunk's loads: its output stores
    constexpr int STORES = OW ? NPV + NPK : 0;
    static_assert(NI == 4, "64-token chunks");

    const int w = P + (OW ? 0 : 4);
    const int l = threadIdx.x & 63, l16 = l & 15, g = l >> 4, lq = l16 >> 2, lr = l16 & 3;
    const int T = a.T;
    const unsigned short* kqh = static_cast<const unsigned short*>(a.q) + static_cast<long long>(bh) * T * DK;
    const unsigned short* vqh = static_cast<const unsigned short*>(a.q2) + static_cast<long long>(bh) * T * DV;
    const unsigned short* qh = static_cast<const unsigned short*>(a.k) + static_cast<long long>(bh) * T * DK;
    const unsigned short* dh = static_cast<const unsigned short*>(a.v) + static_cast<long long>(bh) * T * DV;
    unsigned short* dvh = static_cast<unsigned short*>(a.out) + static_cast<long long>(bh) * T * DV;
    unsigned short* dkh = static_cast<unsigned short*>(a.out2) + static_cast<long long>(bh) * T * DK;
    const LaneOff lk0 = lane_offsets<KRU>(l), lv0 = lane_offsets<VRU>(l);
    // O-wave transpose reads in the permuted output-column order (as the
    // forward's value reads): lane L reads row R0 + 4g + L/4, unit 4a + L%4,
    // half b -- of the dout tile (dv), and of the q tile and the U^T copy (dk)
    const int rowv0 = (4 * g + lq) * VRB, uov0 = (lr ^ swz_mask<VRU>(4 * g + lq)) << 4;
    const int rowk0 = (4 * g + lq) * KRB, uok0 = (lr ^ swz_mask<KRU>(4 * g + lq)) << 4;

    const int nch = (T + C - 1) / C;
    const int c_begin = seg * a.cps;
    const int c_end = (c_begin + a.cps < nch) ? c_begin + a.cps : nch;

    // ---- decay constants (as the forward walk): score (key 16 jt + 4g + r,
    // query 16 IT + l16) decays by gamma^(16 d + l16 - 4g - r), d = IT - jt
    float f0[4], f1_0[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = l16 - 4 * g - r;
        f0[r] = (e < 0) ? 0.f : ex2(static_cast<float>(e) * lg);
        f1_0[r] = ex2(static_cast<float>(16 + e) * lg);
    }
    float gd[IT + 1];
    gd[0] = 1.f;
#pragma unroll
    for (int d = 1; d <= IT; ++d) gd[d] = uni(ex2(static_cast<float>(16 * (d - 1)) * lg));
    const float xi = ex2(static_cast<float>(16 * IT + l16 + 1) * lg);  // gamma^(i+1)
    float zb0[8];  // gamma^(31 - key) for this lane's k-slots; zeta = zb * bj for a full chunk
#pragma unroll
    for (int e = 0; e < 8; ++e) zb0[e] = ex2(static_cast<float>(31 - slot_key(g, e)) * lg);
    float bj[NB];
#pragma unroll
    for (int js = 0; js < NB; ++js) bj[js] = uni(ex2(static_cast<float>(32 * (NB - 1 - js)) * lg));
    const float gC = uni(ex2(static_cast<float>(C) * lg));

    // ---- S-waves: U entering the segment, from the state kernel's slots
    f32x4 sacc[OW ? 1 : SKT][OW ? 1 : NVT];
    if constexpr (!OW) {
#pragma unroll
        for (int mi = 0; mi < SKT; ++mi)
#pragma unroll
            for (int n = 0; n < NVT; ++n) sacc[mi][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (seg > 0) {
            float zacc[SKT];  // unused: no normaliser travels with U
            sum_segment_states<C, DK, DV, kModeRet, P>(a, bh, seg, lg, false, sacc, zacc);
        }
    }

    // bf16 copy of U^T for the O-waves: the lane's 4 values of tile (m, n) are 4
    // consecutive dk of value column 16n + l16
    auto write_state_copy = [&]() {
        if constexpr (!OW) {
            char* sb = reinterpret_cast<char*>(tl.s);
#pragma unroll
            for (int mi = 0; mi < SKT; ++mi) {
                const int m = SKT * P + mi;
#pragma unroll
                for (int n = 0; n < NVT; ++n)
                    *reinterpret_cast<u16x4*>(sb + swz_byte<KRU>(perm_row(16 * n + l16), 2 * m + (g >> 1)) +
                                              (g & 1) * 8) = cvt4_bf16(sacc[mi][n]);
            }
        }
    };

    // Reversed time: chunk row r of the chunk at reversed token t0 is memory
    // row T - 1 - (t0 + r); the chunk's memory rows start at T - t0 - clen.
    const int koffr = dma_offset_rev<KRU>(w, l), voffr = dma_offset_rev<VRU>(w, l);
    auto mem_row0 = [&](long long t0, int cl) -> long long { return cl ? T - t0 - cl : 0; };
    auto chunk_len = [&](int c) {
        const long long t0 = static_cast<long long>(c) * C;
        return (T - t0 < C) ? static_cast<int>(T - t0) : C;
    };
    bf16x8 kf[OW ? 2 : 1][QFK];  // O-waves: k rows (queries of A), double-buffered
    bf16x8 vf[OW ? 2 : 1][QFV];  // O-waves: v rows (queries of B)
    // Issued unconditionally (a chunk past the segment gets a zero-length range).
    auto load_chunk = [&](int c, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const long long t0 = static_cast<long long>(c) * C;
        const int cl = (c < c_end) ? chunk_len(c) : 0;
        const long long mrow = mem_row0(t0, cl);
        const u32x4 wq = rsrc_words(qh + mrow * DK, cl * DK * 2);
        const u32x4 wd = rsrc_words(dh + mrow * DV, cl * DV * 2);
        const unsigned qbase = __builtin_amdgcn_readfirstlane(lds_addr_of(tl.k[buf]));
        const unsigned dbase = __builtin_amdgcn_readfirstlane(lds_addr_of(tl.v[buf]));
#pragma unroll
        for (int m = 0; m < KIW; ++m)
            dma16(wq, qbase + (w + 8 * m) * 1024, static_cast<unsigned>((cl - 1) * DK * 2 + koffr - 8192 * m));
#pragma unroll
        for (int m = 0; m < VIW; ++m)
            dma16(wd, dbase + (w + 8 * m) * 1024, static_cast<unsigned>((cl - 1) * DV * 2 + voffr - 8192 * m));
        if constexpr (OW) {
            const auto rk = make_rsrc(kqh + mrow * DK, cl * DK * 2);
            const auto rv = make_rsrc(vqh + mrow * DV, cl * DV * 2);
            const int row = cl - 1 - (16 * IT + l16);  // negative past a short chunk: read as zeros
#pragma unroll
            for (int ks = 0; ks < QFK; ++ks)
                kf[buf][ks] = __builtin_bit_cast(bf16x8, bload16(rk, static_cast<unsigned>((row * DK + 32 * ks + 8 * g) * 2)));
#pragma unroll
            for (int ks = 0; ks < QFV; ++ks)
                vf[buf][ks] = __builtin_bit_cast(bf16x8, bload16(rv, static_cast<unsigned>((row * DV + 32 * ks + 8 * g) * 2)));
        }
    };

    // decay and mask of one score set, as bf16 operands (two key tiles each)
    auto weigh = [&](const f32x4 (&pacc)[NI], const float (&f1)[4], bf16x8 (&pb)[NB]) {
#pragma unroll
        for (int js = 0; js < NB; ++js)
            if (2 * js <= IT) {
                f32x4 lo = pacc[2 * js], hi = f32x4{0.f, 0.f, 0.f, 0.f};
                const int d0 = IT - 2 * js;
#pragma unroll
                for (int r = 0; r < 4; ++r) lo[r] *= (d0 == 0) ? f0[r] : gd[d0] * f1[r];
                if (2 * js + 1 <= IT) {
                    hi = pacc[2 * js + 1];
                    const int d1 = d0 - 1;
#pragma unroll
                    for (int r = 0; r < 4; ++r) hi[r] *= (d1 == 0) ? f0[r] : gd[d1] * f1[r];
                }
                pb[js] = cat_bf16(cvt4_bf16(lo), cvt4_bf16(hi));
            }
    };

    auto step = [&](int c, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        const long long t0 = static_cast<long long>(c) * C;
        const int clen = (T - t0 < C) ? static_cast<int>(T - t0) : C;
        const bool tail = clen < C;  // uniform; only the last chunk of the walk

        // This chunk's loads were issued during the previous step; the only
        // vector-memory ops issued after them are the previous step's output
        // stores, and vector-memory ops complete in issue order.
        if (c == c_begin) wait_vmcnt<0>();
        else wait_vmcnt<STORES>();
        lds_barrier();  // chunk in LDS everywhere, U^T copy written
        load_chunk(c + 1, std::integral_constant<int, 1 - B>{});

        const unsigned short* qb = tl.k[B];  // q tile: keys of A, values of dk
        const unsigned short* db = tl.v[B];  // dout tile: keys of B, values of dv

        if constexpr (OW) {
            LaneOff lk = lk0, lv = lv0;
            opaque<QFK>(lk);
            opaque<QFV>(lv);
            float f1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                f1[r] = f1_0[r];
                opaque(f1[r]);
            }
            // ---- A^T = Q_tile k^T and B^T = Dout_tile v^T for key tiles jt <= IT
            f32x4 pa[NI], pbs[NI];
#pragma unroll
            for (int jt = 0; jt < NI; ++jt) {
                pa[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                pbs[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < QFK; ++ks) {
                bf16x8 ka[IT + 1];
#pragma unroll
                for (int jt = 0; jt <= IT; ++jt) ka[jt] = b128_at(qb, 16 * jt * KRB + lk.opr[ks]);
#pragma unroll
                for (int jt = 0; jt <= IT; ++jt) pa[jt] = mfma_bf16(ka[jt], kf[B][ks], pa[jt]);
            }
#pragma unroll
            for (int ks = 0; ks < QFV; ++ks) {
                bf16x8 da[IT + 1];
#pragma unroll
                for (int jt = 0; jt <= IT; ++jt) da[jt] = b128_at(db, 16 * jt * VRB + lv.opr[ks]);
#pragma unroll
                for (int jt = 0; jt <= IT; ++jt) pbs[jt] = mfma_bf16(da[jt], vf[B][ks], pbs[jt]);
            }
            bf16x8 wa[NB], wb[NB];
            weigh(pa, f1, wa);
            weigh(pbs, f1, wb);

            int rowv = rowv0, uov = uov0, rowk = rowk0, uok = uok0;
            opaque(rowv);
            opaque(uov);
            opaque(rowk);
            opaque(uok);
            const int row = clen - 1 - (16 * IT + l16);  // rows past the end are dropped by the resource
            const long long mrow = mem_row0(t0, clen);
            // ---- dv^T = xi U^T k^T + Dout^T A^T, per pair of value tiles
            const auto rdv = make_rsrc(dvh + mrow * DV, clen * DV * 2);
#pragma unroll
            for (int pp = 0; pp < NPV; ++pp) {
                const int ua = uov ^ (pp << 6);
                f32x4 o[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int n = 2 * pp + b;
                    o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < QFK; ++ks) o[b] = mfma_bf16(b128_at(tl.s, 16 * n * KRB + lk.opr[ks]), kf[B][ks], o[b]);
                    o[b] *= xi;
#pragma unroll
                    for (int js = 0; 2 * js <= IT; ++js) {
                        const bf16x8 x = cat_bf16(tr_at(db, 32 * js * VRB + rowv + ua + 8 * b),
                                                  tr_at(db, (32 * js + 16) * VRB + rowv + ua + 8 * b));
                        o[b] = mfma_bf16(x, wa[js], o[b]);
                    }
                }
                bstore16_bf(rdv, static_cast<unsigned>((row * DV + 32 * pp + 8 * g) * 2),
                            cat_bf16(cvt4_bf16(o[0]), cvt4_bf16(o[1])));
            }
            // ---- dk^T = xi U v^T + Q^T B^T, per pair of key-channel tiles; U comes
            // from transpose reads of the U^T copy (rows: value channels)
            const auto rdk = make_rsrc(dkh + mrow * DK, clen * DK * 2);
#pragma unroll
            for (int pp = 0; pp < NPK; ++pp) {
                const int ua = uok ^ (pp << 6);
                f32x4 o[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < QFV; ++kb) {
                        const bf16x8 x = cat_bf16(tr_at(tl.s, 32 * kb * KRB + rowk + ua + 8 * b),
                                                  tr_at(tl.s, (32 * kb + 16) * KRB + rowk + ua + 8 * b));
                        o[b] = mfma_bf16(x, vf[B][kb], o[b]);
                    }
                    o[b] *= xi;
#pragma unroll
                    for (int js = 0; 2 * js <= IT; ++js) {
                        const bf16x8 x = cat_bf16(tr_at(qb, 32 * js * KRB + rowk + ua + 8 * b),
                                                  tr_at(qb, (32 * js + 16) * KRB + rowk + ua + 8 * b));
                        o[b] = mfma_bf16(x, wb[js], o[b]);
                    }
                }
                bstore16_bf(rdk, static_cast<unsigned>((row * DK + 32 * pp + 8 * g) * 2),
                            cat_bf16(cvt4_bf16(o[0]), cvt4_bf16(o[1])));
            }
            lds_barrier();  // every O-wave is done reading the old U^T copy
        } else {
            LaneOff lk = lk0, lv = lv0;
            opaque<0>(lk);
            opaque<0>(lv);
            float zb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                zb[e] = zb0[e];
                opaque(zb[e]);
            }
            // ---- zeta-scaled q^T operands of the state update
            bf16x8 kz[SKT][NB];
#pragma unroll
            for (int js = 0; js < NB; ++js) {
                float z[8];
                if (!tail) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) z[e] = zb[e] * bj[js];
                } else {
                    // gamma^(clen - 1 - key) for keys inside the chunk, 0 past its end
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int ex = clen - 1 - 32 * js - slot_key(g, e);
                        z[e] = (ex < 0) ? 0.f : ex2(static_cast<float>(ex) * lg);
                    }
                }
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) kz[mi][js] = kt_scaled<KRU>(qb, js, ((SKT * P + mi) << 5) ^ lk.z16, lk, z);
            }
            // ---- U = gamma^c U + (zeta q)^T dout
            const float gc = tail ? uni(ex2(static_cast<float>(clen) * lg)) : gC;
#pragma unroll
            for (int n = 0; n < NVT; ++n) {
                const int xt = (n << 5) ^ lv.z16;
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) sacc[mi][n] *= gc;
#pragma unroll
                for (int js = 0; js < NB; ++js) {
                    const bf16x8 x = tr_block<VRU>(db, 32 * js, xt, lv);
#pragma unroll
                    for (int mi = 0; mi < SKT; ++mi) sacc[mi][n] = mfma_bf16(kz[mi][js], x, sacc[mi][n]);
                }
            }
            lds_barrier();  // every O-wave is done reading the old U^T copy
            write_state_copy();
        }
#ifdef RET_DEBUG
        // chunk c's q and dout are dead until chunk c + 2 is loaded into them
        lds_poison(tl.k[B], C * DK * 2);
        lds_poison(tl.v[B], C * DV * 2);
#endif
    };

    load_chunk(c_begin, std::integral_constant<int, 0>{});
    write_state_copy();  // ordered before the first read by the first step's barrier
    for (int c = c_begin; c < c_end; c += 2) {
        step(c, std::integral_constant<int, 0>{});
        if (c + 1 < c_end) step(c + 1, std::integral_constant<int, 1>{});
    }
    wait_vmcnt<0>();  // the zero-length tail loads of the last step
}

template <int DK, int DV>
__global__ void __launch_bounds__(kThreads, 1) seg_bwd_kv_kernel(const SegArgs a) {
    constexpr int C = 64;
    __shared__ __attribute__((aligned(16))) unsigned short q0[C * DK];
    __shared__ __attribute__((aligned(16))) unsigned short q1[C * DK];
    __shared__ __attribute__((aligned(16))) unsigned short d0[C * DV];
    __shared__ __attribute__((aligned(16))) unsigned short d1[C * DV];
    __shared__ __attribute__((aligned(16))) unsigned short st[DV * DK];
    const STiles tl{{q0, q1}, {d0, d1}, st, nullptr};
    const int bh = blockIdx.x / a.G, seg = blockIdx.x % a.G;
    const float lg = a.log2g[bh % a.H];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    switch (wave) {
        case 0: bwd_kv_body<DK, DV, 0, true>(a, tl, bh, seg, lg); break;
        case 1: bwd_kv_body<DK, DV, 1, true>(a, tl, bh, seg, lg); break;
        case 2: bwd_kv_body<DK, DV, 2, true>(a, tl, bh, seg, lg); break;
        case 3: bwd_kv_body<DK, DV, 3, true>(a, tl, bh, seg, lg); break;
        case 4: bwd_kv_body<DK, DV, 0, false>(a, tl, bh, seg, lg); break;
        case 5: bwd_kv_body<DK, DV, 1, false>(a, tl, bh, seg, lg); break;
        case 6: bwd_kv_body<DK, DV, 2, false>(a, tl, bh, seg, lg); break;
        default: bwd_kv_body<DK, DV, 3, false>(a, tl, bh, seg, lg); break;
    }
}

template <int DK, int DV>
hipError_t launch_bwd_kv_t(const SegArgs& a, hipStream_t stream) {
    const long long bh = static_cast<long long>(a.B) * a.H;
    if (bh <= 0) return hipSuccess;
    if (bh * a.G > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.G > 1) {
        SegArgs sa = a;
        sa.scps = a.cps;  // 64-token chunks are the state kernel's blocks
        hipLaunchKernelGGL((seg_state_kernel<DK, DV, kModeRet, true>), dim3(static_cast<unsigned>(bh * (a.G - 1) * a.pieces)),
                           dim3(kThreads), 0, stream, sa);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((seg_bwd_kv_kernel<DK, DV>), dim3(static_cast<unsigned>(bh * a.G)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace seg
}  // namespace ret
