// seg_kernel.h -- chunkwise causal retention with the sequence split into
// segments (bf16 in, fp32 accumulate, gfx950).
//
// What is computed is the chunkwise form of the retention operator ("RetNet",
// single-head definition and "Chunked Recurrent Representation"; "Efficient
// and Sparse Transformers" section 6, "Chunkwise form").  With S the fp32
// dk x dv state before a chunk of c <= C tokens and local indices i, j:
//   O_i   = sum_{j<=i} gamma^(i-j) (q_i . k_j) v_j  +  gamma^(i+1) q_i S
//   S_new = gamma^c S + sum_j gamma^(c-1-j) k_j v_j^T
//
// Parallel decomposition.  Each (batch, head) sequence is cut into G
// segments of `cps` chunks.  Because the state recurrence is linear, the state
// entering segment g is a decayed sum of the contributions of the segments
// before it:
//   S_in(g) = sum_{j<g} gamma^(L (g-1-j)) dS_j,
//   dS_j    = sum_{t in segment j} gamma^(end_j - 1 - t) k_t v_t^T,
// with L the segment length in tokens (every segment but the last is full).
//   seg_state_kernel  one workgroup per (b, h, j < G-1) computes dS_j
//                     (reads K and V of the segment once).
//   seg_walk_kernel   one workgroup per (b, h, g) forms S_in(g) from the dS_j,
//                     then walks the chunks of segment g with the whole state
//                     in registers and writes O; the last segment also writes
//                     the final state.
// Every workgroup covers the full value width, so Q K^T is computed once per
// chunk, and each workgroup streams its own slice of the sequence.
//
// Per chunk, wave W (of 4) owns query tiles {W, C/16-1-W} (16 rows each, one
// tile when C = 64) and dk tiles {W*DK/64 ...} of the state with every value
// tile.  All products run on v_mfma_f32_16x16x32_bf16, transposed so that the
// Q K^T accumulators feed the P V product from registers:
//   S^T   = K Q^T            A: K rows (LDS)           B: Q rows (registers)
//   P^T   = S^T (.) D        decay factors per lane
//   O^T   = xi (.) S_prev^T Q^T + V^T P^T
//                            A: bf16 state copy / V^T (LDS transpose reads)
//   S     = gamma^c S + (zeta (.) K)^T V
//                            A: K^T (LDS transpose reads, scaled by zeta)
//                            B: the V^T registers of the output product
// K and V go HBM -> LDS by DMA into double-buffered swizzled tiles, one chunk
// ahead; Q goes HBM -> registers directly in operand layout, one chunk ahead.
#pragma once

#include <type_traits>

#include "internal.h"
#include "kcommon.h"

namespace ret {
namespace seg {

using namespace ::ret::kc;

constexpr int kThreads = 256;

template <int C, int DK, int DV>
struct SCfg {
    static constexpr int NI = C / 16;              // 16-token tiles per chunk
    static constexpr int NS = (NI == 8) ? 2 : 1;   // query tiles per wave
    static constexpr int NB = C / 32;              // 32-token operand blocks per chunk
    static constexpr int NKT = DK / 16;            // dk tiles of the state
    static constexpr int NVT = DV / 16;            // dv tiles of the state
    static constexpr int SKT = NKT / 4;            // dk tiles per wave
    static constexpr int KRU = DK / 8;             // 16-byte units per K (and state copy) row
    static constexpr int VRU = DV / 8;             // 16-byte units per V row
    static constexpr int KIW = C * DK * 2 / 1024 / 4;  // 1-KB DMA instructions per wave, K
    static constexpr int VIW = C * DV * 2 / 1024 / 4;  // same for V
    static constexpr int QF = DK / 32;             // Q operand blocks per query tile
    static constexpr int STATE = DK * DV;          // floats per state
    static_assert(NI == 4 || NI == 8, "chunk must be 64 or 128");
    static_assert(NKT == 4 || NKT == 8, "dk must be 64 or 128");
    static_assert(NVT == 4 || NVT == 8, "dv must be 64 or 128");
};

// Workspace layout of one segment state: tile (m, n) of S (dk tile m, dv
// tile n) occupies 256 floats, lane l's four values S[16m + 4(l/16) + r]
// [16n + l%16] (r = 0..3) at 4 l.  Both kernels use the same ownership, so
// the state moves with one 16-byte load or store per lane and tile.
__device__ __forceinline__ int ws_tile_off(int m, int n, int nvt, int lane) {
    return ((m * nvt + n) << 8) + (lane << 2);
}

// LDS tiles: each buffer is its own __shared__ array, so the compiler can
// tell that a DMA into one buffer does not touch the others.
struct STiles {
    unsigned short* k[2];
    unsigned short* v[2];
    unsigned short* s;  // bf16 copy of S^T, [dv][dk], swizzled (walk kernel)
};

// Per-lane byte offsets, within a chunk, of the 16-byte units that DMA
// instruction (W + 4 m) places at LDS byte 1024 (W + 4 m) + 16 l of a
// swizzled tile with RU units per row and `rowbytes` bytes per global row.
template <int RU, int N, int W>
__device__ __forceinline__ void dma_offsets(unsigned (&off)[N], int rowbytes, int l) {
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const int b = (W + 4 * m) * 1024 + l * 16;
        const int r = b / (RU * 16), su = (b % (RU * 16)) >> 4;
        off[m] = static_cast<unsigned>(r * rowbytes + ((su ^ swz_mask<RU>(r)) << 4));
    }
}

// Transpose read of an operand over tokens from a swizzled bf16 tile: this
// lane receives rows r0 .. r0+3 (r0 = the 16-lane group's base row) of
// column 16 t + l%16, as four consecutive k-slots.
template <int RU>
__device__ __forceinline__ u16x4 tr_rows(const unsigned short* tile, int r0, int t, int lq, int lr) {
    const char* base = reinterpret_cast<const char*>(tile);
    return lds_tr4(reinterpret_cast<const unsigned short*>(
        base + swz_byte<RU>(r0 + lq, 2 * t + (lr >> 1)) + (lr & 1) * 8));
}

template <int RU>
__device__ __forceinline__ bf16x8 row_unit(const unsigned short* tile, int r, int u) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
        reinterpret_cast<const char*>(tile) + swz_byte<RU>(r, u)));
}

// The 8 keys of this lane's k-slots in a 32-token block: 4g + e for e < 4,
// 16 + 4g + (e - 4) otherwise (the layout of two stacked MFMA output tiles).
__device__ __forceinline__ int slot_key(int g, int e) { return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4); }

// A-operand of the state update: K^T rows 16 m .. 16 m + 15 (dk), keys of
// block js, each key scaled by z(js, e).
template <int RU, typename ZF>
__device__ __forceinline__ bf16x8 kt_scaled(const unsigned short* kb, int m, int js, int g, int lq, int lr,
                                            ZF zf) {
    const u16x4 lo = tr_rows<RU>(kb, 32 * js + 4 * g, m, lq, lr);
    const u16x4 hi = tr_rows<RU>(kb, 32 * js + 16 + 4 * g, m, lq, lr);
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = bf2f(lo[e]) * zf(js, e);
        b[e] = bf2f(hi[e]) * zf(js, e + 4);
    }
    return cat_bf16(cvt4_bf16(a), cvt4_bf16(b));
}

// ---------------------------------------------------------------------------
// seg_state_kernel: dS_j for one (b, h) and segment j < G - 1.

template <int C, int DK, int DV, int W>
__device__ __forceinline__ void state_body(const SegArgs& a, const STiles& tl, int bh, int seg, float lg) {
    using Cf = SCfg<C, DK, DV>;
    constexpr int NB = Cf::NB, NVT = Cf::NVT, SKT = Cf::SKT, KRU = Cf::KRU, VRU = Cf::VRU;
    constexpr int KIW = Cf::KIW, VIW = Cf::VIW;
    const int tid = threadIdx.x;
    const int l = tid & 63, l16 = l & 15, g = l >> 4, lq = l16 >> 2, lr = l16 & 3;
    (void)l16;
    const int T = a.T;
    const unsigned short* kh = static_cast<const unsigned short*>(a.k) + static_cast<long long>(bh) * T * DK;
    const unsigned short* vh = static_cast<const unsigned short*>(a.v) + static_cast<long long>(bh) * T * DV;

    float zb[8];  // gamma^(31 - key) for this lane's k-slots
#pragma unroll
    for (int e = 0; e < 8; ++e) zb[e] = exp2f(static_cast<float>(31 - slot_key(g, e)) * lg);
    float bj[NB];  // gamma^(32 (NB - 1 - js))
#pragma unroll
    for (int js = 0; js < NB; ++js) bj[js] = exp2f(static_cast<float>(32 * (NB - 1 - js)) * lg);

    unsigned koff[KIW], voff[VIW];
    dma_offsets<KRU, KIW, W>(koff, DK * 2, l);
    dma_offsets<VRU, VIW, W>(voff, DV * 2, l);

    f32x4 acc[SKT][NVT];
#pragma unroll
    for (int mi = 0; mi < SKT; ++mi)
#pragma unroll
        for (int n = 0; n < NVT; ++n) acc[mi][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int c_first = seg * a.cps, c_last = c_first + a.cps - 1;  // all chunks full

    auto load_chunk = [&](int c, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const long long t0 = static_cast<long long>(c) * C;
        const u32x4 wk = rsrc_words(kh + t0 * DK, C * DK * 2);
        const u32x4 wv = rsrc_words(vh + t0 * DV, C * DV * 2);
        const unsigned kbase = __builtin_amdgcn_readfirstlane(lds_addr_of(tl.k[buf]));
        const unsigned vbase = __builtin_amdgcn_readfirstlane(lds_addr_of(tl.v[buf]));
#pragma unroll
        for (int m = 0; m < KIW; ++m) dma16(wk, kbase + (W + 4 * m) * 1024, koff[m]);
#pragma unroll
        for (int m = 0; m < VIW; ++m) dma16(wv, vbase + (W + 4 * m) * 1024, voff[m]);
    };

    // chunks in reverse order (the walk kernel then finds the segment's first
    // chunks most recently read)
    auto step = [&](int c, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        wait_vmcnt<0>();
        __syncthreads();
        if (c > c_first) load_chunk(c - 1, std::integral_constant<int, 1 - B>{});
        // gamma^(C (c_last - c)): decay from the end of chunk c to the end of the segment
        const float wc = exp2f(static_cast<float>(C) * static_cast<float>(c_last - c) * lg);
        const unsigned short* kb = tl.k[B];
        const unsigned short* vb = tl.v[B];
        bf16x8 kz[SKT][NB];
#pragma unroll
        for (int mi = 0; mi < SKT; ++mi)
#pragma unroll
            for (int js = 0; js < NB; ++js)
                kz[mi][js] = kt_scaled<KRU>(kb, SKT * W + mi, js, g, lq, lr,
                                            [&](int j, int e) { return zb[e] * bj[j] * wc; });
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            bf16x8 vf[NB];
#pragma unroll
            for (int js = 0; js < NB; ++js)
                vf[js] = cat_bf16(tr_rows<VRU>(vb, 32 * js + 4 * g, n, lq, lr),
                                  tr_rows<VRU>(vb, 32 * js + 16 + 4 * g, n, lq, lr));
#pragma unroll
            for (int js = 0; js < NB; ++js)
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) acc[mi][n] = mfma_bf16(kz[mi][js], vf[js], acc[mi][n]);
        }
    };

    load_chunk(c_last, std::integral_constant<int, 0>{});
    for (int c = c_last; c >= c_first; c -= 2) {
        step(c, std::integral_constant<int, 0>{});
        if (c - 1 >= c_first) step(c - 1, std::integral_constant<int, 1>{});
    }

    float* wsj = a.ws + (static_cast<long long>(bh) * (a.G - 1) + seg) * Cf::STATE;
#pragma unroll
    for (int mi = 0; mi < SKT; ++mi)
#pragma unroll
        for (int n = 0; n < NVT; ++n)
            *reinterpret_cast<f32x4*>(wsj + ws_tile_off(SKT * W + mi, n, NVT, l)) = acc[mi][n];
}

// ---------------------------------------------------------------------------
// seg_walk_kernel: outputs of one (b, h, segment g).

template <int C, int DK, int DV, int W>
__device__ __forceinline__ void walk_body(const SegArgs& a, const STiles& tl, int bh, int seg, float lg) {
    using Cf = SCfg<C, DK, DV>;
    constexpr int NI = Cf::NI, NS = Cf::NS, NB = Cf::NB, NVT = Cf::NVT, SKT = Cf::SKT;
    constexpr int KRU = Cf::KRU, VRU = Cf::VRU, QF = Cf::QF, KIW = Cf::KIW, VIW = Cf::VIW;
    constexpr int IT0 = W;
    constexpr int IT1 = (NS == 2) ? NI - 1 - W : W;
    constexpr int ITMAX = IT1;
    // vector-memory ops a thread issues after a chunk's loads: the output stores
    constexpr int STORES = NS * NVT;
    auto its = [](int s) constexpr { return s == 0 ? IT0 : IT1; };

    const int tid = threadIdx.x;
    const int l = tid & 63, l16 = l & 15, g = l >> 4, lq = l16 >> 2, lr = l16 & 3;
    const int T = a.T;
    const unsigned short* qh = static_cast<const unsigned short*>(a.q) + static_cast<long long>(bh) * T * DK;
    const unsigned short* kh = static_cast<const unsigned short*>(a.k) + static_cast<long long>(bh) * T * DK;
    const unsigned short* vh = static_cast<const unsigned short*>(a.v) + static_cast<long long>(bh) * T * DV;
    unsigned short* oh = static_cast<unsigned short*>(a.out) + static_cast<long long>(bh) * T * DV;

    const int nch = (T + C - 1) / C;
    const int c_begin = seg * a.cps;
    const int c_end = (c_begin + a.cps < nch) ? c_begin + a.cps : nch;

    // ---- per-lane decay constants
    // P^T element (key 16 jt + 4g + r, query 16 it + l16) has decay
    // gamma^(16 d + l16 - 4g - r), d = it - jt: f0 for d = 0 (0 above the
    // diagonal), gd[d] * f1 for d >= 1 (both exponents non-negative).
    float f0[4], f1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = l16 - 4 * g - r;
        f0[r] = (e < 0) ? 0.f : exp2f(static_cast<float>(e) * lg);
        f1[r] = exp2f(static_cast<float>(16 + e) * lg);
    }
    float gd[ITMAX + 1];
    gd[0] = 1.f;
#pragma unroll
    for (int d = 1; d <= ITMAX; ++d) gd[d] = exp2f(static_cast<float>(16 * (d - 1)) * lg);
    float xi[NS];  // gamma^(i+1) for this lane's query in each owned tile
#pragma unroll
    for (int s = 0; s < NS; ++s) xi[s] = exp2f(static_cast<float>(16 * its(s) + l16 + 1) * lg);
    float zb[8];  // gamma^(31 - key) for this lane's k-slots; zeta = zb * bj for a full chunk
#pragma unroll
    for (int e = 0; e < 8; ++e) zb[e] = exp2f(static_cast<float>(31 - slot_key(g, e)) * lg);
    float bj[NB];
#pragma unroll
    for (int js = 0; js < NB; ++js) bj[js] = exp2f(static_cast<float>(32 * (NB - 1 - js)) * lg);
    const float gC = exp2f(static_cast<float>(C) * lg);

    // ---- state entering the segment
    f32x4 sacc[SKT][NVT];
#pragma unroll
    for (int mi = 0; mi < SKT; ++mi)
#pragma unroll
        for (int n = 0; n < NVT; ++n) sacc[mi][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (seg > 0) {
        const float* wsb = a.ws + static_cast<long long>(bh) * (a.G - 1) * Cf::STATE;
        const float lseg = static_cast<float>(a.cps) * static_cast<float>(C) * lg;
        for (int j = 0; j < seg; ++j) {
            const float w = exp2f(lseg * static_cast<float>(seg - 1 - j));
            const float* wj = wsb + static_cast<long long>(j) * Cf::STATE;
#pragma unroll
            for (int mi = 0; mi < SKT; ++mi)
#pragma unroll
                for (int n = 0; n < NVT; ++n)
                    sacc[mi][n] += w * *reinterpret_cast<const f32x4*>(wj + ws_tile_off(SKT * W + mi, n, NVT, l));
        }
    }

    // bf16 copy of S^T in LDS: this lane's S[16m + 4g + r][16n + l16], r = 0..3,
    // are 4 consecutive dk of row dv = 16n + l16
    auto write_state_copy = [&]() {
        char* sb = reinterpret_cast<char*>(tl.s);
#pragma unroll
        for (int mi = 0; mi < SKT; ++mi) {
            const int m = SKT * W + mi;
#pragma unroll
            for (int n = 0; n < NVT; ++n)
                *reinterpret_cast<u16x4*>(sb + swz_byte<KRU>(16 * n + l16, 2 * m + (g >> 1)) + (g & 1) * 8) =
                    cvt4_bf16(sacc[mi][n]);
        }
    };

    unsigned koff[KIW], voff[VIW];
    dma_offsets<KRU, KIW, W>(koff, DK * 2, l);
    dma_offsets<VRU, VIW, W>(voff, DV * 2, l);

    uint4 qf[2][NS][QF];  // Q operands, double-buffered in registers

    // Issue the loads of chunk c through range-checked resources (rows past
    // the end of the sequence read as zeros).  Nothing consumes them in the
    // step that issues them.
    auto load_chunk = [&](int c, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const long long t0 = static_cast<long long>(c) * C;
        const int cl = (T - t0 < C) ? static_cast<int>(T - t0) : C;
        const u32x4 wk = rsrc_words(kh + t0 * DK, cl * DK * 2);
        const u32x4 wv = rsrc_words(vh + t0 * DV, cl * DV * 2);
        const unsigned kbase = __builtin_amdgcn_readfirstlane(lds_addr_of(tl.k[buf]));
        const unsigned vbase = __builtin_amdgcn_readfirstlane(lds_addr_of(tl.v[buf]));
#pragma unroll
        for (int m = 0; m < KIW; ++m) dma16(wk, kbase + (W + 4 * m) * 1024, koff[m]);
#pragma unroll
        for (int m = 0; m < VIW; ++m) dma16(wv, vbase + (W + 4 * m) * 1024, voff[m]);
        const auto rq = make_rsrc(qh + t0 * DK, cl * DK * 2);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ks = 0; ks < QF; ++ks)
                qf[buf][s][ks] = bload16(rq, static_cast<unsigned>(((16 * its(s) + l16) * DK + 32 * ks + 8 * g) * 2));
    };

    auto step = [&](int c, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        const long long t0 = static_cast<long long>(c) * C;
        const int clen = (T - t0 < C) ? static_cast<int>(T - t0) : C;
        const bool tail = clen < C;  // uniform; only the last chunk of the sequence

        // This chunk's loads were issued one step ago; the only vector-memory
        // ops issued after them are the previous step's output stores, and
        // vector-memory ops complete in issue order.
        if (c == c_begin) wait_vmcnt<0>();
        else wait_vmcnt<STORES>();
        __syncthreads();  // chunk in LDS everywhere, state copy written
        if (c + 1 < c_end) load_chunk(c + 1, std::integral_constant<int, 1 - B>{});

        const unsigned short* kb = tl.k[B];
        const unsigned short* vb = tl.v[B];

        // ---- S^T tiles = K Q^T for key tiles jt <= query tile
        f32x4 pacc[NS][NI];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int jt = 0; jt < NI; ++jt) pacc[s][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < QF; ++ks) {
            bf16x8 ka[ITMAX + 1];
#pragma unroll
            for (int jt = 0; jt <= ITMAX; ++jt) ka[jt] = row_unit<KRU>(kb, 16 * jt + l16, 4 * ks + g);
#pragma unroll
            for (int jt = 0; jt <= ITMAX; ++jt)
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    if (jt <= its(s))
                        pacc[s][jt] = mfma_bf16(ka[jt], __builtin_bit_cast(bf16x8, qf[B][s][ks]), pacc[s][jt]);
        }

        // ---- zeta-scaled K^T operands of the state update
        bf16x8 kz[SKT][NB];
        if (!tail) {
#pragma unroll
            for (int mi = 0; mi < SKT; ++mi)
#pragma unroll
                for (int js = 0; js < NB; ++js)
                    kz[mi][js] = kt_scaled<KRU>(kb, SKT * W + mi, js, g, lq, lr,
                                                [&](int j, int e) { return zb[e] * bj[j]; });
        } else {
            // gamma^(clen - 1 - key) for keys inside the chunk, 0 past its end
#pragma unroll
            for (int mi = 0; mi < SKT; ++mi)
#pragma unroll
                for (int js = 0; js < NB; ++js)
                    kz[mi][js] = kt_scaled<KRU>(kb, SKT * W + mi, js, g, lq, lr, [&](int j, int e) {
                        const int ex = clen - 1 - 32 * j - slot_key(g, e);
                        return (ex < 0) ? 0.f : exp2f(static_cast<float>(ex) * lg);
                    });
        }

        // ---- decay mask, bf16 P^T operands (two key tiles per operand)
        bf16x8 pb[NS][NB];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int js = 0; js < NB; ++js)
                if (2 * js <= its(s)) {
                    f32x4 lo = pacc[s][2 * js], hi = f32x4{0.f, 0.f, 0.f, 0.f};
                    const int d0 = its(s) - 2 * js;
#pragma unroll
                    for (int r = 0; r < 4; ++r) lo[r] *= (d0 == 0) ? f0[r] : gd[d0] * f1[r];
                    if (2 * js + 1 <= its(s)) {
                        hi = pacc[s][2 * js + 1];
                        const int d1 = d0 - 1;
#pragma unroll
                        for (int r = 0; r < 4; ++r) hi[r] *= (d1 == 0) ? f0[r] : gd[d1] * f1[r];
                    }
                    pb[s][js] = cat_bf16(cvt4_bf16(lo), cvt4_bf16(hi));
                }

        // ---- state decay for this chunk
        const float gc = tail ? exp2f(static_cast<float>(clen) * lg) : gC;
#pragma unroll
        for (int mi = 0; mi < SKT; ++mi)
#pragma unroll
            for (int n = 0; n < NVT; ++n) sacc[mi][n] *= gc;

        // ---- per value tile: O^T tiles, stores, state update
        const auto ro = make_rsrc(oh + t0 * DV, clen * DV * 2);
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            bf16x8 vf[NB];
#pragma unroll
            for (int js = 0; js < NB; ++js)
                vf[js] = cat_bf16(tr_rows<VRU>(vb, 32 * js + 4 * g, n, lq, lr),
                                  tr_rows<VRU>(vb, 32 * js + 16 + 4 * g, n, lq, lr));
            f32x4 oacc[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) oacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < QF; ++ks) {
                const bf16x8 sf = row_unit<KRU>(tl.s, 16 * n + l16, 4 * ks + g);
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    oacc[s] = mfma_bf16(sf, __builtin_bit_cast(bf16x8, qf[B][s][ks]), oacc[s]);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) oacc[s] *= xi[s];
#pragma unroll
            for (int js = 0; js < NB; ++js)
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    if (2 * js <= its(s)) oacc[s] = mfma_bf16(vf[js], pb[s][js], oacc[s]);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int row = 16 * its(s) + l16;  // rows past the end are dropped by the resource
                bstore8(ro, static_cast<unsigned>((row * DV + 16 * n + 4 * g) * 2), cvt4_bf16(oacc[s]));
            }
#pragma unroll
            for (int js = 0; js < NB; ++js)
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) sacc[mi][n] = mfma_bf16(kz[mi][js], vf[js], sacc[mi][n]);
        }

        __syncthreads();  // every wave is done reading the old state copy
        write_state_copy();
    };

    if (c_begin < c_end) load_chunk(c_begin, std::integral_constant<int, 0>{});
    write_state_copy();  // ordered before the first read by the first step's barrier
    for (int c = c_begin; c < c_end; c += 2) {
        step(c, std::integral_constant<int, 0>{});
        if (c + 1 < c_end) step(c + 1, std::integral_constant<int, 1>{});
    }

    if (a.final_state && seg == a.G - 1) {
        float* fs = a.final_state + static_cast<long long>(bh) * DK * DV;
#pragma unroll
        for (int mi = 0; mi < SKT; ++mi) {
            const int m = SKT * W + mi;
#pragma unroll
            for (int n = 0; n < NVT; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) fs[(16 * m + 4 * g + r) * DV + 16 * n + l16] = sacc[mi][n][r];
        }
    }
}

template <int C, int DK, int DV>
__global__ void __launch_bounds__(kThreads, 1) seg_state_kernel(const SegArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned short k0[C * DK];
    __shared__ __attribute__((aligned(16))) unsigned short k1[C * DK];
    __shared__ __attribute__((aligned(16))) unsigned short v0[C * DV];
    __shared__ __attribute__((aligned(16))) unsigned short v1[C * DV];
    const STiles tl{{k0, k1}, {v0, v1}, nullptr};
    const int segs = a.G - 1;
    const int bh = blockIdx.x / segs, seg = blockIdx.x % segs;
    const float lg = a.log2g[bh % a.H];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    switch (wave) {
        case 0: state_body<C, DK, DV, 0>(a, tl, bh, seg, lg); break;
        case 1: state_body<C, DK, DV, 1>(a, tl, bh, seg, lg); break;
        case 2: state_body<C, DK, DV, 2>(a, tl, bh, seg, lg); break;
        default: state_body<C, DK, DV, 3>(a, tl, bh, seg, lg); break;
    }
}

template <int C, int DK, int DV>
__global__ void __launch_bounds__(kThreads, 1) seg_walk_kernel(const SegArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned short k0[C * DK];
    __shared__ __attribute__((aligned(16))) unsigned short k1[C * DK];
    __shared__ __attribute__((aligned(16))) unsigned short v0[C * DV];
    __shared__ __attribute__((aligned(16))) unsigned short v1[C * DV];
    __shared__ __attribute__((aligned(16))) unsigned short st[DV * DK];
    const STiles tl{{k0, k1}, {v0, v1}, st};
    const int bh = blockIdx.x / a.G, seg = blockIdx.x % a.G;
    const float lg = a.log2g[bh % a.H];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    switch (wave) {
        case 0: walk_body<C, DK, DV, 0>(a, tl, bh, seg, lg); break;
        case 1: walk_body<C, DK, DV, 1>(a, tl, bh, seg, lg); break;
        case 2: walk_body<C, DK, DV, 2>(a, tl, bh, seg, lg); break;
        default: walk_body<C, DK, DV, 3>(a, tl, bh, seg, lg); break;
    }
}

template <int C, int DK, int DV>
hipError_t launch_t(const SegArgs& a, hipStream_t stream) {
    const long long bh = static_cast<long long>(a.B) * a.H;
    if (bh <= 0) return hipSuccess;
    if (bh * a.G > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.G > 1) {
        hipLaunchKernelGGL((seg_state_kernel<C, DK, DV>), dim3(static_cast<unsigned>(bh * (a.G - 1))),
                           dim3(kThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((seg_walk_kernel<C, DK, DV>), dim3(static_cast<unsigned>(bh * a.G)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <int C>
hipError_t launch_chunk(const SegArgs& a, int dk, int dv, hipStream_t stream) {
    if (dk == 64 && dv == 64) return launch_t<C, 64, 64>(a, stream);
    if (dk == 64 && dv == 128) return launch_t<C, 64, 128>(a, stream);
    if (dk == 128 && dv == 64) return launch_t<C, 128, 64>(a, stream);
    if (dk == 128 && dv == 128) return launch_t<C, 128, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace seg
}  // namespace ret
