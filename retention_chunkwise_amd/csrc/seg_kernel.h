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
// Waves.  A workgroup has 8 waves (two per SIMD) in two roles (see the
// seg_walk_kernel notes below): waves 0-3 compute outputs, wave P owning
// query tiles {P, C/16-1-P} (16 rows each; one tile when C = 64), which
// balances the causal triangle, over the whole value width; waves 4-7 carry
// the fp32 state, wave 4 + P owning dk tiles {P*DK/64, ...} x every value
// tile.  P is a template parameter (four code variants, each unrolled over its
// exact causal tile set).  All products run on v_mfma_f32_16x16x32_bf16,
// transposed so that the Q K^T accumulators feed the P V product from
// registers:
//   S^T   = K Q^T            A: K rows (LDS)           B: Q rows (registers)
//   P^T   = S^T (.) D        decay factors per lane
//   O^T   = xi (.) S_prev^T Q^T + V^T P^T
//                            A: bf16 state copy / V^T (LDS transpose reads)
//   S     = gamma^c S + (zeta (.) K)^T V
//                            A: K^T (LDS transpose reads, scaled by zeta)
//                            B: V^T (LDS transpose reads)
// K and V go HBM -> LDS by DMA into double-buffered swizzled tiles and Q goes
// HBM -> registers of the wave that uses it, all issued one chunk ahead.  LDS
// addresses are a per-lane offset computed once plus an immediate.
#pragma once

#include <type_traits>

#include "internal.h"
#include "kcommon.h"

namespace ret {
namespace seg {

using namespace ::ret::kc;

constexpr int kThreads = 512;

// What a walk computes.  kModeRet: retention.  kModeLin: causal linear
// attention, phi = elu+1 on q and k, gamma = 1, out / (row sum + eps).
// kModeNorm: retention divided by its decayed score row sum floored at 1 in
// size, the normaliser n = gamma^c n + sum zeta k carried beside the state.
// kModeGroup: kModeNorm, then GroupNorm over each output row.
constexpr int kModeRet = 0, kModeLin = 1, kModeNorm = 2, kModeGroup = 3;

template <int C, int DK, int DV, int MODE = kModeRet>
struct SCfg {
    static constexpr int NI = C / 16;              // 16-token tiles per chunk
    static constexpr int NS = (NI == 8) ? 2 : 1;   // query tiles per wave
    static constexpr int NB = C / 32;              // 32-token operand blocks per chunk
    static constexpr int NKT = DK / 16;            // dk tiles of the state
    static constexpr int NVT = DV / 16;            // dv tiles of the state
    static constexpr int SKT = NKT / 4;            // dk tiles per wave
    static constexpr int NVH = NVT / 2;            // dv tiles per wave (one value half)
    static constexpr int KRU = DK / 8;             // 16-byte units per K (and state copy) row
    static constexpr int VRU = DV / 8;             // 16-byte units per V row
    static constexpr int KIW = C * DK * 2 / 1024 / 8;  // 1-KB DMA instructions per wave, K
    static constexpr int VIW = C * DV * 2 / 1024 / 8;  // same for V
    static constexpr int QF = DK / 32;             // Q operand blocks per query tile
    static constexpr int STATE = DK * DV;          // floats per state
    static constexpr int WS = STATE + (MODE != kModeRet ? DK : 0);  // floats per slot (state, normaliser)
    static_assert(NI == 4 || NI == 8, "chunk must be 64 or 128");
    static_assert(NKT == 4 || NKT == 8, "dk must be 64 or 128");
    static_assert(NVT == 4 || NVT == 8, "dv must be 64 or 128");
    static_assert(KIW >= 1 && VIW >= 1, "every wave issues DMA");
};

// Workspace layout of one segment state: tile (m, n) of S (dk tile m, dv
// tile n) occupies 256 floats, lane l's four values S[16m + 4(l/16) + r]
// [16n + l%16] (r = 0..3) at 4 l, so the state moves with one 16-byte access
// per lane and tile.
__device__ __forceinline__ int ws_tile_off(int m, int n, int nvt, int lane) {
    return ((m * nvt + n) << 8) + (lane << 2);
}

// LDS tiles: each buffer is its own __shared__ array, so the compiler can
// tell that a DMA into one buffer does not touch the others.
struct STiles {
    unsigned short* k[2];
    unsigned short* v[2];
    unsigned short* s;     // bf16 copy of S^T, [dv][dk], swizzled (walk kernel)
    float* z;              // normaliser z, [dk] fp32 (walk kernel, linear attention)
};

// Per-lane pieces of the swizzled LDS addresses (see swz_mask).  With RB the
// row bytes of a tile and R0 % 16 == 0:
//  - operand rows (16 bytes at row R0 + l%16, unit 4 ks + g):
//      R0 RB + opr[ks]
//  - transpose reads (rows R0 + 4g .. +3, value/key tile t):
//      R0 RB + tr + ((t << 5) ^ z16)
struct LaneOff {
    int opr[4];
    int tr;
    int z16;
};

template <int RU>
__device__ __forceinline__ LaneOff lane_offsets(int l) {
    constexpr int RB = RU * 16;
    const int l16 = l & 15, g = l >> 4, lq = l16 >> 2, lr = l16 & 3;
    LaneOff o;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) o.opr[ks] = l16 * RB + (((4 * ks + g) ^ swz_mask<RU>(l16)) << 4);
    const int y = 4 * g + lq;
    o.tr = y * RB + (lr & 1) * 8;
    o.z16 = (swz_mask<RU>(y) ^ (lr >> 1)) << 4;
    return o;
}

__device__ __forceinline__ u16x4 tr_at(const unsigned short* tile, int byte) {
    return lds_tr4(reinterpret_cast<const unsigned short*>(reinterpret_cast<const char*>(tile) + byte));
}

__device__ __forceinline__ bf16x8 b128_at(const unsigned short* tile, int byte) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(tile) + byte));
}

// Operand of 32 tokens (rows R0 .. R0+31) of tile column block t: two
// transpose reads; k-slots 8g + e hold rows R0 + slot_key(g, e).
template <int RU>
__device__ __forceinline__ bf16x8 tr_block(const unsigned short* tile, int R0, int xt, const LaneOff& lo) {
    constexpr int RB = RU * 16;
    return cat_bf16(tr_at(tile, R0 * RB + lo.tr + xt), tr_at(tile, (R0 + 16) * RB + lo.tr + xt));
}

// The 8 keys of this lane's k-slots in a 32-token block: 4g + e for e < 4,
// 16 + 4g + (e - 4) otherwise (the layout of two stacked MFMA output tiles).
__device__ __forceinline__ int slot_key(int g, int e) { return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4); }

// K^T operand (dk tile t, token block js) with each key scaled by z[e].
template <int RU>
__device__ __forceinline__ bf16x8 kt_scaled(const unsigned short* kb, int js, int xt, const LaneOff& lo,
                                            const float (&z)[8]) {
    constexpr int RB = RU * 16;
    const u16x4 a = tr_at(kb, 32 * js * RB + lo.tr + xt);
    const u16x4 b = tr_at(kb, (32 * js + 16) * RB + lo.tr + xt);
    f32x4 x, y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = bf2f(a[e]) * z[e];
        y[e] = bf2f(b[e]) * z[e + 4];
    }
    return cat_bf16(cvt4_bf16(x), cvt4_bf16(y));
}

// 2^x on the transcendental unit (v_exp_f32, about 1 ulp; results below the
// normal range flush to zero, which is harmless for decay factors).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Hides a value from loop-invariant code motion: re-issued in every chunk
// step, it keeps the compiler from hoisting LDS addresses (which then fold
// into the instructions' immediate offsets) and decay products out of the
// chunk loop, where each would hold a register for the whole walk.
__device__ __forceinline__ void opaque(int& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void opaque(float& x) { asm volatile("" : "+v"(x)); }
template <int NOPR>
__device__ __forceinline__ void opaque(LaneOff& o) {
#pragma unroll
    for (int i = 0; i < NOPR; ++i) opaque(o.opr[i]);
    opaque(o.tr);
    opaque(o.z16);
}

// phi(x) = elu(x) + 1 = x + 1 for x > 0, e^x otherwise ("Linear attention",
// the elu+1 feature map), with e^x as 2^(x log2 e) on v_exp_f32.
__device__ __forceinline__ float phi_e1(float x) { return x > 0.f ? x + 1.f : ex2(x * 1.4426950408889634f); }

// phi applied to 8 bf16 values, rounded back to bf16.
__device__ __forceinline__ bf16x8 phi8(const bf16x8& x) {
    const u16x8 e = __builtin_bit_cast(u16x8, x);
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = phi_e1(bf2f(e[i]));
        b[i] = phi_e1(bf2f(e[i + 4]));
    }
    return cat_bf16(cvt4_bf16(a), cvt4_bf16(b));
}

// Sum of 8 bf16 values in fp32.
__device__ __forceinline__ float sum8(const bf16x8& x) {
    const u16x8 e = __builtin_bit_cast(u16x8, x);
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += bf2f(e[i]);
    return t;
}

// Uniform value moved to a scalar register.
__device__ __forceinline__ float uni(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Byte offset, within a chunk, of the 16-byte unit that lane l of DMA
// instruction w (LDS bytes [1024 w, +1024)) places at LDS byte 1024 w + 16 l
// of a swizzled tile with RU units per row.  Instruction w + 8 m reads the
// same offset + 8192 m (the swizzle mask depends on row bits that do not
// change between them).
template <int RU>
__device__ __forceinline__ unsigned dma_offset(int w, int l) {
    const int b = w * 1024 + l * 16;
    const int r = b / (RU * 16), su = (b % (RU * 16)) >> 4;
    return static_cast<unsigned>(r * (RU * 16) + ((su ^ swz_mask<RU>(r)) << 4));
}

// The same unit read in time-reversed order: the chunk's row r lives at memory
// row n - 1 - r of a chunk of n rows, so the offset is (n - 1) * row bytes plus
// this per-lane part (unit offset minus r row bytes; instruction w + 8 m adds
// -8192 m).  Rows past a short chunk come out negative, which the buffer's range
// check turns into zeros.
template <int RU>
__device__ __forceinline__ int dma_offset_rev(int w, int l) {
    const int b = w * 1024 + l * 16;
    const int r = b / (RU * 16), su = (b % (RU * 16)) >> 4;
    return ((su ^ swz_mask<RU>(r)) << 4) - r * (RU * 16);
}

// ---------------------------------------------------------------------------
// seg_state_kernel: dS_j for one (b, h) and segment j < G - 1.

// The segment contribution does not depend on how the segment is blocked, so
// this kernel walks 64-token blocks (C here is the block length) through a
// ring of NBUF LDS buffers, prefetching NBUF-1 blocks ahead.  Blocks run last
// to first (the walk kernel then finds each segment's first chunks most
// recently read).
template <int C, int DK, int DV, int MODE, int NBUF, bool REV>
__device__ __forceinline__ void state_body(const SegArgs& a, unsigned short* kring, unsigned short* vring, int bh,
                                           int seg, int piece, float lg, int w) {
    using Cf = SCfg<C, DK, DV, MODE>;
    constexpr bool LIN = MODE == kModeLin, NRM = MODE >= kModeNorm, ZN = MODE != kModeRet;
    constexpr int NB = Cf::NB, NVT = Cf::NVT, NVH = Cf::NVH, SKT = Cf::SKT, KRU = Cf::KRU, VRU = Cf::VRU;
    constexpr int KIW = Cf::KIW, VIW = Cf::VIW;
    constexpr int OPS = KIW + VIW;  // DMA instructions a thread issues per block
    const int l = threadIdx.x & 63, g = l >> 4;
    const int p = w & 3, h = w >> 2;
    const int T = a.T;
    const unsigned short* kh = static_cast<const unsigned short*>(a.k) + static_cast<long long>(bh) * T * DK;
    const unsigned short* vh = static_cast<const unsigned short*>(a.v) + static_cast<long long>(bh) * T * DV;
    const LaneOff lk0 = lane_offsets<KRU>(l), lv0 = lane_offsets<VRU>(l);

    float zb0[8];  // gamma^(31 - key) for this lane's k-slots
#pragma unroll
    for (int e = 0; e < 8; ++e) zb0[e] = ex2(static_cast<float>(31 - slot_key(g, e)) * lg);

    const unsigned koff = dma_offset<KRU>(w, l), voff = dma_offset<VRU>(w, l);
    const int koffr = dma_offset_rev<KRU>(w, l), voffr = dma_offset_rev<VRU>(w, l);

    f32x4 acc[SKT][NVH];
    float zsum[SKT];  // linear attention: partial column sums of phi(K)
#pragma unroll
    for (int mi = 0; mi < SKT; ++mi) {
        zsum[mi] = 0.f;
#pragma unroll
        for (int ni = 0; ni < NVH; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // this workgroup sums piece `piece` of segment `seg`: blocks [piece nblk, +nblk)
    const int nblk = a.scps / a.pieces;           // blocks per piece, all full
    const long long t_seg = (static_cast<long long>(seg) * a.scps + static_cast<long long>(piece) * nblk) * C;
    const unsigned kring0 = __builtin_amdgcn_readfirstlane(lds_addr_of(kring));
    const unsigned vring0 = __builtin_amdgcn_readfirstlane(lds_addr_of(vring));

    // Block i of the walk is segment block nblk-1-i.  Issued for every i (a
    // block past the segment start gets a zero-length range, which moves no
    // data), so each step issues the same number of DMA instructions.
    auto load_block = [&](int i) {
        const int bi = nblk - 1 - i;
        const long long t0 = t_seg + static_cast<long long>(bi) * C;
        const int bytes = (bi >= 0) ? C : 0;
        // memory row of the block's first row (reversed: its rows run backwards from T - 1 - t0)
        const long long mrow = REV ? (bytes ? T - t0 - C : 0) : t0;
        const u32x4 wk = rsrc_words(kh + mrow * DK, bytes * DK * 2);
        const u32x4 wv = rsrc_words(vh + mrow * DV, bytes * DV * 2);
        const int buf = i % NBUF;
        const unsigned kbase = kring0 + buf * (C * DK * 2), vbase = vring0 + buf * (C * DV * 2);
#pragma unroll
        for (int m = 0; m < KIW; ++m)
            dma16(wk, kbase + (w + 8 * m) * 1024,
                  REV ? static_cast<unsigned>((C - 1) * DK * 2 + koffr - 8192 * m) : koff + 8192u * m);
#pragma unroll
        for (int m = 0; m < VIW; ++m)
            dma16(wv, vbase + (w + 8 * m) * 1024,
                  REV ? static_cast<unsigned>((C - 1) * DV * 2 + voffr - 8192 * m) : voff + 8192u * m);
    };

    for (int i = 0; i < NBUF - 1; ++i) load_block(i);
    for (int i = 0; i < nblk; ++i) {
        // blocks i+1 .. i+NBUF-2 may still be in flight; block i has landed
        wait_vmcnt<(NBUF - 2) * OPS>();
        lds_barrier();  // block i in LDS everywhere; block i-1's buffer is free
#ifdef RET_DEBUG
        {
            const int fb = (i + NBUF - 1) % NBUF;  // block i-1's buffer, refilled next
            lds_poison(kring + fb * (C * DK), C * DK * 2);
            lds_poison(vring + fb * (C * DV), C * DV * 2);
            lds_barrier();
        }
#endif
        load_block(i + NBUF - 1);
        LaneOff lk = lk0, lv = lv0;
        opaque<0>(lk);
        opaque<0>(lv);
        float zb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            zb[e] = zb0[e];
            opaque(zb[e]);
        }
        // gamma^(C i): decay from the end of this block to the end of the piece
        const float wc = uni(ex2(static_cast<float>(C) * static_cast<float>(i) * lg));
        const int buf = i % NBUF;
        const unsigned short* kb = kring + buf * (C * DK);
        const unsigned short* vb = vring + buf * (C * DV);
        bf16x8 kz[SKT][NB];
#pragma unroll
        for (int js = 0; js < NB; ++js) {
            if constexpr (LIN) {
                // phi(k)^T operands and their column sums (the normaliser)
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) {
                    kz[mi][js] = phi8(tr_block<KRU>(kb, 32 * js, ((SKT * p + mi) << 5) ^ lk.z16, lk));
                    zsum[mi] += sum8(kz[mi][js]);
                }
            } else {
                const float bj = uni(ex2(static_cast<float>(32 * (NB - 1 - js)) * lg)) * wc;
                float z[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) z[e] = zb[e] * bj;
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) {
                    kz[mi][js] = kt_scaled<KRU>(kb, js, ((SKT * p + mi) << 5) ^ lk.z16, lk, z);
                    if constexpr (NRM) zsum[mi] += sum8(kz[mi][js]);  // decayed key sums (the normaliser)
                }
            }
        }
#pragma unroll
        for (int ni = 0; ni < NVH; ++ni) {
            const int xt = ((NVH * h + ni) << 5) ^ lv.z16;
#pragma unroll
            for (int js = 0; js < NB; ++js) {
                const bf16x8 vf = tr_block<VRU>(vb, 32 * js, xt, lv);
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) acc[mi][ni] = mfma_bf16(kz[mi][js], vf, acc[mi][ni]);
            }
        }
    }
    wait_vmcnt<0>();  // drain the zero-length tail loads before the workgroup ends

    float* wsj = a.ws + ((static_cast<long long>(bh) * (a.G - 1) + seg) * a.pieces + piece) * Cf::WS;
#pragma unroll
    for (int mi = 0; mi < SKT; ++mi) {
#pragma unroll
        for (int ni = 0; ni < NVH; ++ni)
            *reinterpret_cast<f32x4*>(wsj + ws_tile_off(SKT * p + mi, NVH * h + ni, NVT, l)) = acc[mi][ni];
        if constexpr (ZN) {
            // lanes l, l^16, l^32, l^48 hold the four key groups of column 16m + l%16
            const float zt = sum_over_groups(zsum[mi]);
            if (h == 0 && g == 0) wsj[Cf::STATE + 16 * (SKT * p + mi) + (l & 15)] = zt;
        }
    }
}

// ---------------------------------------------------------------------------
// seg_walk_kernel: outputs of one (b, h, segment g).
//
// Roles.  Waves 0-3 ("O-waves", P = wave) compute the outputs of query tiles
// {P, C/16-1-P} over the full value width; waves 4-7 ("S-waves", P = wave-4)
// carry dk tiles {P*DK/64, ...} x every value tile of the state.  Waves P and
// P + 4 share a SIMD, so the MFMA-heavy output products of one overlap the
// vector work of the other.  Both roles pass the same two barriers per step.
//
// Value-column order of the output products.  O-wave MFMA tiles pair up: row
// 4q + j (q, j < 4) of tile 2a + b holds value column 32a + 8q + 4b + j, so a
// lane's accumulators of the two tiles of a pair are 8 consecutive columns of
// one query row (one 16-byte store).  The bf16 state copy stores its rows in
// the same order: row 16 n + i holds the value column of row i of tile n.

// 16-byte output store.  Plain (cached) on purpose: a store instruction fills
// half of each 128-byte line it touches and the next one fills the other
// half; with a streaming (non-temporal) hint the halves reach HBM separately
// and the write traffic measured 1.34x the output size, without it exactly 1x.
__device__ __forceinline__ void bstore16_bf(__amdgpu_buffer_rsrc_t r, unsigned off, const bf16x8& x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, static_cast<int>(off), 0, 0);
}

// State-copy row of value column dv.
__device__ __forceinline__ int perm_row(int dv) {
    return (dv & ~31) | (((dv >> 2) & 1) << 4) | (((dv >> 3) & 3) << 2) | (dv & 3);
}

// The state entering segment seg, summed into an S-wave's tiles (wave P + 4:
// dk tiles SKT P .. + SKT - 1 by every value tile) from the state kernel's
// workspace:
//   S_in = sum_{j<seg, pieces p} gamma^(L (seg-1-j) + Lp (pieces-1-p)) dS_{j,p}
// and for the normalised modes the normaliser beside it.  Value tiles go in
// groups of NG and SB workspace states of a group are loaded at once, so the
// loads of a batch are in flight together.  tr: the workspace holds the
// states of a walk with key and value roles swapped (read transposed).
template <int C, int DK, int DV, int MODE, int P>
__device__ __forceinline__ void sum_segment_states(const SegArgs& a, int bh, int seg, float lg, bool tr,
                                                   f32x4 (&sacc)[SCfg<C, DK, DV, MODE>::SKT][SCfg<C, DK, DV, MODE>::NVT],
                                                   float (&zacc)[SCfg<C, DK, DV, MODE>::SKT]) {
    using Cf = SCfg<C, DK, DV, MODE>;
    constexpr bool ZN = MODE != kModeRet;
    constexpr int SKT = Cf::SKT, NVT = Cf::NVT, NKT = Cf::NKT;
    constexpr int NG = NVT < 2 ? NVT : 2;  // value tiles per group
    constexpr int SB = 8 / SKT;            // workspace states in flight
    const int l = threadIdx.x & 63, l16 = l & 15, g = l >> 4;
    const float* wsb = a.ws + static_cast<long long>(bh) * (a.G - 1) * a.pieces * Cf::WS;
    const float lseg = static_cast<float>(a.cps) * static_cast<float>(C) * lg;
    const float lpiece = lseg / static_cast<float>(a.pieces);
    const int nslot = seg * a.pieces;
#pragma unroll
    for (int n0 = 0; n0 < NVT; n0 += NG) {
        const bool zg = ZN && n0 == 0;  // the normaliser travels with the first group
        for (int j0 = 0; j0 < nslot; j0 += SB) {
            f32x4 x[SB][SKT][NG];
            float zx[SB][SKT];
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                const int jp = (j0 + b < nslot) ? j0 + b : nslot - 1;  // past the end: reloaded, weight 0
                const float* sj = wsb + static_cast<long long>(jp) * Cf::WS;
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) {
                    const int m = SKT * P + mi;
#pragma unroll
                    for (int nn = 0; nn < NG; ++nn) {
                        const int n = n0 + nn;
                        if (tr) {
                            // S[16m + 4g + r][16n + l16] is element l16 % 4 of lane 16 (l16 / 4) + 4g + r
                            // in tile (n, m) of the transposed state
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                x[b][mi][nn][r] = sj[((n * NKT + m) << 8) + ((16 * (l16 >> 2) + 4 * g + r) << 2) + (l16 & 3)];
                        } else {
                            x[b][mi][nn] = *reinterpret_cast<const f32x4*>(sj + ws_tile_off(m, n, NVT, l));
                        }
                    }
                    zx[b][mi] = zg ? sj[Cf::STATE + 16 * m + l16] : 0.f;
                }
            }
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                const int jp = j0 + b;
                const int j = jp / a.pieces, pc = jp % a.pieces;
                const float wj = (jp < nslot) ? uni(ex2(lseg * static_cast<float>(seg - 1 - j) +
                                                         lpiece * static_cast<float>(a.pieces - 1 - pc)))
                                              : 0.f;
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) {
#pragma unroll
                    for (int nn = 0; nn < NG; ++nn) sacc[mi][n0 + nn] += wj * x[b][mi][nn];
                    if (zg) zacc[mi] += wj * zx[b][mi];
                }
            }
        }
    }
}

template <int C, int DK, int DV, int MODE, int P, bool OW>
__device__ __forceinline__ void walk_body(const SegArgs& a, const STiles& tl, int bh, int seg, float lg) {
    using Cf = SCfg<C, DK, DV, MODE>;
    constexpr bool LIN = MODE == kModeLin, NRM = MODE >= kModeNorm, GRP = MODE == kModeGroup;
    constexpr bool ZN = MODE != kModeRet;  // a normaliser travels with the state
    constexpr int NI = Cf::NI, NS = Cf::NS, NB = Cf::NB, NVT = Cf::NVT, SKT = Cf::SKT;
    constexpr int KRU = Cf::KRU, VRU = Cf::VRU, QF = Cf::QF, KIW = Cf::KIW, VIW = Cf::VIW;
    constexpr int KRB = KRU * 16, VRB = VRU * 16;
    constexpr int NPAIR = NVT / 2;
    constexpr int IT0 = P;
    constexpr int IT1 = (NS == 2) ? NI - 1 - P : P;
    constexpr int ITMAX = IT1;
    // vector-memory ops a thread issues after a chunk's loads: its output stores
    constexpr int STORES = OW ? NS * NPAIR : 0;
    auto its = [](int s) constexpr { return s == 0 ? IT0 : IT1; };

    const int w = P + (OW ? 0 : 4);
    const int l = threadIdx.x & 63, l16 = l & 15, g = l >> 4, lq = l16 >> 2, lr = l16 & 3;
    const int T = a.T;
    const unsigned short* qh = static_cast<const unsigned short*>(a.q) + static_cast<long long>(bh) * T * DK;
    const unsigned short* kh = static_cast<const unsigned short*>(a.k) + static_cast<long long>(bh) * T * DK;
    const unsigned short* vh = static_cast<const unsigned short*>(a.v) + static_cast<long long>(bh) * T * DV;
    unsigned short* oh = static_cast<unsigned short*>(a.out) + static_cast<long long>(bh) * T * DV;
    const LaneOff lk0 = lane_offsets<KRU>(l), lv0 = lane_offsets<VRU>(l);
    // O-wave transpose reads of V in the permuted column order: lane L reads
    // row R0 + 4g + L/4, unit 4a + L%4, half b:  R0 RB + rowo + (uo ^ (a << 6)) + 8 b
    const int rowo0 = (4 * g + lq) * VRB;
    const int uo0 = (lr ^ swz_mask<VRU>(4 * g + lq)) << 4;

    const int nch = (T + C - 1) / C;
    const int c_begin = seg * a.cps;
    const int c_end = (c_begin + a.cps < nch) ? c_begin + a.cps : nch;

    // ---- decay constants
    // P^T element (key 16 jt + 4g + r, query 16 it + l16) has decay
    // gamma^(16 d + l16 - 4g - r), d = it - jt: f0 for d = 0 (0 above the
    // diagonal), gd[d] * f1 for d >= 1 (both exponents non-negative).
    float f0[4], f1_0[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = l16 - 4 * g - r;
        f0[r] = (e < 0) ? 0.f : ex2(static_cast<float>(e) * lg);
        f1_0[r] = ex2(static_cast<float>(16 + e) * lg);
    }
    float gd[ITMAX + 1];
    gd[0] = 1.f;
#pragma unroll
    for (int d = 1; d <= ITMAX; ++d) gd[d] = uni(ex2(static_cast<float>(16 * (d - 1)) * lg));
    float xi[NS];  // gamma^(i+1) for this lane's query in each owned tile
#pragma unroll
    for (int s = 0; s < NS; ++s) xi[s] = ex2(static_cast<float>(16 * its(s) + l16 + 1) * lg);
    float zb0[8];  // gamma^(31 - key) for this lane's k-slots; zeta = zb * bj for a full chunk
#pragma unroll
    for (int e = 0; e < 8; ++e) zb0[e] = ex2(static_cast<float>(31 - slot_key(g, e)) * lg);
    float bj[NB];
#pragma unroll
    for (int js = 0; js < NB; ++js) bj[js] = uni(ex2(static_cast<float>(32 * (NB - 1 - js)) * lg));
    const float gC = uni(ex2(static_cast<float>(C) * lg));

    // ---- S-waves: state (and, for linear attention, normaliser) entering the segment
    f32x4 sacc[OW ? 1 : SKT][OW ? 1 : NVT];
    float zacc[SKT];  // z[16m + l16] of this wave's dk tiles (linear attention)
    if constexpr (!OW) {
#pragma unroll
        for (int mi = 0; mi < SKT; ++mi) {
            zacc[mi] = 0.f;
#pragma unroll
            for (int n = 0; n < NVT; ++n) sacc[mi][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (seg > 0) sum_segment_states<C, DK, DV, MODE, P>(a, bh, seg, lg, !ZN && a.ws_tr, sacc, zacc);
        if (a.init_state) {
            // the state before token 0, decayed over the seg * L tokens before this segment
            const float w0 = uni(ex2(static_cast<float>(a.cps) * static_cast<float>(C) * lg * static_cast<float>(seg)));
            const float* si = a.init_state + static_cast<long long>(bh) * DK * DV;
#pragma unroll
            for (int mi = 0; mi < SKT; ++mi) {
                const int m = SKT * P + mi;
#pragma unroll
                for (int n = 0; n < NVT; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sacc[mi][n][r] += w0 * si[(16 * m + 4 * g + r) * DV + 16 * n + l16];
            }
        }
        if constexpr (LIN) {
            if (a.init_z) {
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi)
                    zacc[mi] += a.init_z[static_cast<long long>(bh) * DK + 16 * (SKT * P + mi) + l16];
            }
        }
    }

    // bf16 copy of S^T in LDS: this lane's S[16m + 4g + r][16n + l16], r = 0..3,
    // are 4 consecutive dk of value column 16n + l16
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
                if (ZN && g == 0) tl.z[16 * m + l16] = zacc[mi];
            }
        }
    };

    const unsigned koff = dma_offset<KRU>(w, l), voff = dma_offset<VRU>(w, l);

    // Issue the loads of chunk c through range-checked resources (rows past
    // the end of the sequence read as zeros).
    auto chunk_len = [&](int c) {
        const long long t0 = static_cast<long long>(c) * C;
        return (T - t0 < C) ? static_cast<int>(T - t0) : C;
    };
    bf16x8 qf[OW ? 2 : 1][NS][QF];  // O-waves: Q operands, double-buffered in registers
    // Issued unconditionally (a chunk past the segment gets a zero-length
    // range, which moves no data): a conditional load would make the
    // compiler's own waits assume the path without it and stall on the
    // loads just issued.
    auto load_chunk = [&](int c, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const long long t0 = static_cast<long long>(c) * C;
        const int cl = (c < c_end) ? chunk_len(c) : 0;
        const u32x4 wk = rsrc_words(kh + t0 * DK, cl * DK * 2);
        const u32x4 wv = rsrc_words(vh + t0 * DV, cl * DV * 2);
        const unsigned kbase = __builtin_amdgcn_readfirstlane(lds_addr_of(tl.k[buf]));
        const unsigned vbase = __builtin_amdgcn_readfirstlane(lds_addr_of(tl.v[buf]));
#pragma unroll
        for (int m = 0; m < KIW; ++m)
            dma16(wk, kbase + (w + 8 * m) * 1024, koff + 8192u * m);
#pragma unroll
        for (int m = 0; m < VIW; ++m)
            dma16(wv, vbase + (w + 8 * m) * 1024, voff + 8192u * m);
        if constexpr (OW) {
            const auto rq = make_rsrc(qh + t0 * DK, cl * DK * 2);
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int ks = 0; ks < QF; ++ks)
                    qf[buf][s][ks] = __builtin_bit_cast(
                        bf16x8, bload16(rq, static_cast<unsigned>(((16 * its(s) + l16) * DK + 32 * ks + 8 * g) * 2)));
        }
    };

    // phi on the K chunk in buffer b, in place; rows past the end (loaded as
    // zeros) stay zero rather than phi(0) = 1
    auto phi_pass = [&](int b, int cl) {
        if constexpr (LIN) {
            constexpr int UPT = C * DK / 8 / kThreads;  // 16-byte units per thread
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                const int u = threadIdx.x + kThreads * i;
                if (u / KRU < cl) {
                    bf16x8* pk = reinterpret_cast<bf16x8*>(tl.k[b] + 8 * u);
                    *pk = phi8(*pk);
                }
            }
        }
    };

    auto step = [&](int c, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        const long long t0 = static_cast<long long>(c) * C;
        const int clen = (T - t0 < C) ? static_cast<int>(T - t0) : C;
        const bool tail = clen < C;  // uniform; only the last chunk of the sequence

        // This chunk's loads were issued during the previous step; the only
        // vector-memory ops issued after them are the previous step's output
        // stores, and vector-memory ops complete in issue order.  Linear
        // attention waits for them at the end of the previous step instead,
        // to apply phi there (the first chunk: here).
        if (c == c_begin) {
            wait_vmcnt<0>();
            if constexpr (LIN) {
                lds_barrier();
                phi_pass(B, clen);
            }
        } else if constexpr (!LIN) {
            wait_vmcnt<STORES>();
        }
        lds_barrier();  // chunk in LDS everywhere (phi applied), state copy written
        load_chunk(c + 1, std::integral_constant<int, 1 - B>{});

        const unsigned short* kb = tl.k[B];
        const unsigned short* vb = tl.v[B];
        // Linear attention: the end of this step waits for chunk c + 1's loads
        // and applies phi to its K in place before the next step's barrier.
        auto end_step = [&]() {
            if constexpr (LIN) {
                wait_vmcnt<STORES>();
                lds_barrier();  // chunk c + 1 in LDS everywhere; chunk c's K read by every wave
                if (c + 1 < c_end) phi_pass(1 - B, chunk_len(c + 1));
            } else {
                lds_barrier();
            }
        };

        if constexpr (OW) {
            LaneOff lk = lk0;
            opaque<QF>(lk);
            float f1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                f1[r] = f1_0[r];
                opaque(f1[r]);
            }
            // ---- Q operands (phi(q) for linear attention)
            bf16x8 qp[NS][QF];
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int ks = 0; ks < QF; ++ks) qp[s][ks] = LIN ? phi8(qf[B][s][ks]) : qf[B][s][ks];

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
                for (int jt = 0; jt <= ITMAX; ++jt) ka[jt] = b128_at(kb, 16 * jt * KRB + lk.opr[ks]);
#pragma unroll
                for (int jt = 0; jt <= ITMAX; ++jt)
#pragma unroll
                    for (int s = 0; s < NS; ++s)
                        if (jt <= its(s)) pacc[s][jt] = mfma_bf16(ka[jt], qp[s][ks], pacc[s][jt]);
            }

            // ---- decay mask, bf16 P^T operands (two key tiles per operand);
            // the row-sum floor sums the fp32 weights before their rounding
            bf16x8 pb[NS][NB];
            float psum[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                psum[s] = 0.f;
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
                        if constexpr (NRM) psum[s] += (lo[0] + lo[1]) + (lo[2] + lo[3]) + ((hi[0] + hi[1]) + (hi[2] + hi[3]));
                        pb[s][js] = cat_bf16(cvt4_bf16(lo), cvt4_bf16(hi));
                    }
            }

            // ---- per-query divisors: the row sum of P plus the earlier tokens'
            // share, q . z_prev (decayed by xi for retention).  Linear attention:
            // 1 / (sum + eps) with the bf16 weights the numerator uses (all
            // positive, so the quotient stays a weighted mean of the values);
            // the row-sum floor: 1 / max(|sum|, 1) with the fp32 weights (signed
            // weights cancel, and their rounding errors must not).
            float rden[NS];
            if constexpr (ZN) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    float tp = 0.f, tz = 0.f;
                    f32x4 ones_acc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (LIN) {
                        // row sums of the bf16 weights on the matrix core: a ones
                        // operand against P^T leaves every key's weight summed in
                        // each row of the tile (all four lane groups alike)
                        const bf16x8 ones = __builtin_bit_cast(bf16x8, u16x8{0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80,
                                                                             0x3f80, 0x3f80, 0x3f80});
#pragma unroll
                        for (int js = 0; js < NB; ++js)
                            if (2 * js <= its(s)) ones_acc = mfma_bf16(ones, pb[s][js], ones_acc);
                    } else {
                        tp = psum[s];
                    }
#pragma unroll
                    for (int ks = 0; ks < QF; ++ks) {
                        const u16x8 e = __builtin_bit_cast(u16x8, qp[s][ks]);
                        const f32x4 z0 = *reinterpret_cast<const f32x4*>(tl.z + 32 * ks + 8 * g);
                        const f32x4 z1 = *reinterpret_cast<const f32x4*>(tl.z + 32 * ks + 8 * g + 4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) tz += bf2f(e[i]) * z0[i] + bf2f(e[i + 4]) * z1[i];
                    }
                    if constexpr (LIN) {
                        rden[s] = 1.f / (ones_acc[0] + sum_over_groups(tz) + a.eps);
                    } else {
                        const float r = sum_over_groups(tp + xi[s] * tz);
                        rden[s] = 1.f / fmaxf(fabsf(r), 1.f);
                    }
                }
            }

            // ---- O^T = xi S_prev^T Q^T + V^T P^T per value-tile pair; 16-byte stores
            int rowo = rowo0, uo = uo0;
            opaque(rowo);
            opaque(uo);
            const auto ro = make_rsrc(oh + t0 * DV, clen * DV * 2);
            // outputs of value-tile pair pa (columns 32 pa .. +31 in the permuted
            // order) for this wave's query tiles, scaled by their divisors
            auto pair_out = [&](int pa, f32x4 (&oacc)[NS][2]) {
                const int uoa = uo ^ (pa << 6);
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int n = 2 * pa + b;
#pragma unroll
                    for (int s = 0; s < NS; ++s) oacc[s][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < QF; ++ks) {
                        const bf16x8 sf = b128_at(tl.s, 16 * n * KRB + lk.opr[ks]);
#pragma unroll
                        for (int s = 0; s < NS; ++s) oacc[s][b] = mfma_bf16(sf, qp[s][ks], oacc[s][b]);
                    }
                    if constexpr (!LIN) {
#pragma unroll
                        for (int s = 0; s < NS; ++s) oacc[s][b] *= xi[s];
                    }
#pragma unroll
                    for (int js = 0; 2 * js <= ITMAX; ++js) {
                        const bf16x8 vf = cat_bf16(tr_at(vb, 32 * js * VRB + rowo + uoa + 8 * b),
                                                   tr_at(vb, (32 * js + 16) * VRB + rowo + uoa + 8 * b));
#pragma unroll
                        for (int s = 0; s < NS; ++s)
                            if (2 * js <= its(s)) oacc[s][b] = mfma_bf16(vf, pb[s][js], oacc[s][b]);
                    }
                }
                if constexpr (ZN) {
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        oacc[s][0] *= rden[s];
                        oacc[s][1] *= rden[s];
                    }
                }
            };
            auto store_pair = [&](int pa, const f32x4 (&oacc)[NS][2]) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const int row = 16 * its(s) + l16;  // rows past the end are dropped by the resource
                    bstore16_bf(ro, static_cast<unsigned>((row * DV + 32 * pa + 8 * g) * 2),
                                cat_bf16(cvt4_bf16(oacc[s][0]), cvt4_bf16(oacc[s][1])));
                }
            };
            if constexpr (GRP) {
                // GroupNorm needs a whole row before any of it is stored, and the
                // row does not fit in registers beside everything else: the first
                // pass only gathers each row's statistics over the value tiles, the
                // second recomputes the products and stores standardised values.
                // Statistics: per pair of value tiles the lane's 8 values give a
                // mean and a sum of squared deviations, merged into the running
                // pair by Chan's pairwise update, then across the four lane groups
                // the same way; no E[x^2] - mean^2 cancellation.
                float mean[NS], m2[NS];
#pragma unroll
                for (int pa = 0; pa < NPAIR; ++pa) {
                    f32x4 oacc[NS][2];
                    pair_out(pa, oacc);
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        const f32x4 t = oacc[s][0] + oacc[s][1];
                        const float mb = ((t[0] + t[1]) + (t[2] + t[3])) * 0.125f;
                        const f32x4 d0 = oacc[s][0] - mb, d1 = oacc[s][1] - mb;
                        float qb = 0.f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) qb += d0[r] * d0[r] + d1[r] * d1[r];
                        if (pa == 0) {
                            mean[s] = mb;
                            m2[s] = qb;
                        } else {
                            // counts 8 pa (running) and 8 (this pair)
                            const float dl = mb - mean[s], wb = 1.f / static_cast<float>(pa + 1);
                            mean[s] += dl * wb;
                            m2[s] += qb + dl * dl * (8.f * static_cast<float>(pa) * wb);
                        }
                    }
                }
                float mu[NS], rstd[NS];
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    // merge equal counts: n = 8 NPAIR per lane, then 16 NPAIR
                    float m = mean[s], q2 = m2[s], n = 8.f * NPAIR;
#pragma unroll
                    for (int x = 16; x <= 32; x <<= 1) {
                        const float mo = __shfl_xor(m, x), qo = __shfl_xor(q2, x);
                        const float dl = mo - m;
                        q2 += qo + dl * dl * (0.5f * n);
                        m = 0.5f * (m + mo);
                        n *= 2.f;
                    }
                    mu[s] = m;
                    rstd[s] = 1.f / sqrtf(q2 * (1.f / DV) + a.gn_eps);
                }
#pragma unroll
                for (int pa = 0; pa < NPAIR; ++pa) {
                    f32x4 oacc[NS][2];
                    pair_out(pa, oacc);
#pragma unroll
                    for (int s = 0; s < NS; ++s)
#pragma unroll
                        for (int b = 0; b < 2; ++b) oacc[s][b] = (oacc[s][b] - mu[s]) * rstd[s];
                    store_pair(pa, oacc);
                }
            } else {
#pragma unroll
                for (int pa = 0; pa < NPAIR; ++pa) {
                    f32x4 oacc[NS][2];
                    pair_out(pa, oacc);
                    store_pair(pa, oacc);
                }
            }
            end_step();  // every O-wave is done reading the old state copy
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
            // ---- zeta-scaled K^T operands of the state update (phi(k)^T, unscaled,
            // for linear attention, with their column sums)
            bf16x8 kz[SKT][NB];
            float zsum[SKT];
#pragma unroll
            for (int mi = 0; mi < SKT; ++mi) zsum[mi] = 0.f;
#pragma unroll
            for (int js = 0; js < NB; ++js) {
                if constexpr (LIN) {
#pragma unroll
                    for (int mi = 0; mi < SKT; ++mi) {
                        kz[mi][js] = tr_block<KRU>(kb, 32 * js, ((SKT * P + mi) << 5) ^ lk.z16, lk);
                        zsum[mi] += sum8(kz[mi][js]);
                    }
                } else {
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
                    for (int mi = 0; mi < SKT; ++mi) {
                        kz[mi][js] = kt_scaled<KRU>(kb, js, ((SKT * P + mi) << 5) ^ lk.z16, lk, z);
                        if constexpr (NRM) zsum[mi] += sum8(kz[mi][js]);  // decayed key sums
                    }
                }
            }

            // ---- S = gamma^c S + (zeta K)^T V   (z += sum phi(k) for linear attention,
            // z = gamma^c z + sum zeta k for the row-sum floor)
            const float gc = tail ? uni(ex2(static_cast<float>(clen) * lg)) : gC;
#pragma unroll
            for (int n = 0; n < NVT; ++n) {
                const int xt = (n << 5) ^ lv.z16;
                if constexpr (!LIN) {
#pragma unroll
                    for (int mi = 0; mi < SKT; ++mi) sacc[mi][n] *= gc;
                }
#pragma unroll
                for (int js = 0; js < NB; ++js) {
                    const bf16x8 vf = tr_block<VRU>(vb, 32 * js, xt, lv);
#pragma unroll
                    for (int mi = 0; mi < SKT; ++mi) sacc[mi][n] = mfma_bf16(kz[mi][js], vf, sacc[mi][n]);
                }
            }
            if constexpr (ZN) {
                // lanes l, l^16, l^32, l^48 hold the four key groups of column 16m + l%16
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi) zacc[mi] = (LIN ? 1.f : gc) * zacc[mi] + sum_over_groups(zsum[mi]);
            }
            end_step();  // every O-wave is done reading the old state copy
            write_state_copy();
        }
#ifdef RET_DEBUG
        // chunk c's K and V are dead until chunk c + 2 is loaded into them
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

    if constexpr (!OW) {
        if (a.final_state && seg == a.G - 1) {
            float* fs = a.final_state + static_cast<long long>(bh) * DK * DV;
#pragma unroll
            for (int mi = 0; mi < SKT; ++mi) {
                const int m = SKT * P + mi;
#pragma unroll
                for (int n = 0; n < NVT; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) fs[(16 * m + 4 * g + r) * DV + 16 * n + l16] = sacc[mi][n][r];
            }
        }
        if constexpr (LIN) {
            if (a.final_z && seg == a.G - 1 && g == 0) {
#pragma unroll
                for (int mi = 0; mi < SKT; ++mi)
                    a.final_z[static_cast<long long>(bh) * DK + 16 * (SKT * P + mi) + l16] = zacc[mi];
            }
        }
    }
}

// State kernel blocking: 64-token blocks, 4-deep ring.
constexpr int kStateBlock = 64;
constexpr int kStateRing = 4;

template <int DK, int DV, int MODE, bool REV>
__global__ void __launch_bounds__(kThreads, 1) seg_state_kernel(const SegArgs a) {
    constexpr bool LIN = MODE == kModeLin;
    __shared__ __attribute__((aligned(16))) unsigned short kring[kStateRing * kStateBlock * DK];
    __shared__ __attribute__((aligned(16))) unsigned short vring[kStateRing * kStateBlock * DV];
    const int slots = (a.G - 1) * a.pieces;
    const int bh = blockIdx.x / slots, slot = blockIdx.x % slots;
    const float lg = LIN ? 0.f : a.log2g[bh % a.H];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    state_body<kStateBlock, DK, DV, MODE, kStateRing, REV>(a, kring, vring, bh, slot / a.pieces, slot % a.pieces, lg,
                                                          wave);
}

template <int C, int DK, int DV, int MODE>
__global__ void __launch_bounds__(kThreads, 1) seg_walk_kernel(const SegArgs a) {
    constexpr bool LIN = MODE == kModeLin;
    __shared__ __attribute__((aligned(16))) unsigned short k0[C * DK];
    __shared__ __attribute__((aligned(16))) unsigned short k1[C * DK];
    __shared__ __attribute__((aligned(16))) unsigned short v0[C * DV];
    __shared__ __attribute__((aligned(16))) unsigned short v1[C * DV];
    __shared__ __attribute__((aligned(16))) unsigned short st[DV * DK];
    float* zp = nullptr;
    if constexpr (MODE != kModeRet) {
        __shared__ __attribute__((aligned(16))) float zs[DK];  // only the normalised modes carry z
        zp = zs;
    }
    const STiles tl{{k0, k1}, {v0, v1}, st, zp};
    const int bh = blockIdx.x / a.G, seg = blockIdx.x % a.G;
    const float lg = LIN ? 0.f : a.log2g[bh % a.H];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    switch (wave) {
        case 0: walk_body<C, DK, DV, MODE, 0, true>(a, tl, bh, seg, lg); break;
        case 1: walk_body<C, DK, DV, MODE, 1, true>(a, tl, bh, seg, lg); break;
        case 2: walk_body<C, DK, DV, MODE, 2, true>(a, tl, bh, seg, lg); break;
        case 3: walk_body<C, DK, DV, MODE, 3, true>(a, tl, bh, seg, lg); break;
        case 4: walk_body<C, DK, DV, MODE, 0, false>(a, tl, bh, seg, lg); break;
        case 5: walk_body<C, DK, DV, MODE, 1, false>(a, tl, bh, seg, lg); break;
        case 6: walk_body<C, DK, DV, MODE, 2, false>(a, tl, bh, seg, lg); break;
        default: walk_body<C, DK, DV, MODE, 3, false>(a, tl, bh, seg, lg); break;
    }
}

// LDS available to one workgroup on gfx950, and what the walk kernel takes.
constexpr int kLdsBytes = 160 * 1024;
template <int C, int DK, int DV, int MODE>
constexpr bool walk_fits() {
    return 2 * C * DK * 2 + 2 * C * DV * 2 + DV * DK * 2 + (MODE != kModeRet ? DK * 4 : 0) <= kLdsBytes;
}
// Variants that are built: they fit in LDS, and linear attention with dk = 128
// runs with 64-token chunks (at 128 its walk kernel would spill registers).
template <int C, int DK, int DV, int MODE>
constexpr bool walk_supported() {
    return walk_fits<C, DK, DV, MODE>() && !(MODE == kModeLin && C == 128 && DK == 128);
}

template <int C, int DK, int DV, int MODE>
hipError_t launch_t(const SegArgs& a, hipStream_t stream) {
    if constexpr (!walk_supported<C, DK, DV, MODE>()) {
        return hipErrorInvalidConfiguration;
    } else {
    const long long bh = static_cast<long long>(a.B) * a.H;
    if (bh <= 0) return hipSuccess;
    if (bh * a.G > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.G > 1 && !a.ws_tr) {
        SegArgs sa = a;
        sa.scps = a.cps * (C / kStateBlock);
        // the state kernel is the same for both normalised retention modes
        constexpr int SMODE = (MODE == kModeGroup) ? kModeNorm : MODE;
        hipLaunchKernelGGL((seg_state_kernel<DK, DV, SMODE, false>), dim3(static_cast<unsigned>(bh * (a.G - 1) * a.pieces)),
                           dim3(kThreads), 0, stream, sa);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((seg_walk_kernel<C, DK, DV, MODE>), dim3(static_cast<unsigned>(bh * a.G)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
    }
}

template <int C, int MODE>
hipError_t launch_chunk(const SegArgs& a, int dk, int dv, hipStream_t stream) {
    if (dk == 64 && dv == 64) return launch_t<C, 64, 64, MODE>(a, stream);
    if (dk == 64 && dv == 128) return launch_t<C, 64, 128, MODE>(a, stream);
    if (dk == 128 && dv == 64) return launch_t<C, 128, 64, MODE>(a, stream);
    if (dk == 128 && dv == 128) return launch_t<C, 128, 128, MODE>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace seg
}  // namespace ret
