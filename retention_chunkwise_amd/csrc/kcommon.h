// kcommon.h -- device helpers shared by the libretention kernels (gfx950):
// bf16 conversions, MFMA wrappers, LDS transpose reads, range-checked buffer
// loads and stores, and LDS-DMA loads with explicit vector-memory waits.
#pragma once

#include <hip/hip_runtime.h>

namespace ret {
namespace kc {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

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

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, let lane L address 8 bytes M[L][0..3]; lane i receives
// {M[i/4 + 4m][i % 4] : m = 0..3}.  With lane L pointing at row r0 + L/4,
// columns c0 + 4 (L % 4) of a row-major bf16 tile, lane i therefore gets rows
// r0..r0+3 of column c0 + i: four consecutive tokens of one column, which is
// the MFMA operand layout for a contraction over tokens.
__device__ __forceinline__ u16x4 lds_tr4(const unsigned short* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(u16x4, r);
}

// Raw buffer access with hardware range checking: a resource covers exactly
// the valid bytes of one chunk, so loads past its end return zeros and stores
// past its end are dropped.  Offsets are 32-bit byte offsets.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    // word 3: 32-bit data format, the standard raw-buffer setting on gfx9-family parts
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, 0x00020000);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
    return uint4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, unsigned off, const u16x4& x) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, static_cast<int>(off), 0, 0);
}

__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, unsigned off, const f32x4& x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, static_cast<int>(off), 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding vector-memory operations (prefetch loads, output stores), which
// the kernels order themselves with wait_vmcnt.  The asm's memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS hazard self-check (builds with -DRET_DEBUG): a buffer that no wave may
// read any more until it is refilled is overwritten with all-ones words, a NaN
// in bf16 and in fp32, by every thread of the workgroup.  A read that a missing
// or misplaced barrier lets through then turns outputs into NaN, where a
// release build would read stale but plausible values.
#ifdef RET_DEBUG
__device__ __forceinline__ void lds_poison(void* p, int bytes) {
    for (int i = static_cast<int>(threadIdx.x) * 16; i < bytes; i += static_cast<int>(blockDim.x) * 16)
        *reinterpret_cast<uint4*>(static_cast<char*>(p) + i) = uint4{~0u, ~0u, ~0u, ~0u};
}
#endif

// Buffer resource words for the LDS-DMA loads (same layout as make_rsrc).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, int bytes) {
    const unsigned long long p = reinterpret_cast<unsigned long long>(base);
    u32x4 r;
    r[0] = static_cast<unsigned>(p);
    r[1] = static_cast<unsigned>(p >> 32) & 0xffffu;  // stride 0
    r[2] = static_cast<unsigned>(bytes);
    r[3] = 0x00020000u;
    return r;
}

// 16 bytes per lane from a range-checked buffer straight into LDS: lane l's
// data lands at LDS byte `lds_addr` + 16 l (lds_addr must be wave-uniform).
// Issued as inline asm on purpose: the compiler's own wait insertion treats
// any LDS-DMA as possibly aliasing every later LDS read and would wait for the
// prefetch right after issuing it.  The kernels wait for these loads
// explicitly (wait_vmcnt) before the barrier that precedes any read.  M0 is
// written here and nowhere else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const u32x4& rsrc, unsigned lds_addr, unsigned voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <typename T>
__device__ __forceinline__ unsigned lds_addr_of(const T* p) {
    typedef __attribute__((address_space(3))) const T lds_t;
    return static_cast<unsigned>(reinterpret_cast<unsigned long>((lds_t*)(p)));
}

// 16-byte unit swizzle of unpadded row-major bf16 tiles whose rows hold RU =
// 8 or 16 units (128 or 256 bytes).  The unit index of row r is XORed with
//   r & 15            (RU = 16)
//   (r >> 1) & 7      (RU = 8)
// Measured on gfx950 (64 four-byte banks): with it, 16-byte operand reads of
// 16 consecutive rows at one unit run at the speed of a contiguous read, and
// 8-byte transpose reads of 4 consecutive rows at two adjacent units run as
// fast as any swizzle tried (those reads are not bank-limited).
template <int RU>
__device__ __forceinline__ int swz_mask(int r) {
    static_assert(RU == 8 || RU == 16, "8 or 16 units per row");
    return (RU == 16) ? (r & 15) : ((r >> 1) & 7);
}

// Byte offset of logical unit u of row r in a tile with RU units per row.
template <int RU>
__device__ __forceinline__ int swz_byte(int r, int u) {
    return r * (RU * 16) + ((u ^ swz_mask<RU>(r)) << 4);
}

}  // namespace kc
}  // namespace ret
