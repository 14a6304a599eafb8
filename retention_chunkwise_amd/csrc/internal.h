// internal.h -- types and launcher declarations shared by the libretention
// translation units.  Not part of the public ABI (see include/retention.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ret {

// Largest head count a single call accepts.  Per-head log2(gamma) values travel
// in the kernel argument block, so the library needs no device buffer for them.
constexpr int kMaxHeads = 256;

// Arguments of the chunk-walk kernel (forward retention and linear attention).
struct WalkArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* final_state;  // may be null
    int B, H, T;
    int dv;              // full value width (the kernel handles one slice of it)
    int nslices;         // dv / (16 * NT)
    int xcd_remap;       // 1: spread (b, h) groups so their slices share an XCD
    float eps;           // linear attention only
    float log2g[kMaxHeads];
};

// Arguments of the recurrent decode-step kernel.
struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    float* state;
    void* out;
    int N, H;
    float gamma[kMaxHeads];
};

// Launchers (host).  They assume validated arguments and return a hipError_t.
hipError_t launch_walk(const WalkArgs& a, bool bf16, int chunk, int dk, int nt,
                       bool linattn, hipStream_t stream);
hipError_t launch_walk_ret_bf16(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream);
hipError_t launch_walk_ret_f32(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream);
hipError_t launch_walk_lin_bf16(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream);
hipError_t launch_walk_lin_f32(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, bool bf16, int dk, int dv,
                         hipStream_t stream);

// Choice of value-slice width (in 16-column MFMA tiles) for the chunk walk:
// the widest slice that still gives at least `target_groups` workgroups.
int choose_walk_nt(long long bh, int dv, int target_groups, bool bf16, int chunk, int dk);

}  // namespace ret
