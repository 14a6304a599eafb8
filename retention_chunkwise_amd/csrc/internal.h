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
    float* final_state;        // may be null
    const float* init_state;   // [B][H][dk][dv] state before token 0; null: zero
    const float* init_z;       // [B][H][dk] normaliser before token 0 (linear attention); null: zero
    float* final_z;            // [B][H][dk] normaliser after the last token (linear attention); may be null
    int B, H, T;
    int dv;              // full value width (the kernel handles one slice of it)
    int nslices;         // dv / (16 * NT)
    int xcd_remap;       // 1: spread (b, h) groups so their slices share an XCD
    int reverse;         // 1: walk the time-reversed sequence (token t at row T - 1 - t); fp32 only
    int G;               // segments per (b, h) (1: walk whole sequences); all but the last are full
    int cps;             // chunks per segment
    int seg_len;         // tokens per full segment (set by the launcher: cps * chunk)
    float* ws;           // [B*H][G-1][dk*dv (+ dk)] fp32 segment states, row-major; unused when G == 1
    int ws_tr;           // retention only: ws already holds the segment states of a walk over the same
                         // segments with key and value roles swapped (dv x dk, row-major); the state
                         // pass is skipped and the walk reads them transposed (ws is then only read)
    float eps;           // linear attention only
    float gn_eps;        // GroupNorm epsilon (normalised retention with GroupNorm only)
    float log2g[kMaxHeads];
};

// Arguments of the recurrent decode-step kernel (retention, or linear
// attention with the elu+1 feature map and its normaliser z).
struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    float* state;
    float* z;     // [N][H][dk], linear attention only
    void* out;
    int N, H;
    float eps;    // linear attention only
    float gamma[kMaxHeads];  // retention only
};

// Arguments of the segment-split forward (bf16; retention, or linear
// attention with the elu+1 feature map): seg_state_kernel then seg_walk_kernel.
struct SegArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* final_state;        // may be null
    const float* init_state;   // [B][H][dk][dv] state before token 0; null: zero
    const float* init_z;       // [B][H][dk] normaliser before token 0 (linear attention); null: zero
    float* final_z;            // [B][H][dk] normaliser after the last token (linear attention); may be null
    float* ws;           // [B*H][G-1][pieces][dk*dv (+ dk)] fp32 segment states (and normalisers);
                         // unused when G == 1
    int B, H, T;
    int G;               // segments per (b, h); every segment but the last is full
    int cps;             // chunks per segment
    int scps;            // state-kernel blocks per segment (set by the launcher)
    int pieces;          // state-kernel workgroups per segment (divides scps)
    float eps;           // linear attention only
    float gn_eps;        // GroupNorm epsilon (normalised retention with GroupNorm only)
    int ws_tr;           // retention only: ws already holds the segment states of a walk over the same
                         // segments with key and value roles swapped (shape dv x dk); the state pass
                         // is skipped and the walk reads them transposed (ws is then only read)
    const void* q2;      // fused backward walk only: the second query input (v), width dv
    void* out2;          // fused backward walk only: the second output (dk), width dk
    float log2g[kMaxHeads];
};

// Arguments of the gated linear attention walk (q, k, v, out fp32 or bf16; log-gates fp32).
struct GlaArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* lg;     // [B][H][T][dk] log-gates (finite, <= 0; values above 0 are taken as 0)
    void* out;
    float* final_state;  // may be null
    int B, H, T;
    int dv;
    int nslices;         // dv / (16 * NT)
    int G;               // segments per (b, h); all but the last are full
    int cps;             // chunks (64 tokens) per segment
    float* ws;           // [B*H][G-1][dk*dv + dk] segment states and log-gate totals; unused when G == 1
};

// Launchers (host).  They assume validated arguments and return a hipError_t.
hipError_t launch_walk(const WalkArgs& a, bool bf16, int chunk, int dk, int nt,
                       bool linattn, hipStream_t stream);
hipError_t launch_walk_ret_bf16(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream);
hipError_t launch_walk_ret_f32(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream);
hipError_t launch_walk_lin_bf16(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream);
hipError_t launch_walk_lin_f32(const WalkArgs& a, int chunk, int dk, int nt, hipStream_t stream);
// fp32 retention with the row-sum floor, and GroupNorm when `group` (value-slice walk).
hipError_t launch_walk_norm_f32(const WalkArgs& a, int chunk, int dk, int nt, bool group, hipStream_t stream);
// GroupNorm over each fp32 row of dv (64 or 128) values, in place.
hipError_t launch_group_norm_rows_f32(float* out, long long rows, int dv, float eps, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, bool bf16, int dk, int dv,
                         hipStream_t stream);
hipError_t launch_decode_lin(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t stream);

hipError_t launch_seg(const SegArgs& a, int chunk, int dk, int dv, bool linattn, hipStream_t stream);
hipError_t launch_seg_c64(const SegArgs& a, int dk, int dv, hipStream_t stream);
hipError_t launch_seg_c128(const SegArgs& a, int dk, int dv, hipStream_t stream);
hipError_t launch_seg_lin_c64(const SegArgs& a, int dk, int dv, hipStream_t stream);
hipError_t launch_seg_lin_c128(const SegArgs& a, int dk, int dv, hipStream_t stream);
// Retention with the row-sum floor, and GroupNorm when `group`.
hipError_t launch_seg_norm(const SegArgs& a, int chunk, int dk, int dv, bool group, hipStream_t stream);
hipError_t launch_seg_norm_c64(const SegArgs& a, int dk, int dv, bool group, hipStream_t stream);
hipError_t launch_seg_norm_c128(const SegArgs& a, int dk, int dv, bool group, hipStream_t stream);
// Fused reverse walk of the backward pass (64-token chunks): with a.q = k,
// a.q2 = v, a.k = q, a.v = dout it writes dv to a.out and dk to a.out2.
hipError_t launch_seg_bwd_kv(const SegArgs& a, int dk, int dv, hipStream_t stream);

// Segment count for the segment-split forward: enough (b, h, segment)
// workgroups to occupy the chip, at least `min_cps` chunks per segment.
// Returns G; *cps receives the chunks per segment (G = ceil(nch / cps)).
int choose_segments(long long bh, int nch, int target_groups, int min_cps, int max_g, int* cps);

// Choice of value-slice width (in 16-column MFMA tiles) for the chunk walk:
// the widest slice that still gives at least `target_groups` workgroups.
int choose_walk_nt(long long bh, int dv, int target_groups, bool bf16, int chunk, int dk);

// Gated linear attention: value-slice width (in 16-column tiles) and launcher.
int gla_choose_nt(long long bh, int dk, int dv);
// Workgroups the GLA walk aims for: two per CU where two fit.
int gla_target_groups(int dk, int nt);
hipError_t launch_gla(const GlaArgs& a, bool bf16, int dk, int nt, hipStream_t stream);

// Widest value slice of the segmented walk whose workgroup fits in LDS (the
// fewest recomputed Q K^T tiles); the segments provide the parallelism.
int choose_walk_nt_wide(int dv, bool bf16, int chunk, int dk, bool linattn);
bool walk_variant_fits(bool bf16, bool linattn, int chunk, int dk, int nt);
bool walk_fits_ret_bf16(int chunk, int dk, int nt);
bool walk_fits_ret_f32(int chunk, int dk, int nt);
bool walk_fits_lin_bf16(int chunk, int dk, int nt);
bool walk_fits_lin_f32(int chunk, int dk, int nt);

}  // namespace ret
