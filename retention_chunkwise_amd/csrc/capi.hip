// capi.hip -- the extern "C" entry points of libretention (include/retention.h).
//
// Every argument is validated on the host before anything is enqueued, so a
// rejected call has no side effect.  The library allocates no device memory:
// the segment-split forward paths take their workspace from the caller.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "../../include/retention.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return RET_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range& a, const Range& b) {
    return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

Range range(const char* name, const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, lo + bytes};
}

int dtype_size(int dtype) {
    if (dtype == RET_F32) return 4;
    if (dtype == RET_BF16) return 2;
    return 0;
}

// product of non-negative factors; false on overflow of size_t
bool mul_ok(size_t& acc, long long f) {
    if (f < 0) return false;
    if (f != 0 && acc > SIZE_MAX / static_cast<size_t>(f)) return false;
    acc *= static_cast<size_t>(f);
    return true;
}

int check_gamma(const char* fn, const float* gamma, int H, float* log2g) {
    for (int h = 0; h < H; ++h) {
        const float g = gamma[h];
        if (!(g > 0.f && g <= 1.f))  // also rejects NaN
            return fail(RET_ERR_GAMMA, "%s: gamma[%d] = %g is outside (0, 1]", fn, h, static_cast<double>(g));
        if (log2g) log2g[h] = static_cast<float>(log2(static_cast<double>(g)));
    }
    return RET_OK;
}

// ---- forward path selection
//
// The plan of a call (path, segment count, value-slice width, linear-attention
// chunk) is a function of its arguments, unless the calling thread has set a
// plan override (retention_set_plan_override), which tests and tuning sweeps
// use to force both paths and many segment counts on the same inputs.  No
// override changes results beyond rounding.
enum class FwdPath { kSlice, kSegment };

struct PlanOverride {
    int path = RET_PATH_AUTO;  // RET_PATH_*
    int segments = 0;          // 0: automatic
    int walk_nt = 0;           // 0: automatic; else a narrower value slice (16-column tiles), slice path
    int lin_chunk = 0;         // 0: automatic; else 64 or 128, bf16 linear attention on the segment path
};
thread_local PlanOverride g_over;

FwdPath choose_fwd_path(int dtype) {
    const bool seg_ok = dtype == RET_BF16;
    if (g_over.path == RET_PATH_SLICE) return FwdPath::kSlice;
    return seg_ok ? FwdPath::kSegment : FwdPath::kSlice;
}

// Plan of a forward call: the path, the segment count G, chunks per segment,
// state-kernel workgroups per segment (segment path), the value-slice width
// (value-slice path), and the workspace they need: (G - 1) * pieces partial
// states per (b, h), none when G == 1.
struct SegPlan {
    FwdPath path = FwdPath::kSegment;
    int chunk = 64;
    int G = 1, cps = 1, pieces = 1, nt = 1;
    size_t ws_bytes = 0;
};

// Segment count fixed by the plan override (false: not fixed).
bool forced_segments(int nch, SegPlan* p) {
    const int forced = g_over.segments;
    if (forced <= 0) return false;
    const int g = (forced < nch) ? forced : (nch > 0 ? nch : 1);
    p->cps = (nch > 0) ? (nch + g - 1) / g : 1;
    p->G = (nch > 0) ? (nch + p->cps - 1) / p->cps : 1;
    return true;
}

bool set_ws_bytes(long long bh, int dk, int dv, bool linattn, SegPlan* p) {
    p->ws_bytes = 0;
    if (p->G > 1) {
        size_t n = 4;
        const long long slot = static_cast<long long>(dk) * dv + (linattn ? dk : 0);
        if (!mul_ok(n, bh) || !mul_ok(n, p->G - 1) || !mul_ok(n, p->pieces) || !mul_ok(n, slot)) return false;
        p->ws_bytes = n;
    }
    return true;
}

// Value-slice path: fp32 walks segments with the widest value slice that
// fits in LDS (Q K^T computed once per segment chunk, the segments give the
// parallelism); a bf16 walk on this path (only when forced) keeps whole
// sequences and narrow slices unless a segment count is forced too.
bool plan_slices(long long bh, int T, int chunk, int dk, int dv, bool linattn, bool bf16, SegPlan* p) {
    p->path = FwdPath::kSlice;
    p->chunk = chunk;
    p->pieces = 1;
    const int nch = (T + chunk - 1) / chunk;
    const bool forced = forced_segments(nch, p);
    if (!bf16 || forced) {
        p->nt = ret::choose_walk_nt_wide(dv, bf16, chunk, dk, linattn);
        const int want = g_over.walk_nt;  // override: a narrower slice, if that variant fits
        if (want > 0 && want < p->nt && (dv / 16) % want == 0 && ret::walk_variant_fits(bf16, linattn, chunk, dk, want))
            p->nt = want;
        if (!forced) {
            p->G = ret::choose_segments(bh * (dv / (16 * p->nt)), nch, 256, 2, 16, &p->cps);
            // plain fp32 retention: the widest slice fills a CU's LDS; with one
            // workgroup per CU or fewer, halve the slice so that two share each CU at
            // the same segment count ([4, 8, 2048, 64]: 37.4 us against 39.5 us).
            // The normalised and linear-attention walks keep whole rows per slice.
            if (!bf16 && !linattn && want == 0 && p->nt >= 2 && bh * (dv / (16 * p->nt)) * p->G <= 256 &&
                ret::walk_variant_fits(bf16, linattn, chunk, dk, p->nt / 2))
                p->nt /= 2;
        }
        // the segment-state kernel addresses one segment's K and V with 32-bit byte offsets:
        // very long sequences take more segments, until a segment's K and V each stay under 2 GiB
        const long long row = static_cast<long long>(dk > dv ? dk : dv) * (bf16 ? 2 : 4);
        while (p->G > 1 && static_cast<long long>(p->cps) * chunk * row >= (1LL << 31)) {
            const int g = p->G + 1;
            p->cps = (nch + g - 1) / g;
            p->G = (nch + p->cps - 1) / p->cps;
        }
    } else {
        p->nt = ret::choose_walk_nt(bh, dv, 256, bf16, chunk, dk);
        p->G = 1;
        p->cps = nch > 0 ? nch : 1;
    }
    return set_ws_bytes(bh, dk, dv, linattn, p);
}

bool plan_segments(long long bh, int T, int chunk, int dk, int dv, bool linattn, SegPlan* p) {
    p->path = FwdPath::kSegment;
    p->chunk = chunk;
    const int nch = (T + chunk - 1) / chunk;
    if (!forced_segments(nch, p)) p->G = ret::choose_segments(bh, nch, 256, 4, 16, &p->cps);
    // state-kernel workgroups per segment: enough to occupy the chip in one
    // round, dividing the segment's 64-token blocks evenly, at most 16 partial
    // states per (b, h) (the walk sums up to that many states on entry)
    const int sblocks = p->cps * (chunk / 64);
    const long long sgroups = bh * (p->G - 1);
    int pieces = (sgroups > 0 && sgroups < 256) ? static_cast<int>(256 / sgroups) : 1;
    if (p->G > 1 && pieces > 16 / (p->G - 1)) pieces = 16 / (p->G - 1);
    if (pieces > sblocks) pieces = sblocks;
    if (pieces < 1) pieces = 1;
    while (pieces > 1 && sblocks % pieces != 0) --pieces;
    p->pieces = pieces;
    return set_ws_bytes(bh, dk, dv, linattn, p);
}

// Internal chunk of the linear-attention forward: bf16 segments use 128
// tokens (64 when dk = 128, where 128 would spill registers); the fp32 walk
// uses 64 (wider value slices fit in LDS); a forced bf16 slice walk 128.
int linattn_chunk(int dk, FwdPath path, bool bf16) {
    if (path == FwdPath::kSegment) {
        const int want = g_over.lin_chunk;  // override: 64 or 128 (128 only with dk = 64)
        if (want == 64 || (want == 128 && dk == 64)) return want;
        return dk == 128 ? 64 : 128;
    }
    return bf16 ? 128 : 64;
}

// The plan a forward call with these arguments will use.
bool plan_fwd(long long bh, int T, int chunk, int dk, int dv, bool linattn, int dtype, SegPlan* p) {
    const FwdPath path = choose_fwd_path(dtype);
    const bool bf16 = dtype == RET_BF16;
    if (linattn) chunk = linattn_chunk(dk, path, bf16);
    if (path == FwdPath::kSegment) return plan_segments(bh, T, chunk, dk, dv, linattn, p);
    return plan_slices(bh, T, chunk, dk, dv, linattn, bf16, p);
}

// Checks the caller's workspace against a plan (before anything is enqueued).
int check_workspace(const char* fn, const SegPlan& p, const void* workspace, size_t ws_bytes,
                    std::initializer_list<Range> others) {
    if (p.ws_bytes == 0) return RET_OK;
    if (!workspace || ws_bytes < p.ws_bytes)
        return fail(RET_ERR_WORKSPACE, "%s: needs a workspace of %zu bytes (got %zu%s)", fn, p.ws_bytes, ws_bytes,
                    workspace ? "" : ", NULL");
    if (!aligned16(workspace)) return fail(RET_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
    const Range rw = range("workspace", workspace, p.ws_bytes);
    for (const Range& o : others)
        if (overlap(rw, o)) return fail(RET_ERR_ALIAS, "%s: workspace overlaps %s", fn, o.name);
    return RET_OK;
}

// State pointers of a forward call: entering token 0 and after the last token
// (each may be null; the normalisers are linear attention only).
struct FwdState {
    const float* init_state = nullptr;
    const float* init_z = nullptr;
    float* final_state = nullptr;
    float* final_z = nullptr;
};

// Launches the segment-split forward (bf16) with a checked plan and workspace.
hipError_t launch_segment_path(const SegPlan& plan, const void* q, const void* k, const void* v, void* out,
                               const FwdState& fst, void* workspace, const float* log2g, float eps, int B, int H,
                               int T, int chunk, int dk, int dv, bool linattn, hipStream_t st,
                               bool ws_transposed = false) {
    ret::SegArgs sa{};
    sa.G = plan.G;
    sa.cps = plan.cps;
    sa.pieces = plan.pieces;
    sa.q = q; sa.k = k; sa.v = v; sa.out = out;
    sa.final_state = fst.final_state; sa.init_state = fst.init_state;
    sa.init_z = fst.init_z; sa.final_z = fst.final_z;
    sa.ws = plan.ws_bytes ? static_cast<float*>(workspace) : nullptr;
    sa.B = B; sa.H = H; sa.T = T; sa.eps = eps;
    sa.ws_tr = ws_transposed ? 1 : 0;
    if (log2g) memcpy(sa.log2g, log2g, sizeof(sa.log2g));
    return ret::launch_seg(sa, chunk, dk, dv, linattn, st);
}

// Plan of one walk of the backward pass: bf16 takes the segment path (its dk
// and dv come from the fused reverse walk), fp32 the value-slice path.
bool plan_bwd_walk(long long bh, int T, int chunk, int dk, int dv, int dtype, SegPlan* p) {
    if (dtype == RET_BF16) return plan_segments(bh, T, chunk, dk, dv, false, p);
    return plan_slices(bh, T, chunk, dk, dv, false, false, p);
}

// The walks of the backward pass: dq = fwd(dout, v, k) with widths (dv, dk)
// (plans[0]); dk = reversed fwd(v, dout, q) with widths (dv, dk) (plans[1])
// and dv = reversed fwd(k, q, dout) with widths (dk, dv) (plans[2]).  bf16
// computes dk and dv in one fused reverse walk of 64-token chunks over the
// plan of the dv walk (plans[1] = plans[2]).  They run one after another on
// one stream (dv, dk or the fused walk, then dq) and share the workspace,
// which must hold the largest plan.
bool plan_bwd(long long bh, int T, int chunk, int dk, int dv, int dtype, SegPlan plans[3], size_t* ws_max) {
    if (!plan_bwd_walk(bh, T, chunk, dv, dk, dtype, &plans[0])) return false;
    if (dtype == RET_BF16) {
        if (!plan_segments(bh, T, 64, dk, dv, false, &plans[2])) return false;
        plans[1] = plans[2];
    } else {
        plans[1] = plans[0];
        if (!plan_bwd_walk(bh, T, chunk, dk, dv, dtype, &plans[2])) return false;
    }
    *ws_max = plans[0].ws_bytes > plans[2].ws_bytes ? plans[0].ws_bytes : plans[2].ws_bytes;
    return true;
}

// Launches the value-slice walk (and its segment-state kernel) with a checked
// plan and workspace.
hipError_t launch_slice_path(const SegPlan& plan, const void* q, const void* k, const void* v, void* out,
                             const FwdState& fst, void* workspace, const float* log2g, float eps, int B, int H,
                             int T, int dk, int dv, bool bf16, bool linattn, hipStream_t st, bool reverse = false,
                             bool ws_transposed = false) {
    ret::WalkArgs a{};
    a.reverse = reverse ? 1 : 0;
    a.ws_tr = ws_transposed ? 1 : 0;
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.final_state = fst.final_state; a.init_state = fst.init_state;
    a.init_z = fst.init_z; a.final_z = fst.final_z;
    a.B = B; a.H = H; a.T = T; a.dv = dv; a.nslices = dv / (16 * plan.nt); a.eps = eps;
    a.G = plan.G; a.cps = plan.cps;
    a.ws = plan.ws_bytes ? static_cast<float*>(workspace) : nullptr;
    if (log2g) memcpy(a.log2g, log2g, sizeof(a.log2g));
    return ret::launch_walk(a, bf16, plan.chunk, dk, plan.nt, linattn, st);
}

// Plan of the gated linear attention walk: 64-token chunks, the widest value
// slice, and enough segments to occupy the chip (at least 2 chunks each).
bool plan_gla(long long bh, int T, int dk, int dv, SegPlan* p) {
    p->chunk = 64;
    p->pieces = 1;
    p->nt = ret::gla_choose_nt(bh, dk, dv);
    const int nch = (T + 63) / 64;
    if (!forced_segments(nch, p))
        p->G = ret::choose_segments(bh * (dv / (16 * p->nt)), nch, ret::gla_target_groups(dk, p->nt), 2, 16, &p->cps);
    return set_ws_bytes(bh, dk, dv, true, p);
}

// Chunk of the normalised walk: with dk = dv = 128 the 128-token walk and its
// normaliser exceed the LDS, so it runs 64-token chunks (same result).
int norm_chunk(int chunk, int dk, int dv) { return (chunk == 128 && dk == 128 && dv == 128) ? 64 : chunk; }

// Plan of a normalised forward: the bf16 segment walk, or the fp32 value-slice
// walk (a normaliser slot travels with each segment state on both).
bool plan_norm(long long bh, int T, int chunk, int dk, int dv, int dtype, SegPlan* p) {
    if (dtype == RET_BF16) return plan_segments(bh, T, norm_chunk(chunk, dk, dv), dk, dv, true, p);
    return plan_slices(bh, T, chunk, dk, dv, true, false, p);
}

}  // namespace

extern "C" {

const char* retention_last_error(void) { return g_err; }

size_t retention_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
    if (B <= 0 || H < 1 || T < 0 || (chunk != 64 && chunk != 128) || (dk != 64 && dk != 128) ||
        (dv != 64 && dv != 128) || !dtype_size(dtype))
        return 0;
    SegPlan plan;
    if (!plan_fwd(static_cast<long long>(B) * H, T, chunk, dk, dv, false, dtype, &plan)) return 0;
    return plan.ws_bytes;
}

size_t linear_attn_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype) {
    if (B <= 0 || H < 1 || T < 0 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128) || !dtype_size(dtype))
        return 0;
    SegPlan plan;
    if (!plan_fwd(static_cast<long long>(B) * H, T, 64, dk, dv, true, dtype, &plan)) return 0;
    return plan.ws_bytes;
}



size_t gla_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype) {
    if (B <= 0 || H < 1 || T < 0 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128) || !dtype_size(dtype)) return 0;
    SegPlan plan;
    if (!plan_gla(static_cast<long long>(B) * H, T, dk, dv, &plan)) return 0;
    return plan.ws_bytes;
}

size_t retention_fwd_normalized_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
    if (B <= 0 || H < 1 || T < 0 || (chunk != 64 && chunk != 128) || (dk != 64 && dk != 128) ||
        (dv != 64 && dv != 128) || (dtype != RET_BF16 && dtype != RET_F32))
        return 0;
    SegPlan plan;
    if (!plan_norm(static_cast<long long>(B) * H, T, chunk, dk, dv, dtype, &plan)) return 0;
    return plan.ws_bytes;
}

size_t retention_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
    if (B <= 0 || H < 1 || T < 0 || (chunk != 64 && chunk != 128) || (dk != 64 && dk != 128) ||
        (dv != 64 && dv != 128) || !dtype_size(dtype))
        return 0;
    SegPlan plans[3];
    size_t n = 0;
    if (!plan_bwd(static_cast<long long>(B) * H, T, chunk, dk, dv, dtype, plans, &n)) return 0;
    return n;
}

int retention_abi_version(void) { return RET_ABI_VERSION; }

int retention_set_plan_override(int fwd_path, int segments, int walk_nt, int lin_chunk) {
    const char* fn = "retention_set_plan_override";
    if (fwd_path != RET_PATH_AUTO && fwd_path != RET_PATH_SLICE && fwd_path != RET_PATH_SEGMENT)
        return fail(RET_ERR_SHAPE, "%s: unknown path %d", fn, fwd_path);
    if (segments < 0 || segments > 65536)
        return fail(RET_ERR_SHAPE, "%s: segments must be 0..65536 (got %d)", fn, segments);
    if (walk_nt != 0 && walk_nt != 1 && walk_nt != 2 && walk_nt != 4 && walk_nt != 8)
        return fail(RET_ERR_SHAPE, "%s: walk_nt must be 0, 1, 2, 4 or 8 (got %d)", fn, walk_nt);
    if (lin_chunk != 0 && lin_chunk != 64 && lin_chunk != 128)
        return fail(RET_ERR_CHUNK, "%s: lin_chunk must be 0, 64 or 128 (got %d)", fn, lin_chunk);
    g_over.path = fwd_path;
    g_over.segments = segments;
    g_over.walk_nt = walk_nt;
    g_over.lin_chunk = lin_chunk;
    return ok();
}

}  // extern "C"

namespace {

// Checks an optional fp32 state tensor of `bytes` bytes: 16-byte aligned and
// overlapping none of `others`.
int check_state_arg(const char* fn, const char* name, const void* p, size_t bytes, std::initializer_list<Range> others) {
    if (!p) return RET_OK;
    if (!aligned16(p)) return fail(RET_ERR_ALIGN, "%s: %s must be 16-byte aligned", fn, name);
    const Range r = range(name, p, bytes);
    for (const Range& o : others)
        if (overlap(r, o)) return fail(RET_ERR_ALIAS, "%s: %s overlaps %s", fn, name, o.name);
    return RET_OK;
}

}  // namespace

// ---- allocation-free forward: the segment states live in a device array of
// the library, not in a caller workspace.  Each GPU the library runs on holds
// its own copy from the first use until the process ends; every call on that
// GPU shares it, so calls that overlap in time on one GPU race.  The segment
// states are written before they are read, so nothing needs clearing between
// calls.
constexpr size_t kScratchBytes = static_cast<size_t>(RET_NOALLOC_MAX_WORKSPACE);
static_assert(kScratchBytes == (size_t{32} << 20), "the header states 32 MiB");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the device that runs `stream` (looked up once
// per device, with that device current).  The array's host-side name is a
// stand-in, not a device address: kernels get this pointer instead.
int scratch_for(const char* fn, hipStream_t stream, void** ptr) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: no device for the stream: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices) return fail(RET_ERR_HIP, "%s: device %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return fail(RET_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(RET_ERR_HIP, "%s: hipSetDevice(%d) failed: %s", fn, dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) static_cast<void>(hipSetDevice(cur));  // the address is known; restoring is best effort
        if (e != hipSuccess || !p)
            return fail(RET_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed: %s", fn, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return RET_OK;
}

// Shared by retention_fwd, retention_fwd_from_state and retention_fwd_noalloc
// (use_scratch: the workspace is the library's device array, not the caller's).
int ret_fwd_impl(const char* fn, const void* q, const void* k, const void* v, const float* gamma, int chunk,
                 const float* initial_state, void* out, float* final_state, int B, int H, int T, int dk, int dv,
                 int dtype, void* workspace, size_t ws_bytes, void* stream, bool use_scratch = false) {
    if (!gamma) return fail(RET_ERR_NULL, "%s: gamma must be non-NULL", fn);
    const int esz = dtype_size(dtype);
    if (!esz) return fail(RET_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (chunk != 64 && chunk != 128)
        return fail(RET_ERR_CHUNK, "%s: chunk must be 64 or 128 (got %d)", fn, chunk);
    if (B < 0 || T < 0 || H < 1 || H > ret::kMaxHeads)
        return fail(RET_ERR_SHAPE, "%s: need B >= 0, T >= 0, 1 <= H <= %d (got B=%d H=%d T=%d)", fn,
                    ret::kMaxHeads, B, H, T);
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
        return fail(RET_ERR_SHAPE, "%s: dk and dv must each be 64 or 128 (got %d, %d)", fn, dk, dv);
    size_t nqk = esz, nv = esz, ns = 4;
    if (!mul_ok(nqk, B) || !mul_ok(nqk, H) || !mul_ok(nqk, T) || !mul_ok(nqk, dk) ||
        !mul_ok(nv, B) || !mul_ok(nv, H) || !mul_ok(nv, T) || !mul_ok(nv, dv) ||
        !mul_ok(ns, B) || !mul_ok(ns, H) || !mul_ok(ns, dk) || !mul_ok(ns, dv))
        return fail(RET_ERR_SHAPE, "%s: tensor sizes overflow", fn);
    if (nqk > 0 && (!q || !k || !v || !out))
        return fail(RET_ERR_NULL, "%s: q, k, v and out must be non-NULL", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(RET_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    ret::WalkArgs a{};
    int rc = check_gamma(fn, gamma, H, a.log2g);
    if (rc) return rc;
    const Range rq = range("q", q, nqk), rk = range("k", k, nqk), rv = range("v", v, nv);
    const Range ro = range("out", out, nv);
    const Range none{"", 0, 0};
    for (const Range& in : {rq, rk, rv})
        if (overlap(ro, in)) return fail(RET_ERR_ALIAS, "%s: out overlaps %s", fn, in.name);
    const Range ri = initial_state ? range("initial_state", initial_state, ns) : none;
    if ((rc = check_state_arg(fn, "final_state", final_state, ns, {rq, rk, rv, ro, ri}))) return rc;
    if ((rc = check_state_arg(fn, "initial_state", initial_state, ns, {ro}))) return rc;
    if (B == 0) return ok();
    const long long bh = static_cast<long long>(B) * H;
    hipStream_t st = static_cast<hipStream_t>(stream);
    FwdState fst;
    fst.init_state = initial_state;
    fst.final_state = final_state;
    SegPlan plan;
    if (!plan_fwd(bh, T, chunk, dk, dv, false, dtype, &plan))
        return fail(RET_ERR_SHAPE, "%s: workspace size overflows", fn);
    if (use_scratch && plan.ws_bytes > 0) {
        if (plan.ws_bytes > kScratchBytes)
            return fail(RET_ERR_WORKSPACE,
                        "%s: these sizes need %zu bytes of segment states, more than the library's %zu-byte device "
                        "array; call retention_fwd with a workspace instead",
                        fn, plan.ws_bytes, kScratchBytes);
        if ((rc = scratch_for(fn, st, &workspace))) return rc;
        ws_bytes = kScratchBytes;
    }
    rc = check_workspace(fn, plan, workspace, ws_bytes,
                         {rq, rk, rv, ro, final_state ? range("final_state", final_state, ns) : none, ri});
    if (rc) return rc;
    const hipError_t e =
        plan.path == FwdPath::kSegment
            ? launch_segment_path(plan, q, k, v, out, fst, workspace, a.log2g, 0.f, B, H, T, chunk, dk, dv, false, st)
            : launch_slice_path(plan, q, k, v, out, fst, workspace, a.log2g, 0.f, B, H, T, dk, dv,
                                dtype == RET_BF16, false, st);
    if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

// Shared by linear_attn_fwd and linear_attn_fwd_from_state.
int lin_fwd_impl(const char* fn, const void* q, const void* k, const void* v, int phi, const float* initial_S,
                 const float* initial_z, void* out, float* final_S, float* final_z, int B, int H, int T, int dk,
                 int dv, int dtype, float eps, void* workspace, size_t ws_bytes, void* stream) {
    const int esz = dtype_size(dtype);
    if (!esz) return fail(RET_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (phi != RET_PHI_ELU1) return fail(RET_ERR_PHI, "%s: unknown feature map %d", fn, phi);
    if (!(eps >= 0.f) || isinf(eps)) return fail(RET_ERR_SHAPE, "%s: eps must be finite and >= 0", fn);
    if (B < 0 || T < 0 || H < 1)
        return fail(RET_ERR_SHAPE, "%s: need B >= 0, T >= 0, H >= 1 (got B=%d H=%d T=%d)", fn, B, H, T);
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
        return fail(RET_ERR_SHAPE, "%s: dk and dv must each be 64 or 128 (got %d, %d)", fn, dk, dv);
    size_t nqk = esz, nv = esz, ns = 4, nz = 4;
    if (!mul_ok(nqk, B) || !mul_ok(nqk, H) || !mul_ok(nqk, T) || !mul_ok(nqk, dk) ||
        !mul_ok(nv, B) || !mul_ok(nv, H) || !mul_ok(nv, T) || !mul_ok(nv, dv) ||
        !mul_ok(ns, B) || !mul_ok(ns, H) || !mul_ok(ns, dk) || !mul_ok(ns, dv) ||
        !mul_ok(nz, B) || !mul_ok(nz, H) || !mul_ok(nz, dk))
        return fail(RET_ERR_SHAPE, "%s: tensor sizes overflow", fn);
    if (nqk > 0 && (!q || !k || !v || !out))
        return fail(RET_ERR_NULL, "%s: q, k, v and out must be non-NULL", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(RET_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    const Range rq = range("q", q, nqk), rk = range("k", k, nqk), rv = range("v", v, nv);
    const Range ro = range("out", out, nv);
    const Range none{"", 0, 0};
    for (const Range& in : {rq, rk, rv})
        if (overlap(ro, in)) return fail(RET_ERR_ALIAS, "%s: out overlaps %s", fn, in.name);
    const Range riS = initial_S ? range("initial_S", initial_S, ns) : none;
    const Range riz = initial_z ? range("initial_z", initial_z, nz) : none;
    const Range rfS = final_S ? range("final_S", final_S, ns) : none;
    int rc;
    if ((rc = check_state_arg(fn, "final_S", final_S, ns, {rq, rk, rv, ro, riS, riz}))) return rc;
    if ((rc = check_state_arg(fn, "final_z", final_z, nz, {rq, rk, rv, ro, riS, riz, rfS}))) return rc;
    if ((rc = check_state_arg(fn, "initial_S", initial_S, ns, {ro}))) return rc;
    if ((rc = check_state_arg(fn, "initial_z", initial_z, nz, {ro}))) return rc;
    if (B == 0) return ok();
    const long long bh = static_cast<long long>(B) * H;
    hipStream_t st = static_cast<hipStream_t>(stream);
    FwdState fst;
    fst.init_state = initial_S;
    fst.init_z = initial_z;
    fst.final_state = final_S;
    fst.final_z = final_z;
    SegPlan plan;
    if (!plan_fwd(bh, T, 64, dk, dv, true, dtype, &plan)) return fail(RET_ERR_SHAPE, "%s: workspace size overflows", fn);
    const Range rfz = final_z ? range("final_z", final_z, nz) : none;
    rc = check_workspace(fn, plan, workspace, ws_bytes, {rq, rk, rv, ro, riS, riz, rfS, rfz});
    if (rc) return rc;
    const hipError_t e =
        plan.path == FwdPath::kSegment
            ? launch_segment_path(plan, q, k, v, out, fst, workspace, nullptr, eps, B, H, T, plan.chunk, dk, dv,
                                  true, st)
            : launch_slice_path(plan, q, k, v, out, fst, workspace, nullptr, eps, B, H, T, dk, dv,
                                dtype == RET_BF16, true, st);
    if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

// Shared argument checks of the two decode steps.  z is the normaliser of the
// linear-attention step (null for retention).
int decode_checks(const char* fn, const void* q, const void* k, const void* v, const float* state, const float* z,
                  bool lin, const void* out, int N, int H, int dk, int dv, int dtype) {
    const int esz = dtype_size(dtype);
    if (!esz) return fail(RET_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
    const int hmax = lin ? 0x7fffffff : ret::kMaxHeads;
    if (N < 0 || H < 1 || H > hmax)
        return fail(RET_ERR_SHAPE, "%s: need N >= 0, 1 <= H <= %d (got N=%d H=%d)", fn, hmax, N, H);
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
        return fail(RET_ERR_SHAPE, "%s: dk and dv must each be 64 or 128 (got %d, %d)", fn, dk, dv);
    size_t nqk = esz, nv = esz, ns = 4, nz = 4;
    if (!mul_ok(nqk, N) || !mul_ok(nqk, H) || !mul_ok(nqk, dk) ||
        !mul_ok(nv, N) || !mul_ok(nv, H) || !mul_ok(nv, dv) ||
        !mul_ok(ns, N) || !mul_ok(ns, H) || !mul_ok(ns, dk) || !mul_ok(ns, dv) ||
        !mul_ok(nz, N) || !mul_ok(nz, H) || !mul_ok(nz, dk))
        return fail(RET_ERR_SHAPE, "%s: tensor sizes overflow", fn);
    if (nqk > 0 && (!q || !k || !v || !state || !out || (lin && !z)))
        return fail(RET_ERR_NULL, lin ? "%s: q, k, v, S, z and out must be non-NULL"
                                      : "%s: q, k, v, state and out must be non-NULL", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state) || !aligned16(out) ||
        (lin && !aligned16(z)))
        return fail(RET_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    const char* sname = lin ? "S" : "state";
    const Range rq = range("q", q, nqk), rk = range("k", k, nqk), rv = range("v", v, nv);
    const Range rs = range(sname, state, ns), ro = range("out", out, nv);
    const Range rz = lin ? range("z", z, nz) : Range{"", 0, 0};
    for (const Range& in : {rq, rk, rv}) {
        if (overlap(rs, in)) return fail(RET_ERR_ALIAS, "%s: %s overlaps %s", fn, sname, in.name);
        if (overlap(ro, in)) return fail(RET_ERR_ALIAS, "%s: out overlaps %s", fn, in.name);
        if (overlap(rz, in)) return fail(RET_ERR_ALIAS, "%s: z overlaps %s", fn, in.name);
    }
    if (overlap(ro, rs)) return fail(RET_ERR_ALIAS, "%s: out overlaps %s", fn, sname);
    if (overlap(rz, rs)) return fail(RET_ERR_ALIAS, "%s: z overlaps S", fn);
    if (overlap(rz, ro)) return fail(RET_ERR_ALIAS, "%s: z overlaps out", fn);
    return RET_OK;
}

// retention_bwd, and retention_bwd_from_fwd when fn_fwd_ws is set: the dq walk
// then reads the forward's segment states instead of running its own state pass.
int bwd_impl(const char* fn, const void* q, const void* k, const void* v, const float* gamma, int chunk,
             const void* dout, const void* fwd_ws, size_t fwd_ws_bytes, bool with_fwd, void* dq, void* dk, void* dv,
             int B, int H, int T, int d_k, int d_v, int dtype, void* workspace, size_t ws_bytes, void* stream) {
    if (!gamma) return fail(RET_ERR_NULL, "%s: gamma must be non-NULL", fn);
    const int esz = dtype_size(dtype);
    if (!esz) return fail(RET_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (chunk != 64 && chunk != 128) return fail(RET_ERR_CHUNK, "%s: chunk must be 64 or 128 (got %d)", fn, chunk);
    if (B < 0 || T < 0 || H < 1 || H > ret::kMaxHeads)
        return fail(RET_ERR_SHAPE, "%s: need B >= 0, T >= 0, 1 <= H <= %d (got B=%d H=%d T=%d)", fn, ret::kMaxHeads, B,
                    H, T);
    if ((d_k != 64 && d_k != 128) || (d_v != 64 && d_v != 128))
        return fail(RET_ERR_SHAPE, "%s: dk and dv must each be 64 or 128 (got %d, %d)", fn, d_k, d_v);
    size_t nqk = esz, nv = esz;
    if (!mul_ok(nqk, B) || !mul_ok(nqk, H) || !mul_ok(nqk, T) || !mul_ok(nqk, d_k) ||
        !mul_ok(nv, B) || !mul_ok(nv, H) || !mul_ok(nv, T) || !mul_ok(nv, d_v))
        return fail(RET_ERR_SHAPE, "%s: tensor sizes overflow", fn);
    if (nqk > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv))
        return fail(RET_ERR_NULL, "%s: q, k, v, dout, dq, dk and dv must be non-NULL", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv))
        return fail(RET_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    float log2g[ret::kMaxHeads] = {};
    int rc = check_gamma(fn, gamma, H, log2g);
    if (rc) return rc;
    const Range rq = range("q", q, nqk), rk = range("k", k, nqk), rv = range("v", v, nv), rdo = range("dout", dout, nv);
    const Range rdq = range("dq", dq, nqk), rdk = range("dk", dk, nqk), rdv = range("dv", dv, nv);
    for (const Range& o : {rdq, rdk, rdv}) {
        for (const Range& in : {rq, rk, rv, rdo})
            if (overlap(o, in)) return fail(RET_ERR_ALIAS, "%s: %s overlaps %s", fn, o.name, in.name);
    }
    if (overlap(rdq, rdk) || overlap(rdq, rdv) || overlap(rdk, rdv))
        return fail(RET_ERR_ALIAS, "%s: the gradient outputs overlap", fn);
    if (B == 0) return ok();
    const long long bh = static_cast<long long>(B) * H;
    SegPlan plans[3];
    size_t need = 0;
    if (!plan_bwd(bh, T, chunk, d_k, d_v, dtype, plans, &need))
        return fail(RET_ERR_SHAPE, "%s: workspace size overflows", fn);
    SegPlan wplan;
    wplan.ws_bytes = need;
    rc = check_workspace(fn, wplan, workspace, ws_bytes, {rq, rk, rv, rdo, rdq, rdk, rdv});
    if (rc) return rc;
    // The forward's segment states, if it left any: Sum gamma^.. k v^T per segment, the transposes
    // of the dq walk's (keys v, values k) over the same segments.
    bool dq_shares = false;
    if (with_fwd) {
        SegPlan fplan;
        if (!plan_fwd(bh, T, chunk, d_k, d_v, false, dtype, &fplan))
            return fail(RET_ERR_SHAPE, "%s: workspace size overflows", fn);
        if (fplan.ws_bytes > 0) {
            if (!fwd_ws || fwd_ws_bytes < fplan.ws_bytes)
                return fail(RET_ERR_WORKSPACE, "%s: the forward's workspace must hold %zu bytes (got %zu%s)", fn,
                            fplan.ws_bytes, fwd_ws_bytes, fwd_ws ? "" : ", NULL");
            if (!aligned16(fwd_ws)) return fail(RET_ERR_ALIGN, "%s: fwd_workspace must be 16-byte aligned", fn);
            const Range rf = range("fwd_workspace", fwd_ws, fplan.ws_bytes);
            for (const Range& o : {rdq, rdk, rdv, range("workspace", workspace, need)})
                if (overlap(rf, o)) return fail(RET_ERR_ALIAS, "%s: fwd_workspace overlaps %s", fn, o.name);
            // the forward's plan must be the one the dq walk uses (it is, unless a plan
            // override changed between the calls; then the dq walk runs its own state pass)
            dq_shares = fplan.path == plans[0].path && fplan.G == plans[0].G && fplan.cps == plans[0].cps &&
                        fplan.chunk == plans[0].chunk &&
                        (fplan.path == FwdPath::kSlice || fplan.pieces == plans[0].pieces);
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const FwdState none;
    // (query input, key input, value input, output, key width, value width, reversed)
    struct Walk {
        const void *a, *b, *c;
        void* o;
        int wk, wv;
        bool rev;
    };
    // fp32: dv first; its segment states sum q_s dout_s^T, the transpose of what the dk walk
    // needs (dout_s q_s^T over the same reversed segments), so the dk walk reads them
    // transposed instead of running its own state pass
    const Walk walks[3] = {{k, q, dout, dv, d_k, d_v, true}, {v, dout, q, dk, d_v, d_k, true},
                           {dout, v, k, dq, d_v, d_k, false}};
    const SegPlan* wplans[3] = {&plans[2], &plans[1], &plans[0]};
    const bool share = plans[1].path == plans[2].path && plans[1].G == plans[2].G && plans[1].cps == plans[2].cps &&
                       plans[1].chunk == plans[2].chunk &&
                       (plans[1].path == FwdPath::kSlice || plans[1].pieces == plans[2].pieces);
    const bool fused = dtype == RET_BF16;
    if (fused) {
        // dk and dv from one reverse walk: queries k (for dv) and v (for dk), keys and
        // values q and dout
        ret::SegArgs sa{};
        sa.G = plans[2].G;
        sa.cps = plans[2].cps;
        sa.pieces = plans[2].pieces;
        sa.q = k; sa.k = q; sa.v = dout; sa.out = dv;
        sa.q2 = v; sa.out2 = dk;
        sa.ws = plans[2].ws_bytes ? static_cast<float*>(workspace) : nullptr;
        sa.B = B; sa.H = H; sa.T = T;
        memcpy(sa.log2g, log2g, sizeof(sa.log2g));
        const hipError_t e = ret::launch_seg_bwd_kv(sa, d_k, d_v, st);
        if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    }
    for (int i = fused ? 2 : 0; i < 3; ++i) {
        const Walk& w = walks[i];
        const SegPlan& pl = *wplans[i];
        const bool tr = (i == 1 && share) || (i == 2 && dq_shares);
        void* ws = (i == 2 && dq_shares) ? const_cast<void*>(fwd_ws) : workspace;  // only read when tr
        // the segment path runs only the forward-time dq walk here (bf16 dk and dv come
        // from the fused walk); the reversed walks of fp32 take the value-slice path
        if (pl.path == FwdPath::kSegment && w.rev)
            return fail(RET_ERR_HIP, "%s: no time-reversed segment walk for this plan", fn);
        const hipError_t e =
            pl.path == FwdPath::kSegment
                ? launch_segment_path(pl, w.a, w.b, w.c, w.o, none, ws, log2g, 0.f, B, H, T, chunk, w.wk,
                                      w.wv, false, st, tr)
                : launch_slice_path(pl, w.a, w.b, w.c, w.o, none, ws, log2g, 0.f, B, H, T, w.wk, w.wv,
                                    false, false, st, w.rev, tr);
        if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    }
    return ok();
}

}  // namespace

extern "C" {

int retention_fwd(const void* q, const void* k, const void* v, const float* gamma, int chunk,
                  void* out, float* final_state, int B, int H, int T, int dk, int dv, int dtype,
                  void* workspace, size_t ws_bytes, void* stream) {
    return ret_fwd_impl("retention_fwd", q, k, v, gamma, chunk, nullptr, out, final_state, B, H, T, dk, dv, dtype,
                        workspace, ws_bytes, stream);
}

int retention_fwd_noalloc(const void* q, const void* k, const void* v, const float* gamma, int chunk, void* out,
                          float* final_state, int B, int H, int T, int dk, int dv, int dtype, void* stream) {
    return ret_fwd_impl("retention_fwd_noalloc", q, k, v, gamma, chunk, nullptr, out, final_state, B, H, T, dk, dv,
                        dtype, nullptr, 0, stream, true);
}

int retention_fwd_from_state(const void* q, const void* k, const void* v, const float* gamma, int chunk,
                             const float* initial_state, void* out, float* final_state, int B, int H, int T,
                             int dk, int dv, int dtype, void* workspace, size_t ws_bytes, void* stream) {
    return ret_fwd_impl("retention_fwd_from_state", q, k, v, gamma, chunk, initial_state, out, final_state, B, H,
                        T, dk, dv, dtype, workspace, ws_bytes, stream);
}

int retention_fwd_normalized(const void* q, const void* k, const void* v, const float* gamma, int chunk, int norm,
                             float eps, void* out, int B, int H, int T, int dk, int dv, int dtype, void* workspace,
                             size_t ws_bytes, void* stream) {
    const char* fn = "retention_fwd_normalized";
    if (!gamma) return fail(RET_ERR_NULL, "%s: gamma must be non-NULL", fn);
    const int esz = dtype_size(dtype);
    if (!esz) return fail(RET_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (norm != RET_NORM_ROWSUM && norm != RET_NORM_GROUP)
        return fail(RET_ERR_SHAPE, "%s: norm must be RET_NORM_ROWSUM or RET_NORM_GROUP (got %d)", fn, norm);
    if (!(eps >= 0.f) || isinf(eps)) return fail(RET_ERR_SHAPE, "%s: eps must be finite and >= 0", fn);
    // a row of equal values (all-zero queries, say) has variance 0: GroupNorm needs eps > 0
    if (norm == RET_NORM_GROUP && !(eps > 0.f))
        return fail(RET_ERR_SHAPE, "%s: GroupNorm needs eps > 0 (got %g)", fn, static_cast<double>(eps));
    if (chunk != 64 && chunk != 128) return fail(RET_ERR_CHUNK, "%s: chunk must be 64 or 128 (got %d)", fn, chunk);
    if (B < 0 || T < 0 || H < 1 || H > ret::kMaxHeads)
        return fail(RET_ERR_SHAPE, "%s: need B >= 0, T >= 0, 1 <= H <= %d (got B=%d H=%d T=%d)", fn, ret::kMaxHeads, B,
                    H, T);
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
        return fail(RET_ERR_SHAPE, "%s: dk and dv must each be 64 or 128 (got %d, %d)", fn, dk, dv);
    size_t nqk = esz, nv = esz;
    if (!mul_ok(nqk, B) || !mul_ok(nqk, H) || !mul_ok(nqk, T) || !mul_ok(nqk, dk) ||
        !mul_ok(nv, B) || !mul_ok(nv, H) || !mul_ok(nv, T) || !mul_ok(nv, dv))
        return fail(RET_ERR_SHAPE, "%s: tensor sizes overflow", fn);
    if (nqk > 0 && (!q || !k || !v || !out)) return fail(RET_ERR_NULL, "%s: q, k, v and out must be non-NULL", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(RET_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    float log2g[ret::kMaxHeads] = {};
    int rc = check_gamma(fn, gamma, H, log2g);
    if (rc) return rc;
    const Range rq = range("q", q, nqk), rk = range("k", k, nqk), rv = range("v", v, nv), ro = range("out", out, nv);
    for (const Range& in : {rq, rk, rv})
        if (overlap(ro, in)) return fail(RET_ERR_ALIAS, "%s: out overlaps %s", fn, in.name);
    SegPlan plan;
    if (!plan_norm(static_cast<long long>(B) * H, T, chunk, dk, dv, dtype, &plan))
        return fail(RET_ERR_SHAPE, "%s: workspace size overflows", fn);
    if (B == 0) return ok();
    if ((rc = check_workspace(fn, plan, workspace, ws_bytes, {rq, rk, rv, ro}))) return rc;
    if (dtype == RET_F32) {
        ret::WalkArgs a{};
        a.q = q; a.k = k; a.v = v; a.out = out;
        a.B = B; a.H = H; a.T = T; a.dv = dv; a.nslices = dv / (16 * plan.nt); a.gn_eps = eps;
        a.G = plan.G; a.cps = plan.cps;
        a.ws = plan.ws_bytes ? static_cast<float*>(workspace) : nullptr;
        memcpy(a.log2g, log2g, sizeof(a.log2g));
        // GroupNorm is fused where one workgroup holds whole rows; where the walk splits a
        // row over value slices it applies the floor, and a row pass standardises in place
        const bool group = norm == RET_NORM_GROUP, fused = plan.nt * 16 == dv;
        hipError_t e = ret::launch_walk_norm_f32(a, plan.chunk, dk, plan.nt, group && fused,
                                                 static_cast<hipStream_t>(stream));
        if (e == hipSuccess && group && !fused)
            e = ret::launch_group_norm_rows_f32(static_cast<float*>(out), static_cast<long long>(B) * H * T, dv, eps,
                                                static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
        return ok();
    }
    chunk = plan.chunk;
    ret::SegArgs sa{};
    sa.G = plan.G; sa.cps = plan.cps; sa.pieces = plan.pieces;
    sa.q = q; sa.k = k; sa.v = v; sa.out = out;
    sa.ws = plan.ws_bytes ? static_cast<float*>(workspace) : nullptr;
    sa.B = B; sa.H = H; sa.T = T; sa.gn_eps = eps;
    memcpy(sa.log2g, log2g, sizeof(sa.log2g));
    const hipError_t e = ret::launch_seg_norm(sa, chunk, dk, dv, norm == RET_NORM_GROUP, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int retention_bwd(const void* q, const void* k, const void* v, const float* gamma, int chunk, const void* dout,
                  void* dq, void* dk, void* dv, int B, int H, int T, int d_k, int d_v, int dtype, void* workspace,
                  size_t ws_bytes, void* stream) {
    return bwd_impl("retention_bwd", q, k, v, gamma, chunk, dout, nullptr, 0, false, dq, dk, dv, B, H, T, d_k, d_v,
                    dtype, workspace, ws_bytes, stream);
}

int retention_bwd_from_fwd(const void* q, const void* k, const void* v, const float* gamma, int chunk,
                           const void* dout, const void* fwd_workspace, size_t fwd_ws_bytes, void* dq, void* dk,
                           void* dv, int B, int H, int T, int d_k, int d_v, int dtype, void* workspace,
                           size_t ws_bytes, void* stream) {
    return bwd_impl("retention_bwd_from_fwd", q, k, v, gamma, chunk, dout, fwd_workspace, fwd_ws_bytes, true, dq, dk,
                    dv, B, H, T, d_k, d_v, dtype, workspace, ws_bytes, stream);
}

int retention_decode_step(const void* q, const void* k, const void* v, const float* gamma,
                          float* state, void* out, int N, int H, int dk, int dv, int dtype,
                          void* stream) {
    const char* fn = "retention_decode_step";
    if (!gamma) return fail(RET_ERR_NULL, "%s: gamma must be non-NULL", fn);
    int rc = decode_checks(fn, q, k, v, state, nullptr, false, out, N, H, dk, dv, dtype);
    if (rc) return rc;
    ret::DecodeArgs a{};
    if ((rc = check_gamma(fn, gamma, H, nullptr))) return rc;
    for (int h = 0; h < H; ++h) a.gamma[h] = gamma[h];
    if (N == 0) return ok();
    a.q = q; a.k = k; a.v = v; a.state = state; a.out = out; a.N = N; a.H = H;
    const hipError_t e = ret::launch_decode(a, dtype == RET_BF16, dk, dv, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int linear_attn_fwd(const void* q, const void* k, const void* v, int phi, void* out, int B, int H,
                    int T, int dk, int dv, int dtype, float eps, void* workspace, size_t ws_bytes,
                    void* stream) {
    return lin_fwd_impl("linear_attn_fwd", q, k, v, phi, nullptr, nullptr, out, nullptr, nullptr, B, H, T, dk, dv,
                        dtype, eps, workspace, ws_bytes, stream);
}

int linear_attn_fwd_from_state(const void* q, const void* k, const void* v, int phi, const float* initial_S,
                               const float* initial_z, void* out, float* final_S, float* final_z, int B, int H,
                               int T, int dk, int dv, int dtype, float eps, void* workspace, size_t ws_bytes,
                               void* stream) {
    return lin_fwd_impl("linear_attn_fwd_from_state", q, k, v, phi, initial_S, initial_z, out, final_S, final_z,
                        B, H, T, dk, dv, dtype, eps, workspace, ws_bytes, stream);
}

int gla_fwd(const void* q, const void* k, const void* v, const float* log_gate, void* out, float* final_state, int B,
            int H, int T, int dk, int dv, int dtype, void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "gla_fwd";
    const int esz = dtype_size(dtype);
    if (!esz) return fail(RET_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (B < 0 || T < 0 || H < 1)
        return fail(RET_ERR_SHAPE, "%s: need B >= 0, T >= 0, H >= 1 (got B=%d H=%d T=%d)", fn, B, H, T);
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
        return fail(RET_ERR_SHAPE, "%s: dk and dv must each be 64 or 128 (got %d, %d)", fn, dk, dv);
    size_t nqk = esz, ng = 4, nv = esz, ns = 4;
    if (!mul_ok(nqk, B) || !mul_ok(nqk, H) || !mul_ok(nqk, T) || !mul_ok(nqk, dk) ||
        !mul_ok(ng, B) || !mul_ok(ng, H) || !mul_ok(ng, T) || !mul_ok(ng, dk) ||
        !mul_ok(nv, B) || !mul_ok(nv, H) || !mul_ok(nv, T) || !mul_ok(nv, dv) ||
        !mul_ok(ns, B) || !mul_ok(ns, H) || !mul_ok(ns, dk) || !mul_ok(ns, dv))
        return fail(RET_ERR_SHAPE, "%s: tensor sizes overflow", fn);
    if (nqk > 0 && (!q || !k || !v || !log_gate || !out))
        return fail(RET_ERR_NULL, "%s: q, k, v, log_gate and out must be non-NULL", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_gate) || !aligned16(out))
        return fail(RET_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    const Range rq = range("q", q, nqk), rk = range("k", k, nqk), rv = range("v", v, nv);
    const Range rg = range("log_gate", log_gate, ng), ro = range("out", out, nv);
    for (const Range& in : {rq, rk, rv, rg})
        if (overlap(ro, in)) return fail(RET_ERR_ALIAS, "%s: out overlaps %s", fn, in.name);
    int rc;
    if ((rc = check_state_arg(fn, "final_state", final_state, ns, {rq, rk, rv, rg, ro}))) return rc;
    if (B == 0) return ok();
    SegPlan plan;
    if (!plan_gla(static_cast<long long>(B) * H, T, dk, dv, &plan)) return fail(RET_ERR_SHAPE, "%s: workspace size overflows", fn);
    if ((rc = check_workspace(fn, plan, workspace, ws_bytes,
                              {rq, rk, rv, rg, ro, final_state ? range("final_state", final_state, ns) : Range{"", 0, 0}})))
        return rc;
    ret::GlaArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.lg = log_gate; a.out = out; a.final_state = final_state;
    a.B = B; a.H = H; a.T = T; a.dv = dv;
    const int nt = plan.nt;
    a.nslices = dv / (16 * nt);
    a.G = plan.G; a.cps = plan.cps;
    a.ws = plan.ws_bytes ? static_cast<float*>(workspace) : nullptr;
    const hipError_t e = ret::launch_gla(a, dtype == RET_BF16, dk, nt, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int linear_attn_decode_step(const void* q, const void* k, const void* v, int phi, float* S, float* z, void* out,
                            int N, int H, int dk, int dv, int dtype, float eps, void* stream) {
    const char* fn = "linear_attn_decode_step";
    if (phi != RET_PHI_ELU1) return fail(RET_ERR_PHI, "%s: unknown feature map %d", fn, phi);
    if (!(eps >= 0.f) || isinf(eps)) return fail(RET_ERR_SHAPE, "%s: eps must be finite and >= 0", fn);
    const int rc = decode_checks(fn, q, k, v, S, z, true, out, N, H, dk, dv, dtype);
    if (rc) return rc;
    if (N == 0) return ok();
    ret::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.state = S; a.z = z; a.out = out; a.N = N; a.H = H; a.eps = eps;
    const hipError_t e = ret::launch_decode_lin(a, dtype == RET_BF16, dk, dv, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RET_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // extern "C"
