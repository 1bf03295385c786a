// C ABI of the top-1 MoE gate: argument validation, workspace plan and launch order.
// The operations and their page citations are documented in include/moe_top1.h.
#include "moe_top1.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "moe_internal.hpp"

namespace moe {

static thread_local char g_err[512] = "";

static moe_status_t fail(moe_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

static moe_status_t hip_fail(hipError_t e, const char* what) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Number of d_W chunks P for T tokens (see expert_nchunks): about eight workgroups per compute
// unit once the output tiles of a chunk are counted (several rounds, so the last partial
// round is short), and chunks of at least MOE_DW_MIN_CHUNK tokens (MOE_DW_MIN_CHUNK_BIG in
// the fp32 large-T tiling, where fewer, longer chunks shrink the partials more than they cost
// the dW workgroups).  The chunk partials then stay within P x (H^2 + H) floats whatever the
// routing skew.  Depends only on (T, H, act), so results are reproducible for a shape.  The
// bf16 kernels get far fewer dW workgroups.  At T = 163,840, H = 512 (16 tiles per chunk, 2
// workgroups per CU, so 512 run at once), 320 plan 20 chunks (1 MB of fp32 partials each; 128
// took the reduce to 35 us): each of 8 balanced experts takes 3 chunks, 384 dW workgroups run in
// one round and the free slots start dX tiles.  512 planned 32, but experts on the rounding
// boundary take 4 or 5 chunks: 36 chunks, 576 workgroups, 64 of them in a second round (step
// 445 against 432 us; 448: 4 chunks each, 512 workgroups, 432 us; 384: 444 us; 256 and 192,
// chunks of 10,240 tokens: 464 and 440 us).
#ifndef MOE_DW_WORKGROUPS
#define MOE_DW_WORKGROUPS 2048
#endif
#ifndef MOE_DW_WORKGROUPS_BF16
#define MOE_DW_WORKGROUPS_BF16 320
#endif
// 256 x 256 d_W tiles (bf16 and large-T fp32 at H = 256, 512): one workgroup per compute unit,
// in a launch of their own, so the budget is one round of 256 workgroups.
#ifndef MOE_DW_WORKGROUPS_BIG
#define MOE_DW_WORKGROUPS_BIG 256
#endif
static int plan_chunks(int64_t T, int H, int NE, int act) {
    const bool f32 = act == MOE_DTYPE_F32;
    const int bt = f32 ? f32_dw_tile(T, H) : bf16_dw_tile(H);
    const int tiles_per_chunk = (H / bt) * (H / bt);
    const int64_t wg = bt == 256 ? MOE_DW_WORKGROUPS_BIG : (f32 ? MOE_DW_WORKGROUPS : MOE_DW_WORKGROUPS_BF16);
    int64_t pmax = (wg + tiles_per_chunk - 1) / tiles_per_chunk;
    // the 256 x 256 tiles run one round of one workgroup per compute unit: plan P so that even
    // the worst case of P + N_E chunks stays within the budget
    if (bt == 256) pmax = pmax - NE > 1 ? pmax - NE : 1;
    int64_t p = T / ((f32 && f32_big_tiles(T, H)) ? MOE_DW_MIN_CHUNK_BIG : MOE_DW_MIN_CHUNK);
    if (p > pmax) p = pmax;
    if (p < 1) p = 1;
    return (int)p;
}

Plan make_plan(int64_t T, int H, int NE, int act) {
    Plan p;
    p.T = T;
    p.H = H;
    p.NE = NE;
    p.act = act;
    p.n_rblk = (int)((T + kRouteTokens - 1) / kRouteTokens);
    p.n_ablk = (int)((T + kAuxTokens - 1) / kAuxTokens);
    if (H > 0) {
        p.chunks = plan_chunks(T, H, NE, act);
        p.n_chunk_max = p.chunks + NE;
    }
    size_t o = 0;
    p.off_hist = o;    o += align256((size_t)p.n_rblk * NE * 4);
    p.off_blkbase = o; o += align256((size_t)p.n_rblk * NE * 4);
    p.off_idx = o;     o += align256((size_t)T * 4);
    p.off_counts = o;  o += align256((size_t)NE * 4);
    p.off_offsets = o; o += align256((size_t)(NE + 1) * 4);
    p.off_paux = o;    o += align256((size_t)p.n_ablk * NE * 4);
    p.off_pdw = o;     o += align256((size_t)p.n_chunk_max * H * H * 4);
    p.off_pdb = o;     o += align256((size_t)p.n_chunk_max * H * 4);
    p.wt_bytes = (act == MOE_DTYPE_F32 && H > 0 && f32_dw_tile(T, H) == 256) ? (size_t)NE * H * H * 4 : 0;
    p.off_wt = o;      o += align256(p.wt_bytes);
    p.total = o;
    return p;
}

// ---------------------------------------------------------------- launch timer
static int g_timer_kernel = -1;
static hipEvent_t g_timer_start = nullptr, g_timer_stop = nullptr;

static ArmedEvents g_armed;
ArmedEvents& armed_events() { return g_armed; }

// The timed kernel's launch carries the events (launch_kernel); if the launcher made no
// launch, they are disarmed again and keep their earlier timestamps.
TimerScope::TimerScope(KernelId k, hipStream_t st) : s(st), on(g_timer_kernel == (int)k) {
    if (on) {
        g_armed.start = g_timer_start;
        g_armed.stop = g_timer_stop;
    }
}
TimerScope::~TimerScope() {
    if (on) g_armed.start = g_armed.stop = nullptr;
}

// ---------------------------------------------------------------- validation
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQ(ptr)                                                                              \
    do {                                                                                      \
        if (!(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s: required pointer '%s' is NULL", fn, #ptr); \
        if (!aligned16(ptr))                                                                  \
            return fail(MOE_ERR_INVALID_ARG, "%s: pointer '%s' is not 16-byte aligned", fn, #ptr); \
    } while (0)
#define OPT(ptr)                                                                              \
    do {                                                                                      \
        if ((ptr) && !aligned16(ptr))                                                         \
            return fail(MOE_ERR_INVALID_ARG, "%s: pointer '%s' is not 16-byte aligned", fn, #ptr); \
    } while (0)

static moe_status_t check_shape(const char* fn, int64_t B, int64_t NH, int64_t H, int64_t NE, int act,
                                bool has_h) {
    if (B <= 0 || NH <= 0 || NE <= 0 || (has_h && H <= 0))
        return fail(MOE_ERR_INVALID_ARG, "%s: sizes must be positive (B=%lld NH=%lld H=%lld NE=%lld)", fn,
                    (long long)B, (long long)NH, (long long)H, (long long)NE);
    if (NE > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "%s: N_E=%lld outside [1, 64]", fn, (long long)NE);
    if (has_h && !(H == 64 || H == 128 || H == 256 || H == 512))
        return fail(MOE_ERR_UNSUPPORTED, "%s: H=%lld not in {64, 128, 256, 512}", fn, (long long)H);
    if (act != MOE_DTYPE_F32 && act != MOE_DTYPE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, act);
    if (B > (int64_t)1 << 31 || NH > (int64_t)1 << 31)
        return fail(MOE_ERR_INVALID_ARG, "%s: B or N_H too large", fn);
    const int64_t T = B * NH;
    const int64_t w = has_h ? (H > NE ? H : NE) : NE;
    if (T >= ((int64_t)1 << 31) / w)
        return fail(MOE_ERR_INVALID_ARG, "%s: T * max(H, N_E) = %lld * %lld must be < 2^31", fn, (long long)T,
                    (long long)w);
    return MOE_OK;
}

static moe_status_t check_ws(const char* fn, const Plan& p, void* ws, size_t ws_bytes) {
    if (!ws) return fail(MOE_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, p.total);
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
    if (ws_bytes < p.total)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, p.total);
    return MOE_OK;
}

template <typename T>
static T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

#define LAUNCH(kid, expr, what)                       \
    do {                                              \
        hipError_t _e;                                \
        {                                             \
            TimerScope _ts(kid, s);                   \
            _e = (expr);                              \
        }                                             \
        if (_e != hipSuccess) return hip_fail(_e, what); \
    } while (0)

static moe_status_t do_route(const float* G, int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* perm,
                             const Plan& p, void* ws, hipStream_t s) {
    int32_t* hist = at<int32_t>(ws, p.off_hist);
    int32_t* blkbase = at<int32_t>(ws, p.off_blkbase);
    LAUNCH(K_ROUTE, launch_route(G, p.T, p.NE, idx, hist, p.n_rblk, s), "route");
    if (perm && scatter_scan_fits(p.n_rblk, p.NE)) {
        LAUNCH(K_SCATTER, launch_scatter_scan(idx, p.T, p.NE, hist, p.n_rblk, counts, offsets, perm, s),
               "scatter+scan");
        return MOE_OK;
    }
    LAUNCH(K_SCAN, launch_scan(hist, p.n_rblk, p.NE, blkbase, counts, offsets, s), "scan");
    if (perm) LAUNCH(K_SCATTER, launch_scatter(idx, p.T, p.NE, blkbase, perm, p.n_rblk, s), "scatter");
    return MOE_OK;
}

// ---------------------------------------------------------------- allocation-free forward
// The forward pass's scratch (routing histograms and block bases) in a file-scope device
// array instead of a caller's workspace.  Each device the library runs on holds its own copy
// of the array for the life of the process; its address on the current device is looked up
// once (hipGetSymbolAddress) at the first call there.  Every call on a device shares that
// device's array: calls that overlap on one device race.  The kernels write every scratch
// word they later read (one histogram row per routing block, then the block bases), so
// nothing needs clearing between calls.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;  // 8 MiB per device
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static moe_status_t scratch_on_current_device(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(MOE_ERR_HIP, "%s: scratch address is NULL", fn);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int st) {
    switch (st) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

const char* moe_kernel_name(int k) {
    static const char* names[K_COUNT] = {"route", "scan", "scatter", "fwd_gemm", "bwd_gemm",
                                         "reduce", "aux", "aux_final", "w_transpose", "lambda_update",
                                         "reduce_axis0", "collapse", "softmax_ce"};
    return (k >= 0 && k < K_COUNT) ? names[k] : nullptr;
}

moe_status_t moe_workspace_bytes(int64_t B, int64_t NH, int64_t H, int64_t NE, int act, size_t* bytes_out) {
    const char* fn = "moe_workspace_bytes";
    if (!bytes_out) return fail(MOE_ERR_INVALID_ARG, "%s: bytes_out is NULL", fn);
    moe_status_t st = check_shape(fn, B, NH, H, NE, act, true);
    if (st != MOE_OK) return st;
    *bytes_out = make_plan(B * NH, (int)H, (int)NE, act).total;
    return MOE_OK;
}

moe_status_t moe_set_launch_timer(int kernel_id, void* ev_start, void* ev_stop) {
    if (kernel_id < 0) {
        g_timer_kernel = -1;
        g_timer_start = g_timer_stop = nullptr;
        return MOE_OK;
    }
    if (kernel_id >= K_COUNT || !ev_start || !ev_stop)
        return fail(MOE_ERR_INVALID_ARG, "moe_set_launch_timer: bad kernel id or NULL event");
    g_timer_start = (hipEvent_t)ev_start;
    g_timer_stop = (hipEvent_t)ev_stop;
    g_timer_kernel = kernel_id;
    return MOE_OK;
}

moe_status_t moe_top1_route(const float* gate_logits, int32_t* expert_idx, int32_t* expert_counts,
                            int32_t* expert_offsets, int32_t* perm, int64_t B, int64_t NH, int64_t NE,
                            void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "moe_top1_route";
    moe_status_t st = check_shape(fn, B, NH, 0, NE, MOE_DTYPE_F32, false);
    if (st != MOE_OK) return st;
    REQ(gate_logits); REQ(expert_idx); REQ(expert_counts); REQ(expert_offsets); REQ(perm);
    // routing needs no H-dependent workspace; size it with the smallest H
    Plan p = make_plan(B * NH, 64, (int)NE, MOE_DTYPE_F32);
    size_t need = p.off_paux;  // hist + blkbase + idx + counts + offsets
    if (!workspace) return fail(MOE_ERR_WORKSPACE, "%s: workspace is NULL", fn);
    if (!aligned16(workspace)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
    if (workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
    return do_route(gate_logits, expert_idx, expert_counts, expert_offsets, perm, p, workspace,
                    (hipStream_t)stream);
}

// The forward GEMM once routing has formed offsets and perm.
static moe_status_t fwd_gemm_only(const void* fused_ctx, const void* W, const float* b, void* routed_ctx,
                                  const int32_t* expert_offsets, const int32_t* perm, const Plan& p, int act,
                                  hipStream_t s) {
    if (act == MOE_DTYPE_F32)
        LAUNCH(K_FWD_GEMM,
               launch_fwd_gemm_f32((const float*)fused_ctx, (const float*)W, b, (float*)routed_ctx,
                                   expert_offsets, perm, p.T, p.H, p.NE, s),
               "fwd gemm");
    else
        LAUNCH(K_FWD_GEMM,
               launch_fwd_gemm_bf16((const uint16_t*)fused_ctx, (const uint16_t*)W, b, (uint16_t*)routed_ctx,
                                    expert_offsets, perm, p.T, p.H, p.NE, s),
               "fwd gemm");
    return MOE_OK;
}

// Arguments of the forward pass checked (shape, pointers); nothing is launched.
static moe_status_t check_fwd_args(const char* fn, const void* fused_ctx, const float* gate_logits, const void* W,
                                   const float* b, const void* routed_ctx, const int32_t* expert_idx,
                                   const int32_t* expert_counts, const int32_t* expert_offsets, const int32_t* perm,
                                   int64_t B, int64_t NH, int64_t H, int64_t NE, int act) {
    moe_status_t st = check_shape(fn, B, NH, H, NE, act, true);
    if (st != MOE_OK) return st;
    REQ(fused_ctx); REQ(gate_logits); REQ(W); REQ(b); REQ(routed_ctx);
    REQ(expert_idx); REQ(expert_counts); REQ(expert_offsets); REQ(perm);
    return MOE_OK;
}

// The forward pass once its arguments are checked; it uses the routing sections of the
// workspace only (histograms and block bases: the plan's bytes below off_idx).
static moe_status_t fwd_launch(const void* fused_ctx, const float* gate_logits, const void* W, const float* b,
                               void* routed_ctx, int32_t* expert_idx, int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* perm, const Plan& p, int act, void* workspace, hipStream_t s) {
    if (act == MOE_DTYPE_F32 && fwd_gemm_f32_gather_fits(p.T, p.H, p.NE, p.n_rblk)) {
        // routing, then one forward launch that also forms perm, counts and offsets
        int32_t* hist = at<int32_t>(workspace, p.off_hist);
        LAUNCH(K_ROUTE, launch_route(gate_logits, p.T, p.NE, expert_idx, hist, p.n_rblk, s), "route");
        LAUNCH(K_FWD_GEMM,
               launch_fwd_gemm_f32_gather((const float*)fused_ctx, (const float*)W, b, (float*)routed_ctx, expert_idx,
                                          hist, p.n_rblk, expert_counts, expert_offsets, perm, p.T, p.H, p.NE,
                                          nullptr, s),
               "fwd gemm");
        return MOE_OK;
    }
    moe_status_t st = do_route(gate_logits, expert_idx, expert_counts, expert_offsets, perm, p, workspace, s);
    if (st != MOE_OK) return st;
    return fwd_gemm_only(fused_ctx, W, b, routed_ctx, expert_offsets, perm, p, act, s);
}

moe_status_t moe_top1_fwd(const void* fused_ctx, const float* gate_logits, const void* W, const float* b,
                          void* routed_ctx, int32_t* expert_idx, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* perm, int64_t B, int64_t NH, int64_t H,
                          int64_t NE, int act, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "moe_top1_fwd";
    moe_status_t st = check_fwd_args(fn, fused_ctx, gate_logits, W, b, routed_ctx, expert_idx, expert_counts,
                                     expert_offsets, perm, B, NH, H, NE, act);
    if (st != MOE_OK) return st;
    const Plan p = make_plan(B * NH, (int)H, (int)NE, act);
    if ((st = check_ws(fn, p, workspace, workspace_bytes)) != MOE_OK) return st;
    return fwd_launch(fused_ctx, gate_logits, W, b, routed_ctx, expert_idx, expert_counts, expert_offsets, perm, p,
                      act, workspace, (hipStream_t)stream);
}


moe_status_t moe_top1_fwd_noalloc(const void* fused_ctx, const float* gate_logits, const void* W, const float* b,
                                  void* routed_ctx, int32_t* expert_idx, int32_t* expert_counts,
                                  int32_t* expert_offsets, int32_t* perm, int64_t B, int64_t NH, int64_t H,
                                  int64_t NE, int act, void* stream) {
    const char* fn = "moe_top1_fwd_noalloc";
    moe_status_t st = check_fwd_args(fn, fused_ctx, gate_logits, W, b, routed_ctx, expert_idx, expert_counts,
                                     expert_offsets, perm, B, NH, H, NE, act);
    if (st != MOE_OK) return st;
    const Plan p = make_plan(B * NH, (int)H, (int)NE, act);
    if (p.off_idx > kNoAllocScratchBytes)
        return fail(MOE_ERR_WORKSPACE,
                    "%s: the routing scratch for ceil(T/256) * N_E = %lld histogram entries needs %zu bytes, more than "
                    "the %zu-byte device array; use moe_top1_fwd with a workspace",
                    fn, (long long)p.n_rblk * NE, p.off_idx, kNoAllocScratchBytes);
    void* ws = nullptr;
    if ((st = scratch_on_current_device(fn, &ws)) != MOE_OK) return st;
    return fwd_launch(fused_ctx, gate_logits, W, b, routed_ctx, expert_idx, expert_counts, expert_offsets, perm, p,
                      act, ws, (hipStream_t)stream);
}

static moe_status_t bwd_impl(const char* fn, const void* dy, int from_mean, const void* fused_ctx, const void* W,
                             const int32_t* expert_offsets, const int32_t* perm, void* d_fused_ctx, float* d_W,
                             float* d_b, int accumulate_dx, int64_t B, int64_t NH, int64_t H, int64_t NE, int act,
                             void* workspace, size_t workspace_bytes, void* stream) {
    moe_status_t st = check_shape(fn, B, NH, H, NE, act, true);
    if (st != MOE_OK) return st;
    REQ(dy); REQ(fused_ctx); REQ(W); REQ(expert_offsets); REQ(perm);
    REQ(d_fused_ctx); REQ(d_W); REQ(d_b);
    const Plan p = make_plan(B * NH, (int)H, (int)NE, act);
    if ((st = check_ws(fn, p, workspace, workspace_bytes)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    float* pdw = at<float>(workspace, p.off_pdw);
    float* pdb = at<float>(workspace, p.off_pdb);
    float* wt = at<float>(workspace, p.off_wt);
    if (from_mean && act == MOE_DTYPE_F32) {
        LAUNCH(K_BWD_GEMM,
               launch_bwd_gemm_f32_from_mean((const float*)dy, (const float*)fused_ctx, (const float*)W,
                                             (float*)d_fused_ctx, accumulate_dx, pdw, pdb, wt, expert_offsets, perm,
                                             p.T, p.H, p.NE, (int)NH, p.chunks, p.n_chunk_max, s),
               "bwd gemm (from mean)");
    } else if (from_mean) {
        LAUNCH(K_BWD_GEMM,
               launch_bwd_gemm_bf16_from_mean((const uint16_t*)dy, (const uint16_t*)fused_ctx, (const uint16_t*)W,
                                              (uint16_t*)d_fused_ctx, accumulate_dx, pdw, pdb, expert_offsets, perm,
                                              p.T, p.H, p.NE, (int)NH, p.chunks, p.n_chunk_max, s),
               "bwd gemm (from mean)");
    } else if (act == MOE_DTYPE_F32) {
        LAUNCH(K_BWD_GEMM,
               launch_bwd_gemm_f32((const float*)dy, (const float*)fused_ctx, (const float*)W, (float*)d_fused_ctx,
                                   accumulate_dx, pdw, pdb, wt, expert_offsets, perm, p.T, p.H, p.NE, p.chunks,
                                   p.n_chunk_max, s),
               "bwd gemm");
    } else {
        LAUNCH(K_BWD_GEMM,
               launch_bwd_gemm_bf16((const uint16_t*)dy, (const uint16_t*)fused_ctx, (const uint16_t*)W,
                                    (uint16_t*)d_fused_ctx,
                                    accumulate_dx, pdw, pdb, expert_offsets, perm, p.T, p.H, p.NE, p.chunks,
                                    p.n_chunk_max, s),
               "bwd gemm");
    }
    LAUNCH(K_REDUCE, launch_reduce_dw(pdw, pdb, expert_offsets, p.T, p.H, p.NE, p.chunks, d_W, d_b, s), "reduce");
    return MOE_OK;
}

moe_status_t moe_top1_bwd(const void* d_routed_ctx, const void* fused_ctx, const void* W,
                          const int32_t* expert_offsets, const int32_t* perm, void* d_fused_ctx, float* d_W,
                          float* d_b, int accumulate_dx, int64_t B, int64_t NH, int64_t H, int64_t NE, int act,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_impl("moe_top1_bwd", d_routed_ctx, 0, fused_ctx, W, expert_offsets, perm, d_fused_ctx, d_W, d_b,
                    accumulate_dx, B, NH, H, NE, act, workspace, workspace_bytes, stream);
}

moe_status_t moe_top1_bwd_from_mean(const void* d_ctx_mean, const void* fused_ctx, const void* W,
                                    const int32_t* expert_offsets, const int32_t* perm, void* d_fused_ctx, float* d_W,
                                    float* d_b, int accumulate_dx, int64_t B, int64_t NH, int64_t H, int64_t NE,
                                    int act, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_impl("moe_top1_bwd_from_mean", d_ctx_mean, 1, fused_ctx, W, expert_offsets, perm, d_fused_ctx, d_W,
                    d_b, accumulate_dx, B, NH, H, NE, act, workspace, workspace_bytes, stream);
}

static moe_status_t aux_impl(const char* fn, const float* gate_logits, const int32_t* expert_counts, float lambda,
                             const float* lambda_dev, float* loss, float* d_gate_logits, float* frac, float* mean_prob,
                             float* probs, int64_t B, int64_t NH, int64_t NE, void* workspace, size_t workspace_bytes,
                             void* stream) {
    moe_status_t st = check_shape(fn, B, NH, 0, NE, MOE_DTYPE_F32, false);
    if (st != MOE_OK) return st;
    REQ(gate_logits); OPT(expert_counts); REQ(loss); REQ(d_gate_logits);
    OPT(frac); OPT(mean_prob); OPT(probs);
    if (!lambda_dev && !isfinite(lambda)) return fail(MOE_ERR_INVALID_ARG, "%s: lambda is not finite", fn);
    Plan p = make_plan(B * NH, 64, (int)NE, MOE_DTYPE_F32);
    const size_t need = p.off_pdw;
    if (!workspace) return fail(MOE_ERR_WORKSPACE, "%s: workspace is NULL", fn);
    if (!aligned16(workspace)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
    if (workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    const int32_t* counts = expert_counts;
    if (!counts) {
        int32_t* c = at<int32_t>(workspace, p.off_counts);
        st = do_route(gate_logits, at<int32_t>(workspace, p.off_idx), c, at<int32_t>(workspace, p.off_offsets),
                      nullptr, p, workspace, s);
        if (st != MOE_OK) return st;
        counts = c;
    }
    float* part = at<float>(workspace, p.off_paux);
    LAUNCH(K_AUX,
           launch_aux_rows(gate_logits, counts, p.T, p.NE, lambda, lambda_dev, d_gate_logits, probs, part, p.n_ablk, s),
           "aux rows");
    LAUNCH(K_AUX_FINAL,
           launch_aux_final(part, counts, p.n_ablk, p.T, p.NE, lambda, lambda_dev, loss, frac, mean_prob, s),
           "aux final");
    return MOE_OK;
}

moe_status_t moe_aux_loss(const float* gate_logits, const int32_t* expert_counts, float lambda, float* loss,
                          float* d_gate_logits, float* frac, float* mean_prob, float* probs, int64_t B,
                          int64_t NH, int64_t NE, void* workspace, size_t workspace_bytes, void* stream) {
    return aux_impl("moe_aux_loss", gate_logits, expert_counts, lambda, nullptr, loss, d_gate_logits, frac, mean_prob,
                    probs, B, NH, NE, workspace, workspace_bytes, stream);
}

moe_status_t moe_aux_loss_lambda_dev(const float* gate_logits, const int32_t* expert_counts, const float* lambda_dev,
                                     float* loss, float* d_gate_logits, float* frac, float* mean_prob, float* probs,
                                     int64_t B, int64_t NH, int64_t NE, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    const char* fn = "moe_aux_loss_lambda_dev";
    if (!lambda_dev) return fail(MOE_ERR_INVALID_ARG, "%s: required pointer 'lambda_dev' is NULL", fn);
    return aux_impl(fn, gate_logits, expert_counts, 0.0f, lambda_dev, loss, d_gate_logits, frac, mean_prob, probs,
                    B, NH, NE, workspace, workspace_bytes, stream);
}

moe_status_t moe_top1_fwd_aux(const void* fused_ctx, const float* gate_logits, const void* W, const float* b,
                              void* routed_ctx, int32_t* expert_idx, int32_t* expert_counts, int32_t* expert_offsets,
                              int32_t* perm, float lambda, const float* lambda_dev, float* loss, float* d_gate_logits,
                              float* frac, float* mean_prob, float* probs, int64_t B, int64_t NH, int64_t H,
                              int64_t NE, int act, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "moe_top1_fwd_aux";
    moe_status_t st = check_shape(fn, B, NH, H, NE, act, true);
    if (st != MOE_OK) return st;
    REQ(fused_ctx); REQ(gate_logits); REQ(W); REQ(b); REQ(routed_ctx);
    REQ(expert_idx); REQ(expert_counts); REQ(expert_offsets); REQ(perm);
    REQ(loss); REQ(d_gate_logits); OPT(frac); OPT(mean_prob); OPT(probs);
    if (lambda_dev && ((uintptr_t)lambda_dev & 3u))
        return fail(MOE_ERR_INVALID_ARG, "%s: lambda_dev is not 4-byte aligned", fn);
    if (!lambda_dev && !isfinite(lambda)) return fail(MOE_ERR_INVALID_ARG, "%s: lambda is not finite", fn);
    const Plan p = make_plan(B * NH, (int)H, (int)NE, act);
    if ((st = check_ws(fn, p, workspace, workspace_bytes)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (act == MOE_DTYPE_F32 && NE <= kAuxFwdMaxExperts && p.n_ablk == p.n_rblk &&
        fwd_gemm_f32_gather_fits(p.T, p.H, p.NE, p.n_rblk)) {
        // two launches: routing (+ the softmax column sums), then the forward GEMM whose grid
        // also writes dG and the loss
        int32_t* hist = at<int32_t>(workspace, p.off_hist);
        float* part = at<float>(workspace, p.off_paux);
        LAUNCH(K_ROUTE, launch_route_part(gate_logits, p.T, p.NE, expert_idx, hist, part, p.n_rblk, s), "route");
        const AuxFwdArgs ax = {gate_logits, part, lambda, lambda_dev, d_gate_logits, probs, loss, frac, mean_prob,
                               p.n_ablk};
        LAUNCH(K_FWD_GEMM,
               launch_fwd_gemm_f32_gather((const float*)fused_ctx, (const float*)W, b, (float*)routed_ctx, expert_idx,
                                          hist, p.n_rblk, expert_counts, expert_offsets, perm, p.T, p.H, p.NE, &ax,
                                          s),
               "fwd gemm + aux");
        return MOE_OK;
    }
    if (NE <= kAuxScatterMaxExperts) {
        // routing with the softmax column sums, then the scatter (which knows the final counts)
        // with dG and, in one extra block, the loss; then the forward GEMM alone
        int32_t* hist = at<int32_t>(workspace, p.off_hist);
        int32_t* blkbase = at<int32_t>(workspace, p.off_blkbase);
        float* part = at<float>(workspace, p.off_paux);
        LAUNCH(K_ROUTE, launch_route_part(gate_logits, p.T, p.NE, expert_idx, hist, part, p.n_rblk, s), "route");
        const AuxFwdArgs ax = {gate_logits, part, lambda, lambda_dev, d_gate_logits, probs, loss, frac, mean_prob,
                               p.n_ablk};
        if (scatter_scan_fits(p.n_rblk, p.NE)) {
            LAUNCH(K_SCATTER,
                   launch_scatter_scan_aux(expert_idx, p.T, p.NE, hist, p.n_rblk, expert_counts, expert_offsets, perm,
                                           ax, s),
                   "scatter+scan + aux");
        } else {
            LAUNCH(K_SCAN, launch_scan(hist, p.n_rblk, p.NE, blkbase, expert_counts, expert_offsets, s), "scan");
            LAUNCH(K_SCATTER,
                   launch_scatter_aux(expert_idx, p.T, p.NE, blkbase, perm, expert_counts, p.n_rblk, ax, s),
                   "scatter + aux");
        }
        return fwd_gemm_only(fused_ctx, W, b, routed_ctx, expert_offsets, perm, p, act, s);
    }
    st = moe_top1_fwd(fused_ctx, gate_logits, W, b, routed_ctx, expert_idx, expert_counts, expert_offsets, perm, B, NH,
                      H, NE, act, workspace, workspace_bytes, stream);
    if (st != MOE_OK) return st;
    return aux_impl(fn, gate_logits, expert_counts, lambda, lambda_dev, loss, d_gate_logits, frac, mean_prob, probs, B,
                    NH, NE, workspace, workspace_bytes, stream);
}

moe_status_t moe_lambda_eff_update(const float* ent_ema, float lambda_floor, float lambda_max_extra,
                                   float entropy_target_frac, int64_t NE, float* lambda_eff, void* stream) {
    const char* fn = "moe_lambda_eff_update";
    if (!ent_ema) return fail(MOE_ERR_INVALID_ARG, "%s: required pointer 'ent_ema' is NULL", fn);
    if (!lambda_eff) return fail(MOE_ERR_INVALID_ARG, "%s: required pointer 'lambda_eff' is NULL", fn);
    if (((uintptr_t)ent_ema & 3u) || ((uintptr_t)lambda_eff & 3u))
        return fail(MOE_ERR_INVALID_ARG, "%s: pointers must be 4-byte aligned", fn);
    if (NE < 2 || NE > kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED, "%s: N_E=%lld outside [2, 64] (ln N_E must be positive)", fn, (long long)NE);
    if (!isfinite(lambda_floor) || !isfinite(lambda_max_extra) || !(entropy_target_frac > 0.0f) ||
        !isfinite(entropy_target_frac))
        return fail(MOE_ERR_INVALID_ARG, "%s: knobs must be finite and the target fraction positive", fn);
    hipStream_t s = (hipStream_t)stream;
    LAUNCH(K_LAMBDA,
           launch_lambda_eff(ent_ema, lambda_floor, lambda_max_extra, entropy_target_frac, (int)NE, lambda_eff, s),
           "lambda update");
    return MOE_OK;
}

// ---------------------------------------------------------------- reduce_axis0
static moe_status_t check_axis0(const char* fn, int64_t n_batch, int64_t n_tail) {
    if (n_batch <= 0 || n_tail <= 0)
        return fail(MOE_ERR_INVALID_ARG, "%s: n_batch and n_tail must be positive", fn);
    if (n_tail >= ((int64_t)1 << 31) || n_batch > ((int64_t)1 << 40) / n_tail)
        return fail(MOE_ERR_INVALID_ARG, "%s: n_batch * n_tail too large", fn);
    return MOE_OK;
}

static size_t axis0_ws(int64_t n_batch, int64_t n_tail) {
    const int64_t R = reduce_axis0_chunks(n_batch, n_tail, n_tail % 4 == 0);
    return R > 1 ? align256((size_t)R * n_tail * 4) : 0;
}

moe_status_t moe_reduce_axis0_workspace_bytes(int64_t n_batch, int64_t n_tail, size_t* bytes_out) {
    const char* fn = "moe_reduce_axis0_workspace_bytes";
    if (!bytes_out) return fail(MOE_ERR_INVALID_ARG, "%s: bytes_out is NULL", fn);
    moe_status_t st = check_axis0(fn, n_batch, n_tail);
    if (st != MOE_OK) return st;
    *bytes_out = axis0_ws(n_batch, n_tail);
    return MOE_OK;
}

moe_status_t moe_reduce_axis0(const float* in, int64_t n_batch, int64_t n_tail, float* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
    const char* fn = "moe_reduce_axis0";
    moe_status_t st = check_axis0(fn, n_batch, n_tail);
    if (st != MOE_OK) return st;
    const bool vec = n_tail % 4 == 0;
    if (!in || !out) return fail(MOE_ERR_INVALID_ARG, "%s: in and out must be non-NULL", fn);
    if (vec ? (!aligned16(in) || !aligned16(out)) : (((uintptr_t)in | (uintptr_t)out) & 3u))
        return fail(MOE_ERR_INVALID_ARG, "%s: in/out must be %d-byte aligned", fn, vec ? 16 : 4);
    const size_t need = axis0_ws(n_batch, n_tail);
    if (need > 0) {
        if (!workspace) return fail(MOE_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
        if (!aligned16(workspace)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
        if (workspace_bytes < need)
            return fail(MOE_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
    }
    hipStream_t s = (hipStream_t)stream;
    LAUNCH(K_REDUCE_AXIS0, launch_reduce_axis0(in, n_batch, n_tail, out, (float*)workspace, vec, s), "reduce_axis0");
    return MOE_OK;
}

// ---------------------------------------------------------------- horizon mean collapse
static moe_status_t collapse_impl(const char* fn, bool bwd, const void* in, void* out, int64_t B, int64_t NH,
                                  int64_t H, int act, void* stream) {
    if (B <= 0 || NH <= 0 || H <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: sizes must be positive", fn);
    if (act != MOE_DTYPE_F32 && act != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
    const int per = act == MOE_DTYPE_F32 ? 4 : 8;
    if (H % per != 0) return fail(MOE_ERR_UNSUPPORTED, "%s: H must be a multiple of %d", fn, per);
    if (NH > ((int64_t)1 << 20) || B * NH > ((int64_t)1 << 40) / H)
        return fail(MOE_ERR_INVALID_ARG, "%s: shape too large", fn);
    if (!in || !out) return fail(MOE_ERR_INVALID_ARG, "%s: in and out must be non-NULL", fn);
    if (!aligned16(in) || !aligned16(out)) return fail(MOE_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    hipStream_t s = (hipStream_t)stream;
    LAUNCH(K_COLLAPSE, launch_collapse(bwd, act, in, out, B, (int)NH, (int)H, s), "collapse");
    return MOE_OK;
}

moe_status_t moe_horizon_mean_collapse_fwd(const void* x, void* ctx_mean, int64_t B, int64_t NH, int64_t H, int act,
                                           void* stream) {
    return collapse_impl("moe_horizon_mean_collapse_fwd", false, x, ctx_mean, B, NH, H, act, stream);
}

moe_status_t moe_horizon_mean_collapse_bwd(const void* d_ctx_mean, void* d_x, int64_t B, int64_t NH, int64_t H,
                                           int act, void* stream) {
    return collapse_impl("moe_horizon_mean_collapse_bwd", true, d_ctx_mean, d_x, B, NH, H, act, stream);
}

// ---------------------------------------------------------------- softmax-CE head
moe_status_t moe_softmax_ce_grad(const float* logits, const int32_t* labels, float* grad, float* ce, int64_t B,
                                 int64_t NH, int64_t A, void* stream) {
    const char* fn = "moe_softmax_ce_grad";
    if (B <= 0 || NH <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: sizes must be positive", fn);
    if (A < 1 || A > 64) return fail(MOE_ERR_UNSUPPORTED, "%s: A=%lld outside [1, 64]", fn, (long long)A);
    if (B > ((int64_t)1 << 40) / NH) return fail(MOE_ERR_INVALID_ARG, "%s: shape too large", fn);
    if (!logits || !labels || !grad || !ce) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (((uintptr_t)logits | (uintptr_t)labels | (uintptr_t)grad | (uintptr_t)ce) & 3u)
        return fail(MOE_ERR_INVALID_ARG, "%s: pointers must be 4-byte aligned", fn);
    hipStream_t s = (hipStream_t)stream;
    LAUNCH(K_SOFTMAX_CE, launch_softmax_ce(logits, labels, B * NH, (int)A, B, grad, ce, s), "softmax-CE");
    return MOE_OK;
}

// ---------------------------------------------------------------- calibration probes
}  // extern "C"
namespace moe {  // peak_probe.hip
hipError_t launch_probe_mfma(int act, int64_t workgroups, int64_t iters, float* sink, int64_t* ticks,
                             hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
}  // namespace moe
extern "C" {

moe_status_t moe_probe_mfma(int act, int64_t workgroups, int64_t iters, float* sink, int64_t* ticks, void* stream) {
    const char* fn = "moe_probe_mfma";
    if (act != MOE_DTYPE_F32 && act != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, act);
    if (workgroups <= 0 || workgroups > (1 << 20) || iters <= 0)
        return fail(MOE_ERR_INVALID_ARG, "%s: workgroups must be in [1, 2^20] and iters positive", fn);
    if (!sink || !ticks) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (((uintptr_t)sink & 3u) || ((uintptr_t)ticks & 7u))
        return fail(MOE_ERR_INVALID_ARG, "%s: sink must be 4-byte and ticks 8-byte aligned", fn);
    const hipError_t e = launch_probe_mfma(act, workgroups, iters, sink, ticks, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "MFMA probe");
    return MOE_OK;
}

moe_status_t moe_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    const char* fn = "moe_probe_copy";
    if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned16(src) || !aligned16(dst)) return fail(MOE_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    if (bytes <= 0 || (bytes & 15) != 0) return fail(MOE_ERR_INVALID_ARG, "%s: bytes must be a positive multiple of 16", fn);
    const hipError_t e = launch_probe_copy(src, dst, bytes, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "copy probe");
    return MOE_OK;
}

}  // extern "C"
