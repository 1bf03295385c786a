// C ABI of the top-1 MoE gate: argument validation, workspace plan and launch order.
// The operations and their page citations are documented in include/moe_top1.h.
#include "moe_top1.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

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
// round is short), and chunks of at least 128 tokens.  The
// chunk partials then stay within P x (H^2 + H) floats whatever the routing skew.  Depends
// only on (T, H), so results are reproducible for a shape.
#ifndef MOE_DW_WORKGROUPS
#define MOE_DW_WORKGROUPS 2048
#endif
#ifndef MOE_DW_MIN_CHUNK
#define MOE_DW_MIN_CHUNK 128
#endif
static int plan_chunks(int64_t T, int H) {
    const int bt = (H >= 128) ? 128 : 64;
    const int tiles_per_chunk = (H / bt) * (H / bt);
    const int64_t pmax = (MOE_DW_WORKGROUPS + tiles_per_chunk - 1) / tiles_per_chunk;
    int64_t p = T / MOE_DW_MIN_CHUNK;
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
        p.chunks = plan_chunks(T, H);
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
    p.off_wt = o;      o += (act == MOE_DTYPE_BF16) ? align256((size_t)NE * H * H * 2) : 0;
    p.total = o;
    return p;
}

// ---------------------------------------------------------------- launch timer
static int g_timer_kernel = -1;
static hipEvent_t g_timer_start = nullptr, g_timer_stop = nullptr;

TimerScope::TimerScope(KernelId k, hipStream_t st) : s(st), on(g_timer_kernel == (int)k) {
    if (on) (void)hipEventRecord(g_timer_start, s);
}
TimerScope::~TimerScope() {
    if (on) (void)hipEventRecord(g_timer_stop, s);
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
                                         "reduce", "aux", "aux_final", "w_transpose"};
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

moe_status_t moe_top1_fwd(const void* fused_ctx, const float* gate_logits, const void* W, const float* b,
                          void* routed_ctx, int32_t* expert_idx, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* perm, int64_t B, int64_t NH, int64_t H,
                          int64_t NE, int act, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "moe_top1_fwd";
    moe_status_t st = check_shape(fn, B, NH, H, NE, act, true);
    if (st != MOE_OK) return st;
    REQ(fused_ctx); REQ(gate_logits); REQ(W); REQ(b); REQ(routed_ctx);
    REQ(expert_idx); REQ(expert_counts); REQ(expert_offsets); REQ(perm);
    const Plan p = make_plan(B * NH, (int)H, (int)NE, act);
    if ((st = check_ws(fn, p, workspace, workspace_bytes)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if ((st = do_route(gate_logits, expert_idx, expert_counts, expert_offsets, perm, p, workspace, s)) != MOE_OK)
        return st;
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

moe_status_t moe_top1_bwd(const void* d_routed_ctx, const void* fused_ctx, const void* W,
                          const int32_t* expert_offsets, const int32_t* perm, void* d_fused_ctx, float* d_W,
                          float* d_b, int accumulate_dx, int64_t B, int64_t NH, int64_t H, int64_t NE, int act,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "moe_top1_bwd";
    moe_status_t st = check_shape(fn, B, NH, H, NE, act, true);
    if (st != MOE_OK) return st;
    REQ(d_routed_ctx); REQ(fused_ctx); REQ(W); REQ(expert_offsets); REQ(perm);
    REQ(d_fused_ctx); REQ(d_W); REQ(d_b);
    const Plan p = make_plan(B * NH, (int)H, (int)NE, act);
    if ((st = check_ws(fn, p, workspace, workspace_bytes)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    float* pdw = at<float>(workspace, p.off_pdw);
    float* pdb = at<float>(workspace, p.off_pdb);
    if (act == MOE_DTYPE_F32) {
        LAUNCH(K_BWD_GEMM,
               launch_bwd_gemm_f32((const float*)d_routed_ctx, (const float*)fused_ctx, (const float*)W,
                                   (float*)d_fused_ctx, accumulate_dx, pdw, pdb, expert_offsets, perm, p.T, p.H,
                                   p.NE, p.chunks, p.n_chunk_max, s),
               "bwd gemm");
    } else {
        uint16_t* wt = at<uint16_t>(workspace, p.off_wt);
        LAUNCH(K_W_TRANSPOSE, launch_transpose_w_bf16((const uint16_t*)W, wt, p.H, p.NE, s), "w transpose");
        LAUNCH(K_BWD_GEMM,
               launch_bwd_gemm_bf16((const uint16_t*)d_routed_ctx, (const uint16_t*)fused_ctx, wt,
                                    (uint16_t*)d_fused_ctx, accumulate_dx, pdw, pdb, expert_offsets, perm, p.T, p.H,
                                    p.NE, p.chunks, p.n_chunk_max, s),
               "bwd gemm");
    }
    LAUNCH(K_REDUCE, launch_reduce_dw(pdw, pdb, expert_offsets, p.T, p.H, p.NE, p.chunks, d_W, d_b, s), "reduce");
    return MOE_OK;
}

moe_status_t moe_aux_loss(const float* gate_logits, const int32_t* expert_counts, float lambda, float* loss,
                          float* d_gate_logits, float* frac, float* mean_prob, float* probs, int64_t B,
                          int64_t NH, int64_t NE, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "moe_aux_loss";
    moe_status_t st = check_shape(fn, B, NH, 0, NE, MOE_DTYPE_F32, false);
    if (st != MOE_OK) return st;
    REQ(gate_logits); OPT(expert_counts); REQ(loss); REQ(d_gate_logits);
    OPT(frac); OPT(mean_prob); OPT(probs);
    if (!isfinite(lambda)) return fail(MOE_ERR_INVALID_ARG, "%s: lambda is not finite", fn);
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
    LAUNCH(K_AUX, launch_aux_rows(gate_logits, counts, p.T, p.NE, lambda, d_gate_logits, probs, part, p.n_ablk, s),
           "aux rows");
    LAUNCH(K_AUX_FINAL, launch_aux_final(part, counts, p.n_ablk, p.T, p.NE, lambda, loss, frac, mean_prob, s),
           "aux final");
    return MOE_OK;
}

}  // extern "C"
