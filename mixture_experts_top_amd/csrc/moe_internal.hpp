// Internal declarations of the top-1 MoE gate library (gfx950 / CDNA4).
//
// The C ABI lives in include/moe_top1.h; this header holds the workspace plan, the
// constants shared by kernels and host code, and the host-side launchers that each
// kernel file provides.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "routing_guard.hpp"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Routing: one workgroup of 256 threads (4 waves) ranks 256 tokens as 4 groups of 64.
constexpr int kRouteThreads = 256;
constexpr int kRouteTokens = 256;
constexpr int kRouteGroups = kRouteTokens / 64;
constexpr int kMaxExperts = 64;
constexpr int kScanThreads = 1024;

// Aux loss: one workgroup of 256 threads covers 256 tokens (one per thread).
constexpr int kAuxThreads = 256;
constexpr int kAuxTokens = 256;

enum KernelId {
    K_ROUTE = 0, K_SCAN, K_SCATTER, K_FWD_GEMM, K_BWD_GEMM, K_REDUCE, K_AUX, K_AUX_FINAL, K_W_TRANSPOSE,
    K_LAMBDA, K_REDUCE_AXIS0, K_COLLAPSE, K_SOFTMAX_CE, K_COUNT
};

// fp32 GEMM tiling, shared by the kernels' launchers and the workspace plan.  Large T:
// 128-row tiles and 128 x 128 d_W tiles (64 for H = 64).  Small T (too few 128-row tiles
// for MOE_ROWS_BIG_TILES_PER_CU per CU): smaller tiles, so that more workgroups hide the
// memory latency that then bounds each one.
#ifndef MOE_ROWS_BIG_TILES_PER_CU
#define MOE_ROWS_BIG_TILES_PER_CU 2
#endif
#ifndef MOE_DW_SMALL_BT
#define MOE_DW_SMALL_BT 64
#endif
// Minimum tokens per d_W chunk (see plan_chunks): small-T tiling, fp32 large-T tiling.  With
// the large-T 128 x 128 dW tiles, 320-token chunks took the imbalanced shape's (81,920 tokens,
// H = 128) backward from 81 to 71 µs against 192 (256: 73, 512: 74, 768: 82 µs); the large-stress
// plan is capped by the workgroup budget first, so it does not change.
#ifndef MOE_DW_MIN_CHUNK
#define MOE_DW_MIN_CHUNK 128
#endif
#ifndef MOE_DW_MIN_CHUNK_BIG
#define MOE_DW_MIN_CHUNK_BIG 320
#endif
inline bool f32_big_tiles(int64_t T, int H) {
    const int64_t nt = H >= 128 ? H / 128 : 1;
    return (T / 128) * nt >= MOE_ROWS_BIG_TILES_PER_CU * 256;
}
// fp32 d_W tiles of 256 x 256 at large T for H = 256, 512: eight wavefronts per workgroup,
// one workgroup per compute unit, in a launch of their own ahead of the dX launch.
#ifndef MOE_F32_DW_BIG
#define MOE_F32_DW_BIG 1
#endif
inline int f32_dw_tile(int64_t T, int H) {
    const int big = H >= 128 ? 128 : 64;
    const int small = MOE_DW_SMALL_BT < H ? MOE_DW_SMALL_BT : H;
    if (!f32_big_tiles(T, H)) return small;
    return (MOE_F32_DW_BIG && H >= 256) ? 256 : big;
}

// bf16 d_W output tile (BT x BT per workgroup): 256 x 256 for H = 256 / 512 (one workgroup of
// four wavefronts per compute unit, each wavefront a 128 x 128 quarter), else H or 128.
#ifndef MOE_BF16_DW_BIG
#define MOE_BF16_DW_BIG 1
#endif
constexpr int bf16_dw_tile(int H) { return (MOE_BF16_DW_BIG && H >= 256) ? 256 : (H >= 128 ? 128 : 64); }

// Chunking of each expert's tokens for the d_W split-K.  With P chunks planned for T
// tokens, expert e (c_e tokens) gets n_e = ceil(c_e P / T) chunks (none if c_e = 0), and
// chunk j covers its tokens [floor(j c_e / n_e), floor((j+1) c_e / n_e)).  So chunks are
// about T / P tokens everywhere, the count follows each expert's share of the tokens, and
// sum_e n_e <= P + N_E.  Chunk ids run expert by expert.  Depends only on (offsets, P, T).
__device__ __forceinline__ int expert_nchunks(int c, int P, int T) {
    return c == 0 ? 0 : (int)(((int64_t)c * P + T - 1) / T);
}

// Cross-lane steps through DPP (data-parallel primitives: a VALU operand read from another
// lane of the same 16-lane row) rather than LDS permutes: each step is one VALU instruction,
// where a permute is an LDS round trip that the next step waits for.  dpp_move returns, in
// every lane, src of the lane that CTRL names, or `id` where that lane lies outside the row.
// CTRL: quad_perm p (0x00 - 0xFF, two bits per lane of a quad), row_shr n (0x110 + n),
// row_ror n (0x120 + n).  The scans and sums below read other lanes' registers (DPP sources,
// readlane), so all 64 lanes of the wavefront must be active where they are called: every
// caller runs them in code that the whole workgroup executes.
template <int CTRL>
__device__ __forceinline__ int dpp_move(int src, int id) {
    return __builtin_amdgcn_update_dpp(id, src, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_move(float src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, src), CTRL, 0xF, 0xF,
                                                                 false));
}

// Inclusive prefix sum over the 64 lanes of a wavefront (every lane holds one term): a
// doubling scan inside each 16-lane row (shifts of 1, 2, 4, 8), then the totals of the rows
// below are added.  Integer sums, so the order does not matter.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int lane = __lane_id();
    v += dpp_move<0x111>(v, 0);
    v += dpp_move<0x112>(v, 0);
    v += dpp_move<0x114>(v, 0);
    v += dpp_move<0x118>(v, 0);
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Inclusive running maximum over the 64 lanes of a wavefront, for non-negative terms (0 is
// the identity the shifts bring in, so a result is always one of the terms or 0).
__device__ __forceinline__ int wave_inclusive_max_nonneg(int v) {
    const int lane = __lane_id();
    v = max(v, dpp_move<0x111>(v, 0));
    v = max(v, dpp_move<0x112>(v, 0));
    v = max(v, dpp_move<0x114>(v, 0));
    v = max(v, dpp_move<0x118>(v, 0));
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    const int below = row > 2 ? max(max(r0, r1), r2) : (row > 1 ? max(r0, r1) : (row > 0 ? r0 : 0));
    return max(v, below);
}

// Sum of v over the 64 lanes of a wavefront, the same bits in every lane: within each quad
// (exchanges with lane ^ 1, then ^ 2: every lane of a quad holds the same sum), across the
// quads of a row (rotations by 4 and 8), then the four row sums of lanes 0, 16, 32, 48 in
// that order.  A fixed order, so the result does not depend on the run.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_move<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_move<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_move<0x124>(v);  // row_ror 4
    v += dpp_move<0x128>(v);  // row_ror 8
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return ((r0 + r1) + r2) + r3;
}

// Lane l < NE: expert l's first position lo in perm and its token count cnt, from offsets
// under the guards of routing_guard.hpp (clamped to [0, T], made non-decreasing by a running
// maximum over the lanes); lanes >= NE get cnt = 0.  One load per lane, no serial chain.
__device__ __forceinline__ void expert_range(const int* __restrict__ offsets, int NE, int T, int& lo, int& cnt) {
    const int lane = __lane_id();
    int a = 0, b = 0;
    if (lane < NE) {
        a = guard_offset(offsets[lane], T);
        b = offsets[lane + 1];
    }
    lo = wave_inclusive_max_nonneg(a);
    cnt = lane < NE ? guard_count(lo, b, T) : 0;
}

// Wavefront-wide lookup of the unit `u` in a list cut expert by expert: lane l < NE holds
// expert l's range (expert_range) and its number of units n_l; a prefix sum over lanes finds
// the expert whose units cover u.  All lanes get the same (uniform) result.  Returns false if
// u is past the last unit.
__device__ __forceinline__ bool wave_find(const int* __restrict__ offsets, int NE, int T, int u, int bm, int P,
                                          bool chunks, int& e, int& j, int& lo, int& cnt, int& n_e) {
    const int lane = __lane_id();
    int l0, c;
    expert_range(offsets, NE, T, l0, c);
    const int n = lane < NE ? (chunks ? expert_nchunks(c, P, T) : (c + bm - 1) / bm) : 0;
    const int incl = wave_inclusive_sum(n);
    const int excl = incl - n;
    const uint64_t hit = __ballot(lane < NE && u >= excl && u < incl);
    if (hit == 0) return false;
    const int le = __ffsll((unsigned long long)hit) - 1;
    e = le;
    j = u - __builtin_amdgcn_readlane(excl, le);
    lo = __builtin_amdgcn_readlane(l0, le);
    cnt = __builtin_amdgcn_readlane(c, le);
    n_e = __builtin_amdgcn_readlane(n, le);
    return true;
}

// M-tile `mt` of rows cut into tiles of bm per expert -> expert e, rows [r0, r1) of perm.
__device__ __forceinline__ bool find_tile(const int* __restrict__ offsets, int NE, int T, int mt, int bm, int& e,
                                          int& r0, int& r1) {
    int j, lo, cnt, n;
    if (!wave_find(offsets, NE, T, mt, bm, 0, false, e, j, lo, cnt, n)) return false;
    r0 = lo + j * bm;
    r1 = min(lo + cnt, r0 + bm);
    return true;
}

// d_W chunk c -> expert e, token positions [t0, t1) of perm (see expert_nchunks).
__device__ __forceinline__ bool find_chunk(const int* __restrict__ offsets, int NE, int P, int T, int c, int& e,
                                           int& t0, int& t1) {
    int j, lo, cnt, n;
    if (!wave_find(offsets, NE, T, c, 1, P, true, e, j, lo, cnt, n)) return false;
    t0 = lo + (int)((int64_t)j * cnt / n);
    t1 = lo + (int)((int64_t)(j + 1) * cnt / n);
    return true;
}

// Token id at position k of perm, guarded (routing_guard.hpp).
__device__ __forceinline__ int load_token(const int* __restrict__ perm, int k, int T) {
    return guard_token(perm[k], T);
}

// Workspace layout for one (T, H, N_E, act).  Every section starts on a 256-byte boundary.
struct Plan {
    int64_t T = 0;
    int H = 0, NE = 0, act = 0;
    int n_rblk = 0;       // routing blocks
    int chunks = 0;       // P: planned d_W chunks (see expert_nchunks)
    int n_chunk_max = 0;  // P + N_E, upper bound of the chunk count
    int n_ablk = 0;       // aux blocks
    size_t off_hist = 0, off_blkbase = 0, off_idx = 0, off_counts = 0, off_offsets = 0;
    size_t off_pdw = 0, off_pdb = 0, off_paux = 0;
    size_t off_wt = 0, wt_bytes = 0;  // W^T per expert (fp32 with 256 x 256 d_W tiles), else empty
    size_t total = 0;
};

Plan make_plan(int64_t T, int H, int NE, int act);

// Launch timer hook (moe_set_launch_timer): brackets launches of one kernel with events.
struct TimerScope {
    hipStream_t s;
    bool on;
    TimerScope(KernelId k, hipStream_t s);
    ~TimerScope();
};

// Events armed by a TimerScope for the next kernel launch (process-wide, like the timer).
struct ArmedEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
ArmedEvents& armed_events();

// Every kernel launch goes through here.  When a TimerScope has armed a pair of events, the
// launch carries them and the command processor records them at the kernel's own start and
// end (hipExtLaunchKernelGGL); otherwise it is a plain launch.  Arguments are converted to the
// kernel's parameter types.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shm, hipStream_t s,
                          Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    ArmedEvents& ev = armed_events();
    if (ev.start != nullptr) {
        const hipEvent_t a = ev.start, b = ev.stop;
        ev.start = ev.stop = nullptr;
        hipExtLaunchKernelGGL(kernel, grid, block, shm, s, a, b, 0u, static_cast<KArgs>(args)...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shm, s, static_cast<KArgs>(args)...);
    }
}

// A launch with explicit start / stop events (either may be null), for a launcher that makes
// several launches under one kernel id: it takes the armed events (take_armed_events) and
// gives the start event to its first launch and the stop event to its last, so the pair
// brackets all of them.
template <typename... KArgs, typename... Args>
inline void launch_kernel_ev(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shm, hipStream_t s,
                             hipEvent_t start, hipEvent_t stop, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    if (start != nullptr || stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, shm, s, start, stop, 0u, static_cast<KArgs>(args)...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shm, s, static_cast<KArgs>(args)...);
}
inline ArmedEvents take_armed_events() {
    ArmedEvents e = armed_events();
    armed_events() = ArmedEvents{};
    return e;
}

// ---- launchers (each returns the hipError_t of its launch) ----
// The aux loss riding on the routing and forward launches: inputs, lambda and outputs of
// moe_aux_loss, plus the softmax column sums that k_route_part wrote (one row per 256-token block).
struct AuxFwdArgs {
    const float* G;
    const float* part;
    float lam;
    const float* lam_dev;
    float* dG;
    float* probs;
    float* loss;
    float* frac;
    float* mean_prob;
    int n_ablk;
};
hipError_t launch_route_part(const float* G, int64_t T, int NE, int32_t* idx, int32_t* hist, float* part,
                             int n_rblk, hipStream_t s);
hipError_t launch_route(const float* G, int64_t T, int NE, int32_t* idx, int32_t* hist,
                        int n_rblk, hipStream_t s);
bool scatter_scan_fits(int n_rblk, int NE);
hipError_t launch_scatter_scan(const int32_t* idx, int64_t T, int NE, const int32_t* hist, int n_rblk,
                               int32_t* counts, int32_t* offsets, int32_t* perm, hipStream_t s);
hipError_t launch_scatter_scan_aux(const int32_t* idx, int64_t T, int NE, const int32_t* hist, int n_rblk,
                                   int32_t* counts, int32_t* offsets, int32_t* perm, const AuxFwdArgs& ax,
                                   hipStream_t s);
hipError_t launch_scatter_aux(const int32_t* idx, int64_t T, int NE, const int32_t* blkbase, int32_t* perm,
                              const int32_t* counts, int n_rblk, const AuxFwdArgs& ax, hipStream_t s);
hipError_t launch_scan(const int32_t* hist, int n_rblk, int NE, int32_t* blkbase,
                       int32_t* counts, int32_t* offsets, hipStream_t s);
hipError_t launch_scatter(const int32_t* idx, int64_t T, int NE, const int32_t* blkbase,
                          int32_t* perm, int n_rblk, hipStream_t s);

// The load-balancing loss carried by the small-T forward launch (N_E <= kAuxFwdMaxExperts):
// part holds the routing kernel's softmax column sums, one row per routing block.
constexpr int kAuxFwdMaxExperts = 8;      // aux carried by the one-pass forward GEMM
constexpr int kAuxScatterMaxExperts = 16;  // aux carried by the routing and scatter launches

bool fwd_gemm_f32_gather_fits(int64_t T, int H, int NE, int n_rblk);
hipError_t launch_fwd_gemm_f32_gather(const float* X, const float* W, const float* bias, float* Y,
                                      const int32_t* idx, const int32_t* hist, int n_rblk, int32_t* counts,
                                      int32_t* offsets, int32_t* perm, int64_t T, int H, int NE,
                                      const AuxFwdArgs* aux, hipStream_t s);
hipError_t launch_fwd_gemm_f32(const float* X, const float* W, const float* bias, float* Y,
                               const int32_t* offsets, const int32_t* perm, int64_t T, int H, int NE,
                               hipStream_t s);
// dX (overwrite or accumulate) and the d_W / d_b chunk partials (wt: the plan's W^T section,
// used with the 256 x 256 d_W tiles)
hipError_t launch_bwd_gemm_f32(const float* dY, const float* X, const float* W, float* dX, int accumulate,
                               float* part_dw, float* part_db, float* wt, const int32_t* offsets, const int32_t* perm,
                               int64_t T, int H, int NE, int P, int n_chunk_max, hipStream_t s);
// same, with row t of dY = d_mean[t / NH] * (1/NH) (backward through a mean over NH horizons)
hipError_t launch_bwd_gemm_f32_from_mean(const float* d_mean, const float* X, const float* W, float* dX,
                                         int accumulate, float* part_dw, float* part_db, float* wt,
                                         const int32_t* offsets, const int32_t* perm, int64_t T, int H, int NE, int NH,
                                         int P, int n_chunk_max, hipStream_t s);
// bf16 storage (raw uint16 patterns), fp32 accumulation
hipError_t launch_fwd_gemm_bf16(const uint16_t* X, const uint16_t* W, const float* bias, uint16_t* Y,
                                const int32_t* offsets, const int32_t* perm, int64_t T, int H, int NE,
                                hipStream_t s);
hipError_t launch_bwd_gemm_bf16(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX,
                                int accumulate, float* part_dw, float* part_db, const int32_t* offsets,
                                const int32_t* perm, int64_t T, int H, int NE, int P, int n_chunk_max,
                                hipStream_t s);
// same, with row t of dY = bf16(d_mean[t / NH] * (1/NH)) (backward through a mean over NH horizons)
hipError_t launch_bwd_gemm_bf16_from_mean(const uint16_t* d_mean, const uint16_t* X, const uint16_t* W, uint16_t* dX,
                                          int accumulate, float* part_dw, float* part_db, const int32_t* offsets,
                                          const int32_t* perm, int64_t T, int H, int NE, int NH, int P,
                                          int n_chunk_max, hipStream_t s);
hipError_t launch_reduce_dw(const float* part_dw, const float* part_db, const int32_t* offsets,
                            int64_t T, int H, int NE, int P, float* dW, float* db, hipStream_t s);

hipError_t launch_aux_rows(const float* G, const int32_t* counts, int64_t T, int NE, float lam, const float* lam_dev,
                           float* dG, float* probs, float* part, int n_ablk, hipStream_t s);
hipError_t launch_aux_final(const float* part, const int32_t* counts, int n_ablk, int64_t T, int NE,
                            float lam, const float* lam_dev, float* loss, float* frac, float* mean_prob,
                            hipStream_t s);
int64_t reduce_axis0_chunks(int64_t n_batch, int64_t n_tail, bool vec);
hipError_t launch_reduce_axis0(const float* in, int64_t n_batch, int64_t n_tail, float* out, float* part, bool vec,
                               hipStream_t s);
hipError_t launch_collapse(bool bwd, int act, const void* in, void* out, int64_t B, int NH, int H, hipStream_t s);
hipError_t launch_softmax_ce(const float* logits, const int32_t* labels, int64_t rows, int A, int64_t B, float* grad,
                             float* ce, hipStream_t s);
hipError_t launch_lambda_eff(const float* ent_ema, float floor_, float max_extra, float target_frac, int K,
                             float* lambda_eff, hipStream_t s);

}  // namespace moe
