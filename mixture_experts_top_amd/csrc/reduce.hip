// Deterministic collapse of the per-chunk d_W / d_b partials over the token axis.
//
// This is the role of reduce_axis0 on the pages: the MoE-gate commit page ("11b96dac6a",
// PERFORMANCE block) collapses its per-token d_W / d_b scratches over (B, N_H), and the
// perf-pass page ("b23f8f2efa", reduce_axis0 entry) gives the design -- a column tile
// read with coalesced 128-byte accesses, a block tree-reduce over the row axis, one
// writer per output and no atomics.  Here the rows are the fixed-size token chunks of
// one expert (chunk partials, not per-token scratch), so the reduced axis is short.
//
// Block (RX x RY, RX RY = 256): tx owns one float4 column, ty sums chunks ty, ty+RY, ... in
// ascending order, and the RY partial sums are added in a fixed order.  An expert with no
// tokens has no chunks and gets +0.0.
#include "moe_internal.hpp"

namespace moe {

namespace {
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
}  // namespace

// Sums rows [cs, cs + n) of a [rows][len] fp32 array into out[col0 : col0 + 4 RX] (float4
// lanes); +0.0 when n == 0.  Thread row ty takes rows ty, ty + RY, ... in order, then the RY
// row sums are added in order.  The rows are loaded NB at a time, every load of a batch
// unconditional (a row index past n re-reads row n - 1, which is not added), so a thread
// waits on one memory round trip per batch rather than one per row.
template <int RY>
__device__ __forceinline__ void column_sum(const float* __restrict__ in, size_t len, int cs, int n, size_t col0,
                                           float* __restrict__ out, f32x4* red) {
    constexpr int RX = 256 / RY, NB = 8;
    const int tx = threadIdx.x % RX, ty = threadIdx.x / RX;
    const size_t col = col0 + 4 * (size_t)tx;
    const bool ok = col < len;
    f32x4 s = f32x4{};
    if (ok && n > 0) {
        for (int c0 = ty; c0 < n; c0 += NB * RY) {
            f32x4 v[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int c = c0 + u * RY;
                v[u] = ld4(in + (size_t)(cs + (c < n ? c : n - 1)) * len + col);
            }
#pragma unroll
            for (int u = 0; u < NB; ++u)
                if (c0 + u * RY < n) s += v[u];
        }
    }
    red[ty * RX + tx] = s;
    __syncthreads();
    if (ty == 0 && ok) {
        f32x4 r = red[tx];
#pragma unroll
        for (int q = 1; q < RY; ++q) r += red[q * RX + tx];
        st4(out + col, r);
    }
    __syncthreads();
}

// grid (H*H/(4 RX) + 1, N_E): x < H*H/(4 RX) -> a column tile of dW[e]; the last x -> db[e].
// RY rows of threads share an expert's chunk rows: 4 when experts have few chunks (wide
// column tiles, few workgroups; 2 when they average fewer than 8), 8 or 16 when they have more
// (more loads in flight).
template <int RY>
__global__ __launch_bounds__(256) void k_reduce_dw(const float* __restrict__ pdw,
                                                   const float* __restrict__ pdb,
                                                   const int* __restrict__ offsets, int H, int NE,
                                                   int P, int T, float* __restrict__ dW,
                                                   float* __restrict__ db) {
    constexpr int RX = 256 / RY;
    __shared__ f32x4 red[256];
    const int e = blockIdx.y;
    // chunk range of expert e: one load per lane (guarded, routing_guard.hpp) and a wavefront
    // prefix sum over the experts
    const int lane = threadIdx.x % 64;
    int lo, cnt;
    expert_range(offsets, NE, T, lo, cnt);
    const int nl = expert_nchunks(cnt, P, T);
    const int incl = wave_inclusive_sum(nl);
    const int cs = __builtin_amdgcn_readlane(incl - nl, e), n = __builtin_amdgcn_readlane(nl, e);
    const size_t HH = (size_t)H * H;
    const int nbx = (int)(HH / (4 * RX));
    if ((int)blockIdx.x < nbx) {
        column_sum<RY>(pdw, HH, cs, n, (size_t)blockIdx.x * 4 * RX, dW + (size_t)e * HH, red);
    } else {
        for (int c0 = 0; c0 < H; c0 += 4 * RX) column_sum<RY>(pdb, H, cs, n, c0, db + (size_t)e * H, red);
    }
}

// Few chunks per expert: one thread per column owns four float4 columns (tid + 256 j, so each
// load instruction reads 1 KB of one row) and sums every chunk of them in chunk order, NB
// chunks per batch with all of a batch's loads unconditional (clamped chunk index), so 4 NB
// loads per thread are in flight at once.  grid (H*H/(16*256) + 1, N_E); the last x does db.
template <int NB>
__global__ __launch_bounds__(256) void k_reduce_dw_wide(const float* __restrict__ pdw,
                                                        const float* __restrict__ pdb,
                                                        const int* __restrict__ offsets, int H, int NE,
                                                        int P, int T, float* __restrict__ dW,
                                                        float* __restrict__ db) {
    constexpr int CPT = 4;
    const int e = blockIdx.y;
    int lo, cnt;
    expert_range(offsets, NE, T, lo, cnt);
    const int nl = expert_nchunks(cnt, P, T);
    const int incl = wave_inclusive_sum(nl);
    const int cs = __builtin_amdgcn_readlane(incl - nl, e), n = __builtin_amdgcn_readlane(nl, e);
    const size_t HH = (size_t)H * H;
    const int nbx = (int)(HH / (4 * 256 * CPT));
    const bool isdb = (int)blockIdx.x >= nbx;
    const float* __restrict__ in = isdb ? pdb : pdw;
    const size_t len = isdb ? (size_t)H : HH;
    float* __restrict__ out = isdb ? db + (size_t)e * H : dW + (size_t)e * HH;
    const size_t c0 = isdb ? 0 : (size_t)blockIdx.x * 4 * 256 * CPT;
    size_t col[CPT];
    bool ok[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        col[j] = c0 + 4 * ((size_t)threadIdx.x + 256 * j);
        ok[j] = col[j] < len;
        if (!ok[j]) col[j] = 0;
    }
    f32x4 s[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) s[j] = f32x4{};
    for (int b0 = 0; b0 < n; b0 += NB) {
        f32x4 v[NB][CPT];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const float* row = in + (size_t)(cs + (b0 + u < n ? b0 + u : n - 1)) * len;
#pragma unroll
            for (int j = 0; j < CPT; ++j) v[u][j] = ld4(row + col[j]);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u)
            if (b0 + u < n)
#pragma unroll
                for (int j = 0; j < CPT; ++j) s[j] += v[u][j];
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        if (ok[j]) st4(out + col[j], s[j]);
}

// Rows of threads per column tile: 16 (narrow tiles, more loads in flight per column) once
// the plan has at least this many chunks, else 4.
#ifndef MOE_REDUCE_RY16_MIN_P
#define MOE_REDUCE_RY16_MIN_P 1024
#endif
// 8 rows of threads when the experts average at least this many chunks each (and the plan
// stays under MOE_REDUCE_RY16_MIN_P): imbalanced shape (T = 81,920, N_E = 8) reduce 8.9 -> 7.0 us
// MOE_REDUCE_RYLOW rows of threads (wider column tiles, half the workgroups) when the experts
// average fewer than MOE_REDUCE_RYLOW_MAX_CPE chunks each: wider-bf16 shape (32 chunks over 8
// experts) reduce 15.8 -> 13.3 us
#ifndef MOE_REDUCE_RYLOW_MAX_CPE
#define MOE_REDUCE_RYLOW_MAX_CPE 8
#endif
#ifndef MOE_REDUCE_RYLOW
#define MOE_REDUCE_RYLOW 2
#endif
#ifndef MOE_REDUCE_WIDE
#define MOE_REDUCE_WIDE 1
#endif
#ifndef MOE_REDUCE_WIDE_MAX_CPE
#define MOE_REDUCE_WIDE_MAX_CPE 8
#endif
#ifndef MOE_REDUCE_RY8_MIN_CPE
#define MOE_REDUCE_RY8_MIN_CPE 16
#endif
hipError_t launch_reduce_dw(const float* part_dw, const float* part_db, const int32_t* offsets, int64_t T, int H,
                            int NE, int P, float* dW, float* db, hipStream_t s) {
    if (MOE_REDUCE_WIDE && P / NE < MOE_REDUCE_WIDE_MAX_CPE && (H * H) % (16 * 256) == 0) {
        const int nbx = H * H / (16 * 256);
        launch_kernel(k_reduce_dw_wide<4>, dim3(nbx + 1, NE), dim3(256), 0, s, part_dw, part_db, offsets, H, NE, P,
                      (int)T, dW, db);
    } else if (P / NE < MOE_REDUCE_RYLOW_MAX_CPE) {
        constexpr int RY = MOE_REDUCE_RYLOW;
        const int nbx = H * H / (4 * (256 / RY));
        launch_kernel(k_reduce_dw<RY>, dim3(nbx + 1, NE), dim3(256), 0, s, part_dw, part_db, offsets, H, NE, P,
                      (int)T, dW, db);
    } else if (P < MOE_REDUCE_RY16_MIN_P && P / NE >= MOE_REDUCE_RY8_MIN_CPE) {
        const int nbx = H * H / (4 * 32);
        launch_kernel(k_reduce_dw<8>, dim3(nbx + 1, NE), dim3(256), 0, s, part_dw, part_db, offsets, H, NE, P,
                      (int)T, dW, db);
    } else if (P >= MOE_REDUCE_RY16_MIN_P) {
        const int nbx = H * H / (4 * 16);
        launch_kernel(k_reduce_dw<16>, dim3(nbx + 1, NE), dim3(256), 0, s, part_dw, part_db, offsets, H, NE, P,
                           (int)T, dW, db);
    } else {
        const int nbx = H * H / (4 * 64);
        launch_kernel(k_reduce_dw<4>, dim3(nbx + 1, NE), dim3(256), 0, s, part_dw, part_db, offsets, H, NE, P,
                           (int)T, dW, db);
    }
    return hipGetLastError();
}

}  // namespace moe
