// Deterministic collapse of the per-chunk d_W / d_b partials over the token axis.
//
// This is the role of reduce_axis0 on the pages: the MoE-gate commit page ("11b96dac6a",
// PERFORMANCE block) collapses its per-token d_W / d_b scratches over (B, N_H), and the
// perf-pass page ("b23f8f2efa", reduce_axis0 entry) gives the design -- a column tile
// read with coalesced 128-byte accesses, a block tree-reduce over the row axis, one
// writer per output and no atomics.  Here the rows are the fixed-size token chunks of
// one expert (chunk partials, not per-token scratch), so the reduced axis is short.
//
// Block (64 x 4): tx owns one float4 column, ty sums chunks ty, ty+4, ... in ascending
// order, and the four partial sums are added in a fixed order.  An expert with no
// tokens has no chunks and gets +0.0.
#include "moe_internal.hpp"

namespace moe {

namespace {
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
}  // namespace

__global__ __launch_bounds__(256) void k_reduce_dw(const float* __restrict__ pdw,
                                                   const float* __restrict__ pdb,
                                                   const int* __restrict__ offsets, int H, int NE,
                                                   int chunk, float* __restrict__ dW,
                                                   float* __restrict__ db) {
    __shared__ f32x4 red[4][64];
    const int e = blockIdx.y;
    int cs = 0;
    for (int i = 0; i < e; ++i) cs += (offsets[i + 1] - offsets[i] + chunk - 1) / chunk;
    const int n = (offsets[e + 1] - offsets[e] + chunk - 1) / chunk;
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
    const size_t HH = (size_t)H * H;
    const int nbx = (int)(HH / 256);
    if ((int)blockIdx.x < nbx) {
        const size_t col = ((size_t)blockIdx.x * 64 + tx) * 4;
        f32x4 s = f32x4{};
        for (int c = ty; c < n; c += 4) s += ld4(pdw + (size_t)(cs + c) * HH + col);
        red[ty][tx] = s;
        __syncthreads();
        if (ty == 0) st4(dW + (size_t)e * HH + col, ((red[0][tx] + red[1][tx]) + red[2][tx]) + red[3][tx]);
    } else {
        for (int c4 = 0; c4 < H / 4; c4 += 64) {
            const int col = (c4 + tx) * 4;
            f32x4 s = f32x4{};
            if (col < H)
                for (int c = ty; c < n; c += 4) s += ld4(pdb + (size_t)(cs + c) * H + col);
            red[ty][tx] = s;
            __syncthreads();
            if (ty == 0 && col < H)
                st4(db + (size_t)e * H + col, ((red[0][tx] + red[1][tx]) + red[2][tx]) + red[3][tx]);
            __syncthreads();
        }
    }
}

hipError_t launch_reduce_dw(const float* part_dw, const float* part_db, const int32_t* offsets, int H,
                            int NE, int chunk, float* dW, float* db, hipStream_t s) {
    const int nbx = H * H / 256;
    hipLaunchKernelGGL(k_reduce_dw, dim3(nbx + 1, NE), dim3(256), 0, s, part_dw, part_db, offsets, H, NE,
                       chunk, dW, db);
    return hipGetLastError();
}

}  // namespace moe
