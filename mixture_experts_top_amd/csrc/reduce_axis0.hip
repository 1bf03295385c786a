// Standalone deterministic column sum: out[j] = sum_r in[r, j] over an [n_batch, n_tail] fp32
// array.  This is the reduce_axis0 primitive of the perf-pass page ("b23f8f2efa",
// reduce_axis0 entry: a column tile read with coalesced accesses, a block tree-reduce over
// rows, no atomics), which the MHA page ("9170d24fe3", trainer and BUG blocks) applies to the
// MoE's per-token d_W scratch with n_batch = B*N_H and n_tail = N_E*H*H.
//
// Two passes of one kernel: pass 1 splits the rows into R fixed chunks (R chosen from the
// shape so the grid fills the GPU), each workgroup summing one column tile of one chunk;
// pass 2 sums the R chunk rows.  Inside a workgroup, 4 rows of threads take every fourth row
// in order and their sums are added in a fixed order.  No atomics; the result depends only
// on the inputs and the shape.
#include "moe_internal.hpp"

namespace moe {

namespace {
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
}  // namespace

// grid (column tiles, chunks); block 64 x 4.  VEC: 4 columns per thread (n_tail % 4 == 0,
// 16-byte aligned rows), else 1.
template <bool VEC>
__global__ __launch_bounds__(256) void k_reduce_axis0(const float* __restrict__ in, int64_t n_batch, int64_t n_tail,
                                                      int64_t rows_per_chunk, float* __restrict__ out) {
    constexpr int W = VEC ? 4 : 1;
    __shared__ float red[4][64 * W];
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = min(n_batch, r0 + rows_per_chunk);
    const int64_t col = ((int64_t)blockIdx.x * 64 + tx) * W;
    const bool ok = col < n_tail;
    float* o = out + (int64_t)blockIdx.y * n_tail;
    if (VEC) {
        f32x4 s = f32x4{};
        if (ok) {
#pragma unroll 8
            for (int64_t r = r0 + ty; r < r1; r += 4)  // read once: non-temporal (6.25 -> 6.93 TB/s)
                s += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(in + r * n_tail + col));
        }
        st4(&red[ty][4 * tx], s);
        __syncthreads();
        if (ty == 0 && ok) {
            const f32x4 a = ld4(&red[0][4 * tx]), b = ld4(&red[1][4 * tx]), c = ld4(&red[2][4 * tx]),
                        d = ld4(&red[3][4 * tx]);
            st4(o + col, ((a + b) + c) + d);
        }
    } else {
        float s = 0.0f;
        if (ok) {
#pragma unroll 8
            for (int64_t r = r0 + ty; r < r1; r += 4) s += in[r * n_tail + col];
        }
        red[ty][tx] = s;
        __syncthreads();
        if (ty == 0 && ok) o[col] = ((red[0][tx] + red[1][tx]) + red[2][tx]) + red[3][tx];
    }
}

// Number of row chunks for pass 1: about 2048 workgroups in total, chunks of >= 64 rows.
int64_t reduce_axis0_chunks(int64_t n_batch, int64_t n_tail, bool vec) {
    const int64_t tiles = (n_tail + (vec ? 256 : 64) - 1) / (vec ? 256 : 64);
    int64_t R = (2048 + tiles - 1) / tiles;
    const int64_t rmax = (n_batch + 63) / 64;
    if (R > rmax) R = rmax;
    if (R < 1) R = 1;
    const int64_t rpc = (n_batch + R - 1) / R;
    return (n_batch + rpc - 1) / rpc;
}

hipError_t launch_reduce_axis0(const float* in, int64_t n_batch, int64_t n_tail, float* out, float* part, bool vec,
                               hipStream_t s) {
    const int64_t R = reduce_axis0_chunks(n_batch, n_tail, vec);
    const int64_t rpc = (n_batch + R - 1) / R;
    const int64_t tiles = (n_tail + (vec ? 256 : 64) - 1) / (vec ? 256 : 64);
    float* dst = (R == 1) ? out : part;
    if (vec) {
        launch_kernel(k_reduce_axis0<true>, dim3((unsigned)tiles, (unsigned)R), dim3(256), 0, s, in, n_batch,
                           n_tail, rpc, dst);
        if (R > 1)
            launch_kernel(k_reduce_axis0<true>, dim3((unsigned)tiles, 1), dim3(256), 0, s, part, R, n_tail, R,
                               out);
    } else {
        launch_kernel(k_reduce_axis0<false>, dim3((unsigned)tiles, (unsigned)R), dim3(256), 0, s, in, n_batch,
                           n_tail, rpc, dst);
        if (R > 1)
            launch_kernel(k_reduce_axis0<false>, dim3((unsigned)tiles, 1), dim3(256), 0, s, part, R, n_tail, R,
                               out);
    }
    return hipGetLastError();
}

}  // namespace moe
