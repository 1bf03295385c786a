// Softmax + cross-entropy gradient head (softmax/cross-entropy page "6cfd7e6691", kernel
// block): for each (b, h) row of A atom logits,
//   p = softmax(z) (shift by the row max, exponentiate, normalise by the row sum)
//   ce[b, h] = -log(max(p[label], 1e-30))
//   grad[b, h, :] = (p - onehot(label)) / B          (mean over the batch)
// and a label of -1 (the sentinel) gives ce = 0 and a zero gradient row; labels outside
// [0, A) are treated the same way.  The page uses one block per row and one thread per atom;
// here one thread owns a row and a workgroup of 256 rows stages its logits and gradients
// through LDS, so every HBM access is a contiguous sweep.  One writer per output, no atomics.
#include "moe_internal.hpp"

namespace moe {

template <int AB>  // A <= AB
__global__ __launch_bounds__(256) void k_softmax_ce(const float* __restrict__ logits, const int* __restrict__ labels,
                                                    int64_t rows, int A, float invB, float* __restrict__ grad,
                                                    float* __restrict__ ce) {
    __shared__ __attribute__((aligned(16))) float tile[256 * AB];
    constexpr int NV = AB / 4;  // 16-byte pieces per thread (256 rows x AB floats at most)
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * 256;
    const int nrows = (int)min((int64_t)256, rows - r0);
    const int64_t base = r0 * A;  // a multiple of 4 (256 rows per block)
    const int n = nrows * A;
    // 16-byte sweeps when both arrays allow them (4-byte aligned pointers are accepted too)
    const bool vec = ((((uintptr_t)logits) | ((uintptr_t)grad)) & 15) == 0;
    const int n4 = vec ? n / 4 : 0;
    // The block's logits are one contiguous range: every 16-byte load of the sweep goes out
    // before the first LDS store (unconditional loads, an index past the range re-reads piece
    // 0 and is not stored), then the rest one float at a time.
    if (vec) {
        const f32x4* src = reinterpret_cast<const f32x4*>(logits + base);
        f32x4 v[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int q = tid + 256 * k;
            v[k] = src[q < n4 ? q : 0];
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int q = tid + 256 * k;
            if (q < n4) reinterpret_cast<f32x4*>(tile)[q] = v[k];
        }
    }
    for (int i = 4 * n4 + tid; i < n; i += 256) tile[i] = logits[base + i];
    __syncthreads();
    if (tid < nrows) {
        float* z = tile + tid * A;
        const int lab = labels[r0 + tid];
        const bool valid = lab >= 0 && lab < A;
        float m = z[0];
        for (int a = 1; a < A; ++a) m = fmaxf(m, z[a]);
        float S = 0.0f;
        for (int a = 0; a < A; ++a) {
            const float e = expf(z[a] - m);
            z[a] = e;
            S += e;
        }
        float p_lab = 0.0f;
        for (int a = 0; a < A; ++a) {
            const float p = z[a] / S;
            if (a == lab) p_lab = p;
            z[a] = valid ? (p - (a == lab ? 1.0f : 0.0f)) * invB : 0.0f;
        }
        ce[r0 + tid] = valid ? -logf(fmaxf(p_lab, 1e-30f)) : 0.0f;
    }
    __syncthreads();
    if (vec) {
        f32x4* dst = reinterpret_cast<f32x4*>(grad + base);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int q = tid + 256 * k;
            // non-temporal: the gradient is not read back here (5.6 -> 5.8 TB/s at B = 131,072,
            // N_H = 8; non-temporal loads of the logits as well measured slower, 5.0)
            if (q < n4) __builtin_nontemporal_store(reinterpret_cast<const f32x4*>(tile)[q], &dst[q]);
        }
    }
    for (int i = 4 * n4 + tid; i < n; i += 256) grad[base + i] = tile[i];
}

hipError_t launch_softmax_ce(const float* logits, const int32_t* labels, int64_t rows, int A, int64_t B, float* grad,
                             float* ce, hipStream_t s) {
    const dim3 grid((unsigned)((rows + 255) / 256));
    const float invB = 1.0f / (float)B;
    if (A <= 32)
        launch_kernel(k_softmax_ce<32>, grid, dim3(256), 0, s, logits, labels, rows, A, invB, grad, ce);
    else
        launch_kernel(k_softmax_ce<64>, grid, dim3(256), 0, s, logits, labels, rows, A, invB, grad, ce);
    return hipGetLastError();
}

}  // namespace moe
