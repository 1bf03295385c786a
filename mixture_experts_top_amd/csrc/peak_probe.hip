// Calibration probes for the roofline figures: what the chip delivers on this machine, against
// the spec-sheet peaks that the roofline fractions divide by.  Not part of the gate.
//
// k_probe_mfma: every wavefront issues `iters` rounds of four independent MFMA chains (so
// each SIMD always has an instruction whose inputs are ready) and records the shader-clock
// and constant-clock ticks it spent; the accumulators end in a checksum per thread so that
// the work cannot be dropped.  k_probe_copy: the STREAM copy, 16-byte loads and stores.
#include "moe_internal.hpp"
#include "moe_top1.h"

namespace moe {

namespace {
typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));

template <int ACT>
__global__ __launch_bounds__(256) void k_probe_mfma(int64_t iters, float* __restrict__ sink,
                                                    int64_t* __restrict__ ticks) {
    const int tid = threadIdx.x;
    f32x16 c0 = f32x16{}, c1 = f32x16{}, c2 = f32x16{}, c3 = f32x16{};
    const int64_t t0 = (int64_t)clock64(), w0 = (int64_t)wall_clock64();
    if constexpr (ACT == MOE_DTYPE_F32) {
        const float a = 0.125f * (float)(tid & 7), b = 1.0f / (float)(1 + (tid & 3));
        for (int64_t i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, b, c3, 0, 0, 0);
        }
    } else {
        pbf16x8 a, b;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            a[j] = (__bf16)(0.125f * (float)((tid + j) & 7));
            b[j] = (__bf16)(1.0f / (float)(1 + ((tid + j) & 3)));
        }
        for (int64_t i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
        }
    }
    const int64_t t1 = (int64_t)clock64(), w1 = (int64_t)wall_clock64();
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
    sink[(int64_t)blockIdx.x * 256 + tid] = s;
    if (tid == 0) {
        ticks[2 * (int64_t)blockIdx.x] = t1 - t0;
        ticks[2 * (int64_t)blockIdx.x + 1] = w1 - w0;
    }
}

__global__ __launch_bounds__(256) void k_probe_copy(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                    int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}
}  // namespace

hipError_t launch_probe_mfma(int act, int64_t workgroups, int64_t iters, float* sink, int64_t* ticks,
                             hipStream_t s) {
    if (act == MOE_DTYPE_F32)
        launch_kernel(k_probe_mfma<MOE_DTYPE_F32>, dim3((unsigned)workgroups), dim3(256), 0, s, iters, sink, ticks);
    else
        launch_kernel(k_probe_mfma<MOE_DTYPE_BF16>, dim3((unsigned)workgroups), dim3(256), 0, s, iters, sink, ticks);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
    const int64_t n = bytes / 16;
    // four workgroups per CU, one 16-byte load and store per step: the fastest of the forms
    // measured on the box (5.8 TB/s at 1 GiB, against 4.2-5.3 TB/s for four or eight loads in
    // flight per thread, non-temporal or not, over 1024-16384 workgroups; hipMemcpy 5.2 TB/s)
    const int64_t grid = n / 256 < 1024 ? (n + 255) / 256 : 1024;
    launch_kernel(k_probe_copy, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const f32x4*>(src),
                  static_cast<f32x4*>(dst), n);
    return hipGetLastError();
}

}  // namespace moe
