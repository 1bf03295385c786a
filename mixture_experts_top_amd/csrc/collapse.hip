// Horizon mean collapse (MHA page "9170d24fe3", new-kernel block): [B, N_H, H] -> [B, H] by
// averaging over the horizon axis, single pass, no cross-thread reduction; its backward
// gives every horizon d_out[b] / N_H.  Both scale by the fp32 reciprocal of N_H.
//
// One thread per (b, 16-byte column group): the forward sums the N_H rows of its column in
// horizon order, so accesses are coalesced along H and the result is deterministic.
// Streams touched once go through non-temporal accesses (no reusable cache lines): measured at
// B = 131,072, N_H = 8, H = 256 fp32, the forward with non-temporal loads and stores 5.40 ->
// 6.19 TB/s, the backward with non-temporal stores 5.25 -> 6.18 TB/s (its reads of d_out as
// non-temporal loads: 4.92 TB/s, slower).
#include "moe_internal.hpp"

namespace moe {

namespace {
__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t to_bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
}  // namespace

__global__ __launch_bounds__(256) void k_collapse_fwd_f32(const float* __restrict__ x, float* __restrict__ out,
                                                          int64_t B, int NH, int H) {
    const int q = H / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= B * q) return;
    const int64_t b = i / q, c = (i % q) * 4;
    const float inv = 1.0f / (float)NH;
    f32x4 s = f32x4{};
    for (int h = 0; h < NH; ++h) s += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + (b * NH + h) * H + c));
    __builtin_nontemporal_store(s * inv, reinterpret_cast<f32x4*>(out + b * H + c));
}

// One thread per (b, 16-byte column group): d_out[b] is read once and written to the N_H rows.
__global__ __launch_bounds__(256) void k_collapse_bwd_f32(const float* __restrict__ dout, float* __restrict__ dx,
                                                          int64_t B, int NH, int H) {
    const int q = H / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over B * q
    if (i >= B * q) return;
    const int64_t b = i / q, c = (i % q) * 4;
    const float inv = 1.0f / (float)NH;
    const f32x4 v = *reinterpret_cast<const f32x4*>(dout + b * H + c) * inv;
    for (int h = 0; h < NH; ++h) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dx + (b * NH + h) * H + c));
}

__global__ __launch_bounds__(256) void k_collapse_fwd_bf16(const uint16_t* __restrict__ x, uint16_t* __restrict__ out,
                                                           int64_t B, int NH, int H) {
    const int q = H / 8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= B * q) return;
    const int64_t b = i / q, c = (i % q) * 8;
    const float inv = 1.0f / (float)NH;
    float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int h = 0; h < NH; ++h) {
        const u16x8 v = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(x + (b * NH + h) * H + c));
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] += bf(v[j]);
    }
    u16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = to_bf(s[j] * inv);
    __builtin_nontemporal_store(o, reinterpret_cast<u16x8*>(out + b * H + c));
}

__global__ __launch_bounds__(256) void k_collapse_bwd_bf16(const uint16_t* __restrict__ dout, uint16_t* __restrict__ dx,
                                                           int64_t B, int NH, int H) {
    const int q = H / 8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over B * q
    if (i >= B * q) return;
    const int64_t b = i / q, c = (i % q) * 8;
    const float inv = 1.0f / (float)NH;
    const u16x8 v = *reinterpret_cast<const u16x8*>(dout + b * H + c);
    u16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = to_bf(bf(v[j]) * inv);
    for (int h = 0; h < NH; ++h) __builtin_nontemporal_store(o, reinterpret_cast<u16x8*>(dx + (b * NH + h) * H + c));
}

hipError_t launch_collapse(bool bwd, int act, const void* in, void* out, int64_t B, int NH, int H, hipStream_t s) {
    const int per = (act == 0) ? 4 : 8;
    const int64_t n = B * (H / per);  // one thread per (b, column group), both directions
    const dim3 grid((unsigned)((n + 255) / 256));
    if (act == 0) {
        if (bwd)
            launch_kernel(k_collapse_bwd_f32, grid, dim3(256), 0, s, (const float*)in, (float*)out, B, NH, H);
        else
            launch_kernel(k_collapse_fwd_f32, grid, dim3(256), 0, s, (const float*)in, (float*)out, B, NH, H);
    } else {
        if (bwd)
            launch_kernel(k_collapse_bwd_bf16, grid, dim3(256), 0, s, (const uint16_t*)in, (uint16_t*)out, B, NH,
                               H);
        else
            launch_kernel(k_collapse_fwd_bf16, grid, dim3(256), 0, s, (const uint16_t*)in, (uint16_t*)out, B, NH,
                               H);
    }
    return hipGetLastError();
}

}  // namespace moe
