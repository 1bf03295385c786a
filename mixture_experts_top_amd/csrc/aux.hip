// Load-balancing auxiliary loss and its gradient w.r.t. the gate logits.
//
// MoE-gate commit page ("11b96dac6a"), summary block: softmax of gate_logits plus the
// load-balancing loss frac . prob_mean x N_EXPERTS, scaled by lambda (lambda = 0.01 in
// the static form that the adaptive-lambda page "2d0e6b6bdc" replaces).  ARCHITECTURE
// block: this loss is the only differentiable signal into the gate.  The softmax is the
// max-shifted form of the softmax/cross-entropy page ("6cfd7e6691").
//
// With frac held constant (it is a count),
//   dL/dG[t, j] = (lambda N_E / T) p[t, j] (frac[j] - sum_e frac[e] p[t, e]).
// dG needs no global quantity other than frac, so one pass over G writes dG and the
// per-block column sums of p; a single-workgroup pass then forms mean_prob and the loss
// in a fixed order (no atomics).
#include "moe_internal.hpp"

namespace moe {

template <int NEB>
__global__ __launch_bounds__(kAuxThreads) void k_aux_rows(const float* __restrict__ G,
                                                          const int* __restrict__ counts, int T,
                                                          int NE, float lam_value,
                                                          const float* __restrict__ lam_dev,
                                                          float* __restrict__ dG,
                                                          float* __restrict__ probs,
                                                          float* __restrict__ part) {
    __shared__ float red[kAuxThreads / 64][NEB];
    const int tid = threadIdx.x;
    static_assert(kAuxTokens == kAuxThreads, "one token per thread");
    const int64_t t = (int64_t)blockIdx.x * kAuxTokens + tid;
    const bool vec = (NE % 4) == 0;
    // this token's logits first, then the counts: every load is unconditional (entries past
    // N_E read entry 0 and are never used), so they all go out before the first wait
    float g[NEB];
    const float* row = G + (t < T ? t : 0) * NE;
    if (vec) {  // entries past N_E re-read the row's first ones; every use is guarded by e < N_E
#pragma unroll
        for (int q = 0; q < NEB / 4; ++q) {
            const f32x4 v = reinterpret_cast<const f32x4*>(row)[4 * q < NE ? q : 0];
            g[4 * q] = v.x; g[4 * q + 1] = v.y; g[4 * q + 2] = v.z; g[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < NEB; ++e) g[e] = row[e < NE ? e : 0];
    }
    int cnt[NEB];
#pragma unroll
    for (int e = 0; e < NEB; ++e) cnt[e] = counts[e < NE ? e : 0];
    const float lam = lam_dev ? lam_dev[0] : lam_value;
    float frac[NEB], psum[NEB];
#pragma unroll
    for (int e = 0; e < NEB; ++e) {  // unguarded so the loads stay unconditional: p[e] = 0 past N_E
        frac[e] = (float)((double)cnt[e] / (double)T);
        psum[e] = 0.0f;
    }
    const float coef = (float)((double)lam * (double)NE / (double)T);
    if (t < T) {
        float m = g[0];
#pragma unroll
        for (int e = 1; e < NEB; ++e)
            if (e < NE) m = fmaxf(m, g[e]);
        float z[NEB], S = 0.0f;
#pragma unroll
        for (int e = 0; e < NEB; ++e) {
            z[e] = (e < NE) ? expf(g[e] - m) : 0.0f;
            S += z[e];
        }
        float p[NEB], sfp = 0.0f;
#pragma unroll
        for (int e = 0; e < NEB; ++e) {
            p[e] = z[e] / S;
            sfp += frac[e] * p[e];
            psum[e] += p[e];
        }
        float* drow = dG + t * NE;
        if (vec) {
#pragma unroll
            for (int q = 0; q < NEB / 4; ++q)
                if (4 * q < NE) {
                    f32x4 v;
                    v.x = coef * p[4 * q] * (frac[4 * q] - sfp);
                    v.y = coef * p[4 * q + 1] * (frac[4 * q + 1] - sfp);
                    v.z = coef * p[4 * q + 2] * (frac[4 * q + 2] - sfp);
                    v.w = coef * p[4 * q + 3] * (frac[4 * q + 3] - sfp);
                    reinterpret_cast<f32x4*>(drow)[q] = v;
                    if (probs)
                        reinterpret_cast<f32x4*>(probs + t * NE)[q] =
                            f32x4{p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]};
                }
        } else {
#pragma unroll
            for (int e = 0; e < NEB; ++e)
                if (e < NE) {
                    drow[e] = coef * p[e] * (frac[e] - sfp);
                    if (probs) probs[t * NE + e] = p[e];
                }
        }
    }
    // column sums of p over the block: butterfly within each wave (every lane ends with
    // the same bits), then the four wave sums in a fixed order.
    const int wave = tid / 64, lane = tid % 64;
#pragma unroll
    for (int e = 0; e < NEB; ++e) {
        float v = psum[e];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) red[wave][e] = v;
    }
    __syncthreads();
    if (tid < NE)
        part[(int64_t)blockIdx.x * NE + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// One workgroup: thread (s, e) sums blocks s, s+S, ... of column e; the S partial sums
// are then added in order; mean_prob, frac and the loss follow.
__global__ __launch_bounds__(256) void k_aux_final(const float* __restrict__ part,
                                                   const int* __restrict__ counts, int nblk, int T,
                                                   int NE, float lam_value, const float* __restrict__ lam_dev,
                                                   float* __restrict__ loss,
                                                   float* __restrict__ frac_out,
                                                   float* __restrict__ mean_prob_out) {
    __shared__ float acc[256];
    __shared__ float mp[kMaxExperts], fr[kMaxExperts];
    int nep = 1;
    while (nep < NE) nep <<= 1;
    const int S = 256 / nep;
    const int tid = threadIdx.x, e = tid % nep, s = tid / nep;
    float v = 0.0f;
    if (e < NE)
#pragma unroll 8
        for (int b = s; b < nblk; b += S) v += part[(int64_t)b * NE + e];
    acc[tid] = v;
    __syncthreads();
    if (tid < NE) {
        float tot = 0.0f;
        for (int q = 0; q < S; ++q) tot += acc[q * nep + tid];
        const float m = (float)((double)tot / (double)T);
        const float f = (float)((double)counts[tid] / (double)T);
        mp[tid] = m;
        fr[tid] = f;
        if (mean_prob_out) mean_prob_out[tid] = m;
        if (frac_out) frac_out[tid] = f;
    }
    __syncthreads();
    if (tid == 0) {
        const float lam = lam_dev ? lam_dev[0] : lam_value;
        double d = 0.0;
        for (int x = 0; x < NE; ++x) d += (double)fr[x] * (double)mp[x];
        loss[0] = (float)((double)lam * (double)NE * d);
    }
}

// Adaptive load-balancing weight (adaptive-lambda page, formula block), one thread:
//   lambda_eff = floor + max_extra * max(0, target - ent_ema) / target,  target = frac_t * ln(K)
__global__ void k_lambda_eff(const float* __restrict__ ent_ema, float floor_, float max_extra, float target_frac,
                             int K, float* __restrict__ lambda_eff) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    const double target = (double)target_frac * log((double)K);
    const double deficit = fmax(0.0, target - (double)ent_ema[0]);
    lambda_eff[0] = (float)((double)floor_ + (double)max_extra * deficit / target);
}

hipError_t launch_lambda_eff(const float* ent_ema, float floor_, float max_extra, float target_frac, int K,
                             float* lambda_eff, hipStream_t s) {
    launch_kernel(k_lambda_eff, dim3(1), dim3(64), 0, s, ent_ema, floor_, max_extra, target_frac, K, lambda_eff);
    return hipGetLastError();
}

hipError_t launch_aux_rows(const float* G, const int32_t* counts, int64_t T, int NE, float lam, const float* lam_dev,
                           float* dG, float* probs, float* part, int n_ablk, hipStream_t s) {
    dim3 grid(n_ablk), block(kAuxThreads);
    if (NE <= 4)
        launch_kernel(k_aux_rows<4>, grid, block, 0, s, G, counts, (int)T, NE, lam, lam_dev, dG, probs, part);
    else if (NE <= 8)
        launch_kernel(k_aux_rows<8>, grid, block, 0, s, G, counts, (int)T, NE, lam, lam_dev, dG, probs, part);
    else if (NE <= 16)
        launch_kernel(k_aux_rows<16>, grid, block, 0, s, G, counts, (int)T, NE, lam, lam_dev, dG, probs, part);
    else if (NE <= 32)
        launch_kernel(k_aux_rows<32>, grid, block, 0, s, G, counts, (int)T, NE, lam, lam_dev, dG, probs, part);
    else
        launch_kernel(k_aux_rows<64>, grid, block, 0, s, G, counts, (int)T, NE, lam, lam_dev, dG, probs, part);
    return hipGetLastError();
}

hipError_t launch_aux_final(const float* part, const int32_t* counts, int n_ablk, int64_t T, int NE,
                            float lam, const float* lam_dev, float* loss, float* frac, float* mean_prob,
                            hipStream_t s) {
    launch_kernel(k_aux_final, dim3(1), dim3(256), 0, s, part, counts, n_ablk, (int)T, NE, lam, lam_dev, loss,
                       frac, mean_prob);
    return hipGetLastError();
}

}  // namespace moe
