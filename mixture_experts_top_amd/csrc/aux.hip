// Load-balancing auxiliary loss and its gradient w.r.t. the gate logits.
//
// MoE-gate commit page ("11b96dac6a"), summary block: softmax of gate_logits plus the
// load-balancing loss frac . prob_mean x N_EXPERTS, scaled by lambda (lambda = 0.01 in
// the static form that the adaptive-lambda page "2d0e6b6bdc" replaces).  ARCHITECTURE
// block: this loss is the only differentiable signal into the gate.  The per-token
// arithmetic is in aux_math.hpp.
//
// dG needs no global quantity other than frac, so one pass over G writes dG and the
// per-block column sums of p; a single-workgroup pass then forms mean_prob and the loss
// in a fixed order (no atomics).
#include "aux_math.hpp"

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
    __shared__ float sfrac[NEB];
    static_assert(kAuxTokens == kAuxThreads, "one token per thread");
    const int tid = threadIdx.x;
    const int64_t t = (int64_t)blockIdx.x * kAuxTokens + tid;
    float g[NEB];
    aux_load_logits<NEB>(G, t, T, NE, g);
    const int cnt_mine = counts[tid < NE ? tid : 0];  // entries past N_E are unused
    const float lam = lam_dev ? lam_dev[0] : lam_value;
    float frac[NEB], psum[NEB];
    aux_frac_table<NEB>(cnt_mine, T, sfrac, frac);
#pragma unroll
    for (int e = 0; e < NEB; ++e) psum[e] = 0.0f;
    if (t < T) {
        float p[NEB];
        aux_softmax<NEB>(g, NE, p);
        aux_grad_row<NEB>(p, frac, aux_coef(lam, NE, T), NE, t, dG, probs);
#pragma unroll
        for (int e = 0; e < NEB; ++e) psum[e] = p[e];
    }
    aux_block_colsum<NEB>(psum, red, NE, part + (int64_t)blockIdx.x * NE);
}

__global__ __launch_bounds__(256) void k_aux_final(const float* __restrict__ part,
                                                   const int* __restrict__ counts, int nblk, int T,
                                                   int NE, float lam_value, const float* __restrict__ lam_dev,
                                                   float* __restrict__ loss,
                                                   float* __restrict__ frac_out,
                                                   float* __restrict__ mean_prob_out) {
    __shared__ float acc[256];
    __shared__ float mp[kMaxExperts], fr[kMaxExperts];
    const int tid = threadIdx.x;
    const int cnt = tid < NE ? counts[tid] : 0;
    const float lam = lam_dev ? lam_dev[0] : lam_value;
    aux_final_block(part, cnt, nblk, T, NE, lam, loss, frac_out, mean_prob_out, acc, mp, fr);
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
