// Per-token arithmetic of the load-balancing auxiliary loss, shared by every kernel that
// computes a part of it (the aux kernels, the routing kernel that also sums the softmax
// columns, and the forward GEMM or the scatter kernels that also write the logit gradient
// and the loss), so that each part gives the same bits wherever it runs.
//
// MoE-gate commit page ("11b96dac6a"), summary block: softmax of the gate logits and the
// loss lambda N_E sum_e frac[e] mean_prob[e]; the softmax is the max-shifted form of the
// softmax/cross-entropy page ("6cfd7e6691").  With frac held constant (it is a count),
//   dL/dG[t, j] = (lambda N_E / T) p[t, j] (frac[j] - sum_e frac[e] p[t, e]).
// NEB is N_E rounded up to a supported register width; entries past N_E are never used
// (they hold zero probability).
#pragma once

#include "moe_internal.hpp"

namespace moe {

// Token t's logits.  Every load is unconditional (a token past T reads token 0's row,
// entries past N_E re-read the row's first ones), so all of them go out before the
// first wait; the caller ignores what such loads return.
template <int NEB>
__device__ __forceinline__ void aux_load_logits(const float* __restrict__ G, int64_t t, int64_t T, int NE,
                                                float (&g)[NEB]) {
    const float* row = G + (t < T ? t : 0) * NE;
    if ((NE % 4) == 0) {
#pragma unroll
        for (int q = 0; q < NEB / 4; ++q) {
            const f32x4 v = reinterpret_cast<const f32x4*>(row)[4 * q < NE ? q : 0];
            g[4 * q] = v.x; g[4 * q + 1] = v.y; g[4 * q + 2] = v.z; g[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < NEB; ++e) g[e] = row[e < NE ? e : 0];
    }
}

// p = softmax(g[0 .. N_E)) with the row maximum subtracted; p[e] = 0 for e >= N_E.
template <int NEB>
__device__ __forceinline__ void aux_softmax(const float (&g)[NEB], int NE, float (&p)[NEB]) {
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
#pragma unroll
    for (int e = 0; e < NEB; ++e) p[e] = z[e] / S;
}

// frac_e = count_e / T (in double, rounded once).
__device__ __forceinline__ float aux_frac_of(int count, int64_t T) { return (float)((double)count / (double)T); }

// Every thread's frac[0 .. NEB) from a per-workgroup table: threads e < NEB form entry e
// from count_mine (their expert's count; entries past N_E are unused) once, instead of every
// thread dividing in double N_E times.  Contains a barrier: every thread calls it.
template <int NEB>
__device__ __forceinline__ void aux_frac_table(int count_mine, int64_t T, float* sfrac, float (&frac)[NEB]) {
    if ((int)threadIdx.x < NEB) sfrac[threadIdx.x] = aux_frac_of(count_mine, T);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NEB; ++e) frac[e] = sfrac[e];
}

__device__ __forceinline__ float aux_coef(float lam, int NE, int64_t T) {
    return (float)((double)lam * (double)NE / (double)T);
}

// Writes dG[t, :] (and probs[t, :] when non-null) for one token.
template <int NEB>
__device__ __forceinline__ void aux_grad_row(const float (&p)[NEB], const float (&frac)[NEB], float coef, int NE,
                                             int64_t t, float* __restrict__ dG, float* __restrict__ probs) {
    float sfp = 0.0f;
#pragma unroll
    for (int e = 0; e < NEB; ++e) sfp += frac[e] * p[e];
    float* drow = dG + t * NE;
    if ((NE % 4) == 0) {
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

// Column sums of p over a workgroup of 256 threads (one token each; psum = 0 for tokens
// past T): each wavefront's sum in the fixed order of wave_sum, then the four wavefront sums
// in a fixed order, written to part_row[0 .. N_E).  Contains a barrier: every thread of the
// workgroup calls it.
template <int NEB>
__device__ __forceinline__ void aux_block_colsum(const float (&psum)[NEB], float (*red)[NEB], int NE,
                                                 float* __restrict__ part_row) {
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
#pragma unroll
    for (int e = 0; e < NEB; ++e) {
        const float v = wave_sum(psum[e]);
        if (lane == 0) red[wave][e] = v;
    }
    __syncthreads();
    if (tid < NE) part_row[tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// v += part[b][e] for b = s, s + S, ... < nblk in ascending order, NB loads in flight.
template <int NB>
__device__ __forceinline__ void aux_colsum_batched(const float* __restrict__ part, int nblk, int NE, int S, int s,
                                                   int e, float& v) {
    for (int b0 = s; b0 < nblk; b0 += NB * S) {
        float pv[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int b = b0 + u * S;
            pv[u] = part[(int64_t)(b < nblk ? b : s) * NE + e];
        }
#pragma unroll
        for (int u = 0; u < NB; ++u)
            if (b0 + u * S < nblk) v += pv[u];
    }
}

// One workgroup of 256 threads: mean_prob from the per-block column sums (thread (s, e)
// sums blocks s, s + S, ... of column e, then the S partial sums are added in order),
// frac from the counts (thread e < N_E passes count_e), and the loss.  acc: 256 floats of
// LDS; mp, fr: kMaxExperts floats each.
__device__ __forceinline__ void aux_final_block(const float* __restrict__ part, int count_mine, int nblk, int64_t T,
                                                int NE, float lam, float* __restrict__ loss,
                                                float* __restrict__ frac_out, float* __restrict__ mean_prob_out,
                                                float* acc, float* mp, float* fr) {
    int nep = 1;
    while (nep < NE) nep <<= 1;
    const int S = 256 / nep;
    const int tid = threadIdx.x, e = tid % nep, s = tid / nep;
    float v = 0.0f;
    if (e < NE && s < nblk) {
        // blocks s, s + S, ... in ascending order, loaded NB at a time (a block past nblk
        // re-reads block s and is not added), so a thread waits once per batch, not once per
        // block: 8 per batch when a thread has at most 8 blocks, else 32
        if (nblk <= 8 * S)
            aux_colsum_batched<8>(part, nblk, NE, S, s, e, v);
        else
            aux_colsum_batched<32>(part, nblk, NE, S, s, e, v);
    }
    acc[tid] = v;
    __syncthreads();
    if (tid < NE) {
        float tot = 0.0f;
        for (int q = 0; q < S; ++q) tot += acc[q * nep + tid];
        const float m = (float)((double)tot / (double)T);
        const float f = aux_frac_of(count_mine, T);
        mp[tid] = m;
        fr[tid] = f;
        if (mean_prob_out) mean_prob_out[tid] = m;
        if (frac_out) frac_out[tid] = f;
    }
    __syncthreads();
    if (tid == 0) {
        double d = 0.0;
        for (int x = 0; x < NE; ++x) d += (double)fr[x] * (double)mp[x];
        loss[0] = (float)((double)lam * (double)NE * d);
    }
}

}  // namespace moe
