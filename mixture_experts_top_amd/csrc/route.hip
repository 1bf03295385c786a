// Routing and the stable counting sort by expert.
//
// Top-1 routing follows the MoE-gate commit page ("11b96dac6a"), summary and
// PERFORMANCE blocks: each (b, h) token goes to the expert with the largest gate logit.
// The page lets one thread scan the logits serially; a strict ">" scan upward from
// expert 0 gives the lowest index among equal maxima, and every thread here does the
// same scan for its own token.
//
// The counting sort (histogram -> scan -> scatter) has no counterpart on the pages; it
// groups the tokens of each expert so that the expert linears become dense GEMMs.
// Ranks inside a block come from wavefront ballots (lane order = token order), so the
// permutation is stable and no atomics are used anywhere.
#include "aux_math.hpp"

namespace moe {

// Ranks each lane's expert among the lanes of its wave with the same expert.
// Returns the rank (number of lower lanes with the same expert); for every expert that
// occurs, the lowest such lane stores the wave's count into cnt[e].
// e < 0 marks an inactive lane.
__device__ __forceinline__ int wave_rank(int e, int* cnt /* nullable */) {
    const int lane = __lane_id();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint64_t active = __ballot(e >= 0);
    int rank = 0;
    while (active) {
        const int leader = __ffsll((unsigned long long)active) - 1;
        const int el = __builtin_amdgcn_readlane(e, leader);
        const uint64_t m = __ballot(e == el);
        if (e == el) rank = __popcll(m & lt);
        if (cnt && lane == leader) cnt[el] = __popcll(m);
        active &= ~m;
    }
    return rank;
}

// One block: tokens [blk*256, blk*256+256), one per thread.  Writes expert_idx (if non-null)
// and the block's histogram hist[blk, :].  The token's logits are loaded all at once
// (aux_load_logits: no load waits on another), then scanned in registers.
template <int NEB>
__global__ __launch_bounds__(kRouteThreads) void k_route(const float* __restrict__ G, int T, int NE,
                                                         int* __restrict__ idx_out,
                                                         int* __restrict__ hist) {
    static_assert(kRouteThreads == kRouteTokens && kRouteGroups == kRouteThreads / 64, "one token per thread");
    __shared__ int cnt[kRouteGroups][kMaxExperts];
    const int tid = threadIdx.x;
    for (int i = tid; i < kRouteGroups * kMaxExperts; i += kRouteThreads) (&cnt[0][0])[i] = 0;
    const int64_t t = (int64_t)blockIdx.x * kRouteTokens + tid;
    float g[NEB];
    aux_load_logits<NEB>(G, t, T, NE, g);
    __syncthreads();
    int e = -1;
    if (t < T) {
        // strict ">" upward from expert 0: the lowest index among equal maxima
        float best = g[0];
        e = 0;
#pragma unroll
        for (int x = 1; x < NEB; ++x)
            if (x < NE && g[x] > best) {
                best = g[x];
                e = x;
            }
        if (idx_out) idx_out[t] = e;
    }
    wave_rank(e, cnt[tid / 64]);
    __syncthreads();
    if (tid < NE) {
        int s = 0;
        for (int g = 0; g < kRouteGroups; ++g) s += cnt[g][tid];
        hist[(int64_t)blockIdx.x * NE + tid] = s;
    }
}

// k_route with the first half of the load-balancing loss folded in: besides expert_idx
// and hist[blk, :], the block's column sums of the gate softmax, part[blk, :] -- the same
// bits k_aux_rows writes for these 256 tokens (aux_math.hpp), so the aux pass that
// follows needs no column sums of its own.  The logits are loaded once for both.
template <int NEB>
__global__ __launch_bounds__(kRouteThreads) void k_route_part(const float* __restrict__ G, int T, int NE,
                                                              int* __restrict__ idx_out, int* __restrict__ hist,
                                                              float* __restrict__ part) {
    static_assert(kRouteThreads == kRouteTokens && kRouteTokens == kAuxTokens && kRouteGroups == 4,
                  "one token per thread, routing blocks = aux blocks");
    __shared__ int cnt[kRouteGroups][kMaxExperts];
    __shared__ float red[kRouteGroups][NEB];
    const int tid = threadIdx.x;
    for (int i = tid; i < kRouteGroups * kMaxExperts; i += kRouteThreads) (&cnt[0][0])[i] = 0;
    const int64_t t = (int64_t)blockIdx.x * kRouteTokens + tid;
    float g[NEB];
    aux_load_logits<NEB>(G, t, T, NE, g);
    __syncthreads();
    int e = -1;
    float psum[NEB];
#pragma unroll
    for (int x = 0; x < NEB; ++x) psum[x] = 0.0f;
    if (t < T) {
        // strict ">" upward from expert 0: the lowest index among equal maxima
        float best = g[0];
        e = 0;
#pragma unroll
        for (int x = 1; x < NEB; ++x)
            if (x < NE && g[x] > best) {
                best = g[x];
                e = x;
            }
        if (idx_out) idx_out[t] = e;
        float p[NEB];
        aux_softmax<NEB>(g, NE, p);
#pragma unroll
        for (int x = 0; x < NEB; ++x) psum[x] = p[x];
    }
    wave_rank(e, cnt[tid / 64]);
    aux_block_colsum<NEB>(psum, red, NE, part + (int64_t)blockIdx.x * NE);  // its barrier orders cnt too
    if (tid < NE) {
        int s = 0;
        for (int w = 0; w < kRouteGroups; ++w) s += cnt[w][tid];
        hist[(int64_t)blockIdx.x * NE + tid] = s;
    }
}

// One workgroup of 1024 threads.  Thread (s, e) owns a contiguous segment of blocks for
// expert e; segment totals are scanned in LDS, then every block gets its global base
// position blkbase[blk, e] = offsets[e] + (tokens of expert e in earlier blocks).
__global__ __launch_bounds__(kScanThreads) void k_scan(const int* __restrict__ hist, int nblk, int NE,
                                                       int* __restrict__ blkbase,
                                                       int* __restrict__ counts,
                                                       int* __restrict__ offsets) {
    __shared__ int tot[kScanThreads];
    __shared__ int ex_off[kMaxExperts + 1];
    int nep = 1;
    while (nep < NE) nep <<= 1;
    const int S = kScanThreads / nep;  // segments per expert
    const int tid = threadIdx.x;
    const int e = tid % nep, s = tid / nep;
    const int L = (nblk + S - 1) / S;
    const int b0 = min(nblk, s * L), b1 = min(nblk, b0 + L);
    int sum = 0;
    if (e < NE)
#pragma unroll 8
        for (int b = b0; b < b1; ++b) sum += hist[(int64_t)b * NE + e];
    tot[s * nep + e] = sum;
    __syncthreads();
    // inclusive scan over s for each e (Hillis-Steele)
    for (int d = 1; d < S; d <<= 1) {
        int v = (s >= d) ? tot[(s - d) * nep + e] : 0;
        __syncthreads();
        tot[s * nep + e] += v;
        __syncthreads();
    }
    if (tid == 0) {
        int acc = 0;
        ex_off[0] = 0;
        for (int x = 0; x < NE; ++x) {
            int c = tot[(S - 1) * nep + x];
            counts[x] = c;
            acc += c;
            ex_off[x + 1] = acc;
        }
        for (int x = 0; x <= NE; ++x) offsets[x] = ex_off[x];
    }
    __syncthreads();
    if (e < NE) {
        int run = ex_off[e] + ((s > 0) ? tot[(s - 1) * nep + e] : 0);
#pragma unroll 8
        for (int b = b0; b < b1; ++b) {
            blkbase[(int64_t)b * NE + e] = run;
            run += hist[(int64_t)b * NE + e];
        }
    }
}

// The aux loss riding on a scatter launch (NEB > 0): the counts are final there, so each
// scatter block also writes dG (and probs) for its 256 tokens -- the tokens of k_aux_rows'
// block of the same index, with the same arithmetic (aux_math.hpp) -- and one extra block
// (blockIdx.x == nblk) forms mean_prob, frac and the loss from the column sums that
// k_route_part wrote in the launch before, as k_aux_final does.
template <int NEB>
__device__ __forceinline__ void scatter_aux_rows(const AuxFwdArgs& ax, const float (&g)[NEB], int count_mine,
                                                 int64_t t, int T, int NE, float* sfrac) {
    const float lam = ax.lam_dev ? ax.lam_dev[0] : ax.lam;
    float frac[NEB];
    aux_frac_table<NEB>(count_mine, T, sfrac, frac);  // contains a barrier
    if (t < T) {
        float p[NEB];
        aux_softmax<NEB>(g, NE, p);
        aux_grad_row<NEB>(p, frac, aux_coef(lam, NE, T), NE, t, ax.dG, ax.probs);
    }
}
__device__ __forceinline__ void scatter_aux_final(const AuxFwdArgs& ax, int count_mine, int T, int NE) {
    __shared__ float acc[256];
    __shared__ float mp[kMaxExperts], fr[kMaxExperts];
    static_assert(kRouteThreads == 256, "aux_final_block runs on 256 threads");
    const float lam = ax.lam_dev ? ax.lam_dev[0] : ax.lam;
    aux_final_block(ax.part, count_mine, ax.n_ablk, T, NE, lam, ax.loss, ax.frac, ax.mean_prob, acc, mp, fr);
}

// Same block decomposition as k_route.  Recomputes the in-block ranks from expert_idx
// and writes perm[blkbase[blk, e] + rank] = t.  With NEB > 0 it also runs the aux rows
// (counts from k_scan, final by then) and, in block nblk, the aux final.
template <int NEB>
__global__ __launch_bounds__(kRouteThreads) void k_scatter(const int* __restrict__ idx, int T, int NE,
                                                           const int* __restrict__ blkbase,
                                                           int* __restrict__ perm, const int* __restrict__ counts,
                                                           AuxFwdArgs ax) {
    __shared__ int cnt[kRouteGroups][kMaxExperts];
    __shared__ int bb[kMaxExperts];
    const int tid = threadIdx.x;
    const int nblk = (int)gridDim.x - (NEB > 0 ? 1 : 0);
    if constexpr (NEB > 0) {
        if ((int)blockIdx.x == nblk) {
            scatter_aux_final(ax, tid < NE ? counts[tid] : 0, T, NE);
            return;
        }
    }
    for (int i = tid; i < kRouteGroups * kMaxExperts; i += kRouteThreads) (&cnt[0][0])[i] = 0;
    if (tid < NE) bb[tid] = blkbase[(int64_t)blockIdx.x * NE + tid];
    __syncthreads();
    const int wave = tid / 64, lane = tid % 64;
    const int64_t base = (int64_t)blockIdx.x * kRouteTokens;
    constexpr int GPW = kRouteGroups / (kRouteThreads / 64);  // groups per wave
    float gl[NEB > 0 ? NEB : 1];
    int cmine = 0;
    if constexpr (NEB > 0) {  // this thread's token (one per thread, as in k_aux_rows) and counts
        aux_load_logits<NEB>(ax.G, base + tid, T, NE, gl);
        cmine = counts[tid < NE ? tid : 0];
    }
    int my_e[GPW], my_rank[GPW];
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int g = wave + j * (kRouteThreads / 64);
        const int64_t t = base + g * 64 + lane;
        const int e = (t < T) ? idx[t] : -1;
        my_e[j] = e;
        my_rank[j] = wave_rank(e, cnt[g]);
    }
    __syncthreads();
    // exclusive prefix over groups, per expert
    if (tid < NE) {
        int run = 0;
        for (int g = 0; g < kRouteGroups; ++g) {
            int c = cnt[g][tid];
            cnt[g][tid] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int g = wave + j * (kRouteThreads / 64);
        const int e = my_e[j];
        if (e >= 0) {
            const int64_t t = base + g * 64 + lane;
            perm[bb[e] + cnt[g][e] + my_rank[j]] = (int)t;
        }
    }
    if constexpr (NEB > 0) {
        __shared__ float sfrac[NEB];
        scatter_aux_rows<NEB>(ax, gl, cmine, base + tid, T, NE, sfrac);
    }
}

// Scatter with the scan folded in, for small histograms (n_blk x N_E entries): every block
// sums the histogram columns itself (all blocks -> counts and offsets, earlier blocks -> its
// own base), so routing is two launches.  Block 0 writes counts and offsets.
static_assert(kRouteGroups == kRouteThreads / 64, "one 64-token group per wavefront");

// With NEB > 0 the aux rows ride on it too (see scatter_aux_rows), and block nblk sums the
// histogram like the others, then runs the aux final.
template <int NEB>
__global__ __launch_bounds__(kRouteThreads) void k_scatter_scan(const int* __restrict__ idx, int T, int NE,
                                                                const int* __restrict__ hist, int nblk,
                                                                int* __restrict__ counts, int* __restrict__ offsets,
                                                                int* __restrict__ perm, AuxFwdArgs ax) {
    __shared__ int cnt[kRouteGroups][kMaxExperts];
    __shared__ int part[2][kRouteThreads];
    __shared__ int bb[kMaxExperts];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const bool final_blk = NEB > 0 && b == nblk;
    // this thread's token's expert: its load goes out first, with the histogram loads behind it
    const int wave = tid / 64, lane = tid % 64;
    const int64_t t = (int64_t)b * kRouteTokens + wave * 64 + lane;
    const int e = (t < T && !final_blk) ? idx[t] : -1;
    float gl[NEB > 0 ? NEB : 1];
    if constexpr (NEB > 0) aux_load_logits<NEB>(ax.G, (int64_t)b * kRouteTokens + tid, T, NE, gl);
    int nep = 1;
    while (nep < NE) nep <<= 1;
    const int S = kRouteThreads / nep;
    {
        const int ec = tid % nep, sg = tid / nep;
        int all = 0, before = 0;
        if (ec < NE && sg < nblk) {
            // 8 loads at a time, all unconditional (a block past nblk re-reads block sg and is
            // not counted): one memory round trip per batch
            for (int x0 = sg; x0 < nblk; x0 += 8 * S) {
                int hv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int x = x0 + u * S;
                    hv[u] = hist[(int64_t)(x < nblk ? x : sg) * NE + ec];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int x = x0 + u * S;
                    if (x < nblk) {
                        all += hv[u];
                        before += (x < b) ? hv[u] : 0;
                    }
                }
            }
        }
        part[0][tid] = all;
        part[1][tid] = before;
    }
    for (int i = tid; i < kRouteGroups * kMaxExperts; i += kRouteThreads) (&cnt[0][0])[i] = 0;
    __syncthreads();
    // tree over the S segments of each expert (integer sums: exact in any order)
    for (int half = S / 2; half >= 1; half >>= 1) {
        if (tid / nep < half) {
            part[0][tid] += part[0][tid + half * nep];
            part[1][tid] += part[1][tid + half * nep];
        }
        __syncthreads();
    }
    if (tid == 0) {
        int acc = 0;
        for (int e = 0; e < NE; ++e) {
            const int tot = part[0][e];
            bb[e] = acc + part[1][e];
            if (b == 0) {
                counts[e] = tot;
                offsets[e] = acc;
            }
            acc += tot;
        }
        if (b == 0) offsets[NE] = acc;
    }
    __syncthreads();
    if constexpr (NEB > 0) {
        if (final_blk) {  // the totals of every expert are in part[0][0 .. N_E)
            scatter_aux_final(ax, tid < NE ? part[0][tid] : 0, T, NE);
            return;
        }
    }
    const int r = wave_rank(e, cnt[wave]);
    __syncthreads();
    if (tid < NE) {
        int run = 0;
        for (int g = 0; g < kRouteGroups; ++g) {
            const int c = cnt[g][tid];
            cnt[g][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    if (e >= 0) perm[bb[e] + cnt[wave][e] + r] = (int)t;
    if constexpr (NEB > 0) {
        __shared__ float sfrac[NEB];
        scatter_aux_rows<NEB>(ax, gl, part[0][tid < NE ? tid : 0], (int64_t)b * kRouteTokens + tid, T, NE, sfrac);
    }
}

bool scatter_scan_fits(int n_rblk, int NE) { return (int64_t)n_rblk * NE <= 4096; }

hipError_t launch_scatter_scan(const int32_t* idx, int64_t T, int NE, const int32_t* hist, int n_rblk,
                               int32_t* counts, int32_t* offsets, int32_t* perm, hipStream_t s) {
    launch_kernel(k_scatter_scan<0>, dim3(n_rblk), dim3(kRouteThreads), 0, s, idx, (int)T, NE, hist, n_rblk,
                  counts, offsets, perm, AuxFwdArgs{});
    return hipGetLastError();
}

hipError_t launch_scatter_scan_aux(const int32_t* idx, int64_t T, int NE, const int32_t* hist, int n_rblk,
                                   int32_t* counts, int32_t* offsets, int32_t* perm, const AuxFwdArgs& ax,
                                   hipStream_t s) {
    const dim3 grid(n_rblk + 1), block(kRouteThreads);
    if (NE <= 4)
        launch_kernel(k_scatter_scan<4>, grid, block, 0, s, idx, (int)T, NE, hist, n_rblk, counts, offsets, perm, ax);
    else if (NE <= 8)
        launch_kernel(k_scatter_scan<8>, grid, block, 0, s, idx, (int)T, NE, hist, n_rblk, counts, offsets, perm, ax);
    else if (NE <= 16)
        launch_kernel(k_scatter_scan<16>, grid, block, 0, s, idx, (int)T, NE, hist, n_rblk, counts, offsets, perm, ax);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_route(const float* G, int64_t T, int NE, int32_t* idx, int32_t* hist, int n_rblk,
                        hipStream_t s) {
    const dim3 grid(n_rblk), block(kRouteThreads);
    if (NE <= 4)
        launch_kernel(k_route<4>, grid, block, 0, s, G, (int)T, NE, idx, hist);
    else if (NE <= 8)
        launch_kernel(k_route<8>, grid, block, 0, s, G, (int)T, NE, idx, hist);
    else if (NE <= 16)
        launch_kernel(k_route<16>, grid, block, 0, s, G, (int)T, NE, idx, hist);
    else if (NE <= 32)
        launch_kernel(k_route<32>, grid, block, 0, s, G, (int)T, NE, idx, hist);
    else
        launch_kernel(k_route<64>, grid, block, 0, s, G, (int)T, NE, idx, hist);
    return hipGetLastError();
}

hipError_t launch_route_part(const float* G, int64_t T, int NE, int32_t* idx, int32_t* hist, float* part,
                             int n_rblk, hipStream_t s) {
    if (NE <= 4)
        launch_kernel(k_route_part<4>, dim3(n_rblk), dim3(kRouteThreads), 0, s, G, (int)T, NE, idx, hist, part);
    else if (NE <= 8)
        launch_kernel(k_route_part<8>, dim3(n_rblk), dim3(kRouteThreads), 0, s, G, (int)T, NE, idx, hist, part);
    else if (NE <= 16)
        launch_kernel(k_route_part<16>, dim3(n_rblk), dim3(kRouteThreads), 0, s, G, (int)T, NE, idx, hist, part);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_scan(const int32_t* hist, int n_rblk, int NE, int32_t* blkbase, int32_t* counts,
                       int32_t* offsets, hipStream_t s) {
    launch_kernel(k_scan, dim3(1), dim3(kScanThreads), 0, s, hist, n_rblk, NE, blkbase, counts,
                       offsets);
    return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* idx, int64_t T, int NE, const int32_t* blkbase, int32_t* perm,
                          int n_rblk, hipStream_t s) {
    launch_kernel(k_scatter<0>, dim3(n_rblk), dim3(kRouteThreads), 0, s, idx, (int)T, NE, blkbase, perm,
                  (const int*)nullptr, AuxFwdArgs{});
    return hipGetLastError();
}

hipError_t launch_scatter_aux(const int32_t* idx, int64_t T, int NE, const int32_t* blkbase, int32_t* perm,
                              const int32_t* counts, int n_rblk, const AuxFwdArgs& ax, hipStream_t s) {
    const dim3 grid(n_rblk + 1), block(kRouteThreads);
    if (NE <= 4)
        launch_kernel(k_scatter<4>, grid, block, 0, s, idx, (int)T, NE, blkbase, perm, counts, ax);
    else if (NE <= 8)
        launch_kernel(k_scatter<8>, grid, block, 0, s, idx, (int)T, NE, blkbase, perm, counts, ax);
    else if (NE <= 16)
        launch_kernel(k_scatter<16>, grid, block, 0, s, idx, (int)T, NE, blkbase, perm, counts, ax);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
