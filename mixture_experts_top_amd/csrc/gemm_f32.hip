// Grouped expert GEMMs in fp32 on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Once tokens are grouped by expert (perm, offsets), the per-token expert linear of the
// MoE-gate commit page ("11b96dac6a", summary and PERFORMANCE blocks) becomes one dense
// GEMM per expert:
//   forward   Y[t]  = W[e] x[t] + b[e]           rows of X gathered through perm
//   backward  dX[t] = W[e]^T dY[t]               same tiling, W read untransposed
//             dW[e] = sum_t dY[t] (outer) x[t]   K = the expert's tokens, split into
//             db[e] = sum_t dY[t]                fixed chunks; partials summed later in
//                                                chunk order (no atomics)
// The page's design (one block per token, one thread per output channel, per-token
// scratch for dW) is replaced by tiles of 128 tokens staged in LDS and fed to MFMA.
//
// v_mfma_f32_32x32x2_f32 operand layout (lane l, half h = l / 32):
//   A[m][k]: m = l % 32, k = h          B[k][n]: n = l % 32, k = h
//   D[m][n] (16 accumulators r): n = l % 32, m = 8 (r / 4) + 4 h + (r % 4)
// The K dimension of consecutive instructions may be assigned to lanes in any order as
// long as A and B agree; here lane half h of step s in a group of 8 covers k = 4h + s, so
// a lane fetches four consecutive k with one 16-byte LDS read when K is contiguous.
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;   // 4 waves, arranged 2 x 2 over the output tile
constexpr int kPad = 4;         // LDS row padding (floats): keeps 16-byte alignment, spreads banks

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Finds the expert and row range of M-tile `mt` when every expert's rows are cut into
// tiles of `bm`.  Returns false if mt is past the last tile.
__device__ __forceinline__ bool find_tile(const int* __restrict__ offsets, int NE, int mt, int bm,
                                          int& e, int& r0, int& r1) {
    int acc = 0;
    for (int i = 0; i < NE; ++i) {
        const int c0 = offsets[i], c1 = offsets[i + 1];
        const int n = (c1 - c0 + bm - 1) / bm;
        if (mt < acc + n) {
            e = i;
            r0 = c0 + (mt - acc) * bm;
            r1 = min(c1, r0 + bm);
            return true;
        }
        acc += n;
    }
    return false;
}

// Workgroup ids are dealt to the 8 XCDs round-robin.  The `per` tiles that share one
// operand block get ids id, id+8, id+16, ... so they land on the same XCD (same L2).
__device__ __forceinline__ void xcd_split(int bid, int per, int& major, int& minor) {
    const int grp = bid / (8 * per), loc = bid % (8 * per);
    major = grp * 8 + loc % 8;
    minor = loc / 8;
}

}  // namespace

// ----------------------------------------------------------------------------------
// Row GEMM: Out[t, n0:n0+BN] = A[t, :] . B[:, n0:n0+BN] (+ bias) for the BM rows of one
// expert tile.  DX = false: B[k][n] = W[e][n][k] (forward).  DX = true: B[k][n] = W[e][k][n].
// ----------------------------------------------------------------------------------
template <int H, int BN, bool DX>
__global__ __launch_bounds__(kThreads) void k_rows_f32(const float* __restrict__ A,
                                                        const float* __restrict__ W,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ Out,
                                                        const int* __restrict__ offsets,
                                                        const int* __restrict__ perm, int NE,
                                                        int accumulate) {
    constexpr int BM = 128, KC = 32;
    constexpr int NT = H / BN;
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int SM = WTM / 32, SN = WTN / 32;
    constexpr int BS_ROWS = DX ? KC : BN;
    constexpr int BS_COLS = DX ? BN + kPad : KC + kPad;
    __shared__ float As[BM][KC + kPad];
    __shared__ float Bs[BS_ROWS][BS_COLS];
    __shared__ int tok[BM];

    int mt, nt;
    xcd_split(blockIdx.x, NT, mt, nt);
    int e, r0, r1;
    if (!find_tile(offsets, NE, mt, BM, e, r0, r1)) return;
    const int rows = r1 - r0;
    const int tid = threadIdx.x;
    if (tid < BM) tok[tid] = (tid < rows) ? perm[r0 + tid] : -1;
    __syncthreads();

    const int n0 = nt * BN;
    const float* __restrict__ We = W + (size_t)e * H * H;
    const int wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wm = wave / 2, wn = wave % 2;

    f32x16 acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = f32x16{};

    for (int k0 = 0; k0 < H; k0 += KC) {
        // A: BM rows x KC, 8 threads per row (128 B each).
#pragma unroll
        for (int i = 0; i < BM / 32; ++i) {
            const int r = tid / 8 + 32 * i, c = 4 * (tid % 8);
            const int t = tok[r];
            f32x4 v = f32x4{};
            if (t >= 0) v = ld4(A + (size_t)t * H + k0 + c);
            st4(&As[r][c], v);
        }
        if (!DX) {
#pragma unroll
            for (int i = 0; i < BN / 32; ++i) {
                const int r = tid / 8 + 32 * i, c = 4 * (tid % 8);
                st4(&Bs[r][c], ld4(We + (size_t)(n0 + r) * H + k0 + c));
            }
        } else {
            constexpr int Q = BN / 4;  // float4 per W row segment
#pragma unroll
            for (int i = 0; i < KC * Q / kThreads; ++i) {
                const int q = tid + kThreads * i;
                const int r = q / Q, c = 4 * (q % Q);
                st4(&Bs[r][c], ld4(We + (size_t)(k0 + r) * H + n0 + c));
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KC; kk += 8) {
            f32x4 a[SM], b[SN];
#pragma unroll
            for (int i = 0; i < SM; ++i) a[i] = ld4(&As[wm * WTM + i * 32 + l32][kk + 4 * h]);
#pragma unroll
            for (int j = 0; j < SN; ++j) {
                if (!DX) {
                    b[j] = ld4(&Bs[wn * WTN + j * 32 + l32][kk + 4 * h]);
                } else {
                    const int c = wn * WTN + j * 32 + l32;
                    b[j] = f32x4{Bs[kk + 4 * h + 0][c], Bs[kk + 4 * h + 1][c], Bs[kk + 4 * h + 2][c],
                                 Bs[kk + 4 * h + 3][c]};
                }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < SM; ++i)
#pragma unroll
                    for (int j = 0; j < SN; ++j) acc[i][j] = mfma32(a[i][s], b[j][s], acc[i][j]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < SN; ++j) {
        const int col = n0 + wn * WTN + j * 32 + l32;
        const float bv = DX ? 0.0f : bias[(size_t)e * H + col];
#pragma unroll
        for (int i = 0; i < SM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * WTM + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                const int t = tok[row];
                if (t >= 0) {
                    float* o = Out + (size_t)t * H + col;
                    float v = acc[i][j][r] + bv;
                    if (DX && accumulate) v = *o + v;
                    *o = v;
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------------
// dW / db partials.  Workgroup (chunk c, tile (ot, it)): the chunk's tokens of one expert,
// output block dW[o0:o0+BT, i0:i0+BT].  M = o, N = i, K = tokens.
//   part_dw[c][o][i] = sum_{t in chunk} dY[t][o] X[t][i]
//   part_db[c][o]    = sum_{t in chunk} dY[t][o]          (tiles with it == 0)
// Token order inside a chunk is fixed (perm order), as is the MFMA accumulation order.
// ----------------------------------------------------------------------------------
template <int H>
__global__ __launch_bounds__(kThreads) void k_dw_f32(const float* __restrict__ dY,
                                                      const float* __restrict__ X,
                                                      float* __restrict__ part_dw,
                                                      float* __restrict__ part_db,
                                                      const int* __restrict__ offsets,
                                                      const int* __restrict__ perm, int NE,
                                                      int chunk) {
    constexpr int BT = (H >= 128) ? 128 : 64;
    constexpr int NTI = H / BT, TPC = NTI * NTI;
    constexpr int KC = 32;
    constexpr int WT = BT / 2, SUB = WT / 32;
    __shared__ float As[KC][BT + kPad];  // dY rows, columns o0..o0+BT
    __shared__ float Bs[KC][BT + kPad];  // X rows, columns i0..i0+BT

    int c, tile;
    xcd_split(blockIdx.x, TPC, c, tile);
    // expert and token range of chunk c
    int e = -1, t0 = 0, t1 = 0;
    {
        int acc = 0;
        for (int i = 0; i < NE; ++i) {
            const int c0 = offsets[i], c1 = offsets[i + 1];
            const int n = (c1 - c0 + chunk - 1) / chunk;
            if (c < acc + n) {
                e = i;
                t0 = c0 + (c - acc) * chunk;
                t1 = min(c1, t0 + chunk);
                break;
            }
            acc += n;
        }
    }
    if (e < 0) return;
    const int o0 = (tile / NTI) * BT, i0 = (tile % NTI) * BT;
    const bool do_db = (tile % NTI) == 0;
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wm = wave / 2, wn = wave % 2;

    f32x16 acc[SUB][SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i)
#pragma unroll
        for (int j = 0; j < SUB; ++j) acc[i][j] = f32x16{};
    float dbacc = 0.0f;

    constexpr int Q = BT / 4;  // float4 per row segment
    for (int k0 = t0; k0 < t1; k0 += KC) {
#pragma unroll
        for (int i = 0; i < KC * Q / kThreads; ++i) {
            const int q = tid + kThreads * i;
            const int r = q / Q, cc = 4 * (q % Q);
            f32x4 va = f32x4{}, vb = f32x4{};
            if (k0 + r < t1) {
                const size_t t = (size_t)perm[k0 + r];
                va = ld4(dY + t * H + o0 + cc);
                vb = ld4(X + t * H + i0 + cc);
            }
            st4(&As[r][cc], va);
            st4(&Bs[r][cc], vb);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KC; kk += 8) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k = kk + 4 * h + s;
                float a[SUB], b[SUB];
#pragma unroll
                for (int i = 0; i < SUB; ++i) a[i] = As[k][wm * WT + i * 32 + l32];
#pragma unroll
                for (int j = 0; j < SUB; ++j) b[j] = Bs[k][wn * WT + j * 32 + l32];
#pragma unroll
                for (int i = 0; i < SUB; ++i)
#pragma unroll
                    for (int j = 0; j < SUB; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
            }
        }
        if (do_db && tid < BT) {
#pragma unroll 8
            for (int k = 0; k < KC; ++k) dbacc += As[k][tid];
        }
        __syncthreads();
    }

    float* __restrict__ P = part_dw + (size_t)c * H * H;
#pragma unroll
    for (int i = 0; i < SUB; ++i)
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
            const int col = i0 + wn * WT + j * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = o0 + wm * WT + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                P[(size_t)row * H + col] = acc[i][j][r];
            }
        }
    if (do_db && tid < BT) part_db[(size_t)c * H + o0 + tid] = dbacc;
}

// ----------------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------------
static inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

template <int H>
static hipError_t rows_f32(bool dx, const float* A, const float* W, const float* bias, float* Out,
                           int accumulate, const int32_t* offsets, const int32_t* perm, int64_t T,
                           int NE, hipStream_t s) {
    constexpr int BN = (H >= 128) ? 128 : H;
    constexpr int NT = H / BN;
    const int mtiles = (int)((T + 127) / 128) + NE;
    const int grid = round_up(mtiles, 8) * NT;
    if (dx)
        hipLaunchKernelGGL((k_rows_f32<H, BN, true>), dim3(grid), dim3(kThreads), 0, s, A, W, bias, Out,
                           offsets, perm, NE, accumulate);
    else
        hipLaunchKernelGGL((k_rows_f32<H, BN, false>), dim3(grid), dim3(kThreads), 0, s, A, W, bias, Out,
                           offsets, perm, NE, accumulate);
    return hipGetLastError();
}

static hipError_t rows_f32_dispatch(bool dx, const float* A, const float* W, const float* bias,
                                    float* Out, int accumulate, const int32_t* offsets,
                                    const int32_t* perm, int64_t T, int H, int NE, hipStream_t s) {
    switch (H) {
        case 64: return rows_f32<64>(dx, A, W, bias, Out, accumulate, offsets, perm, T, NE, s);
        case 128: return rows_f32<128>(dx, A, W, bias, Out, accumulate, offsets, perm, T, NE, s);
        case 256: return rows_f32<256>(dx, A, W, bias, Out, accumulate, offsets, perm, T, NE, s);
        case 512: return rows_f32<512>(dx, A, W, bias, Out, accumulate, offsets, perm, T, NE, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_gemm_f32(const float* X, const float* W, const float* bias, float* Y,
                               const int32_t* offsets, const int32_t* perm, int64_t T, int H, int NE,
                               hipStream_t s) {
    return rows_f32_dispatch(false, X, W, bias, Y, 0, offsets, perm, T, H, NE, s);
}

hipError_t launch_dx_gemm_f32(const float* dY, const float* W, float* dX, int accumulate,
                              const int32_t* offsets, const int32_t* perm, int64_t T, int H, int NE,
                              hipStream_t s) {
    return rows_f32_dispatch(true, dY, W, nullptr, dX, accumulate, offsets, perm, T, H, NE, s);
}

template <int H>
static hipError_t dw_f32(const float* dY, const float* X, float* pdw, float* pdb, const int32_t* offsets,
                         const int32_t* perm, int NE, int chunk, int n_chunk_max, hipStream_t s) {
    constexpr int BT = (H >= 128) ? 128 : 64;
    constexpr int TPC = (H / BT) * (H / BT);
    const int grid = round_up(n_chunk_max, 8) * TPC;
    hipLaunchKernelGGL((k_dw_f32<H>), dim3(grid), dim3(kThreads), 0, s, dY, X, pdw, pdb, offsets, perm, NE,
                       chunk);
    return hipGetLastError();
}

hipError_t launch_dw_gemm_f32(const float* dY, const float* X, float* pdw, float* pdb,
                              const int32_t* offsets, const int32_t* perm, int H, int NE, int chunk,
                              int n_chunk_max, hipStream_t s) {
    switch (H) {
        case 64: return dw_f32<64>(dY, X, pdw, pdb, offsets, perm, NE, chunk, n_chunk_max, s);
        case 128: return dw_f32<128>(dY, X, pdw, pdb, offsets, perm, NE, chunk, n_chunk_max, s);
        case 256: return dw_f32<256>(dY, X, pdw, pdb, offsets, perm, NE, chunk, n_chunk_max, s);
        case 512: return dw_f32<512>(dY, X, pdw, pdb, offsets, perm, NE, chunk, n_chunk_max, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
