// Grouped expert GEMMs with bf16 storage and fp32 accumulation (v_mfma_f32_32x32x16_bf16).
//
// Same operations as the fp32 kernels (MoE-gate commit page "11b96dac6a": the selected
// expert's [H, H] linear plus bias forward; gradients through that expert only), for
// activations and weights stored as bf16.  Accumulation is fp32; routed_ctx and
// d_fused_ctx are rounded to bf16 (nearest even) when stored; d_W / d_b partials stay fp32.
//
// v_mfma_f32_32x32x16_bf16: lane l (half h = l / 32) supplies 8 consecutive k of row
// m = l % 32 of A and of column n = l % 32 of B (k = 8h .. 8h+7); the fp32 result has the
// same lane layout as the fp32 32x32 instruction.  Operands come from LDS tiles:
//   forward  A = X rows, B = W[e] rows (W is [out][in]: K = in is contiguous): one 16-byte read
//   dX       A = dY rows, B = W[e] as stored, a [k = out][n = in] tile whose fragments come from
//            two transposing 8-byte reads (ds_read_b64_tr_b16, see tr_frag)
//   dW       A = dY^T, B = X^T: token rows are transposed in registers while staging
//            (4 tokens x 8 features per thread) so K = tokens is contiguous in LDS.
#include "moe_internal.hpp"

namespace moe {

namespace {

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

__device__ __forceinline__ f32x16 mfma_bf16(u16x8 a, u16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// two values at once with v_cvt_pk_bf16_f32 (nearest even, the same bits as f32_to_bf16 for
// every non-NaN input); lo goes to the lower half
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef int i32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

__device__ __forceinline__ u16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const u16x8*>(p); }
__device__ __forceinline__ void st8(uint16_t* p, u16x8 v) { *reinterpret_cast<u16x8*>(p) = v; }

__device__ __forceinline__ void xcd_split(int bid, int per, int& major, int& minor) {
    const int grp = bid / (8 * per), loc = bid % (8 * per);
    major = grp * 8 + loc % 8;
    minor = loc / 8;
}

}  // namespace

// MFMA B fragment (8 consecutive k of one column n per lane) from a row-major [k][n] bf16 LDS
// tile, through gfx950's transposing LDS read ds_read_b64_tr_b16.  Its lane layout, measured:
// within each group of 16 lanes, output lane i's element q is element (i & 3) of the 8 bytes
// that lane 4 q + (i >> 2) addressed -- so lane j of a group pointing at row j >> 2, columns
// 4 (j & 3) .. + 3 of a 4-row x 16-column block hands lane i the 4 rows of column i; two such
// reads give the 8 k of an operand.  blk: the fragment's first row (k) and column (n); RS: the
// tile's row stride in elements (BN + 32: 64 bytes of padding, where these reads measured
// conflict-free).
typedef short i16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4v* lds_i16x4_ptr;
template <int RS>
__device__ __forceinline__ u16x8 tr_frag(const uint16_t* blk, int lane) {
    const int h = lane / 32, grp = (lane % 32) / 16, j = lane % 16;
    const uint16_t* p = blk + (8 * h + (j >> 2)) * RS + 16 * grp + 4 * (j & 3);
    const i16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p));
    const i16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p + 4 * RS));
    u16x8 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[q] = (uint16_t)lo[q];
        v[4 + q] = (uint16_t)hi[q];
    }
    return v;
}

// Out[t, n0:n0+BN] = A[t, :] . Bw[e][n0:n0+BN, :]^T (+ bias[e] | + Out[t] when accumulating);
// for dX, A = dY and Out[t, n] = sum_k A[t, k] W[e][k, n] (W read as stored, see tr_frag).
#ifndef MOE_BF16_KC
#define MOE_BF16_KC 64  // K slice of the bf16 row GEMM (a multiple of 16)
#endif
#ifndef MOE_BF16_STAGED_STORES
#define MOE_BF16_STAGED_STORES 1  // output tiles go through LDS and out as whole 16-byte row segments
#endif
constexpr int kStPad = 8;  // fp32 staging rows: a stride of 8 (mod 64) floats keeps the two half-waves apart
template <int H, int BN>
struct RowsBf16Smem {
    static constexpr int BM = 128, KC = (MOE_BF16_KC < H) ? MOE_BF16_KC : H, KP = KC + 8;
    static constexpr int RSB = BN + 32;  // dX: row stride of the [k][n] W tile (64 bytes of padding)
    static constexpr size_t a = sizeof(uint16_t) * 2 * BM * KP, tok = 4 * BM;
    static constexpr size_t b = sizeof(uint16_t) * 2 * (BN * KP > KC * RSB ? BN * KP : KC * RSB);
    static constexpr size_t stage = MOE_BF16_STAGED_STORES ? sizeof(float) * BM * (BN + kStPad) : 0;
    static constexpr size_t tok_off = a + b > stage ? a + b : stage;
    static constexpr size_t bytes = tok_off + tok;
};

// K slices of both operands in flight per thread (a ring of registers), fed to two LDS
// buffers: with a 64-wide slice worth ~0.2 us of MFMAs per wave, one slice of prefetch left
// each tile waiting on one memory round trip per slice.
#ifndef MOE_BF16_RING_U8
#define MOE_BF16_RING_U8 16  // 16-byte registers per thread for the slice ring
#endif
template <int H, int BN, bool DX>
__device__ __forceinline__ void rows_bf16_body(char* smem, int bid, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ Bw,
                                               const float* __restrict__ bias,
                                               uint16_t* __restrict__ Out,
                                               const int* __restrict__ offsets,
                                               const int* __restrict__ perm, int NE, int accumulate) {
    constexpr int BM = 128, KC = RowsBf16Smem<H, BN>::KC, KP = KC + 8, NKC = H / KC;
    constexpr int NT = H / BN;
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int SM = WTM / 32, SN = WTN / 32;
    constexpr int TPR = KC / 8, RPP = kThreads / TPR;   // threads per 128-byte row slice, rows per pass
    constexpr int AL = BM / RPP, BL = BN / RPP;
    static_assert(H % KC == 0 && BM % RPP == 0 && BN % RPP == 0, "tile shape");
    constexpr int PF0 = MOE_BF16_RING_U8 / (AL + BL);
    constexpr int PF = PF0 < 1 ? 1 : (PF0 > NKC ? NKC : PF0);
    using SM_ = RowsBf16Smem<H, BN>;
    uint16_t(&As)[2][BM][KP] = *reinterpret_cast<uint16_t(*)[2][BM][KP]>(smem);
    uint16_t(&Bs)[2][BN][KP] = *reinterpret_cast<uint16_t(*)[2][BN][KP]>(smem + SM_::a);
    // dX reads W[e] as stored ([out][in]: K = out is the row index) into a [k][n] tile and takes
    // its fragments with the transposing LDS read
    constexpr int RSB = SM_::RSB, TPRB = BN / 8, RPPB = kThreads / TPRB;
    static_assert(!DX || (KC % RPPB == 0 && KC / RPPB == BL), "dX W tile shape");
    uint16_t(&Bt)[2][KC][RSB] = *reinterpret_cast<uint16_t(*)[2][KC][RSB]>(smem + SM_::a);
    int* tok = reinterpret_cast<int*>(smem + SM_::tok_off);

    int mt, nt;
    xcd_split(bid, NT, mt, nt);
    int e, r0, r1;
    if (!find_tile(offsets, NE, mt, BM, e, r0, r1)) return;
    const int rows = r1 - r0;
    const int tid = threadIdx.x;
    const int n0 = nt * BN;
    const uint16_t* __restrict__ Be = Bw + (size_t)e * H * H;
    const int wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wm = wave / 2, wn = wave % 2;

    // token ids: of this thread's A rows (registers) and of the tile's rows (LDS, epilogue)
    int ta[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int row = tid / TPR + RPP * i;
        ta[i] = (row < rows) ? perm[r0 + row] : -1;
    }
    const int tok_mine = (tid < BM && tid < rows) ? perm[r0 + tid] : -1;
    // the bias is loaded before the K loop: a load still pending in the epilogue's conditional
    // stores would be waited for in each of them, and that wait also waits for every store
    // issued before it
    float bv[SN];

    u16x8 ra[PF][AL], rb[PF][BL];
    auto load_b = [&](int c, int slot) {
#pragma unroll
        for (int i = 0; i < BL; ++i)
            rb[slot][i] = DX ? ld8(Be + (size_t)(c * KC + tid / TPRB + RPPB * i) * H + n0 + 8 * (tid % TPRB))
                             : ld8(Be + (size_t)(n0 + tid / TPR + RPP * i) * H + c * KC + 8 * (tid % TPR));
    };
    const uint16_t* a_src[AL];
    auto load_a = [&](int c, int slot) {
#pragma unroll
        for (int i = 0; i < AL; ++i) ra[slot][i] = ld8(a_src[i] + c * KC);
    };
    auto store_slice = [&](int slot, int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i) st8(&As[buf][tid / TPR + RPP * i][8 * (tid % TPR)], ra[slot][i]);
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            if constexpr (DX)
                st8(&Bt[buf][tid / TPRB + RPPB * i][8 * (tid % TPRB)], rb[slot][i]);
            else
                st8(&Bs[buf][tid / TPR + RPP * i][8 * (tid % TPR)], rb[slot][i]);
        }
    };

    // W does not depend on perm: its loads go out while the token ids are in flight (loads
    // return in issue order).  A padded row reads token 0's row: output rows are independent
    // and padded ones are never stored.  The fences keep loads from sinking to their uses.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < SN; ++j) bv[j] = DX ? 0.0f : bias[(size_t)e * H + n0 + wn * WTN + j * 32 + l32];
#pragma unroll
    for (int c = 0; c < PF; ++c) load_b(c, c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < AL; ++i) a_src[i] = A + (size_t)(ta[i] < 0 ? 0 : ta[i]) * H + 8 * (tid % TPR);
#pragma unroll
    for (int c = 0; c < PF; ++c) load_a(c, c);
    __builtin_amdgcn_sched_barrier(0);
    if (tid < BM) tok[tid] = tok_mine;  // read in the epilogue, after the barriers

    f32x16 acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = f32x16{};

    store_slice(0, 0);
    if (PF < NKC) {
        load_b(PF, 0);
        load_a(PF, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
        const int buf = c & 1;
        if (c + 1 < NKC) {
            store_slice((c + 1) % PF, (c + 1) & 1);
            if (c + 1 + PF < NKC) {
                load_b(c + 1 + PF, (c + 1) % PF);
                load_a(c + 1 + PF, (c + 1) % PF);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int kk = 0; kk < KC; kk += 16) {
            u16x8 a[SM], b[SN];
#pragma unroll
            for (int i = 0; i < SM; ++i) a[i] = ld8(&As[buf][wm * WTM + i * 32 + l32][kk + 8 * h]);
#pragma unroll
            for (int j = 0; j < SN; ++j)
                b[j] = DX ? tr_frag<RSB>(&Bt[buf][kk][wn * WTN + j * 32], lane)
                          : ld8(&Bs[buf][wn * WTN + j * 32 + l32][kk + 8 * h]);
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
        }
        if (c + 1 < NKC) __syncthreads();
    }

    if constexpr (MOE_BF16_STAGED_STORES) {
        // Epilogue through LDS: the fp32 tile (+ bias) is staged row-major over the K-slice
        // buffers, then each thread rounds 8 consecutive values to bf16 and writes them as one
        // 16-byte piece of an output row -- an eighth of the store instructions of writing each
        // lane's 2-byte values straight from the accumulators.  Same roundings as below.
        float(&St)[BM][BN + kStPad] = *reinterpret_cast<float(*)[BM][BN + kStPad]>(smem);
        const bool acc_dx = DX && accumulate;
        __syncthreads();  // every wavefront has read its last K slice
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    St[wm * WTM + i * 32 + 8 * (r / 4) + 4 * h + (r % 4)][wn * WTN + j * 32 + l32] =
                        acc_dx ? acc[i][j][r] : acc[i][j][r] + bv[j];
        __syncthreads();
        constexpr int CPR = BN / 8, RPS = kThreads / CPR, NP = BM / RPS;  // 8-wide pieces per row, rows per pass
        static_assert(kThreads % CPR == 0 && BM % RPS == 0, "staged epilogue shape");
        const int c8 = tid % CPR;
        int tk[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q) tk[q] = tok[q * RPS + tid / CPR];
        u16x8 old[NP];
        if (acc_dx) {  // every load out before the first (conditional) store; padded rows read row 0
#pragma unroll
            for (int q = 0; q < NP; ++q) old[q] = ld8(Out + (size_t)(tk[q] < 0 ? 0 : tk[q]) * H + n0 + 8 * c8);
        }
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const float* src = &St[q * RPS + tid / CPR][8 * c8];
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(src), v1 = *reinterpret_cast<const f32x4*>(src + 4);
            const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            u32x4v pk;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float a = acc_dx ? bf16_to_f32(old[q][2 * u]) + v[2 * u] : v[2 * u];
                const float b = acc_dx ? bf16_to_f32(old[q][2 * u + 1]) + v[2 * u + 1] : v[2 * u + 1];
                pk[u] = pack_bf16x2(a, b);
            }
            if (tk[q] >= 0) st8(Out + (size_t)tk[q] * H + n0 + 8 * c8, __builtin_bit_cast(u16x8, pk));
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < SN; ++j) {
        const int col = n0 + wn * WTN + j * 32 + l32;
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            const int* tr = &tok[wm * WTM + i * 32 + 4 * h];
            if (DX && accumulate) {
                // four rows' current values are loaded before their stores (a padded row reads
                // row 0 and drops it), so the block waits for memory four times, not sixteen
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int tk[4];
                    uint16_t old[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        tk[u] = tr[8 * q + u];
                        old[u] = Out[(size_t)(tk[u] < 0 ? 0 : tk[u]) * H + col];
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (tk[u] >= 0)
                            Out[(size_t)tk[u] * H + col] = f32_to_bf16(bf16_to_f32(old[u]) + acc[i][j][4 * q + u]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = tr[8 * (r / 4) + (r % 4)];
                    if (t >= 0) Out[(size_t)t * H + col] = f32_to_bf16(acc[i][j][r] + bv[j]);
                }
            }
        }
    }
}

// Forward with a column slice of W[e] resident in LDS (H = 256, 512).
//
// The tiled kernel above reads a 128 x 128 tile of each operand from L2 for every output tile:
// at T = 163,840, H = 512 that is 1.3 GB of L2 -> CU traffic for 168 MB of X.  Here a
// workgroup (one per CU, 4 wavefronts) keeps BN columns of W[e] in LDS (BN x H bf16 =
// 128 KB) and each wavefront streams groups of 32 of the expert's tokens through that slice,
// its X rows loaded straight into MFMA operand registers: no LDS traffic for X and no barrier
// between groups.  The NS = H / BN workgroups that cover one range of token groups run on the
// same XCD (blockIdx % 8), so X comes from HBM once and from L2 NS times.  At that shape the
// L2 -> CU requests halve and the forward goes from 134 to 128 us: the X loads, which one group
// of register ring does not cover, still hold it (with X rows served from L1 it takes 81 us).
//
// Operand layouts.  A dot product may take its k in any order if both operands take the same
// one: at k-step s = 4 q + i (i < 4) lane half h supplies the 8 k of 16-byte chunk
// c = 8 q + 4 h + i of its row, so over 4 consecutive k-steps a lane reads 64 contiguous bytes
// of its X row.  LDS row p = l32 + 32 j of the slice holds W[e] row n0 + NB l32 + j: lane l32
// of column block j then produces output feature n0 + NB l32 + j, so a lane's NB results for
// a token are adjacent features and leave as one 2 NB-byte store.  Chunk c of LDS row p sits at
// chunk c ^ (p & 15), so the 16 lanes that read together touch 16 different bank groups.
// Stores go through a buffer descriptor: padded rows of a ragged group get an offset past its
// end and the hardware drops them, so no store is conditional (needs T H 2 < 2^31 bytes).
template <int H>
struct WsBf16 {
    static constexpr int BN = (2 * H * H <= 131072) ? H : 131072 / (2 * H);  // columns per slice
    static constexpr int NB = BN / 32;                                       // 32-wide column blocks
    static constexpr int NS = H / BN;                                        // slices (workgroups per range)
    static constexpr int NSL = H / 128;                                      // 8-k-step slices of a group
};
#ifndef MOE_WS_SUB
#define MOE_WS_SUB 1            // 32-row MFMA blocks per wavefront group (2 spills registers)
#endif
#ifndef MOE_WS_WAVES
#define MOE_WS_WAVES 4          // wavefronts per workgroup, one per SIMD (8 spills registers)
#endif
constexpr int kWsWaves = MOE_WS_WAVES, kWsThreads = 64 * kWsWaves;
constexpr int kWsSub = MOE_WS_SUB;
constexpr int kWsGroup = 32 * kWsSub;  // tokens per wavefront group
#ifndef MOE_WS_BPF
#define MOE_WS_BPF 2            // k-steps of W fragments read ahead
#endif
constexpr int kWsWgs = 256;     // resident-slice grid: a multiple of 8 x NS
// 16-byte chunk of a row that lane half h supplies at k-step s (s < H / 16): a lane reads 64
// contiguous bytes of its row over 4 consecutive k-steps, so the 4 loads that touch one 128-byte
// line go out back to back (spreading each slice's 8 loads over 8 lines instead measured slower:
// forward 128 -> 141 us at T = 163,840, H = 512).
template <int H>
__device__ __forceinline__ constexpr int ws_chunk(int s, int h) {
    return 8 * (s / 4) + 4 * h + (s % 4);
}

// Lane e < N_E: expert e's first sorted position, count, and the exclusive / inclusive prefix
// of its 32-token groups.
struct WsGroups {
    int l0, c, excl, incl;
};
__device__ __forceinline__ WsGroups ws_groups(const int* __restrict__ offsets, int NE) {
    const int lane = __lane_id();
    WsGroups g{0, 0, 0, 0};
    if (lane < NE) {
        g.l0 = offsets[lane];
        g.c = offsets[lane + 1] - g.l0;
    }
    const int n = (g.c + kWsGroup - 1) / kWsGroup;
    g.incl = wave_inclusive_sum(n);
    g.excl = g.incl - n;
    return g;
}
// Token of row `row` of group g (g < 0: no group), -1 for padded rows.  Branch-free; the one
// perm load is unconditional (position 0 when there is no group: callers run only when T > 0).
__device__ __forceinline__ int ws_token(const WsGroups& gt, int NE, const int* __restrict__ perm, int g, int row) {
    const uint64_t hit = __ballot(__lane_id() < NE && g >= gt.excl && g < gt.incl);
    const int le = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
    const int j = g - __builtin_amdgcn_readlane(gt.excl, le);
    const int r0 = hit ? __builtin_amdgcn_readlane(gt.l0, le) + kWsGroup * j : 0;
    const int rows = hit ? min(kWsGroup, __builtin_amdgcn_readlane(gt.c, le) - kWsGroup * j) : 0;
    const int t = perm[r0 + min(row, max(rows - 1, 0))];
    return row < rows ? t : -1;
}

template <int H>
__global__ __launch_bounds__(kWsThreads, 1) void k_fwd_bf16_ws(const uint16_t* __restrict__ X,
                                                              const uint16_t* __restrict__ W,
                                                              const float* __restrict__ bias,
                                                              uint16_t* __restrict__ Y,
                                                              const int* __restrict__ offsets,
                                                              const int* __restrict__ perm, int NE, int T) {
    using C = WsBf16<H>;
    constexpr int BN = C::BN, NB = C::NB, NSL = C::NSL, CPR = H / 8;
    static_assert(NB == 4 || NB == 8, "a lane stores 8 or 16 bytes per row");
    static_assert((BN * CPR) % kWsThreads == 0 && (BN * CPR / kWsThreads) % 8 == 0, "slice load shape");
    __shared__ __attribute__((aligned(16))) uint16_t Ws[BN * H];
    __shared__ __attribute__((aligned(16))) int Tk[kWsWaves][kWsGroup];
    constexpr int SUB = kWsSub;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int xcd = blockIdx.x % 8, a = blockIdx.x / 8;
    const int ns = a % C::NS, NR = (int)gridDim.x / C::NS, rr = (a / C::NS) * 8 + xcd;
    const WsGroups gt = ws_groups(offsets, NE);
    const int Gt = __builtin_amdgcn_readlane(gt.incl, 63);
    const int g0 = (int)((int64_t)Gt * rr / NR), g1 = (int)((int64_t)Gt * (rr + 1) / NR);
    if (g0 >= g1) return;
    const int n0 = ns * BN;
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(Y, (short)0, (int)((int64_t)T * H * 2), 0x00020000);

    // one group of X rows ahead: slice k of the next group replaces slice k.  Row block u of a
    // group is rows 32 u + l32; tok[u] is this lane's token in block u.
    u16x8 ring[NSL][SUB][8];
    auto load_slice = [&](const int (&t)[SUB], int k) {
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
            const uint16_t* src = X + (size_t)(t[u] < 0 ? 0 : t[u]) * H + 8 * ws_chunk<H>(0, h);
#pragma unroll
            for (int s = 0; s < 8; ++s) ring[k][u][s] = ld8(src + 8 * ws_chunk<H>(8 * k + s, 0));
        }
    };
    auto tokens = [&](int gg, int (&t)[SUB]) {
#pragma unroll
        for (int u = 0; u < SUB; ++u) t[u] = ws_token(gt, NE, perm, gg < g1 ? gg : -1, 32 * u + l32);
    };
    // this wavefront's groups: g0 + wave, g0 + wave + kWsWaves, ...
    int g = g0 + wave;
    int tok[SUB], tokn[SUB];
    tokens(g, tok);
    tokens(g + kWsWaves, tokn);
#pragma unroll
    for (int k = 0; k < NSL; ++k) load_slice(tok, k);

    for (int e = 0; e < NE; ++e) {
        const int s0 = max(g0, __builtin_amdgcn_readlane(gt.excl, e));
        const int s1 = min(g1, __builtin_amdgcn_readlane(gt.incl, e));
        if (s0 >= s1) continue;
        __syncthreads();  // every wavefront is done with the previous slice
        const uint16_t* __restrict__ We = W + (size_t)e * H * H;
#pragma unroll
        for (int u0 = 0; u0 < BN * CPR / kWsThreads; u0 += 8) {
            u16x8 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int idx = tid + kWsThreads * (u0 + u), p = idx / CPR, c = idx % CPR;
                v[u] = ld8(We + (size_t)(n0 + NB * (p % 32) + p / 32) * H + 8 * c);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int idx = tid + kWsThreads * (u0 + u), p = idx / CPR, c = idx % CPR;
                st8(&Ws[p * H + 8 * (c ^ (p & 15))], v[u]);
            }
        }
        __syncthreads();
        float bv[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) bv[j] = bias[(size_t)e * H + n0 + NB * l32 + j];

        // groups of this wavefront in [s0, s1): g >= s0 holds because the segments before
        // this one took every earlier group
        for (; g < s1; g += kWsWaves) {
            int toknn[SUB];
            tokens(g + 2 * kWsWaves, toknn);
            // the tokens of the 16 rows per block whose results this lane holds (rows
            // 32 u + 8 v + 4 h + q), through the wavefront's slot in LDS (a wavefront's LDS
            // operations complete in order)
#pragma unroll
            for (int u = 0; u < SUB; ++u) Tk[wave][32 * u + l32] = tok[u];
            i32x4v trow[SUB][4];
#pragma unroll
            for (int u = 0; u < SUB; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    trow[u][v] = *reinterpret_cast<const i32x4v*>(&Tk[wave][32 * u + 8 * v + 4 * h]);
            f32x16 acc[SUB][NB];
#pragma unroll
            for (int u = 0; u < SUB; ++u)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[u][j] = f32x16{};
            // W fragments MOE_WS_BPF k-steps ahead of the MFMAs that use them; the fence keeps
            // the compiler from sinking the reads next to their uses
            constexpr int BPF = MOE_WS_BPF, NKS = 8 * NSL;
            u16x8 bq[BPF + 1][NB];
            auto load_b = [&](int ks) {
                const int c = ws_chunk<H>(ks, h);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    bq[ks % (BPF + 1)][j] = ld8(&Ws[(l32 + 32 * j) * H + 8 * (c ^ (l32 & 15))]);
            };
#pragma unroll
            for (int ks = 0; ks < BPF; ++ks) load_b(ks);
#pragma unroll
            for (int k = 0; k < NSL; ++k) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int ks = 8 * k + s;
                    if (ks + BPF < NKS) load_b(ks + BPF);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < NB; ++j)
#pragma unroll
                        for (int u = 0; u < SUB; ++u)
                            acc[u][j] = mfma_bf16(ring[k][u][s], bq[ks % (BPF + 1)][j], acc[u][j]);
                }
                // slice k of the next group goes out once slice k of this one is consumed
                __builtin_amdgcn_sched_barrier(0x010E);
                load_slice(tokn, k);
                __builtin_amdgcn_sched_barrier(0x010E);
            }
#pragma unroll
            for (int u = 0; u < SUB; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = trow[u][r / 4][r % 4];
                    const int off = t >= 0 ? (t * H + n0 + NB * l32) * 2 : (int)0x80000000;
                    if constexpr (NB == 4) {
                        i32x2v pk;
                        pk[0] = (int)pack_bf16x2(acc[u][0][r] + bv[0], acc[u][1][r] + bv[1]);
                        pk[1] = (int)pack_bf16x2(acc[u][2][r] + bv[2], acc[u][3][r] + bv[3]);
                        __builtin_amdgcn_raw_buffer_store_b64(pk, yr, off, 0, 0);
                    } else {
                        i32x4v pk;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            pk[q] = (int)pack_bf16x2(acc[u][2 * q][r] + bv[2 * q], acc[u][2 * q + 1][r] + bv[2 * q + 1]);
                        __builtin_amdgcn_raw_buffer_store_b128(pk, yr, off, 0, 0);
                    }
                }
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                tok[u] = tokn[u];
                tokn[u] = toknn[u];
            }
        }
    }
}

// d_W / d_b partials for one chunk of one expert's tokens, output tile [o0:o0+BT, i0:i0+BT].
//
// The LDS tiles are [feature][token]; a thread's register transpose writes 4 tokens of 8
// features (rows 8 apart), which with a plain layout puts a wave's 8-byte stores on a few
// banks.  The 16-byte token chunks of row r are therefore XOR-swizzled by (r >> 4) & 7: the
// stores of a wave then cover all 64 banks, and the MFMA fragment reads (16 consecutive rows
// with one swizzle) stay conflict-free.
__device__ __forceinline__ int swz(int row, int k) { return (((k >> 3) ^ ((row >> 4) & 7)) << 3) | (k & 7); }
template <int H>
struct DwBf16Smem {
    static constexpr int BT = (H >= 128) ? 128 : 64, KC = 64, KP = KC + 8;
    static constexpr size_t a = sizeof(uint16_t) * 2 * BT * KP;
    static constexpr size_t bytes = 2 * a;
};

template <int H>
__device__ __forceinline__ void dw_bf16_body(char* smem, int bid, const uint16_t* __restrict__ dY,
                                                       const uint16_t* __restrict__ X,
                                                       float* __restrict__ part_dw, float* __restrict__ part_db,
                                                       const int* __restrict__ offsets,
                                                       const int* __restrict__ perm, int NE, int P, int T) {
    constexpr int BT = (H >= 128) ? 128 : 64;
    constexpr int NTI = H / BT, TPC = NTI * NTI;
    constexpr int KC = 64, KP = KC + 8;
    constexpr int WT = BT / 2, SUB = WT / 32;
    constexpr int ITEMS = (KC / 4) * (BT / 8);  // (4 tokens x 8 features) blocks per stage
    uint16_t(&As)[2][BT][KP] = *reinterpret_cast<uint16_t(*)[2][BT][KP]>(smem);                     // dY^T [o][t]
    uint16_t(&Bs)[2][BT][KP] = *reinterpret_cast<uint16_t(*)[2][BT][KP]>(smem + DwBf16Smem<H>::a);  // X^T  [i][t]

    int c, tile;
    xcd_split(bid, TPC, c, tile);
    int e = -1, t0 = 0, t1 = 0;
    if (!find_chunk(offsets, NE, P, T, c, e, t0, t1)) return;
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

    // Two LDS buffers; per thread IPT items of (4 tokens x 8 features) per tensor, loaded one
    // slice ahead of the MFMAs, transposed in registers when stored.  Token ids are fetched
    // one slice further ahead.
    constexpr int IPT = (ITEMS + kThreads - 1) / kThreads;
    const int nslices = (t1 - t0 + KC - 1) / KC;
    int tk[IPT][4];
    u16x8 va[IPT][4], vb[IPT][4];
    auto load_ids = [&](int sl) {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int q = tid + kThreads * it;
            const int tq = q / (BT / 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = t0 + sl * KC + 4 * tq + j;
                tk[it][j] = (q < ITEMS && sl < nslices && k < t1) ? perm[k] : -1;
            }
        }
    };
    auto load_rows = [&]() {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int fq = (tid + kThreads * it) % (BT / 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                va[it][j] = u16x8{};
                vb[it][j] = u16x8{};
                if (tk[it][j] >= 0) {
                    const size_t t = (size_t)tk[it][j];
                    va[it][j] = ld8(dY + t * H + o0 + 8 * fq);
                    vb[it][j] = ld8(X + t * H + i0 + 8 * fq);
                }
            }
        }
    };
    auto store_rows = [&](int buf) {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int q = tid + kThreads * it;
            if (q < ITEMS) {
                const int tq = q / (BT / 8), fq = q % (BT / 8);
#pragma unroll
                for (int f = 0; f < 8; ++f) {
                    uint2 wa, wb;
                    wa.x = (uint32_t)va[it][0][f] | ((uint32_t)va[it][1][f] << 16);
                    wa.y = (uint32_t)va[it][2][f] | ((uint32_t)va[it][3][f] << 16);
                    wb.x = (uint32_t)vb[it][0][f] | ((uint32_t)vb[it][1][f] << 16);
                    wb.y = (uint32_t)vb[it][2][f] | ((uint32_t)vb[it][3][f] << 16);
                    const int row = 8 * fq + f, k = swz(row, 4 * tq);
                    *reinterpret_cast<uint2*>(&As[buf][row][k]) = wa;
                    *reinterpret_cast<uint2*>(&Bs[buf][row][k]) = wb;
                }
            }
        }
    };

    load_ids(0);
    load_rows();
    load_ids(1);
    store_rows(0);
    __syncthreads();
#pragma unroll 1
    for (int sl = 0; sl < nslices; ++sl) {
        const int buf = sl & 1;
        if (sl + 1 < nslices) {
            load_rows();
            load_ids(sl + 2);
        }
#pragma unroll
        for (int kk = 0; kk < KC; kk += 16) {
            u16x8 a[SUB], b[SUB];
#pragma unroll
            for (int i = 0; i < SUB; ++i) {
                const int row = wm * WT + i * 32 + l32;
                a[i] = ld8(&As[buf][row][swz(row, kk + 8 * h)]);
            }
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
                const int row = wn * WT + j * 32 + l32;
                b[j] = ld8(&Bs[buf][row][swz(row, kk + 8 * h)]);
            }
#pragma unroll
            for (int i = 0; i < SUB; ++i)
#pragma unroll
                for (int j = 0; j < SUB; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
        }
        if (do_db && tid < BT) {
#pragma unroll
            for (int q = 0; q < KC / 8; ++q) {
                const u16x8 v = ld8(&As[buf][tid][swz(tid, 8 * q)]);
#pragma unroll
                for (int j = 0; j < 8; ++j) dbacc += bf16_to_f32(v[j]);
            }
        }
        if (sl + 1 < nslices) store_rows(buf ^ 1);
        __syncthreads();
    }

    float* __restrict__ Pd = part_dw + (size_t)c * H * H;
    if constexpr (MOE_BF16_STAGED_STORES) {
        // the partial tile through LDS (the loop's last barrier freed the buffers), then whole
        // 16-byte row pieces
        static_assert(DwBf16Smem<H>::bytes >= sizeof(float) * BT * (BT + kStPad), "LDS for the staged tile");
        float(&St)[BT][BT + kStPad] = *reinterpret_cast<float(*)[BT][BT + kStPad]>(smem);
#pragma unroll
        for (int i = 0; i < SUB; ++i)
#pragma unroll
            for (int j = 0; j < SUB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    St[wm * WT + i * 32 + 8 * (r / 4) + 4 * h + (r % 4)][wn * WT + j * 32 + l32] = acc[i][j][r];
        __syncthreads();
        constexpr int CPR = BT / 4, RPS = kThreads / CPR;
#pragma unroll
        for (int q = 0; q < BT / RPS; ++q) {
            const int row = q * RPS + tid / CPR, c4 = tid % CPR;
            *reinterpret_cast<f32x4*>(Pd + (size_t)(o0 + row) * H + i0 + 4 * c4) =
                *reinterpret_cast<const f32x4*>(&St[row][4 * c4]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < SUB; ++i)
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
                const int col = i0 + wn * WT + j * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = o0 + wm * WT + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    Pd[(size_t)row * H + col] = acc[i][j][r];
                }
            }
    }
    if (do_db && tid < BT) part_db[(size_t)c * H + o0 + tid] = dbacc;
}

// Kernels.  The backward is one launch: dW / db chunk tiles first, then dX tiles.
template <int H, int BN>
__global__ __launch_bounds__(kThreads) void k_fwd_bf16(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                        const float* __restrict__ bias, uint16_t* __restrict__ Y,
                                                        const int* __restrict__ offsets,
                                                        const int* __restrict__ perm, int NE) {
    __shared__ __attribute__((aligned(16))) char smem[RowsBf16Smem<H, BN>::bytes];
    rows_bf16_body<H, BN, false>(smem, blockIdx.x, X, W, bias, Y, offsets, perm, NE, 0);
}

template <int H, int BN>
__global__ __launch_bounds__(kThreads) void k_bwd_bf16(const uint16_t* __restrict__ dY,
                                                        const uint16_t* __restrict__ X,
                                                        const uint16_t* __restrict__ W, uint16_t* __restrict__ dX,
                                                        int accumulate, float* __restrict__ part_dw,
                                                        float* __restrict__ part_db,
                                                        const int* __restrict__ offsets,
                                                        const int* __restrict__ perm, int NE, int P, int T, int n_dx) {
    constexpr size_t r = RowsBf16Smem<H, BN>::bytes, d = DwBf16Smem<H>::bytes;
    __shared__ __attribute__((aligned(16))) char smem[r > d ? r : d];  // one LDS region, either role
    // longest first: the dW workgroups (a whole chunk each) lead the grid, the dX tiles follow,
    // so the dispatcher evens out the end of the launch
    const int n_dw = (int)gridDim.x - n_dx;
    if ((int)blockIdx.x < n_dw)
        dw_bf16_body<H>(smem, blockIdx.x, dY, X, part_dw, part_db, offsets, perm, NE, P, T);
    else
        rows_bf16_body<H, BN, true>(smem, blockIdx.x - n_dw, dY, W, nullptr, dX, offsets, perm, NE, accumulate);
}

// ---------------------------------------------------------------- launchers
static inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

#ifndef MOE_BF16_WS_FWD
#define MOE_BF16_WS_FWD 1  // H = 256 / 512 forward with the W slice resident in LDS
#endif
template <int H>
static hipError_t fwd_bf16(const uint16_t* X, const uint16_t* W, const float* bias, uint16_t* Y,
                           const int32_t* offsets, const int32_t* perm, int64_t T, int NE, hipStream_t s) {
    if constexpr (H >= 256) {
        if (MOE_BF16_WS_FWD && T * H * 2 < ((int64_t)1 << 31)) {
            launch_kernel((k_fwd_bf16_ws<H>), dim3(kWsWgs), dim3(kWsThreads), 0, s, X, W, bias, Y, offsets, perm, NE,
                          (int)T);
            return hipGetLastError();
        }
    }
    constexpr int BN = (H >= 128) ? 128 : H;
    constexpr int NT = H / BN;
    const int grid = round_up((int)((T + 127) / 128) + NE, 8) * NT;
    launch_kernel((k_fwd_bf16<H, BN>), dim3(grid), dim3(kThreads), 0, s, X, W, bias, Y, offsets, perm, NE);
    return hipGetLastError();
}

template <int H>
static hipError_t bwd_bf16(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX, int accumulate,
                           float* pdw, float* pdb, const int32_t* offsets, const int32_t* perm, int64_t T, int NE,
                           int P, int n_chunk_max, hipStream_t s) {
    constexpr int BN = (H >= 128) ? 128 : H;
    constexpr int NT = H / BN;
    constexpr int BT = (H >= 128) ? 128 : 64;
    constexpr int TPC = (H / BT) * (H / BT);
    const int n_dx = round_up((int)((T + 127) / 128) + NE, 8) * NT;
    const int grid = n_dx + round_up(n_chunk_max, 8) * TPC;
    launch_kernel((k_bwd_bf16<H, BN>), dim3(grid), dim3(kThreads), 0, s, dY, X, W, dX, accumulate, pdw, pdb,
                       offsets, perm, NE, P, (int)T, n_dx);
    return hipGetLastError();
}

hipError_t launch_fwd_gemm_bf16(const uint16_t* X, const uint16_t* W, const float* bias, uint16_t* Y,
                                const int32_t* offsets, const int32_t* perm, int64_t T, int H, int NE,
                                hipStream_t s) {
    switch (H) {
        case 64: return fwd_bf16<64>(X, W, bias, Y, offsets, perm, T, NE, s);
        case 128: return fwd_bf16<128>(X, W, bias, Y, offsets, perm, T, NE, s);
        case 256: return fwd_bf16<256>(X, W, bias, Y, offsets, perm, T, NE, s);
        case 512: return fwd_bf16<512>(X, W, bias, Y, offsets, perm, T, NE, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_gemm_bf16(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX,
                                int accumulate, float* pdw, float* pdb, const int32_t* offsets, const int32_t* perm,
                                int64_t T, int H, int NE, int P, int n_chunk_max, hipStream_t s) {
    switch (H) {
        case 64: return bwd_bf16<64>(dY, X, W, dX, accumulate, pdw, pdb, offsets, perm, T, NE, P, n_chunk_max, s);
        case 128: return bwd_bf16<128>(dY, X, W, dX, accumulate, pdw, pdb, offsets, perm, T, NE, P, n_chunk_max, s);
        case 256: return bwd_bf16<256>(dY, X, W, dX, accumulate, pdw, pdb, offsets, perm, T, NE, P, n_chunk_max, s);
        case 512: return bwd_bf16<512>(dY, X, W, dX, accumulate, pdw, pdb, offsets, perm, T, NE, P, n_chunk_max, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
