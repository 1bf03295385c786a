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
// Eight bf16 values times an fp32 factor, rounded back to bf16 (nearest even): a row of d_routed_ctx
// formed from the horizon mean's gradient, d_mean[b] * (1/N_H), exactly as the collapse backward
// stores it.
__device__ __forceinline__ u16x8 scale8(u16x8 v, float f) {
    u16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32_to_bf16(bf16_to_f32(v[j]) * f);
    return o;
}
__device__ __forceinline__ void st8(uint16_t* p, u16x8 v) { *reinterpret_cast<u16x8*>(p) = v; }
// Non-temporal store, for the GEMM outputs, which no workgroup of the same launch reads back
// (wider-bf16 step 373.5 -> 364 us against plain stores).
__device__ __forceinline__ void st8_nt(uint16_t* p, u16x8 v) { __builtin_nontemporal_store(v, reinterpret_cast<u16x8*>(p)); }

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
template <int H, int BN, bool DX, bool MEAN = false>
__device__ __forceinline__ void rows_bf16_body(char* smem, int bid, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ Bw,
                                               const float* __restrict__ bias,
                                               uint16_t* __restrict__ Out,
                                               const int* __restrict__ offsets,
                                               const int* __restrict__ perm, int NE, int T, int accumulate,
                                               int nh = 1, float inv_nh = 1.0f) {
    // MEAN (dX only): row t of A is bf16(A[t / nh] * inv_nh)
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
    if (!find_tile(offsets, NE, T, mt, BM, e, r0, r1)) return;
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
        ta[i] = (row < rows) ? load_token(perm, r0 + row, T) : -1;
    }
    const int tok_mine = (tid < BM && tid < rows) ? load_token(perm, r0 + tid, T) : -1;
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
        for (int i = 0; i < AL; ++i)
            st8(&As[buf][tid / TPR + RPP * i][8 * (tid % TPR)], MEAN ? scale8(ra[slot][i], inv_nh) : ra[slot][i]);
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
    for (int i = 0; i < AL; ++i) {
        const int t = ta[i] < 0 ? 0 : ta[i];
        a_src[i] = A + (size_t)(MEAN ? t / nh : t) * H + 8 * (tid % TPR);
    }
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
            if (tk[q] >= 0) st8_nt(Out + (size_t)tk[q] * H + n0 + 8 * c8, __builtin_bit_cast(u16x8, pk));
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
__device__ __forceinline__ WsGroups ws_groups(const int* __restrict__ offsets, int NE, int T) {
    WsGroups g{0, 0, 0, 0};
    expert_range(offsets, NE, T, g.l0, g.c);
    const int n = (g.c + kWsGroup - 1) / kWsGroup;
    g.incl = wave_inclusive_sum(n);
    g.excl = g.incl - n;
    return g;
}
// Token of row `row` of group g (g < 0: no group), -1 for padded rows.  Branch-free; the one
// perm load is unconditional (position 0 when there is no group: callers run only when T > 0).
__device__ __forceinline__ int ws_token(const WsGroups& gt, int NE, int T, const int* __restrict__ perm, int g,
                                        int row) {
    const uint64_t hit = __ballot(__lane_id() < NE && g >= gt.excl && g < gt.incl);
    const int le = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
    const int j = g - __builtin_amdgcn_readlane(gt.excl, le);
    const int r0 = hit ? __builtin_amdgcn_readlane(gt.l0, le) + kWsGroup * j : 0;
    const int rows = hit ? min(kWsGroup, __builtin_amdgcn_readlane(gt.c, le) - kWsGroup * j) : 0;
    const int t = load_token(perm, r0 + min(row, max(rows - 1, 0)), T);
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
    const WsGroups gt = ws_groups(offsets, NE, T);
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
        for (int u = 0; u < SUB; ++u) t[u] = ws_token(gt, NE, T, perm, gg < g1 ? gg : -1, 32 * u + l32);
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
//
// BT = 128: four wavefronts of 64 x 64 (this body shares a launch with the dX tiles).
// BT = 256 (H = 256, 512): four wavefronts of 128 x 128 (16 accumulator blocks each, one
// workgroup per compute unit, a launch of its own).  A 128 x 128 tile per chunk re-reads the
// chunk's dY and X columns once per partner tile (four at H = 512) and needs twice the L2 -> CU
// bytes per MFMA; the 256 x 256 tile halves both and halves the LDS fragment reads per MFMA.
__device__ __forceinline__ int swz(int row, int k) { return (((k >> 3) ^ ((row >> 4) & 7)) << 3) | (k & 7); }
template <int BT>
struct DwBf16Smem {
    static constexpr int KC = 64, KP = KC + 8;
    static constexpr size_t a = sizeof(uint16_t) * 2 * BT * KP;
    static constexpr size_t bytes = 2 * a;
};

// PFR: slices of rows in flight (1: one slice ahead, loaded while the current one computes).
// NTH: threads per workgroup (256: wavefronts 2 x 2 over the tile; 512: 2 x 4).
template <int H, int BT, bool MEAN = false, int PFR = 1, int NTH = kThreads>
__device__ __forceinline__ void dw_bf16_body(char* smem, int bid, const uint16_t* __restrict__ dY,
                                             const uint16_t* __restrict__ X, float* __restrict__ part_dw,
                                             float* __restrict__ part_db, const int* __restrict__ offsets,
                                             const int* __restrict__ perm, int NE, int P, int T, int nh = 1,
                                             float inv_nh = 1.0f) {
    // MEAN: row t of dY is bf16(dY[t / nh] * inv_nh)
    constexpr int NTI = H / BT, TPC = NTI * NTI;
    constexpr int KC = DwBf16Smem<BT>::KC, KP = DwBf16Smem<BT>::KP;
    constexpr int WN_W = NTH / 128;                      // wavefronts along the tile's columns
    constexpr int WTM = BT / 2, WTN = BT / WN_W, SUBM = WTM / 32, SUBN = WTN / 32;
    constexpr int ITEMS = (KC / 4) * (BT / 8);  // (4 tokens x 8 features) blocks per stage
    uint16_t(&As)[2][BT][KP] = *reinterpret_cast<uint16_t(*)[2][BT][KP]>(smem);                        // dY^T [o][t]
    uint16_t(&Bs)[2][BT][KP] = *reinterpret_cast<uint16_t(*)[2][BT][KP]>(smem + DwBf16Smem<BT>::a);  // X^T  [i][t]

    int c, tile;
    xcd_split(bid, TPC, c, tile);
    int e = -1, t0 = 0, t1 = 0;
    if (!find_chunk(offsets, NE, P, T, c, e, t0, t1)) return;
    const int o0 = (tile / NTI) * BT, i0 = (tile % NTI) * BT;
    const bool do_db = (tile % NTI) == 0;
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wm = wave / WN_W, wn = wave % WN_W;

    f32x16 acc[SUBM][SUBN];
#pragma unroll
    for (int i = 0; i < SUBM; ++i)
#pragma unroll
        for (int j = 0; j < SUBN; ++j) acc[i][j] = f32x16{};
    float dbacc = 0.0f;

    // Two LDS buffers; per thread IPT items of (4 tokens x 8 features) per tensor, loaded one
    // slice ahead of the MFMAs, transposed in registers when stored.  Token ids are fetched
    // one slice further ahead.
    constexpr int IPT = (ITEMS + NTH - 1) / NTH;
    const int nslices = (t1 - t0 + KC - 1) / KC;
    int tk[IPT][4];
    u16x8 va[IPT][4], vb[IPT][4];
    auto load_ids = [&](int sl) {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int q = tid + NTH * it;
            const int tq = q / (BT / 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = t0 + sl * KC + 4 * tq + j;
                tk[it][j] = (q < ITEMS && sl < nslices && k < t1) ? load_token(perm, k, T) : -1;
            }
        }
    };
    auto load_rows = [&]() {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int fq = (tid + NTH * it) % (BT / 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                va[it][j] = u16x8{};
                vb[it][j] = u16x8{};
                if (tk[it][j] >= 0) {
                    const size_t t = (size_t)tk[it][j];
                    va[it][j] = ld8(dY + (MEAN ? t / nh : t) * H + o0 + 8 * fq);
                    vb[it][j] = ld8(X + t * H + i0 + 8 * fq);
                }
            }
        }
    };
    auto store_rows = [&](int buf) {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int q = tid + NTH * it;
            if (q < ITEMS) {
                const int tq = q / (BT / 8), fq = q % (BT / 8);
                if (MEAN) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) va[it][j] = scale8(va[it][j], inv_nh);
                }
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

    auto compute = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < KC; kk += 16) {
            u16x8 a[SUBM], b[SUBN];
#pragma unroll
            for (int i = 0; i < SUBM; ++i) {
                const int row = wm * WTM + i * 32 + l32;
                a[i] = ld8(&As[buf][row][swz(row, kk + 8 * h)]);
            }
#pragma unroll
            for (int j = 0; j < SUBN; ++j) {
                const int row = wn * WTN + j * 32 + l32;
                b[j] = ld8(&Bs[buf][row][swz(row, kk + 8 * h)]);
            }
#pragma unroll
            for (int i = 0; i < SUBM; ++i)
#pragma unroll
                for (int j = 0; j < SUBN; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
        }
        if (do_db && tid < BT) {
#pragma unroll
            for (int q = 0; q < KC / 8; ++q) {
                const u16x8 v = ld8(&As[buf][tid][swz(tid, 8 * q)]);
#pragma unroll
                for (int j = 0; j < 8; ++j) dbacc += bf16_to_f32(v[j]);
            }
        }
    };

    if constexpr (PFR == 1) {
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
            compute(buf);
            if (sl + 1 < nslices) store_rows(buf ^ 1);
            __syncthreads();
        }
    } else {
        // A ring of PFR slices in registers (one wavefront per SIMD leaves the registers for it):
        // the rows of slices s+1 .. s+PFR and the token ids of the PFR slices after those are in
        // flight while slice s computes.  Loads past the chunk's end read its last token and are
        // zeroed when stored, so no load sits under a branch.
        static_assert(PFR % 2 == 0, "the LDS buffer of slice s0 + u is u % 2");
        int tkr[PFR][IPT][4];
        u16x8 var[PFR][IPT][4], vbr[PFR][IPT][4];
        auto kpos = [&](int sl, int it, int j) { return t0 + sl * KC + 4 * ((tid + NTH * it) / (BT / 8)) + j; };
        auto rids = [&](int sl, int slot) {
#pragma unroll
            for (int it = 0; it < IPT; ++it)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = kpos(sl, it, j);
                    tkr[slot][it][j] = load_token(perm, k < t1 ? k : t1 - 1, T);
                }
        };
        auto rrows = [&](int slot) {
#pragma unroll
            for (int it = 0; it < IPT; ++it) {
                const int fq = (tid + NTH * it) % (BT / 8);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const size_t t = (size_t)tkr[slot][it][j];
                    var[slot][it][j] = ld8(dY + (MEAN ? t / nh : t) * H + o0 + 8 * fq);
                    vbr[slot][it][j] = ld8(X + t * H + i0 + 8 * fq);
                }
            }
        };
        auto rstore = [&](int sl, int slot, int buf) {
#pragma unroll
            for (int it = 0; it < IPT; ++it) {
                const int q = tid + NTH * it;
                if (q < ITEMS) {
                    const int tq = q / (BT / 8), fq = q % (BT / 8);
                    u16x8 wa4[4], wb4[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool v = kpos(sl, it, j) < t1;
                        wa4[j] = v ? (MEAN ? scale8(var[slot][it][j], inv_nh) : var[slot][it][j]) : u16x8{};
                        wb4[j] = v ? vbr[slot][it][j] : u16x8{};
                    }
#pragma unroll
                    for (int f = 0; f < 8; ++f) {
                        uint2 wa, wb;
                        wa.x = (uint32_t)wa4[0][f] | ((uint32_t)wa4[1][f] << 16);
                        wa.y = (uint32_t)wa4[2][f] | ((uint32_t)wa4[3][f] << 16);
                        wb.x = (uint32_t)wb4[0][f] | ((uint32_t)wb4[1][f] << 16);
                        wb.y = (uint32_t)wb4[2][f] | ((uint32_t)wb4[3][f] << 16);
                        const int row = 8 * fq + f, k = swz(row, 4 * tq);
                        *reinterpret_cast<uint2*>(&As[buf][row][k]) = wa;
                        *reinterpret_cast<uint2*>(&Bs[buf][row][k]) = wb;
                    }
                }
            }
        };
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < PFR; ++k) rids(k, k);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < PFR; ++k) rrows(k);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < PFR; ++k) rids(PFR + k, k);
        __builtin_amdgcn_sched_barrier(0);
        rstore(0, 0, 0);
        rrows(0);
        rids(2 * PFR, 0);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
#pragma unroll 1
        for (int s0 = 0; s0 < nslices; s0 += PFR) {
#pragma unroll
            for (int u = 0; u < PFR; ++u) {
                const int sl = s0 + u;
                if (sl >= nslices) break;
                rstore(sl + 1, (u + 1) % PFR, (u + 1) & 1);
                rrows((u + 1) % PFR);
                rids(sl + 1 + 2 * PFR, (u + 1) % PFR);
                __builtin_amdgcn_sched_barrier(0);
                compute(u & 1);
                __syncthreads();
            }
        }
    }

    float* __restrict__ Pd = part_dw + (size_t)c * H * H;
    if constexpr (MOE_BF16_STAGED_STORES) {
        // The partial tile through LDS (the loop's last barrier freed the buffers), then whole
        // 16-byte row pieces; a 256 x 256 tile goes in two halves of 128 rows (the wavefronts
        // with wm = 0, then those with wm = 1).
        constexpr int HR = (DwBf16Smem<BT>::bytes >= sizeof(float) * BT * (BT + kStPad)) ? BT : BT / 2;
        static_assert(DwBf16Smem<BT>::bytes >= sizeof(float) * HR * (BT + kStPad), "LDS for the staged tile");
        float(&St)[HR][BT + kStPad] = *reinterpret_cast<float(*)[HR][BT + kStPad]>(smem);
        constexpr int CPR = BT / 4, RPS = NTH / CPR;
#pragma unroll
        for (int half = 0; half < BT / HR; ++half) {
            if (half > 0) __syncthreads();  // the previous half has been read
            if (HR == BT || wm == half) {
#pragma unroll
                for (int i = 0; i < SUBM; ++i)
#pragma unroll
                    for (int j = 0; j < SUBN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            St[(HR == BT ? wm * WTM : 0) + i * 32 + 8 * (r / 4) + 4 * h + (r % 4)]
                              [wn * WTN + j * 32 + l32] = acc[i][j][r];
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < HR / RPS; ++q) {
                const int row = q * RPS + tid / CPR, c4 = tid % CPR;
                *reinterpret_cast<f32x4*>(Pd + (size_t)(o0 + half * HR + row) * H + i0 + 4 * c4) =
                    *reinterpret_cast<const f32x4*>(&St[row][4 * c4]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < SUBM; ++i)
#pragma unroll
            for (int j = 0; j < SUBN; ++j) {
                const int col = i0 + wn * WTN + j * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = o0 + wm * WTM + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    Pd[(size_t)row * H + col] = acc[i][j][r];
                }
            }
    }
    if (do_db && tid < BT) part_db[(size_t)c * H + o0 + tid] = dbacc;
}

// d_W / d_b partials with 256 x 256 output tiles (H = 256, 512), staged token-major.
//
// The chunk's rows go to LDS as loaded (16-byte stores, no register transpose): tile [t][f],
// 64 tokens x 256 features of dY (o0 ..) and of X (i0 ..), rows of 512 bytes.  The MFMA
// fragments want 8 consecutive tokens of one feature per lane, which gfx950's transposing LDS
// read ds_read_b64_tr_b16 gives (see tr_frag).  The 16-byte chunk c of row t sits at chunk
// c ^ 4 (t & 3): a wavefront's stores (two whole rows) stay conflict-free, and the 8 rows x 64
// bytes of one transposing read spread over all 64 banks twice -- the minimum.
// Eight wavefronts, 2 (o) x 4 (i), each 128 x 64 of the tile (8 accumulator blocks); d_b comes
// from the dY fragments of the wavefronts with wn = 0 (each lane sums its 8 tokens, the two lane
// halves are added at the end).
constexpr int kDwtThreads = 512;
#ifndef MOE_BF16_DWT_RING
#define MOE_BF16_DWT_RING 1  // slices of rows in flight (1, or an even ring; 2 spills registers)
#endif
struct DwtSmem {
    static constexpr int KC = 64, ROWB = 512;                 // tokens per slice, bytes per row
    static constexpr size_t tile = (size_t)KC * ROWB;          // one tensor, one slice: 32 KB
    static constexpr size_t bufs = 4 * tile;                   // 2 buffers x {dY, X}
    static constexpr size_t stage = sizeof(float) * 128 * (256 + kStPad);  // half the output tile
    static constexpr size_t bytes = bufs > stage ? bufs : stage;
};
__device__ __forceinline__ u16x8 tr_frag_swz(const char* tile, int r0, int c0, int lane) {
    // rows r0 .. r0 + 15 (8 per lane half), columns c0 .. c0 + 31 (elements); r0 % 16 == 0, c0 % 32 == 0
    const int h = lane / 32, grp = (lane % 32) / 16, j = lane % 16;
    const int R = r0 + 8 * h + (j >> 2);
    const int C = c0 + 16 * grp + 4 * (j & 3);
    const int off = R * DwtSmem::ROWB + ((((C >> 3) ^ (4 * (j >> 2))) << 4) | ((C & 7) * 2));
    const i16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(tile + off));
    const i16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(tile + off + 4 * DwtSmem::ROWB));
    u16x8 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[q] = (uint16_t)lo[q];
        v[4 + q] = (uint16_t)hi[q];
    }
    return v;
}

template <int H, bool MEAN>
__device__ __forceinline__ void dw_bf16_tr_body(char* smem, int bid, const uint16_t* __restrict__ dY,
                                                const uint16_t* __restrict__ X, float* __restrict__ part_dw,
                                                float* __restrict__ part_db, const int* __restrict__ offsets,
                                                const int* __restrict__ perm, int NE, int P, int T, int nh,
                                                float inv_nh) {
    constexpr int BT = 256, NTI = H / BT, TPC = NTI * NTI;
    constexpr int KC = DwtSmem::KC, ROWB = DwtSmem::ROWB;
    constexpr int SUBM = 4, SUBN = 2;  // 128 x 64 per wavefront
    char* tiles = smem;  // [buf][tensor][KC][ROWB]
    auto tile = [&](int buf, int tensor) { return tiles + (2 * buf + tensor) * DwtSmem::tile; };

    int c, tl;
    xcd_split(bid, TPC, c, tl);
    int e = -1, t0 = 0, t1 = 0;
    if (!find_chunk(offsets, NE, P, T, c, e, t0, t1)) return;
    const int o0 = (tl / NTI) * BT, i0 = (tl % NTI) * BT;
    const bool do_db = (tl % NTI) == 0;
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, l32 = lane % 32;
    const int wm = wave / 4, wn = wave % 4;
    const bool db_wave = do_db && wn == 0;

    f32x16 acc[SUBM][SUBN];
#pragma unroll
    for (int i = 0; i < SUBM; ++i)
#pragma unroll
        for (int j = 0; j < SUBN; ++j) acc[i][j] = f32x16{};
    float dbacc[SUBM] = {0.0f, 0.0f, 0.0f, 0.0f};

    // thread -> (token quad tq, feature chunk fq): 4 tokens x 16 bytes of each tensor per slice;
    // fq runs fastest, so a wavefront's loads of one token cover 512 contiguous bytes
    const int fq = tid % 32, tq = tid / 32;
    const int nslices = (t1 - t0 + KC - 1) / KC;
    // A ring of PF slices in registers: the rows of slices s+1 .. s+PF and the token ids of the
    // PF slices after those are in flight while slice s computes.  Loads past the chunk's end
    // read its last token and are zeroed when stored, so no load sits under a branch.
    constexpr int PF = MOE_BF16_DWT_RING;
    static_assert(PF == 1 || PF % 2 == 0, "the LDS buffer of slice s0 + u is u % 2");
    int tk[PF][4];
    u16x8 va[PF][4], vb[PF][4];
    auto kpos = [&](int sl, int j) { return t0 + sl * KC + 4 * tq + j; };
    auto load_ids = [&](int sl, int slot) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = kpos(sl, j);
            tk[slot][j] = load_token(perm, k < t1 ? k : t1 - 1, T);
        }
    };
    auto load_rows = [&](int slot) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const size_t t = (size_t)tk[slot][j];
            va[slot][j] = ld8(dY + (MEAN ? t / nh : t) * H + o0 + 8 * fq);
            vb[slot][j] = ld8(X + t * H + i0 + 8 * fq);
        }
    };
    auto store_rows = [&](int sl, int slot, int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool v = kpos(sl, j) < t1;
            const int row = 4 * tq + j;
            const int off = row * ROWB + ((fq ^ (4 * j)) << 4);  // row & 3 == j
            st8(reinterpret_cast<uint16_t*>(tile(buf, 0) + off), v ? va[slot][j] : u16x8{});
            st8(reinterpret_cast<uint16_t*>(tile(buf, 1) + off), v ? vb[slot][j] : u16x8{});
        }
    };
    auto compute = [&](int buf) {
        const char* ta = tile(buf, 0);
        const char* tb = tile(buf, 1);
#pragma unroll
        for (int kk = 0; kk < KC; kk += 16) {
            u16x8 a[SUBM], b[SUBN];
#pragma unroll
            for (int i = 0; i < SUBM; ++i) {
                a[i] = tr_frag_swz(ta, kk, wm * 128 + 32 * i, lane);
                if (MEAN) a[i] = scale8(a[i], inv_nh);
            }
#pragma unroll
            for (int j = 0; j < SUBN; ++j) b[j] = tr_frag_swz(tb, kk, wn * 64 + 32 * j, lane);
#pragma unroll
            for (int i = 0; i < SUBM; ++i)
#pragma unroll
                for (int j = 0; j < SUBN; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
            if (db_wave) {
#pragma unroll
                for (int i = 0; i < SUBM; ++i)
#pragma unroll
                    for (int q = 0; q < 8; ++q) dbacc[i] += bf16_to_f32(a[i][q]);
            }
        }
    };

    if constexpr (PF == 1) {
        load_ids(0, 0);
        load_rows(0);
        load_ids(1, 0);
        store_rows(0, 0, 0);
        __syncthreads();
#pragma unroll 1
        for (int sl = 0; sl < nslices; ++sl) {
            const int buf = sl & 1;
            if (sl + 1 < nslices) {
                load_rows(0);
                load_ids(sl + 2, 0);
            }
            compute(buf);
            if (sl + 1 < nslices) store_rows(sl + 1, 0, buf ^ 1);
            __syncthreads();
        }
    } else {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < PF; ++k) load_ids(k, k);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < PF; ++k) load_rows(k);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < PF; ++k) load_ids(PF + k, k);
        __builtin_amdgcn_sched_barrier(0);
        store_rows(0, 0, 0);
        load_rows(0);
        load_ids(2 * PF, 0);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
#pragma unroll 1
        for (int s0 = 0; s0 < nslices; s0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int sl = s0 + u;
                if (sl >= nslices) break;
                store_rows(sl + 1, (u + 1) % PF, (u + 1) & 1);
                load_rows((u + 1) % PF);
                load_ids(sl + 1 + 2 * PF, (u + 1) % PF);
                __builtin_amdgcn_sched_barrier(0);
                compute(u & 1);
                __syncthreads();
            }
        }
    }

    // the partial tile in two halves of 128 rows through LDS (the loop's last barrier freed the
    // buffers), then whole 16-byte row pieces
    float* __restrict__ Pd = part_dw + (size_t)c * H * H;
    float(&St)[128][BT + kStPad] = *reinterpret_cast<float(*)[128][BT + kStPad]>(smem);
    const int h = lane / 32;
    constexpr int CPR = BT / 4, RPS = kDwtThreads / CPR;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (half > 0) __syncthreads();
        if (wm == half) {
#pragma unroll
            for (int i = 0; i < SUBM; ++i)
#pragma unroll
                for (int j = 0; j < SUBN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        St[i * 32 + 8 * (r / 4) + 4 * h + (r % 4)][wn * 64 + j * 32 + l32] = acc[i][j][r];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 128 / RPS; ++q) {
            const int row = q * RPS + tid / CPR, c4 = tid % CPR;
            *reinterpret_cast<f32x4*>(Pd + (size_t)(o0 + half * 128 + row) * H + i0 + 4 * c4) =
                *reinterpret_cast<const f32x4*>(&St[row][4 * c4]);
        }
    }
    if (db_wave) {
#pragma unroll
        for (int i = 0; i < SUBM; ++i) {
            const float tot = dbacc[i] + __shfl_xor(dbacc[i], 32);
            if (lane < 32) part_db[(size_t)c * H + o0 + wm * 128 + 32 * i + l32] = tot;
        }
    }
}

// The same d_W tile fed by direct global -> LDS loads.  Same tile, wavefront grid and LDS row
// layout as dw_bf16_tr_body (token-major rows of 512 bytes, chunk c of row t at c ^ 4 (t & 3)),
// but the rows go from global memory straight into LDS with buffer_load_dwordx4 ... lds
// (lane i's 16 bytes land at the instruction's LDS base + 16 i), through a ring of R stages of
// 32 tokens: the rows of the next R - 1 slices are in flight while a slice computes, and they
// cost no registers.  Each stage is an LDS object of its own, so the compiler can tell the
// stages apart and a read of one stage does not wait for the loads into another.  A slice is
// complete in LDS once this wavefront's vector-memory counter has fallen to the number of loads
// issued after it -- every ring step issues the same six (four row loads, two token ids) in a
// fixed order, with no exit inside a ring cycle -- and visible to every wavefront after the
// barrier that follows.
// Rows past the chunk's end (and the slices that pad the last ring cycle) read zeros: their byte
// offset lies past the end of the buffer.
#ifndef MOE_BF16_DW_DMA
#define MOE_BF16_DW_DMA 1
#endif
#ifndef MOE_BF16_DMA_STAGES
#define MOE_BF16_DMA_STAGES 4
#endif
struct DwdSmem {
    static constexpr int KC = 32, ROWB = 512;            // tokens per slice, bytes per row
    static constexpr size_t tensor = (size_t)KC * ROWB;  // one tensor of one slice: 16 KB
    static constexpr size_t stage = 2 * tensor;          // dY then X
};
static __device__ __attribute__((aligned(16))) uint16_t kZeroRow[512];  // one zero row of up to H = 512
typedef __attribute__((address_space(3))) void* lds_void_ptr;
// LDS-qualified element types, for volatile reads (through a generic pointer a volatile read
// stays a flat access, which also waits on the vector-memory counter)
typedef __attribute__((address_space(3))) int lds_int;
// buffer descriptor word 3 for raw (untyped) buffer accesses on CDNA: 32-bit data format
constexpr int kBufWord3 = 0x00020000;
// a byte offset past the end of any tensor the library takes (fewer than 2^31 bf16 elements):
// a buffer load from it returns zeros
constexpr uint32_t kPastEnd = 0xFFFF0000u;
typedef __attribute__((address_space(3))) u16x8 lds_u16x8;

// s_waitcnt with the vector-memory count at N and the LDS count at 0 (export count untouched)
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

template <int H, bool MEAN, int R>
__device__ __forceinline__ void dw_bf16_dma_body(char* const (&st)[R], int bid, const uint16_t* __restrict__ dY,
                                                 const uint16_t* __restrict__ X, float* __restrict__ part_dw,
                                                 float* __restrict__ part_db, const int* __restrict__ offsets,
                                                 const int* __restrict__ perm, int NE, int P, int T, int nh,
                                                 float inv_nh) {
    static_assert(R >= 3, "ring depth");
    constexpr int BT = 256, NTI = H / BT, TPC = NTI * NTI;
    constexpr int KC = DwdSmem::KC, ROWB = DwdSmem::ROWB;
    constexpr int SUBM = 4, SUBN = 2;  // 128 x 64 per wavefront

    int c, tl;
    xcd_split(bid, TPC, c, tl);
    int e = -1, t0 = 0, t1 = 0;
    if (!find_chunk(offsets, NE, P, T, c, e, t0, t1)) return;
    const int o0 = (tl / NTI) * BT, i0 = (tl % NTI) * BT;
    const bool do_db = (tl % NTI) == 0;
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, l32 = lane % 32;
    const int wm = wave / 4, wn = wave % 4;
    const bool db_wave = do_db && wn == 0;

    f32x16 acc[SUBM][SUBN];
#pragma unroll
    for (int i = 0; i < SUBM; ++i)
#pragma unroll
        for (int j = 0; j < SUBN; ++j) acc[i][j] = f32x16{};
    float dbacc[SUBM] = {0.0f, 0.0f, 0.0f, 0.0f};

    // wavefront w fills rows 4w .. 4w + 3 of each tensor of a stage, two rows per load: in load q,
    // lane i takes row 4w + 2q + (i >> 5) and physical chunk i & 31, i.e. logical chunk
    // (i & 31) ^ 4 (row & 3) with row & 3 = 2q + (i >> 5)
    const int lh = lane >> 5, pch = lane & 31;
    const int lc0 = pch ^ (4 * lh), lc1 = pch ^ (4 * (2 + lh));
    const int nslices = (t1 - t0 + KC - 1) / KC;
    auto row_k = [&](int sl, int q) { return t0 + sl * KC + 4 * wave + 2 * q + lh; };
    // perm entries of the slice whose index is congruent to the slot mod R, as loaded: the
    // guard is applied where the rows are addressed, so no wait for them sits at the ring's back edge
    int tk[R][2];
    auto load_ids = [&](int sl, int slot) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int k = row_k(sl, q);
            tk[slot][q] = perm[k < t1 ? k : (t1 > 0 ? t1 - 1 : 0)];
        }
    };
    // buffer loads through descriptors of the whole of dY and X (bf16 tensors of fewer than 2^31
    // elements, so every byte offset fits 32 bits); a padded row takes an offset past the end,
    // which the range check turns into zeros.  (The buffer form, not global_load_lds: the
    // compiler treats the global form as a flat access and then makes every LDS wait total.)
    const __amdgpu_buffer_rsrc_t y_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)dY, 0, (int)((uint32_t)(MEAN ? T / nh : T) * (uint32_t)H * 2u), kBufWord3);
    const __amdgpu_buffer_rsrc_t x_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)X, 0, (int)((uint32_t)T * (uint32_t)H * 2u), kBufWord3);
    auto dma = [&](int sl, int slot, char* stg) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const bool v = row_k(sl, q) < t1;
            const int lc = q ? lc1 : lc0;
            const uint32_t t = (uint32_t)guard_token(tk[slot][q], T);
            const uint32_t oy = v ? (((MEAN ? t / nh : t) * H + o0 + 8 * lc) * 2u) : kPastEnd;
            const uint32_t ox = v ? ((t * H + i0 + 8 * lc) * 2u) : kPastEnd;
            char* ly = stg + (4 * wave + 2 * q) * ROWB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(y_rs, (lds_void_ptr)ly, 16, (int)oy, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rs, (lds_void_ptr)(ly + DwdSmem::tensor), 16, (int)ox, 0, 0, 0);
        }
    };
    auto compute = [&](const char* stg) {
        const char* ta = stg;
        const char* tb = stg + DwdSmem::tensor;
#pragma unroll
        for (int kk = 0; kk < KC; kk += 16) {
            u16x8 a[SUBM], b[SUBN];
#pragma unroll
            for (int i = 0; i < SUBM; ++i) {
                a[i] = tr_frag_swz(ta, kk, wm * 128 + 32 * i, lane);
                if (MEAN) a[i] = scale8(a[i], inv_nh);
            }
#pragma unroll
            for (int j = 0; j < SUBN; ++j) b[j] = tr_frag_swz(tb, kk, wn * 64 + 32 * j, lane);
#pragma unroll
            for (int i = 0; i < SUBM; ++i)
#pragma unroll
                for (int j = 0; j < SUBN; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
            if (db_wave) {
#pragma unroll
                for (int i = 0; i < SUBM; ++i)
#pragma unroll
                    for (int q = 0; q < 8; ++q) dbacc[i] += bf16_to_f32(a[i][q]);
            }
        }
    };

    // prologue: token ids of slices 0 .. R - 1, then the rows of slices 0 .. R - 2, each followed
    // by the ids of the slice R later (the same six loads per slice as a ring step).  The
    // scheduling barriers keep the loads in this order, which the counts below rely on.
    auto pin = [] {  // no load moves across this point, in the optimiser or the scheduler
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int k = 0; k < R; ++k) load_ids(k, k);
#pragma unroll
    for (int k = 0; k + 1 < R; ++k) {
        pin();
        dma(k, k, st[k]);
        pin();
        load_ids(k + R, k);
    }
    pin();
    // ring step s: wait for slice s (at least the R - 2 later steps' six loads each were issued
    // after its rows), barrier (slice s visible; every wavefront is done with the stage of slice
    // s - 1), rows of slice s + R - 1 into that stage, ids of slice s + 2R - 1, slice s's MFMAs
    // at least one cycle, so the loop has no conditional entry for the prologue's loads to sink
    // into (an empty chunk computes nothing and writes zeros)
    const int ncycles = max(1, (nslices + R - 1) / R);
    int cyc = 0;
#pragma unroll 1
    do {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int s = cyc * R + u;
            wait_vm_lds<6 * (R - 2)>();
            __builtin_amdgcn_s_barrier();
            pin();
            dma(s + R - 1, (u + R - 1) % R, st[(u + R - 1) % R]);
            pin();
            load_ids(s + 2 * R - 1, (u + R - 1) % R);
            pin();
            if (s < nslices) compute(st[u]);
        }
    } while (++cyc < ncycles);
    // every load into LDS must land before the workgroup ends (the LDS is the next one's)
    wait_vm_lds<0>();

    // the partial tile straight from the accumulators: each store writes two 128-byte row pieces
    float* __restrict__ Pd = part_dw + (size_t)c * H * H;
    const int h = lane / 32;
#pragma unroll
    for (int i = 0; i < SUBM; ++i)
#pragma unroll
        for (int j = 0; j < SUBN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                Pd[(size_t)(o0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4)) * H + i0 + wn * 64 + j * 32 + l32] =
                    acc[i][j][r];
    if (db_wave) {
#pragma unroll
        for (int i = 0; i < SUBM; ++i) {
            const float tot = dbacc[i] + __shfl_xor(dbacc[i], 32);
            if (lane < 32) part_db[(size_t)c * H + o0 + wm * 128 + 32 * i + l32] = tot;
        }
    }
}

// W-stationary row GEMM (H = 256 / 512, large T): Out[t, n0 : n0 + 256] = A[t, :] . Wm[n, :]^T
// (+ bias) for the tokens of one expert.  Each of the 256 workgroups (one per compute unit,
// eight wavefronts, two per SIMD) owns a 256-feature slice of W[e] -- each wavefront 32
// features, held in its registers as MFMA operands for the whole K (128 VGPRs at H = 512) --
// and streams a fixed share of the expert-sorted token order through it in groups of 32
// tokens: their rows go to LDS whole (one row per load instruction at H = 512, 16-byte chunk c
// of row r at c ^ (r & 15)), each wavefront reads its MFMA fragments from there, and the fp32
// results are staged in LDS and written a group later by all threads as whole 512-byte pieces
// of output rows.  Against the resident-slice forward (W in LDS, rows loaded straight into
// operand registers, 64 rows per load instruction) a row is fetched by half as many compute
// units and each load touches 8 cache lines instead of 64.  The forward passes W ([n][k]),
// dX passes W^T.
// The token share: slice s of workgroup wg covers positions [v T / V, (v + 1) T / V) of the
// expert-sorted order (V workgroups per slice, the slices of one share on one XCD), cut at
// expert boundaries into segments; each segment loads its expert's W slice once (dX: its W^T
// fragments, through LDS and the transposing read).
#ifndef MOE_BF16_WST
#define MOE_BF16_WST 1
#endif
constexpr int kWstThreads = 512, kWstWgs = 256, kWstGT = 32;
template <int H>
struct WstSmem {
    static constexpr int ROWB = 2 * H;                          // bytes per token row
    static constexpr size_t xbuf = (size_t)kWstGT * ROWB;       // one group's rows
    static constexpr size_t obuf = (size_t)kWstGT * 256 * 4;    // one group's fp32 results [32][256]
    static constexpr size_t ost_off = 2 * xbuf;
    static constexpr size_t bias_off = ost_off + 2 * obuf;
    static constexpr size_t ids_off = bias_off + 256 * 4;       // token ids: [5][32]
    static constexpr size_t bytes = ids_off + 5 * kWstGT * 4;
};
// 256 workgroups when every slice share holds at least 8 groups of 32 tokens
static inline bool bf16_wst(int64_t T, int H) {
    return MOE_BF16_WST && H >= 256 && T >= (int64_t)(kWstWgs / (H / 256)) * 8 * kWstGT;
}

// Rows k0 .. k0 + NR - 1, columns n0 .. n0 + 255 of one expert's W (bf16, rows of H) into an
// LDS stage of 512-byte rows, 16-byte chunk c of row r at c ^ 4 (r & 3) (where the transposing
// reads of tr_frag_swz find them conflict-free), with direct-to-LDS loads, two rows per
// wavefront load and all of them in flight at once; the caller waits and synchronises.
template <int H, int NR, int NWV>
__device__ __forceinline__ void stage_w_rows(char* wst, const uint16_t* __restrict__ We, int k0, int n0, int wave,
                                             int lane) {
    constexpr int PER = NR / 2 / NWV;  // loads per wavefront (NWV of them), two rows each
    static_assert(NR % 32 == 0 && PER % 2 == 0, "rows per stage");
    // wavefront w fills rows 2 PER w .. + 2 PER - 1, four rows (two loads) per step; within a
    // step, lane i takes row 2 q + (i >> 5) of load q and physical chunk i & 31 (r & 3 = 2 q + (i >> 5))
    const int sub = lane >> 5, pc = lane & 31;
    const int off0 = sub * H + 8 * (pc ^ (4 * sub));
    const int off1 = (2 + sub) * H + 8 * (pc ^ (4 * (2 + sub)));
    const uint16_t* src = We + (size_t)(k0 + 2 * PER * wave) * H + n0;
    char* dst = wst + 2 * PER * wave * 512;
    // a loop, not unrolled: unrolled, the compiler keeps every load's address live across the
    // caller's loops (and spills them)
#pragma unroll 1
    for (int j = 0; j < PER; j += 2) {
        __builtin_amdgcn_global_load_lds((const void*)(src + off0), (lds_void_ptr)dst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(src + off1), (lds_void_ptr)(dst + 1024), 16, 0, 0);
        src += 4 * H;
        dst += 2048;
    }
}

template <int H, bool DX, bool MEAN, bool ACC>
__device__ __forceinline__ void rows_bf16_wst_body(char* smem, const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ Wm, const float* __restrict__ bias,
                                                   uint16_t* __restrict__ Out, const int* __restrict__ offsets,
                                                   const int* __restrict__ perm, int NE, int T, int nh,
                                                   float inv_nh) {
    using S = WstSmem<H>;
    constexpr int NS = H / 256, NKS = H / 16, V = kWstWgs / NS;
    constexpr int CPR = S::ROWB / 16;       // 16-byte chunks per row
    constexpr int RPI = kWstThreads / CPR;  // rows per load round
    constexpr int NL = kWstGT / RPI;        // row loads per thread per group
    static_assert(kWstWgs % (8 * NS) == 0 && kWstGT % RPI == 0, "shape");
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, l32 = lane % 32, h = lane / 32;
    const int bid = blockIdx.x;
    const int s = (bid / 8) % NS, v = (bid % 8) + 8 * (bid / (8 * NS));
    const int n0 = 256 * s, fw = 32 * wave;  // this wavefront's features n0 + fw + 0..31
    const int P0 = (int)((int64_t)v * T / V), P1 = (int)((int64_t)(v + 1) * T / V);
    char* const xb0 = smem;
    char* const xb1 = smem + S::xbuf;
    float* const ob0 = reinterpret_cast<float*>(smem + S::ost_off);
    float* const ob1 = reinterpret_cast<float*>(smem + S::ost_off + S::obuf);
    float* const bias_s = reinterpret_cast<float*>(smem + S::bias_off);
    // token ids of group g in ids[g % 5]: written at g - 2, read at g - 1 (its rows' loads) and at
    // g + 1 (its output), so with five buffers no wavefront overwrites ids another still reads
    int(&ids)[5][kWstGT] = *reinterpret_cast<int(*)[5][kWstGT]>(smem + S::ids_off);
    int x_lo, x_cnt;
    expert_range(offsets, NE, T, x_lo, x_cnt);
    const int lrow = tid / CPR, lch = tid % CPR;
    // output pieces: thread -> feature chunk pc (8 features) of rows tid / 32 + 16 i
    const int pc = tid % 32, prow = tid / 32;

    u16x8 wr[NKS];  // features n0 + fw + l32, k 16 ks + 8 h ..
    u16x8 xr[NL];   // the next group's rows, in flight

    auto load_x = [&](const int* gid) {  // a padded row reads the zero row
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int t = gid[lrow + RPI * j];
            const uint16_t* src =
                t >= 0 ? A + (size_t)(MEAN ? t / nh : t) * H + 8 * lch : kZeroRow + 8 * lch;
            xr[j] = ld8(src);
        }
    };
    auto store_x = [&](char* xb) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int r = lrow + RPI * j;
            st8(reinterpret_cast<uint16_t*>(xb + r * S::ROWB + 16 * (lch ^ (r & 15))), xr[j]);
        }
    };
    // fp32 result row r (token), 64 chunks of 4 features: chunk c at c ^ (r & 15)
    auto ost_at = [](float* ob, int r, int c) { return ob + r * 256 + 4 * (c ^ (r & 15)); };
    auto compute = [&](const char* xb, float* ob) {
        const char* row = xb + l32 * S::ROWB;
        f32x16 acc = f32x16{};
        // fragments in batches of 4 k-steps, each batch read before its MFMAs, so the LDS reads
        // overlap the MFMA chain instead of each MFMA waiting for its own read
        constexpr int KB = 4;
#pragma unroll
        for (int k0 = 0; k0 < NKS; k0 += KB) {
            u16x8 xf[KB];
#pragma unroll
            for (int u = 0; u < KB; ++u)
                xf[u] = *reinterpret_cast<const u16x8*>(row + 16 * ((2 * (k0 + u) + h) ^ (l32 & 15)));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                if (MEAN) xf[u] = scale8(xf[u], inv_nh);
                acc = mfma_bf16(wr[k0 + u], xf[u], acc);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane: token l32, features fw + 8 q + 4 h .. + 3
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 val = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
            *reinterpret_cast<f32x4*>(ost_at(ob, l32, (fw >> 2) + 2 * q + h)) = val;
        }
    };
    auto store_out = [&](const float* ob, const int* gid) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = prow + 16 * i;
            const int t = gid[r];
            u16x8 old;
            if (ACC) old = ld8(Out + (size_t)(t < 0 ? 0 : t) * H + n0 + 8 * pc);
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(ost_at(const_cast<float*>(ob), r, 2 * pc));
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(ost_at(const_cast<float*>(ob), r, 2 * pc + 1));
            float vv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            if (!DX) {
                const f32x4 b0 = *reinterpret_cast<const f32x4*>(bias_s + 8 * pc);
                const f32x4 b1 = *reinterpret_cast<const f32x4*>(bias_s + 8 * pc + 4);
                const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int u = 0; u < 8; ++u) vv[u] += bv[u];
            }
            if (ACC) {
#pragma unroll
                for (int u = 0; u < 8; ++u) vv[u] = bf16_to_f32(old[u]) + vv[u];
            }
            u32x4v pk;
#pragma unroll
            for (int u = 0; u < 4; ++u) pk[u] = pack_bf16x2(vv[2 * u], vv[2 * u + 1]);
            if (t >= 0) st8_nt(Out + (size_t)t * H + n0 + 8 * pc, __builtin_bit_cast(u16x8, pk));
        }
    };

    int p = P0;
    while (p < P1) {
        // segment: positions [p, se) of expert e
        const uint64_t hit = __ballot(lane < NE && p >= x_lo && p < x_lo + x_cnt);
        if (hit == 0) break;  // (only with routing that does not cover [0, T))
        const int e = __ffsll((unsigned long long)hit) - 1;
        const int se = min(P1, __builtin_amdgcn_readlane(x_lo, e) + __builtin_amdgcn_readlane(x_cnt, e));
        const int G = (se - p + kWstGT - 1) / kWstGT;
        // this thread's entry of perm in group g, as loaded (an unconditional load of a clamped
        // position, so no wait sits under a branch; the guard and the validity are applied where
        // the id is written to LDS, a group later, so nothing waits for the load here)
        auto group_raw = [&](int g) {
            const int k = p + kWstGT * g + (tid % kWstGT);
            return perm[k < se ? k : se - 1];
        };
        auto group_valid = [&](int g) { return g < G && p + kWstGT * g + (tid % kWstGT) < se; };
        __syncthreads();  // the previous segment is done with the bias, ids and staged results
        if constexpr (!DX) {  // W[e] rows n0 + fw + l32, k contiguous
            const uint16_t* __restrict__ We = Wm + (size_t)e * H * H + (size_t)(n0 + fw + l32) * H + 8 * h;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) wr[ks] = ld8(We + 16 * ks);
        } else {
            // W^T fragments: W[e] rows k (256 at a time) x columns n0 .. n0 + 255 staged in the
            // group buffers (512-byte rows, chunk c of row r at c ^ 4 (r & 3)), read back with the
            // transposing LDS read (8 consecutive k of one column per lane)
            constexpr int WROWS = (2 * S::xbuf + 2 * S::obuf >= 256 * 512) ? 256 : 128;  // rows per stage
            static_assert(2 * S::xbuf + 2 * S::obuf >= (size_t)WROWS * 512 && H % WROWS == 0, "LDS for a W stage");
            char* const wst = smem;
#pragma unroll  // compile-time k0, so the register array wr keeps constant indices
            for (int k0 = 0; k0 < H; k0 += WROWS) {
                if (k0 > 0) __syncthreads();  // the previous stage is read
                stage_w_rows<H, WROWS, kWstThreads / 64>(wst, Wm + (size_t)e * H * H, k0, n0,
                                                         __builtin_amdgcn_readfirstlane(wave), lane);
                wait_vm_lds<0>();
                __syncthreads();
#pragma unroll
                for (int ks = 0; ks < WROWS / 16; ++ks) wr[k0 / 16 + ks] = tr_frag_swz(wst, 16 * ks, fw, lane);
            }
        }
        if (!DX && tid < 256) bias_s[tid] = bias[(size_t)e * H + n0 + tid];
        {
            const int i0 = group_raw(0), i1 = group_raw(1);
            if (tid < kWstGT) {
                ids[0][tid] = group_valid(0) ? guard_token(i0, T) : -1;
                ids[1][tid] = group_valid(1) ? guard_token(i1, T) : -1;
            }
        }
        int idr = group_raw(2);  // ids in flight: of group g + 2 during group g
        __syncthreads();
        load_x(ids[0]);
        // group g: its rows to LDS (and the ids of g + 2); the output of g - 1 to memory; the rows
        // of g + 1 and the ids of g + 3 into flight (after the stores: ahead of them, the stores
        // queue behind the loads and the next wait takes longer); the MFMAs of g
#pragma unroll 1
        for (int g = 0; g < G; ++g) {
            char* const xb = (g & 1) ? xb1 : xb0;
            store_x(xb);
            if (tid < kWstGT) ids[(g + 2) % 5][tid] = group_valid(g + 2) ? guard_token(idr, T) : -1;
            __syncthreads();
            if (g > 0) store_out((g & 1) ? ob0 : ob1, ids[(g - 1) % 5]);
            if (g + 1 < G) load_x(ids[(g + 1) % 5]);
            idr = group_raw(g + 3);
            compute(xb, (g & 1) ? ob1 : ob0);
        }
        __syncthreads();
        store_out(((G - 1) & 1) ? ob1 : ob0, ids[(G - 1) % 5]);
        p = se;
    }
}

// Role-split variant (outputs overwritten, not accumulated).  The single-role body above keeps one
// group of rows in flight: its loads go through registers, and because every wavefront also has
// output stores pending, the wait for those rows is a wait for everything.  Here the first half
// of the NW wavefronts ("loaders") move rows from global memory straight into a ring of three
// LDS stages (buffer_load_dwordx4 ... lds), two groups ahead of the MFMAs, and issue no stores; the
// other half ("storers") write the finished rows and issue no loads into that ring.  Each role's
// loop thus has one kind of memory operation pending and waits for exactly the group it needs.
// All wavefronts run the MFMAs, each on 256 / NW features; bias add and bf16 rounding happen in
// the accumulator registers (the same fp32 add and the same rounding as the single-role body, so
// the results are bit-identical), and the bf16 rows are staged in LDS for the storers.
// NW = 4 (one wavefront per SIMD, 64 features each: W in 256 of its 512 registers at H = 512)
// reads every row fragment from LDS once per two MFMAs, NW = 8 (two per SIMD, 32 features each)
// once per MFMA; NW = 8 measured faster at H = 512 (a single wavefront per SIMD leaves the
// latencies of its LDS reads and loads uncovered).
#ifndef MOE_BF16_WST_ROLES
#define MOE_BF16_WST_ROLES 1
#endif
#ifndef MOE_BF16_WSR_WAVES
#define MOE_BF16_WSR_WAVES 8
#endif
#ifndef MOE_BF16_WSR_KB
#define MOE_BF16_WSR_KB 1
#endif
#ifndef MOE_BF16_WSR_PD
#define MOE_BF16_WSR_PD 3
#endif
static_assert(MOE_BF16_WSR_WAVES == 4 || MOE_BF16_WSR_WAVES == 8, "role-split wavefronts");
template <bool ACC>
constexpr int wst_threads() { return (MOE_BF16_WST_ROLES && !ACC) ? 64 * MOE_BF16_WSR_WAVES : kWstThreads; }
template <int H>
struct WsrSmem {
    static constexpr int ROWB = 2 * H;                          // bytes per token row
    static constexpr int NX = 3;                                // row stages
    static constexpr size_t xbuf = (size_t)kWstGT * ROWB;       // one group's rows
    static constexpr size_t obuf = (size_t)kWstGT * 256 * 2;    // one group's bf16 results [32][256]
    static constexpr size_t ost_off = NX * xbuf;
    static constexpr size_t bias_off = ost_off + 2 * obuf;
    static constexpr size_t ids_off = bias_off + 256 * 4;       // token ids: [4][32]
    static constexpr size_t raw_off = ids_off + 4 * kWstGT * 4; // perm entries as loaded: [4][4 waves][64]
    static constexpr size_t bytes = raw_off + 4 * 4 * 64 * 4;
};

template <int H, bool DX, bool MEAN, int NW>
__device__ __forceinline__ void rows_bf16_wsr_body(char* smem, const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ Wm, const float* __restrict__ bias,
                                                   uint16_t* __restrict__ Out, const int* __restrict__ offsets,
                                                   const int* __restrict__ perm, int NE, int T, int nh,
                                                   float inv_nh) {
    using S = WsrSmem<H>;
    constexpr int NS = H / 256, NKS = H / 16, V = kWstWgs / NS;
    constexpr int CPR = S::ROWB / 16;   // 16-byte chunks per row
    constexpr int RPD = 64 / CPR;       // rows per direct-to-LDS load of one wavefront (64 x 16 bytes)
    constexpr int NB = 8 / NW;          // 32-feature blocks per wavefront
    constexpr int NLW = NW / 2;         // loader wavefronts
    constexpr int RPW = kWstGT / NLW;   // rows per loader wavefront per group
    constexpr int DPG = RPW / RPD;      // direct-to-LDS loads per loader wavefront per group
    constexpr int SW = NW - NLW;        // storer wavefronts
    constexpr int RPL = kWstGT / (2 * SW);  // rows per storer lane per group
    static_assert((NW == 4 || NW == 8) && RPW % RPD == 0 && RPW <= 64 && CPR >= 16, "shape");
    const int tid = threadIdx.x, lane = tid % 64, l32 = lane % 32, h = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const bool loader = wave < NLW;
    const int bid = blockIdx.x;
    const int s = (bid / 8) % NS, v = (bid % 8) + 8 * (bid / (8 * NS));
    const int n0 = 256 * s, fw = 32 * NB * wave;  // this wavefront's features n0 + fw + 0 .. 32 NB - 1
    const int P0 = (int)((int64_t)v * T / V), P1 = (int)((int64_t)(v + 1) * T / V);
    float* const bias_s = reinterpret_cast<float*>(smem + S::bias_off);
    // token ids of group g in ids[g % 4]: written by the loaders when they issue the group's rows
    // (two groups ahead), read by the storers a group after its MFMAs
    int(&ids)[4][kWstGT] = *reinterpret_cast<int(*)[4][kWstGT]>(smem + S::ids_off);
    auto xstage = [&](int g) { return smem + (g % S::NX) * S::xbuf; };
    auto ostage = [&](int g) { return smem + S::ost_off + (g & 1) * S::obuf; };
    int x_lo, x_cnt;
    expert_range(offsets, NE, T, x_lo, x_cnt);

    u16x8 wr[NB][NKS];  // block b: features n0 + fw + 32 b + l32, k 16 ks + 8 h ..

    // MFMAs of one group; the results, plus bias and rounded to bf16, into the group's output
    // stage: row = token l32, 16-byte chunk c (features 8c .. 8c + 7) at c ^ (row & 31).
    // mid(bt) runs after the MFMAs of batch bt are issued: the role's memory work placed there
    // issues while the matrix cores are busy, instead of in a phase of its own.
    constexpr int NBT = NKS / MOE_BF16_WSR_KB;  // batches of the MFMA loop
    auto compute = [&](int g, auto&& mid) {
        const char* row = xstage(g) + l32 * S::ROWB;
        // chunk (2 ks + h) ^ (l32 & 15) of the row, written as 16 (ks / 8) + ((2 (ks % 8) + h) ^
        // (l32 & 15)): the same chunk (the xor touches only the low four bits), but with eight
        // per-lane offsets and the rest an immediate, not one address register per k-step
        auto frag = [&](int ks) {
            return *reinterpret_cast<const u16x8*>(row + 256 * (ks >> 3) + 16 * ((2 * (ks & 7) + h) ^ (l32 & 15)));
        };
        // software-pipelined in batches of KB k-steps, the reads PD batches ahead of the MFMAs
        // that use them, so the LDS serves later batches while the matrix cores work on this one
        // (with all wavefronts reading, then all multiplying, in step, the two would take turns;
        // one batch ahead leaves the LDS latency uncovered)
        constexpr int KB = MOE_BF16_WSR_KB;
        constexpr int PD = MOE_BF16_WSR_PD;
        static_assert(NKS % KB == 0 && PD >= 1 && PD < NBT, "pipeline");
        f32x16 acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
        u16x8 buf[PD + 1][KB];
#pragma unroll
        for (int bt = 0; bt < PD; ++bt)
#pragma unroll
            for (int u = 0; u < KB; ++u) buf[bt][u] = frag(KB * bt + u);
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) {
            if (bt + PD < NBT) {
#pragma unroll
                for (int u = 0; u < KB; ++u) buf[(bt + PD) % (PD + 1)][u] = frag(KB * (bt + PD) + u);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                u16x8 x = buf[bt % (PD + 1)][u];
                if (MEAN) x = scale8(x, inv_nh);
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[b] = mfma_bf16(wr[b][KB * bt + u], x, acc[b]);
            }
            mid(bt);
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane: token l32, features fw + 32 b + 8 q + 4 h .. + 3
        char* const orow = ostage(g) + l32 * 512;
        // the bias reads all issued before the first staging write (which the compiler cannot
        // tell apart from them, so interleaved they would each wait on their own)
        f32x4 bv[NB][4];
        if (!DX) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    bv[b][q] = *reinterpret_cast<const f32x4*>(bias_s + fw + 32 * b + 8 * q + 4 * h);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = fw + 32 * b + 8 * q;
                float vv[4] = {acc[b][4 * q], acc[b][4 * q + 1], acc[b][4 * q + 2], acc[b][4 * q + 3]};
                if (!DX) {
                    vv[0] += bv[b][q].x;
                    vv[1] += bv[b][q].y;
                    vv[2] += bv[b][q].z;
                    vv[3] += bv[b][q].w;
                }
                const i32x2v pk = {(int)pack_bf16x2(vv[0], vv[1]), (int)pack_bf16x2(vv[2], vv[3])};
                *reinterpret_cast<i32x2v*>(orow + 16 * ((f >> 3) ^ (l32 & 31)) + 8 * h) = pk;
            }
    };

    int p = P0;
    while (p < P1) {
        // segment: positions [p, se) of expert e
        const uint64_t hit = __ballot(lane < NE && p >= x_lo && p < x_lo + x_cnt);
        if (hit == 0) break;  // (only with routing that does not cover [0, T))
        const int e = __ffsll((unsigned long long)hit) - 1;
        const int se = min(P1, __builtin_amdgcn_readlane(x_lo, e) + __builtin_amdgcn_readlane(x_cnt, e));
        const int G = (se - p + kWstGT - 1) / kWstGT;
        __syncthreads();  // the previous segment is done with every stage, the bias and the ids
        if constexpr (!DX) {  // W[e] rows n0 + fw + 32 b + l32, k contiguous
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint16_t* __restrict__ We =
                    Wm + (size_t)e * H * H + (size_t)(n0 + fw + 32 * b + l32) * H + 8 * h;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) wr[b][ks] = ld8(We + 16 * ks);
            }
        } else {
            // W^T fragments: W[e] rows k (WROWS at a time) x columns n0 .. n0 + 255 staged in the
            // row and output stages (512-byte rows, chunk c of row r at c ^ 4 (r & 3)), read back
            // with the transposing LDS read (8 consecutive k of one column per lane)
            constexpr int WROWS = (S::bias_off >= 256 * 512) ? 256 : 128;
            static_assert(S::bias_off >= (size_t)WROWS * 512 && H % WROWS == 0, "LDS for a W stage");
            char* const wst = smem;
#pragma unroll
            for (int k0 = 0; k0 < H; k0 += WROWS) {
                if (k0 > 0) __syncthreads();
                stage_w_rows<H, WROWS, NW>(wst, Wm + (size_t)e * H * H, k0, n0, wave, lane);
                wait_vm_lds<0>();
                __syncthreads();
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int ks = 0; ks < WROWS / 16; ++ks)
                        wr[b][k0 / 16 + ks] = tr_frag_swz(wst, 16 * ks, fw + 32 * b, lane);
            }
            __syncthreads();  // every wavefront has its fragments before the rows overwrite the stage
        }
        if (!DX && tid < 256) bias_s[tid] = bias[(size_t)e * H + n0 + tid];
        if (loader) {
            // perm entries of this wavefront's rows RPW wave + (i % RPW) of group g (lane i; clamped
            // positions, validity applied when the group is issued), loaded straight into LDS
            // like the rows.  Nothing in this loop is loaded into registers: the compiler models
            // a direct-to-LDS load as a flat access, and while one is in flight every wait it
            // would insert for a register load is a wait for everything.  The only waits on the
            // vector-memory counter are the explicit ones below, which count these loads too.
            int* const raw_s = reinterpret_cast<int*>(smem + S::raw_off) + 64 * wave;
            // The loads into LDS go through buffer descriptors where they can: the compiler
            // models global_load_lds as a flat access, and while one is in flight every LDS
            // wait it inserts (those of the MFMA loop's fragment reads) becomes a wait for all
            // of them; a buffer load is a plain vector-memory access.
            const __amdgpu_buffer_rsrc_t perm_rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(perm + p), 0, 4 * (se - p), kBufWord3);
            auto load_ids = [&](int g) {
                const int k = min(p + kWstGT * g + RPW * wave + lane % RPW, se - 1) - p;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(perm_rs, (lds_void_ptr)(raw_s + 256 * (g & 3)), 4, 4 * k, 0, 0,
                                                         0);
            };
            // one wavefront load of rows into LDS.  One row per load (H = 512): a descriptor of
            // that row (tt uniform), so the lane offsets are constants; a padded row gets a
            // descriptor of no bytes, which the range check turns into zeros without a memory
            // access (every workgroup reading one zero row would queue on one L2 channel).  Two rows per load (H = 256): a descriptor of the whole of A (fewer than
            // 2^31 bf16 elements: byte offsets fit 32 bits), a padded row taking an offset past
            // the end, which the range check turns into zeros.
            const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)A, 0, (int)((uint32_t)(MEAN ? T / nh : T) * (uint32_t)H * 2u), kBufWord3);
            auto row_dma = [&](int tt, int lc, char* dst) {
                if constexpr (RPD == 1) {
                    const uint16_t* rowp = tt >= 0 ? A + (size_t)(MEAN ? tt / nh : tt) * H : A;
                    const __amdgpu_buffer_rsrc_t rs =
                        __builtin_amdgcn_make_buffer_rsrc((void*)rowp, 0, tt >= 0 ? S::ROWB : 0, kBufWord3);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)dst, 16, 16 * lc, 0, 0, 0);
                } else {
                    const uint32_t off =
                        tt >= 0 ? (((uint32_t)(MEAN ? tt / nh : tt) * H + 8 * lc) * 2u) : kPastEnd;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (lds_void_ptr)dst, 16, (int)off, 0, 0, 0);
                }
            };
            // group g's rows into its stage: load q covers rows RPW wave + RPD q .. + RPD - 1, lane
            // i taking row RPW wave + RPD q + i / CPR and physical chunk i % CPR, which holds
            // logical chunk (i % CPR) ^ (row & 15); padded rows are zeros
            auto issue = [&](int g) {
                const int kb = p + kWstGT * g + RPW * wave;
                const int raw = raw_s[256 * (g & 3) + lane];  // the entry of row lane % RPW
                // every lane writes the id of row lane % RPW (lanes with the same row write the
                // same value), so no branch
                ids[g & 3][RPW * wave + lane % RPW] = kb + lane % RPW < se ? guard_token(raw, T) : -1;
                char* const xs = xstage(g);
#pragma unroll
                for (int q = 0; q < DPG; ++q) {
                    const int sub = lane / CPR, pcl = lane % CPR;
                    const int j = RPD * q + sub, rw = RPW * wave + j;
                    const int rj = RPD == 1 ? __builtin_amdgcn_readlane(raw, RPD * q)
                                            : (sub ? __builtin_amdgcn_readlane(raw, RPD * q + 1)
                                                   : __builtin_amdgcn_readlane(raw, RPD * q));
                    const int tt = kb + j < se ? guard_token(rj, T) : -1;
                    row_dma(tt, pcl ^ (rw & 15), xs + (RPW * wave + RPD * q) * S::ROWB);
                }
            };
            auto pin = [] {  // no memory access moves across this point
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            };
            load_ids(0);
            load_ids(1);
            load_ids(2);
            pin();
            wait_vm_lds<0>();
            pin();
            // groups at or past G are issued too, as zero rows into a stage no one reads any more,
            // so that every iteration has the same loads in flight and every wait one count
            issue(0);
            issue(1);
            // the barriers here wait explicitly: a workgroup fence would also wait for the rows
            // still in flight into LDS.  lgkmcnt(0) covers this wavefront's LDS writes (ids,
            // bias, results); the empty asm and the scheduling barriers keep every memory access
            // on its side of the barrier
            auto ring_barrier = [&] {
                pin();
                wait_vm_lds<DPG>();
                __builtin_amdgcn_s_barrier();
                pin();
            };
            ring_barrier();
            // group g: the ids of g + 3, then, interleaved with the MFMAs of g (one load every
            // STEP batches), the rows of g + 2 into the stage g - 1 used (every wavefront finished
            // it before the barrier); then the wait for the rows of g + 1 (only those of g + 2
            // may stay in flight; the ids are older)
            constexpr int STEP = NBT / DPG;
            static_assert(NBT % DPG == 0 && STEP >= 1, "loads per batch");
#pragma unroll 1
            for (int g = 0; g < G; ++g) {
                load_ids(g + 3);
                pin();
                const int gi = g + 2, kb = p + kWstGT * gi + RPW * wave;
                const int raw = *(volatile const lds_int*)(raw_s + 256 * (gi & 3) + lane);
                char* const xs = xstage(gi);
                int tq[DPG];  // per load: this lane's row's token (-1: padded)
                compute(g, [&](int bt) {
                    if (bt == 0) {
                        ids[gi & 3][RPW * wave + lane % RPW] = kb + lane % RPW < se ? guard_token(raw, T) : -1;
#pragma unroll
                        for (int q = 0; q < DPG; ++q) {
                            const int sub = lane / CPR, j = RPD * q + sub;
                            const int rj = RPD == 1 ? __builtin_amdgcn_readlane(raw, RPD * q)
                                                    : (sub ? __builtin_amdgcn_readlane(raw, RPD * q + 1)
                                                           : __builtin_amdgcn_readlane(raw, RPD * q));
                            tq[q] = kb + j < se ? guard_token(rj, T) : -1;
                        }
                    }
                    if (bt % STEP == STEP - 1) {
                        const int q = bt / STEP;
                        const int sub = lane / CPR, pcl = lane % CPR, rw = RPW * wave + RPD * q + sub;
                        row_dma(tq[q], pcl ^ (rw & 15), xs + (RPW * wave + RPD * q) * S::ROWB);
                    }
                });
                ring_barrier();
            }
            wait_vm_lds<0>();  // the last zero rows land before the stages are used again
        } else {
            // storer wavefront sw: rows 2 sw + i / 32 + 2 SW j, 16-byte chunk i % 32, of a group
            const int sw = wave - NLW;
            auto store = [&](int g) {
                const char* os = ostage(g);
                int t[RPL];
                u16x8 val[RPL];
#pragma unroll
                for (int j = 0; j < RPL; ++j) {
                    const int r = 2 * sw + h + 2 * SW * j;
                    t[j] = ids[g & 3][r];
                    val[j] = *reinterpret_cast<const u16x8*>(os + r * 512 + 16 * (l32 ^ (r & 31)));
                }
                // every LDS read issued before the first store (not one pair per store)
#pragma unroll
                for (int j = 0; j < RPL; ++j) asm volatile("" ::"v"(val[j]), "v"(t[j]));
#pragma unroll
                for (int j = 0; j < RPL; ++j)
                    if (t[j] >= 0) st8_nt(Out + (size_t)t[j] * H + n0 + 8 * l32, val[j]);
            };
            __syncthreads();
            compute(0, [](int) {});
            __syncthreads();
            // group g: the rows of g - 1 written two at a time between the MFMAs of g (read from
            // LDS SS batches before they are stored; volatile, so the reads stay where they are
            // and the waits for them go where the stores use them)
            constexpr int SS = NBT / RPL;
            static_assert(NBT % RPL == 0 && RPL % 2 == 0 && SS >= 1, "stores per batch");
#pragma unroll 1
            for (int g = 1; g < G; ++g) {
                const char* os = ostage(g - 1);
                int t[2];
                u16x8 val[2];
                compute(g, [&](int bt) {
                    if (bt % (2 * SS) == 0) {
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int r = 2 * sw + h + 2 * SW * (2 * (bt / (2 * SS)) + u);
                            t[u] = *(volatile const lds_int*)(&ids[(g - 1) & 3][r]);
                            val[u] = *(volatile const lds_u16x8*)(os + r * 512 + 16 * (l32 ^ (r & 31)));
                        }
                    }
                    if (bt % (2 * SS) == SS) {
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            if (t[u] >= 0) st8_nt(Out + (size_t)t[u] * H + n0 + 8 * l32, val[u]);
                    }
                });
                __syncthreads();
            }
            store(G - 1);
        }
        p = se;
    }
}

template <int H, bool DX, bool MEAN, bool ACC>
__global__ __launch_bounds__(wst_threads<ACC>()) __attribute__((amdgpu_waves_per_eu(
    wst_threads<ACC>() == 256 ? 1 : 2))) void k_rows_bf16_wst(const uint16_t* __restrict__ A,
                                                                const uint16_t* __restrict__ Wm,
                                                                const float* __restrict__ bias,
                                                                uint16_t* __restrict__ Out,
                                                                const int* __restrict__ offsets,
                                                                const int* __restrict__ perm, int NE, int T, int nh,
                                                                float inv_nh) {
    constexpr bool ROLES = MOE_BF16_WST_ROLES && !ACC;
    __shared__ __attribute__((aligned(16))) char smem[ROLES ? WsrSmem<H>::bytes : WstSmem<H>::bytes];
    if constexpr (ROLES)
        rows_bf16_wsr_body<H, DX, MEAN, MOE_BF16_WSR_WAVES>(smem, A, Wm, bias, Out, offsets, perm, NE, T, nh,
                                                            inv_nh);
    else
        rows_bf16_wst_body<H, DX, MEAN, ACC>(smem, A, Wm, bias, Out, offsets, perm, NE, T, nh, inv_nh);
}

// Kernels.  For H <= 128 the backward is one launch: dW / db chunk tiles first, then dX tiles.
// For H = 256 / 512 the 256 x 256 dW tiles take a whole compute unit each (their registers), so
// they run as a launch of their own ahead of the dX launch.
template <int H, int BN>
__global__ __launch_bounds__(kThreads) void k_fwd_bf16(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                        const float* __restrict__ bias, uint16_t* __restrict__ Y,
                                                        const int* __restrict__ offsets,
                                                        const int* __restrict__ perm, int NE, int T) {
    __shared__ __attribute__((aligned(16))) char smem[RowsBf16Smem<H, BN>::bytes];
    rows_bf16_body<H, BN, false>(smem, blockIdx.x, X, W, bias, Y, offsets, perm, NE, T, 0);
}

// ACC: dX is added to the existing contents (a compile-time choice, as in the fp32 kernels).
template <int H, int BN, bool MEAN, bool ACC>
__global__ __launch_bounds__(kThreads) void k_bwd_bf16(const uint16_t* __restrict__ dY,
                                                        const uint16_t* __restrict__ X,
                                                        const uint16_t* __restrict__ W, uint16_t* __restrict__ dX,
                                                        int accumulate, float* __restrict__ part_dw,
                                                        float* __restrict__ part_db,
                                                        const int* __restrict__ offsets,
                                                        const int* __restrict__ perm, int NE, int P, int T, int n_dx,
                                                        int nh, float inv_nh) {
    constexpr int BT = bf16_dw_tile(H);
    constexpr size_t r = RowsBf16Smem<H, BN>::bytes, d = DwBf16Smem<BT>::bytes;
    __shared__ __attribute__((aligned(16))) char smem[r > d ? r : d];  // one LDS region, either role
    // longest first: the dW workgroups (a whole chunk each) lead the grid, the dX tiles follow,
    // so the dispatcher evens out the end of the launch
    const int n_dw = (int)gridDim.x - n_dx;
    if ((int)blockIdx.x < n_dw)
        dw_bf16_body<H, BT, MEAN>(smem, blockIdx.x, dY, X, part_dw, part_db, offsets, perm, NE, P, T, nh, inv_nh);
    else
        rows_bf16_body<H, BN, true, MEAN>(smem, blockIdx.x - n_dw, dY, W, nullptr, dX, offsets, perm, NE, T,
                                          (int)ACC, nh, inv_nh);
}

#ifndef MOE_BF16_DW_RING
#define MOE_BF16_DW_RING 1  // slices in flight in the 256 x 256 d_W kernel (1, or an even ring)
#endif
constexpr int kDwBigThreads = 512;  // 256 x 256 d_W tile: 8 wavefronts of 128 x 64, two per SIMD
#ifndef MOE_BF16_DW_TR
#define MOE_BF16_DW_TR 1  // 256 x 256 d_W tiles staged token-major and read with transposing LDS reads
#endif
template <int H, bool MEAN>
__global__ __launch_bounds__(kDwBigThreads) void k_dw_bf16(const uint16_t* __restrict__ dY,
                                                          const uint16_t* __restrict__ X, float* __restrict__ part_dw,
                                                          float* __restrict__ part_db,
                                                          const int* __restrict__ offsets,
                                                          const int* __restrict__ perm, int NE, int P, int T, int nh,
                                                          float inv_nh) {
    constexpr int BT = bf16_dw_tile(H);
    if constexpr (MOE_BF16_DW_DMA) {
        static_assert(kDwBigThreads == 512 && BT == 256, "direct-to-LDS d_W tile shape");
        constexpr int R = MOE_BF16_DMA_STAGES;
        static_assert(R >= 3 && R <= 5, "stages of 32 KB within the LDS");
        __shared__ __attribute__((aligned(16))) char s0[DwdSmem::stage];
        __shared__ __attribute__((aligned(16))) char s1[DwdSmem::stage];
        __shared__ __attribute__((aligned(16))) char s2[R > 2 ? DwdSmem::stage : 16];
        __shared__ __attribute__((aligned(16))) char s3[R > 3 ? DwdSmem::stage : 16];
        __shared__ __attribute__((aligned(16))) char s4[R > 4 ? DwdSmem::stage : 16];
        char* const all[5] = {s0, s1, s2, s3, s4};
        char* st[R];
#pragma unroll
        for (int k = 0; k < R; ++k) st[k] = all[k];
        dw_bf16_dma_body<H, MEAN, R>(st, blockIdx.x, dY, X, part_dw, part_db, offsets, perm, NE, P, T, nh, inv_nh);
    } else if constexpr (MOE_BF16_DW_TR) {
        static_assert(kDwtThreads == kDwBigThreads && BT == 256, "token-major d_W tile shape");
        __shared__ __attribute__((aligned(16))) char smem[DwtSmem::bytes];
        dw_bf16_tr_body<H, MEAN>(smem, blockIdx.x, dY, X, part_dw, part_db, offsets, perm, NE, P, T, nh, inv_nh);
    } else {
        __shared__ __attribute__((aligned(16))) char smem[DwBf16Smem<BT>::bytes];
        dw_bf16_body<H, BT, MEAN, MOE_BF16_DW_RING, kDwBigThreads>(smem, blockIdx.x, dY, X, part_dw, part_db,
                                                                   offsets, perm, NE, P, T, nh, inv_nh);
    }
}

template <int H, int BN, bool MEAN, bool ACC>
__global__ __launch_bounds__(kThreads) void k_dx_bf16(const uint16_t* __restrict__ dY, const uint16_t* __restrict__ W,
                                                       uint16_t* __restrict__ dX, int accumulate,
                                                       const int* __restrict__ offsets,
                                                       const int* __restrict__ perm, int NE, int T, int nh,
                                                       float inv_nh) {
    __shared__ __attribute__((aligned(16))) char smem[RowsBf16Smem<H, BN>::bytes];
    rows_bf16_body<H, BN, true, MEAN>(smem, blockIdx.x, dY, W, nullptr, dX, offsets, perm, NE, T, (int)ACC, nh,
                                      inv_nh);
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
        if (bf16_wst(T, H)) {
            launch_kernel((k_rows_bf16_wst<H, false, false, false>), dim3(kWstWgs), dim3(wst_threads<false>()), 0, s,
                          X, W,
                          bias, Y, offsets, perm, NE, (int)T, 1, 1.0f);
            return hipGetLastError();
        }
        if (MOE_BF16_WS_FWD && T * H * 2 < ((int64_t)1 << 31)) {
            launch_kernel((k_fwd_bf16_ws<H>), dim3(kWsWgs), dim3(kWsThreads), 0, s, X, W, bias, Y, offsets, perm, NE,
                          (int)T);
            return hipGetLastError();
        }
    }
    constexpr int BN = (H >= 128) ? 128 : H;
    constexpr int NT = H / BN;
    const int grid = round_up((int)((T + 127) / 128) + NE, 8) * NT;
    launch_kernel((k_fwd_bf16<H, BN>), dim3(grid), dim3(kThreads), 0, s, X, W, bias, Y, offsets, perm, NE, (int)T);
    return hipGetLastError();
}

template <int H, bool MEAN, bool ACC>
static hipError_t bwd_bf16(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX, int accumulate,
                           float* pdw, float* pdb, const int32_t* offsets, const int32_t* perm, int64_t T, int NE,
                           int P, int n_chunk_max, int nh, hipStream_t s) {
    constexpr int BN = (H >= 128) ? 128 : H;
    constexpr int NT = H / BN;
    constexpr int BT = bf16_dw_tile(H);
    constexpr int TPC = (H / BT) * (H / BT);
    const float inv_nh = 1.0f / (float)nh;
    const int n_dx = round_up((int)((T + 127) / 128) + NE, 8) * NT;
    const int n_dw = round_up(n_chunk_max, 8) * TPC;
    if constexpr (BT == 256) {
        // the kernel timer (if armed) brackets both launches
        const ArmedEvents ev = take_armed_events();
        launch_kernel_ev((k_dw_bf16<H, MEAN>), dim3(n_dw), dim3(kDwBigThreads), 0, s, ev.start, nullptr, dY, X, pdw, pdb,
                         offsets, perm, NE, P, (int)T, nh, inv_nh);
        if (bf16_wst(T, H)) {
            launch_kernel_ev((k_rows_bf16_wst<H, true, MEAN, ACC>), dim3(kWstWgs), dim3(wst_threads<ACC>()), 0, s,
                             nullptr,
                             ev.stop, dY, W, nullptr, dX, offsets, perm, NE, (int)T, nh, inv_nh);
        } else {
            launch_kernel_ev((k_dx_bf16<H, BN, MEAN, ACC>), dim3(n_dx), dim3(kThreads), 0, s, nullptr, ev.stop, dY, W,
                             dX, accumulate, offsets, perm, NE, (int)T, nh, inv_nh);
        }
    } else {
        launch_kernel((k_bwd_bf16<H, BN, MEAN, ACC>), dim3(n_dx + n_dw), dim3(kThreads), 0, s, dY, X, W, dX, accumulate,
                      pdw, pdb, offsets, perm, NE, P, (int)T, n_dx, nh, inv_nh);
    }
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

template <bool MEAN, bool ACC>
static hipError_t bwd_bf16_h2(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX, float* pdw,
                              float* pdb, const int32_t* offsets, const int32_t* perm, int64_t T, int H, int NE, int P,
                              int n_chunk_max, int nh, hipStream_t s) {
    const int acc = ACC ? 1 : 0;
    switch (H) {
        case 64: return bwd_bf16<64, MEAN, ACC>(dY, X, W, dX, acc, pdw, pdb, offsets, perm, T, NE, P, n_chunk_max, nh, s);
        case 128:
            return bwd_bf16<128, MEAN, ACC>(dY, X, W, dX, acc, pdw, pdb, offsets, perm, T, NE, P, n_chunk_max, nh, s);
        case 256:
            return bwd_bf16<256, MEAN, ACC>(dY, X, W, dX, acc, pdw, pdb, offsets, perm, T, NE, P, n_chunk_max, nh, s);
        case 512:
            return bwd_bf16<512, MEAN, ACC>(dY, X, W, dX, acc, pdw, pdb, offsets, perm, T, NE, P, n_chunk_max, nh, s);
    }
    return hipErrorInvalidValue;
}

template <bool MEAN>
static hipError_t bwd_bf16_h(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX, int accumulate,
                             float* pdw, float* pdb, const int32_t* offsets, const int32_t* perm, int64_t T, int H,
                             int NE, int P, int n_chunk_max, int nh, hipStream_t s) {
    if (accumulate)
        return bwd_bf16_h2<MEAN, true>(dY, X, W, dX, pdw, pdb, offsets, perm, T, H, NE, P, n_chunk_max, nh, s);
    return bwd_bf16_h2<MEAN, false>(dY, X, W, dX, pdw, pdb, offsets, perm, T, H, NE, P, n_chunk_max, nh, s);
}

hipError_t launch_bwd_gemm_bf16(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX,
                                int accumulate, float* pdw, float* pdb, const int32_t* offsets, const int32_t* perm,
                                int64_t T, int H, int NE, int P, int n_chunk_max, hipStream_t s) {
    return bwd_bf16_h<false>(dY, X, W, dX, accumulate, pdw, pdb, offsets, perm, T, H, NE, P, n_chunk_max, 1, s);
}

hipError_t launch_bwd_gemm_bf16_from_mean(const uint16_t* d_mean, const uint16_t* X, const uint16_t* W, uint16_t* dX,
                                          int accumulate, float* pdw, float* pdb, const int32_t* offsets,
                                          const int32_t* perm, int64_t T, int H, int NE, int NH, int P,
                                          int n_chunk_max, hipStream_t s) {
    return bwd_bf16_h<true>(d_mean, X, W, dX, accumulate, pdw, pdb, offsets, perm, T, H, NE, P, n_chunk_max, NH, s);
}

}  // namespace moe
