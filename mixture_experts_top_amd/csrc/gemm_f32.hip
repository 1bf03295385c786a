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
#include "aux_math.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;   // 4 waves, arranged 2 x 2 over the output tile
// K slice staged per LDS buffer (a multiple of 8), per kernel; chosen by measurement.
#ifndef MOE_F32_KC_FWD
#define MOE_F32_KC_FWD 32
#endif
// the small-T forward's one-tile workgroups (one K slice in flight while the previous
// computes): 16-wide slices measured 0.2 us faster than 32 at the pages' shape
#ifndef MOE_F32_KC_FWD_SMALL
#define MOE_F32_KC_FWD_SMALL 16
#endif
#ifndef MOE_F32_KC_DX
#define MOE_F32_KC_DX 16
#endif
#ifndef MOE_F32_KC_DW
#define MOE_F32_KC_DW 16
#endif
constexpr int kPad = 4;         // LDS row padding (floats) for K-contiguous tiles: 16-byte aligned rows
#ifndef MOE_F32_PAD_KN
#define MOE_F32_PAD_KN 8
#endif
// Padding of tiles stored [k][n] and read one float per lane, lanes 32..63 four rows below
// lanes 0..31: a row stride of 8 (mod 64) floats puts the two halves on disjoint LDS banks.
constexpr int kPadKN = MOE_F32_PAD_KN;

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
// Non-temporal stores (the write does not allocate in the cache hierarchy as reusable data),
// for the GEMM outputs, which no workgroup of the same launch reads back.  Measured against
// plain stores: pages-shape step 42.7 -> 41.4 us, imbalanced 117.8 -> 115.4 us, large stress
// 3418 -> 3409 us.  Not for the d_W partials, which the reduce reads back next (the
// imbalanced-shape backward was 1.7 us slower).
__device__ __forceinline__ void st4_nt(float* p, f32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p)); }
__device__ __forceinline__ void st1_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }

// Workgroup ids are dealt to the 8 XCDs round-robin.  The `per` tiles that share one
// operand block get ids id, id+8, id+16, ... so they land on the same XCD (same L2).
__device__ __forceinline__ void xcd_split(int bid, int per, int& major, int& minor) {
    const int grp = bid / (8 * per), loc = bid % (8 * per);
    major = grp * 8 + loc % 8;
    minor = loc / 8;
}

// Token ids of the 16 rows a lane stores from a 32x32 accumulator block: row
// 8 (r / 4) + 4 h + (r % 4) of the block, r = 0..15, read from the tile's id list in LDS
// (tr points at the block's row 4 h) as four 16-byte reads with a single wait, so the
// stores that follow do not each wait on an LDS read.
__device__ __forceinline__ void block_row_ids(const int* tr, int (&tk)[16]) {
    int4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const int4*>(tr + 8 * q);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        tk[4 * q] = v[q].x; tk[4 * q + 1] = v[q].y; tk[4 * q + 2] = v[q].z; tk[4 * q + 3] = v[q].w;
    }
}

// Stores one 32x32 accumulator block: its row 8 (r / 4) + 4 h + (r % 4) goes to token
// tok_of(r) (negative: a padded row, not stored), column `col`.  No load may be pending
// when the conditional stores run: a wait inside them would also wait for every store
// issued before it.  With `prior` the output's current value is added (gradient
// accumulation): four rows' loads go out before their stores (a padded row reads row 0
// and drops it), so the block waits for memory four times, not sixteen.  Reading the ids
// one by one (tok_of from LDS) keeps registers free where they bound occupancy; where
// they do not, store_block_ids takes the ids from registers.
template <class TokOf>
__device__ __forceinline__ void store_block(float* __restrict__ Out, int H, int col, const f32x16& a, float bv,
                                            bool prior, TokOf tok_of) {
    if (prior) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int tk[4];
            float old[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                tk[u] = tok_of(4 * q + u);
                old[u] = Out[(size_t)(tk[u] < 0 ? 0 : tk[u]) * H + col];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (tk[u] >= 0) st1_nt(&Out[(size_t)tk[u] * H + col], old[u] + (a[4 * q + u] + bv));
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = tok_of(r);
            if (t >= 0) st1_nt(&Out[(size_t)t * H + col], a[r] + bv);
        }
    }
}

// store_block with the 16 ids already in registers (block_row_ids): the stores do not
// each wait on an LDS read.
__device__ __forceinline__ void store_block_ids(float* __restrict__ Out, int H, int col, const f32x16& a, float bv,
                                                bool prior, const int (&tk)[16]) {
    if (prior) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float old[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) old[u] = Out[(size_t)(tk[4 * q + u] < 0 ? 0 : tk[4 * q + u]) * H + col];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (tk[4 * q + u] >= 0) st1_nt(&Out[(size_t)tk[4 * q + u] * H + col], old[u] + (a[4 * q + u] + bv));
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (tk[r] >= 0) st1_nt(&Out[(size_t)tk[r] * H + col], a[r] + bv);
    }
}

// Like xcd_split with `per` N-tiles per row tile, but with R consecutive row tiles on one
// XCD: row tile mt runs on XCD (mt / R) % 8.  The dX tiles of the small-T backward use it
// with R = (tokens per dW chunk) / BM, so a dX tile and the dW chunk over the same rows of dY
// (chunk c runs on XCD c % 8) read them through the same L2.  Covers every row tile below
// the grid's count when that count is a multiple of 8 R.
__device__ __forceinline__ void xcd_rows(int bid, int per, int R, int& major, int& minor) {
    const int x = bid % 8, sl = bid / 8;
    minor = sl % per;
    const int r = (sl / per) % R, q = sl / (per * R);
    major = R * (8 * q + x) + r;
}

}  // namespace

// ----------------------------------------------------------------------------------
// Row GEMM: Out[t, n0:n0+BN] = A[t, :] . B[:, n0:n0+BN] (+ bias) for the BM rows of one
// expert tile.  DX = false: B[k][n] = W[e][n][k] (forward).  DX = true: B[k][n] = W[e][k][n].
// K is walked in 32-wide slices with two LDS buffers: the global loads of slice c+1 are
// issued into registers before the MFMAs of slice c, and stored to the other buffer after
// them, so one barrier per slice suffices and load latency hides behind the MFMAs.
// ----------------------------------------------------------------------------------
#ifndef MOE_ONEPASS_STAGED_STORES
#define MOE_ONEPASS_STAGED_STORES 1  // one-tile workgroups store their tile through LDS, whole rows
#endif
template <int BM, int BN, int KC, bool DX>
struct RowsF32Smem {
    static constexpr int BS_ROWS = DX ? KC : BN, BS_COLS = DX ? BN + kPadKN : KC + kPad;
    static constexpr size_t a = sizeof(float) * 2 * BM * (KC + kPad), b = sizeof(float) * 2 * BS_ROWS * BS_COLS;
    // the output tile staged row-major (the one-tile epilogue), over the K-slice buffers
    static constexpr size_t stage = MOE_ONEPASS_STAGED_STORES ? sizeof(float) * BM * (BN + kPadKN) : 0;
    static constexpr size_t tok_off = a + b > stage ? a + b : stage;
    static constexpr size_t bytes = tok_off + 2 * 4 * BM;  // + token ids of the current and the next tile
};

// Persistent: workgroup `wg` of `nwg` computes tiles wg, wg + nwg, ... of the `ntile_ids` tile
// ids (ids past the real tile count are skipped).  The experts' offsets are read once per
// wavefront; during the last K-slice of a tile the next tile's token ids and first K-slice are
// loaded, so that latency overlaps the MFMAs and the epilogue stores.
// WNK: the B tile is read [n][k] (k contiguous), as the forward reads W[e][out][in]; dX passes
// W as stored ([k][n], WNK = false) or its transpose (WNK = true, then read like the forward).
template <int H, int BM, int BN, int KC, bool DX, bool MEAN = false, bool WNK = !DX>
__device__ __forceinline__ void rows_f32_body(char* smem, int wg, int nwg, int ntile_ids,
                                              const float* __restrict__ A, const float* __restrict__ W,
                                              const float* __restrict__ bias, float* __restrict__ Out,
                                              const int* __restrict__ offsets, const int* __restrict__ perm,
                                              int NE, int T, int accumulate, int nh = 1, float inv_nh = 1.0f) {
    // MEAN: row t of A is A[t / nh] * inv_nh (the backward of a mean over nh horizons)
    constexpr int NKC = H / KC;
    constexpr int NT = H / BN;
    constexpr int WM = (BM >= 64) ? 2 : 1, WN = 4 / WM;  // wavefront grid over the tile
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int SM = WTM / 32, SN = WTN / 32;
    static_assert(SM >= 1 && SN >= 1, "wavefront tile must hold a 32x32 block");
    constexpr int TPR = KC / 4, RPP = kThreads / TPR;   // threads per row slice, rows per pass
    // float4 loads per thread per slice; with BM < RPP only the first BM row-threads load A
    constexpr int AL = (BM + RPP - 1) / RPP, BL = BN * KC / (4 * kThreads);
    constexpr bool AFULL = BM % RPP == 0;
    static_assert(KC % 8 == 0 && (AFULL || RPP % BM == 0) && (BN * KC) % (4 * kThreads) == 0, "tile shape");
    constexpr int BS_ROWS = !WNK ? KC : BN;
    constexpr int BS_COLS = !WNK ? BN + kPadKN : KC + kPad;
    using SM_ = RowsF32Smem<BM, BN, KC, !WNK>;
    float(&As)[2][BM][KC + kPad] = *reinterpret_cast<float(*)[2][BM][KC + kPad]>(smem);
    float(&Bs)[2][BS_ROWS][BS_COLS] = *reinterpret_cast<float(*)[2][BS_ROWS][BS_COLS]>(smem + SM_::a);
    int(&tok)[2][BM] = *reinterpret_cast<int(*)[2][BM]>(smem + SM_::tok_off);

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wm = wave / WN, wn = wave % WN;

    // expert table: lane l < NE holds expert l's first row, row count and tile count
    int x_lo, x_cnt;
    expert_range(offsets, NE, T, x_lo, x_cnt);
    const int x_n = (x_cnt + BM - 1) / BM;
    const int x_incl = wave_inclusive_sum(x_n), x_excl = x_incl - x_n;
    auto lookup = [&](int id, int& e, int& r0, int& rows, int& n0) -> bool {
        int mt, nt;
        xcd_split(id, NT, mt, nt);
        const uint64_t hit = __ballot(lane < NE && mt >= x_excl && mt < x_incl);
        if (hit == 0) return false;
        const int le = __ffsll((unsigned long long)hit) - 1;
        const int j = mt - __builtin_amdgcn_readlane(x_excl, le);
        e = le;
        r0 = __builtin_amdgcn_readlane(x_lo, le) + j * BM;
        rows = min(BM, __builtin_amdgcn_readlane(x_cnt, le) - j * BM);
        n0 = nt * BN;
        return true;
    };
    auto next_valid = [&](int id, int& e, int& r0, int& rows, int& n0) -> int {
        for (; id < ntile_ids; id += nwg)
            if (lookup(id, e, r0, rows, n0)) return id;
        return -1;
    };

    int e, r0, rows, n0;
    int id = next_valid(wg, e, r0, rows, n0);
    if (id < 0) return;
    int cur = 0;
    if (tid < BM) tok[cur][tid] = (tid < rows) ? load_token(perm, r0 + tid, T) : -1;
    __syncthreads();

    const float* __restrict__ We = W + (size_t)e * H * H;
    int wn0 = n0;  // column offset the W loads use (switches to the next tile during its prefetch)
    const float* a_src[AL];
    auto set_a_src = [&](const int* t_of_row) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int t = t_of_row[i];
            const int row = MEAN ? t / nh : t;
            a_src[i] = (t >= 0) ? A + (size_t)row * H + 4 * (tid % TPR) : nullptr;
        }
    };
    {
        int t0[AL];
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int row = tid / TPR + RPP * i;
            t0[i] = (AFULL || row < BM) ? tok[cur][row] : -1;
        }
        set_a_src(t0);
    }
    f32x4 ra[AL], rb[BL];
    auto load_slice = [&](int k0) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            ra[i] = a_src[i] ? ld4(a_src[i] + k0) : f32x4{};
            if (MEAN) ra[i] *= inv_nh;
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            if (WNK) {
                const int r = tid / TPR + RPP * i, c = 4 * (tid % TPR);
                rb[i] = ld4(We + (size_t)(wn0 + r) * H + k0 + c);
            } else {
                const int q = tid + kThreads * i, r = q / (BN / 4), c = 4 * (q % (BN / 4));
                rb[i] = ld4(We + (size_t)(k0 + r) * H + wn0 + c);
            }
        }
    };
    auto store_slice = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int row = tid / TPR + RPP * i;
            if (AFULL || row < BM) st4(&As[buf][row][4 * (tid % TPR)], ra[i]);
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            if (WNK) {
                st4(&Bs[buf][tid / TPR + RPP * i][4 * (tid % TPR)], rb[i]);
            } else {
                const int q = tid + kThreads * i;
                st4(&Bs[buf][q / (BN / 4)][4 * (q % (BN / 4))], rb[i]);
            }
        }
    };

    f32x16 acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = f32x16{};

    // LDS fragments of one 8-k group, double-buffered in registers: the reads of group g+1
    // are issued before the MFMAs of group g.
    constexpr int NG = KC / 8;
    f32x4 fa[2][SM], fb[2][SN];
    auto load_frag = [&](int buf, int g, int slot) {
        const int kk = 8 * g + 4 * h;
#pragma unroll
        for (int i = 0; i < SM; ++i) fa[slot][i] = ld4(&As[buf][wm * WTM + i * 32 + l32][kk]);
#pragma unroll
        for (int j = 0; j < SN; ++j) {
            if (WNK) {
                fb[slot][j] = ld4(&Bs[buf][wn * WTN + j * 32 + l32][kk]);
            } else {
                const int cc = wn * WTN + j * 32 + l32;
                fb[slot][j] = f32x4{Bs[buf][kk + 0][cc], Bs[buf][kk + 1][cc], Bs[buf][kk + 2][cc], Bs[buf][kk + 3][cc]};
            }
        }
    };
    auto compute = [&](int buf) {
        load_frag(buf, 0, 0);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g + 1 < NG) load_frag(buf, g + 1, (g + 1) & 1);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < SM; ++i)
#pragma unroll
                    for (int j = 0; j < SN; ++j) acc[i][j] = mfma32(fa[g & 1][i][s], fb[g & 1][j][s], acc[i][j]);
        }
    };

    float bv_cur[SN], bv_next[SN];
#pragma unroll
    for (int j = 0; j < SN; ++j) {
        bv_cur[j] = DX ? 0.0f : bias[(size_t)e * H + n0 + wn * WTN + j * 32 + l32];
        bv_next[j] = 0.0f;
    }
    load_slice(0);
    store_slice(0);
    __syncthreads();
    int gs = 0;  // slices done by this workgroup (LDS buffer parity)
#pragma unroll 1
    for (;;) {
        int e2 = 0, r02 = 0, rows2 = 0, n02 = 0;
        const int nid = next_valid(id + nwg, e2, r02, rows2, n02);
        const bool has_next = nid >= 0;
        // token ids of the next tile: for its epilogue (LDS) and its gathered rows
        int tok_next = -1, tn[AL];
#pragma unroll
        for (int i = 0; i < AL; ++i) tn[i] = -1;
        if (has_next) {
            if (!DX) {
#pragma unroll
                for (int j = 0; j < SN; ++j) bv_next[j] = bias[(size_t)e2 * H + n02 + wn * WTN + j * 32 + l32];
            }
            if (tid < BM && tid < rows2) tok_next = load_token(perm, r02 + tid, T);
#pragma unroll
            for (int i = 0; i < AL; ++i) {
                const int row = tid / TPR + RPP * i;
                if (row < rows2) tn[i] = load_token(perm, r02 + row, T);
            }
        }
#pragma unroll 1
        for (int c = 0; c < NKC; ++c, ++gs) {
            const int buf = gs & 1;
            if (c + 1 < NKC) {
                load_slice((c + 1) * KC);
            } else if (has_next) {
                set_a_src(tn);
                We = W + (size_t)e2 * H * H;
                wn0 = n02;
                load_slice(0);
            }
            compute(buf);
            if (c + 1 < NKC || has_next) store_slice(buf ^ 1);
            __syncthreads();
        }

        // epilogue of this tile (its n0, bias and token ids; the bias was loaded a tile ahead,
        // so no load is pending in the stores)
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            const int* tr = &tok[cur][wm * WTM + i * 32 + 4 * h];
#pragma unroll
            for (int j = 0; j < SN; ++j) {
                store_block(Out, H, n0 + wn * WTN + j * 32 + l32, acc[i][j], bv_cur[j], DX && accumulate,
                            [&](int r) { return tr[8 * (r / 4) + (r % 4)]; });
                acc[i][j] = f32x16{};
            }
        }
        if (!has_next) break;
        if (tid < BM) tok[cur ^ 1][tid] = tok_next;  // read in the next epilogue, after its barriers
#pragma unroll
        for (int j = 0; j < SN; ++j) bv_cur[j] = bv_next[j];
        cur ^= 1;
        id = nid;
        e = e2;
        r0 = r02;
        rows = rows2;
        n0 = n02;
    }
}

// One tile per workgroup, with a ring of PF K-slices in registers: while slice c computes,
// the global loads of the next PF slices are outstanding (PF from MOE_ONEPASS_RING_F4: one
// slice by default), so a tile waits on about three memory round trips (offsets, perm,
// first operands) before its K loop.  Used when the grid has no more tiles than resident
// workgroups, where a tile's latency is the kernel's time.
// Routing outputs, for a forward that forms its tiles' token ids itself (and writes perm,
// counts and offsets) instead of reading the scatter's perm: the expert of every token and
// the per-routing-block expert histogram (256 tokens per block).
struct RouteView {
    const int* idx;
    const int* hist;
    int nblk, T;
    int* counts;
    int* offsets;
    int* perm;
};

// Loads the routing histogram hist[nblk][N_E] (at most 4096 entries) into hs and sums its
// columns into tot (256 ints): afterwards tot[e] holds expert e's token count, e < N_E.
// Integer sums, exact in any order.  Contains barriers: every thread calls it.
// Thread (ec, sg) = (tid % nep, tid / nep) sums blocks sg, sg + S, ... of column ec (nep = N_E
// rounded up to a power of two, S = 256 / nep); the S segment sums of a column are then added
// inside each 16-lane row through DPP rotations (nep <= 8) and across rows through LDS, so the
// whole reduction costs two barriers.
__device__ __forceinline__ void hist_counts_lds(int* hs, int* tot, const int* __restrict__ hist, int nblk, int NE) {
    const int tid = threadIdx.x;
    const int nhist = nblk * NE;
    // every load of a thread out before the first wait (one round trip, not one per entry)
    constexpr int MAXU = 4096 / kThreads;
    const int per = (nhist + kThreads - 1) / kThreads;
    int hv[MAXU];
#pragma unroll
    for (int u = 0; u < MAXU; ++u)
        if (u < per) {
            const int i = tid + kThreads * u;
            hv[u] = hist[i < nhist ? i : nhist - 1];
        }
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        const int i = tid + kThreads * u;
        if (u < per && i < nhist) hs[i] = hv[u];
    }
    int nep = 1;
    while (nep < NE) nep <<= 1;
    const int S = kThreads / nep;
    const int ec = tid % nep, sg = tid / nep;
    int sum = 0;
    if (nep == NE) {
        // entry tid + 256 u is block sg + S u of column ec: this thread's own loads
#pragma unroll
        for (int u = 0; u < MAXU; ++u)
            if (u < per && tid + kThreads * u < nhist) sum += hv[u];
    } else {
        __syncthreads();
        if (ec < NE)
            for (int x = sg; x < nblk; x += S) sum += hs[x * NE + ec];
    }
    // partial sums of column ec: with nep <= 8 the lanes of a row that share ec are summed in
    // registers (rotations keep lane % nep), one value per (row, ec) goes to LDS
    if (nep <= 8) {
        if (nep == 1) sum += dpp_move<0xB1>(sum, 0);
        if (nep <= 2) sum += dpp_move<0x4E>(sum, 0);
        if (nep <= 4) sum += dpp_move<0x124>(sum, 0);
        sum += dpp_move<0x128>(sum, 0);
    }
    // nep <= 8: 16 rows x nep entries at tot[128 ..]; else S entries per column over tot[0 .. 255]
    const bool small = nep <= 8;
    int* red = small ? tot + 128 : tot;
    if (!small || (tid % 16) < nep) red[small ? (tid / 16) * nep + ec : tid] = sum;
    __syncthreads();
    const int nparts = small ? 16 : S;
    int cnt = 0;
    if (tid < NE)
        for (int q = 0; q < nparts; ++q) cnt += red[q * nep + tid];
    if (!small) __syncthreads();  // red overlaps tot[0 .. N_E)
    if (tid < NE) tot[tid] = cnt;
    __syncthreads();
}

// float4 registers per thread for the one-pass slice ring.  4 (one K slice in flight while
// the previous one computes) against 12 (three or four, all of K at H = 128): pages-shape step
// 39.3 -> 38.6 us, and 6 / 8 / 10 in between; every workgroup of these grids starts at once,
// so deeper rings only lengthen the first burst of loads that all of them wait behind.
#ifndef MOE_ONEPASS_RING_F4
#define MOE_ONEPASS_RING_F4 4
#endif
template <int H, int BM, int BN, int KC, bool DX, bool MEAN = false, int XR = 1, bool GATHER = false>
__device__ __forceinline__ void rows_f32_onepass_body(char* smem, int bid, const float* __restrict__ A,
                                                      const float* __restrict__ W, const float* __restrict__ bias,
                                                      float* __restrict__ Out, const int* __restrict__ offsets,
                                                      const int* __restrict__ perm, int NE, int T, int accumulate,
                                                      int nh = 1, float inv_nh = 1.0f, RouteView rv = {}) {
    constexpr int NKC = H / KC;
    constexpr int NT = H / BN;
    constexpr int WM = (BM >= 64) ? 2 : 1, WN = 4 / WM;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int SM = WTM / 32, SN = WTN / 32;
    static_assert(SM >= 1 && SN >= 1, "wavefront tile must hold a 32x32 block");
    constexpr int TPR = KC / 4, RPP = kThreads / TPR;
    constexpr int AL = (BM + RPP - 1) / RPP, BL = BN * KC / (4 * kThreads);
    constexpr bool AFULL = BM % RPP == 0;  // else only the first BM row-threads load A
    static_assert(KC % 8 == 0 && (AFULL || RPP % BM == 0) && (BN * KC) % (4 * kThreads) == 0, "tile shape");
    constexpr int PF0 = MOE_ONEPASS_RING_F4 / (AL + BL);  // float4 registers of slices in flight
    constexpr int PF = PF0 < 1 ? 1 : (PF0 > NKC ? NKC : PF0);
    constexpr int BS_ROWS = DX ? KC : BN;
    constexpr int BS_COLS = DX ? BN + kPadKN : KC + kPad;
    using SM_ = RowsF32Smem<BM, BN, KC, DX>;
    float(&As)[2][BM][KC + kPad] = *reinterpret_cast<float(*)[2][BM][KC + kPad]>(smem);
    float(&Bs)[2][BS_ROWS][BS_COLS] = *reinterpret_cast<float(*)[2][BS_ROWS][BS_COLS]>(smem + SM_::a);
    int(&tok)[2][BM] = *reinterpret_cast<int(*)[2][BM]>(smem + SM_::tok_off);

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wm = wave / WN, wn = wave % WN;

    int mt, nt, e, r0, r1;
    if (XR == 1)
        xcd_split(bid, NT, mt, nt);
    else
        xcd_rows(bid, NT, XR, mt, nt);
    int lo = 0;  // GATHER: the tile's first rank within its expert
    if constexpr (!GATHER) {
        if (!find_tile(offsets, NE, T, mt, BM, e, r0, r1)) return;
    } else {
        // The routing histogram (at most 4096 entries) goes to LDS, over the region the K
        // slices use later; its column sums give every expert's count, hence the tile list.
        static_assert(SM_::a + SM_::b >= sizeof(int) * (4096 + 256 + 8), "LDS for the histogram");
        int* hs = reinterpret_cast<int*>(smem);
        int* part = hs + 4096;
        if (tid < BM) tok[0][tid] = -1;
        hist_counts_lds(hs, part, rv.hist, rv.nblk, NE);
        const int cnt_l = (lane < NE) ? part[lane] : 0;
        const int off_l = wave_inclusive_sum(cnt_l) - cnt_l;
        const int nt_l = (cnt_l + BM - 1) / BM;
        const int tincl = wave_inclusive_sum(nt_l), texcl = tincl - nt_l;
        if (bid == 0 && wave == 0 && lane < NE) {
            rv.counts[lane] = cnt_l;
            rv.offsets[lane] = off_l;
            if (lane == NE - 1) rv.offsets[NE] = off_l + cnt_l;
        }
        const uint64_t hit = __ballot(lane < NE && mt >= texcl && mt < tincl);
        if (hit == 0) return;  // the same for every wavefront of the workgroup
        e = __ffsll((unsigned long long)hit) - 1;
        lo = (mt - __builtin_amdgcn_readlane(texcl, e)) * BM;
        r0 = __builtin_amdgcn_readlane(off_l, e) + lo;
        r1 = r0 + min(BM, __builtin_amdgcn_readlane(cnt_l, e) - lo);
    }
    const int rows = r1 - r0, n0 = nt * BN;
    const float* __restrict__ We = W + (size_t)e * H * H;

    // token ids: of this thread's A rows (registers) and of the tile's rows (LDS, epilogue)
    int ta[AL];
    int tok_mine = -1;
    if constexpr (!GATHER) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int row = tid / TPR + RPP * i;
            ta[i] = (row < rows) ? load_token(perm, r0 + row, T) : -1;
        }
        tok_mine = (tid < BM && tid < rows) ? load_token(perm, r0 + tid, T) : -1;  // to LDS once the loads are out
    }

    f32x4 ra[PF][AL], rb[PF][BL];
    auto load_b = [&](int c, int slot) {
        const int k0 = c * KC;
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            if (!DX) {
                const int r = tid / TPR + RPP * i, cc = 4 * (tid % TPR);
                rb[slot][i] = ld4(We + (size_t)(n0 + r) * H + k0 + cc);
            } else {
                const int q = tid + kThreads * i, r = q / (BN / 4), cc = 4 * (q % (BN / 4));
                rb[slot][i] = ld4(We + (size_t)(k0 + r) * H + n0 + cc);
            }
        }
    };
    const float* a_src[AL];
    auto load_a = [&](int c, int slot) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            ra[slot][i] = ld4(a_src[i] + c * KC);
            if (MEAN) ra[slot][i] *= inv_nh;
        }
    };
    auto store_slice = [&](int slot, int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int row = tid / TPR + RPP * i;
            if (AFULL || row < BM) st4(&As[buf][row][4 * (tid % TPR)], ra[slot][i]);
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            if (!DX) {
                st4(&Bs[buf][tid / TPR + RPP * i][4 * (tid % TPR)], rb[slot][i]);
            } else {
                const int q = tid + kThreads * i;
                st4(&Bs[buf][q / (BN / 4)][4 * (q % (BN / 4))], rb[slot][i]);
            }
        }
    };

    // W does not depend on perm: its loads go out while the token ids are in flight (loads
    // return in issue order, so the ids arrive first).  The fences keep the compiler from
    // sinking loads next to their first use.
    float bv[SN];  // complete before the stores (the K loop waits for every load), see below
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < SN; ++j) bv[j] = DX ? 0.0f : bias[(size_t)e * H + n0 + wn * WTN + j * 32 + l32];
#pragma unroll
    for (int c = 0; c < PF; ++c) load_b(c, c);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (GATHER) {
        // The tile's token ids, while W is in flight: ranks lo .. lo + rows - 1 of expert e, in
        // token order.  Expert e's tokens before routing block x number sum_{x' < x} hist[x'][e];
        // inside a block, ballots over the 4 wavefronts (64 tokens each) rank them in order --
        // the same stable counting sort the scatter kernels perform, so perm is identical.
        static_assert(kRouteTokens == kThreads, "one routing block per workgroup pass");
        int* hs = reinterpret_cast<int*>(smem);
        int* wsc = hs + 4096 + 256;  // per-wave scratch and the found block range
        const int hi = lo + rows;    // ranks [lo, hi)
        {
            const int per = (rv.nblk + kThreads - 1) / kThreads;
            const int x0 = min(tid * per, rv.nblk), x1 = min(x0 + per, rv.nblk);
            int sl = 0;
            for (int x = x0; x < x1; ++x) sl += hs[x * NE + e];
            const int wincl = wave_inclusive_sum(sl);
            if (lane == 63) wsc[wave] = wincl;
            __syncthreads();
            int p = wincl - sl;
            for (int w = 0; w < wave; ++w) p += wsc[w];
            for (int x = x0; x < x1; ++x) {
                const int v = hs[x * NE + e];
                if (p <= lo && lo < p + v) {
                    wsc[4] = x;
                    wsc[5] = p;
                }
                if (p <= hi - 1 && hi - 1 < p + v) wsc[6] = x;
                p += v;
            }
            __syncthreads();
        }
        const int b0 = wsc[4], b1 = wsc[6];
        int pre = wsc[5];
        __syncthreads();  // wsc[0..3] are reused below
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int xb = b0; xb <= b1; xb += 4) {  // the experts of up to 4 blocks in one round trip
            int ex[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = (xb + u) * kRouteTokens + tid;
                ex[u] = (xb + u <= b1 && t < rv.T) ? rv.idx[t] : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (xb + u > b1) break;  // uniform
                const int t = (xb + u) * kRouteTokens + tid;
                const uint64_t m = __ballot(ex[u] == e);
                if (lane == 0) wsc[wave] = __popcll(m);
                __syncthreads();
                int g = pre;
                for (int w = 0; w < wave; ++w) g += wsc[w];
                g += __popcll(m & lt);
                if (ex[u] == e && g >= lo && g < hi) tok[0][g - lo] = t;
                pre += wsc[0] + wsc[1] + wsc[2] + wsc[3];
                __syncthreads();
            }
        }
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int row = tid / TPR + RPP * i;
            ta[i] = ((AFULL || row < BM) && row < rows) ? tok[0][row] : -1;
        }
        if (nt == 0 && tid < rows) rv.perm[r0 + tid] = tok[0][tid];
    }
    // a padded row reads token 0's row: output rows are independent and padded ones are
    // never stored, so no branch is needed around the loads
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int t = ta[i] < 0 ? 0 : ta[i];
        a_src[i] = A + (size_t)(MEAN ? t / nh : t) * H + 4 * (tid % TPR);
    }
#pragma unroll
    for (int c = 0; c < PF; ++c) load_a(c, c);
    __builtin_amdgcn_sched_barrier(0);
    if (!GATHER && tid < BM) tok[0][tid] = tok_mine;  // read in the epilogue, after the barriers

    f32x16 acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = f32x16{};
    constexpr int NG = KC / 8;
    f32x4 fa[2][SM], fb[2][SN];
    auto load_frag = [&](int buf, int g, int fs) {
        const int kk = 8 * g + 4 * h;
#pragma unroll
        for (int i = 0; i < SM; ++i) fa[fs][i] = ld4(&As[buf][wm * WTM + i * 32 + l32][kk]);
#pragma unroll
        for (int j = 0; j < SN; ++j) {
            if (!DX) {
                fb[fs][j] = ld4(&Bs[buf][wn * WTN + j * 32 + l32][kk]);
            } else {
                const int cc = wn * WTN + j * 32 + l32;
                fb[fs][j] = f32x4{Bs[buf][kk + 0][cc], Bs[buf][kk + 1][cc], Bs[buf][kk + 2][cc], Bs[buf][kk + 3][cc]};
            }
        }
    };
    auto compute = [&](int buf) {
        load_frag(buf, 0, 0);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g + 1 < NG) load_frag(buf, g + 1, (g + 1) & 1);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < SM; ++i)
#pragma unroll
                    for (int j = 0; j < SN; ++j) acc[i][j] = mfma32(fa[g & 1][i][s], fb[g & 1][j][s], acc[i][j]);
        }
    };

    store_slice(0, 0);
    if (PF < NKC) {
        load_b(PF, 0);
        load_a(PF, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
        if (c + 1 < NKC) {
            store_slice((c + 1) % PF, (c + 1) & 1);
            if (c + 1 + PF < NKC) {
                load_b(c + 1 + PF, (c + 1) % PF);
                load_a(c + 1 + PF, (c + 1) % PF);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        compute(c & 1);
        if (c + 1 < NKC) __syncthreads();
    }

    if constexpr (MOE_ONEPASS_STAGED_STORES) {
        // Epilogue through LDS: the tile goes to a row-major staging area (over the K-slice
        // buffers), then each output row is written as whole 16-byte segments -- a quarter of
        // the store instructions of storing the accumulator blocks directly, and every row
        // segment in one piece.  Same additions in the same order as store_block.
        float(&St)[BM][BN + kPadKN] = *reinterpret_cast<float(*)[BM][BN + kPadKN]>(smem);
        __syncthreads();  // every wavefront has read its last K slice
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    St[wm * WTM + i * 32 + 8 * (r / 4) + 4 * h + (r % 4)][wn * WTN + j * 32 + l32] = acc[i][j][r] + bv[j];
        __syncthreads();
        constexpr int CPR = BN / 4, RPS = kThreads / CPR, NP = BM / RPS;  // float4 per row, rows per pass
        static_assert(kThreads % CPR == 0 && BM % RPS == 0, "staged epilogue shape");
        const int c4 = tid % CPR;
        int tk[NP];
        f32x4 v[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int row = q * RPS + tid / CPR;
            tk[q] = tok[0][row];
            v[q] = ld4(&St[row][4 * c4]);
        }
        if (DX && accumulate) {
            f32x4 old[NP];  // all loads out before the first (conditional) store; padded rows read row 0
#pragma unroll
            for (int q = 0; q < NP; ++q) old[q] = ld4(Out + (size_t)(tk[q] < 0 ? 0 : tk[q]) * H + n0 + 4 * c4);
#pragma unroll
            for (int q = 0; q < NP; ++q)
                if (tk[q] >= 0) st4_nt(Out + (size_t)tk[q] * H + n0 + 4 * c4, old[q] + v[q]);
        } else {
#pragma unroll
            for (int q = 0; q < NP; ++q)
                if (tk[q] >= 0) st4_nt(Out + (size_t)tk[q] * H + n0 + 4 * c4, v[q]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            int tk[16];
            block_row_ids(&tok[0][wm * WTM + i * 32 + 4 * h], tk);
#pragma unroll
            for (int j = 0; j < SN; ++j)
                store_block_ids(Out, H, n0 + wn * WTN + j * 32 + l32, acc[i][j], bv[j], DX && accumulate, tk);
        }
    }
}

// ----------------------------------------------------------------------------------
// dW / db partials.  Workgroup (chunk c, tile (ot, it)): the chunk's tokens of one expert,
// output block dW[o0:o0+BT, i0:i0+BT].  M = o, N = i, K = tokens.
//   part_dw[c][o][i] = sum_{t in chunk} dY[t][o] X[t][i]
//   part_db[c][o]    = sum_{t in chunk} dY[t][o]          (tiles with it == 0)
// Token order inside a chunk is fixed (perm order), as is the MFMA accumulation order.
// Slices go through two LDS buffers, fed from register rings of rows and token ids.
// ----------------------------------------------------------------------------------
template <int BT, int KC>
struct DwF32Smem {
    static constexpr size_t a = sizeof(float) * 2 * KC * (BT + kPadKN);
    static constexpr size_t bytes = 2 * a;
};

#ifndef MOE_DW_PF
#define MOE_DW_PF 2  // K slices of rows in flight per workgroup of the 256 x 256 dW tiles
#endif
#ifndef MOE_F32_KC_DW_BIG
#define MOE_F32_KC_DW_BIG 16  // tokens per K slice in the 256 x 256 dW tiles
#endif
#ifndef MOE_DW_RING_F4
#define MOE_DW_RING_F4 4  // float4 registers of rows in flight per thread in the smaller dW tiles
#endif
// NTH threads: 256 (wavefronts 2 x 2 over the tile) or 512 (2 x 4, for 256 x 256 tiles).
// PFX: K slices of rows in flight (0: as many as MOE_DW_RING_F4 registers hold, even, at
// least 2).
template <int H, int BT, int KC, bool MEAN = false, int NTH = kThreads, int PFX = 0>
__device__ __forceinline__ void dw_f32_body(char* smem, int bid, const float* __restrict__ dY,
                                                      const float* __restrict__ X,
                                                      float* __restrict__ part_dw,
                                                      float* __restrict__ part_db,
                                                      const int* __restrict__ offsets,
                                                      const int* __restrict__ perm, int NE,
                                                      int P, int T, int nh = 1, float inv_nh = 1.0f) {
    constexpr int NTI = H / BT, TPC = NTI * NTI;
    constexpr int WN_W = NTH / 128;  // wavefronts along the tile's columns
    constexpr int WTM = BT / 2, WTN = BT / WN_W, SUBM = WTM / 32, SUBN = WTN / 32;
    constexpr int Q = BT / 4;                  // float4 per row segment
    constexpr int LD = KC * Q / NTH;      // float4 loads per thread per tensor per slice
    constexpr int PF0 = MOE_DW_RING_F4 / (2 * LD);
    constexpr int PF = PFX > 0 ? PFX : (PF0 < 2 ? 2 : PF0 - PF0 % 2);
    float(&As)[2][KC][BT + kPadKN] = *reinterpret_cast<float(*)[2][KC][BT + kPadKN]>(smem);  // dY rows, o0..o0+BT
    float(&Bs)[2][KC][BT + kPadKN] =
        *reinterpret_cast<float(*)[2][KC][BT + kPadKN]>(smem + DwF32Smem<BT, KC>::a);      // X rows, i0..i0+BT

    int c, tile;
    xcd_split(bid, TPC, c, tile);
    int e = -1, t0 = 0, t1 = 0;
    if (!find_chunk(offsets, NE, P, T, c, e, t0, t1)) return;
    const int o0 = (tile / NTI) * BT, i0 = (tile % NTI) * BT;
    const bool do_db = (tile % NTI) == 0;
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int wm = wave / WN_W, wn = wave % WN_W;
    const int nslices = (t1 - t0 + KC - 1) / KC;

    f32x16 acc[SUBM][SUBN];
#pragma unroll
    for (int i = 0; i < SUBM; ++i)
#pragma unroll
        for (int j = 0; j < SUBN; ++j) acc[i][j] = f32x16{};
    float dbacc = 0.0f;

    // Two register rings: the rows of slices s+1 .. s+PF (slot k % PF for slice k) and the
    // token ids of slices s+1 .. s+2PF (slot k % 2PF) are in flight while slice s computes,
    // so neither the gather nor its index loads wait on memory; every id of the first 2PF
    // slices goes out before the first rows, so the start costs two round trips, not three.
    // Loads past the chunk's end read its last token and are zeroed when stored to LDS, so no
    // load sits in a branch; token ids stay raw in the ring and are guarded where the rows
    // are addressed; the ring loop has no exit inside a cycle.  Each of these, otherwise,
    // makes the compiler wait for every load in flight at the loop's back edge.  (Rings of 4
    // and 8 slices measured no faster at the pages' shape: there every workgroup's first
    // loads arrive as one burst bound by memory bandwidth, and the MFMAs bound the rest.)
    int tk[2 * PF][LD];
    f32x4 ra[PF][LD], rb[PF][LD];
    auto kpos = [&](int sl, int i) { return t0 + sl * KC + (tid + NTH * i) / Q; };
    auto load_ids = [&](int sl, int slot) {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int k = kpos(sl, i);
            tk[slot][i] = perm[k < t1 ? k : t1 - 1];
        }
    };
    auto load_rows = [&](int slot, int islot) {  // ids in tk[islot]; rows go to slot
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int cc = 4 * ((tid + NTH * i) % Q);
            const size_t t = (size_t)guard_token(tk[islot][i], T);
            ra[slot][i] = ld4(dY + (MEAN ? t / nh : t) * H + o0 + cc);
            rb[slot][i] = ld4(X + t * H + i0 + cc);
        }
    };
    auto store_rows = [&](int sl, int slot, int buf) {  // masking here, where the rows have arrived
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int q = tid + NTH * i;
            const bool v = kpos(sl, i) < t1;
            f32x4 av = ra[slot][i];
            if (MEAN) av *= inv_nh;
            st4(&As[buf][q / Q][4 * (q % Q)], v ? av : f32x4{});
            st4(&Bs[buf][q / Q][4 * (q % Q)], v ? rb[slot][i] : f32x4{});
        }
    };

    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 2 * PF; ++k) load_ids(k, k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < PF; ++k) load_rows(k, k);
    __builtin_amdgcn_sched_barrier(0);
    store_rows(0, 0, 0);
    load_rows(0, PF);        // slice PF
    load_ids(2 * PF, 0);     // slice 2PF, over slice 0's ids
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // cycles of 2PF slices start at even slices: the LDS buffer of slice s0 + u is u % 2
    int s0 = 0;
    do {  // whole cycles of 2PF slices; slices past the chunk's end load (clamped), do not compute
#pragma unroll
        for (int u = 0; u < 2 * PF; ++u) {
            const int sl = s0 + u;
            store_rows(sl + 1, (u + 1) % PF, (u + 1) & 1);
            load_rows((u + 1) % PF, (u + 1 + PF) % (2 * PF));  // slice sl + 1 + PF
            load_ids(sl + 1 + 2 * PF, (u + 1) % (2 * PF));
            __builtin_amdgcn_sched_barrier(0);
            if (sl < nslices) {  // uniform; LDS reads and MFMAs only
                const int buf = u & 1;
#pragma unroll
                for (int kk = 0; kk < KC; kk += 8) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int k = kk + 4 * h + q;
                        float a[SUBM], b[SUBN];
#pragma unroll
                        for (int i = 0; i < SUBM; ++i) a[i] = As[buf][k][wm * WTM + i * 32 + l32];
#pragma unroll
                        for (int j = 0; j < SUBN; ++j) b[j] = Bs[buf][k][wn * WTN + j * 32 + l32];
#pragma unroll
                        for (int i = 0; i < SUBM; ++i)
#pragma unroll
                            for (int j = 0; j < SUBN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
                    }
                }
                if (do_db && tid < BT) {
#pragma unroll
                    for (int k = 0; k < KC; ++k) dbacc += As[buf][k][tid];
                }
            }
            __syncthreads();
        }
        s0 += 2 * PF;
    } while (s0 < nslices);

    float* __restrict__ Pd = part_dw + (size_t)c * H * H;
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
    if (do_db && tid < BT) part_db[(size_t)c * H + o0 + tid] = dbacc;
}

// ----------------------------------------------------------------------------------
// Kernels.  The backward is one launch: its first n_dx workgroups are dX tiles and the rest
// are dW / db chunk tiles, so both halves fill the GPU together.
// ----------------------------------------------------------------------------------
// Row tiles per XCD group for the small-T backward's dX tiles (tokens per dW chunk / BM; 1
// switches the alignment off).
#ifndef MOE_DX_XCD_ALIGN
#define MOE_DX_XCD_ALIGN 1
#endif
template <int BM>
constexpr int DX_XR = MOE_DX_XCD_ALIGN ? ((MOE_DW_MIN_CHUNK / BM) > 0 ? MOE_DW_MIN_CHUNK / BM : 1) : 1;

#ifdef MOE_FWD_WAVES_PER_EU
#define MOE_FWD_ATTR __attribute__((amdgpu_waves_per_eu(MOE_FWD_WAVES_PER_EU)))
#else
#define MOE_FWD_ATTR
#endif
template <int H, int BM, int BN, int KC, bool ONE>
__global__ __launch_bounds__(kThreads) MOE_FWD_ATTR void k_fwd_f32(const float* __restrict__ X, const float* __restrict__ W,
                                                       const float* __restrict__ bias, float* __restrict__ Y,
                                                       const int* __restrict__ offsets,
                                                       const int* __restrict__ perm, int NE, int T, int ntile_ids) {
    __shared__ __attribute__((aligned(16))) char smem[RowsF32Smem<BM, BN, KC, false>::bytes];
    if (ONE)
        rows_f32_onepass_body<H, BM, BN, KC, false>(smem, blockIdx.x, X, W, bias, Y, offsets, perm, NE, T, 0);
    else
        rows_f32_body<H, BM, BN, KC, false>(smem, blockIdx.x, gridDim.x, ntile_ids, X, W, bias, Y, offsets, perm,
                                            NE, T, 0);
}

// The load-balancing loss inside the forward launch (its inputs are all known once the
// routing is done): n_ablk workgroups after the GEMM ones write dG (and probs) for 256
// tokens each, and one more forms frac, mean_prob and the loss from the routing kernel's
// softmax column sums.  Each takes the counts from the histogram itself, so none waits on
// another workgroup; the arithmetic is the aux kernels' (aux_math.hpp), bit for bit.
struct AuxFwd {
    const float* G;     // gate logits [T][N_E]
    const float* part;  // per-routing-block softmax column sums [n_ablk][N_E]
    float lam;
    const float* lam_dev;  // lambda on the device, or null
    float* dG;
    float* probs;  // optional
    float* loss;
    float* frac;       // optional
    float* mean_prob;  // optional
    int n_gemm;        // GEMM workgroups before the aux ones
    int n_ablk;
};

template <int NEB>
__device__ __forceinline__ void aux_in_forward(char* smem, int r, const int* __restrict__ hist, int nblk, int T,
                                               int NE, const AuxFwd& ax) {
    int* hs = reinterpret_cast<int*>(smem);
    int* tot = hs + 4096;
    float* acc = reinterpret_cast<float*>(tot + 256);
    float* mp = acc + 256;
    float* fr = mp + kMaxExperts;
    const int64_t t = (int64_t)r * kAuxTokens + threadIdx.x;
    float g[NEB];
    aux_load_logits<NEB>(ax.G, t, T, NE, g);  // unconditional, before the histogram's barriers
    hist_counts_lds(hs, tot, hist, nblk, NE);
    const float lam = ax.lam_dev ? ax.lam_dev[0] : ax.lam;
    if (r < ax.n_ablk) {
        float frac[NEB];
        aux_frac_table<NEB>(tot[(int)threadIdx.x < NE ? threadIdx.x : 0], T, fr, frac);
        if (t < T) {
            float p[NEB];
            aux_softmax<NEB>(g, NE, p);
            aux_grad_row<NEB>(p, frac, aux_coef(lam, NE, T), NE, t, ax.dG, ax.probs);
        }
    } else {
        const int tid = threadIdx.x;
        aux_final_block(ax.part, tid < NE ? tot[tid] : 0, ax.n_ablk, T, NE, lam, ax.loss, ax.frac, ax.mean_prob, acc,
                        mp, fr);
    }
}

// Forward for small T that also forms perm, counts and offsets from the routing outputs, so
// the forward pass is routing + this one launch (the scatter kernel is not needed).  With
// NEB > 0 the grid also carries the load-balancing loss (AuxFwd).
template <int H, int BM, int BN, int KC, int NEB>
__global__ __launch_bounds__(kThreads) void k_fwd_f32_gather(const float* __restrict__ X, const float* __restrict__ W,
                                                             const float* __restrict__ bias, float* __restrict__ Y,
                                                             const int* __restrict__ idx, const int* __restrict__ hist,
                                                             int nblk, int T, int* __restrict__ counts,
                                                             int* __restrict__ offsets, int* __restrict__ perm,
                                                             int NE, AuxFwd ax) {
    __shared__ __attribute__((aligned(16))) char smem[RowsF32Smem<BM, BN, KC, false>::bytes];
    if constexpr (NEB > 0) {
        static_assert(RowsF32Smem<BM, BN, KC, false>::bytes >= sizeof(int) * (4096 + 2 * 256 + 2 * kMaxExperts),
                      "LDS for the aux workgroups");
        if ((int)blockIdx.x >= ax.n_gemm) {
            aux_in_forward<NEB>(smem, (int)blockIdx.x - ax.n_gemm, hist, nblk, T, NE, ax);
            return;
        }
    }
    const RouteView rv{idx, hist, nblk, T, counts, offsets, perm};
    rows_f32_onepass_body<H, BM, BN, KC, false, false, 1, true>(smem, blockIdx.x, X, W, bias, Y, nullptr, nullptr,
                                                                 NE, T, 0, 1, 1.0f, rv);
}

// ACC: dX is added to the existing contents (a compile-time choice: with a run-time flag the
// epilogue carries the load-then-store path and the waits it needs even when it is not taken).
// The one-pass grids (small T) are sized so that every workgroup is resident at once with four
// wavefronts per SIMD; the attribute keeps the register count there (at H = 512 it would spill).
template <int H, int BM, int BN, int BT, int KCX, int KCW, bool MEAN, bool ONE, bool DWF = false, bool ACC = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(ONE && H <= 256 ? 4 : 1)))
void k_bwd_f32(const float* __restrict__ dY, const float* __restrict__ X,
                                                       const float* __restrict__ W, float* __restrict__ dX,
                                                       int accumulate, float* __restrict__ part_dw,
                                                       float* __restrict__ part_db,
                                                       const int* __restrict__ offsets,
                                                       const int* __restrict__ perm, int NE, int P, int T,
                                                       int n_dx, int dx_tile_ids, int nh, float inv_nh) {
    constexpr size_t r = RowsF32Smem<BM, BN, KCX, true>::bytes, d = DwF32Smem<BT, KCW>::bytes;
    __shared__ __attribute__((aligned(16))) char smem[r > d ? r : d];  // one LDS region, either role
    if (DWF) {  // dW workgroups first (the long ones), then n_dx workgroups of a few dX tiles each
        const int n_dw = (int)gridDim.x - n_dx;
        if ((int)blockIdx.x < n_dw)
            dw_f32_body<H, BT, KCW, MEAN>(smem, blockIdx.x, dY, X, part_dw, part_db, offsets, perm, NE, P, T, nh,
                                          inv_nh);
        else
            rows_f32_body<H, BM, BN, KCX, true, MEAN>(smem, blockIdx.x - n_dw, n_dx, dx_tile_ids, dY, W, nullptr, dX,
                                                      offsets, perm, NE, T, (int)ACC, nh, inv_nh);
        return;
    }
    if ((int)blockIdx.x < n_dx) {
        if (ONE)
            rows_f32_onepass_body<H, BM, BN, KCX, true, MEAN, DX_XR<BM>>(smem, blockIdx.x, dY, W, nullptr, dX, offsets,
                                                                          perm, NE, T, (int)ACC, nh, inv_nh);
        else
            rows_f32_body<H, BM, BN, KCX, true, MEAN>(smem, blockIdx.x, n_dx, dx_tile_ids, dY, W, nullptr, dX,
                                                      offsets, perm, NE, T, (int)ACC, nh, inv_nh);
    }
    else
        dw_f32_body<H, BT, KCW, MEAN>(smem, blockIdx.x - n_dx, dY, X, part_dw, part_db, offsets, perm, NE, P, T, nh,
                                  inv_nh);
}

// W-stationary row GEMM (H = 256, large T): Out[t, :] = A[t, :] . Wm[n, :]^T (+ bias) for the
// tokens of one expert.  Each of the 256 workgroups (one per compute unit, eight wavefronts, two
// per SIMD) holds all of W[e] -- each wavefront 32 features for the whole K in its registers as
// MFMA operands (128 VGPRs) -- and streams a fixed share of the expert-sorted token order
// through it in groups of 32 tokens: their rows go to LDS whole (one 1 KB row per load
// instruction, 16-byte chunk c of row r at c ^ (r & 15)), each wavefront reads its fragments
// from there, and the results are staged in LDS and written a group later as whole rows.
// Per group a wavefront issues 128 MFMAs back to back: one barrier per 32 tokens, and no tile
// epilogue between K slices.  The k order (lane half h of MFMA step j in block m takes
// k = 8 m + 4 h + j) and the epilogue's additions are those of the tiled kernels, so the results
// are the same bits.  The forward passes W ([n][k]); dX passes W^T (written by the d_W launch).
// The token share of workgroup v: positions [v T / 256, (v + 1) T / 256) of the expert-sorted
// order, cut at expert boundaries into segments; each segment loads its expert's W once.
#ifndef MOE_F32_WST
#define MOE_F32_WST 1
#endif
constexpr int kF32WstThreads = 512, kF32WstWgs = 256, kF32WstGT = 32;
struct F32WstSmem {
    static constexpr int H = 256, ROWB = 4 * H;                   // bytes per token row
    static constexpr size_t xbuf = (size_t)kF32WstGT * ROWB;      // one group's rows: 32 KB
    static constexpr size_t obuf = (size_t)kF32WstGT * H * 4;     // one group's results: 32 KB
    static constexpr size_t ost_off = 2 * xbuf, bias_off = ost_off + 2 * obuf;
    static constexpr size_t ids_off = bias_off + H * 4;           // token ids: [5][32]
    static constexpr size_t bytes = ids_off + 5 * kF32WstGT * 4;
};
// padded rows of the W-stationary kernel read zeros from these rows and write their results to
// the sink rows (never read), so that no load or store is conditional and every group issues the
// same memory operations.  One row per workgroup of an XCD's 32 (blocks go to the XCDs in turn):
// every workgroup on one row would queue its padded groups on one L2 channel.
constexpr int kF32PadRows = 32;
static __device__ __attribute__((aligned(16))) float kZeroRowF[kF32PadRows * 256];
static __device__ __attribute__((aligned(16))) float kSinkRowF[kF32PadRows * 256];
// 256 workgroups when every share holds at least 8 groups of 32 tokens
static inline bool f32_wst(int64_t T, int H) {
    return MOE_F32_WST && H == 256 && T >= (int64_t)kF32WstWgs * 8 * kF32WstGT;
}

template <bool DX, bool MEAN, bool ACC>
__device__ __forceinline__ void rows_f32_wst_body(char* smem, const float* __restrict__ A,
                                                  const float* __restrict__ Wm, const float* __restrict__ bias,
                                                  float* __restrict__ Out, const int* __restrict__ offsets,
                                                  const int* __restrict__ perm, int NE, int T, int nh,
                                                  float inv_nh) {
    using S = F32WstSmem;
    constexpr int H = S::H, NM = H / 8, GT = kF32WstGT;
    constexpr int CPR = S::ROWB / 16;        // 16-byte chunks per row: 64
    constexpr int RPI = kF32WstThreads / CPR;  // rows per load round: 8
    constexpr int NL = GT / RPI;             // row loads per thread per group: 4
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, l32 = lane % 32, h = lane / 32;
    const int v = blockIdx.x, fw = 32 * wave;
    const int P0 = (int)((int64_t)v * T / kF32WstWgs), P1 = (int)((int64_t)(v + 1) * T / kF32WstWgs);
    char* const xb0 = smem;
    char* const xb1 = smem + S::xbuf;
    float* const ob0 = reinterpret_cast<float*>(smem + S::ost_off);
    float* const ob1 = reinterpret_cast<float*>(smem + S::ost_off + S::obuf);
    float* const bias_s = reinterpret_cast<float*>(smem + S::bias_off);
    // token ids of group g in ids[g % 5]: written at g - 2, read at g - 1 (its rows' loads) and at
    // g + 1 (its output), so with five buffers no wavefront overwrites ids another still reads
    int(&ids)[5][GT] = *reinterpret_cast<int(*)[5][GT]>(smem + S::ids_off);
    int x_lo, x_cnt;
    expert_range(offsets, NE, T, x_lo, x_cnt);
    const int lrow = tid / CPR, lch = tid % CPR;
    // perm [T] int32 through a buffer descriptor (word 3: raw 32-bit accesses on CDNA)
    const __amdgpu_buffer_rsrc_t perm_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)perm, 0, (int)((uint32_t)T * 4u), 0x00020000);

    f32x4 wr[NM];  // feature fw + l32, k 8 m + 4 h .. + 3
    f32x4 xr[NL];  // the next group's rows, in flight

    const int pad_row = 256 * ((blockIdx.x / 8) % kF32PadRows);
    auto load_x_one = [&](const int* gid, int j) {  // a padded row reads a zero row
        const int t = gid[lrow + RPI * j];
        xr[j] = ld4(t >= 0 ? A + (size_t)(MEAN ? t / nh : t) * H + 4 * lch : kZeroRowF + pad_row + 4 * lch);
    };
    auto load_x = [&](const int* gid) {
#pragma unroll
        for (int j = 0; j < NL; ++j) load_x_one(gid, j);
    };
    auto store_x = [&](char* xb) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int r = lrow + RPI * j;
            st4(reinterpret_cast<float*>(xb + r * S::ROWB + 16 * (lch ^ (r & 15))), xr[j]);
        }
    };
    // fp32 result row r (token), 64 chunks of 4 features: chunk c at c ^ (r & 15)
    auto ost_at = [](float* ob, int r, int c) { return ob + r * H + 4 * (c ^ (r & 15)); };
    // mid(b) runs after the b-th batch of MFMAs has been issued (the previous group's output
    // rows, one per batch, so their stores overlap the MFMA chain)
    auto compute = [&](const char* xb, float* ob, auto&& mid) {
        const char* row = xb + l32 * S::ROWB;
        f32x16 acc = f32x16{};
        constexpr int MB = 4;  // fragments read 4 blocks of 8 k ahead of their MFMAs
#pragma unroll
        for (int m0 = 0; m0 < NM; m0 += MB) {
            f32x4 xf[MB];
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                xf[u] = *reinterpret_cast<const f32x4*>(row + 16 * ((2 * (m0 + u) + h) ^ (l32 & 15)));
                if (MEAN) xf[u] *= inv_nh;
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < MB; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc = mfma32(wr[m0 + u][j], xf[u][j], acc);
            __builtin_amdgcn_sched_barrier(0);
            mid(m0 / MB);
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane: token l32, features fw + 8 q + 4 h .. + 3
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 val = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
            *reinterpret_cast<f32x4*>(ost_at(ob, l32, (fw >> 2) + 2 * q + h)) = val;
        }
    };
    // staged results of a group -> rows: thread covers features 4 c .. + 3 of rows tid / 64 + 8 i
    auto store_row = [&](float* ob, const int* gid, int i) {
        const int c = tid % 64;
        f32x4 bq = f32x4{};
        if (!DX) bq = *reinterpret_cast<const f32x4*>(bias_s + 4 * c);
        const int r = tid / 64 + 8 * i;
        const int t = gid[r];
        f32x4 v = *reinterpret_cast<const f32x4*>(ost_at(ob, r, c));
        if (!DX) v = v + bq;
        float* const dst = t >= 0 ? Out + (size_t)t * H + 4 * c : kSinkRowF + pad_row + 4 * c;
        if (ACC) v = ld4(dst) + v;
        st4_nt(dst, v);
    };
    auto store_out = [&](float* ob, const int* gid) {
#pragma unroll
        for (int i = 0; i < GT / 8; ++i) store_row(ob, gid, i);
    };

    int p = P0;
    while (p < P1) {
        // segment: positions [p, se) of expert e
        const uint64_t hit = __ballot(lane < NE && p >= x_lo && p < x_lo + x_cnt);
        if (hit == 0) break;  // (only with routing that does not cover [0, T))
        const int e = __ffsll((unsigned long long)hit) - 1;
        const int se = min(P1, __builtin_amdgcn_readlane(x_lo, e) + __builtin_amdgcn_readlane(x_cnt, e));
        const int G = (se - p + GT - 1) / GT;
        // this thread's entry of perm in group g, as loaded (unconditional, of a clamped position;
        // the guard and the validity are applied where the id is written to LDS, at the end of
        // the group).  A buffer load: unlike a load through the read-only pointer, the compiler
        // keeps it where it is issued instead of sinking it to its use.
        auto group_raw = [&](int g) {
            const int k = p + GT * g + (tid % GT);
            return __builtin_amdgcn_raw_buffer_load_b32(perm_rs, (k < se ? k : se - 1) * 4, 0, 0);
        };
        auto group_valid = [&](int g) { return g < G && p + GT * g + (tid % GT) < se; };
        __syncthreads();  // the previous segment is done with the bias, ids and staged results
        {
            const float* __restrict__ We = Wm + (size_t)e * H * H + (size_t)(fw + l32) * H + 4 * h;
#pragma unroll
            for (int m = 0; m < NM; ++m) wr[m] = ld4(We + 8 * m);
        }
        if (!DX && tid < H) bias_s[tid] = bias[(size_t)e * H + tid];
        {
            const int i0 = group_raw(0), i1 = group_raw(1);
            if (tid < GT) {
                ids[0][tid] = group_valid(0) ? guard_token(i0, T) : -1;
                ids[1][tid] = group_valid(1) ? guard_token(i1, T) : -1;
                ids[4][tid] = -1;  // "group -1": the output stores issued during group 0 go to the sink
            }
        }
        __syncthreads();
        load_x(ids[0]);
        store_x(xb0);  // the rows of group 0, visible after the loop's first barrier
        // group g: barrier (its rows and the ids of g + 1 visible, every wavefront done with group
        // g - 1 and so with the row stage of g + 1); the perm entries of g + 2 into flight; the
        // MFMAs of g with, between its batches, the row loads of g + 1 (first half) and the output
        // rows of g - 1 (second half; none before group 0), one per batch, so the vector-memory work
        // of the eight wavefronts overlaps the MFMA chain instead of queueing behind the barrier
        // (issued all at once there, the row loads alone took about 1,100 of the 20,000 cycles of
        // a group); then the ids of g + 2 and the rows of g + 1 to LDS.  Every wait for a load is
        // in the iteration that issued it, so it counts exactly the memory operations issued after.
        static_assert(NM / 4 >= NL + GT / 8, "a batch for every row load and output row");
#pragma unroll 1
        for (int g = 0; g < G; ++g) {
            __syncthreads();
            const int idr = group_raw(g + 2);
            // keep this load here, ahead of the group's other memory operations (the compiler
            // would otherwise sink it to its use, where waiting for it waits for all of them)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            float* const obp = (g & 1) ? ob0 : ob1;
            const int* const gidp = ids[(g + 4) % 5];
            const int* const gidn = ids[(g + 1) % 5];
            // no condition on g: past the last group the ids are -1 (zero rows loaded, staged and
            // never read), and group -1's ids are -1 (its "outputs" go to the sink row)
            compute((g & 1) ? xb1 : xb0, (g & 1) ? ob1 : ob0, [&](int b) {
                if (b < NL)
                    load_x_one(gidn, b);
                else if (b - NL < GT / 8)
                    store_row(obp, gidp, b - NL);
            });
            // the perm entries of g + 2 are used by every thread from here (an empty asm that takes
            // the value), so the compiler cannot move their load into the branch below
            int idv = idr;
            asm volatile("" : "+v"(idv));
            if (tid < GT) ids[(g + 2) % 5][tid] = group_valid(g + 2) ? guard_token(idv, T) : -1;
            store_x((g & 1) ? xb0 : xb1);
        }
        __syncthreads();
        store_out(((G - 1) & 1) ? ob1 : ob0, ids[(G - 1) % 5]);
        p = se;
    }
}

template <bool DX, bool MEAN, bool ACC>
__global__ __launch_bounds__(kF32WstThreads) void k_rows_f32_wst(const float* __restrict__ A,
                                                                  const float* __restrict__ Wm,
                                                                  const float* __restrict__ bias,
                                                                  float* __restrict__ Out,
                                                                  const int* __restrict__ offsets,
                                                                  const int* __restrict__ perm, int NE, int T,
                                                                  int nh, float inv_nh) {
    __shared__ __attribute__((aligned(16))) char smem[F32WstSmem::bytes];
    rows_f32_wst_body<DX, MEAN, ACC>(smem, A, Wm, bias, Out, offsets, perm, NE, T, nh, inv_nh);
}

// Large T, H = 256 / 512: the 256 x 256 d_W tiles (eight wavefronts of 128 x 64, one workgroup
// per compute unit) in a launch of their own, then the dX tiles as a persistent launch.  A
// 128 x 128 d_W tile re-reads its chunk's dY and X columns once per partner tile; with the
// whole 256 x 256 block per workgroup each chunk row is read once.
constexpr int kDwBigThreads = 512;
// The first N_E workgroups of the launch write Wt[e] = W[e]^T for the dX launch that follows
// (64 x 64 blocks through LDS, rows padded by one float), the rest compute d_W tiles.
template <int H>
__device__ __forceinline__ void transpose_w_body(char* smem, int e, const float* __restrict__ W, float* __restrict__ Wt) {
    float(&tb)[64][65] = *reinterpret_cast<float(*)[64][65]>(smem);
    const float* __restrict__ src = W + (size_t)e * H * H;
    float* __restrict__ dst = Wt + (size_t)e * H * H;
    const int tid = threadIdx.x;
#pragma unroll 1
    for (int b = 0; b < (H / 64) * (H / 64); ++b) {
        const int r0 = (b / (H / 64)) * 64, c0 = (b % (H / 64)) * 64;
        f32x4 v[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {  // 64 rows x 16 float4, two per thread
            const int q = tid + kDwBigThreads * u;
            v[u] = ld4(src + (size_t)(r0 + q / 16) * H + c0 + 4 * (q % 16));
        }
        if (b > 0) __syncthreads();  // the previous block has been read out
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int q = tid + kDwBigThreads * u;
#pragma unroll
            for (int x = 0; x < 4; ++x) tb[4 * (q % 16) + x][q / 16] = v[u][x];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int q = tid + kDwBigThreads * u;
            const int r = q / 16, c = 4 * (q % 16);
            st4(dst + (size_t)(c0 + r) * H + r0 + c, f32x4{tb[r][c], tb[r][c + 1], tb[r][c + 2], tb[r][c + 3]});
        }
    }
}

template <int H, int KCW, bool MEAN>
__global__ __launch_bounds__(kDwBigThreads) void k_dw_f32_big(const float* __restrict__ dY,
                                                               const float* __restrict__ X,
                                                               const float* __restrict__ W, float* __restrict__ Wt,
                                                               float* __restrict__ part_dw,
                                                               float* __restrict__ part_db,
                                                               const int* __restrict__ offsets,
                                                               const int* __restrict__ perm, int NE, int P, int T,
                                                               int nh, float inv_nh) {
    __shared__ __attribute__((aligned(16))) char smem[DwF32Smem<256, KCW>::bytes];
    static_assert(DwF32Smem<256, KCW>::bytes >= sizeof(float) * 64 * 65, "LDS for the transpose");
    if ((int)blockIdx.x < NE) {
        transpose_w_body<H>(smem, blockIdx.x, W, Wt);
        return;
    }
    dw_f32_body<H, 256, KCW, MEAN, kDwBigThreads, MOE_DW_PF>(smem, (int)blockIdx.x - NE, dY, X, part_dw, part_db, offsets, perm,
                                                  NE, P, T, nh, inv_nh);
}

// dX from the transposed weights Wt[e] = W[e]^T (written by the d_W launch), read like the
// forward reads W: 16-byte fragment reads and the forward's 32-wide K slices.
template <int H, int BN, int KCX, bool MEAN, bool ACC>
__global__ __launch_bounds__(kThreads) void k_dx_f32(const float* __restrict__ dY, const float* __restrict__ Wt,
                                                      float* __restrict__ dX, int accumulate,
                                                      const int* __restrict__ offsets, const int* __restrict__ perm,
                                                      int NE, int T, int dx_tile_ids, int nh, float inv_nh) {
    __shared__ __attribute__((aligned(16))) char smem[RowsF32Smem<128, BN, KCX, false>::bytes];
    rows_f32_body<H, 128, BN, KCX, true, MEAN, true>(smem, blockIdx.x, gridDim.x, dx_tile_ids, dY, Wt, nullptr, dX,
                                                     offsets, perm, NE, T, (int)ACC, nh, inv_nh);
}

// ----------------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------------
static inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Tiles: 128 x (128 or H) rows x columns and 128 x 128 d_W tiles at large T; at small T
// MOE_ROWS_SMALL_BM x MOE_ROWS_SMALL_BN and MOE_DW_SMALL_BT (f32_big_tiles decides).
#ifndef MOE_ROWS_SMALL_BM
#define MOE_ROWS_SMALL_BM 64
#endif
#ifndef MOE_ROWS_SMALL_BN
#define MOE_ROWS_SMALL_BN 128
#endif
// The forward's small-T tile may differ from dX's: the forward runs alone, while dX shares
// the resident slots with the dW workgroups.
#ifndef MOE_FWD_SMALL_BM
#define MOE_FWD_SMALL_BM MOE_ROWS_SMALL_BM
#endif
#ifndef MOE_FWD_SMALL_BN
#define MOE_FWD_SMALL_BN 64
#endif
template <int H>
struct F32Tiles {
    static constexpr int BIG_BN = (H >= 128) ? 128 : H;
    static constexpr int BIG_BT = (H >= 128) ? 128 : 64;
    static constexpr int SMALL_BN = (MOE_ROWS_SMALL_BN < H) ? MOE_ROWS_SMALL_BN : H;
    static constexpr int SMALL_BM = (SMALL_BN == 128 || MOE_ROWS_SMALL_BM >= 64) ? MOE_ROWS_SMALL_BM : 64;
    static constexpr int FWD_BN = (MOE_FWD_SMALL_BN < H) ? MOE_FWD_SMALL_BN : H;
    static constexpr int FWD_BM = (FWD_BN == 128 || MOE_FWD_SMALL_BM >= 64) ? MOE_FWD_SMALL_BM : 64;
    static constexpr int SMALL_BT = (MOE_DW_SMALL_BT < H) ? MOE_DW_SMALL_BT : H;
};

template <int H, int BN>
static int rows_grid(int64_t T, int NE, int bm) {
    return round_up((int)((T + bm - 1) / bm) + NE, 8) * (H / BN);
}

template <int H, int BT>
static int dw_grid(int n_chunk_max) {
    constexpr int TPC = (H / BT) * (H / BT);
    return round_up(n_chunk_max, 8) * TPC;
}

// Row-GEMM workgroups once the tile ids reach `from` (0: one workgroup per tile).  Both
// counts are multiples of 8, so every tile id a workgroup takes maps to the XCD of its
// first one.  Forward: two per CU, its occupancy.  dX in the small-T backward when its tiles
// exceed the one-pass limit: one per CU, the dW workgroups fill the rest.
#ifndef MOE_FWD_PERSIST_WGS
#define MOE_FWD_PERSIST_WGS 512
#endif
#ifndef MOE_DX_PERSIST_WGS
#define MOE_DX_PERSIST_WGS 256
#endif
#ifndef MOE_DX_BIG_PERSIST_WGS
#define MOE_DX_BIG_PERSIST_WGS 512  // dX launch of its own (after the 256 x 256 d_W launch): two per CU
#endif
#ifndef MOE_DX_TILES_PER_WG
#define MOE_DX_TILES_PER_WG 1  // dX tiles per workgroup in the large-T backward
#endif
static int persist_wgs(int ids, int wgs, int from) { return (wgs <= 0 || ids < from) ? ids : wgs; }
// Up to this many small-row tiles, a grid of one-tile workgroups with every K slice in
// flight (the tiles fit in the resident slots, so latency, not throughput, bounds them).
#ifndef MOE_FWD_GATHER
#define MOE_FWD_GATHER 1  // small-T forward forms perm itself (routing + one launch)
#endif
#ifndef MOE_ROWS_ONEPASS_MAX_IDS
#define MOE_ROWS_ONEPASS_MAX_IDS 1024
#endif

template <int H>
static hipError_t fwd_f32(const float* X, const float* W, const float* bias, float* Y, const int32_t* offsets,
                          const int32_t* perm, int64_t T, int NE, hipStream_t s) {
    using TL = F32Tiles<H>;
    if (f32_wst(T, H)) {
        launch_kernel((k_rows_f32_wst<false, false, false>), dim3(kF32WstWgs), dim3(kF32WstThreads), 0, s, X, W, bias,
                      Y, offsets, perm, NE, (int)T, 1, 1.0f);
        return hipGetLastError();
    }
    if (f32_big_tiles(T, H)) {
        const int ids = rows_grid<H, TL::BIG_BN>(T, NE, 128);
        const int grid = persist_wgs(ids, MOE_FWD_PERSIST_WGS, MOE_FWD_PERSIST_WGS);
        launch_kernel((k_fwd_f32<H, 128, TL::BIG_BN, MOE_F32_KC_FWD, false>), dim3(grid), dim3(kThreads), 0, s,
                           X, W, bias, Y, offsets, perm, NE, (int)T, ids);
        return hipGetLastError();
    }
    const int ids = rows_grid<H, TL::FWD_BN>(T, NE, TL::FWD_BM);
    if (ids <= MOE_ROWS_ONEPASS_MAX_IDS)
        launch_kernel((k_fwd_f32<H, TL::FWD_BM, TL::FWD_BN, MOE_F32_KC_FWD_SMALL, true>), dim3(ids),
                           dim3(kThreads), 0, s, X, W, bias, Y, offsets, perm, NE, (int)T, ids);
    else
        launch_kernel((k_fwd_f32<H, TL::FWD_BM, TL::FWD_BN, MOE_F32_KC_FWD, false>),
                           dim3(persist_wgs(ids, MOE_FWD_PERSIST_WGS, MOE_FWD_PERSIST_WGS)), dim3(kThreads), 0, s, X,
                           W, bias, Y, offsets, perm, NE, (int)T, ids);
    return hipGetLastError();
}

template <int H, bool MEAN, bool ACC>
static hipError_t bwd_f32(const float* dY, const float* X, const float* W, float* dX, int accumulate, float* pdw,
                          float* pdb, float* wt, const int32_t* offsets, const int32_t* perm, int64_t T, int NE, int P,
                          int n_chunk_max, int nh, hipStream_t s) {
    using TL = F32Tiles<H>;
    const float inv_nh = 1.0f / (float)nh;
    if constexpr (H >= 256) {
        if (f32_dw_tile(T, H) == 256) {
            // the kernel timer (if armed) brackets both launches
            constexpr int TPC = (H / 256) * (H / 256);
            const int dx_ids = rows_grid<H, TL::BIG_BN>(T, NE, 128);
            const ArmedEvents ev = take_armed_events();
            launch_kernel_ev((k_dw_f32_big<H, MOE_F32_KC_DW_BIG, MEAN>), dim3(NE + round_up(n_chunk_max, 8) * TPC),
                             dim3(kDwBigThreads), 0, s, ev.start, nullptr, dY, X, W, wt, pdw, pdb, offsets, perm, NE,
                             P, (int)T, nh, inv_nh);
            if (f32_wst(T, H))
                launch_kernel_ev((k_rows_f32_wst<true, MEAN, ACC>), dim3(kF32WstWgs), dim3(kF32WstThreads), 0, s,
                                 nullptr, ev.stop, dY, wt, nullptr, dX, offsets, perm, NE, (int)T, nh, inv_nh);
            else
                launch_kernel_ev((k_dx_f32<H, TL::BIG_BN, MOE_F32_KC_FWD, MEAN, ACC>),
                                 dim3(persist_wgs(dx_ids, MOE_DX_BIG_PERSIST_WGS, MOE_DX_BIG_PERSIST_WGS)),
                                 dim3(kThreads), 0, s, nullptr, ev.stop, dY, wt, dX, accumulate, offsets, perm, NE,
                                 (int)T, dx_ids, nh, inv_nh);
            return hipGetLastError();
        }
    }
    if (f32_big_tiles(T, H)) {
        // Longest first: the dW workgroups (a whole chunk each) lead the grid and the dX tiles
        // follow, MOE_DX_TILES_PER_WG per workgroup (persistent over those few, so each still
        // prefetches its next tile), so the dispatcher evens out the end of the launch.
        const int dx_ids = rows_grid<H, TL::BIG_BN>(T, NE, 128);
        const int n_dx = round_up((dx_ids + MOE_DX_TILES_PER_WG - 1) / MOE_DX_TILES_PER_WG, 8);
        const int grid = n_dx + dw_grid<H, TL::BIG_BT>(n_chunk_max);
        launch_kernel(
            (k_bwd_f32<H, 128, TL::BIG_BN, TL::BIG_BT, MOE_F32_KC_DX, MOE_F32_KC_DW, MEAN, false, true, ACC>), dim3(grid),
            dim3(kThreads), 0, s, dY, X, W, dX, accumulate, pdw, pdb, offsets, perm, NE, P, (int)T, n_dx, dx_ids, nh,
            inv_nh);
        return hipGetLastError();
    }
    const int xr = DX_XR<TL::SMALL_BM>;
    const int dx_ids = round_up((int)((T + TL::SMALL_BM - 1) / TL::SMALL_BM) + NE, 8 * xr) * (H / TL::SMALL_BN);
    const bool one = dx_ids <= MOE_ROWS_ONEPASS_MAX_IDS;
    const int n_dx = one ? dx_ids : persist_wgs(dx_ids, MOE_DX_PERSIST_WGS, 2 * MOE_DX_PERSIST_WGS);
    const int grid = n_dx + dw_grid<H, TL::SMALL_BT>(n_chunk_max);
    if (one)
        launch_kernel(
            (k_bwd_f32<H, TL::SMALL_BM, TL::SMALL_BN, TL::SMALL_BT, MOE_F32_KC_DX, MOE_F32_KC_DW, MEAN, true, false, ACC>),
            dim3(grid), dim3(kThreads), 0, s, dY, X, W, dX, accumulate, pdw, pdb, offsets, perm, NE, P, (int)T, n_dx,
            dx_ids, nh, inv_nh);
    else
        launch_kernel(
            (k_bwd_f32<H, TL::SMALL_BM, TL::SMALL_BN, TL::SMALL_BT, MOE_F32_KC_DX, MOE_F32_KC_DW, MEAN, false, false, ACC>),
            dim3(grid), dim3(kThreads), 0, s, dY, X, W, dX, accumulate, pdw, pdb, offsets, perm, NE, P, (int)T, n_dx,
            dx_ids, nh, inv_nh);
    return hipGetLastError();
}

template <int H>
static hipError_t fwd_f32_gather(const float* X, const float* W, const float* bias, float* Y, const int32_t* idx,
                                 const int32_t* hist, int n_rblk, int32_t* counts, int32_t* offsets, int32_t* perm,
                                 int64_t T, int NE, const AuxFwdArgs* aux, hipStream_t s) {
    using TL = F32Tiles<H>;
    constexpr int BM = TL::FWD_BM, BN = TL::FWD_BN, KC = MOE_F32_KC_FWD_SMALL;
    const int ids = rows_grid<H, BN>(T, NE, BM);
    AuxFwd ax = {};
    ax.n_gemm = ids;
    if (!aux) {
        launch_kernel(k_fwd_f32_gather<H, BM, BN, KC, 0>, dim3(ids), dim3(kThreads), 0, s, X, W, bias, Y, idx, hist,
                      n_rblk, (int)T, counts, offsets, perm, NE, ax);
        return hipGetLastError();
    }
    ax.G = aux->G;
    ax.part = aux->part;
    ax.lam = aux->lam;
    ax.lam_dev = aux->lam_dev;
    ax.dG = aux->dG;
    ax.probs = aux->probs;
    ax.loss = aux->loss;
    ax.frac = aux->frac;
    ax.mean_prob = aux->mean_prob;
    ax.n_ablk = aux->n_ablk;
    const dim3 grid(ids + ax.n_ablk + 1);
    if (NE <= 4)
        launch_kernel(k_fwd_f32_gather<H, BM, BN, KC, 4>, grid, dim3(kThreads), 0, s, X, W, bias, Y, idx, hist,
                      n_rblk, (int)T, counts, offsets, perm, NE, ax);
    else if (NE <= 8)
        launch_kernel(k_fwd_f32_gather<H, BM, BN, KC, 8>, grid, dim3(kThreads), 0, s, X, W, bias, Y, idx, hist,
                      n_rblk, (int)T, counts, offsets, perm, NE, ax);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int H>
static bool gather_fits_h(int64_t T, int NE) {
    using TL = F32Tiles<H>;
    return rows_grid<H, TL::FWD_BN>(T, NE, TL::FWD_BM) <= MOE_ROWS_ONEPASS_MAX_IDS;
}

bool fwd_gemm_f32_gather_fits(int64_t T, int H, int NE, int n_rblk) {
    if (!MOE_FWD_GATHER || f32_big_tiles(T, H) || (int64_t)n_rblk * NE > 4096) return false;
    switch (H) {
        case 64: return gather_fits_h<64>(T, NE);
        case 128: return gather_fits_h<128>(T, NE);
        case 256: return gather_fits_h<256>(T, NE);
        case 512: return gather_fits_h<512>(T, NE);
    }
    return false;
}

hipError_t launch_fwd_gemm_f32_gather(const float* X, const float* W, const float* bias, float* Y,
                                      const int32_t* idx, const int32_t* hist, int n_rblk, int32_t* counts,
                                      int32_t* offsets, int32_t* perm, int64_t T, int H, int NE,
                                      const AuxFwdArgs* aux, hipStream_t s) {
    if (aux && (NE > kAuxFwdMaxExperts || aux->n_ablk != n_rblk)) return hipErrorInvalidValue;
    switch (H) {
        case 64: return fwd_f32_gather<64>(X, W, bias, Y, idx, hist, n_rblk, counts, offsets, perm, T, NE, aux, s);
        case 128: return fwd_f32_gather<128>(X, W, bias, Y, idx, hist, n_rblk, counts, offsets, perm, T, NE, aux, s);
        case 256: return fwd_f32_gather<256>(X, W, bias, Y, idx, hist, n_rblk, counts, offsets, perm, T, NE, aux, s);
        case 512: return fwd_f32_gather<512>(X, W, bias, Y, idx, hist, n_rblk, counts, offsets, perm, T, NE, aux, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_gemm_f32(const float* X, const float* W, const float* bias, float* Y, const int32_t* offsets,
                               const int32_t* perm, int64_t T, int H, int NE, hipStream_t s) {
    switch (H) {
        case 64: return fwd_f32<64>(X, W, bias, Y, offsets, perm, T, NE, s);
        case 128: return fwd_f32<128>(X, W, bias, Y, offsets, perm, T, NE, s);
        case 256: return fwd_f32<256>(X, W, bias, Y, offsets, perm, T, NE, s);
        case 512: return fwd_f32<512>(X, W, bias, Y, offsets, perm, T, NE, s);
    }
    return hipErrorInvalidValue;
}

template <bool MEAN, bool ACC>
static hipError_t bwd_f32_h2(const float* dY, const float* X, const float* W, float* dX, float* pdw, float* pdb,
                             float* wt, const int32_t* offsets, const int32_t* perm, int64_t T, int H, int NE, int P,
                             int n_chunk_max, int nh, hipStream_t s) {
    const int acc = ACC ? 1 : 0;
    switch (H) {
        case 64:
            return bwd_f32<64, MEAN, ACC>(dY, X, W, dX, acc, pdw, pdb, wt, offsets, perm, T, NE, P, n_chunk_max, nh, s);
        case 128:
            return bwd_f32<128, MEAN, ACC>(dY, X, W, dX, acc, pdw, pdb, wt, offsets, perm, T, NE, P, n_chunk_max, nh, s);
        case 256:
            return bwd_f32<256, MEAN, ACC>(dY, X, W, dX, acc, pdw, pdb, wt, offsets, perm, T, NE, P, n_chunk_max, nh, s);
        case 512:
            return bwd_f32<512, MEAN, ACC>(dY, X, W, dX, acc, pdw, pdb, wt, offsets, perm, T, NE, P, n_chunk_max, nh, s);
    }
    return hipErrorInvalidValue;
}

template <bool MEAN>
static hipError_t bwd_f32_h(const float* dY, const float* X, const float* W, float* dX, int accumulate, float* pdw,
                            float* pdb, float* wt, const int32_t* offsets, const int32_t* perm, int64_t T, int H,
                            int NE, int P, int n_chunk_max, int nh, hipStream_t s) {
    if (accumulate)
        return bwd_f32_h2<MEAN, true>(dY, X, W, dX, pdw, pdb, wt, offsets, perm, T, H, NE, P, n_chunk_max, nh, s);
    return bwd_f32_h2<MEAN, false>(dY, X, W, dX, pdw, pdb, wt, offsets, perm, T, H, NE, P, n_chunk_max, nh, s);
}

hipError_t launch_bwd_gemm_f32(const float* dY, const float* X, const float* W, float* dX, int accumulate,
                               float* pdw, float* pdb, float* wt, const int32_t* offsets, const int32_t* perm,
                               int64_t T, int H, int NE, int P, int n_chunk_max, hipStream_t s) {
    return bwd_f32_h<false>(dY, X, W, dX, accumulate, pdw, pdb, wt, offsets, perm, T, H, NE, P, n_chunk_max, 1, s);
}

hipError_t launch_bwd_gemm_f32_from_mean(const float* d_mean, const float* X, const float* W, float* dX,
                                         int accumulate, float* pdw, float* pdb, float* wt, const int32_t* offsets,
                                         const int32_t* perm, int64_t T, int H, int NE, int NH, int P,
                                         int n_chunk_max, hipStream_t s) {
    return bwd_f32_h<true>(d_mean, X, W, dX, accumulate, pdw, pdb, wt, offsets, perm, T, H, NE, P, n_chunk_max, NH,
                           s);
}

}  // namespace moe
