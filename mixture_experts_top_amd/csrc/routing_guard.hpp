// Guards on caller-provided routing (expert_offsets, perm) before the kernels index with it.
//
// moe_top1_bwd and moe_top1_bwd_from_mean take expert_offsets and perm from the caller
// (normally the outputs of moe_top1_fwd for the same tokens).  The MHA wiring page
// ("9170d24fe3", BUG CAUGHT DURING WIRING block) records what happens when a launch is
// sized from numbers that do not match the buffers: reads past the end and a hard fault
// later.  The kernels therefore never index with these values as given:
//
//   * each offset is clamped to [0, T], and expert e's range starts at the running maximum
//     of the clamped offsets 0..e and ends at max(start, clamped offset e+1).  The ranges
//     are then disjoint, lie in [0, T) and their counts sum to at most T, so the tile and
//     chunk counts stay within the grid and workspace bounds the host computed from T;
//   * every token id read from perm is clamped to [0, T - 1].
//
// For routing that moe_top1_fwd wrote (0 = o_0 <= o_1 <= ... <= o_NE = T, perm a
// permutation of 0 .. T-1) both guards change nothing, so results are unaffected.  For other
// input the outputs are meaningless but every access stays inside the caller's buffers.
//
// The functions are constexpr (so also usable on the host, where a unit test checks them).
#pragma once

namespace moe {

// An offset clamped to [0, T].
constexpr int guard_offset(int v, int T) { return v < 0 ? 0 : (v > T ? T : v); }

// Expert range from its start (the running maximum of the clamped offsets up to its own)
// and its raw end offset: the count, never negative, never past T.
constexpr int guard_count(int start, int next_raw, int T) {
    const int n = guard_offset(next_raw, T);
    return n > start ? n - start : 0;
}

// A token id clamped to [0, T - 1] (T >= 1; one v_med3_i32 on the device).
constexpr int guard_token(int v, int T) { return v < 0 ? 0 : (v >= T ? T - 1 : v); }

}  // namespace moe
