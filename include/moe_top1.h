/*
 * moe_top1.h -- C ABI of the top-1 Mixture-of-Experts gate for AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the commit page "11b96dac6a  Top-1 Mixture-of-Experts
 * gate per Switch Transformer":
 *   - forward   (summary block, PERFORMANCE block): pick the top-1 expert of each
 *               (b, h) token's gate logits and apply that expert's [H, H] linear plus
 *               bias to fused_ctx, giving routed_ctx [B, N_H, H];
 *   - backward  (summary block, ARCHITECTURE block): gradients through the selected
 *               expert's W and bias only, giving d_W, d_b and d_fused_ctx; inactive
 *               experts get exactly zero and the gate gets nothing from this path;
 *               the per-token d_W / d_b contributions are collapsed over the token axis
 *               by a deterministic reduction with no atomics (the reduce_axis0 design of
 *               the perf-pass page "b23f8f2efa");
 *   - aux loss  (summary block): softmax of gate_logits and the load-balancing loss
 *               lambda * N_E * sum_e frac_e * mean_prob_e, with its gradient w.r.t. the
 *               gate logits (frac, a count, is held constant).
 *
 * Notation: T = B * N_H tokens, token t = b * N_H + h.  All tensors are dense,
 * row-major and contiguous:
 *   fused_ctx, routed_ctx, d_routed_ctx, d_fused_ctx   [B, N_H, H]       act dtype
 *   gate_logits, d_gate_logits, probs                  [B, N_H, N_E]     fp32
 *   W                                                  [N_E, H_out, H_in] act dtype (y = W x)
 *   b                                                  [N_E, H]          fp32
 *   d_W                                                [N_E, H, H]       fp32
 *   d_b, expert_counts, frac, mean_prob                [N_E]             fp32 / int32
 *   expert_idx, perm                                   [T]               int32
 *   expert_offsets                                     [N_E + 1]         int32
 * "act dtype" is fp32 (MOE_DTYPE_F32) or bf16 (MOE_DTYPE_BF16, stored as raw 16-bit
 * patterns; products are accumulated in fp32 and rounded to bf16, nearest even, on store).
 *
 * Ownership and execution.  Every pointer argument is a device pointer owned by the
 * caller (except size outputs, which are host pointers).  Calls only enqueue work on the
 * given HIP stream (NULL = the default stream) and return; they never allocate, free or
 * synchronise, keep no state between calls and read nothing back to the host, so they
 * may be captured into a HIP graph.  Buffers must stay valid until the stream has run
 * the call.  Two calls may run concurrently only with distinct workspaces and outputs.
 * Results are bitwise reproducible: every floating-point reduction has a fixed order and
 * no atomics are used.
 *
 * Errors.  Every argument is validated before anything is launched; on error nothing is
 * enqueued and the return value says why (moe_status_string, moe_last_error):
 *   MOE_ERR_INVALID_ARG  a required pointer is NULL or not 16-byte aligned, a size is
 *                        <= 0, T * max(H, N_E) >= 2^31, or lambda is not finite;
 *   MOE_ERR_UNSUPPORTED  H not in {64, 128, 256, 512}, N_E not in [1, 64], or an
 *                        unknown dtype;
 *   MOE_ERR_WORKSPACE    workspace is NULL or smaller than moe_workspace_bytes();
 *   MOE_ERR_HIP          a kernel launch failed (the HIP error text is in moe_last_error).
 * Launch extents are always derived by the library from (B, N_H, H, N_E), never taken
 * from the caller.
 */
#ifndef MOE_TOP1_H
#define MOE_TOP1_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE = 3,
    MOE_ERR_HIP = 4
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* Static text for a status code. */
const char* moe_status_string(int status);

/* Detail of the last error returned on the calling thread (static storage, thread-local). */
const char* moe_last_error(void);

/*
 * Workspace size in bytes (host-only; no device is touched).  One workspace of this size
 * serves moe_top1_route, moe_top1_fwd, moe_top1_bwd and moe_aux_loss for the same
 * (B, N_H, H, N_E, act).  The workspace holds routing histograms and the fixed-size
 * per-chunk partial sums of d_W / d_b; its contents need no initialisation and are
 * meaningless between calls.
 */
moe_status_t moe_workspace_bytes(int64_t B, int64_t NH, int64_t H, int64_t NE, int act,
                                 size_t* bytes_out);

/*
 * Routing half of the forward pass (summary and PERFORMANCE blocks of the MoE-gate page:
 * the top-1 expert of each token's gate logits).
 *   expert_idx[t]     argmax_e gate_logits[t, e]; on equal logits the lowest e wins.
 *   expert_counts[e]  number of tokens routed to e.
 *   expert_offsets    exclusive prefix sum of expert_counts, [0, c_0, c_0+c_1, ..., T].
 *   perm              the tokens of expert 0, then of expert 1, ..., each group in
 *                     ascending token order (a stable counting sort by expert).
 * All four outputs are overwritten; integers are exact.
 */
moe_status_t moe_top1_route(const float* gate_logits, int32_t* expert_idx, int32_t* expert_counts,
                            int32_t* expert_offsets, int32_t* perm,
                            int64_t B, int64_t NH, int64_t NE,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward pass (summary block of the MoE-gate page): moe_top1_route, then
 *   routed_ctx[t, :] = W[e*(t)] @ fused_ctx[t, :] + b[e*(t)]
 * for every token (no capacity limit, no scaling by the gate probability).
 * routed_ctx is overwritten; the routing outputs are as for moe_top1_route and are the
 * inputs of moe_top1_bwd and moe_aux_loss.
 */
moe_status_t moe_top1_fwd(const void* fused_ctx, const float* gate_logits, const void* W,
                          const float* b, void* routed_ctx,
                          int32_t* expert_idx, int32_t* expert_counts, int32_t* expert_offsets,
                          int32_t* perm,
                          int64_t B, int64_t NH, int64_t H, int64_t NE, int act,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_top1_fwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same operation, outputs and kernels as moe_top1_fwd, bit for bit.  Its scratch (the routing
 * histograms and block bases, 2 * ceil(T / 256) * N_E int32, each part rounded up to 256
 * bytes) lives in an 8 MiB device array inside the library, one per device, held from the
 * first call on that device until the process ends; that first call looks up the array's
 * address (hipGetSymbolAddress: no allocation) and should be made before any graph capture.
 * The call allocates and frees nothing.  Every call on one device uses that device's one
 * array, so calls that may overlap on a device (different streams, different host threads)
 * race: serialise them.  Shapes whose scratch exceeds the array (ceil(T / 256) * N_E above
 * about one million entries) return MOE_ERR_WORKSPACE before anything is launched; other
 * errors as moe_top1_fwd.
 */
moe_status_t moe_top1_fwd_noalloc(const void* fused_ctx, const float* gate_logits, const void* W,
                                  const float* b, void* routed_ctx,
                                  int32_t* expert_idx, int32_t* expert_counts, int32_t* expert_offsets,
                                  int32_t* perm,
                                  int64_t B, int64_t NH, int64_t H, int64_t NE, int act, void* stream);

/*
 * Backward pass (summary and ARCHITECTURE blocks of the MoE-gate page), given the
 * expert_offsets and perm written by moe_top1_fwd for the same tokens:
 *   d_fused_ctx[t, :] = W[e*(t)]^T @ d_routed_ctx[t, :]      (overwritten, or added to
 *                                                              the existing contents when
 *                                                              accumulate_dx != 0)
 *   d_W[e] = sum_{t : e*(t) = e} d_routed_ctx[t, :]^T (outer) fused_ctx[t, :]  (overwritten)
 *   d_b[e] = sum_{t : e*(t) = e} d_routed_ctx[t, :]                            (overwritten)
 * expert_offsets and perm are read under guards (each offset clamped to [0, T] and the list
 * made non-decreasing; each token id clamped to [0, T - 1]; see the MHA wiring page
 * "9170d24fe3", BUG CAUGHT DURING WIRING block), so routing that does not belong to these
 * tokens gives meaningless results but no access outside the caller's buffers; routing from
 * moe_top1_fwd is unchanged by them.
 * Experts with no tokens get d_W[e] = d_b[e] = +0.0 exactly.  The token sums are taken
 * per fixed-size chunk of each expert's tokens and the chunk partials are then summed
 * in chunk order (no atomics), so the result depends only on the inputs and the shape.
 * The gate logits get no gradient here.
 */
moe_status_t moe_top1_bwd(const void* d_routed_ctx, const void* fused_ctx, const void* W,
                          const int32_t* expert_offsets, const int32_t* perm,
                          void* d_fused_ctx, float* d_W, float* d_b, int accumulate_dx,
                          int64_t B, int64_t NH, int64_t H, int64_t NE, int act,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Load-balancing aux loss (summary block of the MoE-gate page; softmax in the max-shifted
 * form of the softmax/cross-entropy page "6cfd7e6691"):
 *   p[t, :]       = softmax(gate_logits[t, :])
 *   frac[e]       = expert_counts[e] / T
 *   mean_prob[e]  = (1/T) sum_t p[t, e]
 *   loss          = lambda * N_E * sum_e frac[e] * mean_prob[e]
 *   d_gate_logits[t, j] = (lambda * N_E / T) * p[t, j] * (frac[j] - sum_e frac[e] p[t, e])
 * expert_counts comes from moe_top1_fwd; pass NULL to have it recomputed from the logits.
 * loss [1] and d_gate_logits are written on the device; frac, mean_prob and probs are
 * optional outputs (NULL = not written).
 */
moe_status_t moe_aux_loss(const float* gate_logits, const int32_t* expert_counts, float lambda,
                          float* loss, float* d_gate_logits,
                          float* frac, float* mean_prob, float* probs,
                          int64_t B, int64_t NH, int64_t NE,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Adaptive load-balancing weight, on the device (adaptive-lambda page "2d0e6b6bdc", formula
 * and wiring blocks): a single-thread launch computing
 *   lambda_eff[0] = lambda_floor + lambda_max_extra * max(0, target - ent_ema[0]) / target,
 *   target = entropy_target_frac * ln(N_E),
 * so that moe_aux_loss_lambda_dev can read the weight from device memory with no
 * device-to-host read.  The page's knobs are floor 0.01, max extra 0.09, target fraction 0.7.
 * ent_ema [1] and lambda_eff [1] are fp32 device pointers (4-byte aligned); N_E in [2, 64];
 * the knobs must be finite and the target fraction positive, else MOE_ERR_INVALID_ARG.
 * How ent_ema is produced is up to the caller (the pages do not specify it).
 */
moe_status_t moe_lambda_eff_update(const float* ent_ema, float lambda_floor, float lambda_max_extra,
                                   float entropy_target_frac, int64_t NE, float* lambda_eff, void* stream);

/*
 * moe_aux_loss with lambda read from device memory (lambda_dev [1], fp32, e.g. the output of
 * moe_lambda_eff_update) when the kernels run.  Same outputs, errors and workspace as
 * moe_aux_loss; bitwise equal to it for the same lambda value.
 */
moe_status_t moe_aux_loss_lambda_dev(const float* gate_logits, const int32_t* expert_counts,
                                     const float* lambda_dev, float* loss, float* d_gate_logits,
                                     float* frac, float* mean_prob, float* probs,
                                     int64_t B, int64_t NH, int64_t NE,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward pass and load-balancing aux loss in one call (summary block of the MoE-gate page:
 * the aux loss needs only the gate logits and the routing counts, so it can be formed as
 * soon as the routing is done).  Outputs are those of moe_top1_fwd followed by
 * moe_aux_loss (lambda_dev == NULL) or by moe_aux_loss_lambda_dev (lambda_dev != NULL;
 * `lambda` is then ignored) on the expert_counts just written -- bit for bit, whichever
 * way the library schedules the work.  For fp32 activations, N_E <= 8 and small T the
 * softmax column sums ride on the routing launch and dG / frac / mean_prob / loss on the
 * forward GEMM launch (two launches in all); otherwise, for N_E <= 16, the column sums ride
 * on the routing launch and dG / frac / mean_prob / loss on the scatter launch that forms
 * perm; for N_E > 16 the calls run one after the other.
 * Workspace as moe_top1_fwd.  Errors as moe_top1_fwd and moe_aux_loss; lambda_dev, when
 * given, must be 4-byte aligned.
 */
moe_status_t moe_top1_fwd_aux(const void* fused_ctx, const float* gate_logits, const void* W,
                              const float* b, void* routed_ctx,
                              int32_t* expert_idx, int32_t* expert_counts, int32_t* expert_offsets,
                              int32_t* perm, float lambda, const float* lambda_dev,
                              float* loss, float* d_gate_logits, float* frac, float* mean_prob,
                              float* probs,
                              int64_t B, int64_t NH, int64_t H, int64_t NE, int act,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * reduce_axis0 (perf-pass page "b23f8f2efa", reduce_axis0 entry; MHA page "9170d24fe3",
 * trainer and BUG blocks): out[j] = sum_{r < n_batch} in[r * n_tail + j] for j < n_tail, fp32,
 * with a fixed summation order and no atomics (bitwise reproducible for a shape).  The rows
 * are split into a number of fixed chunks that depends only on (n_batch, n_tail); their
 * partial sums live in the workspace (moe_reduce_axis0_workspace_bytes; may be 0 bytes, and
 * then workspace may be NULL).  When n_tail % 4 == 0, in and out must be 16-byte aligned,
 * else 4-byte aligned.  out is overwritten; in is not modified.
 */
moe_status_t moe_reduce_axis0_workspace_bytes(int64_t n_batch, int64_t n_tail, size_t* bytes_out);
moe_status_t moe_reduce_axis0(const float* in, int64_t n_batch, int64_t n_tail, float* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Horizon mean collapse (MHA page "9170d24fe3", new-kernel block) and its backward:
 *   fwd: ctx_mean[b, :] = (sum_h x[b, h, :]) * (1/N_H)        x [B, N_H, H] -> [B, H]
 *   bwd: d_x[b, h, :]   = d_ctx_mean[b, :] * (1/N_H)          [B, H] -> [B, N_H, H]
 * (1/N_H is the fp32 reciprocal; horizons are summed in order h = 0..N_H-1.)  act as for the
 * gate; H must be a multiple of 4 (fp32) or 8 (bf16); 16-byte aligned pointers.
 */
moe_status_t moe_horizon_mean_collapse_fwd(const void* x, void* ctx_mean, int64_t B, int64_t NH,
                                           int64_t H, int act, void* stream);
moe_status_t moe_horizon_mean_collapse_bwd(const void* d_ctx_mean, void* d_x, int64_t B, int64_t NH,
                                           int64_t H, int act, void* stream);

/*
 * moe_top1_bwd with the horizon mean collapse folded into its input (MHA page "9170d24fe3",
 * new-kernel block): instead of d_routed_ctx [B, N_H, H] it takes d_ctx_mean [B, H] (act
 * dtype: fp32, or bf16 for bf16 activations) and uses
 *   d_routed_ctx[b, h, :] = d_ctx_mean[b, :] * (1/N_H)      (bf16: rounded to bf16, nearest even)
 * while staging the GEMM operands, so d_routed_ctx is never written or read.  Outputs,
 * workspace and errors as moe_top1_bwd; bitwise equal to moe_horizon_mean_collapse_bwd
 * followed by moe_top1_bwd, in either dtype.
 */
moe_status_t moe_top1_bwd_from_mean(const void* d_ctx_mean, const void* fused_ctx, const void* W,
                                    const int32_t* expert_offsets, const int32_t* perm,
                                    void* d_fused_ctx, float* d_W, float* d_b, int accumulate_dx,
                                    int64_t B, int64_t NH, int64_t H, int64_t NE, int act,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Softmax + cross-entropy gradient head (softmax/cross-entropy page "6cfd7e6691", kernel
 * block), per (b, h) row of A atom logits (A in [1, 64]; the page uses 21):
 *   p = softmax(logits[b, h, :]) (max-shifted), ce[b, h] = -log(max(p[label], 1e-30)),
 *   grad[b, h, :] = (p - onehot(label)) * (1/B)
 * label = labels[b, h]; a label of -1 (sentinel), or any label outside [0, A), gives
 * ce = 0 and a zero gradient row.  logits, grad [B, N_H, A] fp32; labels [B, N_H] int32;
 * ce [B, N_H] fp32; 4-byte aligned.  Scaling / summing the loss is left to the caller.
 */
moe_status_t moe_softmax_ce_grad(const float* logits, const int32_t* labels, float* grad, float* ce,
                                 int64_t B, int64_t NH, int64_t A, void* stream);

/*
 * Instrumentation.  While set, every launch of kernel `kernel_id` (MOE_KERNEL_*) made by
 * the calls above carries ev_start and ev_stop, which the command processor records at the
 * kernel's own start and end (hipExtLaunchKernelGGL), so their difference is the kernel's
 * duration.  A call that does not launch that kernel leaves the events untouched.  The
 * events are hipEvent_t handles created by the caller.  Pass kernel_id < 0 to clear.
 * Process-wide setting; not thread-safe against concurrent calls.
 */
enum {
    MOE_KERNEL_ROUTE = 0,        /* argmax + per-block histogram */
    MOE_KERNEL_SCAN = 1,         /* counts, offsets, per-block bases (large inputs) */
    MOE_KERNEL_SCATTER = 2,      /* stable perm (small inputs: with the scan folded in) */
    MOE_KERNEL_FWD_GEMM = 3,     /* grouped forward GEMM + bias */
    MOE_KERNEL_BWD_GEMM = 4,     /* grouped dX GEMM and d_W / d_b chunk partials, one launch */
    MOE_KERNEL_REDUCE = 5,       /* deterministic chunk reduction -> d_W, d_b */
    MOE_KERNEL_AUX = 6,          /* softmax, dG, per-block column sums of p */
    MOE_KERNEL_AUX_FINAL = 7,    /* mean_prob, frac, loss */
    MOE_KERNEL_W_TRANSPOSE = 8,  /* reserved: no kernel of this id is launched any more */
    MOE_KERNEL_LAMBDA = 9,       /* adaptive lambda update */
    MOE_KERNEL_REDUCE_AXIS0 = 10,/* standalone reduce_axis0 */
    MOE_KERNEL_COLLAPSE = 11,    /* horizon mean collapse, forward or backward */
    MOE_KERNEL_SOFTMAX_CE = 12,  /* softmax + cross-entropy gradient head */
    MOE_KERNEL_COUNT = 13
};
moe_status_t moe_set_launch_timer(int kernel_id, void* ev_start, void* ev_stop);

/* Name of a MOE_KERNEL_* id (static text), NULL if out of range. */
const char* moe_kernel_name(int kernel_id);

/*
 * Calibration probes (not part of the gate): what this chip delivers, against the
 * spec-sheet peaks that roofline fractions divide by.  Both only enqueue on `stream`.
 *
 * moe_probe_mfma: `workgroups` workgroups of 256 threads (4 wavefronts); each wavefront
 *   issues `iters` rounds of four independent MFMA chains -- act MOE_DTYPE_F32:
 *   v_mfma_f32_32x32x2_f32 (4,096 flops each), MOE_DTYPE_BF16: v_mfma_f32_32x32x16_bf16
 *   (32,768 flops each) -- so a call performs workgroups * 4 * iters * 4 * (flops per
 *   instruction) flops.  Writes one checksum per thread, sink [workgroups * 256] fp32, and
 *   for each workgroup the shader-clock and constant-clock ticks its first wavefront spent
 *   in the loop, ticks [workgroups][2] int64 (clock64, wall_clock64: their ratio times the
 *   constant clock's rate, hipDeviceAttributeWallClockRate, is the shader clock).
 *   workgroups in [1, 2^20], iters > 0; sink 4-byte and ticks 8-byte aligned.
 * moe_probe_copy: dst[0 .. bytes) = src[0 .. bytes) (the STREAM copy: 16-byte loads and
 *   stores); both 16-byte aligned, bytes a positive multiple of 16, no overlap.
 * Errors: MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED as above, MOE_ERR_HIP on a failed launch.
 */
moe_status_t moe_probe_mfma(int act, int64_t workgroups, int64_t iters, float* sink, int64_t* ticks, void* stream);
moe_status_t moe_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_TOP1_H */
