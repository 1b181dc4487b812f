/*
 * zo.h -- C ABI of the 1.5-SPSA perturb / probe-weight / update library (libzo.so),
 * hand-written HIP kernels for gfx950 (MI355X).
 *
 * The method ("Probe-Space Preconditioning for Fast and Stable Zero-Order Training",
 * described on "Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation"): each step
 * draws n_pert Rademacher probes z_i, evaluates the loss at the clean parameters and at
 * theta +/- eps*z_i (in place, inference mode), turns the 2*n_pert + 1 losses into one
 * weight c_i per probe, and moves theta <- theta - eta * sum_i c_i z_i.
 *
 * Conventions shared by every call
 *  - Parameters are one flat buffer of n elements, fp32 or bf16, in device memory, that
 *    holds the global parameter indices [offset, offset + n).  offset must be a multiple
 *    of 128; a model kept in several buffers gets, per buffer, the same probe bits as one
 *    flat buffer when each buffer is passed with its global offset.
 *  - Probe signs are counter-based: z_j of probe p at step t under seed s is bit
 *    (j mod 32) of word (j / 32) mod 4 of Philox4x32-10 (Salmon et al., SC'11) with
 *    counter (blk_lo, blk_hi, p, t), blk = j / 128, and key (s_lo, s_hi); bit 1 means +1,
 *    bit 0 means -1.  Nothing has to be stored: every call can regenerate the signs.
 *  - A packed probe row ("plane") holds the signs of one probe over [offset, offset+n):
 *    zo_bits_stride(n) bytes, byte m = params offset + 8m .. 8m+7, least significant bit
 *    first (the four Philox words of each 128-param block, little-endian).  Bits past n in
 *    the last block are Philox bits and are never applied.
 *  - Every compute call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  The caller owns every buffer; hot-path calls allocate nothing.  The step's
 *    calls (zo_perturb, zo_perturb2, zo_probe_weights, zo_update, zo_restore_update) only
 *    launch kernels -- no allocation, host synchronisation, attribute call or memset node
 *    (counters are cleared by a kernel) -- so they can be recorded into a HIP graph and
 *    replayed, at every probe count up to ZO_MAX_NPERT and with regenerated or stored
 *    signs.  zo_nonfinite_count and zo_tune_placement synchronise and cannot.
 *  - Return values report argument and launch errors only: ZO_EINVAL is returned before
 *    anything is launched, ZO_EHIP when the HIP runtime reports an error.  Numeric
 *    trouble is not an error (see zo_probe_weights).  n == 0 (or n_pert == 0) is a
 *    valid empty call that launches nothing and returns ZO_OK.
 *  - Threading: one host thread uses a context at a time.  Calls on different streams
 *    that touch the same parameter buffer race, as any two kernels would.  The quadratic
 *    loss calls (zo_quad_loss, zo_quad_loss_probes, zo_lowrank_quad_loss) stage partial
 *    sums in a scratch buffer owned by the context: two of them on one context must not overlap on
 *    different streams (the non-finite counter is updated atomically and may be shared).
 *  - Devices: a context belongs to the device that was current at zo_init; every call
 *    on it must be made with that device current, or it returns ZO_EINVAL.
 *  - Measurement and placement knobs that are not steps of the method (the in-place
 *    streaming diagnostic, the per-buffer choice between one launch and slices per pass)
 *    are declared in zo_placement.h.
 *  - Launch shapes: ZO_UPDATE_WG_PER_CU (default 16) overrides the workgroups per CU of the
 *    update kernel, accepted in [1, 64]; ZO_UPDATE_GENERIC=1 makes the update use its
 *    general kernel at every probe count; ZO_MLP_PROBES_PER_WAVE (default 2; 1, 2, 4 or 8)
 *    sets the probes per wave of zo_mlp_loss_probes.  Each is read once per process, and
 *    results do not depend on them.  The passes over the parameters (zo_perturb,
 *    zo_perturb2, zo_stream_rmw) and the plane generator run one chunk per wave in a
 *    non-persistent grid.
 */
#ifndef ZO_H
#define ZO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct zo_ctx zo_ctx;

typedef enum {
    ZO_OK = 0,
    ZO_EINVAL = 1,        /* bad argument; nothing was launched */
    ZO_EHIP = 2,          /* the HIP runtime reported an error */
    ZO_ENOMEM = 3,        /* host or device allocation failed (zo_init only) */
    ZO_EUNSUPPORTED = 4   /* valid request beyond a documented limit */
} zo_status;

typedef enum { ZO_FP32 = 0, ZO_BF16 = 1 } zo_dtype;

/* Largest n_pert one zo_update call accepts (its sign tables live in LDS). */
#define ZO_MAX_NPERT 512u

/* Device scratch of zo_mlp_loss_pair_noalloc, one static array per GPU (1 MiB). */
#define ZO_NOALLOC_SCRATCH_BYTES (1u << 20)

/* Create a context for probe seed `seed` on the current HIP device.  Allocates the host
 * context and a small device area (the non-finite counter and reduction partials), looks
 * up this device's copy of the library's static scratch, and raises the update kernel's
 * dynamic-LDS limit on this device (so that no later call makes a runtime call besides its
 * launches).  Errors: ZO_EINVAL if out is NULL; ZO_ENOMEM / ZO_EHIP if an allocation or
 * runtime call fails (for example when no GPU is present).  *out is set only on success. */
zo_status zo_init(uint64_t seed, zo_ctx **out);

/* Release a context (NULL is allowed).  Synchronizes the device first. */
zo_status zo_destroy(zo_ctx *ctx);

/* The seed the context was created with. */
uint64_t zo_get_seed(const zo_ctx *ctx);

/* Static description of a status code; never NULL. */
const char *zo_strerror(zo_status status);

/* Bytes of one packed probe row over n parameters: ceil(n / 128) * 16. */
size_t zo_bits_stride(uint64_t n);

/* Probe generator (the packed-bit generator of the abstract of "Probe-Space
 * Preconditioning for Fast and Stable Zero-Order Training"; probes z_i of "How 1.5-SPSA
 * Works").  Writes n_probes consecutive rows for probes probe0 .. probe0+n_probes-1 of
 * step `step` over params [offset, offset+n): row r at d_bits + r*zo_bits_stride(n).
 * d_bits: device, 16-byte aligned, n_probes*zo_bits_stride(n) bytes, written in full.
 * Errors (ZO_EINVAL): ctx or d_bits NULL (with work to do), offset % 128 != 0,
 * d_bits misaligned, offset + n beyond 2^64 - 1. */
zo_status zo_gen_probes(zo_ctx *ctx, uint32_t step, uint32_t probe0, uint32_t n_probes,
                        uint64_t offset, uint64_t n, uint8_t *d_bits, void *stream);

/* In-place perturbation theta_j <- round(theta_j + alpha * z_j) of probe `probe` at
 * `step` ("How 1.5-SPSA Works": losses at theta +/- eps*z_i; the abstract: in place,
 * fused unpack/apply).  fp32: one IEEE add, round to nearest even.  bf16: widen to fp32,
 * one fp32 add, round to nearest even back to bf16.  Restoring is the same call with
 * -alpha.  d_bits NULL regenerates the signs; otherwise it is this probe's packed row
 * over the same [offset, offset+n) (device, 16-byte aligned).
 * d_theta: device, 16-byte aligned, n elements of `dtype`.
 * Errors (ZO_EINVAL): ctx or d_theta NULL (with n > 0), unknown dtype, offset % 128 != 0,
 * misaligned pointers, offset + n beyond 2^64 - 1. */
zo_status zo_perturb(zo_ctx *ctx, void *d_theta, zo_dtype dtype, uint64_t offset,
                     uint64_t n, uint32_t step, uint32_t probe, float alpha,
                     const uint8_t *d_bits, void *stream);

/* Two probes in one in-place pass: theta_j <- round(theta_j + d_j) with
 * d_j = (+/-alpha_a) + (+/-alpha_b) added in fp32 (exact when |alpha_a| == |alpha_b|),
 * then the same add and nearest-even narrow as zo_perturb.  It fuses the restore of
 * probe a (alpha_a = +eps after its -eps point) with the +eps move of probe b, so that a
 * step visits every theta +/- eps*z_i ("How 1.5-SPSA Works") in two passes per probe
 * instead of four; with alpha_b = 0 it is zo_perturb of probe a.
 * d_bits_a / d_bits_b: both NULL (regenerate) or both the probes' packed rows.
 * Errors (ZO_EINVAL): as zo_perturb, or exactly one of the two rows given. */
zo_status zo_perturb2(zo_ctx *ctx, void *d_theta, zo_dtype dtype, uint64_t offset,
                      uint64_t n, uint32_t step, uint32_t probe_a, float alpha_a,
                      uint32_t probe_b, float alpha_b, const uint8_t *d_bits_a,
                      const uint8_t *d_bits_b, void *stream);

/* Probe weights ("How 1.5-SPSA Works" for the central difference; "Probe-Space
 * Preconditioning" for the clean-pass curvature weight), computed in fp64:
 *   g_i = (L+_i - L-_i) / (2 eps),   h_i = ((L+_i + L-_i) - 2 L0) / eps^2,
 *   c_i = g_i / max(|h_i|, delta), rounded once to fp32.
 * eps must be the step actually applied (the fp32 alpha of zo_perturb, widened).
 * A probe with a non-finite L+_i, L-_i or L0 gets c_i = 0 and adds 1 to the context's
 * device counter (read it with zo_nonfinite_count).
 * d_Lp, d_Lm: device, n_pert doubles; d_L0: device, one double; d_c: device, n_pert
 * floats (written).  Errors (ZO_EINVAL): NULL ctx or pointers (with n_pert > 0),
 * eps not finite or zero, delta negative or not finite. */
zo_status zo_probe_weights(zo_ctx *ctx, const double *d_Lp, const double *d_Lm,
                           const double *d_L0, uint32_t n_pert, double eps, double delta,
                           float *d_c, void *stream);

/* Weight forms for zo_probe_weights_ex. */
typedef enum {
    ZO_WEIGHTS_PRECOND = 0,   /* c_i = g_i / max(|h_i|, delta)        (zo_probe_weights) */
    ZO_WEIGHTS_POWER = 1,     /* c_i = g_i / max(|h_i|, delta)^power                      */
    ZO_WEIGHTS_SPSA_MEAN = 2  /* c_i = g_i / n_pert, no clean loss                        */
} zo_weights_mode;

/* The other probe-weight forms of the pages, in fp64 with one rounding to fp32:
 * ZO_WEIGHTS_POWER is the curvature-power weighting of "Probe-Space Preconditioning" (a
 * weight |curvature|^alpha from the clean and perturbed losses that shrinks high-curvature
 * probes; the page's alpha is 0.1; power = 1 is ZO_WEIGHTS_PRECOND, 0 the plain central
 * difference).  ZO_WEIGHTS_SPSA_MEAN is the plain 1SPSA estimator of "How 1.5-SPSA Works"
 * averaged over the probes (no clean pass; d_L0 is not read and may be NULL).  Non-finite
 * losses that a mode reads drop the probe (c_i = 0, counter + 1) as in zo_probe_weights.
 * Errors (ZO_EINVAL): as zo_probe_weights, an unknown mode, or power negative or not finite
 * (ZO_WEIGHTS_POWER).  delta is not read by ZO_WEIGHTS_SPSA_MEAN. */
zo_status zo_probe_weights_ex(zo_ctx *ctx, const double *d_Lp, const double *d_Lm,
                              const double *d_L0, uint32_t n_pert, double eps, double delta,
                              zo_weights_mode mode, double power, float *d_c, void *stream);

/* Multi-probe update theta_j <- round(theta_j - eta * s_j), s_j = sum_i c_i z_ij over
 * probes 0 .. n_pert-1 of `step` (the update box of the ZOO loop flowchart in
 * "Pretraining Transformers Without Backprop: What Two Zero-Order Papers Actually
 * Measure").  Each parameter is read and written once.  s_j is accumulated in fp64
 * through per-8-probe tables of signed partial sums (probes in ascending order within a
 * table, tables in ascending order); then t = (double)theta_j - (double)eta * s_j is
 * rounded once, to nearest even, to the storage type (fp32, or bf16 directly from the
 * double).  The result is deterministic (independent of launch geometry).
 * d_c: device, n_pert floats.  d_bits NULL regenerates; otherwise n_pert packed rows of
 * zo_bits_stride(n) bytes (device, 16-byte aligned), row i = probe i.
 * Errors: ZO_EINVAL as for zo_perturb, or d_c NULL (with n_pert > 0);
 * ZO_EUNSUPPORTED if n_pert > ZO_MAX_NPERT. */
zo_status zo_update(zo_ctx *ctx, void *d_theta, zo_dtype dtype, uint64_t offset,
                    uint64_t n, uint32_t step, const float *d_c, uint32_t n_pert,
                    float eta, const uint8_t *d_bits, void *stream);

/* zo_perturb(restore_probe, restore_alpha) followed by zo_update, in one pass over the
 * parameters -- the restore after the last probe's evaluations ("How 1.5-SPSA Works" on
 * "Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation": parameters moved in place
 * to theta +/- eps*z_i and back) and the update box of the ZOO loop flowchart ("Pretraining
 * Transformers Without Backprop: What Two Zero-Order Papers Actually Measure"):
 *   theta_j <- round(round(theta_j + restore_alpha * z_{restore_probe,j})
 *                    - eta * sum_i c_i z_ij),
 * each rounding exactly the one the two calls make, so the result equals the two calls bit
 * for bit.  This is the last restore of the two-moves-per-probe
 * schedule folded into the update that follows it (the probe weights between them read
 * only the losses), saving one full pass per step; the restore probe's signs come from the
 * update's own sign generation at general probe counts, and at the probe counts where the
 * update runs unrolled (16, 32, 64, 160) from one extra Philox call per lane, i.e. eight
 * extra calls per 128-param block (the eight lanes sharing a block each make one).
 * Arguments as zo_update, plus restore_probe (< n_pert, a
 * probe of the same step; with d_bits, its row is used) and restore_alpha (fp32).
 * Errors: as zo_update, and ZO_EINVAL if restore_probe >= n_pert. */
zo_status zo_restore_update(zo_ctx *ctx, void *d_theta, zo_dtype dtype, uint64_t offset,
                            uint64_t n, uint32_t step, uint32_t restore_probe,
                            float restore_alpha, const float *d_c, uint32_t n_pert, float eta,
                            const uint8_t *d_bits, void *stream);

/* Read the non-finite-probe counter: synchronizes `stream`, then copies it to *out. */
zo_status zo_nonfinite_count(zo_ctx *ctx, void *stream, uint32_t *out);

/* Zero the non-finite-probe counter (asynchronous on `stream`, a small fill kernel). */
zo_status zo_reset_nonfinite(zo_ctx *ctx, void *stream);

/* Diagonal quadratic loss L = 1/2 sum_j a_j theta_j^2, accumulated in fp64, written to
 * d_out (one double).  Stand-in for the model's forward pass ("N forward passes" box of
 * the ZOO loop flowchart) on the synthetic quadratic workloads.  Deterministic: fixed
 * partition into partial sums, reduced in a fixed order.
 * d_theta: device, n elements of dtype, 16-byte aligned; d_a: device, n floats, 16-byte
 * aligned.  Errors (ZO_EINVAL): NULL pointers (with n > 0), unknown dtype, misalignment.
 * n == 0 writes 0. */
zo_status zo_quad_loss(zo_ctx *ctx, const void *d_theta, zo_dtype dtype, const float *d_a,
                       uint64_t n, double *d_out, void *stream);

/* Both losses of n_probes consecutive probes of the same quadratic with each probe applied
 * while theta is read (the perturbation-fused forward of the flowchart's "N forward passes"
 * box for this workload, "Pretraining Transformers Without Backprop: What Two Zero-Order
 * Papers Actually Measure"; the central difference of "How 1.5-SPSA Works" on "Stanford's
 * 1.5-SPSA Trains OPT-30B Without Backpropagation"): d_out_plus[i] = L(theta + alpha z_i) and
 * d_out_minus[i] = L(theta - alpha z_i), i = probe0 + 0 .. n_probes-1, where each perturbed
 * element is the value zo_perturb(+/-alpha) would store from the given theta (one fp32 add;
 * bf16: widen, add, round to nearest even).  theta is read once per four probes and never
 * written; each loss equals zo_perturb followed by zo_quad_loss bit for bit (same partition,
 * order of terms and reductions).  Layouts as zo_quad_loss; offset as zo_perturb (a multiple
 * of 128: the global index of theta[0]); d_bits: NULL to regenerate the signs, else
 * n_probes packed rows of zo_bits_stride(n) bytes each (row i for probe probe0 + i), 16-byte
 * aligned; d_out_plus, d_out_minus: device, n_probes doubles each.  d_out_clean: NULL, or
 * one device double that also receives the loss at theta itself (the step's clean pass),
 * equal bit for bit to zo_quad_loss, summed in the first pass over theta instead of a pass
 * of its own.  Uses the context's loss partials, so calls on one context are ordered by
 * their streams.  Errors (ZO_EINVAL): as zo_quad_loss, offset % 128 != 0 or range overflow,
 * probe indices wrapping past 2^32, misaligned d_bits, NULL outputs (with n_probes > 0).
 * n_probes == 0 computes only the clean loss (nothing without d_out_clean); n == 0 writes
 * zeros. */
zo_status zo_quad_loss_probes(zo_ctx *ctx, const void *d_theta, zo_dtype dtype,
                              const float *d_a, uint64_t offset, uint64_t n, uint32_t step,
                              uint32_t probe0, uint32_t n_probes, float alpha,
                              const uint8_t *d_bits, double *d_out_plus, double *d_out_minus,
                              double *d_out_clean, void *stream);

/* Low-rank-plus-diagonal quadratic loss L = 1/2 sum_j a_j theta_j^2 + 1/2 ||U theta||^2,
 * fp64 accumulation, deterministic.  A synthetic model whose curvature along a probe,
 * sum_j a_j + ||U z||^2, differs from probe to probe -- the landscape on which the clean-pass
 * preconditioner is said to pay off with the condition number ("Probe-Space
 * Preconditioning" on "Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation").
 * d_U: device fp32, r rows of n (row-major, each row contiguous), 16-byte aligned; r = 0
 * gives the diagonal loss.  Errors: ZO_EINVAL as zo_quad_loss or d_U NULL/misaligned with
 * r > 0; ZO_EUNSUPPORTED if r > 16. */
zo_status zo_lowrank_quad_loss(zo_ctx *ctx, const void *d_theta, zo_dtype dtype,
                               const float *d_a, const float *d_U, uint32_t r, uint64_t n,
                               double *d_out, void *stream);

/* Loss of a two-layer MLP classifier -- the model forward of the ZOO loop ("N forward
 * passes, loss only" box of the flowchart in "Pretraining Transformers Without Backprop:
 * What Two Zero-Order Papers Actually Measure") for the small real-model workload:
 *   loss = mean_b [ logsumexp(z_b) - z_b[label_b] ],  z = GELU(X W1^T + b1) W2^T + b2,
 * GELU in its exact erf form.  d_params: device fp32, flat W1 [d_hid x d_in] row-major,
 * b1 [d_hid], W2 [d_out x d_hid] row-major, b2 [d_out], 16-byte aligned.  d_X: device fp32
 * [batch x d_in] row-major, 16-byte aligned.  d_labels: device int64 [batch], each in
 * [0, d_out) (an out-of-range label makes the loss NaN).  The GEMM runs on MFMA in fp32;
 * the partial logits and the cross-entropy are reduced in fp64 in a fixed order
 * (deterministic).  The GEMM's tiles are 32 x 32 where batch and d_hid are multiples of 32,
 * 16 x 16 otherwise, in every MLP entry point alike, so that the entry points agree bit for
 * bit at any one shape.  d_workspace: device, 8-byte aligned, at least
 * zo_mlp_workspace_bytes(...) bytes (enough for every MLP call, zo_mlp_loss_pair
 * included), owned by the caller.  d_loss: device, one double.
 * Limits: batch, d_in, d_hid multiples of 16; 1 <= d_out <= 16.
 * Errors (ZO_EINVAL): NULL pointers, shapes outside the limits, misalignment, a workspace
 * that is too small. */
uint64_t zo_mlp_workspace_bytes(uint32_t batch, uint32_t d_in, uint32_t d_hid,
                                uint32_t d_out);
zo_status zo_mlp_loss(zo_ctx *ctx, const float *d_params, const float *d_X,
                      const int64_t *d_labels, uint32_t batch, uint32_t d_in, uint32_t d_hid,
                      uint32_t d_out, void *d_workspace, uint64_t workspace_bytes,
                      double *d_loss, void *stream);

/* The same loss at theta + alpha * z_probe without touching theta: every parameter is
 * read as theta_j + (+/-alpha) in fp32 -- exactly the value zo_perturb would store -- so the
 * result equals zo_perturb followed by zo_mlp_loss, bit for bit, and a step's 2*n_pert
 * perturbed losses need no pass over the parameters.  offset: global index of
 * d_params[0] (multiple of 128); d_bits: NULL (regenerate) or the probe's packed row over
 * the parameters.  Other arguments and errors as zo_mlp_loss. */
zo_status zo_mlp_loss_perturbed(zo_ctx *ctx, const float *d_params, uint64_t offset,
                                uint32_t step, uint32_t probe, float alpha,
                                const uint8_t *d_bits, const float *d_X,
                                const int64_t *d_labels, uint32_t batch, uint32_t d_in,
                                uint32_t d_hid, uint32_t d_out, void *d_workspace,
                                uint64_t workspace_bytes, double *d_loss, void *stream);

/* Both losses of one probe, at theta + alpha * z_probe (into d_loss_plus) and at
 * theta - alpha * z_probe (into d_loss_minus), in one launch sequence: each parameter is
 * loaded once and read with both signs.  Each result equals zo_mlp_loss_perturbed with
 * +alpha resp. -alpha bit for bit (the two accumulations are independent and ordered as
 * in the single call), so a step's central differences cost n_pert forward launches
 * instead of 2*n_pert.  d_loss_plus, d_loss_minus: device, one double each.  Other
 * arguments as zo_mlp_loss_perturbed; errors as there, plus ZO_EINVAL for a NULL
 * d_loss_minus. */
zo_status zo_mlp_loss_pair(zo_ctx *ctx, const float *d_params, uint64_t offset, uint32_t step,
                           uint32_t probe, float alpha, const uint8_t *d_bits, const float *d_X,
                           const int64_t *d_labels, uint32_t batch, uint32_t d_in,
                           uint32_t d_hid, uint32_t d_out, void *d_workspace,
                           uint64_t workspace_bytes, double *d_loss_plus, double *d_loss_minus,
                           void *stream);

/* Both losses of n_probes consecutive probes probe0 .. probe0 + n_probes - 1:
 * d_loss_plus[i] at theta + alpha * z_{probe0+i} and d_loss_minus[i] at
 * theta - alpha * z_{probe0+i} (device, n_probes doubles each), each equal bit for bit to
 * zo_mlp_loss_perturbed of that probe and sign: the step's forwards of "How 1.5-SPSA Works"
 * (n_pert probes, two losses each) as launch sequences of up to 64 probes, each wave of
 * the MFMA GEMM running two probes (ZO_MLP_PROBES_PER_WAVE: 1, 2, 4 or 8; at most 4 on 32 x 32 tiles) so that every X
 * and W1 operand it loads feeds both signs of each.  d_bits: NULL
 * (regenerate) or n_probes packed rows over the parameters, row i = probe probe0 + i
 * (zo_bits_stride(params) bytes apart, 16-byte aligned).  d_loss_clean: NULL, or one device
 * double that also receives the loss at the unperturbed parameters (the step's clean pass),
 * equal bit for bit to zo_mlp_loss, computed by one more group of waves in the first launch
 * sequence.  d_workspace: device, 8-byte aligned, at least
 * zo_mlp_probes_workspace_bytes(batch, d_in, d_hid, d_out, n_probes) bytes.  Other
 * arguments and limits as zo_mlp_loss_perturbed.  n_probes == 0 computes only the clean
 * loss (nothing without d_loss_clean).  Errors (ZO_EINVAL): as zo_mlp_loss_pair, a
 * workspace below that size, probe indices past 2^32 - 1, misaligned d_bits. */
uint64_t zo_mlp_probes_workspace_bytes(uint32_t batch, uint32_t d_in, uint32_t d_hid,
                                       uint32_t d_out, uint32_t n_probes);
zo_status zo_mlp_loss_probes(zo_ctx *ctx, const float *d_params, uint64_t offset, uint32_t step,
                             uint32_t probe0, uint32_t n_probes, float alpha,
                             const uint8_t *d_bits, const float *d_X, const int64_t *d_labels,
                             uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                             void *d_workspace, uint64_t workspace_bytes, double *d_loss_plus,
                             double *d_loss_minus, double *d_loss_clean, void *stream);

/* zo_mlp_loss_pair for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and the
 * same results, bit for bit, but the partial logits and row losses live in a static device
 * array of ZO_NOALLOC_SCRATCH_BYTES (1 MiB) per GPU, held until the process ends, instead
 * of a caller workspace; the call allocates nothing.  Every call on one GPU shares that
 * GPU's array (nothing in it must start at zero; the kernels write every slot they read),
 * so calls that overlap on one GPU -- on different streams or from different host threads
 * -- race and must not be made.  Arguments, results and errors as zo_mlp_loss_pair without
 * d_workspace / workspace_bytes; ZO_EUNSUPPORTED if zo_mlp_workspace_bytes(batch, d_in,
 * d_hid, d_out) exceeds ZO_NOALLOC_SCRATCH_BYTES (the 128 x 768 -> 3072 -> 2 classifier
 * needs 788,480 bytes). */
zo_status zo_mlp_loss_pair_noalloc(zo_ctx *ctx, const float *d_params, uint64_t offset,
                                   uint32_t step, uint32_t probe, float alpha,
                                   const uint8_t *d_bits, const float *d_X,
                                   const int64_t *d_labels, uint32_t batch, uint32_t d_in,
                                   uint32_t d_hid, uint32_t d_out, double *d_loss_plus,
                                   double *d_loss_minus, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ZO_H */
