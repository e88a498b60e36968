/*
 * kdn.h -- C ABI of the MI355X (gfx950) Kalman Delta Network mixer library.
 *
 * The library computes the KDN sequence-mixer forward pass in its two
 * scan-compatible approximations, Diagonal KDN (d_k variance scalars per
 * head) and Isotropic KDN (one variance scalar per head), and the single-token
 * decode step.  The method is defined on the KDN reading notes (page
 * "Kalman Delta Networks: 不确定性感知的关联记忆"), method part:
 *   - exact filter it approximates: §2, Eq. (12)-(17);
 *   - Diagonal KDN predict/gain: §4, Eq. (23)-(30);
 *   - information scaling mu: §5, Eq. (60)-(65) (gain uses the predicted
 *     variance; mu only shapes the variance carried to the next token);
 *   - Moebius form of the variance recurrence and the affine memory scan:
 *     §6, Eq. (32)-(39), with the Appendix D chunking summarised there;
 *   - Isotropic KDN: §7, Eq. (40) and Appendix C;
 *   - parameters alpha (decay), omega (process noise), r (observation
 *     noise) as inputs, and "scanned training == token-by-token inference":
 *     §8.
 *
 * Per token t and head, with D_t = diag(alpha_t):
 *   Diagonal:  p^ = alpha^2 (.) p + omega;  z = sum_i p^_i k_i^2;
 *              kappa = p^ (.) k / (r + z);
 *              p <- p^ / (1 + (mu/r) k (.) k (.) p^)
 *   Isotropic: a = mean_i alpha_i^2;  b^ = a b + omega;  n = |k|^2;
 *              kappa = b^ k / (r + b^ n);  b <- b^ / (1 + mu n b^ / (d_k r))
 *   Memory (both): S <- D S;  delta = v - S^T k;  S <- S + kappa delta^T;
 *              o = S^T q   (read after this token's write)
 *
 * CONVENTIONS (every entry point)
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never frees caller memory and allocates nothing on the forward or step
 *     paths; scratch space, where a regime needs it, is the caller's
 *     `workspace`.
 *   - Layouts are dense row-major:
 *       activations q,k [B,T,H,dk], v,o [B,T,H,dv] in the io dtype;
 *       alpha [B,T,H,dk] fp32; omega [B,T,H,dk] (diag) or [B,T,H] (iso) fp32;
 *       r [B,T,H] fp32; state S [B,H,dk,dv] fp32 (row i = key channel);
 *       variances p [B,H,dk] (diag) or b [B,H] (iso) fp32.
 *   - io dtype: KDN_F32 or KDN_BF16 for q, k, v and o.  Gates, state and
 *     variances are always fp32.  bf16 runs its chunk contractions on bf16
 *     matrix cores with fp32 accumulation (split-operand products for
 *     Diagonal unless KDN_MATH_BF16 is given, below); fp32 runs them in
 *     fp32.
 *   - Supported sizes: dk in {64, 128} for bf16 and dk = 64 for fp32;
 *     dv a multiple of 64 (bf16) or 32 (fp32), at most 256; B, H >= 1;
 *     T >= 0; B*H*T and every tensor below 2^31 elements.
 *   - Pointers to q, k, v, alpha, omega, o, S0/S_T/S and p0/p_T must be
 *     16-byte aligned.
 *   - Preconditions (documented, not checked per element): r > 0,
 *     0 <= alpha <= 1, omega >= 0, p0/b0 > 0, mu >= 0, all finite.  Outside
 *     them results are unspecified (NaN propagates; nothing faults).
 *   - Strong decay in the chunked forwards (every call here but kdn_step):
 *     the chunk products pair the cumulative decay G_t from a 16-token
 *     chunk's start with its reciprocal.  Where a channel's chunk decays by
 *     more than 2^100 the kernels measure G from a power-of-two reference
 *     inside the chunk (exact up to rounding) down to a chunk product of
 *     2^-224 (about 4e-68).  Below that, fp32 cannot span the chunk: every
 *     alpha of that channel and chunk under 2^-14 (zero included) is taken
 *     as 2^-14 in the memory decay (the variance recurrence keeps the true
 *     alpha), which leaves at most 2^-14 of the previous state row per such
 *     token where the method would leave alpha of it.
 *   - Validation is synchronous: on any invalid argument the call returns a
 *     negative status and launches nothing.  Launch failures return
 *     KDN_ERR_HIP.  Kernel faults surface at the caller's stream
 *     synchronisation.  Results are asynchronous on `stream`.
 *   - Results are deterministic run to run (no floating-point atomics).
 *   - Inputs are never modified, except S and var_state in kdn_step.
 *   - kdn_last_error_message() returns a thread-local description of the
 *     last failure on the calling thread.
 */
#ifndef KDN_H
#define KDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDN_OK = 0,
    KDN_ERR_INVALID_ARG = -1,
    KDN_ERR_UNSUPPORTED = -2,
    KDN_ERR_WORKSPACE = -3,
    KDN_ERR_HIP = -4
} kdn_status;

typedef enum { KDN_F32 = 0, KDN_BF16 = 1 } kdn_dtype;
typedef enum { KDN_DIAG = 0, KDN_ISO = 1 } kdn_variant;

/* Contraction precision of the bf16 forward, OR-ed into io_dtype of
 * kdn_diag_fwd, kdn_iso_fwd, kdn_fwd_ex, kdn_fwd_preact and
 * kdn_fwd_workspace_size (no other call accepts it; nor KDN_OUT_F32 below).
 *
 * By default the Diagonal bf16 forward runs every chunk contraction as three
 * bf16 matrix-core products of split operands, x = hi + lo with hi = bf16(x)
 * and lo = bf16(x - hi), summed in fp32 (hi.hi + lo.hi + hi.lo): about 16
 * significant bits per operand, near fp32 results (~1e-5 relative L2 against
 * an fp64 reference).  This is the higher-precision Diagonal of the KDN
 * reading notes (results part §6: the mixer throughput figure ran Diagonal in
 * FP32 / TF32x3 within a BF16 configuration; conclusions part §2: Diagonal
 * pays for an extra scan and higher-precision compute).  The Isotropic bf16
 * forward runs single bf16 products, as the notes ran it.
 *
 * KDN_MATH_BF16 makes the Diagonal bf16 forward run single bf16 products as
 * well: faster, ~4e-3 relative L2 on o.  With fp32 io it is
 * KDN_ERR_INVALID_ARG. */
enum { KDN_MATH_BF16 = 0x100 };

/* Output dtype flag, OR-ed into io_dtype of the same forward calls: with bf16
 * q, k, v, the Diagonal forward's split-product contractions write o in fp32
 * ([B,T,H,dv] float, 16-byte aligned) instead of rounding it to bf16, so o
 * keeps the contractions' precision.  KDN_ERR_UNSUPPORTED with Isotropic or
 * with KDN_MATH_BF16; KDN_ERR_INVALID_ARG with fp32 io (o is fp32 there
 * already). */
enum { KDN_OUT_F32 = 0x200 };

/* Bytes of device workspace with which kdn_diag_fwd / kdn_iso_fwd (and
 * kdn_fwd_ex) run this shape fastest.  The workspace is optional: a call given
 * less (or NULL) runs the serial walk, with the same results up to rounding.
 * Nonzero only for bf16 io with dk == dv when the serial walk would fill at
 * most a quarter of the chip (B*H*dv/64 workgroups against 256 compute
 * units, MI355X's count, taken as fixed so that the size is a pure function
 * of the shape, whatever the device) and T splits into 4 or 8
 * segments of at least 1024 tokens, each a multiple of 64: the state
 * recurrence is affine in the state over any span of tokens (method part §2
 * and §6 of the KDN reading notes), so the segments run as independent walks
 * whose linear and affine parts a short per-head combine chains, and the
 * segment-entry variances come from the gain scan (method part §6).  The size
 * is then the gain scan's carries, two segment-variance planes and four
 * [B*S,H,dk,dv] fp32 state planes.  Returns 0 for invalid shapes too; the
 * forward call reports those. */
size_t kdn_fwd_workspace_size(int variant, int B, int T, int H, int dk, int dv,
                              int io_dtype);

/*
 * Diagonal KDN forward over T tokens (KDN reading notes, method part §4-§6;
 * Appendix D chunking).
 *   q, k   [B,T,H,dk] io dtype       v, o  [B,T,H,dv] io dtype
 *   alpha  [B,T,H,dk] fp32 decay      omega [B,T,H,dk] fp32 process noise
 *   r      [B,T,H]    fp32 observation noise
 *   S0     [B,H,dk,dv] fp32 initial state, or NULL for zeros
 *   p0     [B,H,dk]    fp32 initial variances, or NULL for ones
 *   mu     information scale (the pages' default is dk)
 *   S_T    [B,H,dk,dv] fp32 final state (required)
 *   p_T    [B,H,dk]    fp32 final variances (required)
 *   workspace / workspace_bytes: optional device scratch, 16-byte aligned;
 *     with kdn_fwd_workspace_size(...) bytes or more, shapes with few heads
 *     and long sequences run split over the sequence (NULL: serial walk).
 *     When it is used it must not overlap any other argument
 *     (KDN_ERR_INVALID_ARG).
 *   stream: a hipStream_t (NULL = the null stream)
 * S_T may alias S0 exactly (each workgroup reads its own columns of the
 * state before it overwrites them).  p_T may alias p0 exactly only when
 * dv <= 64 for bf16 io (dv <= 32 for fp32), i.e. one workgroup per head: with
 * more, every value-tile workgroup reads the initial variances and nothing
 * orders that read before the first tile's final write, so the call returns
 * KDN_ERR_INVALID_ARG (use separate p0 / p_T buffers).  A partial overlap of
 * either pair, or o aliasing q, k or v, is rejected with KDN_ERR_INVALID_ARG.
 */
kdn_status kdn_diag_fwd(int B, int T, int H, int dk, int dv, int io_dtype, float mu,
                        const void* q, const void* k, const void* v,
                        const float* alpha, const float* omega, const float* r,
                        const float* S0, const float* p0,
                        void* o, float* S_T, float* p_T,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Isotropic KDN forward (KDN reading notes, method part §7, Eq. (40);
 * Appendix C).  Same layouts as kdn_diag_fwd except
 *   omega  [B,T,H] fp32 (one process-noise scalar per head and token)
 *   b0     [B,H] fp32 initial variance, or NULL for ones
 *   b_T    [B,H] fp32 final variance (required)
 */
kdn_status kdn_iso_fwd(int B, int T, int H, int dk, int dv, int io_dtype, float mu,
                       const void* q, const void* k, const void* v,
                       const float* alpha, const float* omega, const float* r,
                       const float* S0, const float* b0,
                       void* o, float* S_T, float* b_T,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step, one token per sequence (KDN reading notes, method part
 * §8: token-by-token inference runs the same recurrence as the scan).
 *   variant   KDN_DIAG or KDN_ISO
 *   q, k [B,H,dk], v, o [B,H,dv] io dtype; alpha [B,H,dk] fp32;
 *   omega [B,H,dk] (diag) or [B,H] (iso) fp32; r [B,H] fp32
 *   S         [B,H,dk,dv] fp32, read and overwritten in place
 *   var_state p [B,H,dk] (diag) or b [B,H] (iso) fp32, in place
 * Equivalent to the forward call with T = 1, S0 = S_T = S and
 * p0 = p_T = var_state.
 */
kdn_status kdn_step(int variant, int B, int H, int dk, int dv, int io_dtype, float mu,
                    const void* q, const void* k, const void* v,
                    const float* alpha, const float* omega, const float* r,
                    float* S, float* var_state, void* o, void* stream);

/*
 * Extended forward (either variant) with the trained per-head parameters of
 * the end-to-end network (KDN reading notes, method part §8: a learned scalar
 * initial covariance c_{0,h} I and information scale mu per head) and the
 * effective write strength diagnostic (method part §2:
 * beta_eff_t = k_t^T kappa_t = z_t / (r_t + z_t); its distribution is the
 * results part's §4, Fig. 2).  Arguments as in kdn_diag_fwd / kdn_iso_fwd
 * (variant KDN_DIAG or KDN_ISO; var0 / var_T are p0 / p_T or b0 / b_T), plus
 *   mu_h      [H] fp32 device, nullable: information scale of head h (used
 *             instead of mu; entries must be finite and >= 0, not checked)
 *   c0_h      [H] fp32 device, nullable: initial variance of head h, every
 *             channel (Diagonal) or the head's scalar (Isotropic); only
 *             when var0 is NULL -- giving both is KDN_ERR_INVALID_ARG
 *   beta_eff  [B,T,H] fp32 device, nullable: written with beta_eff of every
 *             token; must not alias r, o, S_T or var_T
 * All three are 4-byte aligned.  With all three NULL the call equals
 * kdn_diag_fwd / kdn_iso_fwd.  In the bf16 forward z_t is the diagonal of the
 * chunk's bf16 key product, so beta_eff carries the same bf16 rounding as
 * the gain it describes.
 */
kdn_status kdn_fwd_ex(int variant, int B, int T, int H, int dk, int dv, int io_dtype, float mu,
                      const float* mu_h, const void* q, const void* k, const void* v,
                      const float* alpha, const float* omega, const float* r, const float* S0,
                      const float* var0, const float* c0_h, void* o, float* S_T, float* var_T,
                      float* beta_eff, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Extended decode step: kdn_step with a per-head information scale mu_h [H]
 * (nullable, as in kdn_fwd_ex) and the token's effective write strength
 * beta_eff [B,H] fp32 (nullable).  Same passages as kdn_fwd_ex.
 */
kdn_status kdn_step_ex(int variant, int B, int H, int dk, int dv, int io_dtype, float mu,
                       const float* mu_h, const void* q, const void* k, const void* v,
                       const float* alpha, const float* omega, const float* r, float* S,
                       float* var_state, void* o, float* beta_eff, void* stream);

/*
 * Exact dense-covariance Kalman memory for small d_k (KDN reading notes,
 * method part §2, Eq. (12)-(17)), with the Diagonal KDN's gates as the
 * transition D_t = diag(alpha_t) and process noise Omega_t = diag(omega_t):
 * the filter whose mean-field projection is Diagonal KDN (method part §4).
 * An ablation and cross-check tool (a serial Riccati step per token), not a
 * throughput path; the information scale mu does not apply to it.
 *   q, k   [B,T,H,dk] io dtype       v, o  [B,T,H,dv] io dtype
 *   alpha, omega [B,T,H,dk] fp32     r     [B,T,H] fp32
 *   S0 [B,H,dk,dv] fp32 (NULL: zeros),  P0 [B,H,dk,dk] fp32 (NULL: identity)
 *   S_T, P_T  final state and covariance (required; may alias S0 / P0
 *             exactly, a partial overlap is KDN_ERR_INVALID_ARG)
 *   beta_eff  [B,T,H] fp32, nullable: z / (r + z), z = k^T P^ k
 * dk in {16, 32, 64}, dv in {16, 32, 64, 128}; fp32 arithmetic throughout.
 */
kdn_status kdn_dense_fwd(int B, int T, int H, int dk, int dv, int io_dtype, const void* q,
                         const void* k, const void* v, const float* alpha, const float* omega,
                         const float* r, const float* S0, const float* P0, void* o, float* S_T,
                         float* P_T, float* beta_eff, void* stream);

/*
 * Forward from the gates' pre-activations (KDN reading notes, method part
 * §8: the end-to-end network produces alpha = sigmoid(a), omega =
 * softplus(w) and r = r_min + softplus(rho) from its projections; the notes
 * use r_min = 0.01).  Arguments as kdn_fwd_ex, with the gates replaced by
 *   a_pre  [B,T,H,dk] io dtype (bf16 or fp32, as q/k/v), 16-byte aligned
 *   w_pre  [B,T,H,dk] (Diagonal) or [B,T,H] (Isotropic), io dtype, 16-byte aligned
 *   r_pre  [B,T,H] io dtype, 16-byte aligned
 *   r_min  > 0 and finite (keeps r > 0)
 * With bf16 io (and fp32 o not requested) the forward reads a_pre (and the
 * Diagonal w_pre) itself and forms alpha (and omega) on chip, with the
 * arithmetic of kdn_gates_from_preact; only r (and the Isotropic per-token
 * omega) pass through the workspace.  With fp32 io an elementwise pre-pass
 * writes all three gates into the workspace and the forward of kdn_fwd_ex
 * runs on them.  Either way the result equals, bit for bit, kdn_fwd_ex on
 * the gates kdn_gates_from_preact returns.  The workspace
 * (kdn_fwd_preact_workspace_size bytes, 16-byte aligned, disjoint from every
 * argument) is sized for the fp32 gates.  Validation happens before anything
 * is launched.  Every finite pre-activation is
 * accepted: a very negative a gives a small or zero alpha (sigmoid saturates
 * to 0 below about -88), which the strong-decay rule above covers.
 */
size_t kdn_fwd_preact_workspace_size(int variant, int B, int T, int H, int dk);
kdn_status kdn_fwd_preact(int variant, int B, int T, int H, int dk, int dv, int io_dtype,
                          float mu, const float* mu_h, const void* q, const void* k,
                          const void* v, const void* a_pre, const void* w_pre, const void* r_pre,
                          float r_min, const float* S0, const float* var0, const float* c0_h,
                          void* o, float* S_T, float* var_T, float* beta_eff, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * The gates alone from their pre-activations (KDN reading notes, method part
 * §8), as the forward from pre-activations forms them:
 *   alpha = sigmoid(a_pre)           [B,T,H,dk]
 *   omega = softplus(w_pre)          [B,T,H,dk] (Diagonal) or [B,T,H] (Isotropic)
 *   r     = r_min + softplus(r_pre)  [B,T,H]
 * Pre-activations in io_dtype (KDN_F32 or KDN_BF16, no flags), outputs fp32;
 * every pointer device memory, 16-byte aligned, non-null when T > 0, and no
 * output overlaps any input or other output.  r_min > 0 and finite.  The
 * sigmoid and softplus use the hardware exp2 / log2 (~1 ulp each; softplus
 * through log1p as log(u) e / (u - 1), u = 1 + e); the same operations form
 * the gates inside the bf16 forward, so its results equal kdn_fwd_ex's on
 * these gates bit for bit.  Asynchronous on `stream`.
 */
kdn_status kdn_gates_from_preact(int variant, int B, int T, int H, int dk, int io_dtype,
                                 const void* a_pre, const void* w_pre, const void* r_pre,
                                 float r_min, float* alpha, float* omega, float* r,
                                 void* stream);

/*
 * Backward pass of Diagonal / Isotropic KDN (the mixer is trained through the
 * scanned recurrence, KDN reading notes, method part §8; the notes print no
 * gradient formulas, so this is the reverse-mode derivative of the
 * recurrences of method part §2, §4-§5 and §7, including the information-
 * scaled variance update).  It returns the gradients of a loss L given
 *   d_o     [B,T,H,dv] io dtype: dL/do
 *   dS_T    [B,H,dk,dv] fp32, nullable (zero): dL/dS_T
 *   dvar_T  shape of var0, fp32, nullable (zero): dL/dp_T or dL/db_T
 * for the forward defined by the same arguments as kdn_fwd_ex (variant,
 * sizes, io_dtype, mu, mu_h, q, k, v, alpha, omega, r, S0, var0, c0_h).
 * Outputs (device, written in full; none may overlap any other buffer):
 *   dq, dk [B,T,H,dk] and dv [B,T,H,dv] in the io dtype
 *   dalpha [B,T,H,dk], domega (the shape of omega), dr [B,T,H] fp32
 *   dS0 [B,H,dk,dv], dvar0 (shape of var0), dmu [B,H] fp32, each nullable:
 *     the gradients by the initial state, the initial variance (also when it
 *     came from c0_h or the default 1; dL/dc0_h sums it over b and, for
 *     Diagonal, channels) and by the information scale each (b,h) used
 *     (dL/dmu_h sums it over b)
 * dk in {64, 128}, dv a multiple of 16 up to 256; fp32 arithmetic whatever
 * the io type.  q, k, v, d_o and alpha are 16-byte aligned, the other fp32
 * arrays 4-byte aligned, dq / dk / dv aligned to their element size.  The
 * forward is recomputed inside: the gain, then the state at every 16th token
 * (Diagonal with bf16 io and dv a multiple of 64: by the forward walk with
 * split-bf16 products, ~1e-5 relative; otherwise in fp32 products).
 * With dv a multiple of 64 the memory part runs in 16-token chunks on the
 * matrix cores (fp32 products); otherwise token by token from stored
 * innovations.  The workspace (kdn_bwd_workspace_size bytes, 16-byte aligned)
 * holds those and per-column-block partial sums.  Diagonal shapes with
 * dk = dv whose B*H*(dv/64) workgroups fill at most half of the chip and
 * whose T splits into 2, 4 or 8 segments of at least 1024 tokens (each a
 * multiple of 64) run split over the sequence with bf16 io: the state map
 * over a span is affine (method part §2, §6), so the reverse pass carries
 * the state adjoint into a segment from its right as M^T dS + (the
 * segment's own part), and the segments run side by side (their entry
 * states from the forward walk with split-bf16 products).  For those shapes
 * kdn_bwd_workspace_size includes the split's planes; a smaller workspace of
 * at least the rest runs the same call without the split.  Deterministic (no
 * atomics).  Asynchronous on `stream`; validation as for the forward.
 */
size_t kdn_bwd_workspace_size(int variant, int B, int T, int H, int dk, int dv);
kdn_status kdn_bwd(int variant, int B, int T, int H, int dk, int dv, int io_dtype, float mu,
                   const float* mu_h, const void* q, const void* k, const void* v,
                   const float* alpha, const float* omega, const float* r, const float* S0,
                   const float* var0, const float* c0_h, const void* d_o, const float* dS_T,
                   const float* dvar_T, void* dq, void* dk_out, void* dv_out, float* dalpha,
                   float* domega, float* dr, float* dS0, float* dvar0, float* dmu,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of kdn_fwd_preact: the gradients by the gates' pre-activations
 * (KDN reading notes, method part §8; d sigmoid(a)/da = alpha (1 - alpha),
 * d softplus(x)/dx = sigmoid(x)).  Arguments as kdn_bwd with the gates
 * replaced by a_pre, w_pre, r_pre and r_min as in kdn_fwd_preact, and their
 * gradients da_pre [B,T,H,dk], dw_pre (shape of w_pre), dr_pre [B,T,H] in
 * fp32 in place of dalpha, domega, dr.  The prologue writes the gates into the
 * front of the workspace (kdn_bwd_preact_workspace_size bytes, 16-byte
 * aligned), kdn_bwd runs on them with the rest of it, then the chain rule is
 * applied in place.  No output and no part of the workspace may overlap the
 * pre-activations.
 */
size_t kdn_bwd_preact_workspace_size(int variant, int B, int T, int H, int dk, int dv);
kdn_status kdn_bwd_preact(int variant, int B, int T, int H, int dk, int dv, int io_dtype,
                          float mu, const float* mu_h, const void* q, const void* k,
                          const void* v, const void* a_pre, const void* w_pre, const void* r_pre,
                          float r_min, const float* S0, const float* var0, const float* c0_h,
                          const void* d_o, const float* dS_T, const float* dvar_T, void* dq,
                          void* dk_out, void* dv_out, float* da_pre, float* dw_pre, float* dr_pre,
                          float* dS0, float* dvar0, float* dmu, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Gain scan alone (the variance recurrence and Kalman gain without the
 * memory), exposed for the chunk-parallel regime's tests and diagnostics.
 * Inputs as in the forward calls (q, v not needed).  Writes
 *   kappa [B,T,H,dk] fp32 gain (nullable),
 *   var_T p_T [B,H,dk] (diag) or b_T [B,H] (iso) fp32 (required).
 * The scan composes the per-channel 2x2 Moebius maps
 *   M_t = [[alpha^2, omega], [u alpha^2, 1 + u omega]]
 * (KDN reading notes, method part §6, Eq. (32)-(39)) within 64-token chunks
 * (one lane per channel for Diagonal, a wavefront scan over the tokens for
 * Isotropic), then applies the chunk summaries to the variance in chunk order
 * to get every chunk's entry variance, then replays each chunk from it.
 * Needs kdn_gain_workspace_size(...) bytes of workspace.
 */
size_t kdn_gain_workspace_size(int variant, int B, int T, int H, int dk);
kdn_status kdn_gain_scan(int variant, int B, int T, int H, int dk, int io_dtype, float mu,
                         const void* k, const float* alpha, const float* omega,
                         const float* r, const float* var0,
                         float* kappa, float* var_T,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * The gain scan above without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and validation
 * as kdn_gain_scan; its scratch (the chunk summaries and carries) is a static
 * device array of kdn_gain_scan_static_max_bytes() bytes (32 MiB) that every
 * GPU the library runs on holds from the library's load until the process
 * ends.  A shape whose kdn_gain_workspace_size exceeds that returns
 * KDN_ERR_WORKSPACE and launches nothing.  The call allocates nothing.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents (nothing in it needs clearing: each call writes what it reads), so
 * calls that overlap on one GPU (concurrent streams, or threads without
 * ordering) race: order them on one stream.
 */
size_t kdn_gain_scan_static_max_bytes(void);
kdn_status kdn_gain_scan_static(int variant, int B, int T, int H, int dk, int io_dtype, float mu,
                                const void* k, const float* alpha, const float* omega,
                                const float* r, const float* var0, float* kappa, float* var_T,
                                void* stream);

const char* kdn_status_string(int status);
const char* kdn_last_error_message(void);

/* Library version, e.g. "kdn-mi355x 0.1.0 gfx950". */
const char* kdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDN_H */
