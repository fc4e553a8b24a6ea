/*
 * s4dplr -- S4 DPLR convolution-mode forward pass on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libs4dplr.so.  Plain pointers and sizes only.  Every device buffer
 * is owned by the caller; the library never allocates device memory.  All
 * launches are asynchronous on the caller's HIP stream; a device fault
 * surfaces at the caller's next synchronisation.
 *
 * What is computed (pages cited by title and section):
 *   "The S4 kernel, from scratch", section 1: H independent single-input
 *   single-output state-space systems x' = A x + B u, y = C x + D u, one per
 *   channel, with complex A (N x N), B, C (N) and a real feed-through D.
 *   Section 2 / "S4" wiki, "Structured Transition Matrix": A = Lambda - P Q^*
 *   with Lambda complex diagonal and P, Q rank 1 (Q = P at initialization).
 *   Section 3: bilinear discretization with step dt.
 *   Section 4: the kernel's generating function at the L roots of unity,
 *   z_l = exp(-2 pi i l / L), is
 *       Khat(z) = 2/(1+z) * (k00 - k01 k10 / (1 + k11)),
 *       k_ab    = sum_n w_ab,n / (g(z) - Lambda_n),  g(z) = (2/dt)(1-z)/(1+z),
 *   with weights w00 = C B, w01 = C P, w10 = conj(Q) B, w11 = conj(Q) P
 *   (elementwise); at z = -1 its limit (dt/2) sum_n C_n B_n.  The inverse FFT
 *   of length L returns the aliased kernel (section 4, "Aliasing"); the
 *   time-domain kernel is its real part:  K[h][k] = Re((1/L) sum_l Khat_l z_l^-k).
 *   Section 5: the causal convolution y = K * u + D u, evaluated by an FFT
 *   zero-padded to 2L:  y[b][h][t] = sum_{j<=t} K[h][j] u[b][h][t-j] + D[h] u[b][h][t].
 *   "S4" wiki, section "S4D": with the diagonal flag the low-rank term is
 *   dropped (P = Q = 0) and only k00 is formed.
 *
 * Layouts (all contiguous, row-major, last index fastest):
 *   lambda, P, Q, B, C : [H][N] complex, interleaved float32 (re, im) -- the
 *                        "(..., 2) real tensor" storage of complex parameters
 *                        ("The S4 kernel, from scratch", section 6).
 *   dt, D              : [H] float32.
 *   K                  : [H][L] float32.
 *   u, y               : [batch][H][L] float32.
 *
 * Limits: L a power of two in [2, 65536] (so 2L <= 131072); 1 <= N <= 256;
 * H >= 1; batch >= 1; batch * H * L < 2^31.  The workspace is at least
 * s4dplr_plan_workspace_bytes() bytes and 256-byte aligned.  Every other
 * device buffer is 8-byte aligned (the kernels move complex values and real
 * samples in pairs); an entry point that gets one that is not returns
 * S4DPLR_ERR_ALIGN before enqueueing anything.
 *
 * Preconditions not checked on the device: Re(Lambda_n) < 0 (a stable
 * system: "The S4 kernel, from scratch", section 6 keeps the real parts
 * negative; "ML//SSM//S4": the discrete eigenvalues then lie inside the unit
 * circle), dt > 0, all values finite.  The library does not test them; a
 * violation gives unspecified (possibly non-finite) outputs but no access
 * outside the buffers.  The Python binding checks them on the host before
 * each call when the environment variable S4DPLR_VALIDATE is 1.
 *
 * Errors: every entry point returns a status code and never aborts or prints.
 * Host-side validation runs before any launch; on a validation error nothing
 * is enqueued.  S4DPLR_ERR_HIP reports a HIP runtime error raised while
 * enqueueing; s4dplr_last_hip_error() returns its hipError_t value.
 */
#ifndef S4DPLR_H
#define S4DPLR_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define S4DPLR_ABI_VERSION 1

typedef enum s4dplr_status {
  S4DPLR_OK = 0,
  S4DPLR_ERR_NULL = 1,        /* a required pointer is NULL                      */
  S4DPLR_ERR_SHAPE = 2,       /* a size is outside the limits above              */
  S4DPLR_ERR_WORKSPACE = 3,   /* workspace NULL-sized or not 256-byte aligned    */
  S4DPLR_ERR_UNSUPPORTED = 4, /* unknown flag bits                               */
  S4DPLR_ERR_HIP = 5,         /* HIP runtime error while enqueueing              */
  S4DPLR_ERR_ALIAS = 6,       /* output buffer overlaps an input it must not     */
  S4DPLR_ERR_TOO_LARGE = 7,   /* plan exceeds the static scratch of *_noalloc    */
  S4DPLR_ERR_ALIGN = 8        /* a device buffer is not 8-byte aligned           */
} s4dplr_status;

/* Plan flag: diagonal state matrix (S4D).  P and Q are ignored (may be NULL). */
#define S4DPLR_DIAGONAL 1u
/* Plan flag (with S4DPLR_DIAGONAL only): zero-order-hold discretization
 * ("The S4 kernel, from scratch", section 3: A-bar = exp(dt a)); kernel
 * generation then evaluates the Vandermonde product
 * K[h][k] = Re(sum_n C_n B-bar_n A-bar_n^k), B-bar_n = B_n (exp(dt a_n) - 1) / a_n,
 * which is the kernel itself (not aliased), and the recurrent view and the
 * backward pass use the same discretization. */
#define S4DPLR_ZOH 2u
/* Plan flag: reserve the workspace buffers of s4dplr_block_forward. */
#define S4DPLR_BLOCK 4u
/* Plan flags, bits 8..11: rank r of the low-rank term ("S4" wiki, "Structured
 * Transition Matrix": A = Lambda - P Q^* with low-rank P, Q, the correction
 * handled by the Woodbury identity), 1 <= r <= 4; a zero field means r = 1.
 * With r > 1, P and Q are [H][r][N] interleaved complex (the r columns of the
 * N x r factors one after another) and the generating function is
 *     Khat(z) = 2/(1+z) * (k00 - k01 (I_r + k11)^{-1} k10),
 * k00 = C R B, k01[j] = C R P_j, k10[i] = Q_i^* R B, k11[i][j] = Q_i^* R P_j,
 * R = (g(z) - Lambda)^{-1}: (r+1)^2 Cauchy sums and an r x r solve per
 * frequency.  Rank r > 1 is supported by s4dplr_kernel_gen,
 * s4dplr_generating_function, s4dplr_forward, s4dplr_forward_noalloc and
 * s4dplr_block_forward; s4dplr_recurrent_prepare and s4dplr_kernel_gen_bwd
 * return ERR_UNSUPPORTED for it, and it cannot be combined with
 * S4DPLR_DIAGONAL (ERR_UNSUPPORTED at plan creation). */
#define S4DPLR_RANK_SHIFT 8
#define S4DPLR_RANK_MASK (0xFu << S4DPLR_RANK_SHIFT)
#define S4DPLR_RANK(r) ((unsigned)(r) << S4DPLR_RANK_SHIFT)

typedef struct s4dplr_plan s4dplr_plan;

/* ABI version of the loaded library (S4DPLR_ABI_VERSION it was built with). */
int s4dplr_abi_version(void);

/* Static English description of a status code; never NULL. */
const char* s4dplr_status_string(s4dplr_status status);

/* hipError_t of the most recent S4DPLR_ERR_HIP on the calling thread (0 if none). */
int s4dplr_last_hip_error(void);

/*
 * Create a plan for H channels of N poles, sequence length L and `batch`
 * input rows per channel.  Host-only: allocates host memory for the plan and
 * its fp64-derived tables, touches no device.  *out receives the plan, or NULL
 * on error.  Errors: ERR_NULL (out), ERR_SHAPE (sizes), ERR_UNSUPPORTED (flags,
 * including a rank field above 4 or a rank above 1 with S4DPLR_DIAGONAL).
 * The plan is immutable after creation and may be used concurrently from
 * several threads and streams, each with its own workspace.
 */
s4dplr_status s4dplr_plan_create(s4dplr_plan** out, int H, int N, int L, int batch,
                                 unsigned flags);

/* Bytes of device workspace the plan needs.  Errors: ERR_NULL. */
s4dplr_status s4dplr_plan_workspace_bytes(const s4dplr_plan* plan, size_t* bytes);

/*
 * Copy the plan's constant tables (frequency nodes, FFT twiddles, real-FFT
 * weights; computed in fp64 on the host, rounded to fp32) into the head of
 * the workspace `ws` on `stream`.  Call once per workspace before the compute
 * entry points; those leave the table region untouched, so the workspace can
 * be reused for any number of calls with the same plan.
 * Errors: ERR_NULL, ERR_WORKSPACE (alignment), ERR_HIP.
 */
s4dplr_status s4dplr_plan_init(const s4dplr_plan* plan, void* ws, hipStream_t stream);

/*
 * Kernel generation ("The S4 kernel, from scratch", sections 3-4): write the
 * time-domain kernel K [H][L] for the DPLR parameters.  lambda, P, Q, B, C
 * are [H][N] interleaved complex; dt is [H].  Q == NULL means Q = P.  With
 * S4DPLR_DIAGONAL, P and Q are ignored.  Device pointers.  K must not overlap
 * the workspace.  Also leaves the kernel's padded spectrum in the workspace
 * (with D = 0).
 * Errors: ERR_NULL, ERR_WORKSPACE, ERR_HIP.
 */
s4dplr_status s4dplr_kernel_gen(const s4dplr_plan* plan, const float* lambda, const float* P,
                                const float* Q, const float* B, const float* C,
                                const float* dt, float* K, void* ws, hipStream_t stream);

/*
 * The generating function alone ("The S4 kernel, from scratch", section 4):
 * khat[h][l] = Khat(z_l) at the L roots of unity z_l = exp(-2 pi i l / L),
 *     Khat(z) = 2/(1+z) * (k00 - k01 k10 / (1 + k11)),
 * the four Cauchy sums over the N poles and the rank-1 Woodbury correction,
 * with the limit (dt/2) sum_n C_n B_n at z = -1.  With S4DPLR_DIAGONAL only
 * k00 is formed ("S4" wiki, "S4D").  khat is [H][L] interleaved complex
 * float32 in natural frequency order; its inverse FFT's real part is the
 * kernel of s4dplr_kernel_gen.  Parameters as for s4dplr_kernel_gen; device
 * pointers.  Needs the plan's tables in ws (s4dplr_plan_init); writes nothing
 * else.  khat must not overlap the inputs or the workspace (ERR_ALIAS).
 * Errors: ERR_NULL, ERR_ALIAS, ERR_WORKSPACE, ERR_UNSUPPORTED (a plan with
 * S4DPLR_ZOH, whose kernel is not built from this function), ERR_HIP.
 */
s4dplr_status s4dplr_generating_function(const s4dplr_plan* plan, const float* lambda,
                                         const float* P, const float* Q, const float* B,
                                         const float* C, const float* dt, float* khat, void* ws,
                                         hipStream_t stream);

/*
 * Causal convolution ("The S4 kernel, from scratch", sections 1 and 5):
 * y[b][h][t] = sum_{j<=t} K[h][j] u[b][h][t-j] + D[h] u[b][h][t], by an FFT
 * zero-padded to 2L.  u, y: [batch][H][L]; K: [H][L]; D: [H] or NULL (D = 0).
 * Device pointers.  y must not overlap u or K (ERR_ALIAS).
 * Errors: ERR_NULL, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP.
 */
s4dplr_status s4dplr_conv_fwd(const s4dplr_plan* plan, const float* u, const float* K,
                              const float* D, float* y, void* ws, hipStream_t stream);

/*
 * The whole convolution-mode forward pass: kernel generation followed by the
 * causal convolution, y = K * u + D u.  Arguments as above; K may be NULL, in
 * which case the time-domain kernel is not written out.  D may be NULL (D = 0).
 * y must not overlap u (ERR_ALIAS).
 * Errors: ERR_NULL, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP.
 */
s4dplr_status s4dplr_forward(const s4dplr_plan* plan, const float* lambda, const float* P,
                             const float* Q, const float* B, const float* C, const float* dt,
                             const float* D, const float* u, float* K, float* y, void* ws,
                             hipStream_t stream);

/*
 * s4dplr_forward without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that forbid
 * allocation): the scratch is a static device array of the library, 64 MiB
 * per GPU, held from its first use on that GPU until the process ends.  Plans
 * whose forward pass needs more (the four-step path at large batch * H, e.g.
 * H = 64, L = 65536, batch = 4) are rejected with ERR_TOO_LARGE; the
 * tiny, mid, long and S4D-Lin workload shapes fit.  Computes exactly what
 * s4dplr_forward computes, with the same kernels, on the current device;
 * stream must belong to it.  Every call computes the plan's tables into the
 * array with a small kernel (the same fp64 formulas as the workspace tables,
 * rounded once; nothing is copied from host memory), then generates the
 * kernel and applies the convolution.  All calls on one GPU share its array: calls that can overlap
 * in time on one GPU (other streams, other threads) race and must be
 * serialized by the caller.  No device memory is allocated or freed.
 * Errors: ERR_NULL, ERR_ALIAS, ERR_TOO_LARGE, ERR_HIP.
 */
s4dplr_status s4dplr_forward_noalloc(const s4dplr_plan* plan, const float* lambda,
                                     const float* P, const float* Q, const float* B,
                                     const float* C, const float* dt, const float* D,
                                     const float* u, float* K, float* y, hipStream_t stream);

/*
 * Apply the convolution with the kernel spectrum already in the workspace:
 * y = K * u + D u for the K and D of the most recent s4dplr_kernel_gen
 * (which uses D = 0), s4dplr_conv_fwd or s4dplr_forward call made with this
 * plan on this workspace and stream order.  For running one layer's kernel
 * over several input batches without generating it again ("The S4 kernel,
 * from scratch", section 5: the kernel is computed once and applied as one
 * long convolution).  Without such a prior call the results are unspecified
 * (every access stays inside the workspace).  u, y: [batch][H][L].
 * Errors: ERR_NULL, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP.
 */
s4dplr_status s4dplr_conv_apply(const s4dplr_plan* plan, const float* u, float* y, void* ws,
                                hipStream_t stream);

/*
 * Recurrent view, stage 1 ("The S4 kernel, from scratch", section 5;
 * "Structured state-space sequence model and S4", "One linear layer, two
 * computational views"): form the per-pole step records of the bilinear
 * system A-bar = (I - dt/2 A)^{-1} (I + dt/2 A), B-bar = (I - dt/2 A)^{-1} dt B
 * (section 3) for A = Lambda - P Q^* ("S4" wiki, "Structured Transition
 * Matrix"), in O(N) per channel through the Sherman-Morrison identity; kept in
 * the workspace for s4dplr_recurrent_scan.  Arguments and layouts as for
 * s4dplr_kernel_gen (Q == NULL means Q = P; with S4DPLR_DIAGONAL, P and Q are
 * ignored).  Device pointers.  Does not touch the convolution state of the
 * workspace.  The records are formed in fp64 and stored as fp32.  For plans
 * with N <= 64, L >= 128 and batch * H < 4096 it also forms, per channel,
 * A-bar^C (fp64 squarings, stored as fp32) for the chunk length C the plan
 * chose, which the chunked form of s4dplr_recurrent_scan uses.
 * Errors: ERR_NULL, ERR_WORKSPACE, ERR_HIP.
 */
s4dplr_status s4dplr_recurrent_prepare(const s4dplr_plan* plan, const float* lambda,
                                       const float* P, const float* Q, const float* B,
                                       const float* C, const float* dt, void* ws,
                                       hipStream_t stream);

/*
 * Recurrent view, stage 2: T steps of
 *     x_t = A-bar x_{t-1} + B-bar u_t,   y_t = Re(C x_t) + D u_t
 * for every (batch, channel) sequence, starting from the state passed in and
 * leaving the state after the last step in its place, so consecutive calls
 * continue one stream (streaming inference).  A zero state at the first call
 * gives y = K_T * u + D u with the untruncated-by-aliasing kernel
 * K_k = Re(C A-bar^k B-bar) (section 4, "the kernel is the impulse response").
 * Uses the records of the latest s4dplr_recurrent_prepare on this workspace
 * in stream order (without one the results are unspecified; every access
 * stays inside the workspace).
 *   u, y  : [batch][H][T] float32 (T need not equal the plan's L).
 *   state : [batch][H][N] complex, interleaved float32 (re, im); read and
 *           written.
 *   D     : [H] float32 or NULL (D = 0).
 * T = 0 is a no-op (u and y may then be NULL).  y must not overlap u, state
 * or the workspace; state must not overlap u or the workspace (ERR_ALIAS).
 * When the plan has a chunk length C (see s4dplr_recurrent_prepare) and the
 * call spans 2 .. L/C chunks, the sequences are scanned chunk by chunk in
 * parallel and joined through A-bar^C (three launches); otherwise each
 * sequence is scanned step by step.  Both compute the same recurrence.
 * Limits: 0 <= T and batch * H * T < 2^31 (ERR_SHAPE).
 * Errors: ERR_NULL, ERR_SHAPE, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP.
 */
s4dplr_status s4dplr_recurrent_scan(const s4dplr_plan* plan, const float* D, const float* u,
                                    int T, float* state, float* y, void* ws,
                                    hipStream_t stream);

/*
 * Backward pass of the causal convolution ("The S4 kernel, from scratch",
 * sections 5 and 6: the layer is trained through the convolution).  Given
 * dy = dloss/dy for y = K * u + D u:
 *   du[b][h][t] = sum_{j=0}^{L-1-t} K[h][j] dy[b][h][t+j] + D[h] dy[b][h][t]
 *   dK[h][j]    = sum_b sum_{t=j}^{L-1} dy[b][h][t] u[b][h][t-j]
 *   dD[h]       = sum_b sum_t dy[b][h][t] u[b][h][t]
 * each by FFTs zero-padded to 2L.  u, dy, du: [batch][H][L]; K, dK: [H][L];
 * D, dD: [H].  Any of du, dK, dD may be NULL (not computed).  du needs K
 * (D may be NULL: D = 0); dK and dD need u.  Outputs are overwritten, not
 * accumulated, and must not overlap the inputs, each other or the workspace
 * (ERR_ALIAS).  Computing du replaces the convolution weights held in the
 * workspace (a later s4dplr_conv_apply then applies the correlation).
 * Errors: ERR_NULL, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP.
 */
s4dplr_status s4dplr_conv_bwd(const s4dplr_plan* plan, const float* u, const float* K,
                              const float* D, const float* dy, float* du, float* dK, float* dD,
                              void* ws, hipStream_t stream);

/*
 * Backward pass of kernel generation ("The S4 kernel, from scratch",
 * sections 3-4): the gradients of loss = sum_{h,k} dK[h][k] K[h][k] with
 * respect to lambda, P, Q, B, C (each [H][N] interleaved complex; the pair
 * (re, im) of an output is (dloss/dRe, dloss/dIm)) and dt ([H]), for K the
 * aliased kernel of s4dplr_kernel_gen.  Inputs as for s4dplr_kernel_gen plus
 * dK [H][L].  Q == NULL means Q = P: dP then includes the path through Q and
 * dQ is ignored.  With S4DPLR_DIAGONAL, dP and dQ are ignored.  Every output
 * may be NULL (not written); outputs are overwritten, not accumulated, and
 * must not overlap the inputs, each other or the workspace (ERR_ALIAS).
 * Errors: ERR_NULL, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP.
 */
s4dplr_status s4dplr_kernel_gen_bwd(const s4dplr_plan* plan, const float* lambda, const float* P,
                                    const float* Q, const float* B, const float* C,
                                    const float* dt, const float* dK, float* dlambda, float* dP,
                                    float* dQ, float* dB, float* dC, float* ddt, void* ws,
                                    hipStream_t stream);

/*
 * The block around the layer ("The S4 kernel, from scratch", section 6: a
 * pre-norm, a GLU-gated projection and a residual connection):
 *   z = LayerNorm_h(x) * gamma + beta   (over the H channels at each (b, t);
 *                                       biased variance, eps = 1e-5),
 *   s = the layer applied to z          (s4dplr_forward with these parameters),
 *   out = x + a * sigmoid(g),  [a; g] = W s + bias  (W: [2H][H] row-major fp32,
 *                                       rows [0, H) values, [H, 2H) gates).
 * x, out: [batch][H][L]; gamma, beta: [H]; bias: [2H]; the layer's parameters
 * as for s4dplr_forward (Q and D may be NULL).  The plan must have been
 * created with S4DPLR_BLOCK.  out may be x itself (in place); otherwise it
 * must not overlap x, and it must never overlap the other inputs or the
 * workspace (ERR_ALIAS).  The projection runs on the bf16 matrix cores with
 * every operand split into two bf16 parts (hi = bf16(v), lo = bf16(v - hi))
 * and the three products hi*hi + hi*lo + lo*hi summed in fp32 accumulators:
 * 16 significant bits per operand, within 6e-6 of the fp64 result on the
 * tested shapes.
 * Limit: batch <= 65535 (ERR_SHAPE).
 * Errors: ERR_NULL, ERR_SHAPE, ERR_ALIAS, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP.
 */
s4dplr_status s4dplr_block_forward(const s4dplr_plan* plan, const float* x, const float* gamma,
                                   const float* beta, const float* lambda, const float* P,
                                   const float* Q, const float* B, const float* C,
                                   const float* dt, const float* D, const float* W,
                                   const float* bias, float* out, void* ws, hipStream_t stream);

/* Release a plan (NULL is ignored).  Host-only. */
void s4dplr_plan_destroy(s4dplr_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* S4DPLR_H */
