/*
 * falcon.h — C ABI of the MI355X (gfx950) Falcon fast-weight forward pass.
 *
 * The operation is the forward pass of "Fast Weight Attention for Continual
 * Learning" (arXiv 2608.27763v1).  Per (batch, head) a fast-weight state S
 * with d_k rows and d_v columns is written once per token with the
 * prefix-aligned pair x_t = phi(k_{t-1}), y_t = v_t, and read after the write
 * with o_t = S_t^T phi(q_t):
 *   - the pair, the sentinel x_1 = 0 and the strict no-op first step:
 *     paperlayer.ai summary, §3 "Autoregressive Next-Latent Prediction",
 *     Appendix, §4.6 and §H.3 "Identification of Drivers";
 *   - the step eta_t = beta_t / (mu_t + lambda_t + eps) (0 if the
 *     denominator is 0), the carry gamma_t = 1 - min(eta_t lambda_t,
 *     1 - eps_gamma): summary §3.1, §C.3, §4.6; agihunt.info explainer
 *     "Method"; sungsoo.github.io post (clamp and log1p paragraph);
 *   - the writes of Falcon-1 (scalar NLMS), Falcon-2 (per value column),
 *     Falcon-3 (window mini-batch, mu_t = lambda_max of the window
 *     covariance), Falcon-1A / Falcon-2A / Falcon-3A (inner-product writes,
 *     scalar / per value column / window): summary §1, §4, §4.3-§4.5, App. F;
 *     explainer "Method";
 *   - the feature map phi = QK-RMSNorm (default) or the identity:
 *     summary §5 and §H.3 "The Falcon-3 Recurrence";
 *   - the recurrent and chunk-parallel forms and the chunk-local log-decay:
 *     summary Figure 2, Figure 4, §D.1 "Chunk-Local Evaluation", §G.1;
 *   - the boundary state for exact continuation (S, the next pair's
 *     feature, the last W-1 pairs): summary §C.7, §4.4; sungsoo.github.io.
 *
 * Conventions for every entry point
 *   - All tensor pointers inside the structs are DEVICE pointers owned by
 *     the caller; the library keeps none of them after a call returns.
 *     The structs themselves (falcon_fwd_args, falcon_state) live in host
 *     memory and are read during the call only.
 *   - Layouts are contiguous row-major with batch, then head, then token,
 *     then feature: q, k [B,H,T,d_k]; v, o [B,H,T,d_v]; beta [B,H,T]
 *     ([B,H,T,d_v] for Falcon-2 and -2A); lambda [B,H,T]; S [B,H,d_k,d_v].
 *   - Errors are returned as negative status codes (falcon_status_str gives
 *     the text).  On any error except FALCON_ERR_HIP nothing is launched.
 *   - falcon_fwd enqueues work on the given stream and returns without
 *     synchronising, allocating or freeing memory.  It is reentrant: the
 *     only process-wide state is a per-device cache of the compute-unit
 *     count (atomic) and the debug switch below, read once.
 *   - Debug mode: with the environment variable FALCON_SYNC_CHECK set to a
 *     value other than "0", every entry point that launches kernels
 *     synchronises the stream after each launch and checks the HIP error
 *     state; the first failing kernel is reported on stderr and the call
 *     returns FALCON_ERR_HIP.  It is read once per process, changes no
 *     result, must not be used under stream capture, and is the library's
 *     only environment switch.
 *   - Data preconditions that are documented, not checked on the device:
 *     beta >= 0 and lambda >= 0 (the pages require non-negative steps and
 *     ridge; the NLMS gain is meant to lie in (0, 2)), finite inputs.
 *   - The same inputs give bitwise-identical outputs (no atomics).
 */
#ifndef FALCON_H
#define FALCON_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FALCON_ABI_VERSION 1
#define FALCON_MAX_WINDOW 8

/* status codes */
#define FALCON_OK 0
#define FALCON_ERR_INVALID_ARG (-1) /* a malformed argument                        */
#define FALCON_ERR_UNSUPPORTED (-2) /* well formed but not implemented (sizes...)  */
#define FALCON_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required  */
#define FALCON_ERR_HIP (-4)         /* a kernel launch failed (hipGetLastError)    */

/* variants: 1/2/3 = scalar, per-column, sliding-window regression;
 * 11/12/13 = scalar, per-column, sliding-window inner-product writes
 * (Falcon-2A: summary "B. Falcon-2A: per-channel inner-product write",
 * §4.3, §4.5, Figures 6-8) */
#define FALCON_V1 1
#define FALCON_V2 2
#define FALCON_V3 3
#define FALCON_V1A 11
#define FALCON_V2A 12
#define FALCON_V3A 13

/* storage type of q, k, v and o */
#define FALCON_BF16 0
#define FALCON_F32 1

/* feature map phi applied to q and k */
#define FALCON_PHI_RMSNORM 0  /* z / sqrt(mean(z^2) + eps_rms); 0 if that is 0/0 */
#define FALCON_PHI_IDENTITY 1 /* the "unkernelized" case                        */

/*
 * Boundary state of a segment (summary §C.7, §4.4).
 *   S       [B,H,d_k,d_v] fp32, device.
 *   x_next  [B,H,d_k] fp32, device: phi(k_T) of the previous segment, the
 *           write feature of this segment's first pair.  Ignored when fresh.
 *   tail_x  [B,H,W-1,d_k] fp32, device; tail_y [B,H,W-1,d_v] fp32, device:
 *           the last pairs, right-aligned and oldest first: slot s holds the
 *           pair that lies W-1-s pairs before this segment's first pair.
 *           Only the last n_tail slots are meaningful.  Unused when W == 1.
 *   n_tail  host int, 0..W-1 (input); written by the library on output as
 *           min(W-1, n_tail_in + T).  Output slots before the valid ones are
 *           zero-filled.
 *   fresh   host int.  Input: nonzero means a new sequence (x_1 = 0 and the
 *           first step is a strict no-op); then x_next is ignored and n_tail
 *           must be 0.  Output: set to 1 only when T == 0 and the input was
 *           fresh, else 0.
 */
typedef struct falcon_state {
    float *S;
    float *x_next;
    float *tail_x;
    float *tail_y;
    int n_tail;
    int fresh;
} falcon_state;

/*
 * Arguments of one forward call.
 *   abi_version  must equal FALCON_ABI_VERSION.
 *   variant      FALCON_V1, _V2, _V3, _V1A, _V2A or _V3A.
 *   dtype        FALCON_BF16 or FALCON_F32 (q, k, v, o).  State, beta and
 *                lambda are always fp32; all arithmetic accumulates in fp32.
 *   phi          FALCON_PHI_RMSNORM or FALCON_PHI_IDENTITY.
 *   batch, heads >= 1; seqlen >= 0; dk, dv in {16, 32, 64, 128}.
 *   chunk        0 = token-recurrent form (every variant);
 *                64 = chunk-parallel form, for Falcon-1 (dk in {32, 64, 128},
 *                any dv), Falcon-2 (bf16: dk in {64, 128}; fp32: dk = 64;
 *                any dv) and Falcon-1A / 3A (dk in {32, 64}, dv <= 64).
 *                A combination that has no chunk-parallel kernel returns
 *                FALCON_ERR_UNSUPPORTED.
 *   window       W >= 1; must be 1 for V1, V2, V1A, V2A; at most FALCON_MAX_WINDOW.
 *   eps >= 0, eps_rms >= 0, 0 < eps_gamma < 1 (defaults 1e-6, 1e-6, 1e-3).
 *   q, k, v      device inputs, 16-byte aligned.
 *   beta, lambda device fp32 inputs, 16-byte aligned.
 *   state_in     NULL: S_0 = 0 and a fresh sequence.
 *   state_out    NULL: the final state is not written.  Must not overlap
 *                state_in.
 *   o            device output [B,H,T,d_v] in dtype.
 *   workspace    device scratch of at least falcon_fwd_workspace_size(args)
 *                bytes, 256-byte aligned; may be NULL when that size is 0.
 */
typedef struct falcon_fwd_args {
    int abi_version;
    int variant;
    int dtype;
    int phi;
    int batch, heads, seqlen, dk, dv;
    int chunk;
    int window;
    float eps, eps_gamma, eps_rms;
    const void *q, *k, *v;
    const float *beta, *lambda;
    const falcon_state *state_in;
    falcon_state *state_out;
    void *o;
    void *workspace;
    size_t workspace_bytes;
} falcon_fwd_args;

/* Bytes of device workspace falcon_fwd needs for these arguments (pointer
 * fields are not read).  Pure host code, no HIP call.  Returns 0 for a
 * malformed or unsupported argument set (falcon_fwd_validate says which). */
size_t falcon_fwd_workspace_size(const falcon_fwd_args *args);

/* Checks every argument rule above without touching the GPU.  Returns
 * FALCON_OK or a negative status.  Pure host code, no HIP call. */
int falcon_fwd_validate(const falcon_fwd_args *args);

/* Forward pass: validates, then enqueues the kernels on `stream` (a
 * hipStream_t; NULL = the default stream).  Returns FALCON_OK or a negative
 * status.  Writes o and, if requested, the device parts of state_out; the
 * host fields state_out->n_tail and ->fresh are written before returning. */
int falcon_fwd(const falcon_fwd_args *args, void *stream);

/* Measurement variant of falcon_fwd for benchmarks and profilers: the same
 * validation and the same kernels on `stream`, and in addition it records
 * events[0] before the first kernel and events[i] after the i-th kernel, for
 * i < n_events.  `events` holds hipEvent_t handles owned by the caller (NULL
 * with n_events == 0 is allowed).  Returns the number of kernels launched
 * (>= 0) or a negative status. */
int falcon_fwd_profile(const falcon_fwd_args *args, void *stream, void *const *events, int n_events);

/* Largest workspace falcon_fwd_noalloc can serve: 64 MiB per GPU. */
#define FALCON_NOALLOC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): falcon_fwd
 * with the workspace taken from a fixed device array of the library
 * (FALCON_NOALLOC_SCRATCH_BYTES, one per GPU, held from the library's first
 * use on that GPU until the process ends) instead of args->workspace, which
 * is ignored.  The caller still provides every input and output.  Nothing is
 * allocated or freed: the first call on a device only looks up that device's
 * array.  Calls whose workspace need (falcon_fwd_workspace_size) exceeds
 * FALCON_NOALLOC_SCRATCH_BYTES return FALCON_ERR_WORKSPACE without
 * launching; a failed lookup returns FALCON_ERR_HIP.  Every call on one GPU
 * uses the same array, which keeps the previous call's contents (no kernel
 * reads workspace it has not written in the same call): calls that overlap
 * in time on one GPU, on any streams or host threads, race and must be
 * ordered by the caller.  Same validation, kernels, results and status codes
 * as falcon_fwd otherwise. */
int falcon_fwd_noalloc(const falcon_fwd_args *args, void *stream);

/*
 * Backward pass of Falcon-1 (summary §D.2 "Backward Pass", §E.3 "Chunk-
 * Parallel Backward Pass", §G.3 "Forward and Backward Algorithms"): the
 * gradients of a scalar loss through one falcon_fwd call of variant
 * FALCON_V1 (window 1), given the gradients that reach its outputs.
 *   - o_t = S_t^T phi(q_t) and S_t = gamma_t S_{t-1} + eta_t x_t r_t^T,
 *     r_t = v_t - S_{t-1}^T x_t, are reversed token by token from the end:
 *     with G_t = dL/dS_t and w_t = G_t^T x_t, G_{t-1} = gamma_t G_t -
 *     eta_t x_t w_t^T; dgamma_t = <G_t, S_{t-1}>, deta_t = w_t . r_t,
 *     dv_t = eta_t w_t, dx_t = eta_t (G_t r_t - S_{t-1} w_t).
 *   - The decay gradient reaches eta_t and lambda_t only where the clamp
 *     alpha_t = min(eta_t lambda_t, 1 - eps_gamma) does not bind
 *     (eta_t lambda_t < 1 - eps_gamma, evaluated in fp32 as in the forward).
 *   - eta_t = beta_t / d_t, d_t = ||x_t||^2 + lambda_t + eps; where d_t = 0
 *     the step is 0 and its gradients are 0 (no 0/0).
 *   - The no-op first step of a fresh sequence is a boundary constant:
 *     d_beta and d_lambda of that token are 0.
 *   - x_t = phi(k_{t-1}) and phi(q_t) are differentiated through phi
 *     (QK-RMSNorm: dz = s g - (s^3 / d_k)(z . g) z, s = (mean(z^2) +
 *     eps_rms)^(-1/2); 0 where mean(z^2) + eps_rms = 0; identity: dz = g).
 *     k_{T-1} feeds only the next segment's first pair: d_k of token T-1 is
 *     phi's product with d_x_next_out (0 when NULL).
 * The forward is recomputed from the inputs (nothing from falcon_fwd is
 * reused).  For T > 0 and d_k, d_v <= 64 the pass is chunk-parallel in
 * 64-token chunks (summary §E.3, §H.1): one chunk of the forward is affine in
 * its entry state, S_end = A S_0 + B, O = G S_0 + ..., so the state gradient
 * crosses a chunk backwards as H <- A^T H + G^T dO, and each chunk's token
 * gradients follow from its entry state and H at its end; the workspace holds
 * per chunk the fp32 records A, B, G^T dO and the chunk's entry state and H
 * (about B*H*ceil(T/64)*(d_k*d_k + 4*d_k*d_v)*4 bytes).  Other shapes run the
 * token-recurrent reverse, keeping the state before every 4th token.  All
 * products are fp32.
 *
 *   abi_version  FALCON_ABI_VERSION.  variant: FALCON_V1 only (other
 *                variants return FALCON_ERR_UNSUPPORTED).
 *   dtype, phi, batch, heads, seqlen (>= 0), dk, dv (in {16, 32, 64, 128}),
 *   eps, eps_gamma, eps_rms: as in falcon_fwd_args.
 *   q, k, v, beta, lambda: the forward's inputs (device, 16-byte aligned).
 *   state_in     the forward's input state, or NULL (fresh, S_0 = 0);
 *                n_tail must be 0.
 *   d_o          [B,H,T,d_v] in dtype: dL/do.
 *   d_S_out      [B,H,d_k,d_v] fp32: dL/dS_T, or NULL (0).
 *   d_x_next_out [B,H,d_k] fp32: dL/d(state_out->x_next), or NULL (0).
 *   d_q, d_k, d_v  [B,H,T,d_k / d_v] in dtype, written.
 *   d_beta, d_lambda  [B,H,T] fp32, written.
 *   d_S_in       [B,H,d_k,d_v] fp32: dL/dS_0, written unless NULL.
 *   d_x_next_in  [B,H,d_k] fp32: dL/d(state_in->x_next), written unless NULL
 *                (0 for a fresh sequence).
 *   No output may overlap an input or another output.
 *   workspace    at least falcon_bwd_workspace_size(args) bytes, 256-byte
 *                aligned.
 * Same conventions as falcon_fwd otherwise (errors, streams, no allocation,
 * reentrancy, bitwise-identical results for identical inputs).
 */
typedef struct falcon_bwd_args {
    int abi_version;
    int variant;
    int dtype;
    int phi;
    int batch, heads, seqlen, dk, dv;
    float eps, eps_gamma, eps_rms;
    const void *q, *k, *v;
    const float *beta, *lambda;
    const falcon_state *state_in;
    const void *d_o;
    const float *d_S_out, *d_x_next_out;
    void *d_q, *d_k, *d_v;
    float *d_beta, *d_lambda;
    float *d_S_in, *d_x_next_in;
    void *workspace;
    size_t workspace_bytes;
} falcon_bwd_args;

/* Bytes of workspace falcon_bwd needs (pointer fields are not read); 0 for
 * an invalid or unsupported argument set.  Pure host code. */
size_t falcon_bwd_workspace_size(const falcon_bwd_args *args);

/* Checks every rule above without touching the GPU.  Pure host code. */
int falcon_bwd_validate(const falcon_bwd_args *args);

/* Backward pass: validates, then enqueues its kernels on `stream` (NULL =
 * the default stream).  Returns FALCON_OK or a negative status. */
int falcon_bwd(const falcon_bwd_args *args, void *stream);

/* Measurement variant of falcon_bwd, with the event convention of
 * falcon_fwd_profile: events[0] before the first kernel, events[i] after the
 * i-th.  Returns the number of kernels launched or a negative status. */
int falcon_bwd_profile(const falcon_bwd_args *args, void *stream, void *const *events, int n_events);

/* Static name of the i-th kernel falcon_bwd launches for these arguments, or
 * NULL (i out of range, invalid arguments).  Pure host code. */
const char *falcon_bwd_kernel_name(const falcon_bwd_args *args, int i);

/* Static name of the i-th kernel (0-based) that falcon_fwd launches for these
 * arguments, or NULL when i is out of range or the arguments are invalid.
 * Pure host code, no HIP call. */
const char *falcon_kernel_name(const falcon_fwd_args *args, int i);

/* Static text for a status code. */
const char *falcon_status_str(int status);

/* FALCON_ABI_VERSION of the built library. */
int falcon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FALCON_H */
