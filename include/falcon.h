/*
 * falcon.h -- C ABI of the MI355X (gfx950) Falcon fast-weight library.
 *
 * The library computes the read-after-write, prefix-shifted, NLMS-normalised
 * delta rule of "Fast Weight Attention for Continual Learning" (arXiv
 * 2608.27763; section and equation numbers below are the paper's) and its
 * inner-product and per-column relatives.  For every (batch b, head h) the
 * fast state S in R^{dk x dv} evolves over t = 1..T as
 *
 *     x_t   = phi(k_{t-1})             x_1 = k_prev, or 0 on a fresh start
 *     eta_t = beta_t / (||x_t||^2 + lam_t + eps)          (Eq. 3.4)
 *             eta_t := 0 if the denominator is 0, and eta_1 := 0 on a fresh
 *             start (Section 3, indexing and causality conventions)
 *     alpha_t = min(eta_t lam_t, 1 - eps_gamma),  gamma_t = 1 - alpha_t
 *             (Section 4.3, "Decay positivity"; applied in every entry point)
 *     FALCON_1 : S_t = gamma_t S_{t-1} + eta_t x_t r_t^T, r_t = v_t - S_{t-1}^T x_t
 *     FALCON_1A: S_t = gamma_t S_{t-1} + eta_t x_t v_t^T            (Section 4.3)
 *     FALCON_2 : per-column gains beta_{t,j}: column j of S follows FALCON_1
 *                with eta_{t,j}, gamma_{t,j}                       (Section 4.2)
 *     FALCON_2A: per-column gains, additive write                  (Eq. 4.7)
 *     o_t = S_t^T phi(q_t)              (read after write, Section 4 summary)
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *    row-major with the last axis fastest, 16-byte aligned.  Layouts:
 *      phi_k, phi_q : [B, H, T, dk]     io dtype
 *      v, o         : [B, H, T, dv]     io dtype
 *      beta         : [B, H, T] (FALCON_1, FALCON_1A) or [B, H, T, dv]
 *                     (FALCON_2, FALCON_2A), float32
 *      lam          : [B, H, T]         float32
 *      S0, S_T, S   : [B, H, dk, dv]    float32 (dv fastest)
 *      k_prev       : [B, H, dk]        io dtype
 *  - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t;
 *    NULL means the legacy default stream).  The library never synchronises
 *    the device, allocates no device memory in these entry points, and keeps
 *    no global mutable state besides two process-wide settings
 *    (falcon_set_wait_limit, falcon_set_f1_launch_form), so concurrent calls
 *    on different streams are safe as long as their output buffers and
 *    workspaces do not overlap.
 *  - Every argument is validated before anything is launched; on error the
 *    call returns a negative falcon_status and touches no memory.
 *  - Launch failures reported by the HIP runtime return FALCON_ERR_HIP.
 *  - Values outside the paper's domain (beta outside (0,2), lam < 0,
 *    non-finite data) are not checked on the device: they propagate
 *    arithmetically (NaN in, NaN out).
 *  - Supported sizes: dk, dv in {16, 32, 64, 128}; chunk C in {16, 32, 64};
 *    any T >= 0 (the last chunk may be ragged); B, H >= 0.
 *  - Arithmetic: the state and every accumulation are float32.  With bf16
 *    I/O the matrix products of the chunked path take bf16 operands with
 *    float32 accumulation; with float32 I/O everything is float32.
 */
#ifndef FALCON_H_
#define FALCON_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FALCON_ABI_VERSION 1

typedef enum {
  FALCON_OK = 0,
  FALCON_ERR_NULL = -1,      /* a required pointer is NULL                    */
  FALCON_ERR_SHAPE = -2,     /* B, H, T < 0, or dk / dv not supported         */
  FALCON_ERR_DTYPE = -3,     /* io_dtype not a falcon_dtype                   */
  FALCON_ERR_CHUNK = -4,     /* chunk size not supported                      */
  FALCON_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned              */
  FALCON_ERR_WORKSPACE = -6, /* workspace missing or smaller than required   */
  FALCON_ERR_VARIANT = -7,   /* variant not a falcon_variant                  */
  FALCON_ERR_HIP = -8,       /* the HIP runtime reported an error at launch  */
  FALCON_ERR_VALUE = -9,     /* eps < 0 / not finite, eps_gamma not in (0,1) */
  FALCON_ERR_ALIAS = -10,    /* an output or the workspace overlaps another
                                argument                                     */
  FALCON_ERR_SCRATCH = -11   /* falcon_fwd_chunked_noalloc: one sequence needs
                                more than FALCON_NOALLOC_SCRATCH_BYTES        */
} falcon_status;

typedef enum {
  FALCON_1 = 1,   /* scalar NLMS regression rule (Section 4, Falcon-1)      */
  FALCON_1A = 2,  /* scalar inner-product rule   (Section 4.3, Falcon-1A)   */
  FALCON_2 = 3,   /* per-column regression rule  (Section 4.2, Falcon-2)    */
  FALCON_2A = 4   /* per-column inner-product    (Section 4.3, Falcon-2A)   */
} falcon_variant;

typedef enum {
  FALCON_F32 = 0,  /* float32 features, values and outputs */
  FALCON_BF16 = 1  /* bfloat16 features, values and outputs (RNE on store) */
} falcon_dtype;

/* Problem description (plain int32 fields so that every language binds it
 * the same way). */
typedef struct {
  int32_t B, H, T;      /* batch, heads, sequence length                    */
  int32_t dk, dv;       /* key-feature and value widths                     */
  int32_t variant;      /* a falcon_variant                                 */
  int32_t io_dtype;     /* a falcon_dtype                                   */
  float eps;            /* step-size stabiliser, >= 0 (Eq. 3.4)             */
  float eps_gamma;      /* positive-decay clamp, in (0, 1) (Section 4.3);
                           the pages give no value, 1e-6 is the default    */
} falcon_problem;

/* Version of this ABI (FALCON_ABI_VERSION of the built library). */
int32_t falcon_abi_version(void);

/* Human-readable name of a status code (static storage, never NULL). */
const char* falcon_status_string(int32_t status);

/*
 * falcon_set_wait_limit -- a process-wide setting of the library.  Some
 * kernels hand data between waves or workgroups through flags in memory;
 * every such wait is bounded and gives up after `polls` polls (default
 * 4194304, about 0.1-0.2 s).  A call in which a wait gave up does not hang:
 * it finishes and reports the failure in its results, every output element
 * and every final-state element of the affected sequences being NaN.
 * Meant for tests of that path and for debugging; calls made while it
 * changes read either value.  polls = 0 makes every such wait give up at
 * once.  Returns the previous limit, or -1 (nothing changed) for polls < 0.
 */
int32_t falcon_set_wait_limit(int32_t polls);

/*
 * falcon_set_f1_launch_form -- the other process-wide setting: how
 * falcon_fwd_chunked runs its Falcon-1 fast path (bf16 I/O, dk = dv = 64,
 * C = 64; every other case ignores it).  Both forms compute the same chunk
 * form with the same roundings and give bit-identical results (paper,
 * Section 4.2, chunk-parallel implementation; Eq. 3.3 per chunk):
 *   FALCON_F1_ONE_LAUNCH (default): one kernel in which chunk workgroups
 *     build the chunk matrices while per-sequence chain workgroups, started
 *     first, carry the state through announced chunks (plus a small fill of
 *     the hand-over flags).  Batches of more than 256 sequences (B H) run the
 *     two-launch form instead: their chains would hold too many workgroup
 *     slots;
 *   FALCON_F1_TWO_LAUNCH: the chunk matrices of all chunks, then the chains.
 * The workspace size is the same for both.  Meant for comparison and
 * debugging; calls made while it changes use either form.  Returns the
 * previous form, or -1 (nothing changed) for any other value.
 */
#define FALCON_F1_ONE_LAUNCH 0
#define FALCON_F1_TWO_LAUNCH 1
int32_t falcon_set_f1_launch_form(int32_t form);

/*
 * falcon_fwd_recurrent -- the recurrent form (paper, Section 4.6 and the
 * complexity table of the juhoplayground post: O(N) sequential scan, O(1)
 * state).  One pass over T per (b, h) with the state held on-chip.
 *
 *  S0      : initial state, or NULL for S_0 = 0.
 *  k_prev  : phi(k_0), the key feature preceding token 1, for continuing a
 *            sequence; NULL selects the fresh-start boundary x_1 = 0,
 *            eta_1 = 0 (even when S0 is not NULL).
 *  o       : output, must not overlap any input.
 *  S_T     : final state, or NULL to skip; may alias S0 exactly.
 */
falcon_status falcon_fwd_recurrent(const falcon_problem* p,
                                   const void* phi_k, const void* phi_q, const void* v,
                                   const float* beta, const float* lam,
                                   const float* S0, const void* k_prev,
                                   void* o, float* S_T, hipStream_t stream);

/*
 * falcon_fwd_chunked -- the chunk-parallel form (paper, Section 4.2
 * "Chunk-parallel implementation" and the SSD-style chunking of the
 * rainbus review: intra-chunk work in parallel, only the fixed-size state
 * passed between chunks).  Same arguments and result as
 * falcon_fwd_recurrent up to float rounding, plus the chunk size C.
 *
 *  C         : chunk length, 16, 32 or 64.
 *  workspace : device scratch of at least falcon_workspace_bytes(p, C)
 *              bytes (may be NULL when that is 0); the bytes the call uses
 *              may overlap no input and no output (FALCON_ERR_ALIAS).
 */
falcon_status falcon_fwd_chunked(const falcon_problem* p,
                                 const void* phi_k, const void* phi_q, const void* v,
                                 const float* beta, const float* lam,
                                 const float* S0, const void* k_prev,
                                 void* o, float* S_T,
                                 int32_t C, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Device scratch needed by falcon_fwd_chunked for this problem and C;
 * returns (size_t)-1 for an invalid problem. */
size_t falcon_workspace_bytes(const falcon_problem* p, int32_t C);

/* Size of the static device buffer behind falcon_fwd_chunked_noalloc. */
#define FALCON_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * falcon_fwd_chunked_noalloc -- falcon_fwd_chunked for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and results as
 * falcon_fwd_chunked, without the workspace: the kernels that need scratch
 * use a static device buffer of FALCON_NOALLOC_SCRATCH_BYTES (64 MiB) that the
 * library holds on every GPU it runs on until the process ends.  When the
 * problem needs more scratch than that, the sequences are processed in
 * groups that fit, one group after another on `stream`; a problem in which a
 * single sequence needs more returns FALCON_ERR_SCRATCH (with bf16 I/O,
 * dk = dv = 64 and C = 64: Falcon-1 beyond T = 130880 tokens, Falcon-1A
 * beyond T = 1048064).  The call allocates nothing.
 *
 * The buffer of a GPU is shared by every call on that GPU and keeps the last
 * call's contents; no part of it needs to start at zero.  Calls that overlap
 * in time on one GPU (different streams or threads without ordering) race on
 * it and must not be made.  `stream` must belong to the current device, whose
 * buffer is used.  The first call on a device looks the buffer up (the HIP
 * runtime's symbol lookup, no allocation); FALCON_ERR_HIP if that fails.
 */
falcon_status falcon_fwd_chunked_noalloc(const falcon_problem* p,
                                         const void* phi_k, const void* phi_q, const void* v,
                                         const float* beta, const float* lam,
                                         const float* S0, const void* k_prev,
                                         void* o, float* S_T, int32_t C, hipStream_t stream);

/*
 * falcon_decode_step -- one read-after-write token for every (b, h) from a
 * carried state: the rule of the paper's Section 4 naming summary (Falcon-1:
 * residual against the state before the write, Eq. 3.3; step size Eq. 3.4;
 * decay clamp of Section 4.3) applied to a single token, which is the
 * recurrent form run at inference with O(1) state per head (complexity table
 * of the juhoplayground post).  The read o = S_t^T phi(q_t) comes after the
 * write.  p->T is ignored.  Validation, status codes and stream semantics are
 * those of the forward entry points; S is both read and written, so it may
 * overlap no other argument.
 *
 *  phi_k_prev : [B, H, dk] io dtype, the PREVIOUS token's key feature x_t.
 *  phi_q, v   : [B, H, dk] / [B, H, dv] io dtype, this token's query, value.
 *  beta       : [B, H] (FALCON_1, 1A) or [B, H, dv] (FALCON_2, 2A), float32.
 *  lam        : [B, H] float32.
 *  S          : [B, H, dk, dv] float32, updated IN PLACE to S_t.
 *  is_first   : [B] bytes or NULL; a nonzero entry marks a sequence whose
 *               current token is t = 1, where eta := 0 and gamma := 1.
 *  o          : [B, H, dv] io dtype, o_t = S_t^T phi(q_t).
 */
falcon_status falcon_decode_step(const falcon_problem* p,
                                 const void* phi_k_prev, const void* phi_q, const void* v,
                                 const float* beta, const float* lam,
                                 float* S, const uint8_t* is_first,
                                 void* o, hipStream_t stream);

/*
 * falcon_bwd_chunked -- gradients of the FALCON_1 forward.  Training
 * differentiates through the update itself (paper, Section 3); this entry
 * point returns, for the scalar loss
 *
 *     L = <dO, o> + <dS_T, S_T>     (o, S_T the result of falcon_fwd_*),
 *
 * the derivatives of L with respect to every input.  It recomputes the
 * forward in 32-token chunks (Section 4.2's chunk-parallel form), runs the
 * state chain forward and the adjoint chain backward, and then the chunk-local
 * reverse mode in parallel over chunks.  All arithmetic is float32.
 *
 * Supported: variant FALCON_1, dk = dv = 64, io dtype float32 or bfloat16,
 * any T >= 0.  Other variants return FALCON_ERR_VARIANT, other widths
 * FALCON_ERR_SHAPE.  The clamp of Section 4.3 is part of the forward: where it
 * binds (eta lam > 1 - eps_gamma) gamma is constant and passes no gradient.
 *
 *  phi_k .. k_prev : the forward's inputs, as in falcon_fwd_chunked.
 *  dO      : [B, H, T, dv] io dtype, dL/do.
 *  dS_T    : [B, H, dk, dv] float32, dL/dS_T, or NULL for zero.
 *  dphi_k, dphi_q : [B, H, T, dk] float32.  dphi_k[..., T-1, :] is 0 (the
 *            last key is read by no token of this call).
 *  dv      : [B, H, T, dv] float32.
 *  dbeta, dlam : [B, H, T] float32.
 *  dS0     : [B, H, dk, dv] float32, dL/dS_0, or NULL to skip.
 *  dk_prev : [B, H, dk] float32, dL/dk_prev, or NULL to skip; ignored (not
 *            written) when k_prev is NULL.
 *  Every output must not overlap any input or another output
 *  (FALCON_ERR_ALIAS).
 *  workspace : device scratch of at least falcon_bwd_workspace_bytes(p)
 *              bytes, 16-byte aligned (per 32-token chunk per (b, h): the
 *              chunk maps, the state entering the chunk, the adjoint
 *              leaving it, the forward factors W, U, T, the gates and
 *              each row's decay gamma; 103,552 bytes).
 */
falcon_status falcon_bwd_chunked(const falcon_problem* p,
                                 const void* phi_k, const void* phi_q, const void* v,
                                 const float* beta, const float* lam,
                                 const float* S0, const void* k_prev,
                                 const void* dO, const float* dS_T,
                                 float* dphi_k, float* dphi_q, float* dv,
                                 float* dbeta, float* dlam, float* dS0, float* dk_prev,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Device scratch needed by falcon_bwd_chunked; (size_t)-1 for an invalid or
 * unsupported problem. */
size_t falcon_bwd_workspace_bytes(const falcon_problem* p);

#ifdef __cplusplus
}
#endif

#endif /* FALCON_H_ */
