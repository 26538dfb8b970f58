/*
 * gdr.h -- C ABI of the MI355X (gfx950) gated delta-rule library (libgdr.so).
 *
 * The operation.  For every batch row b and head h, a state S in R^{d_v x d_k}
 * (row i = value channel i, column j = key channel j, so that S k ~ v) is
 * carried through T tokens:
 *
 *     X_t = S_{t-1} D_t
 *     S_t = X_t (I - beta_t k_t k_t^T) + w_t beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * Sources (the pages define no API; these passages define the computation):
 *   - CARVE technical summary, section 1: the delta-rule family keeps a
 *     fixed-size matrix state with d_v rows and d_k columns.
 *   - CARVE technical summary, section 2.2: the write gate is one scalar w per
 *     head and token, broadcast over the value channels.
 *   - CARVE technical summary, section 2.3 and section 3 item 1: all gating
 *     (the decay D_t and the erase beta_t) acts on the key axis only, which is
 *     what keeps one triangular (WY-form) system per chunk valid.
 *   - SFDA technical summary, core architecture: the transition is applied
 *     before the rank-one erase; the phase-decay diag(alpha e^{i theta}) is
 *     realised as a direct sum of 2x2 rotation-decay blocks (GDR_DECAY_ROT2).
 *   - SFDA technical summary, main contributions: the exact affine chunk
 *     transfer makes the boundary state exact, hence S0 in / S_out out.
 *   - CARVE technical summary, section 2.1 and its limitations paragraph: the
 *     content-aware erase beta_t = sigmoid(b_x,t + U_b m_c), with m_c the mean
 *     of the previous chunk's outputs (none before the second chunk).
 *
 * D_t:  GDR_DECAY_DIAG  D_t = Diag(alpha_t), alpha_t in R^{d_k}.
 *       GDR_DECAY_ROT2  D_t = direct sum over j < d_k/2 of
 *                       gamma_{t,j} [[cos th, -sin th], [sin th, cos th]]
 *                       acting on key channels (2j, 2j+1), th = theta_{t,j}.
 *       GDR_DECAY_DIHEDRAL  as ROT2, except that a block whose gamma has its
 *                       sign bit set is the reflection
 *                       |gamma| [[cos th, sin th], [sin th, -cos th]]
 *                       (SFDA technical summary, finite-state expressivity:
 *                       with reflections the family realises dihedral
 *                       memory).  Products of such blocks do not commute.
 *                       Forward: bf16 io, d_k = d_v in {64, 128}, plain erase
 *                       (else GDR_ERR_UNSUPPORTED); decode: every size.  No
 *                       gated or backward variant.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers (hipMalloc / torch CUDA tensors), owned
 *     by the caller, row-major and contiguous in the layouts given below.  The
 *     library never allocates, frees or synchronises; work is enqueued on the
 *     caller's stream (a hipStream_t passed as void*, NULL = default stream)
 *     and runs asynchronously.  Inputs are only read.
 *   - Argument checks (null pointers, shapes, dtypes, alignment, supported
 *     sizes) run on the host BEFORE any HIP call and return a GDR_ERR_* code
 *     with nothing enqueued.  A failed launch returns GDR_ERR_HIP.  Faults
 *     during execution surface at the caller's next synchronisation.  No C++
 *     exception and no abort crosses this ABI.
 *   - NaN / Inf inputs are not checked; they propagate.
 *   - Calls on different streams touching disjoint outputs may overlap.
 *
 * Decay range.  Every decay factor (alpha, or the block magnitude |gamma|)
 * may take any value in [0, 1], including 0 (a full reset of that key channel,
 * the register/reset construction of the SFDA technical summary, finite-state
 * expressivity) and subnormals.  The chunked kernels pair Gamma_r k with
 * Gamma_r^{-1} k inside a block; a block in which some key channel's running
 * decay falls below e^-40 is computed token by token in fp32 instead, so no
 * legal input produces an overflow or NaN and results stay exact to rounding.
 * Such blocks run several times slower than the matrix-core path.  Factors
 * above 1 are outside the supported domain and are not checked.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 1

typedef enum {
  GDR_OK = 0,
  GDR_ERR_NULL = 1,        /* a required pointer is NULL                        */
  GDR_ERR_SHAPE = 2,       /* a size is non-positive or inconsistent            */
  GDR_ERR_DTYPE = 3,       /* unknown io dtype or decay kind                    */
  GDR_ERR_UNSUPPORTED = 4, /* valid but not built: d_k, d_v, chunk, rank        */
  GDR_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                  */
  GDR_ERR_WORKSPACE = 6,   /* workspace missing or too small                    */
  GDR_ERR_HIP = 7,         /* the HIP runtime rejected a launch                 */
  GDR_ERR_ARG = 8          /* an argument that must be NULL is set, or similar  */
} gdr_status;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;        /* q, k, v and o */
typedef enum { GDR_DECAY_DIAG = 0, GDR_DECAY_ROT2 = 1, GDR_DECAY_DIHEDRAL = 2 } gdr_decay;

/* ------------------------------------------------------------------------ */
/* Chunked forward over a sequence.                                          */
/* ------------------------------------------------------------------------ */
typedef struct gdr_fwd_args {
  int32_t B, T, H;      /* batch, tokens (>= 1), heads                         */
  int32_t dk, dv;       /* key / value channels; supported: dk == dv in        */
                        /* {32, 64, 128}                                       */
  int32_t chunk;        /* L, in {16, 32, 64, 128}.  For the content-aware     */
                        /* erase it is the window of the output mean and       */
                        /* changes the result.  Otherwise it only selects the  */
                        /* WY block size, which changes rounding, not the      */
                        /* result: bf16 io at dk in {64, 128} runs 32-token    */
                        /* blocks whatever the value; fp32 io, dk = 32, a      */
                        /* 16-token content window and T*H*dk >= 2^29 run      */
                        /* min(chunk, 64)-token blocks (32 for fp32 at         */
                        /* dk = 128).                                          */
  int32_t io_dtype;     /* gdr_dtype of q, k, v and o                          */
  int32_t decay;        /* gdr_decay                                           */
  const void *q;        /* [B,T,H,dk] io_dtype                                 */
  const void *k;        /* [B,T,H,dk] io_dtype                                 */
  const void *v;        /* [B,T,H,dv] io_dtype                                 */
  const float *alpha;   /* DIAG: [B,T,H,dk] decays in [0,1].                   */
                        /* ROT2: [B,T,H,dk/2] block magnitudes gamma in [0,1]. */
  const float *theta;   /* ROT2: [B,T,H,dk/2] angles (radians).  DIAG: NULL.   */
  const float *beta;    /* [B,T,H] erase strengths; NULL iff content-aware.    */
  const float *w;       /* [B,T,H] scalar write gates.                         */
  const float *beta_logit; /* content-aware: b_x [B,T,H]; otherwise NULL.      */
  const float *ub_down; /* content-aware: B_h [H, ub_rank, dv]; else NULL.     */
  const float *ub_up;   /* content-aware: a_h [H, ub_rank];     else NULL.     */
                        /* (U_b m = a_h^T (B_h m), one scalar per head)        */
  int32_t ub_rank;      /* content-aware: rank r in [1, 64]; else ignored.     */
  int32_t reserved0;
  float *m_carry;       /* content-aware only, may be NULL: [B,H,dv] fp32.     */
                        /* In: mean output of the chunk before this call (used */
                        /* for the first chunk; NULL = zero).  Out: mean       */
                        /* output of this call's last chunk.  Non-NULL needs   */
                        /* T % chunk == 0.                                     */
  const float *S0;      /* [B,H,dv,dk] fp32 initial state, or NULL for zero.   */
  void *o;              /* [B,T,H,dv] io_dtype output.                         */
  float *S_out;         /* [B,H,dv,dk] fp32 final state, or NULL.  May alias   */
                        /* S0 exactly (in-place update); no partial overlap.   */
  void *workspace;      /* unused by this version: pass NULL / 0.              */
  size_t workspace_bytes;
} gdr_fwd_args;

/* Bytes of workspace gdr_chunk_fwd needs for these arguments (0 today). */
size_t gdr_chunk_fwd_workspace(const gdr_fwd_args *a);

/* Enqueue the forward.  Returns GDR_OK once the kernels are enqueued. */
gdr_status gdr_chunk_fwd(const gdr_fwd_args *a, void *hip_stream);

/* ------------------------------------------------------------------------ */
/* Forward with the gate activation and the q/k normalisation in the kernel. */
/* ------------------------------------------------------------------------ */
/* CARVE technical summary, section 2.3: the decay activation is computed in
 * the kernel from its pre-activation instead of being stored for the whole
 * sequence.  Here
 *
 *     decay_t = exp(-a_h * softplus(x_t)),   softplus(x) = log(1 + e^x),
 *
 * per key channel (DIAG) or per 2x2 block magnitude (ROT2, with the angles in
 * gdr_fwd_args.theta as before), so every decay lies in (0, 1] for a_h >= 0.
 * With qk_l2norm, q and k are raw and each token's q and k are divided by
 * sqrt(sum of squares over d_k + 1e-6) in the kernel.  The result equals
 * gdr_chunk_fwd on the activated, normalised inputs up to rounding.  The
 * decay pre-activation in bf16 halves the decay's bytes (2 instead of 4 per
 * channel and token).
 *
 * Supported: io_dtype BF16, dk == dv in {64, 128}, the plain erase (beta given,
 * no content-aware arguments), T * H * dk < 2^29; otherwise
 * GDR_ERR_UNSUPPORTED.  gdr_fwd_args.alpha must be NULL (the decay comes from
 * decay_x); every other field keeps its meaning. */
typedef struct gdr_gate_args {
  const void *decay_x;  /* bf16 pre-activation: DIAG [B,T,H,dk], ROT2 [B,T,H,dk/2] */
  const float *decay_a; /* [H] per-head scale a_h >= 0 (fp32)                      */
  int32_t qk_l2norm;    /* nonzero: normalise each token's q and k in the kernel   */
  int32_t reserved;     /* must be 0                                               */
} gdr_gate_args;

gdr_status gdr_chunk_fwd_gated(const gdr_fwd_args *a, const gdr_gate_args *g, void *hip_stream);

/* ------------------------------------------------------------------------ */
/* Backward of the forward (plain erase).                                     */
/* ------------------------------------------------------------------------ */
/* The gradients that training needs (the CARVE technical summary reports
 * training throughput; its section 3 item 5 concerns gradient norms): for a
 * scalar loss L with dL/do = grad_o and dL/dS_T = grad_S (NULL: zero), the
 * call writes dL/dq, dL/dk, dL/dv, dL/d(decay) -- alpha (DIAG), or gamma and
 * theta (ROT2) -- dL/dbeta, dL/dw and dL/dS0.  The pages give no backward
 * algorithm; this one is the adjoint of the chunk (WY) form of the forward.
 *
 * It recomputes the forward (storing the state at the start of every 32-token
 * block in the workspace), then runs the blocks in reverse.  Products use
 * fp32 operands; the block-start states come from the forward's bf16 matrix
 * products, so the gradients carry the forward's rounding.
 *
 * Supported: BF16 q, k, v and grad_o; dk == dv in {64, 128}; T * H * dk <
 * 2^29; otherwise GDR_ERR_UNSUPPORTED.  Range: every decay in [0, 1] is
 * supported.  A head with a 32-token block whose decay product in some key
 * channel (or pair) falls below e^-40 is redone token by token in fp32 with no
 * division (exact for decays of 0); such a head costs several times its block
 * form (about 5x the whole call when every head needs it).
 *
 * Layouts (fp32 gradients, same shapes as the inputs):
 *   grad_q, grad_k [B,T,H,dk]; grad_v [B,T,H,dv]; grad_alpha as alpha
 *   ([B,T,H,dk] DIAG, [B,T,H,dk/2] ROT2); grad_theta as theta (ROT2, else
 *   NULL); grad_beta, grad_w [B,T,H]; grad_S0 [B,H,dv,dk] (may be NULL).
 * workspace: device memory of at least gdr_chunk_bwd_workspace(a) bytes,
 * 256-byte aligned; its contents on entry do not matter. */
typedef struct gdr_bwd_args {
  int32_t B, T, H, dk, dv;
  gdr_decay decay;
  const void *q, *k, *v;        /* bf16, as gdr_fwd_args                      */
  const float *alpha, *theta;   /* as gdr_fwd_args                            */
  const float *beta, *w;        /* [B,T,H]                                    */
  const float *S0;              /* [B,H,dv,dk] or NULL (zeros)                */
  const void *grad_o;           /* [B,T,H,dv] bf16                            */
  const float *grad_S;          /* [B,H,dv,dk] or NULL (zeros)                */
  float *grad_q, *grad_k, *grad_v;
  float *grad_alpha, *grad_theta;
  float *grad_beta, *grad_w;
  float *grad_S0;               /* or NULL                                    */
  void *workspace;
  size_t workspace_bytes;
} gdr_bwd_args;

/* Bytes of workspace the call needs (0 when the arguments are invalid). */
size_t gdr_chunk_bwd_workspace(const gdr_bwd_args *a);

gdr_status gdr_chunk_bwd(const gdr_bwd_args *a, void *hip_stream);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same backward on
 * a scratch array inside the library (256 MiB per GPU, held until the process
 * ends) instead of a caller workspace.  a->workspace must be NULL and
 * a->workspace_bytes 0 (else GDR_ERR_ARG); problems whose
 * gdr_chunk_bwd_workspace(a) exceeds 256 MiB return GDR_ERR_WORKSPACE.  Calls
 * that overlap on one GPU share the array and race.  Allocates nothing. */
gdr_status gdr_chunk_bwd_noalloc(const gdr_bwd_args *a, void *hip_stream);

/* Backward of gdr_chunk_fwd_gated: the gradients of the same loss when the
 * decay arrives as its pre-activation (decay = exp(-a_h softplus(x))) and, with
 * qk_l2norm, q and k are raw and normalised per token (CARVE technical summary,
 * section 2.3: the activation computed where it is used).  It runs the plain
 * backward on the activated, normalised inputs and carries the gradients back
 * by the chain rule:
 *   dL/dx = dL/d(decay) decay (-a_h) sigmoid(x),
 *   dL/da_h = sum over batch rows, tokens and channels of
 *             dL/d(decay) decay (-softplus(x)),
 *   dL/dy = (g - u (u . g)) / n   (y = q or k, n = sqrt(y . y + 1e-6), u = y / n,
 *                                  g the gradient of y / n).
 * Arguments: a as for gdr_chunk_bwd, except that a->alpha and a->grad_alpha
 * must be NULL (GDR_ERR_ARG otherwise); q and k are the raw inputs when
 * g->qk_l2norm, and grad_q, grad_k are taken with respect to them.  g as for
 * gdr_chunk_fwd_gated.  gg->grad_decay_x (fp32, decay_x's shape) and
 * gg->grad_decay_a ([H] fp32) receive the gate gradients; theta's gradient
 * (ROT2) goes to a->grad_theta as before.  The workspace holds the activated
 * decay, the normalised q and k, their gradients, one fp32 per token-head, and
 * the plain backward's workspace: at least gdr_chunk_bwd_gated_workspace bytes
 * (0 when the arguments are invalid).  decay_x, decay_a and the gate
 * gradients must be 4-byte aligned (GDR_ERR_ALIGN otherwise).  Supported as
 * gdr_chunk_bwd. */
typedef struct gdr_gate_grads {
  float *grad_decay_x;  /* as decay_x: DIAG [B,T,H,dk], ROT2 [B,T,H,dk/2] */
  float *grad_decay_a;  /* [H]                                            */
} gdr_gate_grads;

size_t gdr_chunk_bwd_gated_workspace(const gdr_bwd_args *a, const gdr_gate_args *g);
gdr_status gdr_chunk_bwd_gated(const gdr_bwd_args *a, const gdr_gate_args *g,
                               const gdr_gate_grads *gg, void *hip_stream);

/* ------------------------------------------------------------------------ */
/* Single-token decode step on N independent states, in place.               */
/* ------------------------------------------------------------------------ */
typedef struct gdr_step_args {
  int32_t N, H;         /* states, heads                                       */
  int32_t dk, dv;       /* dk == dv in {32, 64, 128}                           */
  int32_t io_dtype;     /* gdr_dtype of q, k, v and o                          */
  int32_t decay;        /* gdr_decay                                           */
  const void *q;        /* [N,H,dk]                                            */
  const void *k;        /* [N,H,dk]                                            */
  const void *v;        /* [N,H,dv]                                            */
  const float *alpha;   /* DIAG [N,H,dk]; ROT2 gamma [N,H,dk/2]; in [0,1]      */
  const float *theta;   /* ROT2 [N,H,dk/2]; DIAG NULL                          */
  const float *beta;    /* [N,H]                                               */
  const float *w;       /* [N,H]                                               */
  float *S;             /* [N,H,dv,dk] fp32, read and overwritten with S_t     */
  void *o;              /* [N,H,dv] io_dtype, o = S_t q                        */
} gdr_step_args;

/* One token of the recurrence (same definition as above) for each state. */
gdr_status gdr_step_decode(const gdr_step_args *a, void *hip_stream);

/* ------------------------------------------------------------------------ */
const char *gdr_status_str(gdr_status s);   /* static string, never NULL */
int gdr_abi_version(void);                   /* == GDR_ABI_VERSION        */

#ifdef __cplusplus
}
#endif
#endif /* GDR_H_ */
