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
typedef enum { GDR_DECAY_DIAG = 0, GDR_DECAY_ROT2 = 1 } gdr_decay;

/* ------------------------------------------------------------------------ */
/* Chunked forward over a sequence.                                          */
/* ------------------------------------------------------------------------ */
typedef struct gdr_fwd_args {
  int32_t B, T, H;      /* batch, tokens (>= 1), heads                         */
  int32_t dk, dv;       /* key / value channels; supported: dk == dv in        */
                        /* {32, 64, 128}                                       */
  int32_t chunk;        /* L, in {16, 32, 64, 128}.  For the content-aware     */
                        /* erase it is the window of the output mean and       */
                        /* changes the result.  Otherwise it is the WY block   */
                        /* size and changes only rounding; 128 runs as two     */
                        /* 64-token blocks.                                    */
  int32_t io_dtype;     /* gdr_dtype of q, k, v and o                          */
  int32_t decay;        /* gdr_decay                                           */
  const void *q;        /* [B,T,H,dk] io_dtype                                 */
  const void *k;        /* [B,T,H,dk] io_dtype                                 */
  const void *v;        /* [B,T,H,dv] io_dtype                                 */
  const float *alpha;   /* DIAG: [B,T,H,dk] decays in (0,1].                   */
                        /* ROT2: [B,T,H,dk/2] block magnitudes gamma in (0,1]. */
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
  const float *alpha;   /* DIAG [N,H,dk]; ROT2 gamma [N,H,dk/2]                */
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
