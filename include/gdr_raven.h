/* gdr_raven.h -- C ABI of the Raven routing slot-memory forward (gfx950).
 *
 * Part of libgdr.so (status codes, stream convention and ownership rules as in
 * gdr.h).  Source: "Raven: High-Recall Sequence Modeling with Sparse Memory
 * Routing", technical summary, section 2.1 (routing slot memories: M slots
 * written with per-slot strengths r_t; a dense r is a state-space model, a
 * one-hot time-indexed r with full replacement is sliding-window attention)
 * and section 2.2 (separate key and value slot states, a sigmoid router that
 * keeps the top K scores and normalises them, and the selective decay
 * exp(a_t r_t) that leaves unselected slots frozen).
 *
 * Per batch row b, head h and token t (M = slots, K = topk):
 *
 *   sel_t    = the K slots with the largest z_t (ties: the lower slot index)
 *   r_t[i]   = sigmoid(z_t[i]) / sum_{j in sel_t} sigmoid(z_t[j]),  i in sel_t
 *   lam_t[i] = exp(a_t r_t[i]) for i in sel_t, exactly 1 otherwise
 *   Sk[i]    = lam_t[i] Sk[i] + (1 - lam_t[i]) k_t       (rows of M x d_k)
 *   Sv[i]    = lam_t[i] Sv[i] + (1 - lam_t[i]) v_t       (rows of M x d_v)
 *   o_t      = sum_i softmax_i(scale * Sk[i] . q_t) Sv[i]
 *
 * The read-out is attention over the slots after the update (the page leaves
 * it open; this is the form under which the one-hot router with full
 * replacement is exactly sliding-window attention).  The router's input
 * projection z_t = W x_t is the caller's.
 */
#ifndef GDR_RAVEN_H
#define GDR_RAVEN_H

#include "gdr.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int B, T, H;      /* batch rows, tokens, heads (T >= 1; ragged T allowed)       */
  int dk, dv;       /* key and value widths: dk == dv, 64 or 128                 */
  int slots;        /* M: 64                                                     */
  int topk;         /* K: 1 .. 8                                                 */
  float scale;      /* read-out logit scale (1 / sqrt(dk) for attention)         */
  const void* q;    /* bf16 [B,T,H,dk]                                           */
  const void* k;    /* bf16 [B,T,H,dk]                                           */
  const void* v;    /* bf16 [B,T,H,dv]                                           */
  const void* z;    /* bf16 [B,T,H,slots] router logits, finite (a NaN's order is
                       unspecified)                                              */
  const float* a;   /* fp32 [B,T,H] decay rate, finite and <= 0 (a very negative
                       value replaces a selected slot outright)                  */
  const float* Sk0; /* fp32 [B,H,slots,dk] start key slots, or NULL for zero     */
  const float* Sv0; /* fp32 [B,H,slots,dv] start value slots, or NULL for zero   */
  void* o;          /* bf16 [B,T,H,dv] output (fp32 accumulation, RNE)           */
  float* Sk_out;    /* fp32 [B,H,slots,dk] final key slots, or NULL; may be Sk0  */
  float* Sv_out;    /* fp32 [B,H,slots,dv] final value slots, or NULL; may be Sv0 */
} gdr_raven_args;

/* Raven slot-memory forward on `stream` (a hipStream_t; NULL = the null
 * stream).  All pointers are device memory owned by the caller, 16-byte
 * aligned; the call allocates nothing and does not synchronise.  Every
 * argument is checked on the host before any HIP call:
 *   GDR_ERR_NULL        a required pointer is NULL
 *   GDR_ERR_SHAPE       a size is non-positive, or B*T*H overflows
 *   GDR_ERR_UNSUPPORTED dk != dv, dk not in {64, 128}, slots != 64, topk not in
 *                       [1, 8], or scale not finite
 *   GDR_ERR_ALIGN       a pointer is not 16-byte aligned
 *   GDR_ERR_ARG         an output overlaps an input it must not (S*_out may
 *                       equal S*0 exactly)
 *   GDR_ERR_HIP         the launch failed
 * Numerics: products on the matrix cores with bf16 operands (the state's
 * update coefficients as a bf16 pair, so the fp32 slot state keeps fp32
 * accuracy); router, decays and softmax in fp32.  Each 32-token chunk whose
 * decay over the chunk stays above e^-40 in every slot uses the factored form
 * exp(C_t) exp(-C_s); other chunks use exp(C_t - C_s) directly (exact, slower). */
gdr_status gdr_raven_fwd(const gdr_raven_args* a, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_RAVEN_H */
