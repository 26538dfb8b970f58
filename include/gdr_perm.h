/* gdr_perm.h -- C ABI of the delta rule with partial-permutation transitions
 * (gfx950).
 *
 * Part of libgdr.so (status codes, stream convention and ownership rules as in
 * gdr.h).  Source: "Semidirect Fourier Delta Attention", technical summary,
 * "finite-state expressivity": with partial permutations as the structured
 * control in place of the phase blocks, the kernel-compatible family realises
 * a bounded stack.
 *
 * Per batch row b, head h and token t, with S in R^{d_v x d_k} (rows = value
 * channels, columns = key channels, as in gdr.h):
 *
 *   X_t[:, j] = S[:, src_t[j]]   if 0 <= src_t[j] < d_k, else 0
 *   S        = X_t + beta_t (w_t v_t - X_t k_t) k_t^T
 *   o_t      = S q_t
 *
 * An injective src_t is a partial permutation (for example a stack push: every
 * channel one deeper, channel 0 emptied; a pop: one channel up); any map is
 * computed by the same rule.  Products of such transitions are singular, so
 * there is no chunk-parallel split form: the kernel walks the tokens in order,
 * all value rows of all heads in parallel.
 */
#ifndef GDR_PERM_H
#define GDR_PERM_H

#include <stdint.h>

#include "gdr.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int B, T, H;        /* batch rows, tokens (>= 1), heads                        */
  int dk, dv;         /* dk in {64, 128}; dv a multiple of 32, at most 256       */
  const void* q;      /* bf16 [B,T,H,dk]                                          */
  const void* k;      /* bf16 [B,T,H,dk]                                          */
  const void* v;      /* bf16 [B,T,H,dv]                                          */
  const int16_t* src; /* int16 [B,T,H,dk] source key channel of each channel, or
                         a value outside [0, dk) for a zero column              */
  const float* beta;  /* fp32 [B,T,H] erase strength                              */
  const float* w;     /* fp32 [B,T,H] write gate                                  */
  const float* S0;    /* fp32 [B,H,dv,dk] start state, or NULL for zero           */
  void* o;            /* bf16 [B,T,H,dv] output                                   */
  float* S_out;       /* fp32 [B,H,dv,dk] final state, or NULL; may equal S0      */
} gdr_perm_args;

/* Forward on `stream` (a hipStream_t; NULL = the null stream).  Device
 * pointers owned by the caller, 16-byte aligned; the call allocates nothing and
 * does not synchronise.  Checked on the host before any HIP call:
 *   GDR_ERR_NULL        a required pointer is NULL
 *   GDR_ERR_SHAPE       a size is non-positive, or B*T*H overflows
 *   GDR_ERR_UNSUPPORTED dk not in {64, 128}, or dv not a multiple of 32 in
 *                       [32, 256]
 *   GDR_ERR_ALIGN       a pointer is not 16-byte aligned
 *   GDR_ERR_ARG         S_out overlaps S0 without being equal to it
 *   GDR_ERR_HIP         the launch failed
 * Numerics: fp32 state and arithmetic (q, k, v are read as bf16), o rounded to
 * bf16 (RNE). */
gdr_status gdr_perm_fwd(const gdr_perm_args* a, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_PERM_H */
