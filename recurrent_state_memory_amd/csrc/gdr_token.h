// gdr_token.h -- token-by-token recurrence on a wave's accumulator-resident state
// rows: the exact path the chunked kernels take for a chunk whose decay leaves
// the range of the split (Gamma, Gamma^{-1}) form.
//
// The chunk-WY forms pair K+ = Gamma_r k with Kh = Gamma_r^{-1} k, so a key
// channel whose running product over one chunk falls below ~e^-87 makes
// Gamma^{-1} overflow fp32 (and bf16, which has the same exponent range).  Strong
// forgetting is part of the method: the SFDA page's register/reset construction
// (finite-state expressivity, with delta correction) drives the transition to
// zero.  So every chunk is checked: if every key channel keeps
// Gamma_L >= kMinChunkDecay the split form is exact to rounding (no intermediate
// exceeds e^40 |k|); otherwise the chunk runs here, one token at a time, with the
// state in fp32 and no reciprocal anywhere:
//
//     X = S D_t,  y = X k_t,  S = X + (beta_t w_t) v_t k_t^T - beta_t y k_t^T,
//     o_t = S q_t                                    (per value row of S).
//
// Layout (identical in both chunked kernels): lane l = 16 g + n of the wave owns
// value row n of its 16-row block; Sacc[ct][j] = S[n][16 ct + 4 g + j].
#pragma once
#include <hip/hip_runtime.h>

#include "gdr_mfma.h"

namespace gdr {

// e^-40: below this a chunk's running decay takes the token path.
constexpr float kMinChunkDecay = 4.2483543e-18f;

// True when a channel (pair) keeps the split form in range over the chunk.
// DIAG: g = (Gamma_L of channel 2p, of channel 2p + 1).  ROT2: g = Gamma_L of
// the pair as a complex number (magnitude gamma product, phase theta sum).
template <int DECAY>
__device__ inline bool decay_in_range(f32x2 g) {
  if constexpr (DECAY == 0) {
    return g.x >= kMinChunkDecay && g.y >= kMinChunkDecay;   // false for NaN
  } else {
    return g.x * g.x + g.y * g.y >= kMinChunkDecay * kMinChunkDecay;
  }
}

template <typename T>
__device__ inline f32x4 load4_f32(const T* p);
template <>
__device__ inline f32x4 load4_f32<__bf16>(const __bf16* p) {
  const bf16x4 v = *(const bf16x4*)p;
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <>
__device__ inline f32x4 load4_f32<float>(const float* p) {
  return *(const f32x4*)p;
}

// Sum over the four lanes that share n (lanes n, n + 16, n + 32, n + 48).
__device__ inline float sum_over_g(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Run tokens 0 .. ntok-1 of a chunk from raw inputs in LDS:
//   tr [ntok][DK] fp32: DIAG alpha per channel; ROT2 (gamma cos, gamma sin) per
//                       channel pair, pair p at channels 2p, 2p + 1 (DECAY 2:
//                       the lowest bit of the first value marks a reflection)
//   kr, qr [ntok][ldk]: raw keys and queries (io type)
//   vval(t): value of row n of this wave at token t, as float
//   beta[t], bw[t]: erase strength and beta * w
// emit(t, o) is called on every lane with o = o_t[n] (the same on all four g).
//
// FULL unrolls the loops over the accumulator tiles completely, so the tiles
// are addressed statically (a partial unroll indexes them at run time, a mode
// switch per access: a strong-decay forward takes 17-26 % longer that way);
// scheduling barriers keep each tile's loads in its own iteration.  The full
// unroll raises the register count of the whole kernel, which slowed the
// per-channel-decay pipelined kernel's matrix-core pass by 2.5 %, so callers
// choose it per kernel.
template <int DK, int DECAY, bool FULL = false, typename T, typename Val, typename Emit>
__device__ inline void token_steps(f32x4 (&Sacc)[DK / 16], const float* tr, const T* kr,
                                   const T* qr, int ldk, Val vval,
                                   const float* beta, const float* bw, int ntok, Emit emit) {
  constexpr int NCT = DK / 16;
  constexpr int UNR = FULL ? NCT : 4;
  const int g = (threadIdx.x & 63) >> 4;
  for (int t = 0; t < ntok; ++t) {
    const float* a = tr + t * DK + 4 * g;
    const T* kp = kr + t * ldk + 4 * g;
    float part = 0.f;
#pragma unroll UNR
    for (int ct = 0; ct < NCT; ++ct) {
      if constexpr (FULL) __builtin_amdgcn_sched_barrier(0);
      const f32x4 z = *(const f32x4*)(a + 16 * ct);
      if constexpr (DECAY == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) Sacc[ct][j] *= z[j];
      } else {
#pragma unroll
        for (int j = 0; j < 4; j += 2) {   // S times gamma [[c, -s], [s, c]] on the pair
          const float x0 = Sacc[ct][j], x1 = Sacc[ct][j + 1];
          Sacc[ct][j] = z[j] * x0 + z[j + 1] * x1;
          const float y1 = -z[j + 1] * x0 + z[j] * x1;
          if constexpr (DECAY == 2) {
            // reflection block gamma [[c, s], [s, -c]] when the lowest bit
            // of the first value is set: the second component changes sign
            Sacc[ct][j + 1] = __uint_as_float(__float_as_uint(y1) ^ ((__float_as_uint(z[j]) & 1u) << 31));
          } else {
            Sacc[ct][j + 1] = y1;
          }
        }
      }
      const f32x4 k4 = load4_f32<T>(kp + 16 * ct);
#pragma unroll
      for (int j = 0; j < 4; ++j) part += Sacc[ct][j] * k4[j];
    }
    const float y = sum_over_g(part);
    const float vn = vval(t);
    const float d = bw[t] * vn - beta[t] * y;   // beta (w v - y)
    const T* qp = qr + t * ldk + 4 * g;
    float op = 0.f;
#pragma unroll UNR
    for (int ct = 0; ct < NCT; ++ct) {
      if constexpr (FULL) __builtin_amdgcn_sched_barrier(0);
      const f32x4 k4 = load4_f32<T>(kp + 16 * ct);
      const f32x4 q4 = load4_f32<T>(qp + 16 * ct);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Sacc[ct][j] += d * k4[j];
        op += Sacc[ct][j] * q4[j];
      }
    }
    emit(t, sum_over_g(op));
  }
}

}  // namespace gdr
