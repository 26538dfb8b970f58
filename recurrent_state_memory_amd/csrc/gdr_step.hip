// gdr_step.hip -- single-token decode step on a batch of states, in place.
//
// For each state S (d_v x d_k) and its token: X = S D, y = X k,
// S' = X + beta (w v - y) k^T, o = S' q, i.e. one token of the recurrence
// (SFDA technical summary, core architecture, in the d_v x d_k orientation of
// the CARVE technical summary, section 1).  Each value row of S is independent:
// it is read once and written once, so the step is bound by HBM bandwidth.
//
// Layout: one workgroup per (state, head).  A value row of d_k fp32 is split
// over d_k/8 consecutive lanes, eight channels (two 16-byte loads) per lane; a
// 2x2 rotation block never straddles lanes.  All rows of the workgroup are
// loaded before any is computed to keep many loads in flight.
#include "gdr_kernels.h"
#include "gdr_mfma.h"

namespace gdr {

template <typename T>
__device__ inline void load8f(const T* p, float (&x)[8]);
template <>
__device__ inline void load8f<__bf16>(const __bf16* p, float (&x)[8]) {
  const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
template <>
__device__ inline void load8f<float>(const float* p, float (&x)[8]) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

template <typename T, int DK, int DV, int DECAY>
__global__ __launch_bounds__((DV * DK / 8) < 256 ? (DV * DK / 8) : 256) void gdr_step_kernel(
    StepParams p) {
  constexpr int LPR = DK / 8;                       // lanes per value row
  constexpr int NTH = (DV * LPR) < 256 ? (DV * LPR) : 256;
  constexpr int RPP = NTH / LPR;                    // rows per pass
  constexpr int NPASS = DV / RPP;
  static_assert(NPASS * RPP == DV, "row split");

  const int unit = blockIdx.x;                      // (state, head)
  const int tid = threadIdx.x;
  const int lr = tid % LPR, rw = tid / LPR;
  const int c0 = 8 * lr;

  const T* gq = (const T*)p.q + (size_t)unit * DK;
  const T* gk = (const T*)p.k + (size_t)unit * DK;
  const T* gv = (const T*)p.v + (size_t)unit * DV;
  float* S = p.S + (size_t)unit * DV * DK;

  float srow[NPASS][8];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const float* src = S + (size_t)(ps * RPP + rw) * DK + c0;
    const f32x4 a = *(const f32x4*)src, b = *(const f32x4*)(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      srow[ps][i] = a[i];
      srow[ps][4 + i] = b[i];
    }
  }
  float kx[8], qx[8];
  load8f<T>(gk + c0, kx);
  load8f<T>(gq + c0, qx);
  float vr[NPASS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) vr[ps] = to_f32(gv[ps * RPP + rw]);
  const float beta = p.beta[unit], wg = p.w[unit];

  // DIAG: d0 = alpha; ROT2: d0 = (gamma cos, gamma sin) pairs; DECAY 2 (rotation
  // and reflection blocks): the same with |gamma|, refl[j] set where gamma's
  // sign bit is (the block |gamma| [[c, s], [s, -c]])
  float d0[8], d1[4];
  unsigned refl[4] = {0u, 0u, 0u, 0u};
  if constexpr (DECAY == 0) {
    const float* a = p.alpha + (size_t)unit * DK + c0;
    const f32x4 x = *(const f32x4*)a, y = *(const f32x4*)(a + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d0[i] = x[i];
      d0[4 + i] = y[i];
    }
  } else {
    const float* gm = p.alpha + (size_t)unit * (DK / 2) + c0 / 2;
    const float* th = p.theta + (size_t)unit * (DK / 2) + c0 / 2;
    const f32x4 x = *(const f32x4*)gm, y = *(const f32x4*)th;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float sn, cs;
      sincosf(y[j], &sn, &cs);
      const float g = DECAY == 2 ? __builtin_fabsf(x[j]) : x[j];
      if (DECAY == 2) refl[j] = __float_as_uint(x[j]) >> 31;
      d0[2 * j] = g * cs;
      d0[2 * j + 1] = g * sn;
    }
    (void)d1;
  }

  T* go = (T*)p.o + (size_t)unit * DV;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    float x[8];
    if constexpr (DECAY == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = srow[ps][i] * d0[i];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gc = d0[2 * j], gs = d0[2 * j + 1];
        const float s0 = srow[ps][2 * j], s1 = srow[ps][2 * j + 1];
        x[2 * j] = gc * s0 + gs * s1;
        x[2 * j + 1] = refl[j] ? gs * s0 - gc * s1 : -gs * s0 + gc * s1;
      }
    }
    float y = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) y += x[i] * kx[i];
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) y += __shfl_xor(y, off);
    const float e = beta * (wg * vr[ps] - y);
    float on = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] += e * kx[i];
      on += x[i] * qx[i];
    }
    float* dst = S + (size_t)(ps * RPP + rw) * DK + c0;
    *(f32x4*)dst = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4*)(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) on += __shfl_xor(on, off);
    if (lr == 0) go[ps * RPP + rw] = (T)on;
  }
}

template <typename T, int DK, int DECAY>
static hipError_t step_launch(const StepParams& p, hipStream_t s) {
  constexpr int LPR = DK / 8;
  constexpr int NTH = (DK * LPR) < 256 ? (DK * LPR) : 256;
  hipLaunchKernelGGL((gdr_step_kernel<T, DK, DK, DECAY>), dim3(p.N * p.H), dim3(NTH), 0, s, p);
  return hipGetLastError();
}

template <typename T, int DECAY>
static hipError_t step_dk(const StepParams& p, hipStream_t s) {
  switch (p.DK) {
    case 32: return step_launch<T, 32, DECAY>(p, s);
    case 64: return step_launch<T, 64, DECAY>(p, s);
    case 128: return step_launch<T, 128, DECAY>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_step(const StepParams& p, hipStream_t s) {
  if (p.io_bf16) {
    if (p.decay == 2) return step_dk<__bf16, 2>(p, s);
    return p.decay ? step_dk<__bf16, 1>(p, s) : step_dk<__bf16, 0>(p, s);
  }
  if (p.decay == 2) return step_dk<float, 2>(p, s);
  return p.decay ? step_dk<float, 1>(p, s) : step_dk<float, 0>(p, s);
}

}  // namespace gdr
