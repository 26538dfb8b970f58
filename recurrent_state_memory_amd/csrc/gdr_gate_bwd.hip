// gdr_gate_bwd.hip -- the gated forward's decay activation and q/k
// normalisation around the plain backward, gfx950.
//
// The gated forward (CARVE technical summary, section 2.3: the decay
// activation computed where it is used) runs the recurrence on
//     decay = exp(-a_h softplus(x)),   q / n(q),  k / n(k),   n(y) = sqrt(y . y + 1e-6).
// Its gradients are the plain backward's at those activated, normalised
// inputs, carried back by the chain rule:
//     dL/dx   = dL/d(decay) * decay * (-a_h) * sigmoid(x)
//     dL/da_h = sum over (b, t, channels) of dL/d(decay) * decay * (-softplus(x))
//     dL/dy   = (g - u (u . g)) / n(y),   u = y / n(y),  g = dL/d(y / n(y)).
// gate_prep_kernel forms the decay (fp32) and the normalised q, k (bf16) for
// the plain backward; gate_chain_kernel applies the chain rule; the per-head
// scale's gradient is summed over rows in a fixed order by gate_a_kernel.
// One wave per token-head row; the row's dot products reduce over the wave.
#include <hip/hip_runtime.h>

#include "gdr_kernels.h"

namespace gdr {
namespace gate {
namespace {

constexpr float kEps = 1e-6f;   // as the forward's normalisation
constexpr int kRows = 4;        // rows (waves) per workgroup

__device__ inline float bf2f(const void* p, size_t i) { return (float)((const __bf16*)p)[i]; }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// log(1 + e^x) without overflow, and without losing small values
__device__ inline float softplus(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

// Per-lane part of y . y over a row of DK bf16 values (lane l holds l, l + 64, ...).
template <int DK>
__device__ inline float row_sumsq(const void* y, size_t base, int l) {
  float s = 0.f;
#pragma unroll
  for (int i = l; i < DK; i += 64) {
    const float v = bf2f(y, base + i);
    s += v * v;
  }
  return s;
}

// bf16 pair <-> two floats
__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int DK>
__global__ __launch_bounds__(64 * kRows) void gate_prep_kernel(GateBwdParams p) {
  const int l = threadIdx.x & 63;
  const size_t rows = (size_t)p.B * p.T * p.H;
  const size_t row = (size_t)blockIdx.x * kRows + (threadIdx.x >> 6);
  if (row >= rows) return;   // whole waves leave together
  const int h = (int)(row % p.H);
  const float a = p.a[h];
  if (DK == 128 && p.C == 128) {
    // two neighbouring channels per lane; every load is issued before the
    // first store (stores could alias the inputs as far as the compiler
    // knows, so loads after a store would wait for one more round trip)
    const size_t i = row * 128 + 2 * l;
    const uint32_t ux = *(const uint32_t*)((const __bf16*)p.x + i);
    uint32_t uq = 0u, uk = 0u;
    if (p.norm) {
      uq = *(const uint32_t*)((const __bf16*)p.q_raw + i);
      uk = *(const uint32_t*)((const __bf16*)p.k_raw + i);
    }
    *(float2*)(p.alpha + i) = float2{expf(-a * softplus(bf_lo(ux))), expf(-a * softplus(bf_hi(ux)))};
    if (p.norm) {
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const uint32_t u = which ? uk : uq;
        const float y0 = bf_lo(u), y1 = bf_hi(u);
        const float inv = 1.f / sqrtf(wave_sum(y0 * y0 + y1 * y1) + kEps);
        const __bf16 n0 = (__bf16)(y0 * inv), n1 = (__bf16)(y1 * inv);
        *(uint32_t*)((__bf16*)(which ? p.k_n : p.q_n) + i) =
            (uint32_t)__builtin_bit_cast(uint16_t, n0) | ((uint32_t)__builtin_bit_cast(uint16_t, n1) << 16);
      }
    }
    return;
  }
  if (p.C == 128) {   // two neighbouring channels per lane: 4-byte loads, 8-byte stores
    const size_t i = row * 128 + 2 * l;
    const uint32_t u = *(const uint32_t*)((const __bf16*)p.x + i);
    *(float2*)(p.alpha + i) = float2{expf(-a * softplus(bf_lo(u))), expf(-a * softplus(bf_hi(u)))};
  } else {
    for (int j = l; j < p.C; j += 64) {
      const size_t i = row * p.C + j;
      p.alpha[i] = expf(-a * softplus(bf2f(p.x, i)));
    }
  }
  if (p.norm) {
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const void* y = which ? p.k_raw : p.q_raw;
      __bf16* yn = (__bf16*)(which ? p.k_n : p.q_n);
      const size_t base = row * DK;
      if constexpr (DK == 128) {   // channels 2l, 2l + 1
        const uint32_t u = *(const uint32_t*)((const __bf16*)y + base + 2 * l);
        const float y0 = bf_lo(u), y1 = bf_hi(u);
        const float inv = 1.f / sqrtf(wave_sum(y0 * y0 + y1 * y1) + kEps);
        const __bf16 n0 = (__bf16)(y0 * inv), n1 = (__bf16)(y1 * inv);
        *(uint32_t*)(yn + base + 2 * l) =
            (uint32_t)__builtin_bit_cast(uint16_t, n0) | ((uint32_t)__builtin_bit_cast(uint16_t, n1) << 16);
      } else {
        const float inv = 1.f / sqrtf(wave_sum(row_sumsq<DK>(y, base, l)) + kEps);
#pragma unroll
        for (int i = l; i < DK; i += 64) yn[base + i] = (__bf16)(bf2f(y, base + i) * inv);
      }
    }
  }
}

template <int DK>
__global__ __launch_bounds__(64 * kRows) void gate_chain_kernel(GateBwdParams p) {
  const int l = threadIdx.x & 63;
  const size_t rows = (size_t)p.B * p.T * p.H;
  const size_t row = (size_t)blockIdx.x * kRows + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int h = (int)(row % p.H);
  const float a = p.a[h];
  if (DK == 128 && p.C == 128) {
    // channels 2l, 2l + 1; every load issued before the first store, as in
    // gate_prep_kernel
    const size_t i = row * 128 + 2 * l;
    const uint32_t ux = *(const uint32_t*)((const __bf16*)p.x + i);
    const float2 gal = *(const float2*)(p.grad_alpha + i), al = *(const float2*)(p.alpha + i);
    uint32_t uy[2] = {0u, 0u};
    float2 gn[2] = {};
    if (p.norm) {
      uy[0] = *(const uint32_t*)((const __bf16*)p.q_raw + i);
      uy[1] = *(const uint32_t*)((const __bf16*)p.k_raw + i);
      gn[0] = *(const float2*)(p.grad_qn + i);
      gn[1] = *(const float2*)(p.grad_kn + i);
    }
    const float x0 = bf_lo(ux), x1 = bf_hi(ux);
    const float gd0 = gal.x * al.x, gd1 = gal.y * al.y;   // dL/d(decay) * decay
    // grad_decay_x is only 4-byte aligned: two 4-byte stores
    p.grad_x[i] = gd0 * (-a) * (1.f / (1.f + expf(-x0)));
    p.grad_x[i + 1] = gd1 * (-a) * (1.f / (1.f + expf(-x1)));
    const float ga = wave_sum(-(gd0 * softplus(x0) + gd1 * softplus(x1)));
    if (l == 0) p.ga_rows[row] = ga;
    if (p.norm) {
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const float y0 = bf_lo(uy[which]), y1 = bf_hi(uy[which]);
        const float inv = 1.f / sqrtf(wave_sum(y0 * y0 + y1 * y1) + kEps);
        const float u0 = y0 * inv, u1 = y1 * inv;
        const float ug = wave_sum(u0 * gn[which].x + u1 * gn[which].y);
        *(float2*)((which ? p.grad_k : p.grad_q) + i) = float2{(gn[which].x - u0 * ug) * inv, (gn[which].y - u1 * ug) * inv};
      }
    }
    return;
  }
  float ga = 0.f;
  for (int j = l; j < p.C; j += 64) {
    const size_t i = row * p.C + j;
    const float x = bf2f(p.x, i);
    const float gd = p.grad_alpha[i] * p.alpha[i];   // dL/d(decay) * decay
    p.grad_x[i] = gd * (-a) * (1.f / (1.f + expf(-x)));
    ga -= gd * softplus(x);
  }
  ga = wave_sum(ga);
  if (l == 0) p.ga_rows[row] = ga;
  if (p.norm) {
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const void* y = which ? p.k_raw : p.q_raw;
      const float* gn = which ? p.grad_kn : p.grad_qn;
      float* gy = which ? p.grad_k : p.grad_q;
      const size_t base = row * DK;
      const float inv = 1.f / sqrtf(wave_sum(row_sumsq<DK>(y, base, l)) + kEps);
      float ug = 0.f;
#pragma unroll
      for (int i = l; i < DK; i += 64) ug += bf2f(y, base + i) * inv * gn[base + i];
      ug = wave_sum(ug);
#pragma unroll
      for (int i = l; i < DK; i += 64) gy[base + i] = (gn[base + i] - bf2f(y, base + i) * inv * ug) * inv;
    }
  }
}

// dL/da_h: the rows of head h (every H-th row), summed in a fixed order.
__global__ __launch_bounds__(256) void gate_a_kernel(GateBwdParams p) {
  __shared__ float part[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const size_t n = (size_t)p.B * p.T;   // rows of one head
  float s = 0.f;
  for (size_t i = tid; i < n; i += 256) s += p.ga_rows[i * p.H + h];
  part[tid] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) p.grad_a[h] = part[0];
}

}  // namespace
}  // namespace gate

hipError_t launch_gate_prep(const GateBwdParams& p, hipStream_t s) {
  const size_t rows = (size_t)p.B * p.T * p.H;
  const dim3 grid((unsigned)((rows + gate::kRows - 1) / gate::kRows));
  if (p.DK == 128) hipLaunchKernelGGL(gate::gate_prep_kernel<128>, grid, dim3(64 * gate::kRows), 0, s, p);
  else if (p.DK == 64) hipLaunchKernelGGL(gate::gate_prep_kernel<64>, grid, dim3(64 * gate::kRows), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gate_chain(const GateBwdParams& p, hipStream_t s) {
  const size_t rows = (size_t)p.B * p.T * p.H;
  const dim3 grid((unsigned)((rows + gate::kRows - 1) / gate::kRows));
  if (p.DK == 128) hipLaunchKernelGGL(gate::gate_chain_kernel<128>, grid, dim3(64 * gate::kRows), 0, s, p);
  else if (p.DK == 64) hipLaunchKernelGGL(gate::gate_chain_kernel<64>, grid, dim3(64 * gate::kRows), 0, s, p);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gate::gate_a_kernel, dim3(p.H), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace gdr
