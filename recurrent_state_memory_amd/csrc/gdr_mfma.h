// gdr_mfma.h -- CDNA4 (gfx950) matrix-core fragments shared by the kernels.
//
// Every contraction uses 16x16 output tiles with fp32 accumulation and a
// 32-wide contraction step:
//   bf16 operands: one v_mfma_f32_16x16x32_bf16 per step,
//   fp32 operands: eight v_mfma_f32_16x16x4_f32 per step (full fp32 inputs).
//
// Lane l of a 64-wide wavefront, with n = l % 16 and g = l / 16:
//   accumulator tile C (16x16 fp32): lane holds C[4g + j][n], j = 0..3.
//   operand A (16 x 32): lane holds row n, eight contraction slots.
//   operand B (32 x 16): lane holds column n, the same eight slots.
// Only the pairing of A's and B's slots matters for a contraction, so two slot
// maps are used:
//   "plain": slot s <-> k = 8g + s                      (16-byte LDS reads)
//   "cb"   : slot s <-> k = 4g + s        (s < 4)
//                       k = 16 + 4g + s-4 (s >= 4)      (two 8-byte reads)
// The cb map is exactly what two stacked accumulator tiles hold (rows 4g..4g+3
// of the upper and of the lower tile), so an accumulator can feed the next
// contraction as its B operand without leaving registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ inline int lane_id() { return threadIdx.x & 63; }

// Workgroup barrier that orders LDS only.  All cross-wave communication in the
// kernels goes through LDS, so global loads (prefetches) and global stores
// (outputs) stay in flight across it; __syncthreads() would wait for them.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T>
struct Op;

template <>
struct Op<__bf16> {
  using frag = bf16x8;
  using half4 = bf16x4;
  static __device__ inline void mma(f32x4& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ inline frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
    return z;
  }
  static __device__ inline half4 load4(const __bf16* p) { return *(const bf16x4*)p; }
  static __device__ inline frag load8(const __bf16* p) { return *(const bf16x8*)p; }
  static __device__ inline frag join(half4 lo, half4 hi) {
    frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = lo[i];
      f[4 + i] = hi[i];
    }
    return f;
  }
  static __device__ inline frag neg(frag f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = -f[i];
    return f;
  }
  static __device__ inline frag from_acc(const f32x4& lo, const f32x4& hi) {
    frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = (__bf16)lo[i];
      f[4 + i] = (__bf16)hi[i];
    }
    return f;
  }
  static __device__ inline frag from_acc_half(const f32x4& lo) {
    frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = (__bf16)lo[i];
      f[4 + i] = (__bf16)0.0f;
    }
    return f;
  }
};

template <>
struct Op<float> {
  using frag = f32x8;
  using half4 = f32x4;
  static __device__ inline void mma(f32x4& c, const frag& a, const frag& b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  }
  static __device__ inline frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = 0.0f;
    return z;
  }
  static __device__ inline half4 load4(const float* p) { return *(const f32x4*)p; }
  static __device__ inline frag load8(const float* p) {
    f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    return join(a, b);
  }
  static __device__ inline frag join(half4 lo, half4 hi) {
    frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = lo[i];
      f[4 + i] = hi[i];
    }
    return f;
  }
  static __device__ inline frag neg(frag f) { return -f; }
  static __device__ inline frag from_acc(const f32x4& lo, const f32x4& hi) { return join(lo, hi); }
  static __device__ inline frag from_acc_half(const f32x4& lo) {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return join(lo, z);
  }
};

// A/B operand, plain slot map: rows row0 + n, contraction k0 + 8g + s.
template <typename T>
__device__ inline typename Op<T>::frag load_plain(const T* base, int rs, int row0, int k0) {
  const int l = lane_id();
  return Op<T>::load8(base + (row0 + (l & 15)) * rs + k0 + 8 * (l >> 4));
}

// A operand, cb slot map over a 32-wide step starting at k0.
template <typename T>
__device__ inline typename Op<T>::frag load_cb(const T* base, int rs, int row0, int k0) {
  const int l = lane_id();
  const T* p = base + (row0 + (l & 15)) * rs + k0 + 4 * (l >> 4);
  return Op<T>::join(Op<T>::load4(p), Op<T>::load4(p + 16));
}

// A operand, cb slot map over a 16-wide step (slots 4..7 are zero).
template <typename T>
__device__ inline typename Op<T>::frag load_cb_half(const T* base, int rs, int row0, int k0) {
  const int l = lane_id();
  const T* p = base + (row0 + (l & 15)) * rs + k0 + 4 * (l >> 4);
  typename Op<T>::half4 z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = (T)0.0f;
  return Op<T>::join(Op<T>::load4(p), z);
}

template <typename T>
__device__ inline float to_f32(T x) {
  return (float)x;
}

}  // namespace gdr
