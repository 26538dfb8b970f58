// perm_kernels.h -- host/device interface of the partial-permutation kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {
namespace perm {

struct PermParams {
  int B, T, H, DK, DV;
  const void* q;   // bf16
  const void* k;
  const void* v;
  const int16_t* src;
  const float* beta;
  const float* w;
  const float* S0;
  void* o;         // bf16
  float* S_out;
};

hipError_t launch_perm_fwd(const PermParams& p, hipStream_t stream);

}  // namespace perm
}  // namespace gdr
