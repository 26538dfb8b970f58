// raven_kernels.h -- host/device interface of the Raven slot-memory kernel.
#pragma once
#include <hip/hip_runtime.h>

namespace gdr {
namespace raven {

struct RavenParams {
  int B, T, H, D, topk;   // D = d_k = d_v; the slot count is fixed at 64
  float scale;
  const void* q;    // bf16
  const void* k;
  const void* v;
  const void* z;
  const float* a;
  const float* Sk0;
  const float* Sv0;
  void* o;          // bf16
  float* Sk_out;
  float* Sv_out;
};

constexpr int kSlots = 64;
constexpr int kMaxTopK = 8;

hipError_t launch_raven_fwd(const RavenParams& p, hipStream_t stream);

}  // namespace raven
}  // namespace gdr
