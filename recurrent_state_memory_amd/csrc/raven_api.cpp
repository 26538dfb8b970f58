// raven_api.cpp -- C ABI of the Raven slot-memory forward: argument checks,
// then the launch.  Every check runs on the host before any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/gdr_raven.h"
#include "raven_kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, const void* b, size_t bytes) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + bytes && y < x + bytes;
}

gdr_status check_raven(const gdr_raven_args* a) {
  if (!a) return GDR_ERR_NULL;
  if (a->B <= 0 || a->T <= 0 || a->H <= 0 || a->dk <= 0 || a->dv <= 0 || a->slots <= 0 ||
      a->topk <= 0)
    return GDR_ERR_SHAPE;
  if (a->dk != a->dv || (a->dk != 64 && a->dk != 128)) return GDR_ERR_UNSUPPORTED;
  if (a->slots != gdr::raven::kSlots || a->topk > gdr::raven::kMaxTopK) return GDR_ERR_UNSUPPORTED;
  if (!std::isfinite(a->scale)) return GDR_ERR_UNSUPPORTED;
  // element counts: each product bounded before the next is formed
  const long long bt = (long long)a->B * a->T;
  if (bt >= (1LL << 31)) return GDR_ERR_SHAPE;
  const long long rows = bt * a->H;
  if (rows >= (1LL << 40) / a->dk) return GDR_ERR_SHAPE;
  if (!a->q || !a->k || !a->v || !a->z || !a->a || !a->o) return GDR_ERR_NULL;
  const void* ptrs[] = {a->q, a->k, a->v, a->z, a->a, a->Sk0, a->Sv0, a->o, a->Sk_out, a->Sv_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDR_ERR_ALIGN;
  const size_t sbytes = (size_t)a->B * a->H * a->slots * a->dk * sizeof(float);
  if (a->Sk0 && a->Sk_out && a->Sk0 != a->Sk_out && overlap(a->Sk0, a->Sk_out, sbytes))
    return GDR_ERR_ARG;
  if (a->Sv0 && a->Sv_out && a->Sv0 != a->Sv_out && overlap(a->Sv0, a->Sv_out, sbytes))
    return GDR_ERR_ARG;
  if (a->Sk_out && a->Sv_out && overlap(a->Sk_out, a->Sv_out, sbytes)) return GDR_ERR_ARG;
  if (a->Sk_out && a->Sv0 && overlap(a->Sk_out, a->Sv0, sbytes)) return GDR_ERR_ARG;
  if (a->Sv_out && a->Sk0 && overlap(a->Sv_out, a->Sk0, sbytes)) return GDR_ERR_ARG;
  return GDR_OK;
}

}  // namespace

namespace gdr {
namespace raven {
// Host-side marshalling, separate from the launch so that a host-only build can
// check it.
RavenParams raven_params(const gdr_raven_args* a) {
  RavenParams p{};
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.D = a->dk;
  p.topk = a->topk;
  p.scale = a->scale;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.z = a->z;
  p.a = a->a;
  p.Sk0 = a->Sk0;
  p.Sv0 = a->Sv0;
  p.o = a->o;
  p.Sk_out = a->Sk_out;
  p.Sv_out = a->Sv_out;
  return p;
}
}  // namespace raven
}  // namespace gdr

extern "C" gdr_status gdr_raven_fwd(const gdr_raven_args* a, void* stream) {
  const gdr_status st = check_raven(a);
  if (st != GDR_OK) return st;
  const hipError_t e =
      gdr::raven::launch_raven_fwd(gdr::raven::raven_params(a), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}
