// perm_api.cpp -- C ABI of the partial-permutation forward: argument checks,
// then the launch.  Every check runs on the host before any HIP call.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gdr_perm.h"
#include "perm_kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

gdr_status check_perm(const gdr_perm_args* a) {
  if (!a) return GDR_ERR_NULL;
  if (a->B <= 0 || a->T <= 0 || a->H <= 0 || a->dk <= 0 || a->dv <= 0) return GDR_ERR_SHAPE;
  if ((a->dk != 64 && a->dk != 128) || a->dv % 32 != 0 || a->dv > 256) return GDR_ERR_UNSUPPORTED;
  const long long bt = (long long)a->B * a->T;
  if (bt >= (1LL << 31)) return GDR_ERR_SHAPE;
  const long long rows = bt * a->H;
  if (rows >= (1LL << 40) / 256) return GDR_ERR_SHAPE;
  if ((long long)a->B * a->H * (a->dv / 32) >= (1LL << 31) / 8) return GDR_ERR_SHAPE;
  if (!a->q || !a->k || !a->v || !a->src || !a->beta || !a->w || !a->o) return GDR_ERR_NULL;
  const void* ptrs[] = {a->q, a->k, a->v, a->src, a->beta, a->w, a->S0, a->o, a->S_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDR_ERR_ALIGN;
  if (a->S0 && a->S_out && a->S0 != a->S_out) {
    const char* x = (const char*)a->S0;
    const char* y = (const char*)a->S_out;
    const size_t bytes = (size_t)a->B * a->H * a->dv * a->dk * sizeof(float);
    if (x < y + bytes && y < x + bytes) return GDR_ERR_ARG;
  }
  return GDR_OK;
}

}  // namespace

namespace gdr {
namespace perm {
PermParams perm_params(const gdr_perm_args* a) {
  PermParams p{};
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.DK = a->dk;
  p.DV = a->dv;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.src = a->src;
  p.beta = a->beta;
  p.w = a->w;
  p.S0 = a->S0;
  p.o = a->o;
  p.S_out = a->S_out;
  return p;
}
}  // namespace perm
}  // namespace gdr

extern "C" gdr_status gdr_perm_fwd(const gdr_perm_args* a, void* stream) {
  const gdr_status st = check_perm(a);
  if (st != GDR_OK) return st;
  const hipError_t e =
      gdr::perm::launch_perm_fwd(gdr::perm::perm_params(a), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}
