// gdr_api.cpp -- C ABI of libgdr: argument checks, then kernel dispatch.
//
// Every check runs on the host before any HIP call, so invalid calls are
// rejected (and testable) on a machine without a GPU.
#include <hip/hip_runtime.h>

#include "../../include/gdr.h"
#include "gdr_kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int d) { return d == 32 || d == 64 || d == 128; }

bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64 || c == 128; }

gdr_status check_fwd(const gdr_fwd_args* a) {
  if (!a) return GDR_ERR_NULL;
  if (a->io_dtype != GDR_F32 && a->io_dtype != GDR_BF16) return GDR_ERR_DTYPE;
  if (a->decay != GDR_DECAY_DIAG && a->decay != GDR_DECAY_ROT2) return GDR_ERR_DTYPE;
  if (a->B <= 0 || a->T <= 0 || a->H <= 0 || a->dk <= 0 || a->dv <= 0 || a->chunk <= 0)
    return GDR_ERR_SHAPE;
  if (!supported_d(a->dk) || a->dv != a->dk) return GDR_ERR_UNSUPPORTED;
  if (!supported_chunk(a->chunk)) return GDR_ERR_UNSUPPORTED;
  // element counts must stay within 32-bit row indexing of the kernels
  const long long rows = (long long)a->B * a->T * a->H;
  if (rows * a->dk >= (1LL << 40) || (long long)a->B * a->T >= (1LL << 31)) return GDR_ERR_SHAPE;
  if (!a->q || !a->k || !a->v || !a->alpha || !a->w || !a->o) return GDR_ERR_NULL;
  const bool content = a->beta_logit != nullptr;
  if (content) {
    if (a->beta) return GDR_ERR_ARG;
    if (!a->ub_down || !a->ub_up) return GDR_ERR_NULL;
    if (a->ub_rank < 1 || a->ub_rank > 64) return GDR_ERR_UNSUPPORTED;
    if (a->m_carry && (a->T % a->chunk) != 0) return GDR_ERR_SHAPE;
  } else {
    if (!a->beta) return GDR_ERR_NULL;
    if (a->ub_down || a->ub_up || a->m_carry) return GDR_ERR_ARG;
  }
  if (a->decay == GDR_DECAY_ROT2) {
    if (!a->theta) return GDR_ERR_NULL;
  } else if (a->theta) {
    return GDR_ERR_ARG;
  }
  const void* vec[] = {a->q, a->k, a->v, a->alpha, a->theta, a->o, a->S0, a->S_out};
  for (const void* p : vec)
    if (p && !aligned16(p)) return GDR_ERR_ALIGN;
  if (a->S0 && a->S_out && a->S0 != a->S_out) {
    // reject partial overlap of S0 and S_out
    const char* s0 = (const char*)a->S0;
    const char* s1 = (const char*)a->S_out;
    const size_t bytes = (size_t)a->B * a->H * a->dv * a->dk * sizeof(float);
    if (s0 < s1 + bytes && s1 < s0 + bytes) return GDR_ERR_ARG;
  }
  if (a->workspace_bytes && !a->workspace) return GDR_ERR_WORKSPACE;
  return GDR_OK;
}

gdr_status check_step(const gdr_step_args* a) {
  if (!a) return GDR_ERR_NULL;
  if (a->io_dtype != GDR_F32 && a->io_dtype != GDR_BF16) return GDR_ERR_DTYPE;
  if (a->decay != GDR_DECAY_DIAG && a->decay != GDR_DECAY_ROT2) return GDR_ERR_DTYPE;
  if (a->N <= 0 || a->H <= 0 || a->dk <= 0 || a->dv <= 0) return GDR_ERR_SHAPE;
  if ((long long)a->N * a->H >= (1LL << 31)) return GDR_ERR_SHAPE;
  if (!supported_d(a->dk) || a->dv != a->dk) return GDR_ERR_UNSUPPORTED;
  if (!a->q || !a->k || !a->v || !a->alpha || !a->beta || !a->w || !a->S || !a->o)
    return GDR_ERR_NULL;
  if (a->decay == GDR_DECAY_ROT2) {
    if (!a->theta) return GDR_ERR_NULL;
  } else if (a->theta) {
    return GDR_ERR_ARG;
  }
  const void* vec[] = {a->q, a->k, a->v, a->alpha, a->theta, a->S};
  for (const void* p : vec)
    if (p && !aligned16(p)) return GDR_ERR_ALIGN;
  return GDR_OK;
}

}  // namespace

extern "C" {

size_t gdr_chunk_fwd_workspace(const gdr_fwd_args* a) {
  (void)a;
  return 0;
}

gdr_status gdr_chunk_fwd(const gdr_fwd_args* a, void* hip_stream) {
  const gdr_status st = check_fwd(a);
  if (st != GDR_OK) return st;
  gdr::FwdParams p{};
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.DK = a->dk;
  p.DV = a->dv;
  p.io_bf16 = a->io_dtype == GDR_BF16;
  p.block = gdr::fwd_block_len(a->dk, a->chunk, p.io_bf16);
  p.window = a->chunk;
  p.decay = a->decay;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.alpha = a->alpha;
  p.theta = a->theta;
  p.beta = a->beta;
  p.w = a->w;
  p.beta_logit = a->beta_logit;
  p.ub_down = a->ub_down;
  p.ub_up = a->ub_up;
  p.ub_rank = a->ub_rank;
  p.m_carry = a->m_carry;
  p.S0 = a->S0;
  p.o = a->o;
  p.S_out = a->S_out;
  const hipError_t e = gdr::launch_fwd(p, (hipStream_t)hip_stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

gdr_status gdr_step_decode(const gdr_step_args* a, void* hip_stream) {
  const gdr_status st = check_step(a);
  if (st != GDR_OK) return st;
  gdr::StepParams p{};
  p.N = a->N;
  p.H = a->H;
  p.DK = a->dk;
  p.DV = a->dv;
  p.io_bf16 = a->io_dtype == GDR_BF16;
  p.decay = a->decay;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.alpha = a->alpha;
  p.theta = a->theta;
  p.beta = a->beta;
  p.w = a->w;
  p.S = a->S;
  p.o = a->o;
  const hipError_t e = gdr::launch_step(p, (hipStream_t)hip_stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

const char* gdr_status_str(gdr_status s) {
  switch (s) {
    case GDR_OK: return "ok";
    case GDR_ERR_NULL: return "a required pointer is NULL";
    case GDR_ERR_SHAPE: return "a size is non-positive or inconsistent";
    case GDR_ERR_DTYPE: return "unknown io dtype or decay kind";
    case GDR_ERR_UNSUPPORTED: return "unsupported size (d_k, d_v, chunk or rank)";
    case GDR_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case GDR_ERR_WORKSPACE: return "workspace missing or too small";
    case GDR_ERR_HIP: return "the HIP runtime rejected a launch";
    case GDR_ERR_ARG: return "an argument is set that must be NULL, or buffers overlap";
  }
  return "unknown status";
}

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

}  // extern "C"
