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

bool block_decay(int d) { return d == GDR_DECAY_ROT2 || d == GDR_DECAY_DIHEDRAL; }

gdr_status check_fwd(const gdr_fwd_args* a) {
  if (!a) return GDR_ERR_NULL;
  if (a->io_dtype != GDR_F32 && a->io_dtype != GDR_BF16) return GDR_ERR_DTYPE;
  if (a->decay != GDR_DECAY_DIAG && !block_decay(a->decay)) return GDR_ERR_DTYPE;
  if (a->B <= 0 || a->T <= 0 || a->H <= 0 || a->dk <= 0 || a->dv <= 0 || a->chunk <= 0)
    return GDR_ERR_SHAPE;
  if (!supported_d(a->dk) || a->dv != a->dk) return GDR_ERR_UNSUPPORTED;
  if (!supported_chunk(a->chunk)) return GDR_ERR_UNSUPPORTED;
  // element counts must stay within 32-bit row indexing of the kernels; each
  // product is bounded before the next one is formed, so none can overflow
  const long long bt = (long long)a->B * a->T;   // < 2^62
  if (bt >= (1LL << 31)) return GDR_ERR_SHAPE;
  const long long rows = bt * a->H;              // < 2^62
  if (rows >= (1LL << 40) / a->dk) return GDR_ERR_SHAPE;
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
  if (block_decay(a->decay)) {
    if (!a->theta) return GDR_ERR_NULL;
  } else if (a->theta) {
    return GDR_ERR_ARG;
  }
  // reflection blocks: the pipelined kernel's plain launch only
  if (a->decay == GDR_DECAY_DIHEDRAL &&
      (a->io_dtype != GDR_BF16 || (a->dk != 64 && a->dk != 128) || content ||
       (long long)a->T * a->H >= (1LL << 29) / a->dk))
    return GDR_ERR_UNSUPPORTED;
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
  if (a->decay != GDR_DECAY_DIAG && !block_decay(a->decay)) return GDR_ERR_DTYPE;
  if (a->N <= 0 || a->H <= 0 || a->dk <= 0 || a->dv <= 0) return GDR_ERR_SHAPE;
  if ((long long)a->N * a->H >= (1LL << 31)) return GDR_ERR_SHAPE;
  if (!supported_d(a->dk) || a->dv != a->dk) return GDR_ERR_UNSUPPORTED;
  if (!a->q || !a->k || !a->v || !a->alpha || !a->beta || !a->w || !a->S || !a->o)
    return GDR_ERR_NULL;
  if (block_decay(a->decay)) {
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

namespace gdr {
// WY block length of the sequential-stage kernel: the chunk, at most 64, and
// at most 32 for fp32 operands at d_k = 128 (LDS of one CU).
int fwd_block_len(int dk, int chunk, bool io_bf16) {
  const int lmax = (!io_bf16 && dk == 128) ? 32 : 64;
  return chunk < lmax ? chunk : lmax;
}

// Whether the pipelined kernel takes the call (bf16, d_k = d_v in {64, 128}).
bool fwd_pipe_supported(const FwdParams& p) {
  // buffer resources address one (b, h) with 32-bit byte offsets
  const bool fits = (unsigned long long)p.T * p.H * p.DK * 4ull < (1ull << 31);
  // content-aware: the window must be a whole number of 32-token blocks
  const bool content_ok = p.beta_logit == nullptr || (p.window >= 32 && p.window % 32 == 0);
  return p.io_bf16 && content_ok && (p.DK == 64 || p.DK == 128) && p.DV == p.DK && fits;
}
}  // namespace gdr

namespace {
gdr::FwdParams fwd_params(const gdr_fwd_args* a) {
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
  return p;
}

// The gated forward's own conditions, on top of check_fwd's (which sees
// decay_x in place of alpha).
gdr_status check_gated(const gdr_fwd_args* a, const gdr_gate_args* g) {
  if (!a || !g) return GDR_ERR_NULL;
  if (g->reserved != 0) return GDR_ERR_ARG;
  if (a->alpha) return GDR_ERR_ARG;
  if (!g->decay_x || !g->decay_a) return GDR_ERR_NULL;
  gdr_fwd_args c = *a;
  c.alpha = static_cast<const float*>(g->decay_x);   // checked for presence and alignment only
  const gdr_status st = check_fwd(&c);
  if (st != GDR_OK) return st;
  if (a->io_dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
  if (a->dk != 64 && a->dk != 128) return GDR_ERR_UNSUPPORTED;
  if (a->beta_logit) return GDR_ERR_UNSUPPORTED;
  if (a->decay == GDR_DECAY_DIHEDRAL) return GDR_ERR_UNSUPPORTED;
  // 32-bit byte offsets of the kernel's buffer resources (T * H * dk < 2^29)
  if ((long long)a->T * a->H >= (1LL << 29) / a->dk) return GDR_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(g->decay_a) & 3u) != 0) return GDR_ERR_ALIGN;
  return GDR_OK;
}
// Backward: the workspace holds the block-start states of the forward
// recompute, its output o (not returned), the per-value-tile partial sums and
// one range flag per (b, h, value tile), each region 256-byte aligned.
struct BwdLayout {
  size_t ckpt, o, part, flag, total;
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdLayout bwd_layout(const gdr_bwd_args* a) {
  const size_t nc = (size_t)(a->T + gdr::kBwdBlock - 1) / gdr::kBwdBlock;
  const size_t bth = (size_t)a->B * a->T * a->H;
  BwdLayout w;
  w.ckpt = 0;
  w.o = round256((size_t)a->B * a->H * nc * a->dv * a->dk * sizeof(float));
  w.part = w.o + round256(bth * a->dv * 2);
  w.flag = w.part + round256(gdr::bwd_part_floats(a->B, a->T, a->H, a->dk, a->dv) * sizeof(float));
  w.total = w.flag + round256((size_t)a->B * a->H * (a->dv / gdr::kBwdTile) * sizeof(int));
  return w;
}

// Everything but the workspace size.
gdr_status check_bwd_args(const gdr_bwd_args* a) {
  if (!a) return GDR_ERR_NULL;
  if (a->decay != GDR_DECAY_DIAG && !block_decay(a->decay)) return GDR_ERR_DTYPE;
  if (a->B <= 0 || a->T <= 0 || a->H <= 0 || a->dk <= 0 || a->dv <= 0) return GDR_ERR_SHAPE;
  if ((a->dk != 64 && a->dk != 128) || a->dv != a->dk) return GDR_ERR_UNSUPPORTED;
  if (a->decay == GDR_DECAY_DIHEDRAL) return GDR_ERR_UNSUPPORTED;
  if ((long long)a->B * a->T >= (1LL << 31)) return GDR_ERR_SHAPE;
  // 32-bit byte offsets of the forward's buffer resources (T * H * dk < 2^29)
  if ((long long)a->T * a->H >= (1LL << 29) / a->dk) return GDR_ERR_UNSUPPORTED;
  if ((long long)a->B * a->T * a->H >= (1LL << 40) / a->dk) return GDR_ERR_SHAPE;
  const void* need[] = {a->q, a->k, a->v, a->alpha, a->beta, a->w, a->grad_o, a->grad_q,
                        a->grad_k, a->grad_v, a->grad_alpha, a->grad_beta, a->grad_w};
  for (const void* p : need)
    if (!p) return GDR_ERR_NULL;
  if (a->decay == GDR_DECAY_ROT2) {
    if (!a->theta || !a->grad_theta) return GDR_ERR_NULL;
  } else if (a->theta || a->grad_theta) {
    return GDR_ERR_ARG;
  }
  const void* vec[] = {a->q, a->k, a->v, a->alpha, a->theta, a->beta, a->w, a->S0, a->grad_o,
                       a->grad_S, a->grad_q, a->grad_k, a->grad_v, a->grad_alpha, a->grad_theta,
                       a->grad_beta, a->grad_w, a->grad_S0, a->workspace};
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
  const hipError_t e = gdr::launch_fwd(fwd_params(a), (hipStream_t)hip_stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

gdr_status gdr_chunk_fwd_gated(const gdr_fwd_args* a, const gdr_gate_args* g, void* hip_stream) {
  const gdr_status st = check_gated(a, g);
  if (st != GDR_OK) return st;
  gdr::FwdParams p = fwd_params(a);
  p.gmode = g->qk_l2norm ? 2 : 1;
  p.gate_x = g->decay_x;
  p.gate_a = g->decay_a;
  if (!gdr::fwd_pipe_supported(p)) return GDR_ERR_UNSUPPORTED;
  const hipError_t e = gdr::launch_fwd(p, (hipStream_t)hip_stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

size_t gdr_chunk_bwd_workspace(const gdr_bwd_args* a) {
  if (check_bwd_args(a) != GDR_OK) return 0;
  return bwd_layout(a).total;
}

gdr_status gdr_chunk_bwd(const gdr_bwd_args* a, void* hip_stream) {
  if (!a) return GDR_ERR_NULL;
  return gdr::chunk_bwd_on(a, a->workspace, a->workspace_bytes, (hipStream_t)hip_stream);
}

}  // extern "C"

namespace gdr {
gdr_status chunk_bwd_on(const gdr_bwd_args* a, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  const gdr_status st = check_bwd_args(a);
  if (st != GDR_OK) return st;
  const BwdLayout lay = bwd_layout(a);
  if (!workspace || workspace_bytes < lay.total) return GDR_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GDR_ERR_ALIGN;
  char* ws = (char*)workspace;
  // forward recompute with block-start checkpoints
  gdr::FwdParams f{};
  f.B = a->B;
  f.T = a->T;
  f.H = a->H;
  f.DK = a->dk;
  f.DV = a->dv;
  f.io_bf16 = 1;
  f.block = gdr::kBwdBlock;
  f.window = gdr::kBwdBlock;
  f.decay = a->decay;
  f.q = a->q;
  f.k = a->k;
  f.v = a->v;
  f.alpha = a->alpha;
  f.theta = a->theta;
  f.beta = a->beta;
  f.w = a->w;
  f.S0 = a->S0;
  f.o = ws + lay.o;
  f.S_out = nullptr;
  f.ckpt = (float*)(ws + lay.ckpt);
  if (!gdr::fwd_pipe_supported(f)) return GDR_ERR_UNSUPPORTED;
  hipError_t e = gdr::launch_fwd(f, stream);
  if (e != hipSuccess) return GDR_ERR_HIP;
  gdr::BwdParams p{};
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.DK = a->dk;
  p.DV = a->dv;
  p.decay = a->decay;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.alpha = a->alpha;
  p.theta = a->theta;
  p.beta = a->beta;
  p.w = a->w;
  p.grad_o = a->grad_o;
  p.grad_S = a->grad_S;
  p.grad_q = a->grad_q;
  p.grad_k = a->grad_k;
  p.grad_v = a->grad_v;
  p.grad_alpha = a->grad_alpha;
  p.grad_theta = a->grad_theta;
  p.grad_beta = a->grad_beta;
  p.grad_w = a->grad_w;
  p.grad_S0 = a->grad_S0;
  p.ckpt = (const float*)(ws + lay.ckpt);
  p.part = (float*)(ws + lay.part);
  p.flag = (int*)(ws + lay.flag);
  e = gdr::launch_bwd(p, stream);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // namespace gdr

// ---------------------------------------------------------------- gated backward
namespace {

// Workspace of gdr_chunk_bwd_gated: the activated decay and its gradient, the
// normalised q, k and their gradients (qk_l2norm), one fp32 per token-head
// (its part of dL/da_h), then the plain backward's own workspace.
struct GateLayout {
  size_t alpha, galpha, qn, kn, gqn, gkn, ga, inner, inner_bytes, total;
};

alignas(16) const float kPlaceholder[4] = {0.f, 0.f, 0.f, 0.f};

// The plain backward's arguments for a gated call: the activated decay and its
// gradient in the workspace (placeholders until the workspace is known).
gdr_bwd_args inner_args(const gdr_bwd_args* a) {
  gdr_bwd_args t = *a;
  t.alpha = kPlaceholder;
  t.grad_alpha = const_cast<float*>(kPlaceholder);
  t.workspace = nullptr;
  t.workspace_bytes = 0;
  return t;
}

// Everything but the workspace; gg may be NULL for the size query.
gdr_status check_gated_bwd(const gdr_bwd_args* a, const gdr_gate_args* g, const gdr_gate_grads* gg,
                           bool need_grads) {
  if (!a || !g) return GDR_ERR_NULL;
  if (a->alpha || a->grad_alpha) return GDR_ERR_ARG;
  if (g->reserved != 0) return GDR_ERR_ARG;
  if (!g->decay_x || !g->decay_a) return GDR_ERR_NULL;
  if (need_grads && (!gg || !gg->grad_decay_x || !gg->grad_decay_a)) return GDR_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(g->decay_x) & 3u) != 0) return GDR_ERR_ALIGN;   // read in pairs
  if ((reinterpret_cast<uintptr_t>(g->decay_a) & 3u) != 0) return GDR_ERR_ALIGN;
  if (gg && ((reinterpret_cast<uintptr_t>(gg->grad_decay_x) & 3u) != 0 ||
             (reinterpret_cast<uintptr_t>(gg->grad_decay_a) & 3u) != 0))
    return GDR_ERR_ALIGN;
  const gdr_bwd_args t = inner_args(a);
  return check_bwd_args(&t);
}

GateLayout gate_layout(const gdr_bwd_args* a, bool norm) {
  const size_t rows = (size_t)a->B * a->T * a->H;
  const size_t C = a->decay == GDR_DECAY_ROT2 ? a->dk / 2 : a->dk;
  const gdr_bwd_args t = inner_args(a);
  GateLayout w{};
  size_t o = 0;
  w.alpha = o;
  o += round256(rows * C * sizeof(float));
  w.galpha = o;
  o += round256(rows * C * sizeof(float));
  if (norm) {
    w.qn = o;
    o += round256(rows * a->dk * 2);
    w.kn = o;
    o += round256(rows * a->dk * 2);
    w.gqn = o;
    o += round256(rows * a->dk * sizeof(float));
    w.gkn = o;
    o += round256(rows * a->dk * sizeof(float));
  }
  w.ga = o;
  o += round256(rows * sizeof(float));
  w.inner = o;
  w.inner_bytes = bwd_layout(&t).total;
  w.total = o + w.inner_bytes;
  return w;
}

}  // namespace

extern "C" {

size_t gdr_chunk_bwd_gated_workspace(const gdr_bwd_args* a, const gdr_gate_args* g) {
  if (check_gated_bwd(a, g, nullptr, false) != GDR_OK) return 0;
  return gate_layout(a, g->qk_l2norm != 0).total;
}

gdr_status gdr_chunk_bwd_gated(const gdr_bwd_args* a, const gdr_gate_args* g,
                               const gdr_gate_grads* gg, void* hip_stream) {
  const gdr_status st = check_gated_bwd(a, g, gg, true);
  if (st != GDR_OK) return st;
  const bool norm = g->qk_l2norm != 0;
  const GateLayout lay = gate_layout(a, norm);
  if (!a->workspace || a->workspace_bytes < lay.total) return GDR_ERR_WORKSPACE;
  if (!aligned16(a->workspace)) return GDR_ERR_ALIGN;
  const hipStream_t stream = (hipStream_t)hip_stream;
  char* ws = (char*)a->workspace;
  gdr::GateBwdParams p{};
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.DK = a->dk;
  p.C = a->decay == GDR_DECAY_ROT2 ? a->dk / 2 : a->dk;
  p.norm = norm ? 1 : 0;
  p.x = g->decay_x;
  p.a = g->decay_a;
  p.q_raw = a->q;
  p.k_raw = a->k;
  p.alpha = (float*)(ws + lay.alpha);
  p.q_n = norm ? ws + lay.qn : nullptr;
  p.k_n = norm ? ws + lay.kn : nullptr;
  p.grad_alpha = (const float*)(ws + lay.galpha);
  p.grad_qn = norm ? (const float*)(ws + lay.gqn) : nullptr;
  p.grad_kn = norm ? (const float*)(ws + lay.gkn) : nullptr;
  p.grad_x = gg->grad_decay_x;
  p.grad_q = a->grad_q;
  p.grad_k = a->grad_k;
  p.ga_rows = (float*)(ws + lay.ga);
  p.grad_a = gg->grad_decay_a;
  if (gdr::launch_gate_prep(p, stream) != hipSuccess) return GDR_ERR_HIP;
  gdr_bwd_args t = *a;
  t.alpha = p.alpha;
  t.grad_alpha = (float*)(ws + lay.galpha);
  if (norm) {
    t.q = p.q_n;
    t.k = p.k_n;
    t.grad_q = (float*)(ws + lay.gqn);
    t.grad_k = (float*)(ws + lay.gkn);
  }
  const gdr_status sb = gdr::chunk_bwd_on(&t, ws + lay.inner, lay.inner_bytes, stream);
  if (sb != GDR_OK) return sb;
  return gdr::launch_gate_chain(p, stream) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // extern "C"

extern "C" {

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
