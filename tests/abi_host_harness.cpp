// abi_host_harness.cpp -- the host half of libgdr (argument checks and parameter
// marshalling in gdr_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.
// The kernel launchers are replaced by recorders, so nothing touches a GPU; the
// pointers are fake and never dereferenced.  Built and run by tests/test_abi.py.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gdr.h"
#include "gdr_kernels.h"
#include "gdr_raven.h"
#include "raven_kernels.h"
#include "gdr_perm.h"
#include "perm_kernels.h"

namespace gdr {
static FwdParams g_fwd;
static StepParams g_step;
static BwdParams g_bwd;
static int g_nfwd = 0, g_nstep = 0, g_nbwd = 0;
hipError_t launch_fwd(const FwdParams& p, hipStream_t) {
  g_fwd = p;
  ++g_nfwd;
  return hipSuccess;
}
hipError_t launch_step(const StepParams& p, hipStream_t) {
  g_step = p;
  ++g_nstep;
  return hipSuccess;
}
hipError_t launch_bwd(const BwdParams& p, hipStream_t) {
  g_bwd = p;
  ++g_nbwd;
  return hipSuccess;
}
static GateBwdParams g_gate;
static int g_ngprep = 0, g_ngchain = 0;
hipError_t launch_gate_prep(const GateBwdParams& p, hipStream_t) {
  g_gate = p;
  ++g_ngprep;
  return hipSuccess;
}
hipError_t launch_gate_chain(const GateBwdParams& p, hipStream_t) {
  g_gate = p;
  ++g_ngchain;
  return hipSuccess;
}
namespace raven {
static RavenParams g_rv;
static int g_nrv = 0;
hipError_t launch_raven_fwd(const RavenParams& p, hipStream_t) {
  g_rv = p;
  ++g_nrv;
  return hipSuccess;
}
}  // namespace raven
namespace perm {
static PermParams g_pm;
static int g_npm = 0;
hipError_t launch_perm_fwd(const PermParams& p, hipStream_t) {
  g_pm = p;
  ++g_npm;
  return hipSuccess;
}
}  // namespace perm
}  // namespace gdr

static int g_fail = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

// 16 MiB apart: no two fake buffers overlap for the sizes used here
static void* fake(unsigned k) { return (void*)((uintptr_t)0x1000000u * (k + 1)); }

static gdr_fwd_args good_fwd() {
  gdr_fwd_args a;
  std::memset(&a, 0, sizeof a);
  a.B = 2; a.T = 100; a.H = 4; a.dk = 128; a.dv = 128; a.chunk = 64;
  a.io_dtype = GDR_BF16; a.decay = GDR_DECAY_DIAG;
  a.q = fake(1); a.k = fake(2); a.v = fake(3); a.alpha = (const float*)fake(4);
  a.beta = (const float*)fake(5); a.w = (const float*)fake(6); a.o = fake(7);
  return a;
}

int main() {
  // valid call: reaches the launcher with every field marshalled
  gdr_fwd_args a = good_fwd();
  a.S0 = (const float*)fake(8); a.S_out = (float*)fake(9);
  CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_OK);
  CHECK(gdr::g_nfwd == 1);
  CHECK(gdr::g_fwd.B == 2 && gdr::g_fwd.T == 100 && gdr::g_fwd.H == 4);
  CHECK(gdr::g_fwd.DK == 128 && gdr::g_fwd.DV == 128 && gdr::g_fwd.io_bf16 == 1);
  CHECK(gdr::g_fwd.block == 64 && gdr::g_fwd.window == 64);
  CHECK(gdr::g_fwd.q == a.q && gdr::g_fwd.S0 == a.S0 && gdr::g_fwd.S_out == a.S_out);
  // fp32 at d = 128 runs 32-token blocks
  a.io_dtype = GDR_F32;
  CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_OK && gdr::g_fwd.block == 32);
  // content-aware call
  a = good_fwd();
  a.beta = nullptr; a.beta_logit = (const float*)fake(10); a.ub_down = (const float*)fake(11);
  a.ub_up = (const float*)fake(12); a.ub_rank = 16; a.chunk = 128; a.T = 256;
  a.m_carry = (float*)fake(13);
  CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_OK && gdr::g_fwd.window == 128 && gdr::g_fwd.ub_rank == 16);
  // reflection blocks: marshalled as decay kind 2; other io dtypes and the
  // content-aware erase are refused
  a = good_fwd(); a.decay = GDR_DECAY_DIHEDRAL; a.theta = (const float*)fake(16);
  CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_OK && gdr::g_fwd.decay == 2 && gdr::g_fwd.theta == a.theta);
  const int nrefl = gdr::g_nfwd;
  a.io_dtype = GDR_F32; CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_UNSUPPORTED);
  a.io_dtype = GDR_BF16; a.theta = nullptr; CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_NULL);
  CHECK(gdr::g_nfwd == nrefl);

  // rejected before any launch
  const int before = gdr::g_nfwd;
  CHECK(gdr_chunk_fwd(nullptr, nullptr) == GDR_ERR_NULL);
  a = good_fwd(); a.B = 0; CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_SHAPE);
  a = good_fwd(); a.T = -5; CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_SHAPE);
  a = good_fwd(); a.dk = a.dv = 96; CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_UNSUPPORTED);
  a = good_fwd(); a.chunk = 48; CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_UNSUPPORTED);
  a = good_fwd(); a.io_dtype = 9; CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_DTYPE);
  a = good_fwd(); a.q = (const void*)((const char*)a.q + 4); CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_ALIGN);
  a = good_fwd(); a.theta = (const float*)fake(20); CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_ARG);
  a = good_fwd(); a.S0 = (const float*)fake(30); a.S_out = (float*)((char*)fake(30) + 64);
  CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_ARG);
  a = good_fwd(); a.workspace_bytes = 64; CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_WORKSPACE);
  // extreme sizes: the element-count checks must not overflow
  a = good_fwd(); a.B = 0x7fffffff; a.T = 0x7fffffff; a.H = 0x7fffffff;
  CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_SHAPE);
  a = good_fwd(); a.T = 1 << 30; a.B = 4; CHECK(gdr_chunk_fwd(&a, nullptr) == GDR_ERR_SHAPE);
  CHECK(gdr::g_nfwd == before);

  // gated forward: marshalled with its gate mode, decay from decay_x
  gdr_gate_args g;
  std::memset(&g, 0, sizeof g);
  g.decay_x = fake(14); g.decay_a = (const float*)fake(15); g.qk_l2norm = 1;
  a = good_fwd(); a.alpha = nullptr;
  CHECK(gdr_chunk_fwd_gated(&a, &g, nullptr) == GDR_OK);
  CHECK(gdr::g_fwd.gmode == 2 && gdr::g_fwd.gate_x == g.decay_x && gdr::g_fwd.gate_a == g.decay_a);
  CHECK(gdr::g_fwd.alpha == nullptr && gdr::g_fwd.q == a.q);
  g.qk_l2norm = 0; a.decay = GDR_DECAY_ROT2; a.theta = (const float*)fake(16); a.dk = a.dv = 64;
  CHECK(gdr_chunk_fwd_gated(&a, &g, nullptr) == GDR_OK && gdr::g_fwd.gmode == 1 && gdr::g_fwd.decay == 1);
  const int before_g = gdr::g_nfwd;
  a = good_fwd(); a.alpha = nullptr;
  CHECK(gdr_chunk_fwd_gated(nullptr, &g, nullptr) == GDR_ERR_NULL);
  CHECK(gdr_chunk_fwd_gated(&a, nullptr, nullptr) == GDR_ERR_NULL);
  {
    gdr_gate_args h = g; h.reserved = 1; CHECK(gdr_chunk_fwd_gated(&a, &h, nullptr) == GDR_ERR_ARG);
    h = g; h.decay_x = nullptr; CHECK(gdr_chunk_fwd_gated(&a, &h, nullptr) == GDR_ERR_NULL);
    h = g; h.decay_a = nullptr; CHECK(gdr_chunk_fwd_gated(&a, &h, nullptr) == GDR_ERR_NULL);
    h = g; h.decay_x = (const char*)fake(14) + 2; CHECK(gdr_chunk_fwd_gated(&a, &h, nullptr) == GDR_ERR_ALIGN);
    h = g; h.decay_a = (const float*)((const char*)fake(15) + 2);
    CHECK(gdr_chunk_fwd_gated(&a, &h, nullptr) == GDR_ERR_ALIGN);
  }
  gdr_fwd_args b = a; b.alpha = (const float*)fake(4); CHECK(gdr_chunk_fwd_gated(&b, &g, nullptr) == GDR_ERR_ARG);
  b = a; b.io_dtype = GDR_F32; CHECK(gdr_chunk_fwd_gated(&b, &g, nullptr) == GDR_ERR_UNSUPPORTED);
  b = a; b.dk = b.dv = 32; CHECK(gdr_chunk_fwd_gated(&b, &g, nullptr) == GDR_ERR_UNSUPPORTED);
  b = a; b.beta = nullptr; b.beta_logit = (const float*)fake(10); b.ub_down = (const float*)fake(11);
  b.ub_up = (const float*)fake(12); b.ub_rank = 16;
  CHECK(gdr_chunk_fwd_gated(&b, &g, nullptr) == GDR_ERR_UNSUPPORTED);
  b = a; b.T = 1 << 22; b.H = 1; CHECK(gdr_chunk_fwd_gated(&b, &g, nullptr) == GDR_ERR_UNSUPPORTED);
  b = a; b.beta = nullptr; CHECK(gdr_chunk_fwd_gated(&b, &g, nullptr) == GDR_ERR_NULL);
  CHECK(gdr::g_nfwd == before_g);

  // backward: forward recompute with checkpoints in the workspace, then the
  // backward kernels on the same workspace
  gdr_bwd_args w;
  std::memset(&w, 0, sizeof w);
  w.B = 2; w.T = 100; w.H = 4; w.dk = 128; w.dv = 128; w.decay = GDR_DECAY_DIAG;
  w.q = fake(1); w.k = fake(2); w.v = fake(3); w.alpha = (const float*)fake(4);
  w.beta = (const float*)fake(5); w.w = (const float*)fake(6); w.grad_o = fake(7);
  w.grad_q = (float*)fake(8); w.grad_k = (float*)fake(9); w.grad_v = (float*)fake(10);
  w.grad_alpha = (float*)fake(11); w.grad_beta = (float*)fake(12); w.grad_w = (float*)fake(13);
  const size_t need = gdr_chunk_bwd_workspace(&w);
  // 4 blocks of 32: checkpoints 2*4*4*128*128*4, o 800*128*2, partials 4*800*386*4,
  // range flags 2*4*4 ints (one 256-byte region)
  CHECK(need == (size_t)2 * 4 * 4 * 128 * 128 * 4 + 800 * 128 * 2 + (size_t)4 * 800 * 386 * 4 + 256);
  CHECK(gdr_chunk_bwd(&w, nullptr) == GDR_ERR_WORKSPACE);
  w.workspace = fake(20); w.workspace_bytes = need - 1;
  CHECK(gdr_chunk_bwd(&w, nullptr) == GDR_ERR_WORKSPACE);
  w.workspace_bytes = need;
  const int f_before = gdr::g_nfwd;
  CHECK(gdr_chunk_bwd(&w, nullptr) == GDR_OK);
  CHECK(gdr::g_nfwd == f_before + 1 && gdr::g_nbwd == 1);
  CHECK(gdr::g_fwd.ckpt == (float*)w.workspace && gdr::g_fwd.S_out == nullptr && gdr::g_fwd.o != nullptr);
  CHECK(gdr::g_bwd.ckpt == gdr::g_fwd.ckpt && gdr::g_bwd.grad_q == w.grad_q && gdr::g_bwd.grad_S0 == nullptr);
  CHECK((char*)gdr::g_bwd.part >= (char*)gdr::g_fwd.o + 800 * 128 * 2);
  CHECK((char*)gdr::g_bwd.part + (size_t)4 * 800 * 386 * 4 <= (char*)w.workspace + need);
  CHECK((char*)gdr::g_bwd.flag >= (char*)gdr::g_bwd.part + (size_t)4 * 800 * 386 * 4);
  CHECK((char*)(gdr::g_bwd.flag + 2 * 4 * 4) <= (char*)w.workspace + need);
  {
    gdr_bwd_args x = w; x.dk = x.dv = 32; CHECK(gdr_chunk_bwd(&x, nullptr) == GDR_ERR_UNSUPPORTED);
    CHECK(gdr_chunk_bwd_workspace(&x) == 0);
    x = w; x.grad_beta = nullptr; CHECK(gdr_chunk_bwd(&x, nullptr) == GDR_ERR_NULL);
    x = w; x.theta = (const float*)fake(21); CHECK(gdr_chunk_bwd(&x, nullptr) == GDR_ERR_ARG);
    x = w; x.decay = GDR_DECAY_ROT2; CHECK(gdr_chunk_bwd(&x, nullptr) == GDR_ERR_NULL);
    x = w; x.decay = GDR_DECAY_ROT2; x.theta = (const float*)fake(21); x.grad_theta = (float*)fake(22);
    CHECK(gdr_chunk_bwd(&x, nullptr) == GDR_OK && gdr::g_bwd.decay == 1);
    x.decay = GDR_DECAY_DIHEDRAL; CHECK(gdr_chunk_bwd(&x, nullptr) == GDR_ERR_UNSUPPORTED);
    x = w; x.grad_q = (float*)((char*)fake(8) + 4); CHECK(gdr_chunk_bwd(&x, nullptr) == GDR_ERR_ALIGN);
    x = w; x.T = 0; CHECK(gdr_chunk_bwd(&x, nullptr) == GDR_ERR_SHAPE);
    x = w; x.B = 0x7fffffff; x.T = 0x7fffffff; CHECK(gdr_chunk_bwd(&x, nullptr) == GDR_ERR_SHAPE);
    CHECK(gdr_chunk_bwd(nullptr, nullptr) == GDR_ERR_NULL && gdr_chunk_bwd_workspace(nullptr) == 0);
  }

  // gated backward: activation and normalisation around the plain backward
  {
    gdr_bwd_args gb = w;
    gb.alpha = nullptr;
    gb.grad_alpha = nullptr;
    gb.workspace = nullptr;
    gb.workspace_bytes = 0;
    gdr_gate_args ga;
    std::memset(&ga, 0, sizeof ga);
    ga.decay_x = fake(30); ga.decay_a = (const float*)fake(31); ga.qk_l2norm = 1;
    gdr_gate_grads gg;
    gg.grad_decay_x = (float*)fake(32); gg.grad_decay_a = (float*)fake(33);
    const size_t gneed = gdr_chunk_bwd_gated_workspace(&gb, &ga);
    // decay and its gradient 800*128*4 each, q/k normalised 800*128*2 each and
    // their gradients 800*128*4 each, 800 row sums, then the plain backward's
    const size_t gown = 2 * (size_t)800 * 128 * 4 + 2 * 800 * 128 * 2 + 2 * (size_t)800 * 128 * 4 + 3328;
    CHECK(gneed == gown + need);
    CHECK(gdr_chunk_bwd_gated(&gb, &ga, &gg, nullptr) == GDR_ERR_WORKSPACE);
    gb.workspace = fake(20); gb.workspace_bytes = gneed - 1;
    CHECK(gdr_chunk_bwd_gated(&gb, &ga, &gg, nullptr) == GDR_ERR_WORKSPACE);
    gb.workspace_bytes = gneed;
    const int nb = gdr::g_nbwd;
    CHECK(gdr_chunk_bwd_gated(&gb, &ga, &gg, nullptr) == GDR_OK);
    CHECK(gdr::g_ngprep == 1 && gdr::g_ngchain == 1 && gdr::g_nbwd == nb + 1);
    CHECK(gdr::g_gate.norm == 1 && gdr::g_gate.C == 128 && gdr::g_gate.grad_q == w.grad_q);
    CHECK(gdr::g_bwd.grad_q != w.grad_q && gdr::g_bwd.q == gdr::g_gate.q_n);
    CHECK((const float*)gdr::g_bwd.grad_alpha == gdr::g_gate.grad_alpha && gdr::g_gate.alpha != nullptr);
    CHECK((char*)gdr::g_gate.ga_rows + 800 * 4 <= (char*)gdr::g_bwd.ckpt);
    CHECK((char*)gdr::g_bwd.flag + 2 * 4 * 4 * 4 <= (char*)gb.workspace + gneed);
    gdr_bwd_args x = gb;
    x.alpha = (const float*)fake(4); CHECK(gdr_chunk_bwd_gated(&x, &ga, &gg, nullptr) == GDR_ERR_ARG);
    x = gb; x.grad_alpha = (float*)fake(11); CHECK(gdr_chunk_bwd_gated(&x, &ga, &gg, nullptr) == GDR_ERR_ARG);
    CHECK(gdr_chunk_bwd_gated(&gb, &ga, nullptr, nullptr) == GDR_ERR_NULL);
    CHECK(gdr_chunk_bwd_gated(&gb, nullptr, &gg, nullptr) == GDR_ERR_NULL);
    gdr_gate_args gx = ga; gx.reserved = 1; CHECK(gdr_chunk_bwd_gated(&gb, &gx, &gg, nullptr) == GDR_ERR_ARG);
    gx = ga; gx.decay_a = (const float*)((char*)fake(31) + 2);
    CHECK(gdr_chunk_bwd_gated(&gb, &gx, &gg, nullptr) == GDR_ERR_ALIGN);
    gx = ga; gx.decay_x = (const char*)fake(30) + 2;
    CHECK(gdr_chunk_bwd_gated(&gb, &gx, &gg, nullptr) == GDR_ERR_ALIGN);
    gx = ga; gx.qk_l2norm = 0;
    CHECK(gdr_chunk_bwd_gated_workspace(&gb, &gx) == 2 * (size_t)800 * 128 * 4 + 3328 + need);
    gb.workspace_bytes = gdr_chunk_bwd_gated_workspace(&gb, &gx);
    CHECK(gdr_chunk_bwd_gated(&gb, &gx, &gg, nullptr) == GDR_OK && gdr::g_bwd.grad_q == w.grad_q);
    CHECK(gdr_chunk_bwd_gated_workspace(nullptr, &ga) == 0);
  }

  // decode
  gdr_step_args s;
  std::memset(&s, 0, sizeof s);
  s.N = 256; s.H = 16; s.dk = 128; s.dv = 128; s.io_dtype = GDR_BF16; s.decay = GDR_DECAY_ROT2;
  s.q = fake(1); s.k = fake(2); s.v = fake(3); s.alpha = (const float*)fake(4);
  s.theta = (const float*)fake(5); s.beta = (const float*)fake(6); s.w = (const float*)fake(7);
  s.S = (float*)fake(8); s.o = fake(9);
  CHECK(gdr_step_decode(&s, nullptr) == GDR_OK && gdr::g_nstep == 1 && gdr::g_step.decay == 1);
  s.decay = GDR_DECAY_DIHEDRAL;
  CHECK(gdr_step_decode(&s, nullptr) == GDR_OK && gdr::g_nstep == 2 && gdr::g_step.decay == 2);
  s.decay = GDR_DECAY_ROT2;
  s.N = 0x7fffffff; s.H = 0x7fffffff; CHECK(gdr_step_decode(&s, nullptr) == GDR_ERR_SHAPE);
  CHECK(gdr_step_decode(nullptr, nullptr) == GDR_ERR_NULL);

  // Raven slot memory: marshalled, and rejected before any launch
  {
    gdr_raven_args r;
    std::memset(&r, 0, sizeof r);
    r.B = 2; r.T = 77; r.H = 3; r.dk = r.dv = 128; r.slots = 64; r.topk = 8; r.scale = 0.125f;
    r.q = fake(1); r.k = fake(2); r.v = fake(3); r.z = fake(4); r.a = (const float*)fake(5);
    r.o = fake(6); r.Sk0 = (const float*)fake(7); r.Sv0 = (const float*)fake(8);
    r.Sk_out = (float*)fake(7); r.Sv_out = (float*)fake(8);   // in place
    CHECK(gdr_raven_fwd(&r, nullptr) == GDR_OK && gdr::raven::g_nrv == 1);
    const gdr::raven::RavenParams& p = gdr::raven::g_rv;
    CHECK(p.B == 2 && p.T == 77 && p.H == 3 && p.D == 128 && p.topk == 8 && p.scale == 0.125f);
    CHECK((const void*)p.q == r.q && (const void*)p.z == r.z && p.a == r.a && (void*)p.o == r.o);
    CHECK(p.Sk0 == r.Sk0 && p.Sv_out == r.Sv_out);
    gdr_raven_args x = r; x.topk = 9; CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_UNSUPPORTED);
    x = r; x.topk = 0; CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_SHAPE);
    x = r; x.slots = 32; CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_UNSUPPORTED);
    x = r; x.dv = 64; CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_UNSUPPORTED);
    x = r; x.z = nullptr; CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_NULL);
    x = r; x.a = (const float*)((const char*)fake(5) + 4); CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_ALIGN);
    x = r; x.Sk_out = (float*)((char*)fake(7) + 256); CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_ARG);
    x = r; x.Sv_out = (float*)fake(7); x.Sk_out = nullptr; CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_ARG);
    x = r; x.B = 0x7fffffff; x.T = 0x7fffffff; x.H = 0x7fffffff;
    CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_SHAPE);
    x = r; x.scale = 1.f / 0.f; CHECK(gdr_raven_fwd(&x, nullptr) == GDR_ERR_UNSUPPORTED);
    CHECK(gdr_raven_fwd(nullptr, nullptr) == GDR_ERR_NULL);
    CHECK(gdr::raven::g_nrv == 1);
  }

  // partial permutations: marshalled, and rejected before any launch
  {
    gdr_perm_args a;
    std::memset(&a, 0, sizeof a);
    a.B = 2; a.T = 50; a.H = 3; a.dk = 128; a.dv = 64;
    a.q = fake(1); a.k = fake(2); a.v = fake(3); a.src = (const int16_t*)fake(4);
    a.beta = (const float*)fake(5); a.w = (const float*)fake(6); a.o = fake(7);
    a.S0 = (const float*)fake(8); a.S_out = (float*)fake(8);
    CHECK(gdr_perm_fwd(&a, nullptr) == GDR_OK && gdr::perm::g_npm == 1);
    const gdr::perm::PermParams& p = gdr::perm::g_pm;
    CHECK(p.B == 2 && p.T == 50 && p.H == 3 && p.DK == 128 && p.DV == 64);
    CHECK(p.src == a.src && p.beta == a.beta && p.w == a.w && p.o == a.o && p.S_out == a.S_out);
    gdr_perm_args x = a; x.dv = 40; CHECK(gdr_perm_fwd(&x, nullptr) == GDR_ERR_UNSUPPORTED);
    x = a; x.src = nullptr; CHECK(gdr_perm_fwd(&x, nullptr) == GDR_ERR_NULL);
    x = a; x.S_out = (float*)((char*)fake(8) + 16); CHECK(gdr_perm_fwd(&x, nullptr) == GDR_ERR_ARG);
    x = a; x.B = 0x7fffffff; x.T = 0x7fffffff; CHECK(gdr_perm_fwd(&x, nullptr) == GDR_ERR_SHAPE);
    CHECK(gdr_perm_fwd(nullptr, nullptr) == GDR_ERR_NULL && gdr::perm::g_npm == 1);
  }

  for (int st = -1; st < 12; ++st) CHECK(gdr_status_str((gdr_status)st) != nullptr);
  CHECK(gdr_abi_version() == GDR_ABI_VERSION);
  CHECK(gdr_chunk_fwd_workspace(nullptr) == 0);
  if (g_fail) return 1;
  std::printf("ABI_HARNESS_OK\n");
  return 0;
}
