// gdr_fwd_pipe.hip -- pipelined chunk-WY gated delta-rule forward (bf16 q/k/v/o) for gfx950.
//
// Same computation as gdr_fwd.hip (chunk-WY algebra of the CARVE technical
// summary, section 1.3, and the SFDA constructive chunk-WY theorem / exact
// affine chunk transfer), as a three-stage pipeline inside one workgroup with
// a single workgroup barrier per 32-token step:
//
//   prep waves (4), chunk i+2: load the chunk (issued two chunks ahead; one in
//     the 16-wave content-aware variant),
//     running products of the key-axis transitions (forward and backward,
//     scanned across token segments inside each wave), decayed forms
//     K+ = g_r k, Q+ = g_r q and Kh = Gamma_L^{-T} K- with K- = h_r^T k.
//   solve waves (4), chunk i+1: Gram tiles A = strict_lower(diag(beta) K+ Kh^T)
//     and M = lower_incl(Q+ Kh^T), and the two 16x16 diagonal blocks T00, T11
//     of (I + A)^{-1} as the nilpotent product (I - N)(I + N^2)(I + N^4)(I + N^8)
//     on the matrix cores.
//   consumer waves (one per 16 value channels), chunk i:
//     R  = diag(beta w) V - diag(beta) K+ S^T
//     Dl = (I + A)^{-1} R by blocks: Dl0 = T00 R0, Dl1 = T11 (R1 - A10 Dl0)
//     O  = Q+ S^T + M Dl,   S <- S Gamma_L + Dl^T K- = (S + Dl^T Kh) Gamma_L.
//
// g_r = prod_{s<=r} D_s and h_r = prod_{s>r} D_s inside the chunk, so only one
// reciprocal per key channel (of Gamma_L) is needed; for 2x2 rotation-decay
// blocks the same holds with complex products per channel pair.  Prep outputs
// are triple-buffered and solve outputs double-buffered in LDS.
//
// Content-aware erase (CONTENT): one workgroup covers all value channels of a
// (b, h); beta of each window comes from the previous window's mean output,
// formed by the consumers and read by the solve after one idle step.
#include "gdr_kernels.h"
#include "gdr_mfma.h"

namespace gdr {
namespace pipe {

using bf = __bf16;

__device__ inline f32x2 cmul(f32x2 a, f32x2 b) {
  return f32x2{a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x};
}
__device__ inline f32x2 conj(f32x2 a) { return f32x2{a.x, -a.y}; }

__device__ inline f32x2 bf2_to_f2(uint32_t u) {
  return f32x2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
}
__device__ inline uint32_t f2_to_bf2(f32x2 x) {
  bf16x2 v;
  v[0] = (bf)x.x;
  v[1] = (bf)x.y;
  return *(uint32_t*)&v;
}

// K+, Q+ and Kh rows store the key channels of each 32-channel block in the
// order of the "cb" slot map (gdr_mfma.h): position 8g + s holds channel
// 4g + s (s < 4) or 16 + 4g + s - 4 (s >= 4).  A plain 16-byte fragment read
// then pairs with a fragment built from two stacked accumulator tiles, and a
// contraction of two rows stored this way is unchanged.
__device__ constexpr int cb_pos(int c) {
  return (c & ~31) + 8 * ((c & 15) >> 2) + (((c & 31) >> 4) << 2) + (c & 3);
}

constexpr int L = 32;      // tokens per chunk
constexpr int NWP = 4;     // prep waves
constexpr int NWS = 4;     // solve waves
// LDS bank rules of gfx950 (measured with the bank-conflict counter): 4-byte
// accesses go to 32 banks, lanes 0-31 and 32-63 in separate cycles; 8-byte
// accesses to 64 banks, 32 lanes per cycle; 16-byte reads to 64 banks, 16 lanes
// per cycle in a lane grouping that is not plain lane order.  The strides and
// the swizzle below keep the hot accesses free of conflicts under these rules.
constexpr int RSL = L + 4; // row stride of [.][L] arrays
constexpr int RS16 = 20;   // row stride of 16x16 blocks

template <int DK, int TV>
struct Cfg {
  static constexpr int NWC = TV / 16;            // consumer waves
  static constexpr int NT = (NWP + NWS + NWC) * 64;
  static constexpr int NP = DK / 2;              // channel pairs
  static constexpr int PPW = NP / NWP;           // channel pairs per prep wave
  static constexpr int NSEG = 64 / PPW;          // token segments per prep wave
  static constexpr int TPS = L / NSEG;           // tokens per prep lane
  // K+, Q+ and Kh rows: 128 key channels use an 80-dword stride and, in rows
  // with bit 3 set, 16-byte unit u stored at u ^ 6; so the 16-byte fragment
  // reads of 16 rows and the prep's 4-byte stores of rows 8 apart are both
  // conflict-free.  64 key channels keep a 36-dword stride and no swizzle.
  static constexpr int RSK = DK == 128 ? 160 : DK + 8;
  static constexpr int SWZ = DK == 128 ? 6 : 0;
  static constexpr int RSV = TV + 8;
  static constexpr int NCT = DK / 16;
  static constexpr int NKC = DK / 32;
  static constexpr int VPR = TV / 8;             // 16-byte pieces per value row
  static constexpr int VLD = (L * VPR + NWP * 64 - 1) / (NWP * 64);   // per prep thread
  static_assert(TPS % 4 == 0 && TPS >= 4, "prep split");
  static_assert(L * VPR % (NWP * 64) == 0 || L * VPR < NWP * 64, "value tile load split");
};

// Prep outputs of one chunk (3 slots: written for i+2, read for i+1 and i).
template <int DK, int TV>
struct SlotA {
  using C = Cfg<DK, TV>;
  bf Kp[L * C::RSK];
  bf Qp[L * C::RSK];
  bf KhT[DK * RSL];
  bf V[L * C::RSV];
  float beta[L];   // beta (content-aware: the logit b_x)
  float bw[L];     // beta * w (content-aware: w)
  f32x2 GL[C::NP];
};

// 16-byte LDS reads of beta, bw and GL rely on these offsets
template <int DK, int TV>
constexpr bool slot_aligned() {
  using S = SlotA<DK, TV>;
  return offsetof(S, beta) % 16 == 0 && offsetof(S, bw) % 16 == 0 && offsetof(S, GL) % 16 == 0 &&
         sizeof(S) % 16 == 0;
}
static_assert(slot_aligned<128, 64>() && slot_aligned<128, 32>() && slot_aligned<64, 32>() &&
                  slot_aligned<128, 128>() && slot_aligned<64, 64>(),
              "SlotA alignment");

// Solve outputs of one chunk (2 slots).
struct SlotS {
  bf M[L * RSL];
  bf A10[16 * RS16];
  bf Td[2 * 16 * RS16];
};

template <int DK, int TV>
struct Shared {
  using C = Cfg<DK, TV>;
  SlotA<DK, TV> a[3];
  bf Kh[2][L * C::RSK];
  SlotS s[2];
};

template <int TPS, int VLD>
struct Raw {
  uint32_t k[TPS], q[TPS];
  f32x2 a[TPS];
  uint4 v[VLD];
};

// Buffer resources over one (b, h): element (t, c) of a [B,T,H,X] tensor sits at
// byte (t * H * X + c) * size from the resource base, and the resource ends
// after token T-1, so loads past the sequence return zero without a branch.
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(uint32_t)bytes, 0x00020000);
}

struct Rsrc {
  rsrc_t k, q, a, th, v, beta, w;
  int sk, sa, sv, sb;   // per-token byte strides
};

template <int DK, int TV, int DECAY>
__device__ inline Rsrc make_rsrcs(const FwdParams& p, int b, int h, int v0) {
  const int Tn = p.T, H = p.H, DV = p.DV;
  const size_t bh = (size_t)b * Tn * H + h;
  const size_t rows = (size_t)(Tn - 1) * H + 1;   // token rows up to token T-1 of head h
  Rsrc r;
  r.sk = H * DK * 2;
  r.k = make_rsrc((const bf*)p.k + bh * DK, rows * DK * 2);
  r.q = make_rsrc((const bf*)p.q + bh * DK, rows * DK * 2);
  if constexpr (DECAY == 0) {
    r.sa = H * DK * 4;
    r.a = make_rsrc(p.alpha + bh * DK, rows * DK * 4);
    r.th = r.a;
  } else {
    r.sa = H * (DK / 2) * 4;
    r.a = make_rsrc(p.alpha + bh * (DK / 2), rows * (DK / 2) * 4);
    r.th = make_rsrc(p.theta + bh * (DK / 2), rows * (DK / 2) * 4);
  }
  r.sv = H * DV * 2;
  r.v = make_rsrc((const bf*)p.v + bh * DV + v0, rows * DV * 2 - (size_t)v0 * 2);
  r.sb = H * 4;
  r.beta = make_rsrc(p.beta + bh, rows * 4);
  r.w = make_rsrc(p.w + bh, rows * 4);
  return r;
}

// A or B operand from K+, Q+ or Kh rows: rows row0 + n (row0 a multiple of 16),
// contraction over key positions 32 kk .. 32 kk + 31 in the plain slot map.
template <int DK, int TV>
__device__ inline bf16x8 load_kq(const bf* base, int row0, int kk) {
  using C = Cfg<DK, TV>;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int sw = C::SWZ * ((n >> 3) & 1);
  return *(const bf16x8*)(base + (row0 + n) * C::RSK + (((4 * kk + g) ^ sw) << 3));
}

// Byte offsets: the per-lane part goes in voffset, the per-token part (uniform)
// in soffset.  Both count in the range check of a raw buffer (no stride), so
// tokens at or past T still read as zero.
// PART 0: value tile; 1: key-axis transitions; 2: keys; 3: queries.
template <int DK, int TV, int DECAY, int PART>
__device__ inline void load_part(Raw<Cfg<DK, TV>::TPS, Cfg<DK, TV>::VLD>& R, const Rsrc& rs, int c0, int pp, int seg,
                                 int ptid) {
  using C = Cfg<DK, TV>;
  if constexpr (PART == 0) {
#pragma unroll
    for (int u = 0; u < C::VLD; ++u) {
      const int idx0 = ptid + u * NWP * 64;
      const int idx = idx0 < L * C::VPR ? idx0 : 0;
      const int r = idx / C::VPR, cc = idx % C::VPR;
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs.v, r * rs.sv + cc * 16, c0 * rs.sv, 0);
      R.v[u] = uint4{x[0], x[1], x[2], x[3]};
    }
  } else if constexpr (PART == 1) {
    const int al = seg * C::TPS * rs.sa + (DECAY == 0 ? 8 : 4) * pp;
#pragma unroll
    for (int r = 0; r < C::TPS; ++r) {
      const int as = (c0 + r) * rs.sa;   // uniform
      if constexpr (DECAY == 0) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs.a, al, as, 0);
        R.a[r] = f32x2{__uint_as_float(x[0]), __uint_as_float(x[1])};
      } else {
        R.a[r] = f32x2{__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs.a, al, as, 0)),
                       __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs.th, al, as, 0))};
      }
    }
  } else {
    const int kl = seg * C::TPS * rs.sk + 4 * pp;
#pragma unroll
    for (int r = 0; r < C::TPS; ++r) {
      const int ks = (c0 + r) * rs.sk;   // uniform
      if constexpr (PART == 2) R.k[r] = __builtin_amdgcn_raw_buffer_load_b32(rs.k, kl, ks, 0);
      else R.q[r] = __builtin_amdgcn_raw_buffer_load_b32(rs.q, kl, ks, 0);
    }
  }
}

template <int DK, int TV, int DECAY>
__device__ inline void load_raw(Raw<Cfg<DK, TV>::TPS, Cfg<DK, TV>::VLD>& R, const Rsrc& rs, int c0, int pp, int seg,
                                int ptid) {
  load_part<DK, TV, DECAY, 0>(R, rs, c0, pp, seg, ptid);
  load_part<DK, TV, DECAY, 1>(R, rs, c0, pp, seg, ptid);
  load_part<DK, TV, DECAY, 2>(R, rs, c0, pp, seg, ptid);
  load_part<DK, TV, DECAY, 3>(R, rs, c0, pp, seg, ptid);
}

// Value held by lane l ^ (PPW * d) (d = 1, 2, 4; PPW * d in {8, 16, 32}):
// a row rotation by 8 within rows of 16 lanes (one DPP move), else a backward
// permute through the LDS crossbar, which takes one DS instruction and no VALU
// issue slot (the v_permlane swaps need two copies and a select per value).
template <int PPW>
__device__ inline float xor_lanes(float v, int d, int l) {
  const int dist = PPW * d;
  const unsigned u = __float_as_uint(v);
  if (dist == 8) {
    return __uint_as_float(__builtin_amdgcn_mov_dpp(u, 0x128, 0xf, 0xf, false));   // row_ror:8
  } else {   // LDS crossbar: one DS instruction, no VALU issue
    return __uint_as_float((unsigned)__builtin_amdgcn_ds_bpermute((l ^ dist) << 2, (int)u));
  }
}

// One prep step: decayed key/query forms of 32-token block `it` (raw loads in
// R) into prep slot vs % 3 and the Kh buffer vs % 2 (vs: the block's step).
// With NEXT, the raw loads of the chunk at token cn go into Rn, spread over the
// step in four groups so that the prep waves do not all stall on a full
// vector-memory queue at the start of every step.
template <int DK, int TV, int DECAY, bool NEXT>
__device__ __forceinline__ void prep_chunk(Shared<DK, TV>& sh, const Raw<Cfg<DK, TV>::TPS, Cfg<DK, TV>::VLD>& R,
                                           Raw<Cfg<DK, TV>::TPS, Cfg<DK, TV>::VLD>& Rn, const Rsrc& rs, int cn,
                                           int it, int vs, int Tn, int pw, int l, int pl,
                                           int seg, int pp, int ptid) {
  using C = Cfg<DK, TV>;
  constexpr int PPW = C::PPW, NSEG = C::NSEG, TPS = C::TPS, RSK = C::RSK, RSV = C::RSV,
                VPR = C::VPR;
  SlotA<DK, TV>& A = sh.a[vs % 3];
  bf* Kh = sh.Kh[vs & 1];
  const int c0 = it * L;
  if constexpr (NEXT) load_part<DK, TV, DECAY, 0>(Rn, rs, cn, pp, seg, ptid);
  // transitions of this lane's token segment (identity past the end)
  f32x2 d[TPS];
  if (c0 + L <= Tn) {
#pragma unroll
    for (int r = 0; r < TPS; ++r) d[r] = R.a[r];
  } else {
#pragma unroll
    for (int r = 0; r < TPS; ++r) {
      const bool ok = c0 + seg * TPS + r < Tn;
      d[r].x = ok ? R.a[r].x : 1.f;
      d[r].y = ok ? R.a[r].y : (DECAY == 0 ? 1.f : 0.f);
    }
  }
  if constexpr (DECAY != 0) {
#pragma unroll
    for (int r = 0; r < TPS; ++r) {   // (gamma, theta) -> gamma e^{i theta}
      float sn, cs;
      __sincosf(d[r].y, &sn, &cs);
      d[r] = f32x2{d[r].x * cs, d[r].x * sn};
    }
  }
  auto mulz = [](f32x2 u, f32x2 v) {
    return (DECAY == 0) ? f32x2{u.x * v.x, u.y * v.y} : cmul(u, v);
  };
  const f32x2 one = {1.f, DECAY == 0 ? 1.f : 0.f};
  if constexpr (NEXT) {
    __builtin_amdgcn_sched_barrier(0);
    load_part<DK, TV, DECAY, 1>(Rn, rs, cn, pp, seg, ptid);
  }
  f32x2 run = d[0];
#pragma unroll
  for (int r = 1; r < TPS; ++r) run = mulz(run, d[r]);
#pragma unroll
  for (int u = 0; u < C::VLD; ++u) {
    const int idx = ptid + u * NWP * 64;
    if (idx < L * VPR) {
      const int r = idx / VPR, cc = idx % VPR;
      *(uint4*)(A.V + r * RSV + cc * 8) = R.v[u];
    }
  }
  // products over the earlier (pre) and later (post) segments of this lane's
  // channel pair, and over the whole chunk (tot): a butterfly over the NSEG
  // segments (lanes PPW apart) with cross-lane swaps; every factor is a
  // diagonal or 2x2-rotation transition, so the products commute
  f32x2 pre = one, post = one, tot = run;
#pragma unroll
  for (int d = 1; d < NSEG; d *= 2) {
    const f32x2 tp = {xor_lanes<PPW>(tot.x, d, l), xor_lanes<PPW>(tot.y, d, l)};
    const bool upper = (seg & d) != 0;   // partner block holds earlier segments
    pre = mulz(pre, upper ? tp : one);
    post = mulz(post, upper ? one : tp);
    tot = mulz(tot, tp);
  }
  if (seg == 0) A.GL[pp] = tot;
  if constexpr (NEXT) {
    __builtin_amdgcn_sched_barrier(0);
    load_part<DK, TV, DECAY, 2>(Rn, rs, cn, pp, seg, ptid);
  }
  f32x2 ig;   // Gamma_L^{-T} per channel (pair)
  if constexpr (DECAY == 0) {
    ig = f32x2{__builtin_amdgcn_rcpf(tot.x), __builtin_amdgcn_rcpf(tot.y)};
  } else {
    const float nz = __builtin_amdgcn_rcpf(tot.x * tot.x + tot.y * tot.y);
    ig = f32x2{tot.x * nz, tot.y * nz};
  }
  // running products from the chunk start (gf = Gamma_r) and, for Kh, the
  // product to the chunk end times Gamma_L^{-T} (hb = Gamma_L^{-T} h_r^T)
  f32x2 gfv[TPS], hbv[TPS];
  {
    f32x2 rf = pre;
#pragma unroll
    for (int r = 0; r < TPS; ++r) {
      rf = mulz(rf, d[r]);
      gfv[r] = rf;
    }
    f32x2 rb = (DECAY == 0) ? mulz(post, ig) : cmul(ig, conj(post));
#pragma unroll
    for (int r = TPS - 1; r >= 0; --r) {
      hbv[r] = rb;
      rb = (DECAY == 0) ? mulz(rb, d[r]) : cmul(rb, conj(d[r]));
    }
  }
  // stored position of this channel pair (rows of one lane share bit 3 when
  // segments are 8 tokens, so one swizzled position serves all of them)
  static_assert(C::SWZ == 0 || TPS == 8, "K+/Q+/Kh swizzle assumes 8-token segments");
  const int pc0 = cb_pos(2 * pp);
  const int pc = (((pc0 >> 3) ^ (C::SWZ * (seg & 1))) << 3) | (pc0 & 7);
  float kh0[TPS], kh1[TPS];
#pragma unroll
  for (int r4 = 0; r4 < TPS; r4 += 4) {
    if (NEXT && r4 == (TPS > 4 ? 4 : 0)) {
      __builtin_amdgcn_sched_barrier(0);
      load_part<DK, TV, DECAY, 3>(Rn, rs, cn, pp, seg, ptid);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r4 + u;
      const int row = seg * TPS + r;
      const f32x2 kx = bf2_to_f2(R.k[r]), qx = bf2_to_f2(R.q[r]);
      f32x2 kp, qp, kh;
      const f32x2 gf = gfv[r], hb = hbv[r];
      if constexpr (DECAY == 0) {
        kp = f32x2{kx.x * gf.x, kx.y * gf.y};
        qp = f32x2{qx.x * gf.x, qx.y * gf.y};
        kh = f32x2{kx.x * hb.x, kx.y * hb.y};
      } else {
        kp = cmul(gf, kx);
        qp = cmul(gf, qx);
        kh = cmul(hb, kx);
      }
      *(uint32_t*)(A.Kp + row * RSK + pc) = f2_to_bf2(kp);
      *(uint32_t*)(A.Qp + row * RSK + pc) = f2_to_bf2(qp);
      *(uint32_t*)(Kh + row * RSK + pc) = f2_to_bf2(kh);
      kh0[r] = kh.x;
      kh1[r] = kh.y;
    }
  }
  // Kh transposed: one 16-byte store per channel for 8-token segments
  // (conflict-free at the 18-dword row stride), 8-byte stores otherwise
  if constexpr (TPS == 8) {
    bf16x8 m0, m1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      m0[u] = (bf)kh0[u];
      m1[u] = (bf)kh1[u];
    }
    *(bf16x8*)(A.KhT + (2 * pp) * RSL + seg * TPS) = m0;
    *(bf16x8*)(A.KhT + (2 * pp + 1) * RSL + seg * TPS) = m1;
  } else {
#pragma unroll
    for (int r4 = 0; r4 < TPS; r4 += 4) {
      bf16x4 m0, m1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        m0[u] = (bf)kh0[r4 + u];
        m1[u] = (bf)kh1[r4 + u];
      }
      *(bf16x4*)(A.KhT + (2 * pp) * RSL + seg * TPS + r4) = m0;
      *(bf16x4*)(A.KhT + (2 * pp + 1) * RSL + seg * TPS + r4) = m1;
    }
  }
}

template <int DK, int TV, int DECAY, bool CONTENT>
__global__ __launch_bounds__((NWP + NWS + TV / 16) * 64) void gdr_fwd_pipe_kernel(FwdParams p) {
  using C = Cfg<DK, TV>;
  using O = Op<bf>;
  using frag = O::frag;
  constexpr int NP = C::NP, PPW = C::PPW, NSEG = C::NSEG, TPS = C::TPS, RSK = C::RSK,
                RSV = C::RSV, NCT = C::NCT, NKC = C::NKC, VPR = C::VPR;
  __shared__ __attribute__((aligned(16))) Shared<DK, TV> sh;

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = l & 15, g = l >> 4;

  const int nvt = p.n_vt;
  const int grp = blockIdx.x / (8 * nvt), rem = blockIdx.x % (8 * nvt);
  const int unit = grp * 8 + (rem & 7);
  const int vt = rem >> 3;
  if (unit >= p.n_units) return;
  const int b = unit / p.H, h = unit % p.H;
  const int v0 = vt * TV;
  const int Tn = p.T, H = p.H, DV = p.DV;
  const int nchunks = (Tn + L - 1) / L;   // 32-token blocks
  // Content-aware erase: beta of a window of SPC blocks needs the previous
  // window's mean output, which the consumers finish one step before the
  // solve of the window's first block can use it; so one idle step follows
  // every window.  Block j then runs its prep at step vj = j + j / SPC, its
  // solve at vj + 1 and its consumer at vj + 2; slots rotate by step.
  const int SPC = CONTENT ? p.window / L : 1;
  auto vstep = [&](int j) { return CONTENT ? j + j / SPC : j; };
  auto block_at = [&](int v) {   // block whose prep runs at step v, -1 if idle
    return CONTENT ? ((v % (SPC + 1) == SPC) ? -1 : v - v / (SPC + 1)) : v;
  };
  const int nsteps = vstep(nchunks - 1) + 3;
  // u_h = B_h^T a_h and the mean output of the previous window (the carried
  // mean, or zero, before the first window)
  __shared__ float sU[CONTENT ? TV : 1], sMean[CONTENT ? TV : 1];
  // content-aware: beta and beta*w of a block, computed by the solve for the
  // consumer (one per prep slot)
  __shared__ __attribute__((aligned(16))) float sBc[CONTENT ? 3 : 1][CONTENT ? 2 : 1][L];
  if constexpr (CONTENT) {
    if (tid < TV) {
      float acc = 0.f;
      for (int r = 0; r < p.ub_rank; ++r)
        acc += p.ub_up[h * p.ub_rank + r] * p.ub_down[((size_t)h * p.ub_rank + r) * DV + tid];
      sU[tid] = acc;
      sMean[tid] = p.m_carry ? p.m_carry[(size_t)(b * H + h) * DV + tid] : 0.f;
    }
    lds_barrier();
  }

  if (wv < NWP) {
    // ================================================================ prep
    // Raw loads run two chunks ahead (issued two steps before their use, which
    // covers the memory latency under load), in three register sets with the
    // loop unrolled by three.  They are unconditional (the last chunk is
    // loaded again at the end) so that the outstanding-load count at every use
    // is known statically.
    const int pw = wv;
    // With one block per (b, h) the content-aware launch keeps one workgroup
    // per CU; there the consumer's chain sets the step time, so it issues
    // first, then the prep, then the solve.  (The plain launches run faster
    // at equal priority.)
    if constexpr (CONTENT) __builtin_amdgcn_s_setprio(1);
    const int pl = l % PPW, seg = l / PPW, pp = pw * PPW + pl;
    const int ptid = tid;                       // 0 .. NWP*64-1
    const Rsrc rs = make_rsrcs<DK, TV, DECAY>(p, b, h, v0);
    const int clast = (nchunks - 1) * L;
    auto idle_after = [&](int j) {   // the idle step after a window's last block
      if (CONTENT && j % SPC == SPC - 1 && j + 1 < nchunks) lds_barrier();
    };
    int it = 0;
    if constexpr (C::NT > 12 * 64) {
      // 16 waves leave 128 VGPRs per wave: one chunk ahead, two register sets
      Raw<TPS, C::VLD> R0, R1;
      load_raw<DK, TV, DECAY>(R0, rs, 0, pp, seg, ptid);
      for (; it + 1 < nchunks; it += 2) {
        prep_chunk<DK, TV, DECAY, true>(sh, R0, R1, rs, (it + 1) * L, it, vstep(it), Tn, pw, l, pl,
                                        seg, pp, ptid);
        lds_barrier();
        idle_after(it);
        prep_chunk<DK, TV, DECAY, true>(sh, R1, R0, rs, min((it + 2) * L, clast), it + 1,
                                        vstep(it + 1), Tn, pw, l, pl, seg, pp, ptid);
        lds_barrier();
        idle_after(it + 1);
      }
      if (it < nchunks) {   // odd chunk count: the last chunk is in R0
        prep_chunk<DK, TV, DECAY, false>(sh, R0, R1, rs, 0, it, vstep(it), Tn, pw, l, pl, seg, pp,
                                         ptid);
        lds_barrier();
        ++it;
      }
    } else {
    Raw<TPS, C::VLD> R0, R1, R2;
    load_raw<DK, TV, DECAY>(R0, rs, 0, pp, seg, ptid);
    load_raw<DK, TV, DECAY>(R1, rs, min(L, clast), pp, seg, ptid);
    for (; it + 2 < nchunks; it += 3) {
      prep_chunk<DK, TV, DECAY, true>(sh, R0, R2, rs, (it + 2) * L, it, vstep(it), Tn, pw, l, pl,
                                      seg, pp, ptid);
      lds_barrier();
      idle_after(it);
      prep_chunk<DK, TV, DECAY, true>(sh, R1, R0, rs, min((it + 3) * L, clast), it + 1,
                                      vstep(it + 1), Tn, pw, l, pl, seg, pp, ptid);
      lds_barrier();
      idle_after(it + 1);
      prep_chunk<DK, TV, DECAY, true>(sh, R2, R1, rs, min((it + 4) * L, clast), it + 2,
                                      vstep(it + 2), Tn, pw, l, pl, seg, pp, ptid);
      lds_barrier();
      idle_after(it + 2);
    }
    // one or two chunks left: they are in R0 and R1
    if (it < nchunks) {
      prep_chunk<DK, TV, DECAY, false>(sh, R0, R2, rs, 0, it, vstep(it), Tn, pw, l, pl, seg, pp,
                                       ptid);
      lds_barrier();
      idle_after(it);
      ++it;
    }
    if (it < nchunks) {
      prep_chunk<DK, TV, DECAY, false>(sh, R1, R2, rs, 0, it, vstep(it), Tn, pw, l, pl, seg, pp,
                                       ptid);
      lds_barrier();
      ++it;
    }
    }
    for (int st = vstep(nchunks - 1) + 1; st < nsteps; ++st) lds_barrier();
  } else if (wv < NWP + NWS) {
    // ================================================================ solve
    const int sw = wv - NWP;
    // the last solve wave also stages beta and beta*w (content-aware: the
    // logit b_x and w): loads one block ahead, written into the prep slot of
    // the block being prepared in this step (tokens at or past T read as zero)
    const float* pbeta = CONTENT ? p.beta_logit : p.beta;
    const rsrc_t rb = make_rsrc(pbeta + ((size_t)b * Tn * H + h), ((size_t)(Tn - 1) * H + 1) * 4);
    const rsrc_t rw = make_rsrc(p.w + ((size_t)b * Tn * H + h), ((size_t)(Tn - 1) * H + 1) * 4);
    const int tb = (l < L ? l : L - 1) * H * 4;
    float nbt = 0.f, nwt = 0.f;
    if (sw == NWS - 1) {
      nbt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, tb, 0, 0));
      nwt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, tb, 0, 0));
    }
    float s_win = 0.f;   // content-aware: s_c = u_h . m_c of the current window
    for (int it = 0; it < nsteps; ++it) {
      const int jp = CONTENT ? block_at(it) : it;
      if (sw == NWS - 1 && (CONTENT ? (jp >= 0 && jp < nchunks) : (it < nchunks))) {
        const float bt = nbt, wt = nwt;
        const int cn = min(jp + 1, nchunks - 1) * L * H * 4;   // uniform
        nbt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, tb, cn, 0));
        nwt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, tb, cn, 0));
        if (l < L) {
          sh.a[it % 3].beta[l] = bt;
          sh.a[it % 3].bw[l] = CONTENT ? wt : bt * wt;
        }
      }
      const int vj = it - 1;
      const int j = CONTENT ? (vj >= 0 ? block_at(vj) : -1) : vj;
      if (j >= 0 && j < nchunks) {
        const SlotA<DK, TV>& A = sh.a[vj % 3];
        const bf* Kh = sh.Kh[vj & 1];
        SlotS& S = sh.s[vj & 1];
        if constexpr (CONTENT) {
          if (j % SPC == 0) {   // new window: s_c from the previous window's mean (fixed order)
            float acc = 0.f;
            for (int vv = l; vv < TV; vv += 64) acc += sU[vv] * sMean[vv];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            s_win = acc;
          }
        }
        auto beta_at = [&](int r) {
          if constexpr (CONTENT) return 1.f / (1.f + __expf(-(A.beta[r] + s_win)));
          else return A.beta[r];
        };
        if constexpr (CONTENT) {   // beta and beta*w of this block for the consumer
          if (sw == NWS - 1 && l < L) {
            const float bt = beta_at(l);
            sBc[vj % 3][0][l] = bt;
            sBc[vj % 3][1][l] = bt * A.bw[l];
          }
        }
        if (sw < 2) {
          // diagonal block bb: N and N^T as accumulator tiles, then
          // T_bb = (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8).
          // mul(Q, Y) = C(Q^T Y): a tile feeds the left operand as its transpose.
          const int bb = sw;
          f32x4 g0 = {0.f, 0.f, 0.f, 0.f}, g1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKC; ++kk) {
            const frag kp = load_kq<DK, TV>(A.Kp, 16 * bb, kk);
            const frag kh = load_kq<DK, TV>(Kh, 16 * bb, kk);
            O::mma(g0, kp, kh);   // (K+ Kh^T)[4g+j][n]
            O::mma(g1, kh, kp);   // (K+ Kh^T)[n][4g+j]
          }
          f32x4 Nc, Nt, Pt;
          const float bn = beta_at(16 * bb + n);
          // content-aware: beta of rows 4g..4g+3 (a sigmoid each) for all lanes
          // up front, so that no divergent branch guards them
          f32x4 br = {0.f, 0.f, 0.f, 0.f};
          if constexpr (CONTENT) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) br[jj] = beta_at(16 * bb + 4 * g + jj);
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int rr = 4 * g + jj;
            Nc[jj] = (n < rr) ? (CONTENT ? br[jj] : beta_at(16 * bb + rr)) * g0[jj] : 0.f;   // N[rr][n]
            Nt[jj] = (rr < n) ? bn * g1[jj] : 0.f;                     // N[n][rr]
            Pt[jj] = ((rr == n) ? 1.f : 0.f) - Nt[jj];                  // (I - N)^T
          }
          auto mul = [](const f32x4& Q, const f32x4& Y) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            O::mma(z, O::from_acc_half(Q), O::from_acc_half(Y));
            return z;
          };
          const f32x4 N2 = mul(Nt, Nc), N2t = mul(Nc, Nt);
          const f32x4 N4 = mul(N2t, N2), N4t = mul(N2, N2t);
          const f32x4 N8 = mul(N4t, N4);
          Pt += mul(N2, Pt);
          Pt += mul(N4, Pt);
          Pt += mul(N8, Pt);   // T^T: lane holds T[n][4g..4g+3]
          bf16x4 tv;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) tv[jj] = (bf)Pt[jj];
          *(bf16x4*)(S.Td + (bb * 16 + n) * RS16 + 4 * g) = tv;
        } else {
          // wave 2: A10 and M00; wave 3: M10 and M11.  Y = R1 - A10 Dl0 takes
          // -A10: with rotation decay the solve stores it negated, with
          // diagonal decay the consumer negates it (the faster schedule of each)
#pragma unroll
          for (int ti = 0; ti < 2; ++ti) {
            const bool isA = (sw == 2 && ti == 0);
            const int rb = (sw == 2) ? (ti == 0 ? 1 : 0) : 1;
            const int cbk = (sw == 3) ? ti : 0;
            const bf* src = isA ? A.Kp : A.Qp;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKC; ++kk)
              O::mma(acc, load_kq<DK, TV>(src, 16 * rb, kk), load_kq<DK, TV>(Kh, 16 * cbk, kk));
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int rr = 16 * rb + 4 * g + jj, cc = 16 * cbk + n;
              if (isA) {
                S.A10[(4 * g + jj) * RS16 + n] = (bf)((DECAY != 0 ? -1.f : 1.f) * beta_at(rr) * acc[jj]);
              } else {
                S.M[rr * RSL + cc] = (bf)((cc <= rr) ? acc[jj] : 0.f);
              }
            }
          }
        }
      }
      lds_barrier();
    }
  } else {
    // ============================================================ consumer
    const int cw = wv - NWP - NWS;              // value block of 16 channels
    if constexpr (CONTENT) __builtin_amdgcn_s_setprio(2);
    f32x4 Sacc[NCT];
    const size_t srow = ((size_t)(b * H + h) * DV + v0 + 16 * cw + n) * DK;
    if (p.S0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) Sacc[ct] = *(const f32x4*)(p.S0 + srow + 16 * ct + 4 * g);
    } else {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) Sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // drain the state load here, so that inside the loop only the loop's own
    // output stores are outstanding and no wait on them is needed
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    // o through a buffer resource over this wave's 16 value channels of (b, h):
    // stores past token T-1 fall outside the resource and are dropped.
    const size_t obh = (size_t)b * Tn * H + h;
    const size_t orows = (size_t)(Tn - 1) * H + 1;
    const int ocol = v0 + 16 * cw;
    const rsrc_t ro = make_rsrc((bf*)p.o + obh * DV + ocol, orows * DV * 2 - (size_t)ocol * 2);
    const int so = H * DV * 2;                     // bytes per token row
    const int olane = n * so + 8 * g;              // token n, value channels 4g..4g+3
    float colsum[4] = {0.f, 0.f, 0.f, 0.f};   // content-aware: window sums of 4 channels
    for (int it = 0; it < nsteps; ++it) {
      const int vi = it - 2;
      const int i = CONTENT ? (vi >= 0 ? block_at(vi) : -1) : vi;
      if (CONTENT ? (i >= 0 && i < nchunks) : (i >= 0)) {
        const SlotA<DK, TV>& A = sh.a[vi % 3];
        const SlotS& S = sh.s[vi & 1];
        const int c0 = i * L;
        // R = diag(bw) V - diag(beta) K+ S^T;  Qs^T = (Q+ S^T)^T, kept transposed
        // (lane holds one token and four value channels) for 8-byte o stores
        frag Sf[NKC];
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk) Sf[kk] = O::from_acc(Sacc[2 * kk], Sacc[2 * kk + 1]);
        f32x4 Rt[2], Qs[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 P = {0.f, 0.f, 0.f, 0.f}, Q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKC; ++kk) {
            O::mma(P, load_kq<DK, TV>(A.Kp, 16 * t, kk), Sf[kk]);
            O::mma(Q, Sf[kk], load_kq<DK, TV>(A.Qp, 16 * t, kk));
          }
          const f32x4 bw4 = *(const f32x4*)((CONTENT ? sBc[vi % 3][1] : A.bw) + 16 * t + 4 * g);
          const f32x4 bt4 = *(const f32x4*)((CONTENT ? sBc[vi % 3][0] : A.beta) + 16 * t + 4 * g);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * t + 4 * g + jj;
            Rt[t][jj] = bw4[jj] * (float)A.V[r * RSV + 16 * cw + n] - bt4[jj] * P[jj];
          }
          Qs[t] = Q;
        }
        // Dl by blocks, O = Qs + M Dl
        f32x4 D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
        O::mma(D0, load_cb_half<bf>(S.Td, RS16, 0, 0), O::from_acc_half(Rt[0]));
        const frag d0 = O::from_acc_half(D0);
        f32x4 Y = Rt[1];
        {
          const frag a10 = load_cb_half<bf>(S.A10, RS16, 0, 0);
          O::mma(Y, DECAY != 0 ? a10 : O::neg(a10), d0);
        }
        O::mma(D1, load_cb_half<bf>(S.Td + 16 * RS16, RS16, 0, 0), O::from_acc_half(Y));
        frag Df = d0;   // slots 0..3 from D0, 4..7 from D1
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Df[4 + jj] = (bf)D1[jj];
        // O^T = Qs^T + (M Dl)^T = Qs^T + Dl^T M^T
        f32x4 O0 = Qs[0], O1 = Qs[1];
        O::mma(O0, d0, load_cb_half<bf>(S.M, RSL, 0, 0));
        O::mma(O1, Df, load_cb<bf>(S.M, RSL, 16, 0));
        const bf16x4 ox0 = {(bf)O0[0], (bf)O0[1], (bf)O0[2], (bf)O0[3]};
        const bf16x4 ox1 = {(bf)O1[0], (bf)O1[1], (bf)O1[2], (bf)O1[3]};
        if constexpr (CONTENT) {
          // window sums of the fp32 outputs (tokens past T contribute zero);
          // at a window's last block its per-channel mean goes to LDS, to be
          // read by the solve of the next window's first block
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) colsum[jj] += O0[jj] + O1[jj];
          if (i % SPC == SPC - 1) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              float sum = colsum[jj];
#pragma unroll
              for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off);
              if (n == 0) sMean[16 * cw + 4 * g + jj] = sum * (1.f / (float)(SPC * L));
              colsum[jj] = 0.f;
            }
          }
        }
        // S <- S Gamma_L + Dl^T K- = (S + Dl^T Kh) Gamma_L, since K- = Kh Gamma_L
        // column-wise (per channel, or per rotation pair)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          O::mma(Sacc[ct], load_cb<bf>(A.KhT, RSL, 16 * ct, 0), Df);
          const f32x4 z4 = *(const f32x4*)(A.GL + 8 * ct + 2 * g);   // channels 16ct+4g..+3
#pragma unroll
          for (int jj = 0; jj < 4; jj += 2) {
            const f32x2 z = {z4[jj], z4[jj + 1]};
            const float x0 = Sacc[ct][jj], x1 = Sacc[ct][jj + 1];
            if constexpr (DECAY == 0) {
              Sacc[ct][jj] = x0 * z.x;
              Sacc[ct][jj + 1] = x1 * z.y;
            } else {
              Sacc[ct][jj] = z.x * x0 + z.y * x1;
              Sacc[ct][jj + 1] = -z.y * x0 + z.x * x1;
            }
          }
        }
        {   // o stores last, off the chain from the barrier to the state update
          typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
          __builtin_amdgcn_raw_buffer_store_b64(*(const u32x2*)&ox0, ro, olane, c0 * so, 0);
          __builtin_amdgcn_raw_buffer_store_b64(*(const u32x2*)&ox1, ro, olane, (c0 + 16) * so, 0);
        }
      }
      lds_barrier();
    }
    if (p.S_out) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) *(f32x4*)(p.S_out + srow + 16 * ct + 4 * g) = Sacc[ct];
    }
    if constexpr (CONTENT) {   // the last window's mean (T is a multiple of the window)
      if (p.m_carry && n == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          p.m_carry[(size_t)(b * H + h) * DV + 16 * cw + 4 * g + jj] = sMean[16 * cw + 4 * g + jj];
      }
    }
  }
}

template <int DK, int TV, int DECAY, bool CONTENT = false>
hipError_t launch(const FwdParams& p0, hipStream_t s) {
  FwdParams p = p0;
  p.n_vt = p.DV / TV;
  p.n_units = p.B * p.H;
  const int groups = (p.n_units + 7) / 8;
  hipLaunchKernelGGL((gdr_fwd_pipe_kernel<DK, TV, DECAY, CONTENT>), dim3(groups * 8 * p.n_vt),
                     dim3(Cfg<DK, TV>::NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace pipe

bool fwd_pipe_supported(const FwdParams& p) {
  // buffer resources address one (b, h) with 32-bit byte offsets
  const bool fits = (unsigned long long)p.T * p.H * p.DK * 4ull < (1ull << 31);
  // content-aware: the window must be a whole number of 32-token blocks
  const bool content_ok = p.beta_logit == nullptr || (p.window >= 32 && p.window % 32 == 0);
  return p.io_bf16 && content_ok && (p.DK == 64 || p.DK == 128) && p.DV == p.DK && fits;
}

hipError_t launch_fwd_pipe(const FwdParams& p, hipStream_t s) {
  const bool rot = p.decay != 0;
  if (p.beta_logit != nullptr) {   // content-aware: one workgroup covers all value channels
    if (p.DK == 128) return rot ? pipe::launch<128, 128, 1, true>(p, s) : pipe::launch<128, 128, 0, true>(p, s);
    return rot ? pipe::launch<64, 64, 1, true>(p, s) : pipe::launch<64, 64, 0, true>(p, s);
  }
  if (p.DK == 128) {
    if ((long)p.B * p.H * 2 >= 192) {
      return rot ? pipe::launch<128, 64, 1>(p, s) : pipe::launch<128, 64, 0>(p, s);
    }
    return rot ? pipe::launch<128, 32, 1>(p, s) : pipe::launch<128, 32, 0>(p, s);
  }
  if (p.DK == 64) return rot ? pipe::launch<64, 32, 1>(p, s) : pipe::launch<64, 32, 0>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace gdr
