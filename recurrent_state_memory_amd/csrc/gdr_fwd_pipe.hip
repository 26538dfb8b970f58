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
#include <type_traits>

#include "gdr_kernels.h"
#include "gdr_mfma.h"
#include "gdr_token.h"

namespace gdr {
namespace pipe {

using bf = __bf16;

__device__ inline f32x2 cmul(f32x2 a, f32x2 b) {
  return f32x2{a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x};
}
__device__ inline f32x2 conj(f32x2 a) { return f32x2{a.x, -a.y}; }

// Rotation and reflection blocks (DECAY == 2).  A block acts on a key pair,
// as a complex number x, by x -> w x (rotation-scale) or x -> w conj(x)
// (reflection-scale, |gamma| R(theta) Diag(1, -1)); such maps compose as
// (w1, s1) o (w2, s2) = (w1 c^s1(w2), s1 xor s2) and do not commute.  The
// reflection bit s travels in the lowest mantissa bit of w.x (a 2^-24 relative
// perturbation, far below the bf16 operands), so a map is still one f32x2.
__device__ inline unsigned refl_bit(f32x2 m) { return __float_as_uint(m.x) & 1u; }
__device__ inline f32x2 with_refl(f32x2 w, unsigned s) {
  return f32x2{__uint_as_float((__float_as_uint(w.x) & ~1u) | s), w.y};
}

__device__ inline f32x2 bf2_to_f2(uint32_t u) {
  return f32x2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
}
// Decay from its pre-activation (gated forward): exp(-a softplus(x)), as
// 2^(-a (max(x, 0) log2 e + log2(1 + 2^(-|x| log2 e)))): no overflow for large
// |x|; for x below about -17 softplus(x) < 2^-24 is dropped (an error below one
// fp32 ulp of the decay).
__device__ inline float gate_act(float x, float a) {
  constexpr float kLog2e = 1.44269504088896341f;
  const float t = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);
  const float sp2 = __builtin_fmaxf(x, 0.f) * kLog2e + __builtin_amdgcn_logf(1.f + t);
  return __builtin_amdgcn_exp2f(-a * sp2);
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
  // content-aware erase: the prep loads whole value rows (DK == DV pieces of
  // 8), stores this workgroup's tile and reduces u_h . v_t over the row
  static constexpr int VPRF = DK / 8;
  static constexpr int VLDF = L * VPRF / (NWP * 64);
  static_assert(TPS % 4 == 0 && TPS >= 4, "prep split");
  static_assert(L * VPR % (NWP * 64) == 0 || L * VPR < NWP * 64, "value tile load split");
  static_assert(L * VPRF % (NWP * 64) == 0 && (NWP * 64) % VPRF == 0, "value row load split");
};

// Bytes of one chunk in raw form for the token path (gdr_token.h): the
// transition as fp32 per channel, then raw keys and queries.
template <int DK>
constexpr int raw_bytes() { return L * DK * (4 + 2 + 2); }

template <int DK>
constexpr int raw_pad() {   // bf16 elements that extend Kp|Qp|KhT to raw_bytes()
  constexpr int have = 2 * (2 * L * (DK == 128 ? 160 : DK + 8) + DK * RSL);
  return raw_bytes<DK>() > have ? (raw_bytes<DK>() - have + 15) / 16 * 8 : 8;
}

// Prep outputs of one chunk (3 slots: written for i+2, read for i+1 and i).
// Kp, Qp, KhT and pad are contiguous: a chunk whose decay leaves the split
// form's range holds its raw transition, keys and queries there instead
// (written by the solve, read by the consumer's token path).
template <int DK, int TV>
struct SlotA {
  using C = Cfg<DK, TV>;
  bf Kp[L * C::RSK];
  bf Qp[L * C::RSK];
  bf KhT[DK * RSL];
  bf pad[raw_pad<DK>()];
  bf V[L * C::RSV];
  float beta[L];   // beta (content-aware: the logit b_x)
  float bw[L];     // beta * w (content-aware: w)
  f32x2 GL[C::NP];
  int flag[NWP];   // per prep wave: some channel's Gamma_L is out of range
  float uv[L];     // content-aware: u_h . v_t, the projected row's value
};


// 16-byte LDS reads of beta, bw and GL rely on these offsets
template <int DK, int TV>
constexpr bool slot_aligned() {
  using S = SlotA<DK, TV>;
  return offsetof(S, beta) % 16 == 0 && offsetof(S, bw) % 16 == 0 && offsetof(S, GL) % 16 == 0 &&
         offsetof(S, flag) % 16 == 0 && offsetof(S, uv) % 16 == 0 && offsetof(S, V) % 16 == 0 &&
         sizeof(S) % 16 == 0 &&
         offsetof(S, V) - offsetof(S, Kp) >= (size_t)raw_bytes<DK>();
}
static_assert(slot_aligned<128, 64>() && slot_aligned<128, 32>() && slot_aligned<64, 32>() &&
                  slot_aligned<128, 16>() && slot_aligned<64, 16>(),
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

// raw loads of one prep lane for one chunk
template <int DK, int TV, bool CONTENT>
using RawT = Raw<Cfg<DK, TV>::TPS, CONTENT ? Cfg<DK, TV>::VLDF : Cfg<DK, TV>::VLD>;

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
  int sk, sa, sth, sv, sb;   // per-token byte strides
};

// GMODE > 0 (gated forward): the decay comes as a bf16 pre-activation.
template <int DK, int TV, int DECAY, int GMODE = 0>
__device__ inline Rsrc make_rsrcs(const FwdParams& p, int b, int h, int v0) {
  const int Tn = p.T, H = p.H, DV = p.DV;
  const size_t bh = (size_t)b * Tn * H + h;
  const size_t rows = (size_t)(Tn - 1) * H + 1;   // token rows up to token T-1 of head h
  Rsrc r;
  r.sk = H * DK * 2;
  r.k = make_rsrc((const bf*)p.k + bh * DK, rows * DK * 2);
  r.q = make_rsrc((const bf*)p.q + bh * DK, rows * DK * 2);
  constexpr int GS = GMODE > 0 ? 2 : 4;   // bytes per decay value
  const char* abase = GMODE > 0 ? (const char*)p.gate_x : (const char*)p.alpha;
  if constexpr (DECAY == 0) {
    r.sa = H * DK * GS;
    r.a = make_rsrc(abase + bh * DK * GS, rows * DK * GS);
    r.th = r.a;
    r.sth = r.sa;
  } else {
    r.sa = H * (DK / 2) * GS;
    r.a = make_rsrc(abase + bh * (DK / 2) * GS, rows * (DK / 2) * GS);
    r.sth = H * (DK / 2) * 4;
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
template <int DK, int TV, int DECAY, bool CONTENT, int PART, int GMODE = 0>
__device__ inline void load_part(RawT<DK, TV, CONTENT>& R, const Rsrc& rs, int c0, int pp, int seg,
                                 int ptid) {
  using C = Cfg<DK, TV>;
  if constexpr (PART == 0 && CONTENT) {   // whole value rows (the resource starts at column 0)
#pragma unroll
    for (int u = 0; u < C::VLDF; ++u) {
      const int idx = ptid + u * NWP * 64;
      const int r = idx / C::VPRF, cc = idx % C::VPRF;
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs.v, r * rs.sv + cc * 16, c0 * rs.sv, 0);
      R.v[u] = uint4{x[0], x[1], x[2], x[3]};
    }
  } else if constexpr (PART == 0) {
#pragma unroll
    for (int u = 0; u < C::VLD; ++u) {
      const int idx0 = ptid + u * NWP * 64;
      const int idx = idx0 < L * C::VPR ? idx0 : 0;
      const int r = idx / C::VPR, cc = idx % C::VPR;
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs.v, r * rs.sv + cc * 16, c0 * rs.sv, 0);
      R.v[u] = uint4{x[0], x[1], x[2], x[3]};
    }
  } else if constexpr (PART == 1 && GMODE > 0) {
    // bf16 pre-activations, kept as raw bits: DIAG the channel pair's two
    // values (.x), ROT2 the block's value (.x, low half) and its angle (.y)
    const int al = seg * C::TPS * rs.sa + (DECAY == 0 ? 4 : 2) * pp;
    const int tl = seg * C::TPS * rs.sth + 4 * pp;
#pragma unroll
    for (int r = 0; r < C::TPS; ++r) {
      if constexpr (DECAY == 0) {
        R.a[r] = f32x2{__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs.a, al, (c0 + r) * rs.sa, 0)), 0.f};
      } else {
        R.a[r] = f32x2{__uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs.a, al, (c0 + r) * rs.sa, 0)),
                       __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs.th, tl, (c0 + r) * rs.sth, 0))};
      }
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

template <int DK, int TV, int DECAY, bool CONTENT, int GMODE = 0>
__device__ inline void load_raw(RawT<DK, TV, CONTENT>& R, const Rsrc& rs, int c0, int pp, int seg,
                                int ptid) {
  load_part<DK, TV, DECAY, CONTENT, 0, GMODE>(R, rs, c0, pp, seg, ptid);
  load_part<DK, TV, DECAY, CONTENT, 1, GMODE>(R, rs, c0, pp, seg, ptid);
  load_part<DK, TV, DECAY, CONTENT, 2, GMODE>(R, rs, c0, pp, seg, ptid);
  load_part<DK, TV, DECAY, CONTENT, 3, GMODE>(R, rs, c0, pp, seg, ptid);
}

// Value of the partner lane across bit d (d in {8, 4, 2, 1}) of a 16-lane row,
// by a DPP move inside the row: row mirror (lane i <-> 15 - i), half-row
// mirror (i <-> 7 - i within each 8), then quad swaps (i ^ 2, i ^ 1).  Each
// pairs the lanes of the two halves of the current 2d-lane group, which is all
// a reduce-scatter needs, with no LDS instruction and no wait on one.
__device__ inline float row_partner(float v, int d) {
  const int x = __float_as_int(v);
  int r;
  if (d == 8) r = __builtin_amdgcn_mov_dpp(x, 0x140, 0xf, 0xf, false);
  else if (d == 4) r = __builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, false);
  else if (d == 2) r = __builtin_amdgcn_mov_dpp(x, 0x4e, 0xf, 0xf, false);
  else r = __builtin_amdgcn_mov_dpp(x, 0xb1, 0xf, 0xf, false);
  return __int_as_float(r);
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
// Gated forward (GMODE > 0): the transitions come as bf16 pre-activations with
// the head's scale ga.  With q/k normalisation (GMODE == 2) k and q stay raw
// here: the norms are folded into beta, beta*w and an output scale.
template <int DK, int TV, int DECAY, bool CONTENT, bool NEXT, bool ROBUST, int GMODE = 0>
__device__ __forceinline__ void prep_chunk(Shared<DK, TV>& sh, const RawT<DK, TV, CONTENT>& R,
                                           RawT<DK, TV, CONTENT>& Rn, const Rsrc& rs, int cn,
                                           int it, int vs, int Tn, int pw, int l, int pl,
                                           int seg, int pp, int ptid, int& any_out,
                                           const float (&uh)[8], int vc0, float ga = 0.f) {
  using C = Cfg<DK, TV>;
  constexpr int PPW = C::PPW, NSEG = C::NSEG, TPS = C::TPS, RSK = C::RSK, RSV = C::RSV,
                VPR = C::VPR;
  SlotA<DK, TV>& A = sh.a[vs % 3];
  bf* Kh = sh.Kh[vs & 1];
  const int c0 = it * L;
  if constexpr (NEXT) load_part<DK, TV, DECAY, CONTENT, 0, GMODE>(Rn, rs, cn, pp, seg, ptid);
  // transitions of this lane's token segment (identity past the end)
  f32x2 ain[TPS];
#pragma unroll
  for (int r = 0; r < TPS; ++r) {
    if constexpr (GMODE == 0) {
      ain[r] = R.a[r];
    } else if constexpr (DECAY == 0) {
      const f32x2 x = bf2_to_f2(__float_as_uint(R.a[r].x));
      ain[r] = f32x2{gate_act(x.x, ga), gate_act(x.y, ga)};
    } else {
      ain[r] = f32x2{gate_act(__uint_as_float(__float_as_uint(R.a[r].x) << 16), ga), R.a[r].y};
    }
  }
  f32x2 d[TPS];
  // Tokens past T act as the identity.  Only the last block of a ragged
  // sequence needs that.  The per-channel decay keeps the form the compiler
  // if-converts (compares and selects on every block), which it schedules 3 %
  // faster on the layer workload; for the 2x2 blocks an empty asm keeps the
  // fix behind a real branch (2 % faster on the rotation workload;
  // interleaved A/B).
  if constexpr (DECAY == 0) {
    if (c0 + L <= Tn) {
#pragma unroll
      for (int r = 0; r < TPS; ++r) d[r] = ain[r];
    } else {
#pragma unroll
      for (int r = 0; r < TPS; ++r) {
        const bool ok = c0 + seg * TPS + r < Tn;
        d[r].x = ok ? ain[r].x : 1.f;
        d[r].y = ok ? ain[r].y : 1.f;
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < TPS; ++r) d[r] = ain[r];
    if (c0 + L > Tn) {
      asm volatile("");
#pragma unroll
      for (int r = 0; r < TPS; ++r) {
        const bool ok = c0 + seg * TPS + r < Tn;
        d[r].x = ok ? ain[r].x : 1.f;
        d[r].y = ok ? ain[r].y : 0.f;
      }
    }
  }
  if constexpr (DECAY == 1) {
#pragma unroll
    for (int r = 0; r < TPS; ++r) {   // (gamma, theta) -> gamma e^{i theta}
      float sn, cs;
      __sincosf(d[r].y, &sn, &cs);
      d[r] = f32x2{d[r].x * cs, d[r].x * sn};
    }
  }
  // Reflection blocks: the map of tokens 1..r is (w_1 c^p1(w_2) c^p2(w_3) ...,
  // p_r) with p_i the parity of reflections among tokens 1..i (c: complex
  // conjugate), so conjugating each w_i by the parity before it turns every
  // product into a plain, commuting complex product.  psg[r]: that parity
  // through token r of the chunk, as a sign bit.  The parity of this pair's
  // earlier segments comes from one ballot of the segment parities (bit
  // pl + PPW j: segment j).
  unsigned psg[TPS];
  unsigned ptot = 0u;   // reflection parity of the whole chunk (bit 0)
  if constexpr (DECAY == 2) {
    unsigned sp = 0u;
#pragma unroll
    for (int r = 0; r < TPS; ++r) sp ^= __float_as_uint(d[r].x);   // sign bit of gamma: reflection
    constexpr unsigned long long REP = [] {
      unsigned long long m = 0ull;
      for (int j = 0; j < NSEG; ++j) m |= 1ull << (j * PPW);
      return m;
    }();
    const unsigned long long bm = __ballot((int)sp < 0) >> pl;
    unsigned par = (unsigned)(__popcll(bm & REP & ((1ull << (seg * PPW)) - 1ull)) & 1) << 31;
    ptot = (unsigned)__popcll(bm & REP) & 1u;
#pragma unroll
    for (int r = 0; r < TPS; ++r) {
      float sn, cs;
      __sincosf(d[r].y, &sn, &cs);
      const float gm = __builtin_fabsf(d[r].x);
      const unsigned sr = __float_as_uint(d[r].x) & 0x80000000u;
      d[r] = f32x2{gm * cs, __uint_as_float(__float_as_uint(gm * sn) ^ par)};
      par ^= sr;
      psg[r] = par;
    }
  }
  // products of commuting factors (reflection blocks: conjugated as above)
  auto mulz = [](f32x2 u, f32x2 v) {
    if constexpr (DECAY == 0) return f32x2{u.x * v.x, u.y * v.y};
    else return cmul(u, v);
  };
  const f32x2 one = {1.f, DECAY == 0 ? 1.f : 0.f};
  if constexpr (NEXT) {
    __builtin_amdgcn_sched_barrier(0);
    load_part<DK, TV, DECAY, CONTENT, 1, GMODE>(Rn, rs, cn, pp, seg, ptid);
  }
  f32x2 run = d[0];
#pragma unroll
  for (int r = 1; r < TPS; ++r) run = mulz(run, d[r]);
  if constexpr (CONTENT) {
    // whole rows: the tile (columns vc0 .. vc0 + TV - 1) goes to LDS, and
    // u_h . v_t is reduced over the VPRF lanes that hold token t's row
#pragma unroll
    for (int u = 0; u < C::VLDF; ++u) {
      const int idx = ptid + u * NWP * 64;
      const int r = idx / C::VPRF, cc = idx % C::VPRF;
      const int tc = cc * 8 - vc0;
      if (tc >= 0 && tc < TV) *(uint4*)(A.V + r * RSV + tc) = R.v[u];
      const uint32_t w4[4] = {R.v[u].x, R.v[u].y, R.v[u].z, R.v[u].w};
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 x = bf2_to_f2(w4[e]);
        dot += uh[2 * e] * x.x + uh[2 * e + 1] * x.y;
      }
#pragma unroll
      for (int off = 1; off < C::VPRF; off <<= 1) dot += __shfl_xor(dot, off);
      if (cc == 0) A.uv[r] = dot;
    }
  } else {
#pragma unroll
  for (int u = 0; u < C::VLD; ++u) {
    const int idx = ptid + u * NWP * 64;
    if (idx < L * VPR) {
      const int r = idx / VPR, cc = idx % VPR;
      *(uint4*)(A.V + r * RSV + cc * 8) = R.v[u];
    }
  }
  }
  // products over the earlier (pre) and later (post) segments of this lane's
  // channel pair, and over the whole chunk (tot): a butterfly over the NSEG
  // segments (lanes PPW apart) with cross-lane swaps, each product taken in
  // token order (the partner block of an upper lane holds earlier segments)
  f32x2 pre = one, post = one, tot = run;
#pragma unroll
  for (int d = 1; d < NSEG; d *= 2) {
    const f32x2 tp = {xor_lanes<PPW>(tot.x, d, l), xor_lanes<PPW>(tot.y, d, l)};
    const bool upper = (seg & d) != 0;
    pre = mulz(pre, upper ? tp : one);
    post = mulz(post, upper ? one : tp);
    tot = mulz(tot, tp);
  }
  if (seg == 0) A.GL[pp] = DECAY == 2 ? with_refl(tot, ptot) : tot;
  {   // chunk-level range check of the split form (gdr_token.h)
    const unsigned long long bad = __ballot(!decay_in_range<DECAY>(tot));
    if constexpr (ROBUST) {
      if (l == 0) A.flag[pw] = bad != 0ull;
    } else {
      any_out |= bad != 0ull;
    }
  }
  if constexpr (NEXT) {
    __builtin_amdgcn_sched_barrier(0);
    load_part<DK, TV, DECAY, CONTENT, 2, GMODE>(Rn, rs, cn, pp, seg, ptid);
  }
  f32x2 ig;   // Gamma_L^{-T} per channel (pair)
  if constexpr (DECAY == 0) {
    ig = f32x2{__builtin_amdgcn_rcpf(tot.x), __builtin_amdgcn_rcpf(tot.y)};
  } else {
    const float nz = __builtin_amdgcn_rcpf(tot.x * tot.x + tot.y * tot.y);
    ig = f32x2{tot.x * nz, tot.y * nz};
  }
  (void)ig;
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
      load_part<DK, TV, DECAY, CONTENT, 3, GMODE>(Rn, rs, cn, pp, seg, ptid);
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
      } else if constexpr (DECAY == 1) {
        kp = cmul(gf, kx);
        qp = cmul(gf, qx);
        kh = cmul(hb, kx);
      } else {   // Gamma_r and Gamma_r^{-T} reflect when the parity through r is odd
        const f32x2 kc = {kx.x, __uint_as_float(__float_as_uint(kx.y) ^ psg[r])};
        const f32x2 qc = {qx.x, __uint_as_float(__float_as_uint(qx.y) ^ psg[r])};
        kp = cmul(gf, kc);
        qp = cmul(gf, qc);
        kh = cmul(hb, kc);
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

// Raw form of chunk c0 .. c0+L-1 for the token path, written by the 4 solve
// waves (lane id ix in 0..255: token ix / 8, channels (ix % 8) * DK / 8 ...):
// the transition as fp32 per channel (ROT2: gamma cos theta, gamma sin theta
// per pair), then the raw keys and queries.  Tokens past T read as zero.
// Gated forward: the transition from its pre-activation (scale ga), and with
// GMODE == 2 queries divided by their norms (sums of squares reduced over the
// 8 lanes that hold a token).
template <int DK, int TV, int DECAY, int GMODE = 0>
__device__ inline void stage_raw(SlotA<DK, TV>& A, const Rsrc& rs, int c0, int ix, float ga = 0.f) {
  constexpr int CPL = DK / 8;   // channels per lane
  constexpr int NP8 = CPL / 8;  // 16-byte pieces of keys (or queries) per lane
  static_assert(NWS * 64 == 8 * L, "one solve lane per (token, channel block)");
  char* raw = (char*)A.Kp;
  float* ra = (float*)raw;
  bf* rk = (bf*)(raw + L * DK * 4);
  bf* rq = rk + L * DK;
  const int t = ix >> 3, c = (ix & 7) * CPL;
  const int tok = c0 + t;
  uint4 kk[NP8], qq[NP8];
#pragma unroll
  for (int u = 0; u < NP8; ++u) {
    const auto xk = __builtin_amdgcn_raw_buffer_load_b128(rs.k, (c + 8 * u) * 2, tok * rs.sk, 0);
    const auto xq = __builtin_amdgcn_raw_buffer_load_b128(rs.q, (c + 8 * u) * 2, tok * rs.sk, 0);
    kk[u] = uint4{xk[0], xk[1], xk[2], xk[3]};
    qq[u] = uint4{xq[0], xq[1], xq[2], xq[3]};
  }
  if constexpr (GMODE == 2) {
    // queries divided by their norms; keys stay raw (their norms are folded
    // into the block's beta and beta*w, which the token path uses too)
    float sq = 0.f;
#pragma unroll
    for (int u = 0; u < NP8; ++u) {
      const uint32_t wq[4] = {qq[u].x, qq[u].y, qq[u].z, qq[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 q2 = __builtin_bit_cast(bf16x2, wq[e]);
        sq = __builtin_amdgcn_fdot2_f32_bf16(q2, q2, sq, false);
      }
    }
#pragma unroll
    for (int d = 4; d >= 1; d >>= 1) sq += row_partner(sq, d);
    const float fq = __builtin_amdgcn_rsqf(sq + 1e-6f);
#pragma unroll
    for (int u = 0; u < NP8; ++u) {
      uint32_t wq[4] = {qq[u].x, qq[u].y, qq[u].z, qq[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 b2 = bf2_to_f2(wq[e]);
        wq[e] = f2_to_bf2(f32x2{b2.x * fq, b2.y * fq});
      }
      qq[u] = uint4{wq[0], wq[1], wq[2], wq[3]};
    }
  }
#pragma unroll
  for (int u = 0; u < NP8; ++u) {
    *(uint4*)(rk + t * DK + c + 8 * u) = kk[u];
    *(uint4*)(rq + t * DK + c + 8 * u) = qq[u];
  }
  if constexpr (DECAY == 0 && GMODE == 0) {
#pragma unroll
    for (int u = 0; u < CPL; u += 4) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs.a, (c + u) * 4, tok * rs.sa, 0);
      *(uint4*)(ra + t * DK + c + u) = uint4{x[0], x[1], x[2], x[3]};
    }
  } else if constexpr (DECAY == 0) {
#pragma unroll
    for (int u = 0; u < CPL; u += 8) {   // 8 bf16 pre-activations -> 8 decays
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs.a, (c + u) * 2, tok * rs.sa, 0);
      f32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 v2 = bf2_to_f2(x[e]);
        (e < 2 ? lo : hi)[2 * (e & 1)] = gate_act(v2.x, ga);
        (e < 2 ? lo : hi)[2 * (e & 1) + 1] = gate_act(v2.y, ga);
      }
      *(f32x4*)(ra + t * DK + c + u) = lo;
      *(f32x4*)(ra + t * DK + c + u + 4) = hi;
    }
  } else {
#pragma unroll
    for (int u = 0; u < CPL / 2; u += 4) {   // pairs c/2 + u .. c/2 + u + 3
      float gm4[4];
      if constexpr (GMODE == 0) {
        const auto xg = __builtin_amdgcn_raw_buffer_load_b128(rs.a, (c / 2 + u) * 4, tok * rs.sa, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) gm4[e] = __uint_as_float(xg[e]);
      } else {
        const auto xg = __builtin_amdgcn_raw_buffer_load_b64(rs.a, (c / 2 + u) * 2, tok * rs.sa, 0);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const f32x2 v2 = bf2_to_f2(xg[e]);
          gm4[2 * e] = gate_act(v2.x, ga);
          gm4[2 * e + 1] = gate_act(v2.y, ga);
        }
      }
      const auto xt = __builtin_amdgcn_raw_buffer_load_b128(rs.th, (c / 2 + u) * 4, tok * rs.sth, 0);
      f32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sn, cs;
        __sincosf(__uint_as_float(xt[e]), &sn, &cs);
        if constexpr (DECAY == 2) {   // reflection bit in the lowest bit of the first value
          const float gm = __builtin_fabsf(gm4[e]);
          const f32x2 m = with_refl(f32x2{gm * cs, gm * sn}, __float_as_uint(gm4[e]) >> 31);
          (e < 2 ? lo : hi)[2 * (e & 1)] = m.x;
          (e < 2 ? lo : hi)[2 * (e & 1) + 1] = m.y;
        } else {
          (e < 2 ? lo : hi)[2 * (e & 1)] = gm4[e] * cs;
          (e < 2 ? lo : hi)[2 * (e & 1) + 1] = gm4[e] * sn;
        }
      }
      *(f32x4*)(ra + t * DK + c + 2 * u) = lo;
      *(f32x4*)(ra + t * DK + c + 2 * u + 4) = hi;
    }
  }
}

// CKPT: the backward's forward recompute, which also stores the state at the
// start of every block (p.ckpt).
template <int DK, int TV, int DECAY, bool CONTENT, int GMODE = 0, bool CKPT = false>
__global__ __launch_bounds__((NWP + NWS + TV / 16 + (CONTENT ? 1 : 0)) * 64) void gdr_fwd_pipe_kernel(
    FwdParams p) {
  static_assert(GMODE == 0 || !CONTENT, "the gated forward has the plain erase");
  static_assert(!CKPT || (GMODE == 0 && !CONTENT), "checkpoints are taken by the plain forward");
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
  // Content-aware erase.  Every gate acts on the key axis, so the value rows of
  // S evolve independently and any fixed combination of them does too (CARVE
  // technical summary, section 2.3 and section 3 item 1): the projected row
  // r = u_h^T S follows the same recurrence with value u_h . v_t, and
  // r_t . q_t = u_h . o_t.  So every value-tile workgroup carries r in one extra
  // consumer wave (the projection wave) and forms the window signal
  // s_c = u_h . m_c = (1/window) sum_t r_t . q_t itself, with no exchange
  // between workgroups.  u_h = B_h^T a_h; sMean holds the carried mean of the
  // window before the call (or zero), which gives the first window's signal;
  // sS holds the signal of the window after the last finished one.
  constexpr int NWC = C::NWC;
  __shared__ __attribute__((aligned(16))) float sU[CONTENT ? DK : 1], sMean[CONTENT ? DK : 1];
  __shared__ float sS[1];
  // Gated forward with q/k normalisation.  Dividing k_t by its norm |k_t|
  // (sqrt of the sum of squares + 1e-6) turns the erase beta_t k^ k^T into
  // (beta_t / |k_t|^2) k k^T and the write beta_t w_t v k^T into
  // (beta_t w_t / |k_t|) v k^T, so a block runs on raw k with those two
  // strengths in place of beta and beta*w, exactly; and o_t = S_t q_t / |q_t|.
  // The solve waves form both norms from raw k and q, and sNq holds 1 / |q_t|
  // of a block (one per prep slot) for the consumer.
  constexpr bool GNORM = GMODE == 2;
  __shared__ __attribute__((aligned(16))) float sNq[GNORM ? 3 : 1][GNORM ? L : 1];
  // content-aware: beta and beta*w of a block, computed by the solve for the
  // consumer (one per prep slot)
  __shared__ __attribute__((aligned(16))) float sBc[CONTENT ? 3 : 1][2][L];
  if constexpr (CONTENT) {
    if (tid < DV) {
      float acc = 0.f;
      for (int r = 0; r < p.ub_rank; ++r)
        acc += p.ub_up[h * p.ub_rank + r] * p.ub_down[((size_t)h * p.ub_rank + r) * DV + tid];
      sU[tid] = acc;
      sMean[tid] = p.m_carry ? p.m_carry[(size_t)(b * H + h) * DV + tid] : 0.f;
    }
    lds_barrier();
  }

  // Each role runs the pipeline twice at most.  Pass 1 (ROBUST = false) is the
  // matrix-core path only; the prep records whether any block of this (b, h)
  // left the split form's range, in which case pass 1's results are invalid
  // and pass 2 (ROBUST = true) recomputes the whole (b, h) with a range check
  // per block and the token path for out-of-range blocks, overwriting every
  // output of pass 1 (same lanes, same addresses, in program order).  Keeping
  // the two apart leaves the hot loop free of data-dependent branches, which
  // otherwise cost it ~10 % through a worse instruction schedule.  Every role
  // keeps its state inside its own branch so none of it is live in another.
  __shared__ __attribute__((aligned(16))) int sRedo[NWP];   // read as one int4
  static_assert(NWP == 4, "sRedo is read as one int4");
  auto redo_needed = [&](int bad) {
    if (wv < NWP && (threadIdx.x & 63) == 0) sRedo[wv] = bad;
    lds_barrier();
    const int4 r4 = *(const int4*)sRedo;
    return __builtin_amdgcn_readfirstlane(r4.x | r4.y | r4.z | r4.w) != 0;
  };
  // restart state shared by all roles before pass 2 (content-aware: the
  // carried mean of the window before the call)
  auto reset_for_pass2 = [&]() {
    if constexpr (CONTENT) {
      if (tid < TV) sMean[tid] = p.m_carry ? p.m_carry[(size_t)(b * H + h) * DV + tid] : 0.f;
    }
    lds_barrier();
  };
  if (wv < NWP) {
    auto prep_role = [&](auto robust_tag) -> int {
      constexpr bool ROBUST = decltype(robust_tag)::value;
      int any_bad = 0;
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
    const Rsrc rs = make_rsrcs<DK, TV, DECAY, GMODE>(p, b, h, CONTENT ? 0 : v0);
    const float ga = GMODE > 0 ? p.gate_a[h] : 0.f;   // gated forward: the head's decay scale
    const int clast = (nchunks - 1) * L;
    // content-aware: u_h over the 8 value channels of this lane's row piece
    float uh[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (CONTENT) {
      const int cc = ptid % C::VPRF;
#pragma unroll
      for (int e = 0; e < 8; ++e) uh[e] = sU[cc * 8 + e];
    }
    auto idle_after = [&](int j) {   // the idle step after a window's last block
      if (CONTENT && j % SPC == SPC - 1 && j + 1 < nchunks) lds_barrier();
    };
    int it = 0;
    if constexpr (C::NT > 12 * 64) {
      static_assert(GMODE == 0, "the gated forward runs the three-register-set prep");
      // 16 waves leave 128 VGPRs per wave: one chunk ahead, two register sets
      RawT<DK, TV, CONTENT> R0, R1;
      load_raw<DK, TV, DECAY, CONTENT>(R0, rs, 0, pp, seg, ptid);
      for (; it + 1 < nchunks; it += 2) {
        prep_chunk<DK, TV, DECAY, CONTENT, true, ROBUST>(sh, R0, R1, rs, (it + 1) * L, it, vstep(it), Tn, pw, l, pl,
                                        seg, pp, ptid, any_bad, uh, v0);
        lds_barrier();
        idle_after(it);
        prep_chunk<DK, TV, DECAY, CONTENT, true, ROBUST>(sh, R1, R0, rs, min((it + 2) * L, clast), it + 1,
                                        vstep(it + 1), Tn, pw, l, pl, seg, pp, ptid, any_bad, uh, v0);
        lds_barrier();
        idle_after(it + 1);
      }
      if (it < nchunks) {   // odd chunk count: the last chunk is in R0
        prep_chunk<DK, TV, DECAY, CONTENT, false, ROBUST>(sh, R0, R1, rs, 0, it, vstep(it), Tn, pw, l, pl, seg, pp,
                                         ptid, any_bad, uh, v0);
        lds_barrier();
        ++it;
      }
    } else {
    RawT<DK, TV, CONTENT> R0, R1, R2;
    load_raw<DK, TV, DECAY, CONTENT, GMODE>(R0, rs, 0, pp, seg, ptid);
    load_raw<DK, TV, DECAY, CONTENT, GMODE>(R1, rs, min(L, clast), pp, seg, ptid);
    for (; it + 2 < nchunks; it += 3) {
      prep_chunk<DK, TV, DECAY, CONTENT, true, ROBUST, GMODE>(sh, R0, R2, rs, (it + 2) * L, it, vstep(it), Tn, pw, l, pl,
                                      seg, pp, ptid, any_bad, uh, v0, ga);
      lds_barrier();
      idle_after(it);
      prep_chunk<DK, TV, DECAY, CONTENT, true, ROBUST, GMODE>(sh, R1, R0, rs, min((it + 3) * L, clast), it + 1,
                                      vstep(it + 1), Tn, pw, l, pl, seg, pp, ptid, any_bad, uh, v0, ga);
      lds_barrier();
      idle_after(it + 1);
      prep_chunk<DK, TV, DECAY, CONTENT, true, ROBUST, GMODE>(sh, R2, R1, rs, min((it + 4) * L, clast), it + 2,
                                      vstep(it + 2), Tn, pw, l, pl, seg, pp, ptid, any_bad, uh, v0, ga);
      lds_barrier();
      idle_after(it + 2);
    }
    // one or two chunks left: they are in R0 and R1
    if (it < nchunks) {
      prep_chunk<DK, TV, DECAY, CONTENT, false, ROBUST, GMODE>(sh, R0, R2, rs, 0, it, vstep(it), Tn, pw, l, pl, seg, pp,
                                       ptid, any_bad, uh, v0, ga);
      lds_barrier();
      idle_after(it);
      ++it;
    }
    if (it < nchunks) {
      prep_chunk<DK, TV, DECAY, CONTENT, false, ROBUST, GMODE>(sh, R1, R2, rs, 0, it, vstep(it), Tn, pw, l, pl, seg, pp,
                                       ptid, any_bad, uh, v0, ga);
      lds_barrier();
      ++it;
    }
    }
    for (int st = vstep(nchunks - 1) + 1; st < nsteps; ++st) lds_barrier();
      return any_bad;
    };
    if (redo_needed(prep_role(std::false_type{}))) {
      reset_for_pass2();
      prep_role(std::true_type{});
    }
  } else if (wv < NWP + NWS) {
    auto solve_role = [&](auto robust_tag) {
      constexpr bool ROBUST = decltype(robust_tag)::value;
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
    if (!GNORM && sw == NWS - 1) {
      nbt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, tb, 0, 0));
      nwt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, tb, 0, 0));
    }
    float s_win = 0.f;   // content-aware: s_c = u_h . m_c of the current window
    const Rsrc rss = make_rsrcs<DK, TV, DECAY, GMODE>(p, b, h, v0);
    const float ga = GMODE > 0 ? p.gate_a[h] : 0.f;
    // Normalised gated: lane ix = 64 sw + l holds token ix / 8 of a block and
    // its key and query channels (ix % 8) * DK / 8 ..., loaded at the end of
    // the step before the block's prep step; at the end of that step the 8
    // lanes of a token reduce the sums of squares, and the first of them
    // stages the block's strengths beta / |k|^2 and beta w / |k| and the
    // output scale 1 / |q|.  (A second register set, two steps ahead, would
    // need the solve loop unrolled by two, which slows the plain launches.)
    constexpr int NPC = GNORM ? DK / 64 : 1;   // 16-byte pieces of k (and of q) per lane
    struct GSet {
      uint4 k[NPC], q[NPC];
      float b, w;
    };
    const int ntk = (sw * 64 + l) >> 3;
    const int nvo = ntk * rss.sk + ((sw * 64 + l) & 7) * (DK / 8) * 2;
    auto gnorm_load = [&](GSet& G, int c) {   // block c (tokens past T read as zero)
      const int so = c * L * rss.sk;
#pragma unroll
      for (int u = 0; u < NPC; ++u) {
        const auto xk = __builtin_amdgcn_raw_buffer_load_b128(rss.k, nvo + 16 * u, so, 0);
        const auto xq = __builtin_amdgcn_raw_buffer_load_b128(rss.q, nvo + 16 * u, so, 0);
        G.k[u] = uint4{xk[0], xk[1], xk[2], xk[3]};
        G.q[u] = uint4{xq[0], xq[1], xq[2], xq[3]};
      }
      G.b = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, ntk * H * 4, c * L * H * 4, 0));
      G.w = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, ntk * H * 4, c * L * H * 4, 0));
    };
    auto gnorm_stage = [&](const GSet& G, int it) {
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int u = 0; u < NPC; ++u) {
        const uint32_t wk[4] = {G.k[u].x, G.k[u].y, G.k[u].z, G.k[u].w};
        const uint32_t wq[4] = {G.q[u].x, G.q[u].y, G.q[u].z, G.q[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 k2 = __builtin_bit_cast(bf16x2, wk[e]), q2 = __builtin_bit_cast(bf16x2, wq[e]);
          sk = __builtin_amdgcn_fdot2_f32_bf16(k2, k2, sk, false);
          sq = __builtin_amdgcn_fdot2_f32_bf16(q2, q2, sq, false);
        }
      }
#pragma unroll
      for (int d = 4; d >= 1; d >>= 1) {   // all 8 lanes of the token end with the sums
        sk += row_partner(sk, d);
        sq += row_partner(sq, d);
      }
      if ((l & 7) == 0) {
        const float k2 = sk + 1e-6f;
        sh.a[it % 3].beta[ntk] = G.b * __builtin_amdgcn_rcpf(k2);
        sh.a[it % 3].bw[ntk] = G.b * G.w * __builtin_amdgcn_rsqf(k2);
        sNq[it % 3][ntk] = __builtin_amdgcn_rsqf(sq + 1e-6f);
      }
    };
    GSet G;   // normalised gated: block it during step it
    if constexpr (GNORM) gnorm_load(G, 0);
    for (int it = 0; it < nsteps; ++it) {
      const int jp = CONTENT ? block_at(it) : it;
      // (normalised gated: the block's strengths are staged at the end of the step)
      if (!GNORM && sw == NWS - 1 && (CONTENT ? (jp >= 0 && jp < nchunks) : (it < nchunks))) {
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
          if (j == 0) {   // first window: u_h . (carried mean), fixed-order reduction
            float acc = 0.f;
            for (int vv = l; vv < DV; vv += 64) acc += sU[vv] * sMean[vv];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            s_win = acc;
          } else if (j % SPC == 0) {   // later windows: formed by the projection wave
            s_win = sS[0];
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
        // some channel leaves the split form's range: the consumer runs this
        // chunk token by token from raw inputs staged below (the flag is read
        // now and used after the Gram and inverse work, which then is unused)
        const int4 rflag = ROBUST ? *(const int4*)A.flag : int4{0, 0, 0, 0};
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
        if (ROBUST && __builtin_amdgcn_readfirstlane(rflag.x | rflag.y | rflag.z | rflag.w) != 0) {
          // the other solve waves may still be reading K+ / Q+ of this slot for
          // their Gram tiles; those results are discarded for this chunk
          stage_raw<DK, TV, DECAY, GMODE>(sh.a[vj % 3], rss, j * L, sw * 64 + l, ga);
        }
      }
      if constexpr (GNORM) {   // off the start of the solve's chain
        if (it < nchunks) gnorm_stage(G, it);
        if (it + 1 < nchunks) gnorm_load(G, it + 1);
      }
      lds_barrier();
    }
    };
    solve_role(std::false_type{});
    if (redo_needed(0)) {
      reset_for_pass2();
      solve_role(std::true_type{});
    }
  } else {
    // ============================================================ consumer
    // cw < NWC: value rows v0 + 16 cw + n of S.  Content-aware, cw == NWC is the
    // projection wave: row 0 of its tile is r = u_h^T S with value u_h . v_t,
    // rows 1..15 stay zero; its outputs are not stored, they form the signal.
    const int cw = wv - NWP - NWS;
    f32x4 Sacc[NCT];
    float wmean[4] = {0.f, 0.f, 0.f, 0.f};   // content-aware: last finished window's mean
    auto consumer_role = [&](auto robust_tag, auto xw_tag) {
      constexpr bool ROBUST = decltype(robust_tag)::value;
      constexpr bool XW = decltype(xw_tag)::value;
      if constexpr (CONTENT) __builtin_amdgcn_s_setprio(2);
      const size_t sbh = (size_t)(b * H + h) * DV;
      if constexpr (XW) {
        // r = u_h^T S0: rows n, n + 16, ... summed per lane, then over n
        f32x4 acc[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p.S0) {
          for (int i = n; i < DV; i += 16) {
            const float ui = sU[i];
            const float* row = p.S0 + (sbh + i) * DK + 4 * g;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) acc[ct] += ui * *(const f32x4*)(row + 16 * ct);
          }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float v = acc[ct][jj];
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off);
            Sacc[ct][jj] = n == 0 ? v : 0.f;
          }
        }
      } else {
        const size_t srow = (sbh + v0 + 16 * cw + n) * DK;
        if (p.S0) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) Sacc[ct] = *(const f32x4*)(p.S0 + srow + 16 * ct + 4 * g);
        } else {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) Sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      // drain the state load here, so that inside the loop only the loop's own
      // output stores are outstanding and no wait on them is needed
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      // o through a buffer resource over this wave's 16 value channels of (b, h):
      // stores past token T-1 fall outside the resource and are dropped.
      const size_t obh = (size_t)b * Tn * H + h;
      const size_t orows = (size_t)(Tn - 1) * H + 1;
      const int ocol = XW ? 0 : v0 + 16 * cw;
      const rsrc_t ro = make_rsrc((bf*)p.o + obh * DV + ocol, orows * DV * 2 - (size_t)ocol * 2);
      const int so = H * DV * 2;                     // bytes per token row
      const int olane = n * so + 8 * g;              // token n, value channels 4g..4g+3
      // value of this lane's row n at token r of a chunk
      auto vat = [&](const SlotA<DK, TV>& A, int r) {
        if constexpr (XW) return n == 0 ? A.uv[r] : 0.f;
        else return (float)A.V[r * RSV + 16 * cw + n];
      };
      float colsum[4] = {0.f, 0.f, 0.f, 0.f};   // content-aware: window sums
      int token_next = 0;   // range flag of the slot consumed at the next step
      // One consumer step; TOKEN selects the token path (gdr_token.h) for a
      // chunk whose decay leaves the split form's range.
      auto step = [&](int it, auto token_tag) {
        constexpr bool TOKEN = decltype(token_tag)::value;
        const int vi = it - 2;
        const int i = CONTENT ? (vi >= 0 ? block_at(vi) : -1) : vi;
        if (CONTENT ? (i >= 0 && i < nchunks) : (i >= 0)) {
          const SlotA<DK, TV>& A = sh.a[vi % 3];
          const SlotS& S = sh.s[vi & 1];
          const int c0 = i * L;
          if constexpr (CKPT) {   // the state at the start of block i, for the backward
            float* dst = p.ckpt + (((size_t)(b * H + h) * nchunks + i) * DV + v0 + 16 * cw + n) * DK + 4 * g;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) *(f32x4*)(dst + 16 * ct) = Sacc[ct];
          }
          if constexpr (TOKEN) {
            // raw transition, keys and queries staged by the solve; o_t[n] is
            // stored as one bf16 by the lanes with g == 0
            const char* raw = (const char*)A.Kp;
            const float* bt = CONTENT ? sBc[vi % 3][0] : A.beta;
            const float* bwp = CONTENT ? sBc[vi % 3][1] : A.bw;
            float fsum = 0.f;
            // full unroll where it measured no slower on the ordinary inputs
            token_steps<DK, DECAY, DECAY != 0 || CONTENT, bf>(
                Sacc, (const float*)raw, (const bf*)(raw + L * DK * 4),
                (const bf*)(raw + L * DK * 6), DK, [&](int t) { return vat(A, t); }, bt, bwp,
                min(L, Tn - c0), [&](int t, float ov) {
                  if (!XW && g == 0) {
                    const bf ob = (bf)ov;
                    __builtin_amdgcn_raw_buffer_store_b16(*(const unsigned short*)&ob, ro, 2 * n,
                                                          (c0 + t) * so, 0);
                  }
                  fsum += ov;
                });
            if constexpr (CONTENT) {
              if constexpr (XW) {
                colsum[0] += (n == 0 && g == 0) ? fsum : 0.f;
              } else {
                // value channel 4g + jj is kept by a lane of group g
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                  const float x = __shfl(fsum, 4 * g + jj);
                  colsum[jj] += n == 0 ? x : 0.f;
                }
              }
            }
          } else {
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
                        Rt[t][jj] = bw4[jj] * vat(A, r) - bt4[jj] * P[jj];
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
                    if constexpr (GNORM) {   // o_t = (S_t q_t) / |q_t|: tokens n and 16 + n
                      O0 *= sNq[vi % 3][n];
                      O1 *= sNq[vi % 3][16 + n];
                    }
                    const bf16x4 ox0 = {(bf)O0[0], (bf)O0[1], (bf)O0[2], (bf)O0[3]};
                    const bf16x4 ox1 = {(bf)O1[0], (bf)O1[1], (bf)O1[2], (bf)O1[3]};
                    if constexpr (CONTENT) {
                      // window sums of the fp32 outputs (tokens past T contribute zero);
                      // the projection wave keeps value column 0 only: r_t . q_t
                      if constexpr (XW) {
                        colsum[0] += g == 0 ? O0[0] + O1[0] : 0.f;
                      } else {
          #pragma unroll
                        for (int jj = 0; jj < 4; ++jj) colsum[jj] += O0[jj] + O1[jj];
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
                        } else if constexpr (DECAY == 1) {
                          Sacc[ct][jj] = z.x * x0 + z.y * x1;
                          Sacc[ct][jj + 1] = -z.y * x0 + z.x * x1;
                        } else {
                          // a state row times Gamma_L: conj(w) y, or for a
                          // reflection (symmetric block) w conj(y)
                          const float y1 = -z.y * x0 + z.x * x1;
                          Sacc[ct][jj] = z.x * x0 + z.y * x1;
                          Sacc[ct][jj + 1] = __uint_as_float(__float_as_uint(y1) ^ (refl_bit(z) << 31));
                        }
                      }
                    }
            if constexpr (!XW) {   // o stores last, off the chain to the state update
              typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
              __builtin_amdgcn_raw_buffer_store_b64(*(const u32x2*)&ox0, ro, olane, c0 * so, 0);
              __builtin_amdgcn_raw_buffer_store_b64(*(const u32x2*)&ox1, ro, olane, (c0 + 16) * so, 0);
            }
          }
          if constexpr (CONTENT) {
            if (i % SPC == SPC - 1) {   // a window's last block
              const float inv = 1.f / (float)(SPC * L);
              if constexpr (XW) {
                // its signal, for the solve of the next window's first block
                float sum = colsum[0];
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off);
                sum += __shfl_xor(sum, 16);
                sum += __shfl_xor(sum, 32);
                if (l == 0) sS[0] = sum * inv;
                colsum[0] = 0.f;
              } else {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                  float sum = colsum[jj];
#pragma unroll
                  for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off);
                  wmean[jj] = sum * inv;
                  colsum[jj] = 0.f;
                }
              }
            }
          }
        }
        // the slot of virtual step it - 1 (consumed next step) was completed by
        // the prep before the last barrier; reading its flag now keeps the LDS
        // latency off the start of the next step's chain
        if (ROBUST && it >= 1) {
          const int4 f = *(const int4*)sh.a[(it - 1) % 3].flag;
          token_next = __builtin_amdgcn_readfirstlane(f.x | f.y | f.z | f.w);
        }
        lds_barrier();
      };
      if constexpr (!ROBUST) {
        for (int it = 0; it < nsteps; ++it) step(it, std::false_type{});
      } else {
        // the flag read in step it is that of the chunk consumed in step it + 1
        int it = 0;
        while (it < nsteps) {
          for (; it < nsteps && token_next == 0; ++it) step(it, std::false_type{});
          if (it < nsteps) {
            step(it, std::true_type{});
            ++it;
          }
        }
      }
    };
    if (CONTENT && cw == NWC) {
      consumer_role(std::false_type{}, std::true_type{});
      if (redo_needed(0)) {
        reset_for_pass2();
        consumer_role(std::true_type{}, std::true_type{});
      }
    } else {
      consumer_role(std::false_type{}, std::false_type{});
      if (redo_needed(0)) {
        reset_for_pass2();
        consumer_role(std::true_type{}, std::false_type{});
      }
      if (p.S_out) {
        const size_t srow = ((size_t)(b * H + h) * DV + v0 + 16 * cw + n) * DK;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) *(f32x4*)(p.S_out + srow + 16 * ct + 4 * g) = Sacc[ct];
      }
      if constexpr (CONTENT) {   // the last window's mean (T is a multiple of the window)
        if (p.m_carry && n == 0) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            p.m_carry[(size_t)(b * H + h) * DV + v0 + 16 * cw + 4 * g + jj] = wmean[jj];
        }
      }
    }
  }
}

template <int DK, int TV, int DECAY, bool CONTENT = false, int GMODE = 0, bool CKPT = false>
hipError_t launch(const FwdParams& p0, hipStream_t s) {
  FwdParams p = p0;
  p.n_vt = p.DV / TV;
  p.n_units = p.B * p.H;
  const int groups = (p.n_units + 7) / 8;
  // content-aware: one more wave carries the projected row u_h^T S
  hipLaunchKernelGGL((gdr_fwd_pipe_kernel<DK, TV, DECAY, CONTENT, GMODE, CKPT>), dim3(groups * 8 * p.n_vt),
                     dim3(Cfg<DK, TV>::NT + (CONTENT ? 64 : 0)), 0, s, p);
  return hipGetLastError();
}

}  // namespace pipe

namespace {
// gated forward (decay from its pre-activation; gmode 2 also normalises q, k)
template <int DK, int TV>
hipError_t launch_gated(const FwdParams& p, hipStream_t s) {
  const bool rot = p.decay != 0;
  if (p.gmode == 2) return rot ? pipe::launch<DK, TV, 1, false, 2>(p, s) : pipe::launch<DK, TV, 0, false, 2>(p, s);
  return rot ? pipe::launch<DK, TV, 1, false, 1>(p, s) : pipe::launch<DK, TV, 0, false, 1>(p, s);
}

hipError_t launch_fwd_gated(const FwdParams& p, hipStream_t s) {
  if (p.DK == 128) {
    if ((long)p.B * p.H * 2 >= 192) return launch_gated<128, 64>(p, s);
    return launch_gated<128, 32>(p, s);
  }
  if (p.DK == 64) return launch_gated<64, 32>(p, s);
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_fwd_pipe(const FwdParams& p, hipStream_t s) {
  const bool rot = p.decay != 0;
  // reflection blocks run only in the plain launch
  if (p.decay == 2 && (p.beta_logit != nullptr || p.gmode != 0 || p.ckpt != nullptr)) return hipErrorInvalidValue;
  if (p.beta_logit != nullptr) {
    // content-aware: 16-channel value tiles, each workgroup with its own
    // projection wave (few heads, long sequences: spread over more CUs)
    if (p.DK == 128) return rot ? pipe::launch<128, 16, 1, true>(p, s) : pipe::launch<128, 16, 0, true>(p, s);
    return rot ? pipe::launch<64, 16, 1, true>(p, s) : pipe::launch<64, 16, 0, true>(p, s);
  }
  if (p.gmode != 0) return launch_fwd_gated(p, s);
  if (p.ckpt != nullptr) {   // the backward's forward recompute (tiles as in the plain launch)
    if (p.DK == 128) {
      if ((long)p.B * p.H * 2 >= 192) {
        return rot ? pipe::launch<128, 64, 1, false, 0, true>(p, s) : pipe::launch<128, 64, 0, false, 0, true>(p, s);
      }
      return rot ? pipe::launch<128, 32, 1, false, 0, true>(p, s) : pipe::launch<128, 32, 0, false, 0, true>(p, s);
    }
    if (p.DK == 64) return rot ? pipe::launch<64, 32, 1, false, 0, true>(p, s) : pipe::launch<64, 32, 0, false, 0, true>(p, s);
    return hipErrorInvalidValue;
  }
  if (p.decay == 2) {   // rotation and reflection blocks
    if (p.DK == 128) {
      if ((long)p.B * p.H * 2 >= 192) return pipe::launch<128, 64, 2>(p, s);
      return pipe::launch<128, 32, 2>(p, s);
    }
    if (p.DK == 64) return pipe::launch<64, 32, 2>(p, s);
    return hipErrorInvalidValue;
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
