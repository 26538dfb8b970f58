// gdr_bwd.hip -- backward of the chunked gated delta rule (plain erase), gfx950.
//
// The forward (CARVE technical summary, sections 1 and 2.3; SFDA technical
// summary, core architecture) is, per head and token,
//     S_t = S_{t-1} D_t + beta_t (w_t v_t - S_{t-1} D_t k_t) k_t^T,  o_t = S_t q_t.
// For a 32-token block with start state S and cumulative transitions
// P_r = D_1 ... D_r, with Kp_r = P_r k_r, Qp_r = P_r q_r, Kh_r = P_r^{-T} k_r,
// the deltas Dl (one row per token) solve (I + Diag(beta) N) Dl = Diag(beta)
// (Diag(w) V - Kp S^T) with N = strict_lower(Kp Kh^T); then
// O = Qp S^T + M Dl (M = lower(Qp Kh^T)) and S_end = (S + Dl^T Kh) P_L.
// The backward runs the adjoint of these expressions block by block, last
// block first, carrying G = dL/dS_end:
//     dY = G P_L^T,  dDl = M^T dO + Kh dY^T,  dR = T^T dDl  (T = (I + Diag(beta) N)^{-1}),
//     dA = -dR Dl^T,  dM = lower(dO Dl^T),  dN = strict_lower(Diag(beta) dA),
//     dQp = dO S + dM Kh,  dKp = dN Kh - Diag(beta) dR S,
//     dKh = Dl dY + dM^T Qp + dN^T Kp,
//     dS = dY + dO^T Qp - (Diag(beta) dR)^T Kp   (the G of the previous block),
// and the gradients of q, k, the decay, beta, w and v follow elementwise.
//
// One workgroup (4 waves) per (b, h, 32-channel value tile).  Every product
// runs on the matrix cores with fp32 operands (v_mfma_f32_16x16x4_f32) from
// LDS; G stays in accumulator registers across blocks.  Sums over value
// channels (dq, dk, the decay's log-gradient, dbeta, dw) are written per value
// tile to a partial-sum area and added by bwd_reduce_kernel, which also turns
// the per-token log-gradients into decay gradients by a reverse prefix sum over
// each block.  The state at the start of every block comes from the forward
// recompute (checkpoints).
//
// Range: like the forward's split form, the block form divides by the running
// decay, so it is exact only while each channel's product over a block stays
// at or above e^-40.  bwd_kernel flags every (b, h, value tile) with a block
// outside that range (strong forgetting: decays near or at zero), and
// bwd_token_kernel then redoes the flagged ones token by token in fp32 with no
// division, overwriting every output the block form wrote for them.
#include <hip/hip_runtime.h>

#include "gdr_kernels.h"
#include "gdr_mfma.h"
#include "gdr_token.h"

namespace gdr {
namespace bwd {

constexpr int L = kBwdBlock;   // tokens per block
constexpr int TV = kBwdTile;   // value channels per workgroup
constexpr int NT = 256;        // 4 waves

using F = Op<float>;

template <int DK>
struct Smem {
  static constexpr int PK = DK + 4, PV = TV + 4, PL = L + 4;
  float Kp[L * PK], Qp[L * PK], Kh[L * PK], Gam[L * PK];
  float S[TV * PK], DY[TV * PK];
  float V[L * PV], DO[L * PV], In[L * PV], Dl[L * PV], DDl[L * PV], DR[L * PV], Din[L * PV];
  float N[L * PL], M[L * PL], T[L * PL], DA[L * PL], DM[L * PL];
  float beta[L], w[L];
  float gl[DK];       // DIAG: P_L per channel; ROT2: (re, im) of P_L per pair
  float dl_end[DK];   // block-end term of the decay's log-gradient
  float red[6][L];    // per-token row sums from the waves (dw, dbeta)
};

__device__ inline float bf2f(const __bf16* p, size_t i) { return (float)p[i]; }

// acc += A B over K, 16x16 output tile at rows r0, columns c0, with
// A(r, k) = a[r * ARS + k * ACS] and B(k, c) = b[k * BRS + c * BCS].  fp32
// operands: bf16 ones (one 16x16x32 product per step) measured 16 % faster on
// the layer shape but raise the gradients' error from ~1e-7 to ~4e-3 where the
// block start state is exact.
//
// Operand slot s of a lane in group g (lane = 16 g + n) holds contraction index
// k0 + 4g + (s & 3) + 16 (s >> 2); any bijection works if both operands use it.
// This one puts the lanes of groups g and g + 1, which a 4-byte LDS read serves
// in the same cycle, on rows 4 apart: with every row stride here 4 mod 32
// floats that is 16 banks apart, so the strided (transposed) operand reads are
// free of bank conflicts (rows 8 apart, as in the plain order, share banks).
// An operand contiguous along k is read as two 16-byte pieces, at 4g and 16 + 4g.
template <int ARS, int ACS, int BRS, int BCS, int K>
__device__ inline void mm(f32x4& acc, const float* a, int r0, const float* b, int c0) {
  static_assert(ACS == 1 || ACS % 32 == 4, "strided A rows must be 4 mod 32 floats apart");
  static_assert(BRS == 1 || BRS % 32 == 4, "strided B rows must be 4 mod 32 floats apart");
  const int l = lane_id(), n = l & 15, g = l >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    f32x8 fa, fb;
    if constexpr (ACS == 1) {
      const float* p = a + (r0 + n) * ARS + k0 + 4 * g;
      fa = F::join(*(const f32x4*)p, *(const f32x4*)(p + 16));
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) fa[s] = a[(r0 + n) * ARS + (k0 + 4 * g + (s & 3) + 16 * (s >> 2)) * ACS];
    }
    if constexpr (BRS == 1) {
      const float* p = b + (c0 + n) * BCS + k0 + 4 * g;
      fb = F::join(*(const f32x4*)p, *(const f32x4*)(p + 16));
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) fb[s] = b[(k0 + 4 * g + (s & 3) + 16 * (s >> 2)) * BRS + (c0 + n) * BCS];
    }
    F::mma(acc, fa, fb);
  }
}

// Sum over the 16 lanes that share g (columns n of one accumulator row).
__device__ inline float sum16(float x) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// Unpack 8 bf16 (one 16-byte piece) to fp32 in LDS.
__device__ inline void put8(float* dst, uint4 u, bool ok) {
  const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dst[2 * e] = ok ? __uint_as_float(wds[e] << 16) : 0.f;
    dst[2 * e + 1] = ok ? __uint_as_float(wds[e] & 0xffff0000u) : 0.f;
  }
}

// Raw inputs of one block, held in registers between their global loads and
// their LDS stores, so that the loads of block c - 1 run under the products of
// block c.
template <int DK, int DECAY>
struct BlockRaw {
  static constexpr int SP = TV * DK / 4 / NT;                      // state tile, 16-byte pieces
  static constexpr int KP = L * DK / 8 / NT;                       // keys, queries
  static constexpr int AP = DECAY == 0 ? L * DK / 4 / NT           // DIAG alpha
                                       : (L * DK / 8 + NT - 1) / NT;   // ROT2 gamma, theta
  float bt, wt;
  uint4 uv, ug;
  f32x4 s[SP];
  uint4 kx[KP], qx[KP];
  f32x4 ax[AP], tx[DECAY == 0 ? 1 : AP];
};

// Issues every global load of block c (16-byte pieces); rows at or past T
// repeat the last token (masked when stored).
template <int DK, int DECAY>
__device__ inline void load_block(BlockRaw<DK, DECAY>& R, const BwdParams& p, int unit, size_t bh,
                                  int c, int t0, int nt, int nc, int v0, int tid) {
  using RW = BlockRaw<DK, DECAY>;
  const int H = p.H, DV = p.DV;
  if (tid < L) {
    const size_t row = bh + (size_t)(t0 + min(tid, nt - 1)) * H;
    R.bt = p.beta[row];
    R.wt = p.w[row];
  }
  // v and grad_o tiles: L rows x TV bf16 = 4 pieces of 8 per row
  static_assert(L * TV / 8 <= NT, "one piece of v and of grad_o per thread");
  if (tid < L * TV / 8) {
    const int r = tid / (TV / 8), i8 = tid % (TV / 8);
    const size_t src = (bh + (size_t)(t0 + min(r, nt - 1)) * H) * DV + v0 + 8 * i8;
    R.uv = *(const uint4*)((const __bf16*)p.v + src);
    R.ug = *(const uint4*)((const __bf16*)p.grad_o + src);
  }
  {   // block-start state tile: TV rows x DK fp32
    const float* ck = p.ckpt + ((size_t)unit * nc + c) * DV * DK;   // unit = b * H + h
#pragma unroll
    for (int u = 0; u < RW::SP; ++u) {
      const int e = tid + u * NT, i = e / (DK / 4), j4 = e % (DK / 4);
      R.s[u] = *(const f32x4*)(ck + (size_t)(v0 + i) * DK + 4 * j4);
    }
  }
#pragma unroll
  for (int u = 0; u < RW::KP; ++u) {   // keys and queries: L rows x DK bf16
    const int e = tid + u * NT, r = e / (DK / 8), j8 = e % (DK / 8);
    const size_t src = (bh + (size_t)(t0 + min(r, nt - 1)) * H) * DK + 8 * j8;
    R.kx[u] = *(const uint4*)((const __bf16*)p.k + src);
    R.qx[u] = *(const uint4*)((const __bf16*)p.q + src);
  }
  if constexpr (DECAY == 0) {   // alpha: L x DK
#pragma unroll
    for (int u = 0; u < RW::AP; ++u) {
      const int e = tid + u * NT, r = e / (DK / 4), j4 = e % (DK / 4);
      R.ax[u] = *(const f32x4*)(p.alpha + (bh + (size_t)(t0 + min(r, nt - 1)) * H) * DK + 4 * j4);
    }
  } else {   // gamma and theta: L x DK/2 each
    constexpr int HP = DK / 2;
#pragma unroll
    for (int u = 0; u < RW::AP; ++u) {
      const int e = min(tid + u * NT, L * HP / 4 - 1), r = e / (HP / 4), j4 = e % (HP / 4);
      const size_t src = (bh + (size_t)(t0 + min(r, nt - 1)) * H) * HP + 4 * j4;
      R.ax[u] = *(const f32x4*)(p.alpha + src);
      R.tx[u] = *(const f32x4*)(p.theta + src);
    }
  }
}

// Stores block raw inputs into LDS: k into Kp, q into Qp, the transition into
// Gam (DIAG alpha; ROT2 gamma at even, theta at odd positions); tokens at or
// past T as zero (and as the identity transition).
template <int DK, int DECAY>
__device__ inline void store_block(Smem<DK>& sm, const BwdParams& p, const BlockRaw<DK, DECAY>& R,
                                   int nt, int tid) {
  using RW = BlockRaw<DK, DECAY>;
  constexpr int PK = Smem<DK>::PK, PV = Smem<DK>::PV;
  if (tid < L) {
    const bool ok = tid < nt;
    sm.beta[tid] = ok ? R.bt : 0.f;
    sm.w[tid] = ok ? R.wt : 0.f;
  }
  if (tid < L * TV / 8) {
    const int r = tid / (TV / 8), i8 = tid % (TV / 8);
    const bool ok = r < nt;
    put8(sm.V + r * PV + 8 * i8, R.uv, ok);
    put8(sm.DO + r * PV + 8 * i8, R.ug, ok);
  }
#pragma unroll
  for (int u = 0; u < RW::SP; ++u) {
    const int e = tid + u * NT, i = e / (DK / 4), j4 = e % (DK / 4);
    *(f32x4*)(sm.S + i * PK + 4 * j4) = R.s[u];
  }
#pragma unroll
  for (int u = 0; u < RW::KP; ++u) {
    const int e = tid + u * NT, r = e / (DK / 8), j8 = e % (DK / 8);
    put8(sm.Kp + r * PK + 8 * j8, R.kx[u], r < nt);
    put8(sm.Qp + r * PK + 8 * j8, R.qx[u], r < nt);
  }
  if constexpr (DECAY == 0) {
#pragma unroll
    for (int u = 0; u < RW::AP; ++u) {
      const int e = tid + u * NT, r = e / (DK / 4), j4 = e % (DK / 4);
      const bool ok = r < nt;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) sm.Gam[r * PK + 4 * j4 + q4] = ok ? R.ax[u][q4] : 1.f;
    }
  } else {
    constexpr int HP = DK / 2;
#pragma unroll
    for (int u = 0; u < RW::AP; ++u) {
      const int e = tid + u * NT;
      if (e < L * HP / 4) {
        const int r = e / (HP / 4), j4 = e % (HP / 4);
        const bool ok = r < nt;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          sm.Gam[r * PK + 2 * (4 * j4 + q4)] = ok ? R.ax[u][q4] : 1.f;
          sm.Gam[r * PK + 2 * (4 * j4 + q4) + 1] = ok ? R.tx[u][q4] : 0.f;
        }
      }
    }
  }
}

template <int DK, int DECAY>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
  using Sm = Smem<DK>;
  constexpr int PK = Sm::PK, PV = Sm::PV, PL = Sm::PL;
  constexpr int NCT = DK / 16, CPW = NCT / 4;   // column tiles of a DK-wide matrix per wave
  __shared__ __attribute__((aligned(16))) Sm sm;
  const int tid = threadIdx.x, l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = l & 15, g = l >> 4;
  const int H = p.H, Tn = p.T, DV = p.DV;
  const int vt = blockIdx.x % p.n_vt, unit = blockIdx.x / p.n_vt;
  const int b = unit / H, h = unit % H;
  const int v0 = vt * TV;
  const int nc = (Tn + L - 1) / L;
  const size_t bh = (size_t)b * Tn * H + h;   // token-head row of token t: bh + t * H
  const size_t BTH = (size_t)p.B * Tn * H;
  const __bf16* q = (const __bf16*)p.q;
  const __bf16* k = (const __bf16*)p.k;
  const __bf16* v = (const __bf16*)p.v;
  const __bf16* dO = (const __bf16*)p.grad_o;
  float* Pq = p.part;
  float* Pk = Pq + (size_t)p.n_vt * BTH * DK;
  float* Pl = Pk + (size_t)p.n_vt * BTH * DK;
  float* Pb = Pl + (size_t)p.n_vt * BTH * DK;
  float* Pw = Pb + (size_t)p.n_vt * BTH;
  const int ti2 = wv >> 1, tj2 = wv & 1;   // tile of a 32x32 matrix owned by this wave

  // G = dL/dS at the end of the current block: rows v0 + 16 ti + 4g + j,
  // columns 16 (wv * CPW + c) + n
  f32x4 G[2][CPW];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = v0 + 16 * ti + 4 * g + j, col = 16 * (wv * CPW + c) + n;
        G[ti][c][j] = p.grad_S ? p.grad_S[((size_t)(b * H + h) * DV + row) * DK + col] : 0.f;
      }

  bool bad = false;   // some block's decay product left the block form's range
  BlockRaw<DK, DECAY> raw;
  {
    const int t0 = (nc - 1) * L;
    load_block<DK, DECAY>(raw, p, unit, bh, nc - 1, t0, Tn - t0, nc, v0, tid);
  }
  for (int c = nc - 1; c >= 0; --c) {
    const int t0 = c * L, nt = min(L, Tn - t0);
    // ---------------------------------------------------------------- loads
    // this block's raw inputs (loaded during the previous block) into LDS,
    // then the loads of the next block (c - 1, a full block) are issued
    store_block<DK, DECAY>(sm, p, raw, nt, tid);
    lds_barrier();
    if (c > 0) load_block<DK, DECAY>(raw, p, unit, bh, c - 1, t0 - L, L, nc, v0, tid);
    // cumulative transitions and the decayed key/query forms, in place: every
    // thread takes one token segment of one channel (ROT2: channel pair), and
    // the products of the earlier segments come from a scan over the lanes
    // that hold the same channel (shuffles inside the wave)
    {
      constexpr int NCH = DECAY == 0 ? DK : DK / 2;
      constexpr int NSEG = NT / NCH, CW = 64 / NSEG, TPS = L / NSEG;
      static_assert(NSEG >= 2 && CW * NSEG == 64 && TPS * NSEG == L, "prefix split");
      const int seg = l / CW, j = wv * CW + l % CW, r0 = seg * TPS;
      if constexpr (DECAY == 0) {
        float a[TPS];
        float inc = 1.f;
#pragma unroll
        for (int r = 0; r < TPS; ++r) {
          a[r] = sm.Gam[(r0 + r) * PK + j];
          inc *= a[r];
        }
#pragma unroll
        for (int d = 1; d < NSEG; d *= 2) {
          const float up = __shfl_up(inc, CW * d);
          if (seg >= d) inc *= up;
        }
        const float ex = __shfl_up(inc, CW);
        float gam = seg > 0 ? ex : 1.f;
#pragma unroll
        for (int r = 0; r < TPS; ++r) {
          const int rr = r0 + r;
          gam *= a[r];
          const float kk = sm.Kp[rr * PK + j], qq = sm.Qp[rr * PK + j];
          sm.Gam[rr * PK + j] = gam;
          sm.Kp[rr * PK + j] = gam * kk;
          sm.Qp[rr * PK + j] = gam * qq;
          sm.Kh[rr * PK + j] = kk * __builtin_amdgcn_rcpf(gam);
        }
        if (seg == NSEG - 1) {
          sm.gl[j] = gam;
          bad |= !(gam >= kMinChunkDecay);   // also true for NaN
        }
      } else {
        const int pr = j;
        float dr[TPS], di[TPS];
        float ir = 1.f, ii = 0.f;
#pragma unroll
        for (int r = 0; r < TPS; ++r) {
          const float gm = sm.Gam[(r0 + r) * PK + 2 * pr], th = sm.Gam[(r0 + r) * PK + 2 * pr + 1];
          float sn, cs;
          __sincosf(th, &sn, &cs);
          dr[r] = gm * cs;
          di[r] = gm * sn;
          const float nr = ir * dr[r] - ii * di[r], ni = ir * di[r] + ii * dr[r];
          ir = nr;
          ii = ni;
        }
#pragma unroll
        for (int d = 1; d < NSEG; d *= 2) {
          const float ur = __shfl_up(ir, CW * d), ui = __shfl_up(ii, CW * d);
          if (seg >= d) {
            const float nr = ir * ur - ii * ui, ni = ir * ui + ii * ur;
            ir = nr;
            ii = ni;
          }
        }
        const float er = __shfl_up(ir, CW), ei = __shfl_up(ii, CW);
        float zr = seg > 0 ? er : 1.f, zi = seg > 0 ? ei : 0.f;
#pragma unroll
        for (int r = 0; r < TPS; ++r) {
          const int rr = r0 + r;
          const float nr = zr * dr[r] - zi * di[r], ni = zr * di[r] + zi * dr[r];
          zr = nr;
          zi = ni;
          const float k0 = sm.Kp[rr * PK + 2 * pr], k1 = sm.Kp[rr * PK + 2 * pr + 1];
          const float q0 = sm.Qp[rr * PK + 2 * pr], q1 = sm.Qp[rr * PK + 2 * pr + 1];
          const float iz = __builtin_amdgcn_rcpf(zr * zr + zi * zi);
          const float hr = zr * iz, hi = zi * iz;   // P^{-T} on a pair: z / |z|^2
          sm.Gam[rr * PK + 2 * pr] = zr;
          sm.Gam[rr * PK + 2 * pr + 1] = zi;
          sm.Kp[rr * PK + 2 * pr] = zr * k0 - zi * k1;
          sm.Kp[rr * PK + 2 * pr + 1] = zr * k1 + zi * k0;
          sm.Qp[rr * PK + 2 * pr] = zr * q0 - zi * q1;
          sm.Qp[rr * PK + 2 * pr + 1] = zr * q1 + zi * q0;
          sm.Kh[rr * PK + 2 * pr] = hr * k0 - hi * k1;
          sm.Kh[rr * PK + 2 * pr + 1] = hr * k1 + hi * k0;
        }
        if (seg == NSEG - 1) {
          sm.gl[2 * pr] = zr;
          sm.gl[2 * pr + 1] = zi;
          bad |= !(zr * zr + zi * zi >= kMinChunkDecay * kMinChunkDecay);
        }
      }
    }
    lds_barrier();
    // ------------------------------------------- N, M and inner = w v - Kp S^T
    {
      f32x4 an = {0.f, 0.f, 0.f, 0.f}, am = an, ai = an;
      mm<PK, 1, 1, PK, DK>(an, sm.Kp, 16 * ti2, sm.Kh, 16 * tj2);
      mm<PK, 1, 1, PK, DK>(am, sm.Qp, 16 * ti2, sm.Kh, 16 * tj2);
      mm<PK, 1, 1, PK, DK>(ai, sm.Kp, 16 * ti2, sm.S, 16 * tj2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * ti2 + 4 * g + j, s = 16 * tj2 + n;
        sm.N[r * PL + s] = s < r ? an[j] : 0.f;
        sm.M[r * PL + s] = s <= r ? am[j] : 0.f;
        sm.In[r * PV + s] = sm.w[r] * sm.V[r * PV + s] - ai[j];
      }
    }
    lds_barrier();
    // ------------------- T = (I + A)^{-1} with A = Diag(beta) N strictly lower, so
    // A^32 = 0 and T = (I - A)(I + A^2)(I + A^4)(I + A^8)(I + A^16): four
    // squarings and four products on the matrix cores, each wave one 16x16
    // tile of each (DM, DDl and DR, written later in the block, hold the
    // intermediate powers and partial products); then T Diag(beta) in DA
    {
      static_assert(Sm::PV == PL, "the scratch matrices share the L x L stride");
      for (int e = tid; e < L * L; e += NT) {
        const int r = e / L, c2 = e % L;
        const float a = sm.beta[r] * sm.N[r * PL + c2];   // N is 0 on and above the diagonal
        sm.DM[r * PL + c2] = a;
        sm.T[r * PL + c2] = (r == c2 ? 1.f : 0.f) - a;
      }
      lds_barrier();
      const int r0 = 16 * ti2, cc0 = 16 * tj2;
      auto tile_load = [&](const float* m) {
        f32x4 t;
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = m[(r0 + 4 * g + j) * PL + cc0 + n];
        return t;
      };
      auto tile_store = [&](float* m, const f32x4& t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) m[(r0 + 4 * g + j) * PL + cc0 + n] = t[j];
      };
      float* Xc = sm.DM;
      float* Xn = sm.DDl;
      {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        mm<PL, 1, PL, 1, L>(x, Xc, r0, Xc, cc0);   // A^2
        tile_store(Xn, x);
      }
      lds_barrier();
      { float* t_ = Xc; Xc = Xn; Xn = t_; }
      float* Pc = sm.T;
      float* Pn = sm.DR;
#pragma unroll 1
      for (int m = 0; m < 4; ++m) {
        f32x4 pv = tile_load(Pc);
        mm<PL, 1, PL, 1, L>(pv, Pc, r0, Xc, cc0);   // P (I + A^(2^(m+1)))
        tile_store(Pn, pv);
        if (m < 3) {
          f32x4 x = {0.f, 0.f, 0.f, 0.f};
          mm<PL, 1, PL, 1, L>(x, Xc, r0, Xc, cc0);   // the next power
          tile_store(Xn, x);
        }
        lds_barrier();
        { float* t_ = Pc; Pc = Pn; Pn = t_; }
        { float* t_ = Xc; Xc = Xn; Xn = t_; }
      }
      // four swaps: the product is back in T
      for (int e = tid; e < L * L; e += NT) {
        const int r = e / L, c2 = e % L;
        sm.DA[r * PL + c2] = sm.T[r * PL + c2] * sm.beta[c2];
      }
    }
    lds_barrier();
    // ----------------------------------------------- Dl = T Diag(beta) inner
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm<PL, 1, PV, 1, L>(acc, sm.DA, 16 * ti2, sm.In, 16 * tj2);
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.Dl[(16 * ti2 + 4 * g + j) * PV + 16 * tj2 + n] = acc[j];
    }
    lds_barrier();
    // ---- Y = S + Dl^T Kh, S_end = Y P_L, dY = G P_L^T, block-end decay term
    f32x4 dYr[2][CPW];
    {
      float te[CPW][2];   // per column tile: DIAG sum_i G S_end; ROT2 (da, dphi) of the pair
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) te[cc][0] = te[cc][1] = 0.f;
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
          const int col0 = 16 * (wv * CPW + cc), ch = col0 + n;
          f32x4 y;
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = sm.S[(16 * ti + 4 * g + j) * PK + ch];
          mm<1, PV, PK, 1, L>(y, sm.Dl, 16 * ti, sm.Kh, col0);
          if constexpr (DECAY == 0) {
            const float z = sm.gl[ch];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              te[cc][0] += G[ti][cc][j] * (y[j] * z);
              dYr[ti][cc][j] = G[ti][cc][j] * z;
            }
          } else {
            const bool even = (n & 1) == 0;
            const float zr = sm.gl[ch & ~1], zi = sm.gl[ch | 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float yo = __shfl_xor(y[j], 1), go = __shfl_xor(G[ti][cc][j], 1);
              const float y0 = even ? y[j] : yo, y1 = even ? yo : y[j];
              const float g0 = even ? G[ti][cc][j] : go, g1 = even ? go : G[ti][cc][j];
              // a state row is multiplied by conj(z) (the transition acts on
              // the right), the adjoint row by z
              const float s0 = y0 * zr + y1 * zi, s1 = y1 * zr - y0 * zi;   // S_end pair
              const float d0 = g0 * zr - g1 * zi, d1 = g0 * zi + g1 * zr;   // dY pair
              dYr[ti][cc][j] = even ? d0 : d1;
              if (even) {   // d/da of conj(z) is conj(z), d/dphi is -i conj(z)
                te[cc][0] += g0 * s0 + g1 * s1;
                te[cc][1] += g0 * s1 - g1 * s0;
              }
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) sm.DY[(16 * ti + 4 * g + j) * PK + ch] = dYr[ti][cc][j];
        }
      }
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        const int ch = 16 * (wv * CPW + cc) + n;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          te[cc][e] += __shfl_xor(te[cc][e], 16);
          te[cc][e] += __shfl_xor(te[cc][e], 32);
        }
        if (g == 0) {
          if constexpr (DECAY == 0) {
            sm.dl_end[ch] = te[cc][0];
          } else if ((n & 1) == 0) {
            sm.dl_end[ch >> 1] = te[cc][0];
            sm.dl_end[DK / 2 + (ch >> 1)] = te[cc][1];
          }
        }
      }
    }
    lds_barrier();
    // ------------------------------------------ dDl = M^T dO + Kh dY^T  [L x TV]
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm<1, PL, PV, 1, L>(acc, sm.M, 16 * ti2, sm.DO, 16 * tj2);
      mm<PK, 1, 1, PK, DK>(acc, sm.Kh, 16 * ti2, sm.DY, 16 * tj2);
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.DDl[(16 * ti2 + 4 * g + j) * PV + 16 * tj2 + n] = acc[j];
    }
    lds_barrier();
    // ------------ dR = T^T dDl; dinner = beta dR; grad_v; dw and dbeta row sums
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm<1, PL, PV, 1, L>(acc, sm.T, 16 * ti2, sm.DDl, 16 * tj2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * ti2 + 4 * g + j, i = 16 * tj2 + n;
        const float din = sm.beta[r] * acc[j];
        sm.DR[r * PV + i] = acc[j];
        sm.Din[r * PV + i] = din;
        if (r < nt) p.grad_v[(bh + (size_t)(t0 + r) * H) * DV + v0 + i] = sm.w[r] * din;
        const float pw = sum16(din * sm.V[r * PV + i]);
        const float pb = sum16(acc[j] * sm.In[r * PV + i]);
        if (n == 0) {
          sm.red[tj2][r] = pw;
          sm.red[2 + tj2][r] = pb;
        }
      }
    }
    lds_barrier();
    // --------------------- dA = -dR Dl^T -> dN; dM = lower(dO Dl^T); dbeta part
    {
      f32x4 da = {0.f, 0.f, 0.f, 0.f}, dm = da;
      mm<PV, 1, 1, PV, TV>(da, sm.DR, 16 * ti2, sm.Dl, 16 * tj2);
      mm<PV, 1, 1, PV, TV>(dm, sm.DO, 16 * ti2, sm.Dl, 16 * tj2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * ti2 + 4 * g + j, s = 16 * tj2 + n;
        const float a = -da[j];
        const float pb = sum16(s < r ? a * sm.N[r * PL + s] : 0.f);
        if (n == 0) sm.red[4 + tj2][r] = pb;
        sm.DA[r * PL + s] = s < r ? sm.beta[r] * a : 0.f;   // dN
        sm.DM[r * PL + s] = s <= r ? dm[j] : 0.f;
      }
    }
    lds_barrier();
    // ------------------------- dQp, dKp, dKh [L x DK] and the per-tile partials
    if (tid < L && tid < nt) {
      const size_t row = bh + (size_t)(t0 + tid) * H;
      Pw[(size_t)vt * BTH + row] = sm.red[0][tid] + sm.red[1][tid];
      Pb[(size_t)vt * BTH + row] = sm.red[2][tid] + sm.red[3][tid] + sm.red[4][tid] + sm.red[5][tid];
    }
#pragma unroll 1
    for (int ti = 0; ti < 2; ++ti) {
#pragma unroll 1
      for (int cc = 0; cc < CPW; ++cc) {
        const int col0 = 16 * (wv * CPW + cc), ch = col0 + n;
        f32x4 dq = {0.f, 0.f, 0.f, 0.f}, dkp = dq, dkp2 = dq, dkh = dq;
        mm<PV, 1, PK, 1, TV>(dq, sm.DO, 16 * ti, sm.S, col0);
        mm<PL, 1, PK, 1, L>(dq, sm.DM, 16 * ti, sm.Kh, col0);
        mm<PL, 1, PK, 1, L>(dkp, sm.DA, 16 * ti, sm.Kh, col0);
        mm<PV, 1, PK, 1, TV>(dkp2, sm.Din, 16 * ti, sm.S, col0);
        mm<PV, 1, PK, 1, TV>(dkh, sm.Dl, 16 * ti, sm.DY, col0);
        mm<1, PL, PK, 1, L>(dkh, sm.DM, 16 * ti, sm.Qp, col0);
        mm<1, PL, PK, 1, L>(dkh, sm.DA, 16 * ti, sm.Kp, col0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * ti + 4 * g + j;
          const float gq = dq[j], gkp = dkp[j] - dkp2[j], gkh = dkh[j];
          const float kp = sm.Kp[r * PK + ch], qp = sm.Qp[r * PK + ch], kh = sm.Kh[r * PK + ch];
          const size_t row = bh + (size_t)(t0 + r) * H;
          const size_t o = ((size_t)vt * BTH + row) * DK;
          if constexpr (DECAY == 0) {
            const float gam = sm.Gam[r * PK + ch];
            float dl = kp * gkp - kh * gkh + qp * gq;
            if (r == nt - 1) dl += sm.dl_end[ch];
            if (r < nt) {
              Pq[o + ch] = gam * gq;
              Pk[o + ch] = gam * gkp + gkh * __builtin_amdgcn_rcpf(gam);
              Pl[o + ch] = dl;
            }
          } else {
            // pairs (2p, 2p + 1) sit in adjacent lanes
            const bool even = (n & 1) == 0;
            const float zr = sm.Gam[r * PK + (ch & ~1)], zi = sm.Gam[r * PK + (ch | 1)];
            const float o_q = __shfl_xor(gq, 1), o_kp = __shfl_xor(gkp, 1), o_kh = __shfl_xor(gkh, 1);
            const float x_kp = __shfl_xor(kp, 1), x_qp = __shfl_xor(qp, 1), x_kh = __shfl_xor(kh, 1);
            // components 0 and 1 of each pair
            const float q0 = even ? gq : o_q, q1 = even ? o_q : gq;
            const float a0 = even ? gkp : o_kp, a1 = even ? o_kp : gkp;
            const float h0 = even ? gkh : o_kh, h1 = even ? o_kh : gkh;
            const float Kp0 = even ? kp : x_kp, Kp1 = even ? x_kp : kp;
            const float Qp0 = even ? qp : x_qp, Qp1 = even ? x_qp : qp;
            const float Kh0 = even ? kh : x_kh, Kh1 = even ? x_kh : kh;
            // dq = conj(z) dQp; dk = conj(z) dKp + conj(z) / |z|^2 dKh
            const float iz = __builtin_amdgcn_rcpf(zr * zr + zi * zi);
            const float dq0 = zr * q0 + zi * q1, dq1 = zr * q1 - zi * q0;
            const float dk0 = zr * a0 + zi * a1 + iz * (zr * h0 + zi * h1);
            const float dk1 = zr * a1 - zi * a0 + iz * (zr * h1 - zi * h0);
            // log-magnitude and angle gradients of the pair's running product
            float da = Kp0 * a0 + Kp1 * a1 - (Kh0 * h0 + Kh1 * h1) + Qp0 * q0 + Qp1 * q1;
            float dphi = (-a0 * Kp1 + a1 * Kp0) + (-h0 * Kh1 + h1 * Kh0) + (-q0 * Qp1 + q1 * Qp0);
            const int pr = ch >> 1;
            if (r == nt - 1) {
              da += sm.dl_end[pr];
              dphi += sm.dl_end[DK / 2 + pr];
            }
            if (r < nt) {
              Pq[o + ch] = even ? dq0 : dq1;
              Pk[o + ch] = even ? dk0 : dk1;
              Pl[o + (even ? pr : DK / 2 + pr)] = even ? da : dphi;
            }
          }
        }
      }
    }
    // --------------------- dS = dY + dO^T Qp - dinner^T Kp: G of the previous block
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        const int col0 = 16 * (wv * CPW + cc);
        f32x4 acc = dYr[ti][cc], acc2 = {0.f, 0.f, 0.f, 0.f};
        mm<1, PV, PK, 1, L>(acc, sm.DO, 16 * ti, sm.Qp, col0);
        mm<1, PV, PK, 1, L>(acc2, sm.Din, 16 * ti, sm.Kp, col0);
        G[ti][cc] = acc - acc2;
      }
    }
    lds_barrier();
  }
  if (p.grad_S0) {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = v0 + 16 * ti + 4 * g + j, col = 16 * (wv * CPW + cc) + n;
          p.grad_S0[((size_t)(b * H + h) * DV + row) * DK + col] = G[ti][cc][j];
        }
  }
  // one flag per workgroup, written whether set or not (no clearing needed)
  __shared__ int bad_w[4];
  const bool wbad = __ballot(bad) != 0ull;
  if (l == 0) bad_w[wv] = wbad ? 1 : 0;
  lds_barrier();
  if (tid == 0) p.flag[blockIdx.x] = bad_w[0] | bad_w[1] | bad_w[2] | bad_w[3];
}

// ------------------------------------------------------------------------------
// Token path of the backward for a flagged (b, h, value tile): the reverse mode
// of the token recurrence itself,
//     X = S_{t-1} D_t,  e = w_t v_t - X k_t,  S_t = X + beta_t e k_t^T,  o_t = S_t q_t,
// per value row (rows are independent under key-axis transitions):
//     g += dO_t q_t;            dq_t += dO_t S_t
//     gk = g . k_t;             dbeta_t += e gk;  dw_t += beta v gk;  dv_t = w beta gk
//     dX = g - beta gk k_t;     dk_t += beta e g - beta gk X
//     g = dX D_t^T;             d(decay)_t from dX and S_{t-1}
// with the sums over rows.  S_{t-1} comes from recomputing each block forward
// from its checkpoint: once over the block keeping the state at every eighth
// token in LDS, then per group of 8 tokens (last group first) again from that
// state, keeping the group's 8 states in registers.  fp32 throughout and no
// division, so decays of 0 are exact.
//
// Layout: a wave holds 8 rows (lanes 8c + r: row r, channels c*DK/8 ..), so a
// row's dot products reduce over lanes 8, 16 and 32 apart and the sums over
// rows over 8 neighbouring lanes (DPP).  The decay's partial sums go out per
// token as dL/d(alpha) (DIAG) or dL/d(gamma), dL/d(theta) (ROT2) -- already the
// transition's own gradients, which bwd_reduce_kernel adds up without its
// prefix sum for flagged heads.

template <int DK>
struct TokSmem {
  static constexpr int NG = L / 8;   // groups of 8 tokens
  __bf16 K[L * DK], Q[L * DK];
  float Z[L * DK];            // DIAG alpha; ROT2 (gamma cos theta, gamma sin theta) per pair
  float V[L * TV], DO[L * TV];
  float beta[L], w[L];
  float sub[NG][TV * DK];     // the state before tokens 0, 8, 16, 24 of the block
  float ev[L][TV];            // per token and row: e = w v - X k, from the first forward pass
  float red[8][4][3 * DK];    // per token of a group, per wave: dq, dk, d(decay) row sums
  float redb[8][4][2];        // dbeta, dw row sums
};

// sum over the 8 neighbouring lanes 8c .. 8c + 7; every lane gets it (no lane
// reads outside its row, so bound_ctrl never applies; with it set the compiler
// folds each move into the add as a DPP operand)
__device__ inline float sum8_rows(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, true));    // lane ^ 1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, true));    // lane ^ 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, true));   // 7 - lane in 8
  return x;
}
// sum over the lanes r, r + 8, ..., r + 56 (one row's channel slices)
__device__ inline float sum_row_slices(float x) {
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <int DK, int DECAY>
__global__ __launch_bounds__(NT) void bwd_token_kernel(BwdParams p) {
  if (p.flag[blockIdx.x] == 0) return;   // uniform over the workgroup
  using Sm = TokSmem<DK>;
  constexpr int CPL = DK / 8;            // channels per lane
  __shared__ __attribute__((aligned(16))) Sm sm;
  const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
  const int r = l & 7, cs = l >> 3, row = 8 * wv + r, ch0 = cs * CPL;
  const int H = p.H, Tn = p.T, DV = p.DV;
  const int vt = blockIdx.x % p.n_vt, unit = blockIdx.x / p.n_vt;
  const int b = unit / H, h = unit % H;
  const int v0 = vt * TV;
  const int nc = (Tn + L - 1) / L;
  const size_t bh = (size_t)b * Tn * H + h;
  const size_t BTH = (size_t)p.B * Tn * H;
  const __bf16* q = (const __bf16*)p.q;
  const __bf16* k = (const __bf16*)p.k;
  const __bf16* v = (const __bf16*)p.v;
  const __bf16* dO = (const __bf16*)p.grad_o;
  float* Pq = p.part;
  float* Pk = Pq + (size_t)p.n_vt * BTH * DK;
  float* Pl = Pk + (size_t)p.n_vt * BTH * DK;
  float* Pb = Pl + (size_t)p.n_vt * BTH * DK;
  float* Pw = Pb + (size_t)p.n_vt * BTH;
  const size_t srow = ((size_t)(b * H + h) * DV + v0 + row) * DK + ch0;   // this lane's state slice

  float gr[CPL];   // dL/dS of this lane's row slice after the token being undone
#pragma unroll
  for (int e = 0; e < CPL; ++e) gr[e] = p.grad_S ? p.grad_S[srow + e] : 0.f;

  // this lane's slice of X = S D_t
  auto transition = [&](const float (&s)[CPL], float (&x)[CPL], int t) {
    const float* z = sm.Z + t * DK + ch0;
#pragma unroll
    for (int e = 0; e < CPL; e += 2) {
      if constexpr (DECAY == 0) {
        x[e] = s[e] * z[e];
        x[e + 1] = s[e + 1] * z[e + 1];
      } else {   // S times the block gamma [[c, -s], [s, c]]: zr = gamma c, zi = gamma s
        x[e] = z[e] * s[e] + z[e + 1] * s[e + 1];
        x[e + 1] = -z[e + 1] * s[e] + z[e] * s[e + 1];
      }
    }
  };
  auto keys = [&](float (&kk)[CPL], const __bf16* src) {   // CPL bf16 as 16-byte pieces
#pragma unroll
    for (int e8 = 0; e8 < CPL; e8 += 8) {
      const uint4 u4 = *(const uint4*)(src + e8);
      const uint32_t wds[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kk[e8 + 2 * j] = __uint_as_float(wds[j] << 16);
        kk[e8 + 2 * j + 1] = __uint_as_float(wds[j] & 0xffff0000u);
      }
    }
  };
  // one token forward: s <- S_t from s = S_{t-1}; the first pass over a block
  // forms e = w v - X k with a row dot product and keeps it, the later passes
  // (the group recomputes) read it back, so only the first has the serial
  // cross-lane reduction
  auto fwd_token = [&](float (&s)[CPL], int t, bool first) {
    float x[CPL], kk[CPL];
    transition(s, x, t);
    keys(kk, sm.K + t * DK + ch0);
    float ev;
    if (first) {
      float y = 0.f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) y += x[e] * kk[e];
      ev = sm.w[t] * sm.V[t * TV + row] - sum_row_slices(y);
      if (cs == 0) sm.ev[t][row] = ev;
    } else {
      ev = sm.ev[t][row];
    }
    const float cf = sm.beta[t] * ev;
#pragma unroll
    for (int e = 0; e < CPL; ++e) s[e] = x[e] + cf * kk[e];
  };

  for (int c = nc - 1; c >= 0; --c) {
    const int t0 = c * L, nt = min(L, Tn - t0);
    // ------------------------------------------------ stage the block's inputs
    for (int e = tid; e < L * DK / 8; e += NT) {
      const int tt = e / (DK / 8), j8 = e % (DK / 8);
      uint4 kk = {0u, 0u, 0u, 0u}, qq = kk;
      if (tt < nt) {
        const size_t src = (bh + (size_t)(t0 + tt) * H) * DK + 8 * j8;
        kk = *(const uint4*)(k + src);
        qq = *(const uint4*)(q + src);
      }
      *(uint4*)(sm.K + tt * DK + 8 * j8) = kk;
      *(uint4*)(sm.Q + tt * DK + 8 * j8) = qq;
    }
    if constexpr (DECAY == 0) {
      for (int e = tid; e < L * DK / 4; e += NT) {
        const int tt = e / (DK / 4), j4 = e % (DK / 4);
        f32x4 a = {1.f, 1.f, 1.f, 1.f};
        if (tt < nt) a = *(const f32x4*)(p.alpha + (bh + (size_t)(t0 + tt) * H) * DK + 4 * j4);
        *(f32x4*)(sm.Z + tt * DK + 4 * j4) = a;
      }
    } else {
      for (int e = tid; e < L * DK / 2; e += NT) {
        const int tt = e / (DK / 2), pr = e % (DK / 2);
        float zr = 1.f, zi = 0.f;
        if (tt < nt) {
          const size_t src = (bh + (size_t)(t0 + tt) * H) * (DK / 2) + pr;
          float sn, cn;
          __sincosf(p.theta[src], &sn, &cn);
          const float gm = p.alpha[src];
          zr = gm * cn;
          zi = gm * sn;
        }
        sm.Z[tt * DK + 2 * pr] = zr;
        sm.Z[tt * DK + 2 * pr + 1] = zi;
      }
    }
    for (int e = tid; e < L * TV; e += NT) {
      const int tt = e / TV, i = e % TV;
      float vv = 0.f, gg = 0.f;
      if (tt < nt) {
        const size_t src = (bh + (size_t)(t0 + tt) * H) * DV + v0 + i;
        vv = (float)v[src];
        gg = (float)dO[src];
      }
      sm.V[e] = vv;
      sm.DO[e] = gg;
    }
    if (tid < L) {
      const bool ok = tid < nt;
      const size_t src = bh + (size_t)(t0 + tid) * H;
      sm.beta[tid] = ok ? p.beta[src] : 0.f;
      sm.w[tid] = ok ? p.w[src] : 0.f;
    }
    lds_barrier();
    // ------------- forward over the block, keeping the state before every 8th token
    {
      float s[CPL];
      const float* ck = p.ckpt + ((size_t)unit * nc + c) * DV * DK + (size_t)(v0 + row) * DK + ch0;
#pragma unroll
      for (int e = 0; e < CPL; e += 4) *(f32x4*)(s + e) = *(const f32x4*)(ck + e);
      for (int t = 0; t < nt; ++t) {
        if ((t & 7) == 0) {
#pragma unroll
          for (int e = 0; e < CPL; e += 4)
            *(f32x4*)(sm.sub[t >> 3] + row * DK + ch0 + e) = *(const f32x4*)(s + e);
        }
        fwd_token(s, t, true);
      }
    }
    // ------------------------------------ groups of 8 tokens, last group first
    for (int grp = (nt - 1) >> 3; grp >= 0; --grp) {
      float st[8][CPL];   // the state before each token of the group
      {
        float s[CPL];
#pragma unroll
        for (int e = 0; e < CPL; e += 4) *(f32x4*)(s + e) = *(const f32x4*)(sm.sub[grp] + row * DK + ch0 + e);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int e = 0; e < CPL; ++e) st[u][e] = s[e];
          if (u < 7 && 8 * grp + u < nt) fwd_token(s, 8 * grp + u, false);
        }
      }
#pragma unroll
      for (int u = 7; u >= 0; --u) {
        const int t = 8 * grp + u;
        if (t < nt) {
          float x[CPL], kk[CPL], qq[CPL];
          transition(st[u], x, t);
          keys(kk, sm.K + t * DK + ch0);
          keys(qq, sm.Q + t * DK + ch0);
          const float bt = sm.beta[t], wt = sm.w[t], vr = sm.V[t * TV + row];
          const float ev = sm.ev[t][row];   // w v - X k
          const float dor = sm.DO[t * TV + row];
          float dq[CPL], dk[CPL], dz[CPL];
          float gk = 0.f;
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            dq[e] = dor * (x[e] + bt * ev * kk[e]);   // dO_t S_t
            gr[e] += dor * qq[e];
            gk += gr[e] * kk[e];
          }
          gk = sum_row_slices(gk);
          const float bg = bt * gk;
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            const float dx = gr[e] - bg * kk[e];
            dk[e] = bt * ev * gr[e] - bg * x[e];
            gr[e] = dx;   // dX for now
          }
          // through the transition: g = dX D^T, and the decay's gradient
          const float* z = sm.Z + t * DK + ch0;
#pragma unroll
          for (int e = 0; e < CPL; e += 2) {
            const float d0 = gr[e], d1 = gr[e + 1];
            const float s0 = st[u][e], s1 = st[u][e + 1];
            if constexpr (DECAY == 0) {
              gr[e] = d0 * z[e];
              gr[e + 1] = d1 * z[e + 1];
              dz[e] = d0 * s0;
              dz[e + 1] = d1 * s1;
            } else {
              const float zr = z[e], zi = z[e + 1];
              gr[e] = zr * d0 - zi * d1;
              gr[e + 1] = zi * d0 + zr * d1;
              dz[e] = d0 * s0 + d1 * s1;       // d/d(gamma c)
              dz[e + 1] = d0 * s1 - d1 * s0;   // d/d(gamma s)
            }
          }
          // sums over the wave's 8 rows; lanes of row 0 keep them
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            dq[e] = sum8_rows(dq[e]);
            dk[e] = sum8_rows(dk[e]);
            dz[e] = sum8_rows(dz[e]);
          }
          const float pb = sum8_rows(ev * gk), pw = sum8_rows(bt * vr * gk);
          if (r == 0) {
#pragma unroll
            for (int e = 0; e < CPL; e += 4) {
              *(f32x4*)(&sm.red[u][wv][ch0 + e]) = *(const f32x4*)(dq + e);
              *(f32x4*)(&sm.red[u][wv][DK + ch0 + e]) = *(const f32x4*)(dk + e);
              *(f32x4*)(&sm.red[u][wv][2 * DK + ch0 + e]) = *(const f32x4*)(dz + e);
            }
          }
          if (l == 0) {
            sm.redb[u][wv][0] = pb;
            sm.redb[u][wv][1] = pw;
          }
          if (cs == 0) p.grad_v[(bh + (size_t)(t0 + t) * H) * DV + v0 + row] = wt * bg;
        }
      }
      lds_barrier();
      // the workgroup's sums for the group's tokens -> this tile's partials
      for (int idx = tid; idx < 8 * 3 * DK; idx += NT) {
        const int u = idx / (3 * DK), rem = idx % (3 * DK), qd = rem / DK, ch = rem % DK;
        const int t = 8 * grp + u;
        if (t >= nt) continue;
        const float sum = sm.red[u][0][rem] + sm.red[u][1][rem] + sm.red[u][2][rem] + sm.red[u][3][rem];
        const size_t trow = bh + (size_t)(t0 + t) * H;
        const size_t o = ((size_t)vt * BTH + trow) * DK;
        if (qd == 0) {
          Pq[o + ch] = sum;
        } else if (qd == 1) {
          Pk[o + ch] = sum;
        } else if constexpr (DECAY == 0) {
          Pl[o + ch] = sum;
        } else if ((ch & 1) == 0) {
          // (d/d(gamma c), d/d(gamma s)) -> d/d(gamma) = dzr c + dzi s,
          // d/d(theta) = dzi (gamma c) - dzr (gamma s)
          const float dzi = sm.red[u][0][rem + 1] + sm.red[u][1][rem + 1] + sm.red[u][2][rem + 1] +
                            sm.red[u][3][rem + 1];
          const int pr = ch >> 1;
          float sn, cn;
          __sincosf(p.theta[trow * (DK / 2) + pr], &sn, &cn);
          const float zr = sm.Z[t * DK + ch], zi = sm.Z[t * DK + ch + 1];
          Pl[o + pr] = sum * cn + dzi * sn;
          Pl[o + DK / 2 + pr] = dzi * zr - sum * zi;
        }
      }
      if (tid < 16) {
        const int u = tid >> 1, which = tid & 1, t = 8 * grp + u;
        if (t < nt) {
          const float sum = sm.redb[u][0][which] + sm.redb[u][1][which] + sm.redb[u][2][which] +
                            sm.redb[u][3][which];
          const size_t trow = bh + (size_t)(t0 + t) * H;
          (which == 0 ? Pb : Pw)[(size_t)vt * BTH + trow] = sum;
        }
      }
      lds_barrier();
    }
  }
  if (p.grad_S0) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) p.grad_S0[srow + e] = gr[e];
  }
}

// Sums the value tiles' partials; turns the per-token log-gradients of the
// running decay into gradients of each token's decay by a reverse prefix sum
// over the block (a token's decay enters every running product from it to
// the block's end).  One workgroup of DK threads per (b, h, block).
template <int DK, int DECAY>
__global__ __launch_bounds__(DK) void bwd_reduce_kernel(BwdParams p) {
  const int H = p.H, Tn = p.T;
  const int nc = (Tn + L - 1) / L;
  const int c = blockIdx.x % nc, unit = blockIdx.x / nc;
  const int b = unit / H, h = unit % H;
  const int t0 = c * L, nt = min(L, Tn - t0);
  const int j = threadIdx.x;
  const size_t bh = (size_t)b * Tn * H + h;
  const size_t BTH = (size_t)p.B * Tn * H;
  constexpr int nvt = DK / TV;   // value tiles (d_v = d_k here; the launcher checks it)
  const float* Pq = p.part;
  const float* Pk = Pq + (size_t)nvt * BTH * DK;
  const float* Pl = Pk + (size_t)nvt * BTH * DK;
  const float* Pb = Pl + (size_t)nvt * BTH * DK;
  const float* Pw = Pb + (size_t)nvt * BTH;
  // flagged heads: the token path's partials are already the decay's gradients
  const bool direct = p.flag[unit * nvt] != 0;
  // Rows go in groups of RG, last first; a group's loads are all issued before
  // its stores (the outputs may alias the partials as far as the compiler
  // knows, so a load after a store would wait for it).
  constexpr int RG = 4;
  float acc0 = 0.f, acc1 = 0.f;
  for (int r0 = nt - 1; r0 >= 0; r0 -= RG) {
    float sq[RG], sk[RG], sl0[RG], sl1[RG], al[RG], sb[RG], sw[RG];
#pragma unroll
    for (int u = 0; u < RG; ++u) {
      sq[u] = sk[u] = sl0[u] = sl1[u] = sb[u] = sw[u] = 0.f;
      al[u] = 1.f;
      const int r = r0 - u;
      if (r < 0) continue;
      const size_t row = bh + (size_t)(t0 + r) * H;
#pragma unroll
      for (int t = 0; t < nvt; ++t) {
        const size_t o = ((size_t)t * BTH + row) * DK;
        sq[u] += Pq[o + j];
        sk[u] += Pk[o + j];
        if (DECAY == 0) {
          sl0[u] += Pl[o + j];
        } else if (j < DK / 2) {
          sl0[u] += Pl[o + j];
          sl1[u] += Pl[o + DK / 2 + j];
        }
      }
      if (!direct) {
        if (DECAY == 0) al[u] = p.alpha[row * DK + j];
        else if (j < DK / 2) al[u] = p.alpha[row * (DK / 2) + j];
      }
      if (j == 0) {
#pragma unroll
        for (int t = 0; t < nvt; ++t) {
          sb[u] += Pb[(size_t)t * BTH + row];
          sw[u] += Pw[(size_t)t * BTH + row];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RG; ++u) {
      const int r = r0 - u;
      if (r < 0) continue;
      const size_t row = bh + (size_t)(t0 + r) * H;
      p.grad_q[row * DK + j] = sq[u];
      p.grad_k[row * DK + j] = sk[u];
      if (DECAY == 0) {
        acc0 += sl0[u];
        p.grad_alpha[row * DK + j] = direct ? sl0[u] : acc0 / al[u];
      } else if (j < DK / 2) {
        acc0 += sl0[u];
        acc1 += sl1[u];
        p.grad_alpha[row * (DK / 2) + j] = direct ? sl0[u] : acc0 / al[u];
        p.grad_theta[row * (DK / 2) + j] = direct ? sl1[u] : acc1;
      }
      if (j == 0) {
        p.grad_beta[row] = sb[u];
        p.grad_w[row] = sw[u];
      }
    }
  }
}

template <int DK, int DECAY>
hipError_t launch_dk(const BwdParams& p0, hipStream_t s) {
  BwdParams p = p0;
  p.n_vt = p.DV / TV;
  const int nc = (p.T + L - 1) / L;
  hipLaunchKernelGGL((bwd_kernel<DK, DECAY>), dim3(p.B * p.H * p.n_vt), dim3(NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // same grid: each workgroup reads the flag bwd_kernel wrote for it
  hipLaunchKernelGGL((bwd_token_kernel<DK, DECAY>), dim3(p.B * p.H * p.n_vt), dim3(NT), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_reduce_kernel<DK, DECAY>), dim3(p.B * p.H * nc), dim3(DK), 0, s, p);
  return hipGetLastError();
}

}  // namespace bwd

hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
  const bool rot = p.decay != 0;
  if (p.DK == 128 && p.DV == 128) return rot ? bwd::launch_dk<128, 1>(p, s) : bwd::launch_dk<128, 0>(p, s);
  if (p.DK == 64 && p.DV == 64) return rot ? bwd::launch_dk<64, 1>(p, s) : bwd::launch_dk<64, 0>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace gdr
