// perm_fwd.hip -- delta rule with partial-permutation transitions, gfx950.
//
// SFDA technical summary, finite-state expressivity: partial permutations as
// the structured control realise a bounded stack.  Per token the key-axis
// transition selects columns of the state (column j <- column src[j], or zero),
// then the delta-rule erase and write follow:
//
//   X = S D_t;  S = X + beta (w v - X k) k^T;  o = S q.
//
// Products of such transitions are singular (a dropped channel never comes
// back), so the split chunk form (which needs Gamma^-1) does not exist here;
// the kernel walks the tokens in order.  Value rows evolve independently under
// key-axis transitions, so every row runs on its own: a wave carries 8 rows
// (8 lanes per row, d_k/8 channels per lane, fp32 in registers) and needs no
// other wave within a chunk -- the column selection goes through the wave's own
// LDS row buffer (a source outside [0, d_k) is mapped at staging to a column
// that always holds 0, so the gather has no test), the two dot products through
// DPP butterflies inside each group of 8 lanes.  Workgroups (one head, 32 value
// rows) stage 16 tokens of k, q (as fp32), the source maps, v, beta and w in
// LDS, with the next chunk's loads in flight; the value blocks of one head
// share an XCD, so keys, queries and maps come from its L2 after the first
// reader.  Staging also classifies every token's map (the same for all rows):
// the identity and the two unit shifts of a bounded stack (push: channel j
// takes j - 1 and channel 0 empties; pop: j takes j + 1 and the last empties)
// then move the row in registers (one DPP move across the row's lanes), and
// only other maps use the LDS selection.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "perm_kernels.h"

namespace gdr {
namespace perm {
namespace {

using bf = __bf16;
constexpr int L = 16;      // tokens per staged chunk
constexpr int NT = 256;    // 4 waves x 8 rows = 32 value rows per workgroup
constexpr int RPW = 8;     // rows per wave (8 lanes per row)
constexpr int ROWS = 4 * RPW;

constexpr int kGeneral = 0, kIdentity = 1, kDown = 2, kUp = 3;

// Keys and queries in LDS as fp32 rows of KRS floats: the 16-channel slice of
// lane group c starts at 20 c (d_k = 128), so the eight slices one wave reads
// per token sit in distinct banks; 8-channel slices (d_k = 64) need no padding.
template <int D>
constexpr int kq_pad() { return D / 8 == 16 ? 4 : 0; }
template <int D>
constexpr int kq_rs() { return D + 8 * kq_pad<D>(); }

template <int D>
struct Sh {
  float Kc[L * kq_rs<D>()];   // keys and queries, unpacked from bf16 at staging
  float Qc[L * kq_rs<D>()];
  int16_t Sc[L * D];       // source channel, or D (the zero column) where there is none
  bf Vc[L * ROWS];
  float Bc[L];             // beta
  float Wc[L];             // w
  int Kind[L];             // the token's map: kGeneral, kIdentity, kDown or kUp
  float Rb[4][RPW][D + 4]; // per wave, per row: the row for the column selection; [D] = 0
  bf Oc[L * ROWS];
};

// sum over 8 aligned lanes; every lane gets the same value (no lane reads
// outside its row, so bound_ctrl never applies; with it set the compiler folds
// each move into the add as a DPP operand)
__device__ inline float row_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, true));
  return x;
}

__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ inline uint32_t src_fix(uint32_t pair, int d) {   // two int16 sources -> [0, d]
  const int a = (int)(int16_t)(pair & 0xffffu), b = (int)(int16_t)(pair >> 16);
  const uint32_t ua = (a >= 0 && a < d) ? (uint32_t)a : (uint32_t)d;
  const uint32_t ub = (b >= 0 && b < d) ? (uint32_t)b : (uint32_t)d;
  return ua | (ub << 16);
}

// Which of the three structured maps 8 consecutive fixed sources (channels
// j0 .. j0 + 7; D stands for "none") agree with: bit 0 identity, bit 1 down
// (j <- j - 1), bit 2 up (j <- j + 1).
template <int D>
__device__ inline unsigned classify8(const uint32_t (&fx)[4], int j0) {
  bool id = true, dn = true, up = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = j0 + i;
    const int sv = (int)((fx[i >> 1] >> (16 * (i & 1))) & 0xffffu);
    id = id && sv == j;
    dn = dn && sv == (j >= 1 ? j - 1 : D);
    up = up && sv == (j + 1 < D ? j + 1 : D);
  }
  return (id ? 1u : 0u) | (dn ? 2u : 0u) | (up ? 4u : 0u);
}

template <int D>
__global__ __launch_bounds__(NT) void perm_fwd_kernel(PermParams p) {
  constexpr int CPL = D / 8;           // key channels per lane
  constexpr int PPT = D / 8;           // 16-byte pieces per token row (bf16 / int16)
  constexpr int NPIECE = L * PPT;      // such pieces per chunk per tensor (<= NT)
  __shared__ __attribute__((aligned(16))) Sh<D> sh;

  // value blocks of one head on one XCD (workgroup ids 8 apart)
  const int NVB = p.DV / ROWS;
  const int id = blockIdx.x, xcd = id & 7, vb = (id >> 3) % NVB, grp = (id >> 3) / NVB;
  const int bh = grp * 8 + xcd;
  if (bh >= p.B * p.H) return;
  const int b = bh / p.H, h = bh % p.H;
  const int T = p.T, H = p.H, DV = p.DV, v0 = vb * ROWS;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l >> 3, cg = l & 7;
  const int vrow = v0 + RPW * w + r;
  const size_t row0 = (size_t)b * T * H + h;
  const bf* qg = static_cast<const bf*>(p.q) + row0 * D;
  const bf* kg = static_cast<const bf*>(p.k) + row0 * D;
  const bf* vg = static_cast<const bf*>(p.v) + row0 * DV + v0;
  const int16_t* sg = p.src + row0 * D;
  const float* betag = p.beta + row0;
  const float* wg = p.w + row0;
  bf* og = static_cast<bf*>(p.o) + row0 * DV + v0;
  const size_t tokd = (size_t)H * D, tokv = (size_t)H * DV;

  float x[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) x[e] = 0.f;
  if (p.S0) {
    const size_t so = ((size_t)bh * DV + vrow) * D + cg * CPL;
#pragma unroll
    for (int e = 0; e < CPL; e += 4) {
      const float4 s4 = *(const float4*)(p.S0 + so + e);
      x[e] = s4.x;
      x[e + 1] = s4.y;
      x[e + 2] = s4.z;
      x[e + 3] = s4.w;
    }
  }
  float* rbuf = sh.Rb[w][r];
  if (cg == 0) rbuf[D] = 0.f;   // the zero column

  // ---- chunk loads into registers (tokens past T read the last token; the
  // token loop never reaches them), then into LDS
  uint4 rk, rq, rs, rv;
  float rb = 0.f;
  const int pt = tid / PPT, pch = (tid % PPT) * 8;   // piece of k, q, src (tid < NPIECE)
  auto load_chunk = [&](int c) {
    const int c0 = c * L;
    {
      const int t = c0 + (tid < NPIECE ? pt : 0);
      const size_t off = (size_t)(t < T ? t : T - 1) * tokd + (tid < NPIECE ? pch : 0);
      rk = *(const uint4*)(kg + off);
      rq = *(const uint4*)(qg + off);
      rs = *(const uint4*)(sg + off);
    }
    {
      const int t = c0 + ((tid >> 2) & (L - 1));
      rv = *(const uint4*)(vg + (size_t)(t < T ? t : T - 1) * tokv + 8 * (tid & 3));
    }
    {
      const int t = c0 + (tid & (L - 1));
      const size_t off = (size_t)(t < T ? t : T - 1) * H;
      rb = (tid & L) ? wg[off] : betag[off];
    }
  };
  auto fill_lds = [&]() {
    const uint32_t fx[4] = {src_fix(rs.x, D), src_fix(rs.y, D), src_fix(rs.z, D), src_fix(rs.w, D)};
    const unsigned cls = tid < NPIECE ? classify8<D>(fx, pch) : 0u;
    if (tid < NPIECE) {
      const int kq = pt * kq_rs<D>() + pch + (pch / CPL) * kq_pad<D>();
      *(float4*)(sh.Kc + kq) = float4{bf_lo(rk.x), bf_hi(rk.x), bf_lo(rk.y), bf_hi(rk.y)};
      *(float4*)(sh.Kc + kq + 4) = float4{bf_lo(rk.z), bf_hi(rk.z), bf_lo(rk.w), bf_hi(rk.w)};
      *(float4*)(sh.Qc + kq) = float4{bf_lo(rq.x), bf_hi(rq.x), bf_lo(rq.y), bf_hi(rq.y)};
      *(float4*)(sh.Qc + kq + 4) = float4{bf_lo(rq.z), bf_hi(rq.z), bf_lo(rq.w), bf_hi(rq.w)};
      *(uint4*)(sh.Sc + pt * D + pch) = uint4{fx[0], fx[1], fx[2], fx[3]};
    }
    {   // a token's PPT pieces sit in PPT consecutive lanes of one wave
      static_assert(64 % PPT == 0 && NPIECE % 64 == 0, "pieces of a token in one wave");
      const unsigned long long bi = __ballot((cls & 1u) != 0u), bd = __ballot((cls & 2u) != 0u),
                               bu = __ballot((cls & 4u) != 0u);
      const int sh0 = l & ~(PPT - 1);
      const unsigned long long all = (PPT == 64 ? ~0ull : ((1ull << PPT) - 1ull)) << sh0;
      if (tid < NPIECE && (l & (PPT - 1)) == 0) {
        sh.Kind[pt] = (bi & all) == all ? kIdentity
                    : (bd & all) == all ? kDown
                    : (bu & all) == all ? kUp : kGeneral;
      }
    }
    if (tid < 4 * L) *(uint4*)(sh.Vc + (tid >> 2) * ROWS + 8 * (tid & 3)) = rv;
    if (tid < L) sh.Bc[tid] = rb;
    else if (tid < 2 * L) sh.Wc[tid - L] = rb;
  };

  const int nchunks = (T + L - 1) / L;
  load_chunk(0);
  fill_lds();
  if (nchunks > 1) load_chunk(1);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * L;
    const int tn = T - c0 < L ? T - c0 : L;
    // the chunk's map kinds, 2 bits per token, in one scalar register
    unsigned kbits = 0u;
#pragma unroll
    for (int i = 0; i < L; ++i) kbits |= (unsigned)__builtin_amdgcn_readfirstlane(sh.Kind[i]) << (2 * i);
#pragma unroll 1
    for (int t = 0; t < tn; ++t) {
      const int base = t * D + cg * CPL;
      // this token's keys, queries, value and gates first: none depends on the row
      float kf[CPL], qf[CPL];
      const int kqb = t * kq_rs<D>() + cg * (CPL + kq_pad<D>());
#pragma unroll
      for (int e = 0; e < CPL; e += 4) {
        *(float4*)(kf + e) = *(const float4*)(sh.Kc + kqb + e);
        *(float4*)(qf + e) = *(const float4*)(sh.Qc + kqb + e);
      }
      const float vr = (float)sh.Vc[t * ROWS + RPW * w + r];
      const float bt = sh.Bc[t], wt = sh.Wc[t];
      // Each kind of map runs the whole token on its own: the row is read in
      // its selected order and updated in place (a shift writes channel e
      // from channel e -+ 1, highest first for the push), so the four paths
      // leave the row in the same registers and need no merge moves.
      //   y = (S D) . k;  S D + beta (w v - y) k^T;  o = S . q
      float op;
      const int kind = (int)((kbits >> (2 * t)) & 3u);
      if (kind == kIdentity) {
        float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < CPL; ++e) a4[e & 3] += x[e] * kf[e];
        const float coef = bt * (wt * vr - row_sum((a4[0] + a4[1]) + (a4[2] + a4[3])));
        float b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          x[e] += coef * kf[e];
          b4[e & 3] += x[e] * qf[e];
        }
        op = row_sum((b4[0] + b4[1]) + (b4[2] + b4[3]));
      } else if (kind == kDown) {   // channel e takes e - 1; channel 0 empties
        // row_shr:1 -- lane l - 1 holds the channels just below
        const float in = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[CPL - 1]), 0x111, 0xf, 0xf, false));
        const float x0 = cg == 0 ? 0.f : in;
        float a4[4] = {x0 * kf[0], 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 1; e < CPL; ++e) a4[e & 3] += x[e - 1] * kf[e];
        const float coef = bt * (wt * vr - row_sum((a4[0] + a4[1]) + (a4[2] + a4[3])));
        float b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = CPL - 1; e >= 1; --e) {
          x[e] = x[e - 1] + coef * kf[e];
          b4[e & 3] += x[e] * qf[e];
        }
        x[0] = x0 + coef * kf[0];
        b4[0] += x[0] * qf[0];
        op = row_sum((b4[0] + b4[1]) + (b4[2] + b4[3]));
      } else if (kind == kUp) {   // channel e takes e + 1; the last channel empties
        // row_shl:1 -- lane l + 1 holds the channels just above
        const float in = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[0]), 0x101, 0xf, 0xf, false));
        const float xl = cg == 7 ? 0.f : in;
        float a4[4] = {0.f, 0.f, 0.f, xl * kf[CPL - 1]};
#pragma unroll
        for (int e = 0; e < CPL - 1; ++e) a4[e & 3] += x[e + 1] * kf[e];
        const float coef = bt * (wt * vr - row_sum((a4[0] + a4[1]) + (a4[2] + a4[3])));
        float b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < CPL - 1; ++e) {
          x[e] = x[e + 1] + coef * kf[e];
          b4[e & 3] += x[e] * qf[e];
        }
        x[CPL - 1] = xl + coef * kf[CPL - 1];
        b4[3] += x[CPL - 1] * qf[CPL - 1];
        op = row_sum((b4[0] + b4[1]) + (b4[2] + b4[3]));
      } else {   // any other map: through this row's LDS buffer (source D reads the zero)
        uint32_t sw[CPL / 2];
#pragma unroll
        for (int e = 0; e < CPL; e += 8) {
          const uint4 s4 = *(const uint4*)(sh.Sc + base + e);
          sw[e / 2] = s4.x;
          sw[e / 2 + 1] = s4.y;
          sw[e / 2 + 2] = s4.z;
          sw[e / 2 + 3] = s4.w;
        }
#pragma unroll
        for (int e = 0; e < CPL; e += 4)
          *(float4*)(rbuf + cg * CPL + e) = float4{x[e], x[e + 1], x[e + 2], x[e + 3]};
#pragma unroll
        for (int e = 0; e < CPL; ++e) x[e] = rbuf[e & 1 ? sw[e >> 1] >> 16 : sw[e >> 1] & 0xffffu];
        float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < CPL; ++e) a4[e & 3] += x[e] * kf[e];
        const float coef = bt * (wt * vr - row_sum((a4[0] + a4[1]) + (a4[2] + a4[3])));
        float b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          x[e] += coef * kf[e];
          b4[e & 3] += x[e] * qf[e];
        }
        op = row_sum((b4[0] + b4[1]) + (b4[2] + b4[3]));
      }
      if (cg == 0) sh.Oc[t * ROWS + RPW * w + r] = (bf)op;
    }
    __syncthreads();
    if (tid < 4 * tn) {
      const int t = tid >> 2;
      *(uint4*)(og + (size_t)(c0 + t) * tokv + 8 * (tid & 3)) =
          *(const uint4*)(sh.Oc + t * ROWS + 8 * (tid & 3));
    }
    if (c + 1 < nchunks) {
      fill_lds();
      if (c + 2 < nchunks) load_chunk(c + 2);
    }
    __syncthreads();
  }

  if (p.S_out) {
    const size_t so = ((size_t)bh * DV + vrow) * D + cg * CPL;
#pragma unroll
    for (int e = 0; e < CPL; e += 4)
      *(float4*)(p.S_out + so + e) = float4{x[e], x[e + 1], x[e + 2], x[e + 3]};
  }
}

}  // namespace

hipError_t launch_perm_fwd(const PermParams& p, hipStream_t s) {
  const int nvb = p.DV / ROWS;   // DV is a multiple of 32
  const int groups = (p.B * p.H + 7) / 8;
  const dim3 grid(groups * 8 * nvb);
  if (p.DK == 128) {
    hipLaunchKernelGGL(perm_fwd_kernel<128>, grid, dim3(NT), 0, s, p);
  } else if (p.DK == 64) {
    hipLaunchKernelGGL(perm_fwd_kernel<64>, grid, dim3(NT), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace perm
}  // namespace gdr
