// raven_fwd.hip -- Raven routing slot memory, chunked forward for gfx950.
//
// Raven technical summary, sections 2.1 and 2.2: M = 64 slots per head with a
// key state Sk (M x D) and a value state Sv (M x D); per token a sigmoid router
// keeps the top K logits and normalises them (r_t), the selected slots decay by
// lam = exp(a_t r_t) towards the token (S <- lam S + (1 - lam) x), unselected
// slots stay frozen, and the output is attention over the slots after the update.
//
// One workgroup of 4 waves per (b, h) walks the sequence in 32-token chunks.
// Within a chunk, with P[t][i] the product of slot i's factors lam over tokens
// 0..t of the chunk (1 where the slot is not selected), P(s,t] = P[t] / P[s]
// the product over s < u <= t, and om[s][i] = 1 - lam_s[i]:
//
//   Sk_t[i] . q_t = P[t][i] (q_t . Sk_0[i]) + sum_{s<=t} om[s][i] P(s,t][i] (q_t . k_s)
//   o_t = sum_i p[t][i] P[t][i] Sv_0[i] + sum_{s<=t} A[t][s] v_s,
//         A[t][s] = sum_i p[t][i] om[s][i] P(s,t][i]
//   S_end[i] = P[end][i] S_0[i] + sum_s om[s][i] P(s,end][i] x_s
//
// Where every slot's product over the chunk stays above e^-40, P(s,t] splits
// into P[t] (om[s] / P[s]) and all three sums are products on the matrix cores;
// otherwise the chunk forms the two token-pair sums with running products of
// the factors (exact, VALU).  Products, not sums of log-decays: after a factor
// of 0 (a replaced slot) a sum would absorb the later, milder decays.  The
// chunk-end update uses the suffix products P(s,end] <= 1, split into a bf16
// pair so that the fp32 slot state keeps fp32 accuracy.
//
// Both states stay in MFMA accumulators for the whole sequence: wave w holds
// Sk^T for slots 16w..16w+15 (all channels; the accumulators feed q . Sk
// directly as the B operand) and Sv for channels (D/4)w.. (all slots; they feed
// p . Sv the same way).
//
// Routing: lane (token t, group of 8 slots) sorts its 8 keys (the bf16 logit in
// an order-preserving 16-bit code above 0xffff - slot, so that equal logits go
// to the lower slot) with a 19-comparator network, then three DPP exchanges
// inside the 8 lanes of the token merge the sorted lists to the top 8 of all 64.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_mfma.h"
#include "raven_kernels.h"

namespace gdr {
namespace raven {
namespace {

using bf = __bf16;
constexpr int L = 32;        // tokens per chunk
constexpr int M = kSlots;    // 64
constexpr int NT = 256;      // 4 waves
constexpr float kSplitMin = 4.2483543e-18f;   // e^-40: smallest chunk product for the split form

template <int D>
struct Sh {
  static constexpr int RQ = D + 8;   // bf16 rows [t][ch]
  static constexpr int RT = L + 8;   // bf16 rows [x][t]
  static constexpr int RF = M + 4;   // fp32 rows [t][slot]
  static constexpr int RM = M + 8;   // bf16 rows [t][slot]
  static constexpr int RK = L + 4;   // fp32 rows [t][s]
  bf Qs[L * RQ];
  bf Ks[L * RQ];
  bf Kt[D * RT];        // keys as [channel][token]
  bf Vt[D * RT];        // values as [channel][token]
  bf Os[L * RQ];        // output staging
  bf Zs[L * M];         // router logits [t][slot]
  float As[L];          // decay rate per token
  float lam[L * RF];    // a_t r_t[i] (0: not selected) from the router, then e^(a_t r_t[i])
  float Lc[L * RF];     // P[t][i], the product through token t
  float G[L * RF];      // q_t . Sk_0[i]; then the logits; then the softmax
  float QKf[L * RK];    // q_t . k_s, s <= t (0 above)
  bf QKm[L * RT];
  bf Bis[M * RT];       // om / P as [slot][token]
  bf Bsi[L * RM];       // the same as [token][slot]
  bf Ehi[M * RT];       // om P(s,end] as [slot][token], high and low bf16 parts
  bf Elo[M * RT];
  bf PL[L * RM];        // p P  [t][slot]
  bf Ab[L * RT];        // A  [t][s]
  float Lend[M];        // P[end]
  int sel[L * 8];       // selected slots of each token, by rank
  int flag;             // a slot leaves the split form's range in this chunk
};

__device__ inline unsigned dpp_u(unsigned x, int ctrl) {
  int r;
  if (ctrl == 0xb1) r = __builtin_amdgcn_mov_dpp((int)x, 0xb1, 0xf, 0xf, false);        // lane ^ 1
  else if (ctrl == 0x4e) r = __builtin_amdgcn_mov_dpp((int)x, 0x4e, 0xf, 0xf, false);   // lane ^ 2
  else r = __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xf, 0xf, false);                    // 7 - lane in 8
  return (unsigned)r;
}
__device__ inline float dpp_f(float x, int ctrl) { return __uint_as_float(dpp_u(__float_as_uint(x), ctrl)); }

// order-preserving code of a bf16 value (-0 taken as +0), above 0xffff - slot
__device__ inline unsigned route_key(unsigned u16, int slot) {
  u16 &= 0xffffu;
  if (u16 == 0x8000u) u16 = 0u;
  const unsigned ord = (u16 & 0x8000u) ? (~u16 & 0xffffu) : (u16 | 0x8000u);
  return (ord << 16) | (0xffffu - (unsigned)slot);
}
__device__ inline int key_slot(unsigned key) { return (int)(0xffffu - (key & 0xffffu)); }

__device__ inline void ce(unsigned& a, unsigned& b) {   // a >= b after
  const unsigned hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}
__device__ inline void sort8_desc(unsigned (&x)[8]) {
  ce(x[0], x[1]); ce(x[2], x[3]); ce(x[4], x[5]); ce(x[6], x[7]);
  ce(x[0], x[2]); ce(x[1], x[3]); ce(x[4], x[6]); ce(x[5], x[7]);
  ce(x[1], x[2]); ce(x[5], x[6]); ce(x[0], x[4]); ce(x[3], x[7]);
  ce(x[1], x[5]); ce(x[2], x[6]);
  ce(x[1], x[4]); ce(x[3], x[6]);
  ce(x[2], x[4]); ce(x[3], x[5]);
  ce(x[3], x[4]);
}
// top 8 of this lane's sorted list and its partner's (both descending)
__device__ inline void merge8(unsigned (&x)[8], int ctrl) {
  unsigned y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = dpp_u(x[j], ctrl);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = x[j] > y[7 - j] ? x[j] : y[7 - j];   // bitonic
  ce(x[0], x[4]); ce(x[1], x[5]); ce(x[2], x[6]); ce(x[3], x[7]);
  ce(x[0], x[2]); ce(x[1], x[3]); ce(x[4], x[6]); ce(x[5], x[7]);
  ce(x[0], x[1]); ce(x[2], x[3]); ce(x[4], x[5]); ce(x[6], x[7]);
}

// component-wise (a select of the whole struct goes through the stack)
__device__ inline uint4 keep_if(bool ok, const uint4& x) {
  return uint4{ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u};
}

__device__ inline float sigm(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void raven_fwd_kernel(RavenParams p) {
  using O = Op<bf>;
  using S = Sh<D>;
  constexpr int RQ = S::RQ, RT = S::RT, RF = S::RF, RM = S::RM, RK = S::RK;
  constexpr int NCT = D / 16;       // channel tiles of Sk^T held by each wave
  constexpr int VCT = D / 64;       // value-channel tiles of Sv held by each wave
  constexpr int CW = D / 4;         // value channels per wave
  constexpr int PPT = D / 8;        // 16-byte pieces per token row
  constexpr int NPAIR = 16 * PPT;   // (token pair, 8-channel block) units of a chunk
  __shared__ __attribute__((aligned(16))) S sh;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, n = l & 15, g = l >> 4;
  const int bh = blockIdx.x, b = bh / p.H, h = bh % p.H;
  const int T = p.T, H = p.H, K = p.topk;
  const size_t row0 = (size_t)b * T * H + h;          // (b, t = 0, h)
  const size_t tok = (size_t)H * D;                   // token stride of q, k, v, o
  const bf* qg = static_cast<const bf*>(p.q) + row0 * D;
  const bf* kg = static_cast<const bf*>(p.k) + row0 * D;
  const bf* vg = static_cast<const bf*>(p.v) + row0 * D;
  const bf* zg = static_cast<const bf*>(p.z) + row0 * M;
  const float* ag = p.a + row0;
  bf* og = static_cast<bf*>(p.o) + row0 * D;
  const int nchunks = (T + L - 1) / L;

  // ---- slot states in accumulators
  f32x4 SkT[NCT];       // rows: channels 16ct + 4g + j; columns: slots 16w + n
  f32x4 Sv[4][VCT];     // rows: slots 16st + 4g + j; columns: channels CW w + 16vt + n
  {
    const size_t sb = (size_t)bh * M * D;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      SkT[ct] = p.Sk0 ? *(const f32x4*)(p.Sk0 + sb + (size_t)(16 * w + n) * D + 16 * ct + 4 * g)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int vt = 0; vt < VCT; ++vt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          Sv[st][vt][j] = p.Sv0 ? p.Sv0[sb + (size_t)(16 * st + 4 * g + j) * D + CW * w + 16 * vt + n] : 0.f;
  }

  // ---- raw chunk loads (registers), then into LDS.  Lane (tid < NPAIR) takes
  // tokens 2tp, 2tp + 1 of channels 8cb .. 8cb + 7, so that the transposed
  // copies are written as whole dwords (two tokens of one channel).
  // Tokens past T load from the last token (a valid address, so that no
  // select waits on the load here) and are zeroed when written to LDS.
  uint4 rq[2], rk[2], rv[2], rz;
  float ra = 0.f;
  unsigned okm = 0u;   // bit u: token 2tp + u valid; bit 2: router row valid; bit 3: rate valid
  const int tp = tid & 15, cb = tid >> 4;
  const int cbl = tid < NPAIR ? cb : 0;
  auto load_chunk = [&](int c) {
    const int c0 = c * L;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = c0 + 2 * tp + u;
      okm = (okm & ~(1u << u)) | ((tid < NPAIR && t < T) ? 1u << u : 0u);
      const size_t off = (size_t)(t < T ? t : T - 1) * tok + 8 * cbl;
      rq[u] = *(const uint4*)(qg + off);
      rk[u] = *(const uint4*)(kg + off);
      rv[u] = *(const uint4*)(vg + off);
    }
    {
      const int t = c0 + (tid >> 3), s8 = (tid & 7) * 8;
      okm = (okm & ~4u) | (t < T ? 4u : 0u);
      rz = *(const uint4*)(zg + (size_t)(t < T ? t : T - 1) * H * M + s8);
    }
    {
      const int t = c0 + (tid & (L - 1));
      okm = (okm & ~8u) | ((tid < L && t < T) ? 8u : 0u);
      ra = ag[(size_t)(t < T ? t : T - 1) * H];
    }
  };
  auto fill_lds = [&]() {
    if (tid < NPAIR) {
      const int ch = 8 * cb;
      const bool ok0 = okm & 1u, ok1 = okm & 2u;
      const uint4 q0 = keep_if(ok0, rq[0]), q1 = keep_if(ok1, rq[1]);
      const uint4 ka = keep_if(ok0, rk[0]), kb = keep_if(ok1, rk[1]);
      const uint4 va = keep_if(ok0, rv[0]), vb = keep_if(ok1, rv[1]);
      *(uint4*)(sh.Qs + (2 * tp) * RQ + ch) = q0;
      *(uint4*)(sh.Qs + (2 * tp + 1) * RQ + ch) = q1;
      *(uint4*)(sh.Ks + (2 * tp) * RQ + ch) = ka;
      *(uint4*)(sh.Ks + (2 * tp + 1) * RQ + ch) = kb;
      const uint32_t k0[4] = {ka.x, ka.y, ka.z, ka.w};
      const uint32_t k1[4] = {kb.x, kb.y, kb.z, kb.w};
      const uint32_t v0[4] = {va.x, va.y, va.z, va.w};
      const uint32_t v1[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {   // channels ch + 2e (low halves) and ch + 2e + 1 (high)
        *(uint32_t*)(sh.Kt + (ch + 2 * e) * RT + 2 * tp) = (k0[e] & 0xffffu) | (k1[e] << 16);
        *(uint32_t*)(sh.Kt + (ch + 2 * e + 1) * RT + 2 * tp) = (k0[e] >> 16) | (k1[e] & 0xffff0000u);
        *(uint32_t*)(sh.Vt + (ch + 2 * e) * RT + 2 * tp) = (v0[e] & 0xffffu) | (v1[e] << 16);
        *(uint32_t*)(sh.Vt + (ch + 2 * e + 1) * RT + 2 * tp) = (v0[e] >> 16) | (v1[e] & 0xffff0000u);
      }
    }
    *(uint4*)(sh.Zs + (tid >> 3) * M + (tid & 7) * 8) = keep_if(okm & 4u, rz);
    if (tid < L) sh.As[tid] = (okm & 8u) ? ra : 0.f;
  };

  load_chunk(0);
  fill_lds();
  if (tid == 0) sh.flag = 0;
  if (nchunks > 1) load_chunk(1);
  lds_barrier();

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * L;
    // ---------------- routing: lane = (token t, slots 8 g8 .. 8 g8 + 7)
    {
      const int t = tid >> 3, g8 = tid & 7;
      const uint4 zz = *(const uint4*)(sh.Zs + t * M + 8 * g8);
      const uint32_t zw[4] = {zz.x, zz.y, zz.z, zz.w};
      unsigned own[8], top[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        own[e] = route_key(e & 1 ? zw[e >> 1] >> 16 : zw[e >> 1], 8 * g8 + e);
        top[e] = own[e];
      }
      sort8_desc(top);
      merge8(top, 0xb1);
      merge8(top, 0x4e);
      merge8(top, 0x141);
      unsigned thr = top[0];
      int mine = -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j == K - 1) thr = top[j];
        if (j == g8) mine = j < K ? key_slot(top[j]) : -1;
      }
      // sigmoid of each own slot; the selected ones' sum over the token's 8 lanes
      float sg[8], part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (e & 1 ? zw[e >> 1] >> 16 : zw[e >> 1]) & 0xffffu;
        sg[e] = sigm(__uint_as_float(bits << 16));
        part += own[e] >= thr ? sg[e] : 0.f;
      }
      part += dpp_f(part, 0xb1);
      part += dpp_f(part, 0x4e);
      part += dpp_f(part, 0x141);
      const float at = sh.As[t];
      const float inv = __builtin_amdgcn_rcpf(part);
      float lv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) lv[e] = own[e] >= thr ? at * (sg[e] * inv) : 0.f;
      *(f32x4*)(sh.lam + t * RF + 8 * g8) = f32x4{lv[0], lv[1], lv[2], lv[3]};
      *(f32x4*)(sh.lam + t * RF + 8 * g8 + 4) = f32x4{lv[4], lv[5], lv[6], lv[7]};
      sh.sel[t * 8 + g8] = mine;
    }
    // ---------------- q . Sk_0 (accumulators as the B operand) and q . k
    {
      typename O::frag skb[D / 32];
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) skb[ks] = O::from_acc(SkT[2 * ks], SkT[2 * ks + 1]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) O::mma(acc, load_cb<bf>(sh.Qs, RQ, 16 * tt, 32 * ks), skb[ks]);
#pragma unroll
      for (int j = 0; j < 4; ++j) sh.G[(16 * tt + 4 * g + j) * RF + 16 * w + n] = acc[j];
    }
    }
    {
      const int tt = w == 0 ? 0 : 1, st = w == 2 ? 1 : 0;   // tiles (0,0) (1,0) (1,1); wave 3: (0,1)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (w < 3) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          O::mma(acc, load_plain<bf>(sh.Qs, RQ, 16 * tt, 32 * ks), load_plain<bf>(sh.Ks, RQ, 16 * st, 32 * ks));
      }
      const int ttw = w < 3 ? tt : 0, stw = w < 3 ? st : 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * ttw + 4 * g + j, s = 16 * stw + n;
        const float m = s <= t ? acc[j] : 0.f;
        sh.QKf[t * RK + s] = m;
        sh.QKm[t * RT + s] = (bf)m;
      }
    }
    lds_barrier();
    // ---------------- factors and their products: lane = (slot i, tokens 8qq .. 8qq + 7)
    {
      const int i = 16 * w + n, qq = g;
      float lm[8], fp[8], sp[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) lm[u] = __expf(sh.lam[(8 * qq + u) * RF + i]);
      float run = 1.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        run *= lm[u];
        fp[u] = run;   // product over this quarter's tokens through u
      }
      sp[7] = 1.f;
#pragma unroll
      for (int u = 6; u >= 0; --u) sp[u] = sp[u + 1] * lm[u + 1];   // over u+1 .. 7
      const float q0 = __shfl(run, n), q1 = __shfl(run, n + 16), q2 = __shfl(run, n + 32),
                  q3 = __shfl(run, n + 48);
      const float e2 = q0 * q1, e3 = e2 * q2, pend = e3 * q3;
      const float pre = qq == 0 ? 1.f : qq == 1 ? q0 : qq == 2 ? e2 : e3;
      const float q23 = q2 * q3;
      const float post = qq == 3 ? 1.f : qq == 2 ? q3 : qq == 1 ? q23 : q1 * q23;
      bf16x8 eh, el, bb;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = 8 * qq + u;
        const float lc = pre * fp[u];
        const float om = 1.f - lm[u];
        sh.lam[t * RF + i] = lm[u];
        sh.Lc[t * RF + i] = lc;
        const float e = om * (sp[u] * post);
        const bf ehi = (bf)e;
        eh[u] = ehi;
        el[u] = (bf)(e - (float)ehi);
        const bf bs = (bf)(om * __builtin_amdgcn_rcpf(lc));   // used only where pend >= e^-40
        bb[u] = bs;
        sh.Bsi[t * RM + i] = bs;
      }
      *(bf16x8*)(sh.Ehi + i * RT + 8 * qq) = eh;
      *(bf16x8*)(sh.Elo + i * RT + 8 * qq) = el;
      *(bf16x8*)(sh.Bis + i * RT + 8 * qq) = bb;
      if (qq == 0) sh.Lend[i] = pend;
      if (qq == 3 && !(pend >= kSplitMin)) sh.flag = 1;
    }
    lds_barrier();
    const bool split = sh.flag == 0;
    // ---------------- logits
    if (split) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        O::mma(y, load_plain<bf>(sh.QKm, RT, 16 * tt, 0), load_plain<bf>(sh.Bis, RT, 16 * w, 0));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int idx = (16 * tt + 4 * g + j) * RF + 16 * w + n;
          sh.G[idx] = p.scale * (sh.Lc[idx] * (sh.G[idx] + y[j]));
        }
      }
    } else {
      // exact: from s = t down to 0, pr = P(s,t] (running product), then P[t]
      const int t = l & 31, i0 = 16 * w + 8 * (l >> 5);
#pragma unroll 1
      for (int e = 0; e < 8; ++e) {
        const int i = i0 + e;
        float x = 0.f, pr = 1.f;
#pragma unroll 4
        for (int s = L - 1; s >= 0; --s) {
          const float lm = sh.lam[s * RF + i];
          if (s <= t) {
            x += (1.f - lm) * pr * sh.QKf[t * RK + s];
            pr *= lm;
          }
        }
        sh.G[t * RF + i] = p.scale * (x + pr * sh.G[t * RF + i]);
      }
    }
    lds_barrier();
    // ---------------- softmax over the slots: lane = (token t, 8 slots)
    {
      const int t = tid >> 3, g8 = tid & 7;
      const f32x4 xa = *(const f32x4*)(sh.G + t * RF + 8 * g8);
      const f32x4 xb = *(const f32x4*)(sh.G + t * RF + 8 * g8 + 4);
      float x[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = fmaxf(mx, dpp_f(mx, 0xb1));
      mx = fmaxf(mx, dpp_f(mx, 0x4e));
      mx = fmaxf(mx, dpp_f(mx, 0x141));
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = __expf(x[e] - mx);
        sum += x[e];
      }
      sum += dpp_f(sum, 0xb1);
      sum += dpp_f(sum, 0x4e);
      sum += dpp_f(sum, 0x141);
      const float inv = __builtin_amdgcn_rcpf(sum);
      bf16x8 pl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] *= inv;
        pl[e] = (bf)(x[e] * sh.Lc[t * RF + 8 * g8 + e]);
      }
      *(f32x4*)(sh.G + t * RF + 8 * g8) = f32x4{x[0], x[1], x[2], x[3]};
      *(f32x4*)(sh.G + t * RF + 8 * g8 + 4) = f32x4{x[4], x[5], x[6], x[7]};
      *(bf16x8*)(sh.PL + t * RM + 8 * g8) = pl;
    }
    lds_barrier();
    // ---------------- A[t][s]
    if (split) {
      const int tt = w == 0 ? 0 : 1, st = w == 2 ? 1 : 0;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (w < 3) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          O::mma(acc, load_plain<bf>(sh.PL, RM, 16 * tt, 32 * ks), load_plain<bf>(sh.Bsi, RM, 16 * st, 32 * ks));
      }
      const int ttw = w < 3 ? tt : 0, stw = w < 3 ? st : 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * ttw + 4 * g + j, s = 16 * stw + n;
        sh.Ab[t * RT + s] = (bf)(s <= t ? acc[j] : 0.f);
      }
    } else {
      const int t = tid >> 3, s0 = 4 * (tid & 7);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + u;
        float acc = 0.f;
        if (s <= t) {
#pragma unroll 1
          for (int kk = 0; kk < K; ++kk) {
            const int i = sh.sel[s * 8 + kk];
            float pr = 1.f;   // P(s,t]
#pragma unroll 1
            for (int u = s + 1; u <= t; ++u) pr *= sh.lam[u * RF + i];
            acc += sh.G[t * RF + i] * ((1.f - sh.lam[s * RF + i]) * pr);
          }
        }
        sh.Ab[t * RT + s] = (bf)acc;
      }
    }
    lds_barrier();
    // ---------------- output (old Sv in the accumulators as the B operand)
    typename O::frag svb[2][VCT];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int vt = 0; vt < VCT; ++vt) svb[ks][vt] = O::from_acc(Sv[2 * ks][vt], Sv[2 * ks + 1][vt]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int vt = 0; vt < VCT; ++vt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) O::mma(acc, load_cb<bf>(sh.PL, RM, 16 * tt, 32 * ks), svb[ks][vt]);
        O::mma(acc, load_plain<bf>(sh.Ab, RT, 16 * tt, 0), load_plain<bf>(sh.Vt, RT, CW * w + 16 * vt, 0));
#pragma unroll
        for (int j = 0; j < 4; ++j) sh.Os[(16 * tt + 4 * g + j) * RQ + CW * w + 16 * vt + n] = (bf)acc[j];
      }
    }
    // ---------------- slot states to the chunk end
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const f32x4 le = *(const f32x4*)(sh.Lend + 16 * st + 4 * g);
      const auto eh = load_plain<bf>(sh.Ehi, RT, 16 * st, 0);
      const auto el = load_plain<bf>(sh.Elo, RT, 16 * st, 0);
#pragma unroll
      for (int vt = 0; vt < VCT; ++vt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) Sv[st][vt][j] *= le[j];
        const auto vb = load_plain<bf>(sh.Vt, RT, CW * w + 16 * vt, 0);
        O::mma(Sv[st][vt], eh, vb);
        O::mma(Sv[st][vt], el, vb);
      }
    }
    {
      const float le = sh.Lend[16 * w + n];
      const auto eh = load_plain<bf>(sh.Ehi, RT, 16 * w, 0);
      const auto el = load_plain<bf>(sh.Elo, RT, 16 * w, 0);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int j = 0; j < 4; ++j) SkT[ct][j] *= le;
        const auto kb = load_plain<bf>(sh.Kt, RT, 16 * ct, 0);
        O::mma(SkT[ct], kb, eh);
        O::mma(SkT[ct], kb, el);
      }
    }
    lds_barrier();
    // ---------------- o stores; next chunk into LDS; loads of the one after
    {
      const int t = tid >> 3, pc = tid & 7;
      constexpr int CPL = D / 8;   // channels per lane
      if (c0 + t < T) {
#pragma unroll
        for (int u = 0; u < CPL / 8; ++u)
          *(uint4*)(og + (size_t)(c0 + t) * tok + pc * CPL + 8 * u) =
              *(const uint4*)(sh.Os + t * RQ + pc * CPL + 8 * u);
      }
    }
    if (c + 1 < nchunks) {
      fill_lds();
      if (c + 2 < nchunks) load_chunk(c + 2);
    }
    if (tid == 0) sh.flag = 0;
    lds_barrier();
  }

  // ---- final states
  const size_t sb = (size_t)bh * M * D;
  if (p.Sk_out) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      *(f32x4*)(p.Sk_out + sb + (size_t)(16 * w + n) * D + 16 * ct + 4 * g) = SkT[ct];
  }
  if (p.Sv_out) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int vt = 0; vt < VCT; ++vt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          p.Sv_out[sb + (size_t)(16 * st + 4 * g + j) * D + CW * w + 16 * vt + n] = Sv[st][vt][j];
  }
}

}  // namespace

hipError_t launch_raven_fwd(const RavenParams& p, hipStream_t s) {
  if (p.D == 128) {
    hipLaunchKernelGGL(raven_fwd_kernel<128>, dim3(p.B * p.H), dim3(NT), 0, s, p);
  } else if (p.D == 64) {
    hipLaunchKernelGGL(raven_fwd_kernel<64>, dim3(p.B * p.H), dim3(NT), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace raven
}  // namespace gdr
