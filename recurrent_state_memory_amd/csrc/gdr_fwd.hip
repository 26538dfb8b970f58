// gdr_fwd.hip -- fused chunk-parallel (WY-form) gated delta-rule forward for gfx950.
//
// One workgroup owns one (batch b, head h, value tile) and walks the sequence
// chunk by chunk, keeping its rows of the state S in matrix-core accumulators
// (fp32) for the whole sequence.  Value rows of S evolve independently because
// every gate acts on the key axis (CARVE technical summary, section 2.3 and
// section 3 item 1), so a value tile needs nothing from the other tiles.
//
// Per chunk of L tokens (r = 0..L-1) with start state S0 and running products
// Gamma_r of the key-axis transitions, the chunk-WY algebra is
//   K+ = Gamma_r k_r, Q+ = Gamma_r q_r, Kh = Gamma_r^{-T} k_r, K- = Gamma_L^T Kh
//   A  = strict_lower(diag(beta) K+ Kh^T),   M = lower_incl(Q+ Kh^T)
//   W  = (I + A)^{-1} diag(beta) K+,         U = (I + A)^{-1} diag(beta w) V
//   Dl = U - W S0^T,   O = Q+ S0^T + M Dl,   S_L = S0 Gamma_L + Dl^T K-
// (CARVE technical summary, section 1.3: one triangular system per chunk;
// SFDA technical summary, constructive chunk-WY theorem and the exact affine
// chunk transfer).  Stages inside the chunk loop:
//   P  load q, k, transition and gates; running products of the transitions
//      (per-channel decay, or complex products for 2x2 rotation-decay blocks);
//      decayed forms K+, Kh, Q+, K-^T into LDS.
//   G  Gram tiles A and M on the matrix cores.
//   D  16x16 diagonal blocks of (I + A)^{-1} by forward substitution (fp32).
//   WU W and U by blocked forward substitution over 16-token blocks, with the
//      off-diagonal updates on the matrix cores; W to LDS, U stays in registers.
//   S  Dl, O and the state update on the matrix cores; o to HBM.
// With the content-aware erase (CARVE technical summary, section 2.1), the
// workgroup covers all value channels, so at each window boundary it reduces
// its own fp32 outputs to the window mean m and forms the next window's erase
// gates sigmoid(b_x + u_h . m) with u_h = B_h^T a_h.
#include "gdr_kernels.h"
#include "gdr_mfma.h"
#include "gdr_token.h"

namespace gdr {

__device__ inline f32x2 cmul(f32x2 a, f32x2 b) {
  f32x2 r;
  r.x = a.x * b.x - a.y * b.y;
  r.y = a.x * b.y + a.y * b.x;
  return r;
}

template <typename T>
struct Pair;
template <>
struct Pair<__bf16> {
  static __device__ inline f32x2 load(const __bf16* p) {
    bf16x2 v = *(const bf16x2*)p;
    f32x2 r = {(float)v[0], (float)v[1]};
    return r;
  }
  static __device__ inline void store(__bf16* p, f32x2 x) {
    bf16x2 v;
    v[0] = (__bf16)x.x;
    v[1] = (__bf16)x.y;
    *(bf16x2*)p = v;
  }
};
template <>
struct Pair<float> {
  static __device__ inline f32x2 load(const float* p) { return *(const f32x2*)p; }
  static __device__ inline void store(float* p, f32x2 x) { *(f32x2*)p = x; }
};

template <typename T>
__device__ inline void store4(T* p, const float (&x)[4]);
template <>
__device__ inline void store4<__bf16>(__bf16* p, const float (&x)[4]) {
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (__bf16)x[i];
  *(bf16x4*)p = v;
}
template <>
__device__ inline void store4<float>(float* p, const float (&x)[4]) {
  f32x4 v = {x[0], x[1], x[2], x[3]};
  *(f32x4*)p = v;
}


// Raw (unconverted) inputs of one chunk for one thread, loaded without
// branches (token indices are clamped; invalid tokens are masked on use).
template <typename T>
struct RawPair;
template <>
struct RawPair<__bf16> {
  using type = uint32_t;
  static __device__ inline uint32_t load(const __bf16* p) { return *(const uint32_t*)p; }
  static __device__ inline f32x2 cvt(uint32_t u) {
    return f32x2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
  }
};
template <>
struct RawPair<float> {
  using type = f32x2;
  static __device__ inline f32x2 load(const float* p) { return *(const f32x2*)p; }
  static __device__ inline f32x2 cvt(f32x2 u) { return u; }
};

template <typename T, int TPS, int NVL>
struct RawChunk {
  typename RawPair<T>::type k[TPS], q[TPS];
  f32x2 a[TPS];   // per-channel decay: the alpha pair; rotation: (gamma, theta)
  uint4 v[NVL];   // 16-byte pieces of the value tile
  float bt, wt;   // erase strength (or its logit) and write gate of token tid
};

template <typename T, int DK, int L, int TV, int DECAY, bool CONTENT, typename Raw>
__device__ inline void load_raw(Raw& R, const FwdParams& p, int c0, int pp, int seg, int tid,
                                int b, int h, int v0) {
  constexpr int NP = DK / 2, NT = TV / 16 * 64;
  constexpr int NSEG0 = NT / NP;
  constexpr int NSEG = NSEG0 < L / 4 ? NSEG0 : L / 4;
  constexpr int TPS = L / NSEG;
  constexpr int VEC = 16 / sizeof(T), VPR = TV / VEC;
  const int Tn = p.T, H = p.H, DV = p.DV;
  const T* gk = (const T*)p.k;
  const T* gq = (const T*)p.q;
  const T* gv = (const T*)p.v;
#pragma unroll
  for (int r = 0; r < TPS; ++r) {
    int t = c0 + seg * TPS + r;
    t = t < Tn ? t : Tn - 1;
    const size_t base = (size_t)(b * Tn + t) * H + h;
    R.k[r] = RawPair<T>::load(gk + base * DK + 2 * pp);
    R.q[r] = RawPair<T>::load(gq + base * DK + 2 * pp);
    if constexpr (DECAY == 0) {
      R.a[r] = *(const f32x2*)(p.alpha + base * DK + 2 * pp);
    } else {
      R.a[r] = f32x2{p.alpha[base * NP + pp], p.theta[base * NP + pp]};
    }
  }
#pragma unroll
  for (int i = 0; i < (int)(sizeof(R.v) / sizeof(R.v[0])); ++i) {
    int idx = tid + i * NT;
    idx = idx < L * VPR ? idx : 0;
    const int r = idx / VPR, cc = idx % VPR;
    int t = c0 + r;
    t = t < Tn ? t : Tn - 1;
    R.v[i] = *(const uint4*)(gv + ((size_t)(b * Tn + t) * H + h) * DV + v0 + cc * VEC);
  }
  {
    int t = c0 + (tid < L ? tid : L - 1);
    t = t < Tn ? t : Tn - 1;
    const size_t gi = (size_t)(b * Tn + t) * H + h;
    R.bt = CONTENT ? p.beta_logit[gi] : p.beta[gi];
    R.wt = p.w[gi];
  }
}

template <typename T, int DK, int L, int TV, int DECAY, bool CONTENT>
struct FwdCfg {
  static constexpr int NW = TV / 16;             // waves; wave w owns value block w
  static constexpr int NT = NW * 64;
  static constexpr int NB = L / 16;              // 16-token blocks per chunk
  static constexpr int NP = DK / 2;              // channel pairs
  static constexpr int NSEG0 = NT / NP;
  static constexpr int NSEG = NSEG0 < L / 4 ? NSEG0 : L / 4;   // token segments in prep
  static constexpr int TPS = L / NSEG;           // tokens per prep thread
  static constexpr int RSK = DK + 8;             // row stride of [L][DK] arrays
  static constexpr int RSL = L + 4;              // row stride of [.][L] arrays
  static constexpr int RST = 20;                 // row stride of 16x16 diagonal blocks
  static constexpr int RSV = TV + 8;             // row stride of the V tile
  static constexpr int NCT = DK / 16;            // key-channel tiles
  static constexpr int NKC = DK / 32;            // 32-wide steps over key channels
  static constexpr int NKT = (NB + 1) / 2;       // 32-wide steps over tokens
  static constexpr int NCW = NCT / NW;           // W channel tiles per wave
  static constexpr int NVL0 = (L * (int)sizeof(T) + 63) / 64;
  static constexpr int NVL = NVL0 < 1 ? 1 : NVL0;  // 16-byte value loads per thread
  static_assert(TV % 16 == 0 && NCT % NW == 0, "tile split");
  static_assert(NSEG >= 1 && TPS % 4 == 0, "prep split");
  static constexpr size_t LDS =
      sizeof(T) * (3ull * L * RSK + (size_t)DK * RSL + 2ull * L * RSL + NB * 16ull * RST +
                   (size_t)L * RSV) +
      4ull * (NB * 16 * 17 + 2 * L) + 8ull * (NP + NSEG * NP) +
      (CONTENT ? 4ull * (2 * TV + 2 * 64) : 0);
  static_assert(LDS <= 160 * 1024, "LDS budget of one gfx950 CU");
};

template <typename T, int DK, int L, int TV, int DECAY, bool CONTENT>
__global__ __launch_bounds__(TV / 16 * 64) void gdr_fwd_kernel(FwdParams p) {
  using C = FwdCfg<T, DK, L, TV, DECAY, CONTENT>;
  using O = Op<T>;
  using frag = typename O::frag;
  constexpr int NW = C::NW, NT = C::NT, NB = C::NB, NP = C::NP, NSEG = C::NSEG,
                TPS = C::TPS, RSK = C::RSK, RSL = C::RSL, RST = C::RST, RSV = C::RSV,
                NCT = C::NCT, NKC = C::NKC, NKT = C::NKT, NCW = C::NCW;

  __shared__ __attribute__((aligned(16))) T sKp[L * RSK];
  // Kh (reused for W after stage G) and K-^T, contiguous: a chunk that takes the
  // token path keeps its fp32 transition [L][DK] there instead
  __shared__ __attribute__((aligned(16))) T sKhKm[L * RSK + DK * RSL];
  static_assert(sizeof(T) * (L * RSK + DK * RSL) >= sizeof(float) * L * DK, "raw transition");
  T* const sKh = sKhKm;
  T* const sKmT = sKhKm + L * RSK;
  __shared__ __attribute__((aligned(16))) T sQp[L * RSK];
  __shared__ __attribute__((aligned(16))) T sA[L * RSL];
  __shared__ __attribute__((aligned(16))) T sM[L * RSL];
  __shared__ __attribute__((aligned(16))) T sTd[NB * 16 * RST];
  __shared__ __attribute__((aligned(16))) T sV[L * RSV];
  __shared__ float sAd[NB * 16 * 17];
  __shared__ float sBeta[L];
  __shared__ float sBW[L];
  __shared__ f32x2 sGL[NP];
  __shared__ f32x2 sSeg[NSEG * NP];
  __shared__ float sU[CONTENT ? TV : 1];      // u_h = B_h^T a_h
  __shared__ float sMean[CONTENT ? TV : 1];   // previous window's mean output
  __shared__ float sRed[CONTENT ? 64 : 1];
  __shared__ float sS[CONTENT ? 64 : 1];
  __shared__ int sFlag[NW];   // per wave: a channel's chunk decay leaves the split form's range

  const int tid = threadIdx.x;
  const int l = tid & 63, wv = tid >> 6;
  const int n = l & 15, g = l >> 4;

  // XCD-aware placement: consecutive workgroup ids go to different XCDs, so
  // the value tiles of one (b, h) get ids 8 apart and share an XCD's L2.
  const int nvt = p.n_vt;
  const int grp = blockIdx.x / (8 * nvt), rem = blockIdx.x % (8 * nvt);
  const int unit = grp * 8 + (rem & 7);
  const int vt = rem >> 3;
  if (unit >= p.n_units) return;
  const int b = unit / p.H, h = unit % p.H;
  const int v0 = vt * TV;
  const int Tn = p.T, H = p.H, DV = p.DV;

  const T* __restrict__ gq = (const T*)p.q;
  const T* __restrict__ gk = (const T*)p.k;
  const T* __restrict__ gv = (const T*)p.v;
  T* __restrict__ go = (T*)p.o;

  // Upper blocks of A and M are never written by stage G; zero them once.
  for (int idx = tid; idx < L * L; idx += NT) {
    const int r = idx / L, cc = idx % L;
    if ((cc >> 4) > (r >> 4)) {
      sA[r * RSL + cc] = (T)0.0f;
      sM[r * RSL + cc] = (T)0.0f;
    }
  }

  // State rows v0 + 16 wv + n, as transposed accumulator tiles:
  // Sacc[ct][j] = S[v][16 ct + 4 g + j].
  f32x4 Sacc[NCT];
  {
    const size_t srow = ((size_t)(b * H + h) * DV + v0 + 16 * wv + n) * DK;
    if (p.S0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) Sacc[ct] = *(const f32x4*)(p.S0 + srow + 16 * ct + 4 * g);
    } else {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) Sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  float colsum = 0.f;   // content-aware: running sum of this lane's output column
  if constexpr (CONTENT) {
    // u_h[v] = sum_r a_h[r] B_h[r][v]
    for (int vv = tid; vv < TV; vv += NT) {
      float acc = 0.f;
      for (int r = 0; r < p.ub_rank; ++r)
        acc += p.ub_up[h * p.ub_rank + r] * p.ub_down[((size_t)h * p.ub_rank + r) * DV + v0 + vv];
      sU[vv] = acc;
      sMean[vv] = p.m_carry ? p.m_carry[(size_t)(b * H + h) * DV + v0 + vv] : 0.f;
    }
    lds_barrier();
    if (wv == 0) {
      float acc = 0.f;
      for (int vv = l; vv < TV; vv += 64) acc += sU[vv] * sMean[vv];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      if (l == 0) sS[0] = acc;
    }
    lds_barrier();
  }

  const bool prep = tid < NP * NSEG;
  // threads outside the prep split load a valid (unused) address instead of branching
  const int pp = tid % NP, seg = (tid / NP) % NSEG;
  const int nchunks = (Tn + L - 1) / L;

  using RP = RawPair<T>;
  using Raw = RawChunk<T, TPS, C::NVL>;
  Raw R;
  load_raw<T, DK, L, TV, DECAY, CONTENT>(R, p, 0, pp, seg, tid, b, h, v0);

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * L;

    // ------------------------------------------------------------ stage P1
    f32x2 cum[TPS];
    if (prep) {
      f32x2 run = {1.f, DECAY == 0 ? 1.f : 0.f};
#pragma unroll
      for (int r = 0; r < TPS; ++r) {
        const bool ok = c0 + seg * TPS + r < Tn;
        if constexpr (DECAY == 0) {
          const f32x2 a = ok ? R.a[r] : f32x2{1.f, 1.f};
          run.x *= a.x;
          run.y *= a.y;
        } else {
          const float gm = ok ? R.a[r].x : 1.f;
          const float th = ok ? R.a[r].y : 0.f;
          float sn, cs;
          __sincosf(th, &sn, &cs);
          run = cmul(run, f32x2{gm * cs, gm * sn});
        }
        cum[r] = run;
      }
      sSeg[seg * NP + pp] = run;
    }
    if (tid < L) {
      const bool ok = c0 + tid < Tn;
      float bt = R.bt;
      if constexpr (CONTENT) bt = 1.f / (1.f + __expf(-(bt + sS[0])));
      bt = ok ? bt : 0.f;
      sBeta[tid] = bt;
      sBW[tid] = ok ? bt * R.wt : 0.f;
    }
    {
      constexpr int VEC = 16 / sizeof(T), VPR = TV / VEC;
#pragma unroll
      for (int i = 0; i < C::NVL; ++i) {
        const int idx = tid + i * NT;
        if (idx < L * VPR) {
          const int r = idx / VPR, cc = idx % VPR;
          const bool ok = c0 + r < Tn;
          uint4 val;
          val.x = ok ? R.v[i].x : 0u;
          val.y = ok ? R.v[i].y : 0u;
          val.z = ok ? R.v[i].z : 0u;
          val.w = ok ? R.v[i].w : 0u;
          *(uint4*)(sV + r * RSV + cc * VEC) = val;
        }
      }
    }
    lds_barrier();

    // ------------------------------------------------------------ stage P2
    // running products before this segment (pre) and over the chunk (tot); the
    // chunk takes the token path (gdr_token.h) when some channel's Gamma_L
    // leaves the split form's range
    f32x2 pre = {1.f, DECAY == 0 ? 1.f : 0.f};
    f32x2 tot = pre;
    bool in_range = true;
    if (prep) {
#pragma unroll
      for (int s = 0; s < NSEG; ++s) {
        const f32x2 x = sSeg[s * NP + pp];
        if constexpr (DECAY == 0) {
          if (s < seg) {
            pre.x *= x.x;
            pre.y *= x.y;
          }
          tot.x *= x.x;
          tot.y *= x.y;
        } else {
          if (s < seg) pre = cmul(pre, x);
          tot = cmul(tot, x);
        }
      }
      if (seg == 0) sGL[pp] = tot;
      in_range = decay_in_range<DECAY>(tot);
    }
    {
      const unsigned long long bad = __ballot(!in_range);
      if (l == 0) sFlag[wv] = bad != 0ull;
    }
    lds_barrier();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any_bad |= sFlag[w];
    const bool token_path = __builtin_amdgcn_readfirstlane(any_bad) != 0;
    if (prep && token_path) {
      // raw keys and queries into K+ and Q+, the transition (ROT2: gamma cos,
      // gamma sin per pair) as fp32 into Kh|K-^T
      float* sTr = (float*)sKhKm;
#pragma unroll
      for (int r = 0; r < TPS; ++r) {
        const int row = seg * TPS + r;
        Pair<T>::store(sKp + row * RSK + 2 * pp, RP::cvt(R.k[r]));
        Pair<T>::store(sQp + row * RSK + 2 * pp, RP::cvt(R.q[r]));
        f32x2 z = R.a[r];
        if constexpr (DECAY != 0) {
          float sn, cs;
          __sincosf(z.y, &sn, &cs);
          z = f32x2{z.x * cs, z.x * sn};
        }
        *(f32x2*)(sTr + row * DK + 2 * pp) = z;
      }
    } else if (prep) {
#pragma unroll
      for (int r4 = 0; r4 < TPS; r4 += 4) {
        float km0[4], km1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = r4 + u;
          const int row = seg * TPS + r;
          const bool ok = c0 + row < Tn;
          f32x2 k2 = RP::cvt(R.k[r]), q2 = RP::cvt(R.q[r]);
          if (!ok) k2 = q2 = f32x2{0.f, 0.f};
          f32x2 kp, kh, qp, km;
          if constexpr (DECAY == 0) {
            const f32x2 gc = {pre.x * cum[r].x, pre.y * cum[r].y};
            const f32x2 inv = {__builtin_amdgcn_rcpf(gc.x), __builtin_amdgcn_rcpf(gc.y)};
            kp = f32x2{k2.x * gc.x, k2.y * gc.y};
            kh = f32x2{k2.x * inv.x, k2.y * inv.y};
            qp = f32x2{q2.x * gc.x, q2.y * gc.y};
            km = f32x2{k2.x * (tot.x * inv.x), k2.y * (tot.y * inv.y)};
          } else {
            const f32x2 z = cmul(pre, cum[r]);
            const float nz = __builtin_amdgcn_rcpf(z.x * z.x + z.y * z.y);
            const f32x2 zi = {z.x * nz, z.y * nz};          // Gamma^{-T} block
            kp = cmul(z, k2);
            kh = cmul(zi, k2);
            qp = cmul(z, q2);
            km = cmul(f32x2{tot.x, -tot.y}, kh);          // Gamma_L^T Kh
          }
          Pair<T>::store(sKp + row * RSK + 2 * pp, kp);
          Pair<T>::store(sKh + row * RSK + 2 * pp, kh);
          Pair<T>::store(sQp + row * RSK + 2 * pp, qp);
          km0[u] = km.x;
          km1[u] = km.y;
        }
        const int col = seg * TPS + r4;
        store4<T>(sKmT + (2 * pp) * RSL + col, km0);
        store4<T>(sKmT + (2 * pp + 1) * RSL + col, km1);
      }
    }
    // prefetch the next chunk's inputs; they land while this chunk computes
    if (c + 1 < nchunks)
      load_raw<T, DK, L, TV, DECAY, CONTENT>(R, p, c0 + L, pp, seg, tid, b, h, v0);
    lds_barrier();

    if (token_path) {
      // ---------------------------------------------------------- token path
      token_steps<DK, DECAY, false, T>(
          Sacc, (const float*)sKhKm, sKp, sQp, RSK,
          [&](int t) { return (float)sV[t * RSV + 16 * wv + n]; }, sBeta, sBW,
          min(L, Tn - c0), [&](int t, float ov) {
            if (g == 0) {
              go[((size_t)(b * Tn + c0 + t) * H + h) * DV + v0 + 16 * wv + n] = (T)ov;
              if constexpr (CONTENT) colsum += ov;
            }
          });
    } else {
    // ------------------------------------------------------------ stage G
    {
      constexpr int NTRI = NB * (NB + 1) / 2;
      for (int ti = wv; ti < 2 * NTRI; ti += NW) {
        const int which = ti / NTRI;   // 0: A, 1: M
        const int tt = ti % NTRI;
        int rb = 0;
        while ((rb + 1) * (rb + 2) / 2 <= tt) ++rb;
        const int cb = tt - rb * (rb + 1) / 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const T* src = which ? sQp : sKp;
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk)
          O::mma(acc, load_plain<T>(src, RSK, 16 * rb, 32 * kk),
                 load_plain<T>(sKh, RSK, 16 * cb, 32 * kk));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = 16 * rb + 4 * g + j, cc = 16 * cb + n;
          if (which == 0) {
            const float val = (cc < rr) ? sBeta[rr] * acc[j] : 0.f;
            sA[rr * RSL + cc] = (T)val;
            if (rb == cb) sAd[(rb * 16 + 4 * g + j) * 17 + n] = val;
          } else {
            sM[rr * RSL + cc] = (T)((cc <= rr) ? acc[j] : 0.f);
          }
        }
      }
    }
    lds_barrier();

    // ------------------------------------------------------------ stage D
    if (tid < L) {
      const int bb = tid >> 4, cc = tid & 15;
      float tcol[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == cc) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= sAd[(bb * 16 + i) * 17 + j] * tcol[j];
        tcol[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sTd[(bb * 16 + i) * RST + cc] = (T)tcol[i];
    }
    lds_barrier();

    // ------------------------------------------------------------ stage WU
    f32x4 Uacc[NB];
    {
      f32x4 Wacc[NCW][NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        Uacc[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw) Wacc[cw][bb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        f32x4 y[NCW], u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = 16 * bb + 4 * g + j;
          const float be = sBeta[rr];
#pragma unroll
          for (int cw = 0; cw < NCW; ++cw) {
            const int cb = wv + cw * NW;
            y[cw][j] = be * to_f32(sKp[rr * RSK + 16 * cb + n]);
          }
          u[j] = sBW[rr] * to_f32(sV[rr * RSV + 16 * wv + n]);
        }
#pragma unroll
        for (int kk = 0; 2 * kk < bb; ++kk) {
          const bool half = (2 * kk + 1 >= bb);
          frag a = half ? load_cb_half<T>(sA, RSL, 16 * bb, 32 * kk)
                        : load_cb<T>(sA, RSL, 16 * bb, 32 * kk);
          a = O::neg(a);
#pragma unroll
          for (int cw = 0; cw < NCW; ++cw) {
            const frag bf = half ? O::from_acc_half(Wacc[cw][2 * kk])
                                 : O::from_acc(Wacc[cw][2 * kk], Wacc[cw][2 * kk + 1]);
            O::mma(y[cw], a, bf);
          }
          const frag bu = half ? O::from_acc_half(Uacc[2 * kk])
                               : O::from_acc(Uacc[2 * kk], Uacc[2 * kk + 1]);
          O::mma(u, a, bu);
        }
        const frag at = load_cb_half<T>(sTd + bb * 16 * RST, RST, 0, 0);
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw) O::mma(Wacc[cw][bb], at, O::from_acc_half(y[cw]));
        O::mma(Uacc[bb], at, O::from_acc_half(u));
      }
      T* sW = sKh;
#pragma unroll
      for (int cw = 0; cw < NCW; ++cw) {
        const int cb = wv + cw * NW;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sW[(16 * bb + 4 * g + j) * RSK + 16 * cb + n] = (T)Wacc[cw][bb][j];
      }
    }
    lds_barrier();

    // ------------------------------------------------------------ stage S
    {
      const T* sW = sKh;
      frag Sf[NKC];
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) Sf[kk] = O::from_acc(Sacc[2 * kk], Sacc[2 * kk + 1]);
      f32x4 Dl[NB], Qs[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        f32x4 P = {0.f, 0.f, 0.f, 0.f}, Q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk) {
          O::mma(P, load_cb<T>(sW, RSK, 16 * i, 32 * kk), Sf[kk]);
          O::mma(Q, load_cb<T>(sQp, RSK, 16 * i, 32 * kk), Sf[kk]);
        }
        Dl[i] = Uacc[i] - P;
        Qs[i] = Q;
      }
      frag Df[NKT];
#pragma unroll
      for (int kk = 0; kk < NKT; ++kk)
        Df[kk] = (2 * kk + 1 < NB) ? O::from_acc(Dl[2 * kk], Dl[2 * kk + 1])
                                   : O::from_acc_half(Dl[2 * kk]);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        f32x4 acc = Qs[i];
#pragma unroll
        for (int kk = 0; kk <= i / 2; ++kk) {
          const frag a = (2 * kk + 1 < NB) ? load_cb<T>(sM, RSL, 16 * i, 32 * kk)
                                           : load_cb_half<T>(sM, RSL, 16 * i, 32 * kk);
          O::mma(acc, a, Df[kk]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = c0 + 16 * i + 4 * g + j;
          if (t < Tn) {
            go[((size_t)(b * Tn + t) * H + h) * DV + v0 + 16 * wv + n] = (T)acc[j];
            if constexpr (CONTENT) colsum += acc[j];
          }
        }
      }
      // S <- S Gamma_L  (accumulator rows are key channels)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if constexpr (DECAY == 0) {
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const f32x2 z = sGL[(16 * ct + 4 * g + j) >> 1];
            Sacc[ct][j] *= z.x;
            Sacc[ct][j + 1] *= z.y;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const f32x2 z = sGL[(16 * ct + 4 * g + j) >> 1];
            const float x0 = Sacc[ct][j], x1 = Sacc[ct][j + 1];
            Sacc[ct][j] = z.x * x0 + z.y * x1;
            Sacc[ct][j + 1] = -z.y * x0 + z.x * x1;
          }
        }
        // + Dl^T K-
#pragma unroll
        for (int kk = 0; kk < NKT; ++kk) {
          const frag a = (2 * kk + 1 < NB) ? load_cb<T>(sKmT, RSL, 16 * ct, 32 * kk)
                                           : load_cb_half<T>(sKmT, RSL, 16 * ct, 32 * kk);
          O::mma(Sacc[ct], a, Df[kk]);
        }
      }
    }

    }   // split form

    if constexpr (CONTENT) {
      const int cend = c0 + L;
      if (cend % p.window == 0 || cend >= Tn) {
        // window finished: mean of this window's outputs per value channel
        float s = colsum;
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        const int wstart = (cend - 1) / p.window * p.window;
        const int wlen = (cend < Tn ? cend : Tn) - wstart;
        lds_barrier();   // everyone is done reading sS for this window
        if (g == 0) sMean[16 * wv + n] = s / (float)wlen;
        colsum = 0.f;
        lds_barrier();
        if (wv == 0) {
          float acc = 0.f;
          for (int vv = l; vv < TV; vv += 64) acc += sU[vv] * sMean[vv];
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
          if (l == 0) sS[0] = acc;
        }
      }
    }
    lds_barrier();
  }

  if (p.S_out) {
    const size_t srow = ((size_t)(b * H + h) * DV + v0 + 16 * wv + n) * DK;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) *(f32x4*)(p.S_out + srow + 16 * ct + 4 * g) = Sacc[ct];
  }
  if constexpr (CONTENT) {
    if (p.m_carry && tid < TV) p.m_carry[(size_t)(b * H + h) * DV + v0 + tid] = sMean[tid];
  }
}

// ---------------------------------------------------------------- dispatch
template <typename T, int DK, int L, int TV, int DECAY, bool CONTENT>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  const int nvt = p.DV / TV;
  FwdParams q = p;
  q.n_vt = nvt;
  q.n_units = p.B * p.H;
  const int groups = (q.n_units + 7) / 8;
  dim3 grid(groups * 8 * nvt), block(TV / 16 * 64);
  hipLaunchKernelGGL((gdr_fwd_kernel<T, DK, L, TV, DECAY, CONTENT>), grid, block, 0, stream, q);
  return hipGetLastError();
}

template <typename T, int DK, int L, int DECAY, bool CONTENT>
static hipError_t pick_tv(const FwdParams& p, hipStream_t s) {
  if constexpr (CONTENT) {
    return launch_one<T, DK, L, DK, DECAY, true>(p, s);   // one workgroup per (b, h)
  } else if constexpr (DK == 128) {
    // fill the chip: 64-wide value tiles unless that leaves most CUs idle
    if ((long)p.B * p.H * 2 >= 192) return launch_one<T, DK, L, 64, DECAY, false>(p, s);
    return launch_one<T, DK, L, 32, DECAY, false>(p, s);
  } else {
    return launch_one<T, DK, L, 32, DECAY, false>(p, s);
  }
}

template <typename T, int DK, int DECAY, bool CONTENT>
static hipError_t pick_l(const FwdParams& p, hipStream_t s) {
  // fp32 operands at d_k = 128 fit the LDS of one CU only with 32-token blocks
  constexpr int LMAX = (sizeof(T) == 4 && DK == 128) ? 32 : 64;
  const int L = p.block < LMAX ? p.block : LMAX;
  if (L == 16) return pick_tv<T, DK, 16, DECAY, CONTENT>(p, s);
  if (L == 32) return pick_tv<T, DK, 32, DECAY, CONTENT>(p, s);
  if constexpr (LMAX >= 64) return pick_tv<T, DK, 64, DECAY, CONTENT>(p, s);
  return hipErrorInvalidValue;
}

template <typename T, int DECAY, bool CONTENT>
static hipError_t pick_dk(const FwdParams& p, hipStream_t s) {
  switch (p.DK) {
    case 32: return pick_l<T, 32, DECAY, CONTENT>(p, s);
    case 64: return pick_l<T, 64, DECAY, CONTENT>(p, s);
    case 128: return pick_l<T, 128, DECAY, CONTENT>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t pick_variant(const FwdParams& p, hipStream_t s) {
  const bool content = p.beta_logit != nullptr;
  if (p.decay == 0) {
    return content ? pick_dk<T, 0, true>(p, s) : pick_dk<T, 0, false>(p, s);
  }
  return content ? pick_dk<T, 1, true>(p, s) : pick_dk<T, 1, false>(p, s);
}

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  if (fwd_pipe_supported(p)) return launch_fwd_pipe(p, stream);
  // the gated forward and reflection blocks run only pipelined
  if (p.gmode != 0 || p.decay == 2) return hipErrorInvalidValue;
  if (p.io_bf16) return pick_variant<__bf16>(p, stream);
  return pick_variant<float>(p, stream);
}

}  // namespace gdr
