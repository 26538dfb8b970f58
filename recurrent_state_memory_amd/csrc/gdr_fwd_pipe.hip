// gdr_fwd_pipe.hip -- pipelined chunk-WY gated delta-rule forward (bf16 q/k/v/o) for gfx950.
//
// Same computation as gdr_fwd.hip (chunk-WY algebra of the CARVE technical
// summary, section 1.3, and the SFDA constructive chunk-WY theorem / exact
// affine chunk transfer), organised so that the state-independent work of
// chunk c+1 overlaps the state-dependent work of chunk c inside one
// workgroup:
//
//   producer waves (4): load chunk c+1 (issued one chunk ahead), running
//     products of the key-axis transitions, decayed forms K+, Q+, Kh, K-^T,
//     Gram tiles A = strict_lower(diag(beta) K+ Kh^T), M = lower_incl(Q+ Kh^T),
//     and the two 16x16 diagonal blocks T00, T11 of (I + A)^{-1};
//   consumer waves (one per 16 value channels): for chunk c,
//     R  = diag(beta w) V - diag(beta) K+ S^T
//     Dl = (I + A)^{-1} R by blocks: Dl0 = T00 R0, Dl1 = T11 (R1 - A10 Dl0)
//     O  = Q+ S^T + M Dl,   S <- S Gamma_L + Dl^T K-.
//
// The chunk length is 32 tokens (two 16-token blocks).  The consumer-side
// buffers are double-buffered in LDS; one workgroup-wide barrier separates
// each of the three phases of an iteration, and both roles pass the same
// number of barriers.
//
// Running products without reciprocals: with g_r = prod_{s<=r} D_s (forward)
// and h_r = prod_{s>r} D_s (backward) inside the chunk, K+ = g_r k,
// Q+ = g_r q, K- = h_r^T k, and Kh = Gamma_r^{-T} k = Gamma_L^{-T} K-, so only
// one reciprocal per key channel (of Gamma_L) is needed per chunk.  For 2x2
// rotation-decay blocks the same holds with complex products per channel pair.
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

constexpr int L = 32;      // tokens per chunk
constexpr int NWP = 4;     // producer waves
constexpr int RSL = L + 4; // row stride of [.][L] arrays
constexpr int RS16 = 20;   // row stride of 16x16 blocks

template <int DK, int TV>
struct Cfg {
  static constexpr int NWC = TV / 16;            // consumer waves
  static constexpr int NT = (NWP + NWC) * 64;
  static constexpr int NP = DK / 2;              // channel pairs
  static constexpr int NSEG0 = NWP * 64 / NP;
  static constexpr int NSEG = NSEG0 < L / 4 ? NSEG0 : L / 4;
  static constexpr int TPS = L / NSEG;           // tokens per producer thread
  static constexpr int RSK = DK + 8;
  static constexpr int RSV = TV + 8;
  static constexpr int NCT = DK / 16;
  static constexpr int NKC = DK / 32;
  static constexpr int VPR = TV / 8;             // 16-byte pieces per value row
  static_assert(TPS % 4 == 0 && TPS >= 4, "prep split");
  static_assert(L * VPR <= NWP * 64, "value tile load split");
};

// Consumer-side buffers of one chunk (double-buffered).
template <int DK, int TV>
struct Buf {
  using C = Cfg<DK, TV>;
  bf Kp[L * C::RSK];
  bf Qp[L * C::RSK];
  bf KmT[DK * RSL];
  bf M[L * RSL];
  bf A10[16 * RS16];
  bf Td[2 * 16 * RS16];
  bf V[L * C::RSV];
  float beta[L];
  float bw[L];
  f32x2 GL[C::NP];
};

template <int DK, int TV>
struct Shared {
  using C = Cfg<DK, TV>;
  Buf<DK, TV> buf[2];
  bf Kh[L * C::RSK];
  float Ad[2 * 16 * 17];
  f32x2 segF[C::NSEG * C::NP];
};

template <int TPS>
struct Raw {
  uint32_t k[TPS], q[TPS];
  f32x2 a[TPS];
  uint4 v;
  float bt, wt;
};

template <int DK, int TV, int DECAY>
__device__ inline void load_raw(Raw<Cfg<DK, TV>::TPS>& R, const FwdParams& p, int c0, int pp,
                                int seg, int ptid, int b, int h, int v0) {
  using C = Cfg<DK, TV>;
  const int Tn = p.T, H = p.H;
  const bf* gk = (const bf*)p.k;
  const bf* gq = (const bf*)p.q;
  const bf* gv = (const bf*)p.v;
#pragma unroll
  for (int r = 0; r < C::TPS; ++r) {
    int t = c0 + seg * C::TPS + r;
    t = t < Tn ? t : Tn - 1;
    const size_t base = (size_t)(b * Tn + t) * H + h;
    R.k[r] = *(const uint32_t*)(gk + base * DK + 2 * pp);
    R.q[r] = *(const uint32_t*)(gq + base * DK + 2 * pp);
    if constexpr (DECAY == 0) {
      R.a[r] = *(const f32x2*)(p.alpha + base * DK + 2 * pp);
    } else {
      R.a[r] = f32x2{p.alpha[base * C::NP + pp], p.theta[base * C::NP + pp]};
    }
  }
  {
    const int idx = ptid < L * C::VPR ? ptid : 0;
    const int r = idx / C::VPR, cc = idx % C::VPR;
    int t = c0 + r;
    t = t < Tn ? t : Tn - 1;
    R.v = *(const uint4*)(gv + ((size_t)(b * Tn + t) * H + h) * p.DV + v0 + cc * 8);
  }
  {
    int t = c0 + (ptid < L ? ptid : L - 1);
    t = t < Tn ? t : Tn - 1;
    const size_t gi = (size_t)(b * Tn + t) * H + h;
    R.bt = p.beta[gi];
    R.wt = p.w[gi];
  }
}

template <int DK, int TV, int DECAY>
__global__ __launch_bounds__((NWP + TV / 16) * 64) void gdr_fwd_pipe_kernel(FwdParams p) {
  using C = Cfg<DK, TV>;
  using O = Op<bf>;
  using frag = O::frag;
  constexpr int NP = C::NP, NSEG = C::NSEG, TPS = C::TPS, RSK = C::RSK, RSV = C::RSV,
                NCT = C::NCT, NKC = C::NKC, VPR = C::VPR;
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
  const int nchunks = (Tn + L - 1) / L;

  if (wv < NWP) {
    // =============================================================== producer
    const int ptid = tid;                       // 0 .. NWP*64-1
    const bool prep = ptid < NP * NSEG;
    const int pp = ptid % NP, seg = (ptid / NP) % NSEG;
    Raw<TPS> R;
    load_raw<DK, TV, DECAY>(R, p, 0, pp, seg, ptid, b, h, v0);

    auto produce = [&](int j) {
      Buf<DK, TV>& B = sh.buf[j & 1];
      const int c0 = j * L;
      // ---- phase 1: running products inside this thread's segment
      f32x2 cf[TPS], cb[TPS];
      if (prep) {
        f32x2 d[TPS];
#pragma unroll
        for (int r = 0; r < TPS; ++r) {
          const bool ok = c0 + seg * TPS + r < Tn;
          if constexpr (DECAY == 0) {
            d[r] = ok ? R.a[r] : f32x2{1.f, 1.f};
          } else {
            float sn, cs;
            __sincosf(ok ? R.a[r].y : 0.f, &sn, &cs);
            const float gm = ok ? R.a[r].x : 1.f;
            d[r] = f32x2{gm * cs, gm * sn};
          }
        }
        f32x2 run = {1.f, DECAY == 0 ? 1.f : 0.f};
#pragma unroll
        for (int r = 0; r < TPS; ++r) {
          if constexpr (DECAY == 0) {
            run = f32x2{run.x * d[r].x, run.y * d[r].y};
          } else {
            run = cmul(run, d[r]);
          }
          cf[r] = run;
        }
        f32x2 bk = {1.f, DECAY == 0 ? 1.f : 0.f};
#pragma unroll
        for (int r = TPS - 1; r >= 0; --r) {
          cb[r] = bk;   // product over later tokens of the segment
          if constexpr (DECAY == 0) {
            bk = f32x2{bk.x * d[r].x, bk.y * d[r].y};
          } else {
            bk = cmul(bk, d[r]);
          }
        }
        sh.segF[seg * NP + pp] = run;
      }
      if (ptid < L) {
        const bool ok = c0 + ptid < Tn;
        B.beta[ptid] = ok ? R.bt : 0.f;
        B.bw[ptid] = ok ? R.bt * R.wt : 0.f;
      }
      if (ptid < L * VPR) {
        const int r = ptid / VPR, cc = ptid % VPR;
        const uint4 zero = {0u, 0u, 0u, 0u};
        *(uint4*)(B.V + r * RSV + cc * 8) = (c0 + r < Tn) ? R.v : zero;
      }
      __syncthreads();
      // ---- phase 2: decayed forms
      if (prep) {
        f32x2 pre = {1.f, DECAY == 0 ? 1.f : 0.f}, post = pre, tot = pre;
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
          const f32x2 x = sh.segF[s * NP + pp];
          if constexpr (DECAY == 0) {
            if (s < seg) pre = f32x2{pre.x * x.x, pre.y * x.y};
            if (s > seg) post = f32x2{post.x * x.x, post.y * x.y};
            tot = f32x2{tot.x * x.x, tot.y * x.y};
          } else {
            if (s < seg) pre = cmul(pre, x);
            if (s > seg) post = cmul(post, x);
            tot = cmul(tot, x);
          }
        }
        if (seg == 0) B.GL[pp] = tot;
        // Kh = Gamma_L^{-T} K-: per-channel 1/G (diag) or z_L/|z_L|^2 (rotation)
        f32x2 ig;
        if constexpr (DECAY == 0) {
          ig = f32x2{__builtin_amdgcn_rcpf(tot.x), __builtin_amdgcn_rcpf(tot.y)};
        } else {
          const float nz = __builtin_amdgcn_rcpf(tot.x * tot.x + tot.y * tot.y);
          ig = f32x2{tot.x * nz, tot.y * nz};
        }
#pragma unroll
        for (int r4 = 0; r4 < TPS; r4 += 4) {
          float km0[4], km1[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = r4 + u;
            const int row = seg * TPS + r;
            const bool ok = c0 + row < Tn;
            f32x2 kx = bf2_to_f2(R.k[r]), qx = bf2_to_f2(R.q[r]);
            if (!ok) kx = qx = f32x2{0.f, 0.f};
            f32x2 kp, qp, km, kh;
            if constexpr (DECAY == 0) {
              const f32x2 gf = {pre.x * cf[r].x, pre.y * cf[r].y};
              const f32x2 gb = {cb[r].x * post.x, cb[r].y * post.y};
              kp = f32x2{kx.x * gf.x, kx.y * gf.y};
              qp = f32x2{qx.x * gf.x, qx.y * gf.y};
              km = f32x2{kx.x * gb.x, kx.y * gb.y};
              kh = f32x2{km.x * ig.x, km.y * ig.y};
            } else {
              const f32x2 zf = cmul(pre, cf[r]);
              const f32x2 zb = cmul(cb[r], post);
              kp = cmul(zf, kx);
              qp = cmul(zf, qx);
              km = cmul(conj(zb), kx);
              kh = cmul(ig, km);
            }
            *(uint32_t*)(B.Kp + row * RSK + 2 * pp) = f2_to_bf2(kp);
            *(uint32_t*)(B.Qp + row * RSK + 2 * pp) = f2_to_bf2(qp);
            *(uint32_t*)(sh.Kh + row * RSK + 2 * pp) = f2_to_bf2(kh);
            km0[u] = km.x;
            km1[u] = km.y;
          }
          const int col = seg * TPS + r4;
          bf16x4 v0v, v1v;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            v0v[u] = (bf)km0[u];
            v1v[u] = (bf)km1[u];
          }
          *(bf16x4*)(B.KmT + (2 * pp) * RSL + col) = v0v;
          *(bf16x4*)(B.KmT + (2 * pp + 1) * RSL + col) = v1v;
        }
      }
      if (j + 1 < nchunks) load_raw<DK, TV, DECAY>(R, p, c0 + L, pp, seg, ptid, b, h, v0);
      __syncthreads();
      // ---- phase 3: Gram tiles and the diagonal inverse blocks
      if (wv == 0) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKC; ++kk)
            O::mma(acc, load_plain<bf>(B.Kp, RSK, 16 * bb, 32 * kk),
                   load_plain<bf>(sh.Kh, RSK, 16 * bb, 32 * kk));
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int rr = 4 * g + jj;
            sh.Ad[(bb * 16 + rr) * 17 + n] = (n < rr) ? B.beta[16 * bb + rr] * acc[jj] : 0.f;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (l < 32) {
          const int bb = l >> 4, cc = l & 15;
          const float* Ab = sh.Ad + bb * 16 * 17;
          float tcol[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float acc = (i == cc) ? 1.f : 0.f;
#pragma unroll
            for (int jj = 0; jj < i; ++jj) acc -= Ab[i * 17 + jj] * tcol[jj];
            tcol[i] = acc;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) B.Td[(bb * 16 + i) * RS16 + cc] = (bf)tcol[i];
        }
      } else {
        // wave 1: A10 and M00; wave 2: M10; wave 3: M11
        const int ntile = (wv == 1) ? 2 : 1;
        for (int ti = 0; ti < ntile; ++ti) {
          const int kind = (wv == 1 && ti == 0) ? 0 : 1;          // 0: A10, 1: an M tile
          const int rb = (wv == 1) ? (ti == 0 ? 1 : 0) : 1;
          const int cbk = (wv == 3) ? 1 : 0;
          const bf* src = kind == 0 ? B.Kp : B.Qp;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKC; ++kk)
            O::mma(acc, load_plain<bf>(src, RSK, 16 * rb, 32 * kk),
                   load_plain<bf>(sh.Kh, RSK, 16 * cbk, 32 * kk));
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int rr = 16 * rb + 4 * g + jj, cc = 16 * cbk + n;
            if (kind == 0) {
              B.A10[(4 * g + jj) * RS16 + n] = (bf)(B.beta[rr] * acc[jj]);
            } else {
              B.M[rr * RSL + cc] = (bf)((cc <= rr) ? acc[jj] : 0.f);
            }
          }
        }
      }
      __syncthreads();
    };

    produce(0);
    for (int i = 0; i < nchunks; ++i) {
      if (i + 1 < nchunks) {
        produce(i + 1);
      } else {
        __syncthreads();
        __syncthreads();
        __syncthreads();
      }
    }
  } else {
    // =============================================================== consumer
    const int cw = wv - NWP;                    // value block of 16 channels
    f32x4 Sacc[NCT];
    const size_t srow = ((size_t)(b * H + h) * DV + v0 + 16 * cw + n) * DK;
    if (p.S0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) Sacc[ct] = *(const f32x4*)(p.S0 + srow + 16 * ct + 4 * g);
    } else {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) Sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf* go = (bf*)p.o;
    __syncthreads();   // prologue: chunk 0 is being prepared
    __syncthreads();
    __syncthreads();
    for (int i = 0; i < nchunks; ++i) {
      const Buf<DK, TV>& B = sh.buf[i & 1];
      const int c0 = i * L;
      // ---- phase 1: R = diag(bw) V - diag(beta) K+ S^T, Qs = Q+ S^T
      frag Sf[NKC];
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk) Sf[kk] = O::from_acc(Sacc[2 * kk], Sacc[2 * kk + 1]);
      f32x4 Rt[2], Qs[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 P = {0.f, 0.f, 0.f, 0.f}, Q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk) {
          O::mma(P, load_cb<bf>(B.Kp, RSK, 16 * t, 32 * kk), Sf[kk]);
          O::mma(Q, load_cb<bf>(B.Qp, RSK, 16 * t, 32 * kk), Sf[kk]);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * t + 4 * g + jj;
          Rt[t][jj] = B.bw[r] * (float)B.V[r * RSV + 16 * cw + n] - B.beta[r] * P[jj];
        }
        Qs[t] = Q;
      }
      __syncthreads();
      // ---- phase 2: Dl by blocks, O = Qs + M Dl, store o
      f32x4 D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
      O::mma(D0, load_cb_half<bf>(B.Td, RS16, 0, 0), O::from_acc_half(Rt[0]));
      f32x4 Y = Rt[1];
      O::mma(Y, O::neg(load_cb_half<bf>(B.A10, RS16, 0, 0)), O::from_acc_half(D0));
      O::mma(D1, load_cb_half<bf>(B.Td + 16 * RS16, RS16, 0, 0), O::from_acc_half(Y));
      const frag Df = O::from_acc(D0, D1);
      f32x4 O0 = Qs[0], O1 = Qs[1];
      O::mma(O0, load_cb_half<bf>(B.M, RSL, 0, 0), O::from_acc_half(D0));
      O::mma(O1, load_cb<bf>(B.M, RSL, 16, 0), Df);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int t0 = c0 + 4 * g + jj, t1 = t0 + 16;
        const int col = v0 + 16 * cw + n;
        if (t0 < Tn) go[((size_t)(b * Tn + t0) * H + h) * DV + col] = (bf)O0[jj];
        if (t1 < Tn) go[((size_t)(b * Tn + t1) * H + h) * DV + col] = (bf)O1[jj];
      }
      __syncthreads();
      // ---- phase 3: S <- S Gamma_L + Dl^T K-
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int jj = 0; jj < 4; jj += 2) {
          const f32x2 z = B.GL[(16 * ct + 4 * g + jj) >> 1];
          const float x0 = Sacc[ct][jj], x1 = Sacc[ct][jj + 1];
          if constexpr (DECAY == 0) {
            Sacc[ct][jj] = x0 * z.x;
            Sacc[ct][jj + 1] = x1 * z.y;
          } else {
            Sacc[ct][jj] = z.x * x0 + z.y * x1;
            Sacc[ct][jj + 1] = -z.y * x0 + z.x * x1;
          }
        }
        O::mma(Sacc[ct], load_cb<bf>(B.KmT, RSL, 16 * ct, 0), Df);
      }
      __syncthreads();
    }
    if (p.S_out) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) *(f32x4*)(p.S_out + srow + 16 * ct + 4 * g) = Sacc[ct];
    }
  }
}

template <int DK, int TV, int DECAY>
hipError_t launch(const FwdParams& p0, hipStream_t s) {
  FwdParams p = p0;
  p.n_vt = p.DV / TV;
  p.n_units = p.B * p.H;
  const int groups = (p.n_units + 7) / 8;
  hipLaunchKernelGGL((gdr_fwd_pipe_kernel<DK, TV, DECAY>), dim3(groups * 8 * p.n_vt),
                     dim3(Cfg<DK, TV>::NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace pipe

bool fwd_pipe_supported(const FwdParams& p) {
  return p.io_bf16 && p.beta_logit == nullptr && (p.DK == 64 || p.DK == 128) && p.DV == p.DK;
}

hipError_t launch_fwd_pipe(const FwdParams& p, hipStream_t s) {
  const bool rot = p.decay != 0;
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
