// gdr_kernels.h -- launch interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

struct FwdParams {
  int B, T, H, DK, DV;
  int block;    // WY block length used by the kernel (16, 32 or 64)
  int window;   // content-aware window (the caller's chunk); unused otherwise
  int io_bf16;  // 1: bf16 q/k/v/o, 0: fp32
  int decay;    // 0: per-channel decay, 1: 2x2 rotation-decay blocks
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* theta;
  const float* beta;
  const float* w;
  const float* beta_logit;
  const float* ub_down;
  const float* ub_up;
  int ub_rank;
  float* m_carry;
  const float* S0;
  void* o;
  float* S_out;
  int n_vt;      // value tiles per (b, h); set by the launcher
  int n_units;   // B * H; set by the launcher
  // gated forward: 0 off; 1 decay from the bf16 pre-activation gate_x with the
  // per-head scale gate_a; 2 also L2-normalises each token's q and k
  int gmode;
  const void* gate_x;
  const float* gate_a;
  // backward's forward recompute: when set, the state at the start of every
  // 32-token block, [B, H, ceil(T / 32), DV, DK] fp32
  float* ckpt;
};

// Backward of the plain-erase forward (gdr_bwd.hip).  Inputs as the forward
// (bf16 q, k, v, grad_o), fp32 gradients out; ckpt holds the block-start
// states from the forward recompute, part the per-value-tile partial sums.
struct BwdParams {
  int B, T, H, DK, DV;
  int decay;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* theta;
  const float* beta;
  const float* w;
  const void* grad_o;
  const float* grad_S;   // gradient of S_T, or null
  float* grad_q;
  float* grad_k;
  float* grad_v;
  float* grad_alpha;
  float* grad_theta;
  float* grad_beta;
  float* grad_w;
  float* grad_S0;        // or null
  const float* ckpt;
  float* part;           // partial sums, bwd_part_floats() floats
  int* flag;             // per (b, h, value tile): a block left the block form's range
  int n_vt;              // value tiles per (b, h); set by the launcher
};

struct StepParams {
  int N, H, DK, DV;
  int io_bf16;
  int decay;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* theta;
  const float* beta;
  const float* w;
  float* S;
  void* o;
};

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
// pipelined bf16 forward (gdr_fwd_pipe.hip) for the plain erase, d_k = d_v in {64, 128}
bool fwd_pipe_supported(const FwdParams& p);
hipError_t launch_fwd_pipe(const FwdParams& p, hipStream_t stream);
hipError_t launch_step(const StepParams& p, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);

// The gated forward's activation and normalisation around the plain backward
// (gdr_gate_bwd.hip): rows are token-heads (b, t, h), C = DK (per-channel
// decay) or DK / 2 (2x2 blocks) decay channels per row.
struct GateBwdParams {
  int B, T, H, DK, C;
  int norm;                 // q and k normalised per token
  const void* x;            // bf16 decay pre-activation [B,T,H,C]
  const float* a;           // [H]
  const void* q_raw;        // bf16 [B,T,H,DK]
  const void* k_raw;
  float* alpha;             // prep: exp(-a softplus(x)) [B,T,H,C]
  void* q_n;                // prep (norm): bf16 l2-normalised q, k
  void* k_n;
  const float* grad_alpha;  // from the plain backward
  const float* grad_qn;     // from the plain backward (norm)
  const float* grad_kn;
  float* grad_x;            // [B,T,H,C]
  float* grad_q;            // raw-input gradients (norm)
  float* grad_k;
  float* ga_rows;           // per row: its contribution to dL/da_h
  float* grad_a;            // [H]
};
hipError_t launch_gate_prep(const GateBwdParams& p, hipStream_t stream);
hipError_t launch_gate_chain(const GateBwdParams& p, hipStream_t stream);
// block length of the backward (and of the forward's checkpoints) and the
// value-tile width of the backward kernel
constexpr int kBwdBlock = 32;
constexpr int kBwdTile = 32;
// floats of the partial-sum area: per value tile and token-head, dq, dk and
// the decay's log-gradient (DK each), then dbeta and dw
inline size_t bwd_part_floats(int B, int T, int H, int DK, int DV) {
  return (size_t)(DV / kBwdTile) * B * T * H * (3 * (size_t)DK + 2);
}
// The backward on a given workspace (argument and size checks included);
// gdr_chunk_bwd passes the caller's, gdr_chunk_bwd_noalloc its static scratch.
gdr_status chunk_bwd_on(const gdr_bwd_args* a, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);
int fwd_block_len(int dk, int chunk, bool io_bf16);

}  // namespace gdr
