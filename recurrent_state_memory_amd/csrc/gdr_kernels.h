// gdr_kernels.h -- launch interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
int fwd_block_len(int dk, int chunk, bool io_bf16);

}  // namespace gdr
