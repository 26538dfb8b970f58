// gdr_noalloc.hip -- the backward for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid hipMalloc): gdr_chunk_bwd_noalloc runs gdr_chunk_bwd's kernels on a
// fixed scratch array that lives in the library's code object instead of a
// caller-provided workspace.
//
// The array is a file-scope device global, so every GPU that loads the
// library holds its own copy (kScratchBytes) until the process ends.  Host
// code never uses the array's name as an address: on the first call on a
// device, with that device current, hipGetSymbolAddress gives the device
// address, which is kept per device and passed to the kernels.  Every call on
// one GPU uses the same array: calls that overlap on one GPU (different
// streams, or different host threads) race.  Nothing in the array has to start
// at zero: the forward recompute writes every checkpoint and the backward
// every partial sum before they are read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdr.h"
#include "gdr_kernels.h"

namespace {

constexpr size_t kScratchBytes = (size_t)256 << 20;   // 256 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array (looked up once per device).
gdr_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GDR_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return GDR_OK;
}

}  // namespace

extern "C" gdr_status gdr_chunk_bwd_noalloc(const gdr_bwd_args* a, void* hip_stream) {
  if (!a) return GDR_ERR_NULL;
  if (a->workspace || a->workspace_bytes) return GDR_ERR_ARG;   // the scratch replaces it
  const size_t need = gdr_chunk_bwd_workspace(a);
  if (need == 0) return gdr::chunk_bwd_on(a, nullptr, 0, (hipStream_t)hip_stream);   // reports why
  if (need > kScratchBytes) return GDR_ERR_WORKSPACE;
  void* ws = nullptr;
  const gdr_status st = scratch_address(&ws);
  if (st != GDR_OK) return st;
  return gdr::chunk_bwd_on(a, ws, kScratchBytes, (hipStream_t)hip_stream);
}
