// fa2_noalloc.hip -- fa2_backward with the library's own fixed workspace, for callers that
// cannot allocate device memory (graph capture, tight serving loops, harnesses that forbid
// hipMalloc). The backward's only scratch is its workspace (-D and LSE*log2(e) per query row,
// written by the preprocess and read by the dK/dV and dQ kernels); here it lives in a
// file-scope device array instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa2.h"
#include "fa2_launch.h"

namespace {

// One copy per GPU, created when the library's code is loaded on that device. In host code
// the name `scratch` is only a stand-in for the symbol, not a device address: host code uses
// the address that scratch_address() looks up, never the name.
__device__ __align__(256) char scratch[FA2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on the first call on
// that device (with it current) and kept for the life of the process.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int fa2_backward_noalloc(const void* q, const void* k, const void* v, const float* o,
                                    const float* lse, const void* dO, float* dq, float* dk,
                                    float* dv, int B, int Hq, int Hkv, int N, int d, int causal,
                                    float scale, hipStream_t stream) {
  if (fa2_backward_workspace_size(B, Hq, N) > FA2_NOALLOC_SCRATCH_BYTES)
    return FA2_ERR_SCRATCH_LIMIT;
  bool empty = false;
  const int st = fa2::backward_check_args(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d,
                                          scale, &empty);
  if (st != FA2_OK || empty) return st;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return FA2_ERR_HIP;
  return fa2_backward(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, ws,
                      FA2_NOALLOC_SCRATCH_BYTES, stream);
}
