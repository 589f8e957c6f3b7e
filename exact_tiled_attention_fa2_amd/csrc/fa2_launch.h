// fa2_launch.h -- internal interface between the C-ABI layer and the kernel launchers.
// Arguments reaching these functions have already been validated by fa2_abi.cpp.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa2 {

struct AttnShape {
  int B, Hq, Hkv, N, d;
  int causal;
  float scale;
  int window = -1;  // causal sliding window: query i sees keys i - window .. i; < 0: none
};

// Window value the kernels use when there is none: larger than any supported N.
constexpr int kNoWindow = 0x3fffffff;

// The window the kernels see: none (kNoWindow) unless 0 <= window < N - 1. A window of N - 1 or
// more hides no key of any row, so it is plain causal attention; mapping it here keeps the
// kernels' index arithmetic (key + window, query - window) far from int overflow whatever value
// the caller passed.
inline int kernel_window(const AttnShape& s) {
  return (s.window >= 0 && s.window < s.N - 1) ? s.window : kNoWindow;
}

hipError_t launch_forward(const void* q, const void* k, const void* v, float* o, float* lse,
                          const AttnShape& s, hipStream_t stream);

// FP8 forward (d = 128): q8, k8, v8 are FP8 E4M3FN codes standing for code * scale; the
// workspace receives V widened to bf16 (forward_fp8_workspace_bytes).
size_t forward_fp8_workspace_bytes(const AttnShape& s);
hipError_t launch_forward_fp8(const void* q8, const void* k8, const void* v8, float q_scale,
                              float k_scale, float v_scale, float* o, float* lse,
                              const AttnShape& s, void* ws, hipStream_t stream);

// Backward workspace: D at [0, R) and LSE*log2(e) at [R, 2R) floats, R = B*Hq*N.
hipError_t launch_bwd_preprocess(const float* o, const void* dO, const float* lse, float* ws,
                                 const AttnShape& s, hipStream_t stream);

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                           const float* ws, float* dk, float* dv, const AttnShape& s,
                           hipStream_t stream);

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                         const float* ws, float* dq, const AttnShape& s, hipStream_t stream);

// dQ with the preprocess folded in: also fills the workspace (as launch_bwd_preprocess) from
// o and lse, for a launch_bwd_dkdv after it.
hipError_t launch_bwd_dq_pre(const void* q, const void* k, const void* v, const void* dO,
                             const float* o, const float* lse, float* ws, float* dq,
                             const AttnShape& s, hipStream_t stream);

// fa2_backward's checks of its sizes and its non-workspace buffers (status codes of fa2.h);
// sets *empty for a problem with nothing to compute. Launches nothing.
int backward_check_args(const void* q, const void* k, const void* v, const float* o,
                        const float* lse, const void* dO, float* dq, float* dk, float* dv, int B,
                        int Hq, int Hkv, int N, int d, float scale, bool* empty);

// Decode: s.N is unused; Nq query rows against Nk cache rows. The workspace holds the partial
// results of the cache chunks (decode_workspace_bytes, 0 when one chunk suffices).
size_t decode_workspace_bytes(const AttnShape& s, int Nq, int Nk);
hipError_t launch_decode(const void* q, const void* k, const void* v, float* o, float* lse,
                         const AttnShape& s, int Nq, int Nk, float* ws, hipStream_t stream);

}  // namespace fa2
