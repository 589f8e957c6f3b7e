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
};

hipError_t launch_forward(const void* q, const void* k, const void* v, float* o, float* lse,
                          const AttnShape& s, hipStream_t stream);

hipError_t launch_bwd_preprocess(const float* o, const void* dO, float* delta, const AttnShape& s,
                                 hipStream_t stream);

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                           const float* delta, const void* dO, float* dk, float* dv,
                           const AttnShape& s, hipStream_t stream);

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                         const float* delta, const void* dO, float* dq, const AttnShape& s,
                         hipStream_t stream);

}  // namespace fa2
