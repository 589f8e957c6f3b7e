// fa2_abi.cpp -- the C ABI of the attention library: argument validation, then launches.
//
// Every check runs on the host before anything is enqueued, so a rejected call launches
// nothing and writes no output. The rules are the ones documented in include/fa2.h.
#include "../../include/fa2.h"

#include <math.h>
#include <stdint.h>

#include "fa2_launch.h"

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void* p, uint64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape checks. Returns FA2_OK and sets *empty when nothing needs computing.
int check_shape(int B, int Hq, int Hkv, int N, int d, float scale, bool* empty) {
  *empty = false;
  if (B < 0 || N < 0 || Hq < 0 || Hkv < 0) return FA2_ERR_BAD_SHAPE;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA2_ERR_BAD_GQA;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED_HEAD_DIM;
  if (!isfinite(scale) || scale == 0.0f) return FA2_ERR_BAD_SCALE;
  if (B == 0 || N == 0) {
    *empty = true;
    return FA2_OK;
  }
  // Kernels address one head with 32-bit byte offsets of fp32 rows: N*d*4 < 2^31.
  if ((int64_t)N * d * 4 >= ((int64_t)1 << 31)) return FA2_ERR_BAD_SHAPE;
  // Grid size (one workgroup per 64-row block per head, at most) must fit a 32-bit count.
  if ((int64_t)B * Hq * ((N + 63) / 64) >= ((int64_t)1 << 31)) return FA2_ERR_BAD_SHAPE;
  if ((int64_t)B * Hq >= ((int64_t)1 << 24)) return FA2_ERR_BAD_SHAPE;
  return FA2_OK;
}

}  // namespace

extern "C" {

const char* fa2_status_string(int status) {
  switch (status) {
    case FA2_OK: return "FA2_OK";
    case FA2_ERR_NULL_POINTER: return "FA2_ERR_NULL_POINTER";
    case FA2_ERR_BAD_SHAPE: return "FA2_ERR_BAD_SHAPE";
    case FA2_ERR_UNSUPPORTED_HEAD_DIM: return "FA2_ERR_UNSUPPORTED_HEAD_DIM";
    case FA2_ERR_BAD_GQA: return "FA2_ERR_BAD_GQA";
    case FA2_ERR_BAD_SCALE: return "FA2_ERR_BAD_SCALE";
    case FA2_ERR_MISALIGNED: return "FA2_ERR_MISALIGNED";
    case FA2_ERR_ALIASING: return "FA2_ERR_ALIASING";
    case FA2_ERR_WORKSPACE: return "FA2_ERR_WORKSPACE";
    case FA2_ERR_HIP: return "FA2_ERR_HIP";
    default: return "FA2_UNKNOWN";
  }
}

int fa2_forward(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
                int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, Hq, Hkv, N, d, scale, &empty);
  if (st != FA2_OK || empty) return st;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA2_ERR_MISALIGNED;
  const uint64_t rows_q = (uint64_t)B * Hq * N, rows_kv = (uint64_t)B * Hkv * N;
  const Range in[3] = {range_of(q, rows_q * d * 2), range_of(k, rows_kv * d * 2),
                       range_of(v, rows_kv * d * 2)};
  const Range out[2] = {range_of(o, rows_q * d * 4), range_of(lse, rows_q * 4)};
  for (const Range& r : out)
    for (const Range& x : in)
      if (overlaps(r, x)) return FA2_ERR_ALIASING;
  if (overlaps(out[0], out[1])) return FA2_ERR_ALIASING;
  fa2::AttnShape s{B, Hq, Hkv, N, d, causal != 0, scale};
  return fa2::launch_forward(q, k, v, o, lse, s, stream) == hipSuccess ? FA2_OK : FA2_ERR_HIP;
}

size_t fa2_backward_workspace_size(int B, int Hq, int N) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  uint64_t bytes = (uint64_t)B * Hq * N * 4;
  return (size_t)((bytes + 255) & ~(uint64_t)255);
}

int fa2_backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
                 const void* dO, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int N,
                 int d, int causal, float scale, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, Hq, Hkv, N, d, scale, &empty);
  if (st != FA2_OK || empty) return st;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA2_ERR_NULL_POINTER;
  if (!workspace || workspace_bytes < fa2_backward_workspace_size(B, Hq, N))
    return FA2_ERR_WORKSPACE;
  const void* ptrs[10] = {q, k, v, o, lse, dO, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA2_ERR_MISALIGNED;
  const uint64_t rows_q = (uint64_t)B * Hq * N, rows_kv = (uint64_t)B * Hkv * N;
  const Range in[6] = {range_of(q, rows_q * d * 2),  range_of(k, rows_kv * d * 2),
                       range_of(v, rows_kv * d * 2), range_of(o, rows_q * d * 4),
                       range_of(lse, rows_q * 4),    range_of(dO, rows_q * d * 2)};
  const Range out[4] = {range_of(dq, rows_q * d * 4), range_of(dk, rows_kv * d * 4),
                        range_of(dv, rows_kv * d * 4),
                        range_of(workspace, fa2_backward_workspace_size(B, Hq, N))};
  for (int i = 0; i < 4; ++i) {
    for (const Range& x : in)
      if (overlaps(out[i], x)) return FA2_ERR_ALIASING;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out[j])) return FA2_ERR_ALIASING;
  }
  fa2::AttnShape s{B, Hq, Hkv, N, d, causal != 0, scale};
  hipError_t e = fa2::launch_backward(q, k, v, o, lse, dO, dq, dk, dv, s,
                                      static_cast<float*>(workspace), stream);
  return e == hipSuccess ? FA2_OK : FA2_ERR_HIP;
}

}  // extern "C"
