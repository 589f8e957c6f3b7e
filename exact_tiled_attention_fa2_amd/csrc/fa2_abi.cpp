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

// Head dims each entry point supports.
enum HeadDims { DIMS_64_128, DIMS_64_128_256 };

bool head_dim_ok(int d, HeadDims dims) {
  return d == 64 || d == 128 || (dims == DIMS_64_128_256 && d == 256);
}

// Shared shape checks. Returns FA2_OK and sets *empty when nothing needs computing.
int check_shape(int B, int Hq, int Hkv, int N, int d, float scale, bool* empty,
                HeadDims dims = DIMS_64_128) {
  *empty = false;
  if (B < 0 || N < 0 || Hq < 0 || Hkv < 0) return FA2_ERR_BAD_SHAPE;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA2_ERR_BAD_GQA;
  if (!head_dim_ok(d, dims)) return FA2_ERR_UNSUPPORTED_HEAD_DIM;
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

struct Buf {
  const void* p;
  uint64_t bytes;
};

// NULL, alignment and overlap rules for one call: outputs must not overlap inputs or each
// other; inputs may overlap each other (they are only read).
int check_buffers(const Buf* in, int nin, const Buf* out, int nout) {
  for (int i = 0; i < nin; ++i)
    if (!in[i].p) return FA2_ERR_NULL_POINTER;
  for (int i = 0; i < nout; ++i)
    if (!out[i].p) return FA2_ERR_NULL_POINTER;
  for (int i = 0; i < nin; ++i)
    if (!aligned16(in[i].p)) return FA2_ERR_MISALIGNED;
  for (int i = 0; i < nout; ++i)
    if (!aligned16(out[i].p)) return FA2_ERR_MISALIGNED;
  for (int i = 0; i < nout; ++i) {
    const Range r = range_of(out[i].p, out[i].bytes);
    for (int j = 0; j < nin; ++j)
      if (overlaps(r, range_of(in[j].p, in[j].bytes))) return FA2_ERR_ALIASING;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(r, range_of(out[j].p, out[j].bytes))) return FA2_ERR_ALIASING;
  }
  return FA2_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA2_OK : FA2_ERR_HIP; }

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
    case FA2_ERR_BAD_WINDOW: return "FA2_ERR_BAD_WINDOW";
    case FA2_ERR_SCRATCH_LIMIT: return "FA2_ERR_SCRATCH_LIMIT";
    default: return "FA2_UNKNOWN";
  }
}

}  // extern "C"

namespace {

int forward_impl(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
                 int Hkv, int N, int d, int causal, int window, float scale, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, Hq, Hkv, N, d, scale, &empty, DIMS_64_128_256);
  if (st != FA2_OK || empty) return st;
  const uint64_t rq = (uint64_t)B * Hq * N, rkv = (uint64_t)B * Hkv * N;
  const Buf in[3] = {{q, rq * d * 2}, {k, rkv * d * 2}, {v, rkv * d * 2}};
  const Buf out[2] = {{o, rq * d * 4}, {lse, rq * 4}};
  st = check_buffers(in, 3, out, 2);
  if (st != FA2_OK) return st;
  // A window that hides nothing (window >= N - 1) is plain causal attention: the same launch
  // configuration and kernels as fa2_forward, so the results are bitwise those of causal.
  if (window >= N - 1) window = -1;
  fa2::AttnShape s{B, Hq, Hkv, N, d, causal != 0, scale, window};
  return hip_status(fa2::launch_forward(q, k, v, o, lse, s, stream));
}

}  // namespace

extern "C" {

int fa2_forward(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
                int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  return forward_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, -1, scale, stream);
}

int fa2_forward_window(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                       int Hq, int Hkv, int N, int d, int window, float scale, hipStream_t stream) {
  if (window < 0) return FA2_ERR_BAD_WINDOW;
  return forward_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, 1, window, scale, stream);
}

size_t fa2_backward_workspace_size(int B, int Hq, int N) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  uint64_t bytes = (uint64_t)B * Hq * N * 8;
  return (size_t)((bytes + 255) & ~(uint64_t)255);
}

namespace {

// The workspace is written by the preprocess and read by the other two steps.
int check_workspace(const void* ws, size_t ws_bytes, int B, int Hq, int N) {
  if (!ws || ws_bytes < fa2_backward_workspace_size(B, Hq, N)) return FA2_ERR_WORKSPACE;
  return FA2_OK;
}

}  // namespace

}  // extern "C"

namespace fa2 {

int backward_check_args(const void* q, const void* k, const void* v, const float* o,
                        const float* lse, const void* dO, float* dq, float* dk, float* dv, int B,
                        int Hq, int Hkv, int N, int d, float scale, bool* empty) {
  int st = check_shape(B, Hq, Hkv, N, d, scale, empty, DIMS_64_128_256);
  if (st != FA2_OK || *empty) return st;
  const uint64_t rq = (uint64_t)B * Hq * N, rkv = (uint64_t)B * Hkv * N;
  const Buf in[6] = {{q, rq * d * 2}, {k, rkv * d * 2}, {v, rkv * d * 2},
                     {o, rq * d * 4}, {lse, rq * 4},     {dO, rq * d * 2}};
  const Buf out[3] = {{dq, rq * d * 4}, {dk, rkv * d * 4}, {dv, rkv * d * 4}};
  return check_buffers(in, 6, out, 3);
}

}  // namespace fa2

namespace {

int backward_impl(const void* q, const void* k, const void* v, const float* o, const float* lse,
                  const void* dO, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int N,
                  int d, int causal, int window, float scale, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  bool empty = false;
  int st = fa2::backward_check_args(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d, scale, &empty);
  if (st != FA2_OK || empty) return st;
  const uint64_t rq = (uint64_t)B * Hq * N, rkv = (uint64_t)B * Hkv * N;
  const Buf in[6] = {{q, rq * d * 2}, {k, rkv * d * 2}, {v, rkv * d * 2},
                     {o, rq * d * 4}, {lse, rq * 4},     {dO, rq * d * 2}};
  const Buf out[3] = {{dq, rq * d * 4}, {dk, rkv * d * 4}, {dv, rkv * d * 4}};
  st = check_workspace(workspace, workspace_bytes, B, Hq, N);
  if (st != FA2_OK) return st;
  const Buf all_in[9] = {in[0], in[1], in[2], in[3], in[4], in[5], out[0], out[1], out[2]};
  const Buf ws[1] = {{workspace, fa2_backward_workspace_size(B, Hq, N)}};
  st = check_buffers(all_in, 9, ws, 1);
  if (st != FA2_OK) return st;
  if (window >= N - 1) window = -1;  // hides nothing: plain causal, as in forward_impl
  fa2::AttnShape s{B, Hq, Hkv, N, d, causal != 0, scale, window};
  float* w = static_cast<float*>(workspace);
  hipError_t e = fa2::launch_bwd_dq_pre(q, k, v, dO, o, lse, w, dq, s, stream);
  if (e == hipSuccess) e = fa2::launch_bwd_dkdv(q, k, v, dO, w, dk, dv, s, stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

int fa2_backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
                 const void* dO, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int N,
                 int d, int causal, float scale, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d, causal, -1, scale,
                       workspace, workspace_bytes, stream);
}

int fa2_backward_window(const void* q, const void* k, const void* v, const float* o,
                        const float* lse, const void* dO, float* dq, float* dk, float* dv, int B,
                        int Hq, int Hkv, int N, int d, int window, float scale, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  if (window < 0) return FA2_ERR_BAD_WINDOW;
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d, 1, window, scale,
                       workspace, workspace_bytes, stream);
}

size_t fa2_forward_fp8_workspace_size(int B, int Hkv, int N, int d) {
  if (B <= 0 || Hkv <= 0 || N <= 0 || d != 128) return 0;
  fa2::AttnShape s{B, Hkv, Hkv, N, d, 0, 1.0f};
  return fa2::forward_fp8_workspace_bytes(s);
}

int fa2_forward_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                    float v_scale, float* o, float* lse, int B, int Hq, int Hkv, int N, int d,
                    int causal, float scale, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  if (B < 0 || N < 0 || Hq < 0 || Hkv < 0) return FA2_ERR_BAD_SHAPE;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA2_ERR_BAD_GQA;
  if (d != 128) return FA2_ERR_UNSUPPORTED_HEAD_DIM;
  if (!isfinite(scale) || scale == 0.0f) return FA2_ERR_BAD_SCALE;
  for (float f : {q_scale, k_scale, v_scale})
    if (!isfinite(f) || !(f > 0.0f)) return FA2_ERR_BAD_SCALE;
  bool empty = false;
  int st = check_shape(B, Hq, Hkv, N, d, scale, &empty);
  if (st != FA2_OK || empty) return st;
  const uint64_t rq = (uint64_t)B * Hq * N, rkv = (uint64_t)B * Hkv * N;
  const Buf in[3] = {{q, rq * d}, {k, rkv * d}, {v, rkv * d}};
  const Buf out[2] = {{o, rq * d * 4}, {lse, rq * 4}};
  st = check_buffers(in, 3, out, 2);
  if (st != FA2_OK) return st;
  const size_t need = fa2_forward_fp8_workspace_size(B, Hkv, N, d);
  if (!workspace || workspace_bytes < need) return FA2_ERR_WORKSPACE;
  const Buf all[5] = {in[0], in[1], in[2], out[0], out[1]};
  const Buf ws[1] = {{workspace, need}};
  st = check_buffers(all, 5, ws, 1);
  if (st != FA2_OK) return st;
  fa2::AttnShape s{B, Hq, Hkv, N, d, causal != 0, scale};
  return hip_status(fa2::launch_forward_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, s, workspace, stream));
}

size_t fa2_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || Hq % Hkv || (d != 64 && d != 128)) return 0;
  fa2::AttnShape s{B, Hq, Hkv, 0, d, 0, 1.0f};
  return fa2::decode_workspace_bytes(s, Nq, Nk);
}

int fa2_decode(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
               int Hkv, int Nq, int Nk, int d, int causal, float scale, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || Nq < 0 || Nk < 0 || Hq < 0 || Hkv < 0) return FA2_ERR_BAD_SHAPE;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA2_ERR_BAD_GQA;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED_HEAD_DIM;
  if (!isfinite(scale) || scale == 0.0f) return FA2_ERR_BAD_SCALE;
  if (B == 0 || Nq == 0) return FA2_OK;
  if (Nk == 0 || (causal && Nq > Nk)) return FA2_ERR_BAD_SHAPE;  // some row would see no key
  if ((int64_t)Nk * d * 4 >= ((int64_t)1 << 31)) return FA2_ERR_BAD_SHAPE;
  if ((int64_t)(Hq / Hkv) * Nq * d * 4 >= ((int64_t)1 << 31)) return FA2_ERR_BAD_SHAPE;
  if ((int64_t)B * Hq * Nq >= ((int64_t)1 << 28) || (int64_t)B * Hkv >= ((int64_t)1 << 24))
    return FA2_ERR_BAD_SHAPE;
  const uint64_t rq = (uint64_t)B * Hq * Nq, rkv = (uint64_t)B * Hkv * Nk;
  const Buf in[3] = {{q, rq * d * 2}, {k, rkv * d * 2}, {v, rkv * d * 2}};
  const Buf out[2] = {{o, rq * d * 4}, {lse, rq * 4}};
  int st = check_buffers(in, 3, out, 2);
  if (st != FA2_OK) return st;
  const size_t need = fa2_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FA2_ERR_WORKSPACE;
    const Buf all[5] = {in[0], in[1], in[2], out[0], out[1]};
    const Buf ws[1] = {{workspace, need}};
    st = check_buffers(all, 5, ws, 1);
    if (st != FA2_OK) return st;
  }
  fa2::AttnShape s{B, Hq, Hkv, 0, d, causal != 0, scale};
  return hip_status(fa2::launch_decode(q, k, v, o, lse, s, Nq, Nk, static_cast<float*>(workspace), stream));
}

int fa2_backward_preprocess(const float* o, const void* dO, const float* lse, void* workspace,
                            size_t workspace_bytes, int B, int Hq, int N, int d,
                            hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, Hq, 1, N, d, 1.0f, &empty, DIMS_64_128_256);
  if (st != FA2_OK || empty) return st;
  const uint64_t rq = (uint64_t)B * Hq * N;
  const Buf in[3] = {{o, rq * d * 4}, {dO, rq * d * 2}, {lse, rq * 4}};
  st = check_buffers(in, 3, nullptr, 0);
  if (st != FA2_OK) return st;
  st = check_workspace(workspace, workspace_bytes, B, Hq, N);
  if (st != FA2_OK) return st;
  const Buf ws[1] = {{workspace, fa2_backward_workspace_size(B, Hq, N)}};
  st = check_buffers(in, 3, ws, 1);
  if (st != FA2_OK) return st;
  fa2::AttnShape s{B, Hq, 1, N, d, 0, 1.0f};
  return hip_status(fa2::launch_bwd_preprocess(o, dO, lse, static_cast<float*>(workspace), s, stream));
}

int fa2_backward_dkdv(const void* q, const void* k, const void* v, const void* dO,
                      const void* workspace, size_t workspace_bytes, float* dk, float* dv,
                      int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                      hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, Hq, Hkv, N, d, scale, &empty, DIMS_64_128_256);
  if (st != FA2_OK || empty) return st;
  st = check_workspace(workspace, workspace_bytes, B, Hq, N);
  if (st != FA2_OK) return st;
  const uint64_t rq = (uint64_t)B * Hq * N, rkv = (uint64_t)B * Hkv * N;
  const Buf in[5] = {{q, rq * d * 2}, {k, rkv * d * 2}, {v, rkv * d * 2}, {dO, rq * d * 2},
                     {workspace, fa2_backward_workspace_size(B, Hq, N)}};
  const Buf out[2] = {{dk, rkv * d * 4}, {dv, rkv * d * 4}};
  st = check_buffers(in, 5, out, 2);
  if (st != FA2_OK) return st;
  fa2::AttnShape s{B, Hq, Hkv, N, d, causal != 0, scale};
  return hip_status(fa2::launch_bwd_dkdv(q, k, v, dO, static_cast<const float*>(workspace), dk, dv, s, stream));
}

int fa2_backward_dq_preprocess(const void* q, const void* k, const void* v, const float* o,
                               const float* lse, const void* dO, void* workspace,
                               size_t workspace_bytes, float* dq, int B, int Hq, int Hkv, int N,
                               int d, int causal, float scale, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, Hq, Hkv, N, d, scale, &empty, DIMS_64_128_256);
  if (st != FA2_OK || empty) return st;
  st = check_workspace(workspace, workspace_bytes, B, Hq, N);
  if (st != FA2_OK) return st;
  const uint64_t rq = (uint64_t)B * Hq * N, rkv = (uint64_t)B * Hkv * N;
  const Buf in[6] = {{q, rq * d * 2}, {k, rkv * d * 2}, {v, rkv * d * 2},
                     {o, rq * d * 4}, {lse, rq * 4},     {dO, rq * d * 2}};
  const Buf out[2] = {{dq, rq * d * 4}, {workspace, fa2_backward_workspace_size(B, Hq, N)}};
  st = check_buffers(in, 6, out, 2);
  if (st != FA2_OK) return st;
  fa2::AttnShape s{B, Hq, Hkv, N, d, causal != 0, scale};
  return hip_status(fa2::launch_bwd_dq_pre(q, k, v, dO, o, lse, static_cast<float*>(workspace), dq, s, stream));
}

int fa2_backward_dq(const void* q, const void* k, const void* v, const void* dO,
                    const void* workspace, size_t workspace_bytes, float* dq, int B, int Hq,
                    int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, Hq, Hkv, N, d, scale, &empty, DIMS_64_128_256);
  if (st != FA2_OK || empty) return st;
  st = check_workspace(workspace, workspace_bytes, B, Hq, N);
  if (st != FA2_OK) return st;
  const uint64_t rq = (uint64_t)B * Hq * N, rkv = (uint64_t)B * Hkv * N;
  const Buf in[5] = {{q, rq * d * 2}, {k, rkv * d * 2}, {v, rkv * d * 2}, {dO, rq * d * 2},
                     {workspace, fa2_backward_workspace_size(B, Hq, N)}};
  const Buf out[1] = {{dq, rq * d * 4}};
  st = check_buffers(in, 5, out, 1);
  if (st != FA2_OK) return st;
  fa2::AttnShape s{B, Hq, Hkv, N, d, causal != 0, scale};
  return hip_status(fa2::launch_bwd_dq(q, k, v, dO, static_cast<const float*>(workspace), dq, s, stream));
}

}  // extern "C"
