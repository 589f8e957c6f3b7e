"""Exact tiled attention (FlashAttention-2 style) for AMD MI355X, Python binding.

The compute lives in ``libfa2.so`` (HIP kernels for gfx950 behind a C ABI, declared in
``include/fa2.h``). This module only marshals arguments to it: the functions named like the
C entry points take raw device addresses (ints) or torch tensors and return the C status.
``forward``/``backward`` are thin conveniences that allocate outputs with torch (device
memory and streams only) and raise on a non-zero status.

There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa2.so")

FA2_OK = 0
STATUS_NAMES = {
    0: "FA2_OK", 1: "FA2_ERR_NULL_POINTER", 2: "FA2_ERR_BAD_SHAPE", 3: "FA2_ERR_UNSUPPORTED_HEAD_DIM",
    4: "FA2_ERR_BAD_GQA", 5: "FA2_ERR_BAD_SCALE", 6: "FA2_ERR_MISALIGNED", 7: "FA2_ERR_ALIASING",
    8: "FA2_ERR_WORKSPACE", 9: "FA2_ERR_HIP", 10: "FA2_ERR_BAD_WINDOW", 11: "FA2_ERR_SCRATCH_LIMIT",
}
NOALLOC_SCRATCH_BYTES = 16 << 20  # FA2_NOALLOC_SCRATCH_BYTES
EXPORTED = ("fa2_forward", "fa2_backward", "fa2_backward_workspace_size", "fa2_backward_preprocess",
            "fa2_backward_dkdv", "fa2_backward_dq", "fa2_backward_dq_preprocess", "fa2_forward_window",
            "fa2_backward_window", "fa2_decode_workspace_size", "fa2_decode", "fa2_forward_fp8_workspace_size",
            "fa2_forward_fp8", "fa2_backward_noalloc", "fa2_status_string")

_lib = None


class Fa2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s returned %s (%d)" % (where, STATUS_NAMES.get(status, "?"), status))
        self.status = status


def load() -> ctypes.CDLL:
    """Load libfa2.so; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfa2.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    p, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa2_forward.restype = i
    lib.fa2_forward.argtypes = [p, p, p, p, p, i, i, i, i, i, i, f, p]
    lib.fa2_backward.restype = i
    lib.fa2_backward.argtypes = [p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, f, p, ctypes.c_size_t, p]
    lib.fa2_backward_workspace_size.restype = ctypes.c_size_t
    lib.fa2_backward_workspace_size.argtypes = [i, i, i]
    lib.fa2_backward_preprocess.restype = i
    z = ctypes.c_size_t
    lib.fa2_backward_preprocess.argtypes = [p, p, p, p, z, i, i, i, i, p]
    lib.fa2_backward_dkdv.restype = i
    lib.fa2_backward_dkdv.argtypes = [p, p, p, p, p, z, p, p, i, i, i, i, i, i, f, p]
    lib.fa2_backward_dq.restype = i
    lib.fa2_backward_dq.argtypes = [p, p, p, p, p, z, p, i, i, i, i, i, i, f, p]
    lib.fa2_backward_dq_preprocess.restype = i
    lib.fa2_backward_dq_preprocess.argtypes = [p, p, p, p, p, p, p, z, p, i, i, i, i, i, i, f, p]
    lib.fa2_forward_window.restype = i
    lib.fa2_forward_window.argtypes = [p, p, p, p, p, i, i, i, i, i, i, f, p]
    lib.fa2_backward_window.restype = i
    lib.fa2_backward_window.argtypes = [p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, f, p, z, p]
    lib.fa2_decode_workspace_size.restype = z
    lib.fa2_decode_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.fa2_decode.restype = i
    lib.fa2_decode.argtypes = [p, p, p, p, p, i, i, i, i, i, i, i, f, p, z, p]
    lib.fa2_forward_fp8_workspace_size.restype = z
    lib.fa2_forward_fp8_workspace_size.argtypes = [i, i, i, i]
    lib.fa2_forward_fp8.restype = i
    lib.fa2_forward_fp8.argtypes = [p, p, p, f, f, f, p, p, i, i, i, i, i, i, f, p, z, p]
    lib.fa2_backward_noalloc.restype = i
    lib.fa2_backward_noalloc.argtypes = [p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, f, p]
    lib.fa2_status_string.restype = ctypes.c_char_p
    lib.fa2_status_string.argtypes = [i]
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    # torch tensor: the library reads plain row-major buffers, so a strided view would be
    # read with the wrong layout
    if not x.is_contiguous():
        raise ValueError("tensor arguments must be contiguous (row-major [B, H, N, d]); got strides %s"
                         % (tuple(x.stride()),))
    return x.data_ptr()


def _expect(name, x, dtype):
    if x.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, x.dtype))


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream  # torch.cuda.Stream


def _torch_stream(s, device):
    """Stream for the torch conveniences: the caller's, else torch's current stream on
    ``device`` (so the launch is ordered after the work that produced the inputs there)."""
    if s is not None:
        return s
    import torch
    return torch.cuda.current_stream(device)


def _check_tensors(specs):
    """Host-side checks of the torch conveniences, before anything is launched: every tensor
    lives on one GPU and has the shape the call implies. The C ABI receives bare pointers and
    cannot tell a host buffer or a short tensor from a good one.

    ``specs``: (name, tensor, expected shape tuple)."""
    for name, x, shape in specs:
        if tuple(x.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), tuple(shape)))
    dev = specs[0][1].device
    if dev.type != "cuda":
        raise ValueError("%s must be a GPU tensor, got device %s" % (specs[0][0], dev))
    for name, x, _ in specs:
        if x.device != dev:
            raise ValueError("%s is on %s, expected %s (all tensors on one GPU)" % (name, x.device, dev))


def _four_dims(name, x):
    if x.dim() != 4:
        raise ValueError("%s must be 4-D [B, H, N, d], got shape %s" % (name, tuple(x.shape)))
    return tuple(x.shape)


# ---------------------------------------------------------------- C entry points, same names

def fa2_forward(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream=None) -> int:
    return load().fa2_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                              int(bool(causal)), float(scale), _stream(stream))


def fa2_backward_workspace_size(B, Hq, N) -> int:
    return int(load().fa2_backward_workspace_size(B, Hq, N))


def fa2_backward(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale,
                 workspace, workspace_bytes, stream=None) -> int:
    return load().fa2_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                               _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                               _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa2_backward_preprocess(o, dO, lse, workspace, workspace_bytes, B, Hq, N, d, stream=None) -> int:
    return load().fa2_backward_preprocess(_ptr(o), _ptr(dO), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                                          B, Hq, N, d, _stream(stream))


def fa2_backward_dkdv(q, k, v, dO, workspace, workspace_bytes, dk, dv, B, Hq, Hkv, N, d, causal, scale,
                      stream=None) -> int:
    return load().fa2_backward_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(workspace), int(workspace_bytes),
                                    _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                                    _stream(stream))


def fa2_backward_dq(q, k, v, dO, workspace, workspace_bytes, dq, B, Hq, Hkv, N, d, causal, scale,
                    stream=None) -> int:
    return load().fa2_backward_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(workspace), int(workspace_bytes),
                                  _ptr(dq), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                                  _stream(stream))


def fa2_backward_dq_preprocess(q, k, v, o, lse, dO, workspace, workspace_bytes, dq, B, Hq, Hkv, N, d,
                               causal, scale, stream=None) -> int:
    return load().fa2_backward_dq_preprocess(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                             _ptr(workspace), int(workspace_bytes), _ptr(dq), B, Hq, Hkv,
                                             N, d, int(bool(causal)), float(scale), _stream(stream))


def fa2_forward_window(q, k, v, o, lse, B, Hq, Hkv, N, d, window, scale, stream=None) -> int:
    return load().fa2_forward_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                                     int(window), float(scale), _stream(stream))


def fa2_backward_window(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d, window, scale,
                        workspace, workspace_bytes, stream=None) -> int:
    return load().fa2_backward_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                                      _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(window), float(scale),
                                      _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa2_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d) -> int:
    return int(load().fa2_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d))


def fa2_decode(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, workspace, workspace_bytes,
               stream=None) -> int:
    return load().fa2_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                             int(bool(causal)), float(scale), _ptr(workspace), int(workspace_bytes),
                             _stream(stream))


def fa2_forward_fp8_workspace_size(B, Hkv, N, d) -> int:
    return int(load().fa2_forward_fp8_workspace_size(B, Hkv, N, d))


def fa2_forward_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, scale,
                    workspace, workspace_bytes, stream=None) -> int:
    return load().fa2_forward_fp8(_ptr(q), _ptr(k), _ptr(v), float(q_scale), float(k_scale), float(v_scale),
                                  _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                                  _ptr(workspace), int(workspace_bytes), _stream(stream))


def fa2_backward_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale,
                         stream=None) -> int:
    return load().fa2_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                                       _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                                       _stream(stream))


def fa2_status_string(status: int) -> str:
    return load().fa2_status_string(int(status)).decode()


# ------------------------------------------------------------ torch conveniences (memory only)

def _dims(q, k):
    B, Hq, N, d = _four_dims("q", q)
    Hkv = _four_dims("k", k)[1]
    return B, Hq, Hkv, N, d


def forward(q, k, v, causal: bool, scale: float, stream=None, window: int | None = None):
    """O (fp32) and LSE (fp32) for bf16 device tensors q [B,Hq,N,d], k/v [B,Hkv,N,d].

    ``window`` (with ``causal``): query i sees keys i - window .. i (fa2_forward_window)."""
    import torch
    for name, x in (("q", q), ("k", k), ("v", v)):
        _expect(name, x, torch.bfloat16)
    B, Hq, Hkv, N, d = _dims(q, k)
    _check_tensors([("q", q, (B, Hq, N, d)), ("k", k, (B, Hkv, N, d)), ("v", v, (B, Hkv, N, d))])
    stream = _torch_stream(stream, q.device)
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if window is None:
        st = fa2_forward(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream)
    else:
        if not causal:
            raise ValueError("a sliding window is defined for causal attention only")
        st = fa2_forward_window(q, k, v, o, lse, B, Hq, Hkv, N, d, window, scale, stream)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_forward" if window is None else "fa2_forward_window")
    return o, lse


def backward(q, k, v, o, lse, dO, causal: bool, scale: float, stream=None, workspace=None,
             window: int | None = None):
    """dQ, dK, dV (fp32) of sum(O * dO) for the outputs of :func:`forward` (same ``window``)."""
    import torch
    for name, x in (("q", q), ("k", k), ("v", v), ("dO", dO)):
        _expect(name, x, torch.bfloat16)
    _expect("o", o, torch.float32)
    _expect("lse", lse, torch.float32)
    B, Hq, Hkv, N, d = _dims(q, k)
    specs = [("q", q, (B, Hq, N, d)), ("k", k, (B, Hkv, N, d)), ("v", v, (B, Hkv, N, d)),
             ("o", o, (B, Hq, N, d)), ("lse", lse, (B, Hq, N)), ("dO", dO, (B, Hq, N, d))]
    if workspace is not None:
        specs.append(("workspace", workspace, tuple(workspace.shape)))
    _check_tensors(specs)
    stream = _torch_stream(stream, q.device)
    dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=q.device)
    need = fa2_backward_workspace_size(B, Hq, N)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    if window is None:
        st = fa2_backward(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale,
                          workspace, wbytes, stream)
    else:
        if not causal:
            raise ValueError("a sliding window is defined for causal attention only")
        st = fa2_backward_window(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, N, d, window, scale,
                                 workspace, wbytes, stream)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_backward" if window is None else "fa2_backward_window")
    return dq, dk, dv


def decode(q, k, v, causal: bool, scale: float, stream=None, workspace=None):
    """O (fp32) and LSE (fp32) of q [B,Hq,Nq,d] against the cache k, v [B,Hkv,Nk,d] (bf16);
    causal rows are the newest tokens (row i sees keys j <= Nk - Nq + i)."""
    import torch
    for name, x in (("q", q), ("k", k), ("v", v)):
        _expect(name, x, torch.bfloat16)
    B, Hq, Nq, d = _four_dims("q", q)
    Hkv, Nk = _four_dims("k", k)[1:3]
    specs = [("q", q, (B, Hq, Nq, d)), ("k", k, (B, Hkv, Nk, d)), ("v", v, (B, Hkv, Nk, d))]
    if workspace is not None:
        specs.append(("workspace", workspace, tuple(workspace.shape)))
    _check_tensors(specs)
    stream = _torch_stream(stream, q.device)
    o = torch.empty((B, Hq, Nq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    need = fa2_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = fa2_decode(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, workspace, wbytes, stream)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_decode")
    return o, lse


def forward_fp8(q8, k8, v8, scales, causal: bool, scale: float, stream=None, workspace=None):
    """O, LSE (fp32) of attention over FP8 E4M3FN codes (uint8 device tensors q8 [B,Hq,N,d],
    k8/v8 [B,Hkv,N,d]) standing for codes * (q_scale, k_scale, v_scale) = ``scales``."""
    import torch
    for name, x in (("q8", q8), ("k8", k8), ("v8", v8)):
        _expect(name, x, torch.uint8)
    B, Hq, N, d = _four_dims("q8", q8)
    Hkv = _four_dims("k8", k8)[1]
    specs = [("q8", q8, (B, Hq, N, d)), ("k8", k8, (B, Hkv, N, d)), ("v8", v8, (B, Hkv, N, d))]
    if workspace is not None:
        specs.append(("workspace", workspace, tuple(workspace.shape)))
    _check_tensors(specs)
    stream = _torch_stream(stream, q8.device)
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q8.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device)
    need = fa2_forward_fp8_workspace_size(B, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q8.device)
    st = fa2_forward_fp8(q8, k8, v8, *scales, o, lse, B, Hq, Hkv, N, d, causal, scale, workspace,
                         workspace.numel() * workspace.element_size(), stream)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_forward_fp8")
    return o, lse
