"""The C-ABI library on the host: it loads, exports what include/fa2.h declares, and rejects
invalid arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import exact_tiled_attention_fa2_amd as fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa2.LIB_PATH):
        import importlib
        importlib.import_module("exact_tiled_attention_fa2_amd.build").build()
    return fa2.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa2.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(fa2_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fa2.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in fa2.STATUS_NAMES.items():
        assert fa2.fa2_status_string(code) == name
    assert fa2.fa2_status_string(99) == "FA2_UNKNOWN"


def test_workspace_size(lib):
    assert fa2.fa2_backward_workspace_size(4, 16, 4096) == 4 * 16 * 4096 * 8
    assert fa2.fa2_backward_workspace_size(1, 1, 3) == 256
    assert fa2.fa2_backward_workspace_size(1, 1, 33) == 512
    assert fa2.fa2_backward_workspace_size(0, 16, 4096) == 0
    assert fa2.fa2_backward_workspace_size(-1, 16, 4096) == 0


# Fake, distinct, 16-byte-aligned device addresses: never dereferenced because every call
# below is rejected by host-side validation before any launch.
BASE = 1 << 40
def P(i):
    return BASE + i * (1 << 32)


def fwd(**kw):
    a = dict(q=P(0), k=P(1), v=P(2), o=P(3), lse=P(4), B=1, Hq=2, Hkv=1, N=128, d=64, causal=1, scale=0.125)
    a.update(kw)
    return fa2.fa2_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"],
                           a["d"], a["causal"], a["scale"])


def bwd(**kw):
    a = dict(q=P(0), k=P(1), v=P(2), o=P(3), lse=P(4), dO=P(5), dq=P(6), dk=P(7), dv=P(8),
             B=1, Hq=2, Hkv=1, N=128, d=64, causal=1, scale=0.125, ws=P(9), wsb=1 << 20)
    a.update(kw)
    return fa2.fa2_backward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["dq"], a["dk"], a["dv"],
                            a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["scale"],
                            a["ws"], a["wsb"])


@pytest.mark.parametrize("call", [fwd, bwd])
def test_validation_codes(lib, call):
    assert call(d=96) == 3 and call(d=192) == 3 and call(d=32) == 3
    # d = 256 is supported; checked here only together with another invalid argument, so
    # nothing is ever launched on these fake addresses.
    assert call(d=256, scale=0.0) == 5 and call(d=256, q=P(0) + 8) == 6
    assert call(Hq=3, Hkv=2) == 4 and call(Hkv=0) == 4 and call(Hq=0) == 4
    assert call(B=-1) == 2 and call(N=-5) == 2
    assert call(N=1 << 22, d=128) == 2           # N*d*4 bytes >= 2^31
    assert call(scale=float("nan")) == 5 and call(scale=float("inf")) == 5 and call(scale=0.0) == 5
    assert call(q=P(0) + 8) == 6
    assert call(q=None) == 1
    assert call(B=0) == 0 and call(N=0) == 0      # empty problems: nothing to do
    assert call(B=0, q=None) == 0


def test_forward_aliasing(lib):
    assert fwd(o=P(0)) == 7                       # o overlaps q
    assert fwd(lse=P(3) + 4096) == 7              # lse inside o
    assert fwd(o=P(1) + 1024) == 7                # o inside k
    assert fwd(lse=P(2) - 16) == 7                # lse range reaches into v


def test_backward_aliasing_and_workspace(lib):
    assert bwd(dq=P(5)) == 7                      # dq overlaps dO
    assert bwd(dk=P(7) + 16, dv=P(7) + 16) == 7   # dk and dv overlap
    assert bwd(ws=P(4)) == 7                      # workspace overlaps lse
    assert bwd(ws=None) == 8
    assert bwd(wsb=fa2.fa2_backward_workspace_size(1, 2, 128) - 1) == 8
    assert bwd(ws=P(9) + 4) == 6


def test_phase_entry_points_validate(lib):
    W = fa2.fa2_backward_workspace_size(1, 2, 64)
    pre = lambda **k: fa2.fa2_backward_preprocess(k.get("o", P(3)), k.get("dO", P(5)), k.get("lse", P(4)),
                                                  k.get("ws", P(9)), k.get("wsb", W), 1, 2, 64, k.get("d", 64))
    assert pre(d=96) == 3
    assert pre(ws=P(3) + 64) == 7          # workspace overlaps o
    assert pre(o=None) == 1
    assert pre(ws=None) == 8 and pre(wsb=W - 1) == 8
    assert fa2.fa2_backward_preprocess(P(3), P(5), P(4), P(9), W, 0, 2, 64, 64) == 0
    args = [P(0), P(1), P(2), P(5), P(9), W]
    assert fa2.fa2_backward_dkdv(*args, P(7), P(8), 1, 2, 1, 64, 128, 1, float("nan")) == 5
    assert fa2.fa2_backward_dkdv(*args, P(7), P(7), 1, 2, 1, 64, 64, 1, 0.1) == 7
    assert fa2.fa2_backward_dkdv(*args, P(7), P(8), 1, 3, 2, 64, 64, 1, 0.1) == 4
    assert fa2.fa2_backward_dkdv(P(0), P(1), P(2), P(5), P(9), W - 4, P(7), P(8), 1, 2, 1, 64, 64, 1, 0.1) == 8
    assert fa2.fa2_backward_dq(*args, P(0), 1, 2, 1, 64, 64, 1, 0.1) == 7
    assert fa2.fa2_backward_dq(*args, P(9), 1, 2, 1, 64, 64, 1, 0.1) == 7   # dq over the workspace
    assert fa2.fa2_backward_dq(*args, P(6) + 4, 1, 2, 1, 64, 64, 1, 0.1) == 6
    assert fa2.fa2_backward_dq(*args, P(6), 1, 2, 1, 64, 32, 1, 0.1) == 3
    assert fa2.fa2_backward_dq(*args, P(6), 1, 2, 1, 64, 192, 1, 0.1) == 3
    assert fa2.fa2_backward_dkdv(*args, P(7), P(8), 1, 2, 1, 64, 256, 1, 0.0) == 5   # d=256 accepted
    assert pre(d=192) == 3


def test_fused_dq_preprocess_validates(lib):
    W = fa2.fa2_backward_workspace_size(1, 2, 64)

    def dqp(**k):
        a = dict(q=P(0), k=P(1), v=P(2), o=P(3), lse=P(4), dO=P(5), ws=P(9), wsb=W, dq=P(6), B=1, Hq=2, Hkv=1,
                 N=64, d=64, scale=0.1)
        a.update(k)
        return fa2.fa2_backward_dq_preprocess(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["ws"], a["wsb"],
                                              a["dq"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], 1, a["scale"])
    assert dqp(d=96) == 3 and dqp(d=192) == 3
    assert dqp(Hkv=3) == 4
    assert dqp(scale=0.0) == 5
    assert dqp(o=None) == 1 and dqp(lse=None) == 1 and dqp(dq=None) == 1
    assert dqp(ws=None) == 8 and dqp(wsb=W - 1) == 8
    assert dqp(ws=P(3) + 64) == 7          # workspace (written here) overlaps o
    assert dqp(ws=P(6)) == 7               # workspace overlaps dq
    assert dqp(dq=P(4)) == 7               # dq overlaps lse
    assert dqp(dq=P(6) + 4) == 6
    assert dqp(B=0) == 0                   # empty: nothing enqueued


def fwdw(**kw):
    a = dict(q=P(0), k=P(1), v=P(2), o=P(3), lse=P(4), B=1, Hq=2, Hkv=1, N=128, d=64, window=16, scale=0.125)
    a.update(kw)
    return fa2.fa2_forward_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"],
                                  a["d"], a["window"], a["scale"])


def bwdw(**kw):
    a = dict(q=P(0), k=P(1), v=P(2), o=P(3), lse=P(4), dO=P(5), dq=P(6), dk=P(7), dv=P(8),
             B=1, Hq=2, Hkv=1, N=128, d=64, window=16, scale=0.125, ws=P(9), wsb=1 << 20)
    a.update(kw)
    return fa2.fa2_backward_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["dq"], a["dk"],
                                   a["dv"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["window"],
                                   a["scale"], a["ws"], a["wsb"])


@pytest.mark.parametrize("call", [fwdw, bwdw])
def test_window_entry_points_validate(lib, call):
    assert call(window=-1) == 10 and call(window=-100, d=96) == 10   # the window is checked first
    assert call(d=96) == 3 and call(Hq=3, Hkv=2) == 4 and call(scale=0.0) == 5
    assert call(q=P(0) + 8) == 6 and call(q=None) == 1
    assert call(B=0) == 0 and call(N=0) == 0 and call(B=0, window=0) == 0
    assert call(o=P(0)) == 7 if call is fwdw else call(dq=P(5)) == 7


def test_window_backward_workspace(lib):
    assert bwdw(ws=None) == 8
    assert bwdw(wsb=fa2.fa2_backward_workspace_size(1, 2, 128) - 1) == 8


def dec(**kw):
    a = dict(q=P(0), k=P(1), v=P(2), o=P(3), lse=P(4), B=1, Hq=8, Hkv=2, Nq=1, Nk=4096, d=128, causal=1,
             scale=0.1, ws=P(9), wsb=1 << 26)
    a.update(kw)
    return fa2.fa2_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
                          a["d"], a["causal"], a["scale"], a["ws"], a["wsb"])


def test_decode_validation(lib):
    assert dec(d=256) == 3 and dec(d=96) == 3 and dec(Hq=6, Hkv=4) == 4 and dec(scale=float("nan")) == 5
    assert dec(Nk=0) == 2 and dec(Nq=8, Nk=7) == 2 and dec(Nq=-1) == 2
    assert dec(q=None) == 1 and dec(k=P(1) + 4) == 6 and dec(o=P(1)) == 7
    assert dec(Nq=0) == 0 and dec(B=0) == 0
    need = fa2.fa2_decode_workspace_size(1, 8, 2, 1, 4096, 128)
    assert need > 0 and need % 256 == 0
    assert dec(ws=None) == 8 and dec(wsb=need - 1) == 8 and dec(ws=P(3)) == 7


def test_decode_workspace_size(lib):
    # a short cache needs no partial results; degenerate shapes need none either
    assert fa2.fa2_decode_workspace_size(64, 32, 8, 1, 64, 128) == 0
    assert fa2.fa2_decode_workspace_size(1, 8, 2, 1, 0, 128) == 0
    assert fa2.fa2_decode_workspace_size(1, 8, 3, 1, 100, 128) == 0
    big = fa2.fa2_decode_workspace_size(1, 8, 2, 4, 1 << 16, 128)
    R = 4 * 4
    assert big >= 2 * R * 129 * 4 and big % 256 == 0


def test_fp8_validation(lib):
    W = fa2.fa2_forward_fp8_workspace_size(1, 1, 128, 128)
    assert W == 128 * 128 * 2 and fa2.fa2_forward_fp8_workspace_size(1, 1, 128, 64) == 0
    f = lambda **k: fa2.fa2_forward_fp8(k.get("q", P(0)), P(1), P(2), k.get("qs", 0.1), 0.1, k.get("vs", 0.1),
                                        k.get("o", P(3)), P(4), 1, 2, 1, 128, k.get("d", 128), 1, k.get("sc", 0.1),
                                        k.get("ws", P(9)), k.get("wsb", W))
    assert f(d=64) == 3 and f(d=256) == 3 and f(qs=0.0) == 5 and f(vs=-1.0) == 5 and f(qs=float("inf")) == 5
    assert f(sc=0.0) == 5 and f(q=None) == 1 and f(q=P(0) + 4) == 6 and f(o=P(1)) == 7
    assert f(ws=None) == 8 and f(wsb=W - 1) == 8 and f(ws=P(3)) == 7


def test_binding_rejects_strided_views_and_wrong_dtypes(lib):
    # The library reads plain row-major buffers: the binding refuses a strided view (and the
    # conveniences a wrong dtype) before anything reaches it. CPU tensors are fine for this:
    # nothing is launched.
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    view = q[:, :, ::2]
    assert not view.is_contiguous()
    o = torch.zeros(1, 2, 4, 64)
    lse = torch.zeros(1, 2, 4)
    with pytest.raises(ValueError, match="contiguous"):
        fa2.fa2_forward(view, view, view, o, lse, 1, 2, 2, 4, 64, True, 0.125)
    with pytest.raises(TypeError, match="bfloat16"):
        fa2.forward(q.float(), q, q, True, 0.125)
    with pytest.raises(TypeError, match="uint8"):
        fa2.forward_fp8(q, q, q, (1.0, 1.0, 1.0), True, 0.125)


def test_binding_rejects_host_tensors_and_wrong_shapes(lib):
    # The C ABI sees bare pointers: a host buffer or a tensor shorter than the sizes imply would
    # reach the kernels. The torch conveniences refuse both before anything is launched (CPU
    # tensors here, so nothing could be launched anyway).
    import torch
    bf = torch.bfloat16
    q = torch.zeros(1, 4, 64, 64, dtype=bf)
    k = torch.zeros(1, 2, 64, 64, dtype=bf)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa2.forward(q, k, k, True, 0.125)
    with pytest.raises(ValueError, match="k has shape"):
        fa2.forward(q, torch.zeros(1, 2, 32, 64, dtype=bf), k, True, 0.125)
    with pytest.raises(ValueError, match="v has shape"):
        fa2.forward(q, k, torch.zeros(1, 2, 64, 32, dtype=bf), True, 0.125)
    with pytest.raises(ValueError, match="4-D"):
        fa2.forward(q[0], k, k, True, 0.125)
    o = torch.zeros(1, 4, 64, 64)
    lse = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError, match="lse has shape"):
        fa2.backward(q, k, k, o, torch.zeros(1, 4, 63), q, True, 0.125)
    with pytest.raises(ValueError, match="dO has shape"):
        fa2.backward(q, k, k, o, lse, torch.zeros(1, 4, 64, 32, dtype=bf), True, 0.125)
    with pytest.raises(ValueError, match="o has shape"):
        fa2.backward(q, k, k, torch.zeros(1, 2, 64, 64), lse, q, True, 0.125)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa2.backward(q, k, k, o, lse, q, True, 0.125)
    with pytest.raises(ValueError, match="v has shape"):
        fa2.decode(q, k, torch.zeros(1, 2, 65, 64, dtype=bf), True, 0.125)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa2.decode(q[:, :, :1], k, k, True, 0.125)
    u8 = torch.uint8
    with pytest.raises(ValueError, match="k8 has shape"):
        fa2.forward_fp8(torch.zeros(1, 4, 64, 128, dtype=u8), torch.zeros(1, 2, 64, 64, dtype=u8),
                        torch.zeros(1, 2, 64, 128, dtype=u8), (1.0, 1.0, 1.0), True, 0.125)


def test_noalloc_limit_checked_first(lib):
    # fa2_backward_noalloc serves problems whose workspace fits its fixed device buffer; larger
    # ones are refused before anything else (fake pointers: nothing is launched).
    f = lambda B, Hq, N, **k: fa2.fa2_backward_noalloc(P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8),
                                                      B, Hq, k.get("Hkv", 1), N, k.get("d", 64), 1, 0.125)
    assert fa2.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert fa2.fa2_backward_workspace_size(1, 32, 65536) == fa2.NOALLOC_SCRATCH_BYTES  # 2^21 rows fit
    assert f(1, 32, 65536 + 8) == 11 and f(2, 32769, 32) == 11
    assert f(1, 2, 128, d=96) == 3 and f(0, 2, 128) == 0 and f(-1, 2, 128) == 2
