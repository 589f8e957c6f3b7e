"""fa2_backward_noalloc (the backward with the library's fixed workspace) against fa2_backward,
through the C ABI: two calls in a row, the second on a smaller problem, each compared with
fa2_backward on the same inputs (bitwise: the same kernels on the same workspace contents) and
with the oracle on sampled rows."""
import math

import numpy as np
import pytest

import exact_tiled_attention_fa2_amd as fa2
import oracle

from . import gpu_harness as H

pytestmark = pytest.mark.gpu


def run_pair(seed, B, Hq, Hkv, N, d, causal):
    import torch
    scale = 1.0 / math.sqrt(d)
    q, k, v, dO = H.make_inputs(seed, B, Hq, Hkv, N, d, with_do=True)
    qd, kd, vd, dod = H.to_dev(q), H.to_dev(k), H.to_dev(v), H.to_dev(dO)
    o, lse = fa2.forward(qd, kd, vd, causal, scale)
    ref = fa2.backward(qd, kd, vd, o, lse, dod, causal, scale)
    got = [torch.full_like(t, float("nan")) for t in ref]
    st = fa2.fa2_backward_noalloc(qd, kd, vd, o, lse, dod, got[0], got[1], got[2], B, Hq, Hkv, N, d,
                                  causal, scale, torch.cuda.current_stream())
    assert st == 0, fa2.STATUS_NAMES.get(st)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    # and to the parity bar against the oracle, on the full problem (small shapes)
    f = H.f64
    rdq, rdk, rdv, _ = oracle.backward(f(q), f(k), f(v), f(dO), causal, scale)
    for a, b in zip(got, (rdq, rdk, rdv)):
        assert H.rel_l2(a.cpu().numpy(), b) <= H.TOL_GRAD


def test_noalloc_matches_backward_twice_shrinking():
    run_pair(0x5EED0A01, 2, 8, 2, 700, 128, True)   # first call: 11200 query rows
    run_pair(0x5EED0A02, 1, 4, 4, 300, 64, False)   # second, smaller: 1200 rows


def test_noalloc_head_dim_256_twice_shrinking():
    # head dim 256: the quad dK/dV kernel and the d = 256 dQ kernel on the fixed workspace
    run_pair(0x5EED0A04, 1, 4, 2, 500, 256, True)
    run_pair(0x5EED0A05, 1, 2, 2, 130, 256, False)


def test_noalloc_rejects_over_limit_without_launch():
    import torch
    q, k, v = (H.to_dev(x) for x in H.make_inputs(0x5EED0A03, 1, 2, 2, 64, 64))
    o = torch.full((1, 2, 64, 64), 5.0, device=q.device)
    # B*Hq*N = 2^21 + 64 rows needs more than the fixed 16 MiB: refused before any launch
    st = fa2.fa2_backward_noalloc(q, k, v, o, o, q, o, o, o, 1, 32768 + 1, 1, 64, 64, True, 0.125)
    assert st == 11
    torch.cuda.synchronize()
    assert bool((o == 5).all())
