"""GPU parity of the sliding-window entry points (fa2_forward_window, fa2_backward_window)
against the fp64 oracle with the same window: query i sees keys max(0, i - W) .. i."""
import math

import numpy as np
import pytest

import exact_tiled_attention_fa2_amd as fa2
import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def run(q, k, v, dO, window, scale, backward=True):
    import torch
    qd, kd, vd = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    o, lse = fa2.forward(qd, kd, vd, True, scale, window=window)
    grads = None
    if backward:
        grads = fa2.backward(qd, kd, vd, o, lse, H.to_dev(dO), True, scale, window=window)
    torch.cuda.synchronize()
    return o, lse, grads


def check_window(seed, B, Hq, Hkv, N, d, W, scale=None, sample=None, backward=True):
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q, k, v, dO = H.make_inputs(seed, B, Hq, Hkv, N, d, with_do=True)
    o, lse, grads = run(q, k, v, dO, W, scale, backward)
    if sample is None:
        qrows = np.tile(np.arange(N, dtype=np.int32), (B * Hq, 1))
        krows = np.tile(np.arange(N, dtype=np.int32), (B * Hkv, 1))
    else:
        qrows = H.sample_rows(seed, B * Hq, N, sample)
        krows = H.sample_rows(seed ^ 0xABCDEF, B * Hkv, N, sample)
    fq, fk, fv, fdo = H.f64(q), H.f64(k), H.f64(v), H.f64(dO)
    ro, rl = oracle.forward(fq, fk, fv, True, scale, rows=qrows, window=W)
    go, gl = H.gather_rows(o, qrows), H.gather_rows(lse, qrows)
    eo, el = H.max_abs(go, ro), H.max_abs(gl, rl)
    msg = "window W=%d B=%d Hq=%d Hkv=%d N=%d d=%d: O %.3e LSE %.3e" % (W, B, Hq, Hkv, N, d, eo, el)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert eo <= H.TOL_O and el <= H.TOL_LSE, msg
    if backward:
        dq, dk, dv = grads
        rdq, rdk, rdv, _ = oracle.backward(fq, fk, fv, fdo, True, scale, qrows=qrows, krows=krows, window=W)
        gdq, gdk, gdv = H.gather_rows(dq, qrows), H.gather_rows(dk, krows), H.gather_rows(dv, krows)
        for name, g in (("dQ", gdq), ("dK", gdk), ("dV", gdv)):
            assert np.all(np.isfinite(g)), name
        eq, ek, ev = H.rel_l2(gdq, rdq), H.rel_l2(gdk, rdk), H.rel_l2(gdv, rdv)
        msg += " dQ %.3e dK %.3e dV %.3e" % (eq, ek, ev)
        assert eq <= H.TOL_GRAD and ek <= H.TOL_GRAD and ev <= H.TOL_GRAD, msg
    print(msg)


# Windows around the 64-key tile and 256-row query block edges, ragged lengths, GQA.
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("W", [0, 1, 31, 63, 64, 65, 100, 255, 256, 300])
def test_window_small_full(W, d):
    check_window(6000 + W, 1, 2, 1, 700, d, W)


@pytest.mark.parametrize("N", [1, 7, 64, 65, 129, 257, 513, 1000])
def test_window_ragged_lengths(N):
    check_window(6100 + N, 1, 2, 2, N, 128, 50)
    check_window(6200 + N, 1, 2, 1, N, 64, 200)


def test_window_head_dim_256():
    check_window(6800, 1, 4, 2, 700, 256, 100)
    check_window(6801, 1, 2, 1, 333, 256, 0)
    # windows ending inside and on the edge of the 32-key quads and 64-key dK/dV workgroups
    check_window(6802, 1, 4, 1, 500, 256, 31)
    check_window(6803, 1, 2, 2, 300, 256, 64)


@pytest.mark.parametrize("Hkv", [1, 2, 8])
def test_window_gqa(Hkv):
    check_window(6300 + Hkv, 2, 8, Hkv, 600, 128, 120)


def test_window_negative_scale():
    check_window(6400, 1, 4, 2, 450, 128, 77, scale=-0.11)


def test_window_long_sampled():
    # Sliding-window prefill shape: 8K tokens, a 1K window.
    check_window(6500, 1, 8, 2, 8192, 128, 1024, sample=256)


def test_window_largest_sequence_accepted():
    # N = 2^22 - 1 at d = 128 with a 1000-key window: workgroups whose first visible tile lies
    # millions of keys into the head, and 32-bit in-head offsets at the top of their range. dK/dV
    # at keys 0, N - 1 and a few between; the oracle's statistics only for the rows that see them.
    B, Hq, Hkv, N, d, W = 1, 1, 1, (1 << 22) - 1, 128, 1000
    scale = 1.0 / math.sqrt(d)
    seed = 0x5EED0A06
    q, k, v, dO = H.make_inputs(seed, B, Hq, Hkv, N, d, with_do=True)
    o, lse, (dq, dk, dv) = run(q, k, v, dO, W, scale)
    keys = np.array([0, 1, 4095, N // 2, N - W - 1, N - W, N - 2, N - 1], dtype=np.int32)
    qrows = np.unique(np.concatenate([H.sample_rows(seed, 1, N, 14)[0], [0, N - 1]])).astype(np.int32)
    seen = np.concatenate([np.arange(j, min(j + W, N - 1) + 1) for j in keys])
    stat_rows = np.unique(np.concatenate([qrows, seen])).astype(np.int32)[None]
    fq, fk, fv, fdo = H.f64(q), H.f64(k), H.f64(v), H.f64(dO)
    ro, rl = oracle.forward(fq, fk, fv, True, scale, rows=qrows[None], window=W)
    go, gl = H.gather_rows(o, qrows[None]), H.gather_rows(lse, qrows[None])
    eo, el = H.max_abs(go, ro), H.max_abs(gl, rl)
    stats = H.causal_row_stats(fq, fk, fv, fdo, scale, stat_rows, window=W)
    rdq, rdk, rdv, _ = oracle.backward(fq, fk, fv, fdo, True, scale, qrows=qrows[None], krows=keys[None],
                                       stats=stats, window=W)
    gdq = H.gather_rows(dq, qrows[None])
    gdk, gdv = H.gather_rows(dk, keys[None]), H.gather_rows(dv, keys[None])
    eq, ek, ev = H.rel_l2(gdq, rdq), H.rel_l2(gdk, rdk), H.rel_l2(gdv, rdv)
    msg = "window W=%d N=%d: O %.3e LSE %.3e dQ %.3e dK %.3e dV %.3e" % (W, N, eo, el, eq, ek, ev)
    print(msg)
    for g in (go, gl, gdq, gdk, gdv):
        assert np.all(np.isfinite(g))
    assert eo <= H.TOL_O and el <= H.TOL_LSE, msg
    assert eq <= H.TOL_GRAD and ek <= H.TOL_GRAD and ev <= H.TOL_GRAD, msg


def test_window_eight_wave_blocks_sampled():
    # windows of more than 4096 keys on long sequences and large grids run 8-wave workgroups
    # (shorter windows run 4-wave ones, like the shapes above)
    check_window(6600, 1, 192, 48, 4500, 128, 4200, sample=32, backward=False)


def test_wide_window_is_causal():
    """A window of N - 1 or more gives exactly fa2_forward / fa2_backward with causal = 1."""
    import torch
    B, Hq, Hkv, N, d = 1, 4, 2, 600, 128
    q, k, v, dO = H.make_inputs(6600, B, Hq, Hkv, N, d, with_do=True)
    qd, kd, vd, dod = H.to_dev(q), H.to_dev(k), H.to_dev(v), H.to_dev(dO)
    o, lse = fa2.forward(qd, kd, vd, True, 0.1)
    grads = fa2.backward(qd, kd, vd, o, lse, dod, True, 0.1)
    for W in (N - 1, N, 1 << 20, 2**31 - 1):  # 2^31 - 1: the usual 'unbounded' sentinel
        ow, lw = fa2.forward(qd, kd, vd, True, 0.1, window=W)
        gw = fa2.backward(qd, kd, vd, ow, lw, dod, True, 0.1, window=W)
        torch.cuda.synchronize()
        assert torch.equal(o, ow) and torch.equal(lse, lw)
        for a, b in zip(grads, gw):
            assert torch.equal(a, b)


def test_window_rejected_without_launch():
    import torch
    q, k, v = (H.to_dev(x) for x in H.make_inputs(6700, 1, 2, 2, 64, 64))
    o = torch.full((1, 2, 64, 64), 5.0, device=q.device)
    lse = torch.full((1, 2, 64), 5.0, device=q.device)
    assert fa2.fa2_forward_window(q, k, v, o, lse, 1, 2, 2, 64, 64, -3, 0.125) == 10
    torch.cuda.synchronize()
    assert bool((o == 5).all() and (lse == 5).all())
