"""GPU backward parity: fa2_backward (fed by fa2_forward's O and LSE) against the fp64 oracle."""
import math

import numpy as np
import pytest

import exact_tiled_attention_fa2_amd as fa2
import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def run_fwd_bwd(q, k, v, dO, causal, scale, stream=None):
    import torch
    qd, kd, vd, dod = H.to_dev(q), H.to_dev(k), H.to_dev(v), H.to_dev(dO)
    o, lse = fa2.forward(qd, kd, vd, causal, scale, stream=stream)
    dq, dk, dv = fa2.backward(qd, kd, vd, o, lse, dod, causal, scale, stream=stream)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def check_backward(seed, B, Hq, Hkv, N, d, causal, scale=None, sample=None):
    q, k, v, dO = H.make_inputs(seed, B, Hq, Hkv, N, d, with_do=True)
    return check_backward_on(q, k, v, dO, causal, scale, seed=seed, sample=sample)


def check_backward_on(q, k, v, dO, causal, scale=None, seed=0, sample=None):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse, dq, dk, dv = run_fwd_bwd(q, k, v, dO, causal, scale)
    if sample is None:
        qrows = np.tile(np.arange(N, dtype=np.int32), (B * Hq, 1))
        krows = np.tile(np.arange(N, dtype=np.int32), (B * Hkv, 1))
    else:
        qrows = H.sample_rows(seed, B * Hq, N, sample)
        krows = H.sample_rows(seed ^ 0xABCDEF, B * Hkv, N, sample)
    rdq, rdk, rdv, _ = oracle.backward(H.f64(q), H.f64(k), H.f64(v), H.f64(dO), causal, scale,
                                       qrows=qrows, krows=krows)
    gdq, gdk, gdv = H.gather_rows(dq, qrows), H.gather_rows(dk, krows), H.gather_rows(dv, krows)
    for name, g in (("dQ", gdq), ("dK", gdk), ("dV", gdv)):
        assert np.all(np.isfinite(g)), name
    eq, ek, ev = H.rel_l2(gdq, rdq), H.rel_l2(gdk, rdk), H.rel_l2(gdv, rdv)
    print("bwd B=%d Hq=%d Hkv=%d N=%d d=%d causal=%d scale=%.4g: dQ %.3e dK %.3e dV %.3e"
          % (B, Hq, Hkv, N, d, causal, scale, eq, ek, ev))
    assert eq <= H.TOL_GRAD and ek <= H.TOL_GRAD and ev <= H.TOL_GRAD
    return dq, dk, dv, dO


def check_backward_long_causal(seed, B, Hq, Hkv, N, d, nq=32, nk=64):
    """Causal backward at a long sequence, checked exactly where that is cheap: dQ at sampled
    query rows (each needs only its own row of the softmax) and dK/dV at the last nk keys (only
    the last nk queries see them). The oracle's row statistics for those rows come from its own
    forward: m = LSE, l = 1, D = dO . O (the identity the CPU pins tie to sum_j P dP)."""
    scale = 1.0 / math.sqrt(d)
    q, k, v, dO = H.make_inputs(seed, B, Hq, Hkv, N, d, with_do=True)
    o, lse, dq, dk, dv = run_fwd_bwd(q, k, v, dO, True, scale)
    qrows = H.sample_rows(seed, B * Hq, N, nq)
    tail = np.arange(N - nk, N, dtype=np.int32)
    stat_rows = np.concatenate([qrows, np.tile(tail, (B * Hq, 1))], axis=1)
    q64, k64, v64, dO64 = H.f64(q), H.f64(k), H.f64(v), H.f64(dO)
    m, l, D = H.causal_row_stats(q64, k64, v64, dO64, scale, stat_rows)
    krows = np.tile(tail, (B * Hkv, 1))
    rdq, rdk, rdv, _ = oracle.backward(q64, k64, v64, dO64, True, scale, qrows=qrows, krows=krows,
                                       stats=(m, l, D))
    gdq, gdk, gdv = H.gather_rows(dq, qrows), H.gather_rows(dk, krows), H.gather_rows(dv, krows)
    eq, ek, ev = H.rel_l2(gdq, rdq), H.rel_l2(gdk, rdk), H.rel_l2(gdv, rdv)
    print("bwd long B=%d Hq=%d Hkv=%d N=%d d=%d: dQ %.3e dK %.3e dV %.3e" % (B, Hq, Hkv, N, d, eq, ek, ev))
    assert eq <= H.TOL_GRAD and ek <= H.TOL_GRAD and ev <= H.TOL_GRAD


def test_prefill_shape_backward_long_rows():
    # the benchmark's workload: B=2, H=32, N=8192, d=128, causal
    check_backward_long_causal(0x5EED0006, 2, 32, 32, 8192, 128)


def test_backward_largest_sequence_accepted():
    # N = 2^22 - 1 at d = 128, the longest sequence fa2_backward accepts: the fp32 dQ/dK/dV and O
    # rows of the head end just under 2^31 bytes, the top of every kernel's 32-bit in-head offsets
    check_backward_long_causal(0x5EED0A03, 1, 1, 1, (1 << 22) - 1, 128, nq=16, nk=64)


def test_backward_largest_sequence_accepted_head_dim_256():
    # N = 2^21 - 1 at d = 256 (quad dK/dV, dQ with one 32-row block per wave)
    check_backward_long_causal(0x5EED0A04, 1, 1, 1, (1 << 21) - 1, 256, nq=16, nk=64)


def check_backward_full_statistics(seed, B, Hq, Hkv, N, d, slices):
    """Causal dK/dV at 256 sampled keys of the given (batch, KV head) slices -- keys 0-15 (whose
    query walks are the longest), key N-1 and 239 drawn keys -- against the oracle with the
    full-row statistics of the query heads that share each KV head; dQ at 256 sampled rows of the
    first query head of each group."""
    scale = 1.0 / math.sqrt(d)
    q, k, v, dO = H.make_inputs(seed, B, Hq, Hkv, N, d, with_do=True)
    o, lse, dq, dk, dv = run_fwd_bwd(q, k, v, dO, True, scale)
    rows = H.sample_rows(seed ^ 0x5A5A, len(slices), N, 256)
    G = Hq // Hkv
    for i, (b, g) in enumerate(slices):
        q64, dO64 = H.f64(q[b:b + 1, g * G:(g + 1) * G]), H.f64(dO[b:b + 1, g * G:(g + 1) * G])
        k64, v64 = H.f64(k[b:b + 1, g:g + 1]), H.f64(v[b:b + 1, g:g + 1])
        rr = rows[i:i + 1]
        assert set(range(16)) <= set(rr[0].tolist()) and N - 1 in rr[0]
        stats = oracle.row_stats(q64, k64, v64, dO64, True, scale)
        rdq, rdk, rdv, _ = oracle.backward(q64, k64, v64, dO64, True, scale, qrows=np.tile(rr, (G, 1)), krows=rr,
                                           stats=stats)
        idx = np.asarray(rr[0], dtype=np.int64)
        gdq = dq[b, g * G].cpu().numpy().astype(np.float64)[idx]
        gdk = dk[b, g].cpu().numpy().astype(np.float64)[idx]
        gdv = dv[b, g].cpu().numpy().astype(np.float64)[idx]
        eq, ek, ev = H.rel_l2(gdq, rdq[0, 0]), H.rel_l2(gdk, rdk[0, 0]), H.rel_l2(gdv, rdv[0, 0])
        print("bwd B%d Hq%d Hkv%d N%d d%d slice (%d, %d), full statistics: dQ %.3e dK %.3e dV %.3e"
              % (B, Hq, Hkv, N, d, b, g, eq, ek, ev))
        assert eq <= H.TOL_GRAD and ek <= H.TOL_GRAD and ev <= H.TOL_GRAD
        # the longest walks on their own: keys 0-15
        assert np.all(idx[:16] == np.arange(16))
        assert H.rel_l2(gdk[:16], rdk[0, 0, :16]) <= H.TOL_GRAD and H.rel_l2(gdv[:16], rdv[0, 0, :16]) <= H.TOL_GRAD


def test_prefill_shape_backward_sampled_keys_full_statistics():
    # the benchmark's workload: B=2, H=32, N=8192, d=128, causal
    check_backward_full_statistics(0x5EED0006, 2, 32, 32, 8192, 128, ((0, 5), (1, 27)))


def test_gqa_long_backward_sampled_keys_full_statistics():
    # B=1, Hq=32, Hkv=8, N=32768: one KV head's dK/dV sums over its four query heads
    check_backward_full_statistics(0x5EED0B00, 1, 32, 8, 32768, 128, ((0, 3),))


def test_head_dim_256_backward_sampled_keys_full_statistics():
    # the d = 256 extra's shape (dK/dV by quads of waves split over head-dim halves)
    check_backward_full_statistics(0x5EED0008, 2, 16, 16, 8192, 256, ((1, 9),))


def test_gqa_long_backward_long_rows():
    check_backward_long_causal(0x5EED0B00, 1, 32, 8, 32768, 128, nq=16)


def test_head_dim_256_backward_long_rows():
    # the d = 256 benchmark extra's shape, B=2, H=16, N=8192 (quad dK/dV, two-stage dQ ring)
    check_backward_long_causal(0x5EED0008, 2, 16, 16, 8192, 256)


def test_training_step_causal_sampled():
    check_backward(0x5EED0005, 4, 16, 16, 4096, 128, True, sample=256)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("profile", ["growing", "shrinking"])
def test_score_range_stress(profile, causal):
    # keys scaled along the sequence: large reference jumps between tiles, or tiles that
    # contribute nothing (the backward recomputes P from the forward's LSE)
    N = 700
    q, k, v, dO = H.make_inputs(0x57E7, 1, 4, 2, N, 128, with_do=True)
    j = np.arange(N, dtype=np.float64)
    factors = 1.0 + (j if profile == "growing" else N - 1 - j) / 8.0
    check_backward_on(q, H.scale_rows(k, factors), v, dO, causal, seed=0x57E7)


def test_near_one_hot_backward():
    q, k, v, dO = H.make_inputs(0x57E8, 1, 4, 2, 500, 128, with_do=True)
    check_backward_on(q, k, v, dO, True, scale=8.0, seed=0x57E8)


def test_small_full():
    check_backward(0x5EED0001, 1, 2, 2, 256, 64, False)
    check_backward(0x5EED0001, 1, 2, 2, 256, 128, True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 63, 64, 65, 127, 128, 129, 200, 257, 500])
def test_ragged_lengths(N, d, causal):
    check_backward(2000 + N, 1, 2, 1, N, d, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 129, 300, 420, 640, 900, 1100])
def test_block_pairing_counts(N, d, causal):
    # One KV head per query head: the dK/dV workgroups take four 128-key blocks each (one from
    # each run of the blocks in length order) and the dQ workgroups pairs of query blocks, so N
    # runs over 1 to 9 key blocks (odd and even counts, a middle block that is its own mirror,
    # workgroups whose last runs are partial or empty) and ragged tails.
    check_backward(2500 + N, 1, 2, 2, N, d, causal)


@pytest.mark.parametrize("Hkv", [1, 2, 4, 8])
def test_gqa_ratios(Hkv):
    check_backward(3000 + Hkv, 2, 8, Hkv, 300, 128, True)
    check_backward(3100 + Hkv, 1, 8, Hkv, 190, 64, False)


@pytest.mark.parametrize("scale", [-0.15, 0.02, 0.7])
def test_scales(scale):
    check_backward(4000, 1, 4, 2, 250, 128, True, scale=scale)
    check_backward(4001, 1, 2, 2, 130, 64, False, scale=scale)


def test_gradient_invariants_on_gpu():
    """sum_j dV_j = sum_i dO_i over the group, sum_j dK_j = 0 (per KV head)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 700, 128
    dq, dk, dv, dO = check_backward(4100, B, Hq, Hkv, N, d, True)
    dv = dv.cpu().numpy().astype(np.float64); dk = dk.cpu().numpy().astype(np.float64)
    do = H.f64(dO)
    G = Hq // Hkv
    for g in range(Hkv):
        want = do[0, g * G:(g + 1) * G].sum(axis=(0, 1))
        assert H.max_abs(dv[0, g].sum(axis=0), want) <= 2e-2 * max(1.0, np.abs(want).max())
        assert np.abs(dk[0, g].sum(axis=0)).max() <= 2e-2 * np.abs(dk[0, g]).sum(axis=0).max()


def test_backward_deterministic_and_stream():
    import torch
    q, k, v, dO = H.make_inputs(4200, 2, 8, 4, 900, 128, with_do=True)
    a = run_fwd_bwd(q, k, v, dO, True, 0.1)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_fwd_bwd(q, k, v, dO, True, 0.1, stream=s)
    s.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_concurrent_calls_on_two_streams():
    """Two host threads drive forward + backward on their own streams at the same time; the
    library keeps no state between calls, so each result equals the one computed alone."""
    import threading
    import torch
    cases = [(H.make_inputs(4250, 2, 8, 2, 1500, 128, with_do=True), True, 0.09),
             (H.make_inputs(4251, 1, 4, 4, 700, 64, with_do=True), False, 0.125)]
    dev = [tuple(H.to_dev(x) for x in arrs) for arrs, _, _ in cases]
    torch.cuda.synchronize()

    def fwd_bwd(i, stream):
        (qd, kd, vd, dod), (_, causal, scale) = dev[i], cases[i]
        o, lse = fa2.forward(qd, kd, vd, causal, scale, stream=stream)
        return (o, lse) + fa2.backward(qd, kd, vd, o, lse, dod, causal, scale, stream=stream)

    alone = [fwd_bwd(i, None) for i in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = [[], []]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(4):
                    results[i].append(fwd_bwd(i, streams[i]))
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for st in streams:
        st.synchronize()
    assert not errors, errors
    for i in range(2):
        assert len(results[i]) == 4
        for res in results[i]:
            for x, y in zip(res, alone[i]):
                assert torch.equal(x, y)


def test_backward_rejects_small_workspace():
    import torch
    q, k, v, dO = H.make_inputs(4300, 1, 2, 2, 64, 64, with_do=True)
    qd, kd, vd, dod = H.to_dev(q), H.to_dev(k), H.to_dev(v), H.to_dev(dO)
    o, lse = fa2.forward(qd, kd, vd, False, 0.125)
    ws = torch.empty(16, dtype=torch.uint8, device=qd.device)
    dq = torch.full((1, 2, 64, 64), 3.0, device=qd.device)
    dk = torch.full((1, 2, 64, 64), 3.0, device=qd.device)
    dv = torch.full((1, 2, 64, 64), 3.0, device=qd.device)
    st = fa2.fa2_backward(qd, kd, vd, o, lse, dod, dq, dk, dv, 1, 2, 2, 64, 64, 0, 0.125, ws, 16)
    assert st == 8
    torch.cuda.synchronize()
    assert bool((dq == 3).all() and (dk == 3).all() and (dv == 3).all())


@pytest.mark.parametrize("d", [64, 128, 256])
def test_phases_match_composed_backward(d):
    """fa2_backward_dq_preprocess then fa2_backward_dkdv, on one stream, give fa2_backward's
    bits; the three-step form (preprocess, dK/dV, dQ) sums D in another order and agrees to
    rounding."""
    import torch
    B, Hq, Hkv, N = 1, 4, 2, 333
    q, k, v, dO = H.make_inputs(4400 + d, B, Hq, Hkv, N, d, with_do=True)
    qd, kd, vd, dod = H.to_dev(q), H.to_dev(k), H.to_dev(v), H.to_dev(dO)
    o, lse = fa2.forward(qd, kd, vd, True, 0.09)
    dq, dk, dv = fa2.backward(qd, kd, vd, o, lse, dod, True, 0.09)
    W = fa2.fa2_backward_workspace_size(B, Hq, N)
    ws = torch.full((W,), 0xFF, dtype=torch.uint8, device=qd.device)   # NaN patterns
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    assert fa2.fa2_backward_dq_preprocess(qd, kd, vd, o, lse, dod, ws, W, dq2, B, Hq, Hkv, N, d, True, 0.09) == 0
    assert fa2.fa2_backward_dkdv(qd, kd, vd, dod, ws, W, dk2, dv2, B, Hq, Hkv, N, d, True, 0.09) == 0
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    ws3 = torch.empty(W, dtype=torch.uint8, device=qd.device)
    dq3, dk3, dv3 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    assert fa2.fa2_backward_preprocess(o, dod, lse, ws3, W, B, Hq, N, d) == 0
    assert fa2.fa2_backward_dkdv(qd, kd, vd, dod, ws3, W, dk3, dv3, B, Hq, Hkv, N, d, True, 0.09) == 0
    assert fa2.fa2_backward_dq(qd, kd, vd, dod, ws3, W, dq3, B, Hq, Hkv, N, d, True, 0.09) == 0
    torch.cuda.synchronize()
    R = B * Hq * N
    w2, w3 = ws.view(torch.float32)[:2 * R], ws3.view(torch.float32)[:2 * R]
    assert float((w2 - w3).abs().max()) <= 1e-6 * (1 + float(w3.abs().max()))
    for a, b in ((dq, dq3), (dk, dk3), (dv, dv3)):
        assert float((a - b).norm() / b.norm()) <= 1e-3


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_preprocess_workspace_layout(d, fused):
    """fa2_backward_preprocess (or fa2_backward_dq_preprocess, which does the same step inside
    the dQ kernel) leaves -D (D_i = sum_c dO_ic O_ic) at floats [0, R) and LSE * log2(e) at
    [R, 2R), R = B*Hq*N, as the header documents."""
    import torch
    B, Hq, Hkv, N = 2, 3, 3, 100 + 31 * fused   # fused: rows past the last 256-row block too
    q, k, v, dO = H.make_inputs(4500 + d, B, Hq, Hkv, N, d, with_do=True)
    qd, kd, vd, dod = H.to_dev(q), H.to_dev(k), H.to_dev(v), H.to_dev(dO)
    o, lse = fa2.forward(qd, kd, vd, True, 0.1)
    W = fa2.fa2_backward_workspace_size(B, Hq, N)
    ws = torch.full((W // 4,), float("nan"), dtype=torch.float32, device=qd.device)
    if fused:
        dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=qd.device)
        assert fa2.fa2_backward_dq_preprocess(qd, kd, vd, o, lse, dod, ws, W, dq, B, Hq, Hkv, N, d, True, 0.1) == 0
    else:
        assert fa2.fa2_backward_preprocess(o, dod, lse, ws, W, B, Hq, N, d) == 0
    torch.cuda.synchronize()
    R = B * Hq * N
    got = ws.cpu().numpy().astype(np.float64)
    o64 = o.cpu().numpy().astype(np.float64)
    want_negd = -np.einsum("bhnc,bhnc->bhn", H.f64(dO), o64).reshape(-1)
    want_lse2 = lse.cpu().numpy().astype(np.float64).reshape(-1) * np.log2(np.e)
    assert np.abs(got[:R] - want_negd).max() <= 1e-5 * (1 + np.abs(want_negd).max())
    assert np.abs(got[R:2 * R] - want_lse2).max() <= 1e-5 * (1 + np.abs(want_lse2).max())
    # -D against the oracle's D = sum_j P_ij dP_ij (a different route to the same value).
    _, _, D = oracle.row_stats(H.f64(q), H.f64(k), H.f64(v), H.f64(dO), True, 0.1)
    assert np.abs(-got[:R] - D.reshape(-1)).max() <= 2e-2 * (1 + np.abs(D).max())


# Head dim 256: dK/dV by quads of waves (S and dP once, dV and dK split over head-dim halves,
# P and dS handed over through LDS; 64-key workgroups, so N = 63, 64, 65, 129 cross their edges),
# dQ with one 32-row block per wave and a two-stage K/V ring.
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 129, 257, 500])
def test_head_dim_256_ragged(N, causal):
    check_backward(9000 + N, 1, 2, 1, N, 256, causal)


def test_head_dim_256_gqa_long_scale():
    check_backward(9100, 2, 8, 2, 400, 256, True)
    check_backward(9101, 1, 4, 4, 2048, 256, True, sample=256)
    check_backward(9102, 1, 4, 2, 300, 256, False, scale=-0.06)
    check_backward(9103, 1, 8, 1, 333, 256, True)  # all query heads on one KV head


@pytest.mark.parametrize("N", [129, 385, 640, 1000])
def test_d256_dq_block_pairs(N):
    # At d = 256 a dQ workgroup takes two pairs of 128-row query blocks: 2 to 8 blocks here.
    check_backward(9200 + N, 1, 2, 2, N, 256, True)
