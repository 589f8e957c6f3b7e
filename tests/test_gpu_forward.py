"""GPU forward parity: libfa2's fa2_forward against the fp64 oracle on seeded inputs."""
import math

import numpy as np
import pytest

import exact_tiled_attention_fa2_amd as fa2
import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def run_forward(q, k, v, causal, scale, stream=None):
    import torch
    qd, kd, vd = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    o, lse = fa2.forward(qd, kd, vd, causal, scale, stream=stream)
    torch.cuda.synchronize()
    return o, lse


def check_forward(seed, B, Hq, Hkv, N, d, causal, scale=None, sample=None):
    q, k, v = H.make_inputs(seed, B, Hq, Hkv, N, d)
    return check_forward_on(q, k, v, causal, scale, seed=seed, sample=sample)


def check_forward_on(q, k, v, causal, scale=None, seed=0, sample=None):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = run_forward(q, k, v, causal, scale)
    if sample is None:
        rows = np.tile(np.arange(N, dtype=np.int32), (B * Hq, 1))
    else:
        rows = H.sample_rows(seed, B * Hq, N, sample)
    ro, rl = oracle.forward(H.f64(q), H.f64(k), H.f64(v), causal, scale, rows=rows)
    go = H.gather_rows(o, rows)
    gl = H.gather_rows(lse, rows)
    eo, el = H.max_abs(go, ro), H.max_abs(gl, rl)
    print("fwd B=%d Hq=%d Hkv=%d N=%d d=%d causal=%d scale=%.4g: O err %.3e LSE err %.3e"
          % (B, Hq, Hkv, N, d, causal, scale, eo, el))
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert eo <= H.TOL_O, eo
    assert el <= H.TOL_LSE, el
    return eo, el


# The five workloads: small, medium, LLM-prefill (causal), grouped-query long context.
def test_small_noncausal_full():
    check_forward(0x5EED0001, 1, 2, 2, 256, 64, False)


def test_medium_noncausal_full():
    check_forward(0x5EED0002, 4, 16, 16, 2048, 64, False)


def test_prefill_causal_sampled():
    check_forward(0x5EED0003, 2, 32, 32, 8192, 128, True, sample=256)


def test_gqa_long_causal_sampled():
    check_forward(0x5EED0004, 1, 32, 8, 32768, 128, True, sample=256)


def test_training_shape_forward_sampled():
    check_forward(0x5EED0005, 4, 16, 16, 4096, 128, True, sample=256)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 63, 64, 65, 127, 129, 255, 256, 257, 300, 1000])
def test_ragged_lengths(N, d, causal):
    check_forward(1000 + N, 1, 2, 1, N, d, causal)


@pytest.mark.parametrize("Hkv", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_gqa_ratios(Hkv, d):
    check_forward(77 + Hkv, 2, 8, Hkv, 333, d, True)


# Online-softmax stress: the reference is raised only when a row's tile max passes it by more than
# 8 (log2 units). Keys scaled up along the sequence make almost every tile raise it by a large
# jump; scaled down, later tiles contribute nothing; a huge scale makes each row nearly one-hot.
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("profile", ["growing", "shrinking", "steps"])
def test_score_range_stress(profile, causal, d):
    N = 1000
    q, k, v = H.make_inputs(0x57E5 + d, 1, 4, 2, N, d)
    j = np.arange(N, dtype=np.float64)
    factors = {"growing": 1.0 + j / 8.0,                       # score spread x126 by the end
               "shrinking": 1.0 + (N - 1 - j) / 8.0,
               "steps": 2.0 ** np.floor(j / 64.0) / 64.0}[profile]  # doubles every tile
    check_forward_on(q, H.scale_rows(k, factors), v, causal, seed=0x57E5)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_near_one_hot_rows(causal, d):
    q, k, v = H.make_inputs(0x57E6, 1, 4, 4, 700, d)
    check_forward_on(q, k, v, causal, scale=8.0, seed=0x57E6)


def test_largest_sequence_accepted():
    # N = 2^22 - 1 is the longest sequence accepted at d = 128 (fp32 rows of one head stay under
    # 2^31 bytes); every buffer's 32-bit in-head offsets reach the top of their range here.
    check_forward(0x5EED0A00, 1, 1, 1, (1 << 22) - 1, 128, True, sample=24)


def test_largest_sequence_accepted_head_dim_256():
    # N = 2^21 - 1 at d = 256 (the split-role kernel): fp32 rows of one head just under 2^31 bytes
    check_forward(0x5EED0A01, 1, 1, 1, (1 << 21) - 1, 256, True, sample=16)


def test_largest_sequence_accepted_head_dim_64():
    # N = 2^23 - 1 at d = 64: the same limit, the longest key walk any forward runs
    check_forward(0x5EED0A02, 1, 1, 1, (1 << 23) - 1, 64, True, sample=16)


# At d = 128, workgroups hold 8 waves (256 query rows) when the grid of such blocks reaches four
# per CU for causal N >= 2048 (B*Hq*ceil(N/256) >= 1024), six per CU for non-causal N > 4096, else 4
# waves (128 rows); the shapes above mostly run 4-wave blocks, these 8-wave ones, with ragged ends,
# grouped heads and both mask modes.
def _eight_waves(B, Hq, N, causal):
    wg8 = B * Hq * ((N + 255) // 256)
    return N >= 2048 and wg8 >= 1024 if causal else N > 4096 and wg8 >= 1536


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [(1, 192, 48, 4200, 128, True), (1, 96, 96, 4500, 128, False),
                                                 (2, 64, 8, 4353, 128, False), (1, 128, 128, 5000, 128, True),
                                                 (2, 48, 16, 2900, 128, True), (8, 16, 16, 2048, 128, True)])
def test_eight_wave_blocks_sampled(B, Hq, Hkv, N, d, causal):
    assert d == 128 and _eight_waves(B, Hq, N, causal)
    check_forward(0x8A0 + N + Hq, B, Hq, Hkv, N, d, causal, sample=48)


@pytest.mark.parametrize("B,Hq", [(1, 3), (3, 5), (2, 4), (1, 16)])
def test_head_counts_and_grid_mapping(B, Hq):
    # B*Hq divisible by 8 uses the per-XCD head mapping, otherwise the plain one.
    check_forward(500 + B * Hq, B, Hq, 1, 777, 128, True)
    check_forward(600 + B * Hq, B, Hq, Hq, 520, 64, False)


@pytest.mark.parametrize("scale", [-0.2, 0.01, 1.0, 3.0])
def test_scales(scale):
    check_forward(900, 1, 4, 2, 300, 128, True, scale=scale)
    check_forward(901, 1, 4, 4, 200, 64, False, scale=scale)


def test_closed_forms_on_gpu():
    """q = 0: O_i = mean of the visible V rows, LSE_i = ln(count); causal row 0 = V_0."""
    B, Hq, Hkv, N, d = 1, 2, 1, 300, 128
    q, k, v = H.make_inputs(31, B, Hq, Hkv, N, d)
    q0 = np.zeros_like(q)
    vv = H.f64(v)
    for causal in (False, True):
        o, lse = run_forward(q0, k, v, causal, 0.125)
        o = o.cpu().numpy(); lse = lse.cpu().numpy()
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        mean = np.cumsum(vv[0, 0], axis=0) / cnt[:, None] if causal else np.broadcast_to(vv[0, 0].mean(0), (N, d))
        for h in range(Hq):
            assert H.max_abs(o[0, h], mean) <= 2e-3
            assert H.max_abs(lse[0, h], np.log(cnt)) <= 1e-4
    o, lse = run_forward(q, k, v, True, 0.125)
    assert H.max_abs(o.cpu().numpy()[0, :, 0], np.broadcast_to(vv[0, 0, 0], (Hq, d))) <= 1e-6


def test_deterministic_and_stream():
    import torch
    q, k, v = H.make_inputs(44, 2, 8, 2, 1500, 128)
    o1, l1 = run_forward(q, k, v, True, 0.09)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = run_forward(q, k, v, True, 0.09, stream=s)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_rejected_call_writes_nothing():
    import torch
    q, k, v = H.make_inputs(5, 1, 2, 2, 64, 64)
    qd, kd, vd = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    o = torch.full((1, 2, 64, 64), 7.0, device=qd.device)
    lse = torch.full((1, 2, 64), 7.0, device=qd.device)
    st = fa2.fa2_forward(qd, kd, vd, o, lse, 1, 2, 2, 64, 96, 0, 0.1)
    assert st == 3  # FA2_ERR_UNSUPPORTED_HEAD_DIM
    st = fa2.fa2_forward(qd, kd, vd, o, lse, 1, 2, 2, 64, 64, 0, float("nan"))
    assert st == 5
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())


# Head dim 256 without a window: split roles (A waves: S, softmax, O columns 0-127; B waves: O
# columns 128-255 from P in LDS, with A's rescale factors), 128-row blocks, 32-key tiles.
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 128, 129, 300, 1000])
def test_head_dim_256_ragged(N, causal):
    check_forward(8000 + N, 1, 2, 1, N, 256, causal)


def test_head_dim_256_gqa_and_long():
    check_forward(8100, 2, 8, 2, 777, 256, True)
    check_forward(8101, 1, 4, 4, 4096, 256, True, sample=256)
    check_forward(8102, 1, 4, 2, 2048, 256, False, scale=-0.05)
    check_forward(8103, 1, 2, 1, 65536, 256, True, sample=24)
