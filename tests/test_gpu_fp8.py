"""GPU parity of fa2_forward_fp8 (Q, K, V as FP8 E4M3FN codes with per-tensor scales) against the
fp64 oracle on the exactly dequantised values. The bars are the bf16 path's: S = Q K^T of two
E4M3 operands is exact per product in fp32, V is widened exactly, so only accumulation order
and the bf16 rounding of P separate the result from exact attention over those values."""
import math

import numpy as np
import pytest

import exact_tiled_attention_fa2_amd as fa2
import oracle
import seedgen
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def to_dev_u8(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes)).to(H.device())


def check_fp8(seed, B, Hq, Hkv, N, d, causal, scales=(1 / 32, 1 / 32, 1 / 32), scale=None, sample=None):
    import torch
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qs, ks, vs = scales
    q8 = seedgen.normal_e4m3(seed, "q", (B, Hq, N, d), 1.0 / qs)
    k8 = seedgen.normal_e4m3(seed, "k", (B, Hkv, N, d), 1.0 / ks)
    v8 = seedgen.normal_e4m3(seed, "v", (B, Hkv, N, d), 1.0 / vs)
    o, lse = fa2.forward_fp8(to_dev_u8(q8), to_dev_u8(k8), to_dev_u8(v8), scales, causal, scale)
    torch.cuda.synchronize()
    if sample is None:
        rows = np.tile(np.arange(N, dtype=np.int32), (B * Hq, 1))
    else:
        rows = H.sample_rows(seed, B * Hq, N, sample)
    dq = lambda c, s: seedgen.e4m3_to_f64(c) * s
    ro, rl = oracle.forward(dq(q8, qs), dq(k8, ks), dq(v8, vs), causal, scale, rows=rows)
    go, gl = H.gather_rows(o, rows), H.gather_rows(lse, rows)
    eo, el = H.max_abs(go, ro), H.max_abs(gl, rl)
    msg = "fp8 B=%d Hq=%d Hkv=%d N=%d d=%d causal=%d scales=%s: O %.3e LSE %.3e" % (
        B, Hq, Hkv, N, d, causal, scales, eo, el)
    print(msg)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl)), msg
    assert eo <= H.TOL_O and el <= H.TOL_LSE, msg


def test_fp8_prefill_causal_sampled():
    check_fp8(0x5EED0003, 2, 32, 32, 8192, 128, True, sample=256)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 257, 1000])
def test_fp8_ragged(N, causal):
    check_fp8(9500 + N, 1, 2, 1, N, 128, causal)


def test_fp8_gqa_scales_and_sign():
    check_fp8(9600, 2, 8, 2, 700, 128, True, scales=(1 / 16, 1 / 64, 1 / 8))
    check_fp8(9601, 1, 4, 4, 500, 128, False, scales=(0.05, 0.02, 0.5), scale=-0.07)
    check_fp8(9602, 1, 32, 8, 4096, 128, True, sample=128)


def test_fp8_largest_sequence_accepted():
    # N = 2^22 - 1: FP8 Q/K rows of 128 bytes and the widened bf16 V (1 GiB workspace) at the
    # longest sequence fa2_forward_fp8 accepts
    check_fp8(0x5EED0A07, 1, 1, 1, (1 << 22) - 1, 128, True, sample=16)


def test_fp8_eight_wave_blocks_sampled():
    # N > 4096 and B*Hq*ceil(N/256) >= 1536: 8-wave workgroups, ragged end, grouped heads
    check_fp8(9700, 1, 192, 48, 4200, 128, True, sample=48)


def test_fp8_rejects_without_launch():
    import torch
    q8 = to_dev_u8(seedgen.normal_e4m3(9700, "q", (1, 2, 64, 128), 32.0))
    o = torch.full((1, 2, 64, 128), 7.0, device=q8.device)
    lse = torch.full((1, 2, 64), 7.0, device=q8.device)
    ws = torch.empty(fa2.fa2_forward_fp8_workspace_size(1, 2, 64, 128), dtype=torch.uint8, device=q8.device)
    nb = ws.numel()
    assert fa2.fa2_forward_fp8(q8, q8, q8, 0.0, 1.0, 1.0, o, lse, 1, 2, 2, 64, 128, 1, 0.1, ws, nb) == 5
    assert fa2.fa2_forward_fp8(q8, q8, q8, 1.0, 1.0, 1.0, o, lse, 1, 2, 2, 64, 64, 1, 0.1, ws, nb) == 3
    assert fa2.fa2_forward_fp8(q8, q8, q8, 1.0, 1.0, 1.0, o, lse, 1, 2, 2, 64, 128, 1, 0.1, ws, nb - 1) == 8
    torch.cuda.synchronize()
    assert bool((o == 7).all() and (lse == 7).all())
