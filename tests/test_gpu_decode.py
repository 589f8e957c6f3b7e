"""GPU parity of fa2_decode (Nq query rows over an Nk-row KV cache, causal aligned to the end of
the cache) against the fp64 oracle's decode on seeded inputs."""
import math

import numpy as np
import pytest

import exact_tiled_attention_fa2_amd as fa2
import oracle
import seedgen
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def decode_inputs(seed, B, Hq, Hkv, Nq, Nk, d):
    q = seedgen.normal_bf16(seed, seedgen.TENSOR_IDS["q"], (B, Hq, Nq, d))
    k = seedgen.normal_bf16(seed, seedgen.TENSOR_IDS["k"], (B, Hkv, Nk, d))
    v = seedgen.normal_bf16(seed, seedgen.TENSOR_IDS["v"], (B, Hkv, Nk, d))
    return q, k, v


def check_decode(seed, B, Hq, Hkv, Nq, Nk, d, causal, scale=None):
    import torch
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q, k, v = decode_inputs(seed, B, Hq, Hkv, Nq, Nk, d)
    o, lse = fa2.decode(H.to_dev(q), H.to_dev(k), H.to_dev(v), causal, scale)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(H.f64(q), H.f64(k), H.f64(v), causal, scale)
    go, gl = o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    eo, el = H.max_abs(go, ro), H.max_abs(gl, rl)
    msg = ("decode B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d split ws=%d: O %.3e LSE %.3e"
           % (B, Hq, Hkv, Nq, Nk, d, causal, fa2.fa2_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d), eo, el))
    print(msg)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl)), msg
    assert eo <= H.TOL_O and el <= H.TOL_LSE, msg
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nk", [1, 2, 63, 64, 65, 300, 1001, 4096])
def test_decode_single_token(Nk, causal, d):
    check_decode(7000 + Nk, 2, 8, 2, 1, Nk, d, causal)


@pytest.mark.parametrize("Hq,Hkv,Nq", [(8, 8, 1), (8, 8, 16), (32, 8, 4), (32, 8, 5), (64, 8, 3), (4, 1, 40)])
def test_decode_row_blocks(Hq, Hkv, Nq):
    # G * Nq rows per KV group: one 32-row block, exactly 32, or several
    check_decode(7100 + Hq + Nq, 1, Hq, Hkv, Nq, 2000, 128, True)
    check_decode(7200 + Hq + Nq, 1, Hq, Hkv, Nq, 777, 64, False)


@pytest.mark.parametrize("Nk", [32768, 65536])
def test_decode_long_cache(Nk):
    # many cache chunks merged per row
    check_decode(7300, 1, 32, 8, 1, Nk, 128, True)
    check_decode(7301, 1, 8, 1, 2, Nk, 128, True)


def test_decode_largest_cache():
    # Nk = 2^22 - 1, the longest cache accepted at d = 128: 32-bit in-head offsets at the top of
    # their range, and 2048 chunks merged per row
    check_decode(7310, 1, 8, 1, 1, (1 << 22) - 1, 128, True)


def test_decode_more_chunks_than_merge_threads():
    # one KV head over 131072 keys: 512 chunks per row, more than the merge has threads
    check_decode(7302, 1, 8, 1, 1, 131072, 128, True)
    check_decode(7303, 1, 4, 1, 1, 131072, 64, False)


def test_decode_square_and_scales():
    check_decode(7400, 1, 4, 2, 300, 300, 128, True)           # Nq = Nk: ordinary causal attention
    check_decode(7401, 1, 4, 2, 7, 500, 128, True, scale=-0.09)
    check_decode(7402, 2, 16, 4, 2, 3000, 64, False, scale=0.3)


def test_decode_near_one_hot_rows():
    # scale 8 on N(0,1) inputs: each row is dominated by one or two keys, spread over the chunks
    check_decode(7403, 2, 8, 2, 3, 5000, 128, True, scale=8.0)
    check_decode(7404, 1, 8, 8, 1, 20000, 64, False, scale=8.0)


def test_decode_deterministic():
    import torch
    q, k, v = (H.to_dev(x) for x in decode_inputs(7500, 4, 32, 8, 2, 20000, 128))
    a = fa2.decode(q, k, v, True, 0.1)
    b = fa2.decode(q, k, v, True, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_small_workspace_rejected():
    import torch
    q, k, v = (H.to_dev(x) for x in decode_inputs(7600, 1, 8, 2, 1, 50000, 128))
    need = fa2.fa2_decode_workspace_size(1, 8, 2, 1, 50000, 128)
    assert need > 0
    o = torch.full((1, 8, 1, 128), 4.0, device=q.device)
    lse = torch.full((1, 8, 1), 4.0, device=q.device)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    assert fa2.fa2_decode(q, k, v, o, lse, 1, 8, 2, 1, 50000, 128, 1, 0.1, ws, need - 256) == 8
    torch.cuda.synchronize()
    assert bool((o == 4).all() and (lse == 4).all())
