"""Shared helpers of the GPU parity tests: seeded inputs on the device, oracle comparisons.

Inputs come from ``seedgen`` (the same bf16 bytes go to the GPU library and, widened exactly
to fp64, to the oracle). Expected values come only from ``oracle``.
"""
from __future__ import annotations

import numpy as np

import oracle
import seedgen

# Parity bars for bf16 inputs with fp32 accumulation.
TOL_O = 1e-2        # max-abs error of O
TOL_LSE = 1e-3      # max-abs error of LSE
TOL_GRAD = 2e-2     # relative L2 error of dQ, dK, dV


def device():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray):
    """uint16 bf16 bit patterns -> torch.bfloat16 device tensor (bit-exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device()).view(torch.bfloat16)


def make_inputs(seed, B, Hq, Hkv, N, d, with_do=False):
    return seedgen.attention_inputs(seed, B, Hq, Hkv, N, d, with_do=with_do)


def f64(bits):
    return seedgen.bf16_bits_to_f64(bits)


def gather_rows(t, rows):
    """t [B,H,N,...] (torch) -> numpy [B,H,R,...] at per-slice rows [B*H, R]."""
    import torch
    B, H, N = t.shape[:3]
    flat = t.reshape(B * H, N, *t.shape[3:])
    idx = torch.as_tensor(rows, dtype=torch.long, device=t.device)
    out = flat[torch.arange(B * H, device=t.device)[:, None], idx]
    return out.reshape(B, H, idx.shape[1], *t.shape[3:]).cpu().numpy().astype(np.float64)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def rel_l2(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def sample_rows(seed, nslices, N, count=256):
    return seedgen.sample_rows_all(seed, nslices, N, count)


def causal_row_stats(q64, k64, v64, dO64, scale, stat_rows, window=-1):
    """The oracle's backward row statistics (m, l, D), [B,Hq,N] each, filled only at the per-slice
    rows ``stat_rows`` [B*Hq, R] of a causal problem (with a sliding window if ``window`` >= 0;
    the oracle's row statistics of just those rows). Other entries are left at m = 0, l = 1,
    D = 0 and must not be read (causal dK/dV of the keys whose queries are all in ``stat_rows``,
    and dQ of a row, read only their own rows)."""
    B, Hq, N = q64.shape[:3]
    sm, sl, sD = oracle.row_stats(q64, k64, v64, dO64, True, scale, rows=stat_rows, window=window)
    m = np.zeros((B, Hq, N))
    l = np.ones((B, Hq, N))
    D = np.zeros((B, Hq, N))
    for s in range(B * Hq):
        b, h = divmod(s, Hq)
        m[b, h, stat_rows[s]] = sm[b, h]
        l[b, h, stat_rows[s]] = sl[b, h]
        D[b, h, stat_rows[s]] = sD[b, h]
    return m, l, D


def to_bf16_bits(x):
    """Round finite values to bf16 (round to nearest, ties to even) and return the bit patterns:
    builds test inputs from transformed seeded values (both sides then read the same bytes)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def scale_rows(bits, factors):
    """bf16 tensor [B,H,N,d] with row n multiplied by factors[n], re-rounded to bf16."""
    x = seedgen.bf16_bits_to_f64(bits) * np.asarray(factors, dtype=np.float64)[None, None, :, None]
    return to_bf16_bits(x)

