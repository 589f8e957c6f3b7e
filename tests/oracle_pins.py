"""Pins of the fp64 oracle: facts fixed by the mathematics, not by the oracle itself.

Each ``pin_*`` function takes an :class:`oracle.Oracle` and raises ``AssertionError`` when the
oracle disagrees with the fact it checks. ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with planted mistakes and requires
every mistake to be caught by at least one pin.

The pages print no attention value for any input, so the pins are closed forms of the
standard softmax(scale * Q K^T) V definition, its invariants, hand-worked tiny cases
(``golden/handworked.json``), library routines that compute the same thing (torch's fp64
scaled_dot_product_attention and autograd), and central finite differences for the backward.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), what + ": non-finite values"
    assert err <= tol, "%s: max abs err %.3e > %.1e" % (what, err, tol)


# ----------------------------------------------------------------------------- forward pins

def pin_constant_scores(orc):
    """q = 0 makes every visible score equal: O_i = mean of visible V rows, LSE_i = ln(count)."""
    rng = _rng(1)
    B, Hq, Hkv, N, d = 2, 4, 2, 9, 5
    q = np.zeros((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    for causal in (False, True):
        o, lse = orc.forward(q, k, v, causal, 0.37)
        for b in range(B):
            for hq in range(Hq):
                g = hq // (Hq // Hkv)
                for i in range(N):
                    n = i + 1 if causal else N
                    _close(o[b, hq, i], v[b, g, :n].mean(axis=0), 1e-12, "const-score O")
                    _close(lse[b, hq, i], math.log(n), 1e-12, "const-score LSE")


def pin_causal_first_row(orc):
    """Causal row 0 sees only key 0: O_0 = V_0 and LSE_0 = scale * <q_0, k_0>."""
    rng = _rng(2)
    B, Hq, Hkv, N, d = 1, 2, 1, 6, 7
    q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
    scale = 0.41
    o, lse = orc.forward(q, k, v, True, scale)
    for hq in range(Hq):
        _close(o[0, hq, 0], v[0, 0, 0], 1e-14, "causal row0 O")
        _close(lse[0, hq, 0], scale * float(q[0, hq, 0] @ k[0, 0, 0]), 1e-13, "causal row0 LSE")


def pin_single_key(orc):
    """N = 1: O = V_0 and LSE = scale * <q, k>, causal or not."""
    rng = _rng(3)
    q, k, v = rng.standard_normal((1, 1, 1, 3)), rng.standard_normal((1, 1, 1, 3)), rng.standard_normal((1, 1, 1, 3))
    for causal in (False, True):
        o, lse = orc.forward(q, k, v, causal, 1.7)
        _close(o[0, 0, 0], v[0, 0, 0], 1e-15, "N=1 O")
        _close(lse[0, 0, 0], 1.7 * float(q[0, 0, 0] @ k[0, 0, 0]), 1e-14, "N=1 LSE")


def pin_two_keys_logistic(orc):
    """Two keys: softmax is the logistic of the score gap, O_i = sig(s0-s1) v0 + sig(s1-s0) v1."""
    rng = _rng(4)
    N, d, scale = 2, 3, 0.8
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    o, lse = orc.forward(q, k, v, False, scale)
    for i in range(N):
        gap = scale * float(q[0, 0, i] @ (k[0, 0, 0] - k[0, 0, 1]))
        w0 = 1.0 / (1.0 + math.exp(-gap))
        _close(o[0, 0, i], w0 * v[0, 0, 0] + (1.0 - w0) * v[0, 0, 1], 1e-14, "two-key O")
        s0, s1 = scale * float(q[0, 0, i] @ k[0, 0, 0]), scale * float(q[0, 0, i] @ k[0, 0, 1])
        _close(lse[0, 0, i], np.logaddexp(s0, s1), 1e-14, "two-key LSE")


def pin_dominant_score(orc):
    """A score above all others by a gap G selects its V row: |O_i - V_j*| <= 2 max|V| (N-1) e^-G."""
    rng = _rng(5)
    N, d, scale = 12, 4, 0.5
    k = rng.uniform(-1, 1, (1, 1, N, d))
    k[0, 0, 7] = [100.0, 0.0, 0.0, 0.0]
    q = np.zeros((1, 1, N, d))
    q[0, 0, :, 0] = 1.0
    q[0, 0, :, 1] = rng.uniform(-1, 1, N)
    v = rng.standard_normal((1, 1, N, d))
    o, lse = orc.forward(q, k, v, False, scale)
    for i in range(N):
        s = scale * (k[0, 0] @ q[0, 0, i])
        gap = s[7] - np.max(np.delete(s, 7))
        assert gap >= 40
        bound = 2 * np.abs(v).max() * (N - 1) * math.exp(-gap)
        _close(o[0, 0, i], v[0, 0, 7], max(bound, 1e-14), "dominant O")
        _close(lse[0, 0, i], s[7], 1e-12, "dominant LSE")


def pin_joint_permutation(orc):
    """Permuting key and value rows together leaves non-causal O and LSE unchanged."""
    rng = _rng(6)
    B, Hq, Hkv, N, d = 1, 4, 2, 11, 6
    q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
    perm = rng.permutation(N)
    o1, l1 = orc.forward(q, k, v, False, 0.3)
    o2, l2 = orc.forward(q, k[:, :, perm], v[:, :, perm], False, 0.3)
    _close(o1, o2, 1e-12, "perm O")
    _close(l1, l2, 1e-12, "perm LSE")


def pin_key_shift(orc):
    """Adding u to every key row shifts each score row by scale <q_i,u>: O unchanged, LSE_i += scale <q_i,u>."""
    rng = _rng(7)
    B, Hq, Hkv, N, d = 1, 2, 1, 10, 5
    q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
    u = rng.standard_normal(d)
    for causal in (False, True):
        o1, l1 = orc.forward(q, k, v, causal, 0.6)
        o2, l2 = orc.forward(q, k + u, v, causal, 0.6)
        _close(o1, o2, 1e-12, "shift O")
        _close(l2 - l1, 0.6 * (q @ u), 1e-12, "shift LSE")


def pin_value_affine(orc):
    """O is affine in V: O(a V + b) = a O(V) + b (rows of P sum to one)."""
    rng = _rng(8)
    B, Hq, Hkv, N, d = 1, 2, 2, 8, 4
    q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
    for causal in (False, True):
        o1, _ = orc.forward(q, k, v, causal, 0.9)
        o2, _ = orc.forward(q, k, -2.5 * v + 0.75, causal, 0.9)
        _close(o2, -2.5 * o1 + 0.75, 1e-12, "affine O")


def pin_hand_worked(orc):
    """Tiny cases worked out by hand (golden/handworked.json, derivations inside)."""
    with open(os.path.join(GOLDEN, "handworked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v, dO = (np.array(eval_exprs(c[n]), dtype=np.float64) for n in ("q", "k", "v", "dO"))
        o, lse = orc.forward(q, k, v, c["causal"], c["scale"])
        _close(o, np.array(eval_exprs(c["O"])), 1e-14, c["name"] + " O")
        _close(lse, np.array(eval_exprs(c["LSE"])), 1e-14, c["name"] + " LSE")
        dq, dk, dv, _ = orc.backward(q, k, v, dO, c["causal"], c["scale"])
        _close(dq, np.array(eval_exprs(c["dQ"])), 1e-14, c["name"] + " dQ")
        _close(dk, np.array(eval_exprs(c["dK"])), 1e-14, c["name"] + " dK")
        _close(dv, np.array(eval_exprs(c["dV"])), 1e-14, c["name"] + " dV")


def eval_exprs(x):
    """Fixture values are numbers or strings like "3/4*ln(3)" (math only: ln, numbers, + - * /)."""
    if isinstance(x, list):
        return [eval_exprs(y) for y in x]
    if isinstance(x, str):
        allowed = set("0123456789.+-*/() lnsqrt")
        assert set(x) <= allowed, x
        return float(eval(x, {"__builtins__": {}}, {"ln": math.log, "sqrt": math.sqrt}))
    return float(x)


def pin_torch_sdpa(orc):
    """Agreement with torch's fp64 CPU scaled_dot_product_attention (an independent library routine)."""
    import torch
    import torch.nn.functional as F
    rng = _rng(9)
    for (B, Hq, Hkv, N, d, causal) in [(2, 4, 4, 17, 8, False), (1, 6, 2, 33, 16, True),
                                        (2, 8, 1, 5, 4, True), (1, 2, 2, 64, 32, False)]:
        q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
        scale = 1.0 / math.sqrt(d) * 1.3
        o, lse = orc.forward(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                             enable_gqa=(Hq != Hkv))
        _close(o, ref.numpy(), 1e-12, "sdpa O")
        # LSE through torch.logsumexp of the same library's scores
        kk = tk.repeat_interleave(Hq // Hkv, dim=1)
        s = torch.matmul(tq, kk.transpose(-1, -2).contiguous()) * scale
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, "sdpa LSE")


def pin_sampled_rows_match_full(orc):
    """Row-restricted forward/backward equal the same rows of the full computation."""
    rng = _rng(10)
    B, Hq, Hkv, N, d = 2, 4, 2, 23, 6
    q, k, v, dO = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)))
    rows_q = np.stack([np.sort(rng.choice(N, 5, replace=False)) for _ in range(B * Hq)]).astype(np.int32)
    rows_k = np.stack([np.sort(rng.choice(N, 4, replace=False)) for _ in range(B * Hkv)]).astype(np.int32)
    for causal in (False, True):
        of, lf = orc.forward(q, k, v, causal, 0.5)
        os_, ls = orc.forward(q, k, v, causal, 0.5, rows=rows_q)
        dqf, dkf, dvf, full_stats = orc.backward(q, k, v, dO, causal, 0.5)
        dqs, dks, dvs, _ = orc.backward(q, k, v, dO, causal, 0.5, qrows=rows_q, krows=rows_k)
        part_stats = orc.row_stats(q, k, v, dO, causal, 0.5, rows=rows_q)
        for s in range(B * Hq):
            b, h = divmod(s, Hq)
            for part, full in zip(part_stats, full_stats):
                assert np.array_equal(part[b, h], full[b, h, rows_q[s]])
            assert np.array_equal(os_[b, h], of[b, h, rows_q[s]])
            assert np.array_equal(ls[b, h], lf[b, h, rows_q[s]])
            assert np.array_equal(dqs[b, h], dqf[b, h, rows_q[s]])
        for s in range(B * Hkv):
            b, g = divmod(s, Hkv)
            assert np.array_equal(dks[b, g], dkf[b, g, rows_k[s]])
            assert np.array_equal(dvs[b, g], dvf[b, g, rows_k[s]])


# ---------------------------------------------------------------------------- backward pins

def _loss(orc, q, k, v, dO, causal, scale):
    o, _ = orc.forward(q, k, v, causal, scale, threads=1)
    return float(np.sum(o * dO))


def pin_finite_differences(orc, shapes=None):
    """Gradients of L = sum(O * dO) agree with central differences of the forward (rel. 1e-6)."""
    rng = _rng(11)
    if shapes is None:
        shapes = [(1, hq, hkv, n, d) for (hq, hkv) in ((1, 1), (2, 1), (2, 2))
                  for n in (1, 2, 3, 5, 8) for d in (1, 2, 4)]
    for idx, (B, Hq, Hkv, N, d) in enumerate(shapes):
        for causal in (False, True):
            q, k, v, dO = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)))
            scale = 0.7
            dq, dk, dv, _ = orc.backward(q, k, v, dO, causal, scale, threads=1)
            for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
                fd = np.zeros_like(x)
                it = np.nditer(x, flags=["multi_index"])
                for _ in it:
                    mi = it.multi_index
                    h = 1e-6 * max(1.0, abs(x[mi]))
                    xp = x.copy(); xp[mi] += h
                    xm = x.copy(); xm[mi] -= h
                    args_p = {"q": q, "k": k, "v": v}; args_m = dict(args_p)
                    key = name[1].lower()
                    args_p[key] = xp; args_m[key] = xm
                    fd[mi] = (_loss(orc, args_p["q"], args_p["k"], args_p["v"], dO, causal, scale)
                              - _loss(orc, args_m["q"], args_m["k"], args_m["v"], dO, causal, scale)) / (2 * h)
                ref = max(np.linalg.norm(fd), 1e-3)
                err = np.linalg.norm(g - fd) / ref
                assert np.all(np.isfinite(g)), name + " non-finite"
                assert err <= 1e-6, "FD %s shape %s causal %s rel err %.3e" % (name, (B, Hq, Hkv, N, d), causal, err)


def pin_backward_invariants(orc):
    """sum_j dV_j = sum_i dO_i, sum_j dK_j = 0 (per KV head), D_i = rowsum(dO_i * O_i)."""
    rng = _rng(12)
    B, Hq, Hkv, N, d = 2, 6, 3, 19, 8
    q, k, v, dO = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)))
    G = Hq // Hkv
    for causal in (False, True):
        o, _ = orc.forward(q, k, v, causal, 0.35)
        dq, dk, dv, (m, l, D) = orc.backward(q, k, v, dO, causal, 0.35)
        for b in range(B):
            for g in range(Hkv):
                _close(dv[b, g].sum(axis=0), dO[b, g * G:(g + 1) * G].sum(axis=(0, 1)), 1e-11, "sum dV")
                _close(dk[b, g].sum(axis=0), np.zeros(d), 1e-11, "sum dK")
        _close(D, np.sum(dO * o, axis=-1), 1e-12, "D identity")
        # the statistics reproduce the forward's LSE
        _, lse = orc.forward(q, k, v, causal, 0.35)
        _close(m + np.log(l), lse, 1e-12, "stats LSE")


def pin_torch_autograd(orc):
    """Agreement with torch fp64 autograd through scaled_dot_product_attention (GQA included)."""
    import torch
    import torch.nn.functional as F
    rng = _rng(13)
    for (B, Hq, Hkv, N, d, causal) in [(1, 4, 2, 13, 8, True), (2, 2, 2, 9, 4, False), (1, 8, 2, 21, 16, True)]:
        q, k, v, dO = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)))
        scale = 0.25
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=(Hq != Hkv))
        (out * torch.from_numpy(dO)).sum().backward()
        dq, dk, dv, _ = orc.backward(q, k, v, dO, causal, scale)
        _close(dq, tq.grad.numpy(), 1e-12, "autograd dQ")
        _close(dk, tk.grad.numpy(), 1e-12, "autograd dK")
        _close(dv, tv.grad.numpy(), 1e-12, "autograd dV")


def pin_gqa_equals_expanded(orc):
    """GQA equals MHA on K/V repeated per query head; dK/dV are the group sums of the MHA grads."""
    rng = _rng(14)
    B, Hq, Hkv, N, d = 1, 6, 2, 10, 4
    G = Hq // Hkv
    q, k, v, dO = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)))
    ke, ve = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (False, True):
        o1, l1 = orc.forward(q, k, v, causal, 0.5)
        o2, l2 = orc.forward(q, ke, ve, causal, 0.5)
        _close(o1, o2, 1e-14, "gqa O")
        _close(l1, l2, 1e-14, "gqa LSE")
        dq1, dk1, dv1, _ = orc.backward(q, k, v, dO, causal, 0.5)
        dq2, dk2, dv2, _ = orc.backward(q, ke, ve, dO, causal, 0.5)
        _close(dq1, dq2, 1e-14, "gqa dQ")
        _close(dk1, dk2.reshape(B, Hkv, G, N, d).sum(axis=2), 1e-13, "gqa dK")
        _close(dv1, dv2.reshape(B, Hkv, G, N, d).sum(axis=2), 1e-13, "gqa dV")


# ------------------------------------------------------------------- sliding-window pins

def _band_mask(N, window):
    """True where key j is visible to query i: i - window <= j <= i."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    return (j <= i) & (j >= i - window)


def pin_window_zero_and_one(orc):
    """Window 0: row i sees only key i (O_i = V_i, LSE_i = s_ii). Window 1: two keys, the
    logistic closed form O_i = w V_{i-1} + (1 - w) V_i with w = 1 / (1 + e^(s_ii - s_i,i-1))."""
    rng = _rng(15)
    B, Hq, Hkv, N, d = 1, 4, 2, 11, 6
    q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
    sc = 0.45
    G = Hq // Hkv
    o0, l0 = orc.forward(q, k, v, True, sc, window=0)
    o1, l1 = orc.forward(q, k, v, True, sc, window=1)
    for hq in range(Hq):
        g = hq // G
        for i in range(N):
            sii = sc * float(q[0, hq, i] @ k[0, g, i])
            _close(o0[0, hq, i], v[0, g, i], 1e-12, "window-0 O")
            _close(l0[0, hq, i], sii, 1e-12, "window-0 LSE")
            if i == 0:
                _close(o1[0, hq, 0], v[0, g, 0], 1e-12, "window-1 row 0")
                continue
            sprev = sc * float(q[0, hq, i] @ k[0, g, i - 1])
            w = 1.0 / (1.0 + math.exp(sii - sprev))
            _close(o1[0, hq, i], w * v[0, g, i - 1] + (1 - w) * v[0, g, i], 1e-12, "window-1 O")
            _close(l1[0, hq, i], math.log(math.exp(sii) + math.exp(sprev)), 1e-12, "window-1 LSE")


def pin_window_torch(orc):
    """Forward and backward with a window agree with torch fp64 attention and autograd under an
    explicit band mask; a window of N - 1 or more is plain causal attention."""
    import torch
    import torch.nn.functional as F
    rng = _rng(16)
    for (B, Hq, Hkv, N, d, W) in [(1, 4, 2, 23, 8, 5), (2, 2, 1, 17, 4, 3), (1, 2, 2, 9, 16, 8),
                                  (1, 2, 2, 12, 4, 40)]:
        q, k, v, dO = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)))
        sc = 0.3
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        mask = torch.from_numpy(_band_mask(N, W))
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=sc, enable_gqa=(Hq != Hkv))
        (ref * torch.from_numpy(dO)).sum().backward()
        o, lse = orc.forward(q, k, v, True, sc, window=W)
        _close(o, ref.detach().numpy(), 1e-12, "window sdpa O")
        kk = tk.detach().repeat_interleave(Hq // Hkv, dim=1)
        s = torch.matmul(tq.detach(), kk.transpose(-1, -2).contiguous()) * sc
        s = s.masked_fill(~mask, float("-inf"))
        _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, "window LSE")
        dq, dk, dv, _ = orc.backward(q, k, v, dO, True, sc, window=W)
        _close(dq, tq.grad.numpy(), 1e-12, "window autograd dQ")
        _close(dk, tk.grad.numpy(), 1e-12, "window autograd dK")
        _close(dv, tv.grad.numpy(), 1e-12, "window autograd dV")
        if W >= N - 1:
            oc, lc = orc.forward(q, k, v, True, sc)
            assert np.array_equal(o, oc) and np.array_equal(lse, lc), "wide window != causal"


def pin_window_locality(orc):
    """Keys and values more than W positions before a query do not affect its output."""
    rng = _rng(17)
    B, Hq, Hkv, N, d, W = 1, 2, 1, 20, 5, 4
    q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
    o, lse = orc.forward(q, k, v, True, 0.6, window=W)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :6] = rng.standard_normal((B, Hkv, 6, d)) * 5
    v2[:, :, :6] = rng.standard_normal((B, Hkv, 6, d)) * 5
    o2, lse2 = orc.forward(q, k2, v2, True, 0.6, window=W)
    rows = np.arange(6 + W, N)  # rows whose window starts at key 6 or later
    assert np.array_equal(o[:, :, rows], o2[:, :, rows]) and np.array_equal(lse[:, :, rows], lse2[:, :, rows])
    assert not np.allclose(o[:, :, 6 + W - 1], o2[:, :, 6 + W - 1]), "row 5 + W must see key 5"


# ----------------------------------------------------------------------------- decode pins

def pin_decode_square_is_forward(orc):
    """With Nq = Nk the decode alignment is the ordinary top-left one: decode equals forward."""
    rng = _rng(18)
    B, Hq, Hkv, N, d = 1, 4, 2, 13, 6
    q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
    for causal in (False, True):
        o1, l1 = orc.decode(q, k, v, causal, 0.4)
        o2, l2 = orc.forward(q, k, v, causal, 0.4)
        _close(o1, o2, 1e-13, "decode square O")
        _close(l1, l2, 1e-13, "decode square LSE")


def pin_decode_torch(orc):
    """Agreement with torch fp64 attention under an explicit end-aligned causal mask (query i
    sees keys j <= Nk - Nq + i), grouped-query heads included."""
    import torch
    import torch.nn.functional as F
    rng = _rng(19)
    for (B, Hq, Hkv, Nq, Nk, d) in [(2, 8, 2, 1, 37, 8), (1, 4, 4, 3, 20, 16), (1, 6, 2, 5, 5, 4),
                                    (1, 2, 1, 4, 70, 32)]:
        q = rng.standard_normal((B, Hq, Nq, d))
        k, v = (rng.standard_normal((B, Hkv, Nk, d)) for _ in range(2))
        sc = 0.35
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        mask = torch.from_numpy(np.arange(Nk)[None, :] <= (Nk - Nq + np.arange(Nq))[:, None])
        for causal in (False, True):
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask if causal else None, scale=sc,
                                                 enable_gqa=(Hq != Hkv))
            o, lse = orc.decode(q, k, v, causal, sc)
            _close(o, ref.numpy(), 1e-12, "decode sdpa O")
            s = torch.matmul(tq, tk.repeat_interleave(Hq // Hkv, dim=1).transpose(-1, -2).contiguous()) * sc
            if causal:
                s = s.masked_fill(~mask, float("-inf"))
            _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, "decode LSE")


def pin_decode_single_rows(orc):
    """One decoded row sees the whole cache, causal or not; a one-key cache returns V_0 and
    LSE = scale <q, k_0>."""
    rng = _rng(21)
    q = rng.standard_normal((1, 2, 1, 5))
    k, v = rng.standard_normal((1, 1, 9, 5)), rng.standard_normal((1, 1, 9, 5))
    a = orc.decode(q, k, v, True, 0.7)
    b = orc.decode(q, k, v, False, 0.7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    o, lse = orc.decode(q, k[:, :, :1], v[:, :, :1], True, 0.7)
    for h in range(2):
        _close(o[0, h, 0], v[0, 0, 0], 1e-15, "one-key O")
        _close(lse[0, h, 0], 0.7 * float(q[0, h, 0] @ k[0, 0, 0]), 1e-15, "one-key LSE")


def pin_decode_split_merge(orc):
    """Attention over a cache equals the logsumexp-weighted merge of attention over its two
    halves: LSE = ln(e^LSE1 + e^LSE2), O = e^(LSE1-LSE) O1 + e^(LSE2-LSE) O2."""
    rng = _rng(22)
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 3, 40, 8
    q = rng.standard_normal((B, Hq, Nq, d))
    k, v = (rng.standard_normal((B, Hkv, Nk, d)) for _ in range(2))
    o, lse = orc.decode(q, k, v, False, 0.5)
    o1, l1 = orc.decode(q, k[:, :, :17], v[:, :, :17], False, 0.5)
    o2, l2 = orc.decode(q, k[:, :, 17:], v[:, :, 17:], False, 0.5)
    L = np.logaddexp(l1, l2)
    _close(lse, L, 1e-12, "merged LSE")
    _close(o, np.exp(l1 - L)[..., None] * o1 + np.exp(l2 - L)[..., None] * o2, 1e-12, "merged O")


FORWARD_PINS = [pin_constant_scores, pin_causal_first_row, pin_single_key, pin_two_keys_logistic,
                pin_dominant_score, pin_joint_permutation, pin_key_shift, pin_value_affine,
                pin_torch_sdpa]
BACKWARD_PINS = [pin_backward_invariants, pin_torch_autograd, pin_gqa_equals_expanded]
BOTH_PINS = [pin_hand_worked, pin_sampled_rows_match_full, pin_finite_differences]
WINDOW_PINS = [pin_window_zero_and_one, pin_window_torch, pin_window_locality]
DECODE_PINS = [pin_decode_square_is_forward, pin_decode_torch, pin_decode_single_rows, pin_decode_split_merge]
ALL_PINS = FORWARD_PINS + BACKWARD_PINS + BOTH_PINS + WINDOW_PINS + DECODE_PINS
