"""Pins for the attention oracle that do not reuse its own formula.

Each ``pin_*`` takes an implementation with the oracle's signature
``impl(q, k, v, scale, causal, row_chunk=...) -> (O, lse)`` on float64 [N, d]
slices and raises AssertionError when the implementation disagrees with what
the definition of attention (page "FlashAttention与TensorRT 10集成", section
"算子融合的极致优化": scale, mask, softmax, weighted sum) and mathematics fix.
The same pins run against deliberately broken copies of the oracle in
``test_oracle.py`` to show that each plausible mistake is caught.
"""
from __future__ import annotations

import numpy as np
import torch

try:
    import mpmath
except ImportError:  # pragma: no cover - mpmath ships with this image
    mpmath = None


def _rand(rng, n, d, scale=1.0):
    # values representable in binary16, as real inputs are
    return (rng.standard_normal((n, d)) * scale).astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------- brute force
def brute_force(q, k, v, scale, causal, dps=50):
    """Scalar loops at ``dps`` significant digits.

    lse is formed as ln(sum_j exp(S_ij)) with no max subtraction, and O as
    sum_j exp(S_ij - lse_i) V_j, a different route from the oracle's.
    """
    mpmath.mp.dps = dps
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i in range(n):
        scores = []
        for j in range(k.shape[0]):
            if causal and j > i:
                continue
            acc = mpmath.mpf(0)
            for c in range(d):
                acc += mpmath.mpf(q[i, c]) * mpmath.mpf(k[j, c])
            scores.append((j, mpmath.mpf(scale) * acc))
        if not scores:
            lse[i] = -np.inf
            continue
        total = mpmath.fsum(mpmath.exp(s) for _, s in scores)
        row_lse = mpmath.log(total)
        lse[i] = float(row_lse)
        for c in range(v.shape[1]):
            o[i, c] = float(mpmath.fsum(mpmath.exp(s - row_lse) * mpmath.mpf(v[j, c]) for j, s in scores))
    return o, lse


def pin_brute_force(impl):
    rng = np.random.default_rng(11)
    cases = [(1, 4, 0.5), (2, 3, 0.125), (3, 8, -0.3), (7, 4, 1.7), (16, 8, 0.35), (9, 1, 2.0)]
    for n, d, scale in cases:
        q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
        for causal in (False, True):
            o_ref, lse_ref = brute_force(q, k, v, scale, causal)
            for chunk in (1024, 3):
                o, lse = impl(q, k, v, scale, causal, row_chunk=chunk)
                assert np.abs(o - o_ref).max() <= 1e-12 * max(1.0, np.abs(o_ref).max()), (n, d, causal, chunk)
                assert np.abs(lse - lse_ref).max() <= 1e-12 * max(1.0, np.abs(lse_ref).max()), (n, d, causal, chunk)


# ---------------------------------------------------------------- library case
def pin_torch_sdpa(impl):
    """torch's float64 CPU scaled_dot_product_attention and logsumexp.

    Positive scales only: torch's causal math path takes the square root of
    the scale and returns NaN for a negative one (negative scales are pinned
    by the brute force instead).
    """
    rng = np.random.default_rng(12)
    for n, d, scale in ((5, 16, 0.25), (64, 64, 0.125), (130, 64, 0.125), (97, 128, 1 / np.sqrt(128)), (40, 32, 0.2)):
        q, k, v = _rand(rng, n, d, 2.0), _rand(rng, n, d, 2.0), _rand(rng, n, d)
        tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        for causal in (False, True):
            o_t = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=float(scale))[0, 0]
            s = float(scale) * (tq[0, 0] @ tk[0, 0].transpose(0, 1))
            if causal:
                s = s.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
            lse_t = torch.logsumexp(s, dim=-1)
            for chunk in (1024, 16):
                o, lse = impl(q, k, v, scale, causal, row_chunk=chunk)
                assert np.abs(o - o_t.numpy()).max() <= 1e-10, (n, d, causal, chunk)
                assert np.abs(lse - lse_t.numpy()).max() <= 1e-10 * max(1.0, float(lse_t.abs().max())), (n, d, causal)


# ---------------------------------------------------------------- closed forms
def pin_closed_forms(impl):
    rng = np.random.default_rng(13)
    n, d = 37, 16
    q, k = _rand(rng, n, d, 3.0), _rand(rng, n, d, 3.0)
    # constant V rows -> every output row is that constant
    const = rng.standard_normal(d)
    v = np.broadcast_to(const, (n, d)).copy()
    for causal in (False, True):
        o, _ = impl(q, k, v, 0.7, causal)
        assert np.allclose(o, v, rtol=0, atol=1e-13)
    # a single key returns its V row; lse is its scaled score
    q1, k1, v1 = _rand(rng, 1, d), _rand(rng, 1, d), _rand(rng, 1, d)
    for causal in (False, True):
        o, lse = impl(q1, k1, v1, 0.4, causal)
        assert np.allclose(o, v1, rtol=0, atol=1e-15)
        assert abs(lse[0] - 0.4 * float(q1[0] @ k1[0])) <= 1e-13
    # causal row 0 sees only key 0
    v = _rand(rng, n, d)
    o, lse = impl(q, k, v, 0.3, True)
    assert np.allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) <= 1e-12
    # zero scale: uniform weights -> plain mean (prefix mean when causal)
    o, lse = impl(q, k, v, 0.0, False)
    assert np.allclose(o, np.tile(v.mean(axis=0), (n, 1)), rtol=0, atol=1e-13)
    assert np.allclose(lse, np.log(n), rtol=0, atol=1e-13)
    o, lse = impl(q, k, v, 0.0, True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(o, prefix, rtol=0, atol=1e-13)
    assert np.allclose(lse, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-13)
    # two keys: the weight of key 0 is the logistic function of the score gap
    q2, k2, v2 = _rand(rng, 2, d), _rand(rng, 2, d), _rand(rng, 2, d)
    o, lse = impl(q2, k2, v2, 0.5, False)
    for i in range(2):
        s0, s1 = 0.5 * float(q2[i] @ k2[0]), 0.5 * float(q2[i] @ k2[1])
        w0 = 1.0 / (1.0 + np.exp(s1 - s0))
        assert np.allclose(o[i], w0 * v2[0] + (1 - w0) * v2[1], rtol=0, atol=1e-14)
        assert abs(lse[i] - (max(s0, s1) + np.log1p(np.exp(-abs(s0 - s1))))) <= 1e-13
    # a dominant key (score gap of 60 after scaling) takes all the weight
    kd = np.zeros((n, d)); kd[5, 0] = 1.0
    qd = np.zeros((n, d)); qd[:, 0] = 60.0
    o, _ = impl(qd, kd, v, 1.0, False)
    assert np.allclose(o, np.tile(v[5], (n, 1)), rtol=0, atol=1e-12)
    # scores of 1000 must not overflow: the row maximum is what gets subtracted
    qd[:, 0] = 1000.0
    o, lse = impl(qd, kd, v, 1.0, False)
    assert np.array_equal(o, np.tile(v[5], (n, 1))) and np.array_equal(lse, np.full(n, 1000.0))


# ---------------------------------------------------------------- invariants
def pin_invariants(impl):
    rng = np.random.default_rng(14)
    # V = identity makes O the probability matrix itself
    n = d = 24
    q, k = _rand(rng, n, d, 2.0), _rand(rng, n, d, 2.0)
    eye = np.eye(n)
    for causal in (False, True):
        p, lse = impl(q, k, eye, 0.6, causal, row_chunk=5)
        assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        assert (p >= 0).all() and (p <= 1).all()
        if causal:
            assert not np.triu(p, 1).any()
        # P_ij = exp(S_ij - lse_i): recover the scores from P and lse
        s = 0.6 * q @ k.T
        vis = np.tril(np.ones((n, n), bool)) if causal else np.ones((n, n), bool)
        assert np.allclose(np.log(p[vis]), (s - lse[:, None])[vis], rtol=0, atol=1e-11)
    n, d = 50, 32
    q, k, v = _rand(rng, n, d, 2.0), _rand(rng, n, d, 2.0), _rand(rng, n, d)
    o, lse = impl(q, k, v, 0.3, False)
    # convex combination of V rows
    assert (o <= v.max(axis=0) + 1e-13).all() and (o >= v.min(axis=0) - 1e-13).all()
    # permuting keys and values together changes nothing (no mask)
    perm = rng.permutation(n)
    o2, lse2 = impl(q, k[perm], v[perm], 0.3, False)
    assert np.allclose(o2, o, rtol=0, atol=1e-13) and np.allclose(lse2, lse, rtol=0, atol=1e-12)
    # permuting queries permutes outputs
    o3, lse3 = impl(q[perm], k, v, 0.3, False)
    assert np.allclose(o3, o[perm], rtol=0, atol=1e-13) and np.allclose(lse3, lse[perm], rtol=0, atol=1e-12)
    for causal in (False, True):
        o, lse = impl(q, k, v, 0.3, causal, row_chunk=7)
        # shifting every key by u shifts each score row by scale*q_i.u
        u = rng.standard_normal(d)
        o4, lse4 = impl(q, k + u, v, 0.3, causal, row_chunk=7)
        assert np.allclose(o4, o, rtol=0, atol=1e-12)
        assert np.allclose(lse4, lse + 0.3 * q @ u, rtol=0, atol=1e-11)
        # V -> aV + c maps O -> aO + c
        o5, lse5 = impl(q, k, -2.5 * v + 0.75, 0.3, causal, row_chunk=7)
        assert np.allclose(o5, -2.5 * o + 0.75, rtol=0, atol=1e-12)
        assert np.array_equal(lse5, lse)
        # rows of the causal output only depend on the keys up to them
        if causal:
            m = 20
            o6, lse6 = impl(q[:m], k[:m], v[:m], 0.3, True)
            assert np.allclose(o6, o[:m], rtol=0, atol=1e-13) and np.allclose(lse6, lse[:m], rtol=0, atol=1e-12)


ALL_PINS = (pin_closed_forms, pin_invariants, pin_torch_sdpa, pin_brute_force)
