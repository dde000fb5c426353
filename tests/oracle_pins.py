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


# ------------------------------------------------------------- packed batches
# ``impl_varlen(q, k, v, cu, scale, causal) -> (O [total,H,d], lse [H,total])``
# on packed float64 [total, H, d] inputs.

def _packed(rng, lengths, H, d, scale=1.0):
    total = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    mk = lambda: (rng.standard_normal((total, H, d)) * scale).astype(np.float16).astype(np.float64)
    return mk(), mk(), mk(), cu


def pin_varlen_brute_force(impl_varlen):
    """Every (sequence, head) against the mpmath loops on that sequence's rows
    alone; lengths include empty sequences and single rows."""
    if mpmath is None:  # pragma: no cover
        return
    rng = np.random.default_rng(5)
    lengths = [3, 0, 1, 6, 2]
    H, d = 2, 4
    q, k, v, cu = _packed(rng, lengths, H, d, 1.5)
    for causal in (False, True):
        o, lse = impl_varlen(q, k, v, cu, 0.45, causal)
        assert o.shape == q.shape and lse.shape == (H, q.shape[0])
        for b in range(len(lengths)):
            r0, r1 = cu[b], cu[b + 1]
            for h in range(H):
                ob, lb = brute_force(q[r0:r1, h], k[r0:r1, h], v[r0:r1, h], 0.45, causal)
                assert np.allclose(o[r0:r1, h], ob, rtol=0, atol=1e-12), (b, h, causal)
                assert np.allclose(lse[h, r0:r1], lb, rtol=0, atol=1e-12), (b, h, causal)


def pin_varlen_equal_lengths_are_dense(impl_varlen):
    """Equal lengths: the packed problem is the dense [B, H, N, d] one, whose
    oracle is pinned on its own."""
    from oracle import attention as dense_attention

    rng = np.random.default_rng(6)
    B, N, H, d = 3, 9, 2, 8
    q, k, v, cu = _packed(rng, [N] * B, H, d)
    dense = lambda x: x.reshape(B, N, H, d).transpose(0, 2, 1, 3)
    for causal in (False, True):
        o, lse = impl_varlen(q, k, v, cu, 0.3, causal)
        od, ld = dense_attention(dense(q), dense(k), dense(v), 0.3, causal)
        assert np.allclose(dense(o), od, rtol=0, atol=1e-13)
        assert np.allclose(lse.reshape(H, B, N).transpose(1, 0, 2), ld, rtol=0, atol=1e-12)


def pin_varlen_sequence_order(impl_varlen):
    """Reordering the packed sequences reorders the outputs block by block: no
    row sees another sequence."""
    rng = np.random.default_rng(7)
    lengths = [5, 1, 8, 3]
    H, d = 2, 8
    q, k, v, cu = _packed(rng, lengths, H, d)
    o, lse = impl_varlen(q, k, v, cu, 0.25, True)
    order = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in order])
    cu2 = np.concatenate([[0], np.cumsum([lengths[b] for b in order])])
    o2, lse2 = impl_varlen(q[rows], k[rows], v[rows], cu2, 0.25, True)
    assert np.allclose(o2, o[rows], rtol=0, atol=1e-13)
    assert np.allclose(lse2, lse[:, rows], rtol=0, atol=1e-12)


VARLEN_PINS = (pin_varlen_brute_force, pin_varlen_equal_lengths_are_dense, pin_varlen_sequence_order)


# ------------------------------------------------------------------ backward
# ``impl_bwd(q, k, v, do, scale, causal) -> (dQ, dK, dV)`` on float64 [N, d]
# slices; the forward oracle (pinned above) defines the function differentiated.

def pin_bwd_finite_differences(impl_bwd):
    """Central differences of L = sum(dO * O) through the forward oracle."""
    from oracle import attention_slice

    rng = np.random.default_rng(21)
    for n, d, scale, causal in [(4, 3, 0.7, False), (5, 2, -0.4, True), (1, 3, 0.5, True), (6, 4, 1.1, True)]:
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        dq, dk, dv = impl_bwd(q, k, v, do, scale, causal)
        loss = lambda qq, kk, vv: float((attention_slice(qq, kk, vv, scale, causal)[0] * do).sum())
        eps = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                args_p[name], args_m[name] = xp, xm
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            assert np.allclose(g, num, rtol=1e-6, atol=1e-7), (name, n, d, causal, np.abs(g - num).max())


def pin_bwd_torch_autograd(impl_bwd):
    """torch autograd in float64 on the CPU through explicit softmax attention."""
    rng = np.random.default_rng(22)
    for n, d, scale, causal in [(7, 8, 0.35, False), (9, 4, 0.8, True), (16, 16, 0.25, True)]:
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        s = scale * tq @ tk.T
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        o = torch.softmax(s, dim=1) @ tv
        o.backward(torch.tensor(do))
        dq, dk, dv = impl_bwd(q, k, v, do, scale, causal)
        for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.allclose(mine, ref.numpy(), rtol=0, atol=1e-10)


def pin_bwd_identities(impl_bwd):
    """Sums fixed by the softmax: rows of P sum to 1 and rows of dS to 0, so
    sum_j dV_j = sum_i dO_i and sum_j dK_j = 0; causal row 0 sees one key,
    so dQ_0 = 0 and the last key only feeds the last query."""
    rng = np.random.default_rng(23)
    n, d = 12, 6
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = impl_bwd(q, k, v, do, 0.6, causal)
        assert np.allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-12)
        assert np.allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-12)
        if causal:
            assert np.allclose(dq[0], 0.0, rtol=0, atol=1e-14)
            # key n-1 is seen only by query n-1, with probability P[n-1, n-1]
            s_last = 0.6 * q[-1] @ k.T
            p_last = np.exp(s_last - s_last.max())
            p_last /= p_last.sum()
            assert np.allclose(dv[-1], p_last[-1] * do[-1], rtol=0, atol=1e-12)
    zero = impl_bwd(q, k, v, np.zeros_like(do), 0.6, True)
    assert all(np.array_equal(g, np.zeros_like(g)) for g in zero)


BACKWARD_PINS = (pin_bwd_identities, pin_bwd_torch_autograd, pin_bwd_finite_differences)


# ------------------------------------------------------------------ dropout
# ``impl`` is a module-like object with the functions of ``oracle/dropout.py``:
# philox4x32_10, keep_threshold, dropout_bytes, attention_dropout_slice.

def pin_dropout_philox_known_answers(impl):
    """The generator against the published known-answer vectors."""
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")
    for vec in json.load(open(path))["vectors"]:
        ctr = np.array([int(x, 16) for x in vec["counter"]], dtype=np.uint64)
        key = np.array([int(x, 16) for x in vec["key"]], dtype=np.uint64)
        out = impl.philox4x32_10(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in vec["output"]], vec


def pin_dropout_rate_zero_is_attention(impl):
    """p = 0 keeps every score with weight 1: the forward oracle's result."""
    from oracle import attention_slice

    rng = np.random.default_rng(31)
    q, k, v = _rand(rng, 70, 8), _rand(rng, 70, 8), _rand(rng, 70, 8)
    for causal in (False, True):
        o, lse = impl.attention_dropout_slice(q, k, v, 0.4, causal, 0.0, 123, 0, 0)
        o_ref, lse_ref = attention_slice(q, k, v, 0.4, causal)
        assert np.allclose(o, o_ref, rtol=0, atol=1e-13)
        assert np.allclose(lse, lse_ref, rtol=0, atol=1e-13)


def pin_dropout_lse_is_undropped(impl):
    """Dropout acts after the softmax: lse is the forward oracle's for any rate."""
    from oracle import attention_slice

    rng = np.random.default_rng(32)
    q, k, v = _rand(rng, 40, 8), _rand(rng, 40, 8), _rand(rng, 40, 8)
    _, lse = impl.attention_dropout_slice(q, k, v, 0.7, True, 0.5, 9, 3, 5)
    assert np.allclose(lse, attention_slice(q, k, v, 0.7, True)[1], rtol=0, atol=1e-13)


def pin_dropout_structure(impl):
    """Q = 0 and V = I: P_ij = 1/n_i over the n_i visible keys, so
    O_ij = [u_ij < t] * (256/t) / n_i exactly, with u the slice's bytes."""
    n = 48
    q = np.zeros((n, n))
    v = np.eye(n)
    for p, causal, seed, offset, bh in ((0.6, False, 5, 0, 0), (0.1, True, 2**40 + 7, 11, 3),
                                        (1 - 1 / 256, False, 77, 1, 2)):
        t = impl.keep_threshold(p)
        o, _ = impl.attention_dropout_slice(q, q, v, 1.0, causal, p, seed, offset, bh)
        keep = impl.dropout_bytes(n, n, bh, seed, offset) < t
        visible = np.arange(n)[None, :] <= np.arange(n)[:, None] if causal else np.ones((n, n), bool)
        n_i = visible.sum(axis=1, keepdims=True)
        expect = np.where(keep & visible, (256.0 / t) / n_i, 0.0)
        assert np.allclose(o, expect, rtol=1e-14, atol=0), (p, causal)


def pin_dropout_thresholds(impl):
    """t = floor(256 (1 - p) + 1/2): fixed values, and invalid rates refused."""
    for p, t in ((0.0, 256), (0.1, 230), (0.5, 128), (0.25, 192), (1 - 1 / 256, 1), (0.998, 1)):
        assert impl.keep_threshold(p) == t, (p, t)
    for bad in (-0.1, 1.0, 0.999, float("nan")):
        try:
            impl.keep_threshold(bad)
        except ValueError:
            continue
        raise AssertionError(f"rate {bad} accepted")


def pin_dropout_byte_statistics(impl):
    """Bytes of a large slice are uniform (chi-square over 256 bins) and the
    kept fraction is t/256 within six standard deviations."""
    u = impl.dropout_bytes(512, 512, 7, 2024, 0).ravel()
    counts = np.bincount(u, minlength=256)
    expect = u.size / 256
    chi2 = ((counts - expect) ** 2 / expect).sum()
    assert chi2 < 400, chi2  # 255 degrees of freedom: mean 255, sd 22.6
    for p in (0.1, 0.5, 0.9):
        t = impl.keep_threshold(p)
        frac = (u < t).mean()
        sd = np.sqrt(t / 256 * (1 - t / 256) / u.size)
        assert abs(frac - t / 256) < 6 * sd, (p, frac)


def pin_dropout_streams_independent(impl):
    """Changing the row, slice, offset or either half of the seed gives another
    stream: two streams agree on a byte with probability 1/256."""
    base = impl.dropout_bytes(64, 256, 3, 0x1234_5678_9ABC, 5)
    others = [
        impl.dropout_bytes(64, 256, 4, 0x1234_5678_9ABC, 5),        # slice
        impl.dropout_bytes(64, 256, 3, 0x1234_5678_9ABC, 6),        # offset
        impl.dropout_bytes(64, 256, 3, 0x1234_5678_9ABD, 5),        # seed, low word
        impl.dropout_bytes(64, 256, 3, 0x1235_5678_9ABC, 5),        # seed, high word
    ]
    for o in others:
        agree = (o == base).mean()
        assert agree < 0.02, agree
    rows = (base[1:] == base[:-1]).mean()  # neighbouring query rows
    assert rows < 0.02, rows
    cols = (base[:, 1:] == base[:, :-1]).mean()  # neighbouring keys
    assert cols < 0.02, cols


def pin_dropout_unbiased(impl):
    """The mean over many seeds approaches the output without dropout (the
    scale 256/t makes each kept weight an unbiased estimate)."""
    from oracle import attention_slice

    rng = np.random.default_rng(33)
    n, d, p = 8, 4, 0.5
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    runs = np.stack([impl.attention_dropout_slice(q, k, v, 0.5, False, p, s, 0, 0)[0] for s in range(600)])
    ref = attention_slice(q, k, v, 0.5, False)[0]
    sem = runs.std(axis=0) / np.sqrt(len(runs))
    assert np.all(np.abs(runs.mean(axis=0) - ref) < 6 * sem + 1e-12)


DROPOUT_PINS = (pin_dropout_philox_known_answers, pin_dropout_thresholds, pin_dropout_rate_zero_is_attention,
                pin_dropout_lse_is_undropped, pin_dropout_structure, pin_dropout_byte_statistics,
                pin_dropout_streams_independent, pin_dropout_unbiased)


# ------------------------------------------------------------------ QKV projection
# ``impl(x, w, bias, H, d) -> (Q, K, V)`` as ``oracle.qkv_projection``.

def pin_proj_brute_force(impl):
    """Scalar loops over every output element of a tiny case."""
    rng = np.random.default_rng(41)
    B, N, D, H, d = 2, 3, 5, 2, 3
    x = rng.standard_normal((B, N, D))
    w = rng.standard_normal((3 * H * d, D))
    bias = rng.standard_normal(3 * H * d)
    outs = impl(x, w, bias, H, d)
    for s in range(3):
        assert outs[s].shape == (B, H, N, d)
        for b in range(B):
            for h in range(H):
                for n in range(N):
                    for c in range(d):
                        f = s * H * d + h * d + c
                        ref = bias[f] + sum(x[b, n, kk] * w[f, kk] for kk in range(D))
                        assert abs(outs[s][b, h, n, c] - ref) < 1e-12, (s, b, h, n, c)


def pin_proj_torch_linear(impl):
    """torch's float64 linear layer, then view/permute into [3, B, H, N, d]."""
    rng = np.random.default_rng(42)
    B, N, D, H, d = 2, 7, 16, 3, 4
    x = rng.standard_normal((B, N, D))
    w = rng.standard_normal((3 * H * d, D))
    bias = rng.standard_normal(3 * H * d)
    y = torch.nn.functional.linear(torch.tensor(x), torch.tensor(w), torch.tensor(bias))
    ref = y.view(B, N, 3, H, d).permute(2, 0, 3, 1, 4).numpy()
    outs = impl(x, w, bias, H, d)
    for s in range(3):
        assert np.allclose(outs[s], ref[s], rtol=0, atol=1e-12), s
    outs = impl(x, w, None, H, d)
    y = torch.nn.functional.linear(torch.tensor(x), torch.tensor(w))
    ref = y.view(B, N, 3, H, d).permute(2, 0, 3, 1, 4).numpy()
    for s in range(3):
        assert np.allclose(outs[s], ref[s], rtol=0, atol=1e-12), s


def pin_proj_one_hot(impl):
    """One token with one input feature and one weight row: a single 1 lands
    at the (tensor, batch, head, token, column) the layout names."""
    B, N, D, H, d = 2, 5, 8, 3, 4
    for b0, n0, k0, s0, h0, c0 in ((1, 3, 6, 2, 1, 3), (0, 0, 0, 0, 0, 0), (1, 4, 2, 1, 2, 1)):
        x = np.zeros((B, N, D))
        x[b0, n0, k0] = 1.0
        w = np.zeros((3 * H * d, D))
        w[s0 * H * d + h0 * d + c0, k0] = 1.0
        outs = impl(x, w, None, H, d)
        for s in range(3):
            want = np.zeros((B, H, N, d))
            if s == s0:
                want[b0, h0, n0, c0] = 1.0
            assert np.array_equal(outs[s], want), (s, b0, n0, k0, s0, h0, c0)


def pin_proj_bias_only(impl):
    """x = 0: every token of every batch carries the bias of its feature."""
    B, N, D, H, d = 2, 3, 4, 2, 5
    bias = np.arange(3 * H * d, dtype=np.float64)
    outs = impl(np.zeros((B, N, D)), np.ones((3 * H * d, D)), bias, H, d)
    for s in range(3):
        for h in range(H):
            for c in range(d):
                assert np.all(outs[s][:, h, :, c] == bias[s * H * d + h * d + c])


PROJECTION_PINS = (pin_proj_brute_force, pin_proj_torch_linear, pin_proj_one_hot, pin_proj_bias_only)
