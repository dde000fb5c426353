"""The oracle against what the pages and mathematics fix (CPU only)."""
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_attention
from tests import oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_passes_pin(pin):
    pin(oracle.attention_slice)


# Each entry plants one plausible mistake in the oracle's own source.  Every
# mutant must fail at least one pin, or the pins are too weak to trust.
MUTANTS = {
    "dropped scale": ("s = np.float64(scale) * (q[r0:r1] @ k.T)", "s = (q[r0:r1] @ k.T)"),
    "q and k swapped": ("q[r0:r1] @ k.T", "k[r0:r1] @ q.T"),
    "diagonal masked": ("keys > rows", "keys >= rows"),
    "upper triangle kept": ("keys > rows", "keys < rows"),
    "chunk offset lost in mask": ("rows = np.arange(r0, r1)[:, None]", "rows = np.arange(0, r1 - r0)[:, None]"),
    "row dropped per chunk": ("r1 = min(n_q, r0 + row_chunk)", "r1 = min(n_q, r0 + row_chunk - 1)"),
    "max over wrong axis": ("m = s.max(axis=1, initial=-np.inf)", "m = s.max(axis=0, initial=-np.inf)"),
    "no max subtraction in lse": ("lse[r0:r1][seen] = m[seen] + np.log(l)", "lse[r0:r1][seen] = np.log(l)"),
    "log base 2": ("m[seen] + np.log(l)", "m[seen] + np.log2(l)"),
    "sum over wrong axis": ("l = p.sum(axis=1)", "l = p.sum(axis=0)"),
    "unnormalised output": ("(p / l[:, None]) @ v", "p @ v"),
    "keys used as values": ("(p / l[:, None]) @ v", "(p / l[:, None]) @ k"),
    "max dropped from exp": ("p = np.exp(s[seen] - m[seen][:, None])", "p = np.exp(s[seen])"),
    "exp sign flipped": ("p = np.exp(s[seen] - m[seen][:, None])", "p = np.exp(m[seen][:, None] - s[seen])"),
}


def _mutant(old, new, name="attention_slice"):
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation site {old!r} not found: update MUTANTS"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return getattr(mod, name)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    impl = _mutant(*MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except Exception as e:  # an assertion or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"mutant '{name}' passed every pin"


@pytest.mark.parametrize("pin", pins.VARLEN_PINS, ids=lambda f: f.__name__)
def test_varlen_oracle_passes_pin(pin):
    pin(oracle.attention_varlen)


VARLEN_MUTANTS = {
    "sequence end one row late": ("r0, r1 = cu[b], cu[b + 1]", "r0, r1 = cu[b], cu[b + 1] + 1"),
    "sequences all start at row 0": ("r0, r1 = cu[b], cu[b + 1]", "r0, r1 = 0, cu[b + 1]"),
    "queries of head 0 for every head": ("attention_slice(q[r0:r1, h]", "attention_slice(q[r0:r1, 0]"),
    "last sequence skipped": ("range(len(cu) - 1)", "range(len(cu) - 2)"),
    "values of the wrong head": ("v[r0:r1, h], scale", "v[r0:r1, H - 1 - h], scale"),
}


@pytest.mark.parametrize("name", sorted(VARLEN_MUTANTS))
def test_varlen_pins_catch_planted_mistake(name):
    impl = _mutant(*VARLEN_MUTANTS[name], name="attention_varlen")
    caught = False
    for pin in pins.VARLEN_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except Exception:  # an assertion or a crash both count as caught
            caught = True
            break
    assert caught, f"mutant '{name}' passed every varlen pin"


BWD_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "backward.py")


@pytest.mark.parametrize("pin", pins.BACKWARD_PINS, ids=lambda f: f.__name__)
def test_backward_oracle_passes_pin(pin):
    pin(oracle.attention_backward_slice)


BACKWARD_MUTANTS = {
    "dQ scale dropped": ("dq = np.float64(scale) * (ds @ k)", "dq = (ds @ k)"),
    "dK from dS instead of dS^T": ("dk = np.float64(scale) * (ds.T @ q)", "dk = np.float64(scale) * (ds @ q)"),
    "row term dropped": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "row term over columns": ("(p * dp).sum(axis=1, keepdims=True)", "(p * dp).sum(axis=0, keepdims=True)"),
    "dV from P instead of P^T": ("dv = p.T @ do", "dv = p @ do"),
    "dP with V for dO": ("dp = do @ v.T", "dp = v @ do.T"),
    "P not normalised": ("p[seen] /= l[seen][:, None]", "pass"),
    "diagonal masked": ("> np.arange(n_q)[:, None]", ">= np.arange(n_q)[:, None]"),
    "dQ from K^T": ("dq = np.float64(scale) * (ds @ k)", "dq = np.float64(scale) * (ds.T @ k)"),
}


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_pins_catch_planted_mistake(name):
    old, new = BACKWARD_MUTANTS[name]
    src = open(BWD_SRC).read()
    assert src.count(old) >= 1, f"mutation site {old!r} not found"
    mod = types.ModuleType("oracle_bwd_mutant")
    exec(compile(src.replace(old, new), "oracle_bwd_mutant", "exec"), mod.__dict__)
    caught = False
    for pin in pins.BACKWARD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod.attention_backward_slice)
        except Exception:  # an assertion or a crash both count as caught
            caught = True
            break
    assert caught, f"mutant '{name}' passed every backward pin"


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # values fixed by the OCP E4M3 definition
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6 and ours[0x38] == 1.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and not np.isinf(ours).any()


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 16, 5000, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    ours = oracle.decode_bf16_bits(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)
    assert oracle.decode_bf16_bits(np.array([0x3F80, 0xC000], np.uint16)).tolist() == [1.0, -2.0]


def test_dequantize_applies_descale_exactly():
    codes = np.array([0x38, 0x7E, 0xB0, 0x00], np.uint8)  # 1, 448, -0.5, 0
    s = np.float32(0.0123)
    x = oracle.dequantize(codes, "fp8", float(s))
    assert x.tolist() == [float(s), 448 * float(s), -0.5 * float(s), 0.0]


def test_attention_batched_matches_slices_and_sample():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((2, 3, 20, 8)) for _ in range(3))
    o, lse = oracle.attention(q, k, v, 0.3, True)
    for b in range(2):
        for h in range(3):
            o1, l1 = oracle.attention_slice(q[b, h], k[b, h], v[b, h], 0.3, True)
            assert np.array_equal(o[b, h], o1) and np.array_equal(lse[b, h], l1)
    sl = oracle.slice_sample(8, 32)
    assert sl[:2] == [(0, 0), (7, 31)] and len(set(sl)) == 8 == len(sl)
    assert sl == oracle.slice_sample(8, 32)
    assert oracle.slice_sample(1, 2) == [(0, 0), (0, 1)]
    o2, _ = oracle.attention(q, k, v, 0.3, True, slices=[(1, 2)])
    assert np.isnan(o2[0, 0]).all() and np.array_equal(o2[1, 2], o[1, 2])


def test_fully_masked_row_reading():
    # not reachable with equal query/key lengths; a key-less query gives O = 0, lse = -inf
    o, lse = oracle.attention_slice(np.ones((2, 4)), np.ones((0, 4)), np.ones((0, 4)), 1.0, False)
    assert not o.any() and np.isneginf(lse).all()


DROP_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "dropout.py")


@pytest.mark.parametrize("pin", pins.DROPOUT_PINS, ids=lambda f: f.__name__)
def test_dropout_oracle_passes_pin(pin):
    from oracle import dropout

    pin(dropout)


DROPOUT_MUTANTS = {
    "multipliers swapped": ("prod0 = np.uint64(PHILOX_M0) * c0", "prod0 = np.uint64(PHILOX_M1) * c0"),
    "key not bumped": ("k0 = (k0 + np.uint64(PHILOX_W0)) & _LOW32", "k0 = k0"),
    "high and low halves swapped": ("(prod1 >> _SHIFT32) ^ c1 ^ k0, prod1 & _LOW32",
                                    "(prod1 & _LOW32) ^ c1 ^ k0, prod1 >> _SHIFT32"),
    "nine rounds": ("for _ in range(10):", "for _ in range(9):"),
    "threshold truncated": ("math.floor(256.0 * (1.0 - p) + 0.5)", "math.floor(256.0 * (1.0 - p))"),
    "kept on equality": ("keep = dropout_bytes(n_q, n_k, bh, seed, offset) < t",
                         "keep = dropout_bytes(n_q, n_k, bh, seed, offset) <= t"),
    "no rescale": ("o = ((p * keep) @ v) * (256.0 / t)", "o = ((p * keep) @ v)"),
    "rescale by 1/(1-p)": ("o = ((p * keep) @ v) * (256.0 / t)", "o = ((p * keep) @ v) / (1.0 - p_drop)"),
    "dropout before normalising": ("p[seen] /= l[seen][:, None]",
                                   "p *= dropout_bytes(n_q, n_k, bh, seed, offset) < keep_threshold(p_drop); "
                                   "l = p.sum(axis=1); p[seen] /= l[seen][:, None]"),
    "row not in counter": ("ctr[..., 1] = i[:, None]", "ctr[..., 1] = 0"),
    "slice not in counter": ("ctr[..., 2] = bh", "ctr[..., 2] = 0"),
    "offset ignored": ("ctr[..., 3] = offset & 0xFFFFFFFF", "ctr[..., 3] = 0"),
    "seed high word ignored": ("(seed >> 32) & 0xFFFFFFFF", "0"),
    "one call per 32 keys": ("w = words[:, 2 * g + s, q]", "w = words[:, 2 * g, q]"),
}


@pytest.mark.parametrize("name", sorted(DROPOUT_MUTANTS))
def test_dropout_pins_catch_planted_mistake(name):
    old, new = DROPOUT_MUTANTS[name]
    src = open(DROP_SRC).read()
    assert src.count(old) >= 1, f"mutation site {old!r} not found"
    mod = types.ModuleType("oracle_dropout_mutant")
    exec(compile(src.replace(old, new), "oracle_dropout_mutant", "exec"), mod.__dict__)
    caught = False
    for pin in pins.DROPOUT_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:  # an assertion or a crash both count as caught
            caught = True
            break
    assert caught, f"mutant '{name}' passed every dropout pin"


PROJ_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "projection.py")


@pytest.mark.parametrize("pin", pins.PROJECTION_PINS, ids=lambda f: f.__name__)
def test_projection_oracle_passes_pin(pin):
    pin(oracle.qkv_projection)


PROJECTION_MUTANTS = {
    "bias ignored": ("y = y + np.asarray(bias, dtype=np.float64)[None, None, :]", "y = y"),
    "weight not transposed": ("y = x @ w.T", "y = x @ w.reshape(w.shape[1], w.shape[0])"),
    "heads and columns swapped": ("y.reshape(B, N, 3, H, d).transpose(2, 0, 3, 1, 4)",
                                  "y.reshape(B, N, 3, d, H).transpose(2, 0, 4, 1, 3)"),
    "tokens and heads swapped": ("transpose(2, 0, 3, 1, 4)", "transpose(2, 0, 1, 3, 4).reshape(3, B, H, N, d)"),
    "per-head interleaved split": ("y.reshape(B, N, 3, H, d).transpose(2, 0, 3, 1, 4)",
                                   "y.reshape(B, N, H, 3, d).transpose(3, 0, 2, 1, 4)"),
    "Q and K exchanged": ("return y[0], y[1], y[2]", "return y[1], y[0], y[2]"),
}


@pytest.mark.parametrize("name", sorted(PROJECTION_MUTANTS))
def test_projection_pins_catch_planted_mistake(name):
    old, new = PROJECTION_MUTANTS[name]
    src = open(PROJ_SRC).read()
    assert src.count(old) >= 1, f"mutation site {old!r} not found"
    mod = types.ModuleType("oracle_projection_mutant")
    exec(compile(src.replace(old, new), "oracle_projection_mutant", "exec"), mod.__dict__)
    caught = False
    for pin in pins.PROJECTION_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod.qkv_projection)
        except Exception:  # an assertion or a crash both count as caught
            caught = True
            break
    assert caught, f"mutant '{name}' passed every projection pin"
