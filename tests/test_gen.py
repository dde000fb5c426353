"""Seeded generator: determinism, storage rounding, fp8 quantiser, byte sizes."""
import json
import os

import numpy as np
import pytest
import torch

from io_aware_attention_fwd_amd import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_deterministic_by_seed_and_order():
    a = gen.make(1, 2, 33, 64, "f16", seed=0)
    b = gen.make(1, 2, 33, 64, "f16", seed=0)
    c = gen.make(1, 2, 33, 64, "f16", seed=1)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert np.array_equal(x, y)
    assert not np.array_equal(a.q, c.q)
    # draw order is Q, then K, then V from one stream
    rng = np.random.default_rng(0)
    q = rng.standard_normal(size=(1, 2, 33, 64), dtype=np.float32)
    k = rng.standard_normal(size=(1, 2, 33, 64), dtype=np.float32)
    assert np.array_equal(a.q, q.astype(np.float16))
    assert np.array_equal(a.k, k.astype(np.float16))


@pytest.mark.parametrize("dtype,np_dtype", [("f16", np.float16), ("bf16", np.uint16), ("fp8", np.uint8)])
def test_shapes_and_storage_types(dtype, np_dtype):
    x = gen.make(2, 3, 17, 128, dtype)
    for t in (x.q, x.k, x.v):
        assert t.shape == (2, 3, 17, 128)
        assert t.dtype == np_dtype
        assert t.flags.c_contiguous


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4096).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 4096),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.0e38], np.float32)])
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_quantiser_scale_saturation_and_error():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(size=(4, 64, 64)).astype(np.float32)
    codes, s = gen.quantize_e4m3(x)
    assert s == pytest.approx(float(np.abs(x).max()) / 448.0, rel=1e-6)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.isfinite(vals).all()
    assert np.abs(vals).max() == 448.0  # the amax element lands on the top code
    # RNE with 3 mantissa bits: relative error <= 2^-4 for normals, abs <= 2^-10 for subnormals
    y = x.astype(np.float64) / s
    err = np.abs(vals - y)
    assert (err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-12).all()
    # the amax element of either sign maps to the extreme finite code, never NaN
    z = np.array([0.5, -3.0, 1.0], np.float32)
    cz, sz = gen.quantize_e4m3(z)
    assert cz[1] == 0xFE and sz == pytest.approx(3.0 / 448.0)


def test_structured_inputs_are_exact():
    for dtype in ("f16", "bf16", "fp8"):
        x = gen.structured(1, 1, 200, 64, dtype, period=64)
        assert x.descale == {"q": 1.0, "k": 1.0, "v": 1.0}
        if dtype == "f16":
            v = x.v.astype(np.float64)
            q = x.q.astype(np.float64)
        elif dtype == "bf16":
            v = (x.v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            q = (x.q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        else:
            v = torch.from_numpy(x.v).view(torch.float8_e4m3fn).double().numpy()
            q = torch.from_numpy(x.q).view(torch.float8_e4m3fn).double().numpy()
        j = np.arange(200)[:, None]
        c = np.arange(64)[None, :]
        assert np.array_equal(v[0, 0], ((j // 64 + c) % 7).astype(np.float64))
        assert not q.any()


def test_kv_bytes_match_page_memory_table():
    """K+V footprint equals the 'KV 缓存' column of the benchmark page's memory tables."""
    with open(os.path.join(GOLDEN, "kv_cache_memory.json")) as f:
        table = json.load(f)
    for row in table["rows"]:
        nbytes = gen.nbytes_kv(table["B"], table["H"], row["N"], table["d"], table["elem_bytes"])
        assert nbytes == row["kv_cache_MB"] * 2 ** 20
        assert nbytes == row["fa2_total_MB"] * 2 ** 20  # attention matrix: 0 MB
