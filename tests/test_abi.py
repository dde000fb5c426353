"""C ABI of libfa.so without a GPU: symbols, version, error codes.

Only argument-rejection paths are exercised; they return before any HIP call,
so these run on a machine with no GPU.  No test here passes arguments that
would launch a kernel.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

from io_aware_attention_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _header():
    return open(HEADER).read()


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|void|char|float)\s*\**\s*(fa_\w+)\s*\(", text, flags=re.M)))


def _codes():
    return {name: int(val) for name, val in re.findall(r"(FA_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", _header())}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.library_path()):
        pytest.fail("libfa.so is not built; run __graft_entry__.build()")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared_functions()
    assert declared == ["fa_bwd", "fa_bwd_noalloc", "fa_fwd", "fa_fwd_dropout", "fa_fwd_fp8", "fa_fwd_tile",
                        "fa_fwd_varlen", "fa_qkv_proj", "fa_strerror", "fa_version"]
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.library_path()], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)$", out, flags=re.M))
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_matches_header(lib):
    ver = int(re.search(r"#define FA_VERSION (\d+)", _header()).group(1))
    assert _lib.fa_version() == ver


def test_strerror_covers_every_code(lib):
    codes = _codes()
    assert codes["FA_OK"] == 0 and len(codes) == 11
    texts = {_lib.fa_strerror(c) for c in codes.values()}
    assert len(texts) == len(codes) and "unknown error code" not in texts
    assert _lib.fa_strerror(12345) == "unknown error code"


# Fake, well-aligned, non-overlapping addresses: every call below is rejected
# before the library touches them.  Should a validation bug ever let one
# through, the library would launch on these addresses, so the rejection tests
# only run where no GPU is visible.
no_gpu = pytest.mark.skipif(__import__("torch").cuda.is_available(),
                            reason="fake device addresses must never reach a real GPU")
BASE = 0x7F0000000000
SPAN = 1 << 36


def _args(**kw):
    a = dict(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, lse=BASE + 4 * SPAN,
             B=2, H=4, N=1000, d=64, scale=0.125, causal=0, dtype=_lib.FA_DTYPE_F16, stream=None)
    a.update(kw)
    return a


def _call(**kw):
    a = _args(**kw)
    return _lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                       a["causal"], a["dtype"], a["stream"])


def _call8(descale=(1.0, 1.0, 1.0), **kw):
    a = _args(**kw)
    return _lib.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                           a["causal"], descale[0], descale[1], descale[2], a["stream"])


@pytest.mark.parametrize("case,kw,code", [
    ("null q", dict(q=None), "FA_ERR_NULL_PTR"),
    ("null lse", dict(lse=None), "FA_ERR_NULL_PTR"),
    ("B=0", dict(B=0), "FA_ERR_SHAPE"),
    ("H<0", dict(H=-3), "FA_ERR_SHAPE"),
    ("N=0", dict(N=0), "FA_ERR_SHAPE"),
    ("slice >= 2 GiB", dict(N=(1 << 31) // (64 * 2)), "FA_ERR_SHAPE"),
    ("too many workgroups", dict(B=1 << 16, H=1 << 14, N=1 << 10), "FA_ERR_SHAPE"),
    ("d=32", dict(d=32), "FA_ERR_HEADDIM"),
    ("d=96", dict(d=96), "FA_ERR_HEADDIM"),
    ("dtype=3", dict(dtype=3), "FA_ERR_DTYPE"),
    ("dtype=-1", dict(dtype=-1), "FA_ERR_DTYPE"),
    ("scale nan", dict(scale=math.nan), "FA_ERR_SCALE"),
    ("scale inf", dict(scale=math.inf), "FA_ERR_SCALE"),
    ("q misaligned", dict(q=BASE + 8), "FA_ERR_ALIGN"),
    ("o misaligned", dict(o=BASE + 3 * SPAN + 2), "FA_ERR_ALIGN"),
    ("lse misaligned", dict(lse=BASE + 4 * SPAN + 2), "FA_ERR_ALIGN"),
    ("o is q", dict(o=BASE), "FA_ERR_ALIAS"),
    ("o overlaps v tail", dict(o=BASE + 2 * SPAN + 16 * 1024), "FA_ERR_ALIAS"),
    ("lse inside k", dict(lse=BASE + SPAN + 4096), "FA_ERR_ALIAS"),
    ("lse inside o", dict(lse=BASE + 3 * SPAN + 64), "FA_ERR_ALIAS"),
])
@no_gpu
def test_fa_fwd_rejects(lib, case, kw, code):
    assert _call(**kw) == _codes()[code], case


@pytest.mark.parametrize("descale,kw,code", [
    ((math.nan, 1.0, 1.0), {}, "FA_ERR_SCALE"),
    ((1.0, math.inf, 1.0), {}, "FA_ERR_SCALE"),
    ((1.0, 1.0, -math.inf), {}, "FA_ERR_SCALE"),
    ((1e30, 1e30, 1.0), {}, "FA_ERR_SCALE"),  # folded multiplier overflows float32
    ((1.0, 1.0, 1.0), dict(d=256), "FA_ERR_HEADDIM"),
    ((1.0, 1.0, 1.0), dict(k=None), "FA_ERR_NULL_PTR"),
    ((1.0, 1.0, 1.0), dict(N=(1 << 31) // 64), "FA_ERR_SHAPE"),
])
@no_gpu
def test_fa_fwd_fp8_rejects(lib, descale, kw, code):
    assert _call8(descale, **kw) == _codes()[code]


def _calld(p_drop=0.1, seed=1, offset=0, **kw):
    a = _args(**kw)
    return _lib.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                               a["causal"], a["dtype"], p_drop, seed, offset, a["stream"])


@pytest.mark.parametrize("p_drop,kw,code", [
    (-0.01, {}, "FA_ERR_DROPOUT"),
    (1.0, {}, "FA_ERR_DROPOUT"),
    (math.nan, {}, "FA_ERR_DROPOUT"),
    (0.999, {}, "FA_ERR_DROPOUT"),  # t = floor(0.256 + 1/2) = 0 keeps nothing
    (0.1, dict(dtype=_lib.FA_DTYPE_FP8_E4M3), "FA_ERR_DTYPE"),
    (0.1, dict(dtype=7), "FA_ERR_DTYPE"),
    (0.1, dict(v=None), "FA_ERR_NULL_PTR"),
    (0.1, dict(d=96), "FA_ERR_HEADDIM"),
    (0.1, dict(N=0), "FA_ERR_SHAPE"),
    (0.1, dict(scale=math.inf), "FA_ERR_SCALE"),
    (0.1, dict(o=BASE + 3 * SPAN + 4), "FA_ERR_ALIGN"),
    (0.1, dict(o=BASE + SPAN), "FA_ERR_ALIAS"),
])
@no_gpu
def test_fa_fwd_dropout_rejects(lib, p_drop, kw, code):
    assert _calld(p_drop, **kw) == _codes()[code]


def _callp(**kw):
    a = dict(x=BASE, w=BASE + SPAN, bias=BASE + 2 * SPAN, q=BASE + 3 * SPAN, k=BASE + 4 * SPAN, v=BASE + 5 * SPAN,
             B=2, N=100, D=256, H=4, d=64, dtype=_lib.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return _lib.fa_qkv_proj(a["x"], a["w"], a["bias"], a["q"], a["k"], a["v"], a["B"], a["N"], a["D"], a["H"], a["d"],
                            a["dtype"], a["stream"])


@pytest.mark.parametrize("case,kw,code", [
    ("null x", dict(x=None), "FA_ERR_NULL_PTR"),
    ("null v", dict(v=None), "FA_ERR_NULL_PTR"),
    ("N=0", dict(N=0), "FA_ERR_SHAPE"),
    ("D=96", dict(D=96), "FA_ERR_SHAPE"),
    ("D=0", dict(D=0), "FA_ERR_SHAPE"),
    ("X of 2 GiB", dict(B=1, N=1 << 14, D=1 << 16), "FA_ERR_SHAPE"),
    ("d=32", dict(d=32), "FA_ERR_HEADDIM"),
    ("fp8", dict(dtype=_lib.FA_DTYPE_FP8_E4M3), "FA_ERR_DTYPE"),
    ("x misaligned", dict(x=BASE + 2), "FA_ERR_ALIGN"),
    ("bias misaligned", dict(bias=BASE + 2 * SPAN + 4), "FA_ERR_ALIGN"),
    ("q is x", dict(q=BASE), "FA_ERR_ALIAS"),
    ("k inside w", dict(k=BASE + SPAN + 1024), "FA_ERR_ALIAS"),
    ("v overlaps q", dict(v=BASE + 3 * SPAN + 4096), "FA_ERR_ALIAS"),
    ("q on the bias", dict(q=BASE + 2 * SPAN), "FA_ERR_ALIAS"),
])
@no_gpu
def test_fa_qkv_proj_rejects(lib, case, kw, code):
    assert _callp(**kw) == _codes()[code], case


def _callv(**kw):
    a = dict(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, lse=BASE + 4 * SPAN, cu=BASE + 5 * SPAN,
             B=3, H=4, total=1000, max_seqlen=600, d=64, scale=0.125, causal=1, dtype=_lib.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return _lib.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["B"], a["H"], a["total"],
                              a["max_seqlen"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("case,kw,code", [
    ("null cu_seqlens", dict(cu=None), "FA_ERR_NULL_PTR"),
    ("null o", dict(o=None), "FA_ERR_NULL_PTR"),
    ("B=0", dict(B=0), "FA_ERR_SHAPE"),
    ("max_seqlen=0", dict(max_seqlen=0), "FA_ERR_SHAPE"),
    ("total<0", dict(total=-1), "FA_ERR_SHAPE"),
    # one packed row is H*d*2 bytes; max_seqlen rows of it must stay below 2 GiB
    ("slice >= 2 GiB", dict(H=64, d=128, max_seqlen=(1 << 31) // (64 * 128 * 2)), "FA_ERR_SHAPE"),
    ("d=80", dict(d=80), "FA_ERR_HEADDIM"),
    ("dtype=7", dict(dtype=7), "FA_ERR_DTYPE"),
    ("scale nan", dict(scale=math.nan), "FA_ERR_SCALE"),
    ("cu misaligned", dict(cu=BASE + 5 * SPAN + 2), "FA_ERR_ALIGN"),
    ("v misaligned", dict(v=BASE + 2 * SPAN + 4), "FA_ERR_ALIGN"),
    ("o is k", dict(o=BASE + SPAN), "FA_ERR_ALIAS"),
    ("lse inside o", dict(lse=BASE + 3 * SPAN + 256), "FA_ERR_ALIAS"),
    ("no rows", dict(total=0), "FA_OK"),  # valid: nothing to enqueue, no HIP call
])
@no_gpu
def test_fa_fwd_varlen_rejects(lib, case, kw, code):
    assert _callv(**kw) == _codes()[code], case


def _callb(**kw):
    a = dict(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, lse=BASE + 4 * SPAN, do=BASE + 5 * SPAN,
             dq=BASE + 6 * SPAN, dk=BASE + 7 * SPAN, dv=BASE + 8 * SPAN, delta=BASE + 9 * SPAN,
             B=2, H=4, N=1000, d=64, scale=0.125, causal=1, dtype=_lib.FA_DTYPE_F16, stream=None)
    a.update(kw)
    return _lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["delta"],
                       a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("case,kw,code", [
    ("null dout", dict(do=None), "FA_ERR_NULL_PTR"),
    ("null delta", dict(delta=None), "FA_ERR_NULL_PTR"),
    ("fp8", dict(dtype=_lib.FA_DTYPE_FP8_E4M3), "FA_ERR_DTYPE"),
    ("dtype=9", dict(dtype=9), "FA_ERR_DTYPE"),
    ("N=0", dict(N=0), "FA_ERR_SHAPE"),
    ("slice >= 2 GiB", dict(N=(1 << 31) // (64 * 2)), "FA_ERR_SHAPE"),
    ("d=256", dict(d=256), "FA_ERR_HEADDIM"),
    ("scale inf", dict(scale=math.inf), "FA_ERR_SCALE"),
    ("dk misaligned", dict(dk=BASE + 7 * SPAN + 8), "FA_ERR_ALIGN"),
    ("delta misaligned", dict(delta=BASE + 9 * SPAN + 1), "FA_ERR_ALIGN"),
    ("dq is q", dict(dq=BASE), "FA_ERR_ALIAS"),
    ("dv inside dout", dict(dv=BASE + 5 * SPAN + 4096), "FA_ERR_ALIAS"),
    ("delta inside dk", dict(delta=BASE + 7 * SPAN + 64), "FA_ERR_ALIAS"),
    ("dk overlaps dq", dict(dk=BASE + 6 * SPAN + 2 * 4 * 1000 * 64 * 2 - 16), "FA_ERR_ALIAS"),
])
@no_gpu
def test_fa_bwd_rejects(lib, case, kw, code):
    assert _callb(**kw) == _codes()[code], case


def test_python_wrapper_rejects_mismatched_shapes():
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        _lib.fwd(q, torch.zeros(1, 2, 9, 64, dtype=torch.float16), q, 0.1)
    with pytest.raises(TypeError):
        _lib.fwd(q.float(), q.float(), q.float(), 0.1)
    with pytest.raises(TypeError):
        _lib.fwd_varlen(q[0], q[0], q[0], torch.zeros(3, dtype=torch.int64), 8, 0.1)
    with pytest.raises(ValueError):
        _lib.fwd_varlen(q, q, q, torch.zeros(3, dtype=torch.int32), 8, 0.1)


# ---- fa_fwd_tile: the kernel shape a call runs (host logic, no HIP call)
def _tile(N, d, causal, dtype, mode=_lib.FA_TILE_DENSE):
    return _lib.fwd_tile(N, d, causal, dtype, mode)


def _compiled_tiles():
    """(FA_TILE string, d64 only, d128 only) of every compiled shape, read from the variant table."""
    src = open(os.path.join(ROOT, "io_aware_attention_fwd_amd", "csrc", "fa_variants.h")).read()
    body = re.search(r"kVariants\[\] = \{(.*?)\};", src, re.S).group(1)
    tiles = ["x".join(t.replace(" ", "").split(",")) for t in re.findall(r"\{([\d,\s]+)\}", body)]
    d64 = {int(i) for i in re.findall(r"v == (\d+)", re.search(r"d64_only\(int v\) \{(.*?)\}", src).group(1))}
    d128 = {int(i) for i in re.findall(r"v == (\d+)", re.search(r"d128_only\(int v\) \{(.*?)\}", src).group(1))}
    return [(t, i in d64, i in d128) for i, t in enumerate(tiles)]


def test_tile_query_rejects(lib):
    t = (ctypes.c_int * 5)()
    codes = _codes()
    assert _lib.fa_fwd_tile(100, 64, 0, 0, 0, None) == codes["FA_ERR_NULL_PTR"]
    assert _lib.fa_fwd_tile(0, 64, 0, 0, 0, t) == codes["FA_ERR_SHAPE"]
    assert _lib.fa_fwd_tile(100, 64, 0, 0, 7, t) == codes["FA_ERR_SHAPE"]
    assert _lib.fa_fwd_tile(100, 96, 0, 0, 0, t) == codes["FA_ERR_HEADDIM"]
    assert _lib.fa_fwd_tile(100, 64, 0, 5, 0, t) == codes["FA_ERR_DTYPE"]
    assert _lib.fa_fwd_tile(100, 64, 0, _lib.FA_DTYPE_FP8_E4M3, _lib.FA_TILE_DROPOUT, t) == codes["FA_ERR_DTYPE"]


def test_tile_query_honours_fa_tile(lib, monkeypatch):
    """FA_TILE selects any shape compiled for the call's head dimension; one
    compiled for the other head dimension, or an unknown string, falls back
    to the default, and the query reports the fallback."""
    for d in (64, 128):
        monkeypatch.delenv("FA_TILE", raising=False)
        default = _tile(300, d, False, _lib.FA_DTYPE_F16)
        for tile, d64, d128 in _compiled_tiles():
            monkeypatch.setenv("FA_TILE", tile)
            ok = not (d64 and d != 64) and not (d128 and d != 128)
            assert _tile(300, d, False, _lib.FA_DTYPE_F16) == (tile if ok else default), (tile, d)
            # dropout kernels exist for the default shapes only: FA_TILE is ignored there
            monkeypatch.delenv("FA_TILE")
            want = _tile(300, d, False, _lib.FA_DTYPE_F16, _lib.FA_TILE_DROPOUT)
            monkeypatch.setenv("FA_TILE", tile)
            assert _tile(300, d, False, _lib.FA_DTYPE_F16, _lib.FA_TILE_DROPOUT) == want
        monkeypatch.setenv("FA_TILE", "1x2x3x4x5")
        assert _tile(300, d, False, _lib.FA_DTYPE_F16) == default


def test_tile_query_defaults_are_compiled_shapes(lib, monkeypatch):
    monkeypatch.delenv("FA_TILE", raising=False)
    compiled = {t: (a, b) for t, a, b in _compiled_tiles()}
    for d in (64, 128):
        for dt in (_lib.FA_DTYPE_F16, _lib.FA_DTYPE_BF16, _lib.FA_DTYPE_FP8_E4M3):
            for causal in (False, True):
                for N in (1, 1000, 4096, 8192, 16384):
                    modes = [_lib.FA_TILE_DENSE, _lib.FA_TILE_VARLEN]
                    if dt != _lib.FA_DTYPE_FP8_E4M3:
                        modes.append(_lib.FA_TILE_DROPOUT)
                    for mode in modes:
                        t = _tile(N, d, causal, dt, mode)
                        d64, d128 = compiled[t]
                        assert not (d64 and d != 64) and not (d128 and d != 128), (t, d)


# ---- with the host stand-ins for the launchers (the sanitizer build of
# tests/host_build), calls that pass validation are counted instead of
# launched, so accepted edge cases can be driven without a GPU too.
def _stub_counter(lib):
    try:
        return ctypes.c_int.in_dll(lib, "fa_stub_launches")
    except ValueError:
        return None


@pytest.mark.parametrize("kw", [dict(), dict(N=1), dict(B=1, H=1, N=3), dict(scale=0.0), dict(scale=-2.5),
                                dict(causal=1), dict(d=128, dtype=_lib.FA_DTYPE_BF16),
                                dict(dtype=_lib.FA_DTYPE_FP8_E4M3), dict(stream=0x1234)])
def test_accepted_calls_reach_the_launcher_once(lib, kw):
    counter = _stub_counter(lib)
    if counter is None:
        pytest.skip("needs the host build whose launchers are stand-ins (FA_LIBRARY)")
    before = counter.value
    assert _call(**kw) == 0
    assert counter.value == before + 1
    assert _call8(**{k: v for k, v in kw.items() if k != "dtype"}) == 0
    assert counter.value == before + 2


# ---- fa_bwd_noalloc: fa_bwd without the workspace argument
def _calln(**kw):
    a = dict(q=BASE, k=BASE + SPAN, v=BASE + 2 * SPAN, o=BASE + 3 * SPAN, lse=BASE + 4 * SPAN, do=BASE + 5 * SPAN,
             dq=BASE + 6 * SPAN, dk=BASE + 7 * SPAN, dv=BASE + 8 * SPAN,
             B=2, H=4, N=1000, d=64, scale=0.125, causal=1, dtype=_lib.FA_DTYPE_F16, stream=None)
    a.update(kw)
    return _lib.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                               a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("case,kw,code", [
    ("null dq", dict(dq=None), "FA_ERR_NULL_PTR"),
    ("fp8", dict(dtype=_lib.FA_DTYPE_FP8_E4M3), "FA_ERR_DTYPE"),
    ("N=0", dict(N=0), "FA_ERR_SHAPE"),
    ("d=80", dict(d=80), "FA_ERR_HEADDIM"),
    ("scale nan", dict(scale=math.nan), "FA_ERR_SCALE"),
    ("scale huge", dict(scale=3e38), "FA_ERR_SCALE"),
    ("one row past the workspace", dict(B=1, H=1, N=(1 << 22) + 1), "FA_ERR_SCRATCH"),
    ("B*H*N past the workspace", dict(B=8, H=64, N=8193), "FA_ERR_SCRATCH"),
    ("dk misaligned", dict(dk=BASE + 7 * SPAN + 8), "FA_ERR_ALIGN"),
    ("dv inside v", dict(dv=BASE + 2 * SPAN + 1024), "FA_ERR_ALIAS"),
    ("dq overlaps dk", dict(dq=BASE + 7 * SPAN - 64), "FA_ERR_ALIAS"),
])
@no_gpu
def test_fa_bwd_noalloc_rejects(lib, case, kw, code):
    assert _calln(**kw) == _codes()[code], case


@pytest.mark.parametrize("kw", [dict(), dict(B=1, H=1, N=1 << 22), dict(B=4, H=32, N=8192, d=128),
                                dict(dtype=_lib.FA_DTYPE_BF16, causal=0)])
def test_noalloc_accepted_up_to_the_workspace(lib, kw):
    counter = _stub_counter(lib)
    if counter is None:
        pytest.skip("needs the host build whose launchers are stand-ins (FA_LIBRARY)")
    before = counter.value
    assert _calln(**kw) == 0
    assert counter.value == before + 1
