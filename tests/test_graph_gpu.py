"""The library's calls inside a captured HIP graph, as a serving loop would
replay them: the forward pass, and the backward pass through fa_bwd_noalloc
(the entry point for callers that cannot allocate).  Neither records a memory
set or an allocation, so a captured call is just its kernels.  Each graph is
replayed several times with eager work between the replays (new inputs
copied into the captured buffers, an eager call on them, synchronizations),
and every replay must equal the eager call bit for bit.
"""
import math

import pytest
import torch

from io_aware_attention_fwd_amd import _lib, gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def _bits(t):
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16) if t.element_size() == 2 else t


@pytest.mark.parametrize("dtype,d,causal", [("f16", 64, False), ("bf16", 64, True), ("bf16", 128, False),
                                            ("f16", 128, True), ("fp8", 64, False)])
def test_forward_graph_replays(dtype, d, causal):
    print(f"[graph fwd] {dtype} d={d} causal={causal} B2 H4 N700", flush=True)
    B, H, N = 2, 4, 700
    scale = 1 / math.sqrt(d)
    q, k, v = gu.to_device(gen.make(B, H, N, d, dtype, seed=11))
    o_dtype = torch.bfloat16 if dtype == "fp8" else q.dtype
    o = torch.empty((B, H, N, d), dtype=o_dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a call before capture (code object loaded, tile chosen)
        _lib.fwd(q, k, v, scale, causal, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _lib.fwd(q, k, v, scale, causal, out=o, lse=lse)
    for r in range(REPLAYS):
        nq, nk, nv = gu.to_device(gen.make(B, H, N, d, dtype, seed=20 + r))
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        o_ref, lse_ref = _lib.fwd(q, k, v, scale, causal)  # eager, into fresh tensors
        torch.cuda.synchronize()
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(o), _bits(o_ref)), f"replay {r}: O differs from the eager call"
        assert torch.equal(_bits(lse), _bits(lse_ref)), f"replay {r}: lse differs from the eager call"


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, False), ("f16", 64, True)])
def test_backward_noalloc_graph_replays(dtype, d, causal):
    print(f"[graph bwd] {dtype} d={d} causal={causal} B2 H4 N600", flush=True)
    B, H, N = 2, 4, 600
    scale = 1 / math.sqrt(d)
    dt = {"f16": _lib.FA_DTYPE_F16, "bf16": _lib.FA_DTYPE_BF16}[dtype]
    q, k, v = gu.to_device(gen.make(B, H, N, d, dtype, seed=31))
    do = gu.to_device(gen.make(B, H, N, d, dtype, seed=32))[0]
    o, lse = _lib.fwd(q, k, v, scale, causal)
    grads = [torch.empty_like(q) for _ in range(3)]

    def call(stream):
        return _lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   do.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                                   B, H, N, d, scale, causal, dt, stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the first call on a device looks up the static array's address
        assert call(side.cuda_stream) == 0
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = call(torch.cuda.current_stream().cuda_stream)
    assert rc == 0, _lib.fa_strerror(rc)
    for r in range(REPLAYS):
        ndo = gu.to_device(gen.make(B, H, N, d, dtype, seed=40 + r))[0]
        do.copy_(ndo)
        ref = _lib.bwd(q, k, v, o, lse, do, scale, causal)  # eager fa_bwd, caller-provided workspace
        torch.cuda.synchronize()
        for t in grads:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), grads, ref):
            assert torch.equal(_bits(a), _bits(b)), f"replay {r}: {name} differs from the eager call"
