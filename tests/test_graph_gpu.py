"""The entry points can be captured into a HIP graph: the library makes no
synchronising call, no memset and no host round trip, and its workspaces are
stream-ordered allocations, which capture records as graph nodes.  Each
captured graph is replayed several times with eager work and synchronisation
between the replays, and every replay must give the eager call's bits.
"""
import pytest

from parity_util import to_device
from tiled_attention_13_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _dev(shape, seed):
    q, k, v = make_inputs(Workload("graph", *shape, "bf16", True, seed))
    return tuple(to_device(a, "bf16") for a in (q, k, v))


def _capture_and_replay(call, outs, expected):
    """Warm up on a side stream, capture ``call`` (which writes into ``outs``),
    then replay it four times, clearing ``outs`` eagerly before each replay."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(outs, expected)):
            assert torch.equal(x, y), f"replay {rep}: output {i} differs from the eager call"


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp8pv"])
def test_fwd_graph_replays_match_eager(gpu_lib, dtype):
    import torch
    from tiled_attention_13_amd import fwd
    q, k, v = _dev((1, 4, 2048, 128), 201)
    o_ref, l_ref = fwd(q, k, v, causal=True, dtype=dtype)
    o_ref, l_ref = o_ref.clone(), l_ref.clone()
    out, lse = torch.empty_like(q), torch.empty_like(l_ref)
    _capture_and_replay(lambda: fwd(q, k, v, causal=True, dtype=dtype, out=out, lse=lse), (out, lse), (o_ref, l_ref))


def test_bwd_graph_replays_match_eager(gpu_lib):
    import torch
    from tiled_attention_13_amd import bwd, fwd
    q, k, v = _dev((1, 4, 1024, 64), 202)
    o, lse = fwd(q, k, v, causal=True)
    g = torch.Generator(device="cpu").manual_seed(203)
    do = torch.randn(q.shape, generator=g).to("cuda").to(torch.bfloat16)
    ref = [t.clone() for t in bwd(q, k, v, o, do, lse, causal=True)]
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    _capture_and_replay(lambda: bwd(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv), (dq, dk, dv), ref)
