"""A whole step (tile pass, forward, backward) captured as a HIP graph and
replayed: every replay must reproduce the eager results bit for bit (the
kernels are deterministic), with eager steps and synchronisations between the
replays.  The library records no memset or allocation, so the calls capture
as plain kernel nodes."""
import numpy as np
import pytest

from column_sparse_masked_amd import masks as M

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cache", [True, False], ids=["tile_cache", "recompute"])
def test_graph_replays_match_eager(cache):
    import torch
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bf16, to_device_bounds
    from _parity import say
    w = M.custom(M.sliding_window_bounds(1536, 400), B=1, H=3, Sq=1536, D=128, seed=61)
    say("[graph] capture and replay")
    q, k, v, do = w.draw()
    tq, tk, tv, tdo = (to_device_bf16(x) for x in (q, k, v, do))
    tb = to_device_bounds(w.bounds)
    att = MaskedAttention.for_workload(w)
    outs = [torch.empty_like(tq), torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=tq.device),
            torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)]

    def step(o, lse, dq, dk, dv):
        att.tile_bounds(tb)
        att.forward(tq, tk, tv, tb, o=o, lse=lse)
        att.backward(tq, tk, tv, o, tdo, lse, tb, dq=dq, dk=dk, dv=dv)

    ref = [torch.empty_like(x) for x in outs]
    step(*ref)
    if cache:
        att.reserve_tile_cache()
        step(*ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*outs)
    torch.cuda.synchronize()
    other = [torch.empty_like(x) for x in outs]
    for rep in range(3):
        for x in outs:
            x.view(torch.uint8).fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), outs, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: {name} differs"
        step(*other)   # eager work between the replays
        torch.cuda.synchronize()
        for a, b in zip(other, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_fp8_forward_graph_replays_match_eager():
    """The tile pass and the fp8 forward captured together: every replay
    reproduces the eager O and LSE bit for bit, with eager calls between."""
    import torch
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bounds, to_device_u8
    from _parity import say
    w = M.custom(M.causal_document_bounds([700, 300, 536]), B=1, H=3, Sq=1536, D=128, seed=62)
    say("[graph] fp8 forward capture and replay")
    q8, k8, v8, ds = M.fp8_inputs(w.draw())
    t8 = [to_device_u8(c) for c in (q8, k8, v8)]
    tb = to_device_bounds(w.bounds)
    att = MaskedAttention.for_workload(w)
    shape_o, shape_l = (w.B, w.H, w.Sq, w.D), (w.B, w.H, w.Sq)

    def new_outs():
        return [torch.empty(shape_o, dtype=torch.bfloat16, device=tb.device),
                torch.empty(shape_l, dtype=torch.float32, device=tb.device)]

    def step(o, lse):
        att.tile_bounds(tb)
        att.forward_fp8(*t8, ds, tb, o=o, lse=lse)

    ref, outs, other = new_outs(), new_outs(), new_outs()
    step(*ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*outs)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in outs:
            x.view(torch.uint8).fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse"), outs, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: {name} differs"
        step(*other)
        torch.cuda.synchronize()
        for a, b in zip(other, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
