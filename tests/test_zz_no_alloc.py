"""fm_attn_bwd_noalloc (the backward for callers that cannot allocate: its
Delta row terms live in the library's static scratch array) against
fm_attn_bwd with a caller workspace, through the C ABI.

Two calls in a row on one GPU, the second on a smaller problem, so that the
second runs over the first's leftovers in the scratch array; each must match
fm_attn_bwd bit for bit (the same kernels run), and the second is also
checked against the fp64 oracle within the backward's tolerances."""
import numpy as np
import pytest

from column_sparse_masked_amd import masks as M
from _parity import check_full, say

pytestmark = pytest.mark.gpu


def _both_backwards(w, tensors):
    import torch
    from column_sparse_masked_amd import _lib
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bf16, to_device_bounds
    q, k, v, do = tensors
    tq, tk, tv, tdo = (to_device_bf16(x) for x in (q, k, v, do))
    tb = to_device_bounds(w.bounds)
    att = MaskedAttention.for_workload(w)
    att.tile_bounds(tb)
    o, lse = att.forward(tq, tk, tv, tb)
    ref = att.backward(tq, tk, tv, o, tdo, lse, tb)
    got = [torch.full_like(x, 3.0) for x in ref]
    _lib.fm_attn_bwd_noalloc(att.p, tq, tk, tv, o, tdo, lse, tb, att.buf.tileinfo, *got)
    torch.cuda.synchronize()
    return (o, lse), ref, got


def test_noalloc_backward_matches_workspace_backward():
    cases = [
        M.custom(M.sliding_window_bounds(2048, 700), B=1, H=4, Sq=2048, D=128, seed=51, name="sliding"),
        M.custom(M.causal_document_bounds([300, 111, 289]), B=1, H=2, Sq=700, D=64, seed=52, name="docs"),
    ]
    for i, w in enumerate(cases):
        say(f"[noalloc] call {i}: {w.name} B={w.B} H={w.H} Sq={w.Sq} D={w.D}")
        tensors = w.draw()
        (o, lse), ref, got = _both_backwards(w, tensors)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert np.array_equal(a.view(dtype=__import__("torch").int16).cpu().numpy(),
                                  b.view(dtype=__import__("torch").int16).cpu().numpy()), \
                f"call {i}: {name} of the no-alloc backward differs from fm_attn_bwd"
        if i == 1:
            res = {"o": o.float().cpu().numpy().astype(np.float64),
                   "lse": lse.cpu().numpy().astype(np.float64)}
            res.update({n: t.float().cpu().numpy().astype(np.float64) for n, t in zip(("dq", "dk", "dv"), got)})
            check_full(w, res, tensors, f"noalloc {w.name}")
