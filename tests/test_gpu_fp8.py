"""GPU parity of the fp8 forward (fm_attn_fwd_fp8, through the C ABI) against
the oracle's exact attention of the decoded E4M3 inputs, within the tolerance
contract derived in _parity.py (per-element bound from E4M3 rounding of P,
tensor rel-L2 <= 2^-4, LSE as tight as the bf16 forward's).

Small problems are compared in full: several tiles, ragged tails, shared and
per-head masks, Sq != Sk, long lists, out-of-range bounds, fully masked rows,
everything masked and the empty key set.  The 8K sliding-window workload is
compared on sampled rows in the benchmark's launch configuration.
"""
import numpy as np
import pytest

from column_sparse_masked_amd import masks as M
from _parity import check_fp8, check_tileinfo, run_gpu_fp8, say

pytestmark = pytest.mark.gpu


def _extreme_bounds(S):
    j = np.arange(S)
    b = np.empty((S, 4), np.int64)
    b[:, 0] = np.where(j % 3 == 0, -2 ** 31, 400)
    b[:, 1] = np.where(j % 3 == 0, 2 ** 31 - 1, 400)
    b[:, 2] = -7
    b[:, 3] = j
    return b.astype(np.int32)


CASES = {
    "sliding_ragged_S1000": lambda: M.custom(M.sliding_window_bounds(1000, 200), B=2, H=2, Sq=1000, D=128,
                                             seed=51, name="sliding"),
    "causal_docs_S1300": lambda: M.custom(M.causal_document_bounds([700, 13, 587]), B=1, H=3, Sq=1300,
                                          D=128, seed=52),
    "unmasked_S700": lambda: M.custom(M.empty_bounds(700, 700), B=1, H=2, Sq=700, D=128, seed=53),
    "per_head_random_Sq333_Sk517": lambda: M.custom(
        None, B=2, H=3, Sq=333, D=128, seed=54,
        per_head_bounds=np.random.default_rng(55).integers(-20, 353, size=(2, 3, 517, 4)).astype(np.int32)),
    "masked_rows_100_140": lambda: M.custom(
        np.stack([np.full(512, 100), np.full(512, 140), np.zeros(512), np.arange(512)], 1).astype(np.int32),
        B=1, H=2, Sq=512, D=128, seed=56),
    "everything_masked_S260": lambda: M.custom(np.tile(np.array([0, 260, 0, 0], np.int32), (260, 1)),
                                               B=1, H=2, Sq=260, D=128, seed=57),
    "tiny_S17": lambda: M.custom(M.causal_document_bounds([5, 12]), B=2, H=2, Sq=17, D=128, seed=58),
    "extreme_int32_bounds": lambda: M.custom(_extreme_bounds(300), B=1, H=2, Sq=300, D=128, seed=59),
    "long_lists_unmasked_S4000": lambda: M.custom(M.empty_bounds(4000, 4000), B=1, H=2, Sq=4000, D=128,
                                                  seed=60),
    "share_question_S1500": lambda: M.custom(
        M.share_question_bounds(300, M.composition(np.random.default_rng(3), 1200, 4)),
        B=1, H=2, Sq=1500, D=128, seed=61),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_small_problem_parity(name):
    w = CASES[name]()
    say(f"[fp8] {name}: B={w.B} H={w.H} Hm={w.Hm} Sq={w.Sq} Sk={w.Sk}")
    q8, k8, v8, ds = M.fp8_inputs(w.draw())
    go, gl, att = run_gpu_fp8(w, (q8, k8, v8), ds)
    check_tileinfo(w, att.read_tileinfo())
    check_fp8(w, go, gl, (q8, k8, v8), ds, label=name)


@pytest.mark.parametrize("name", ["sliding_ragged_S1000", "causal_docs_S1300", "tiny_S17", "share_question_S1500"])
def test_fp8_pair_mode_parity(name):
    """A tileinfo built for pairs of query blocks (fwd_rows 256): the fp8
    forward takes two tickets per queue entry, one per query block, and none
    for the missing second block of an odd last pair."""
    w = CASES[name]()
    say(f"[fp8 pairs] {name}: B={w.B} H={w.H} Hm={w.Hm} Sq={w.Sq} Sk={w.Sk}")
    q8, k8, v8, ds = M.fp8_inputs(w.draw())
    go, gl, att = run_gpu_fp8(w, (q8, k8, v8), ds, fwd_rows=256)
    check_tileinfo(w, att.read_tileinfo(), 256)
    check_fp8(w, go, gl, (q8, k8, v8), ds, label=name + " (pairs)")


def test_fp8_empty_key_set():
    w = M.custom(np.zeros((0, 4), np.int32), B=1, H=2, Sq=200, D=128, seed=62)
    say("[fp8] empty key set")
    q8, k8, v8, ds = M.fp8_inputs(w.draw())
    go, gl, _ = run_gpu_fp8(w, (q8, k8, v8), ds)
    assert (go == 0).all() and np.isposinf(gl).all()


def test_fp8_repeated_and_interleaved_calls():
    """Same tileinfo: fp8 forward, bf16 forward, fp8 forward again: the two
    fp8 results are bit-identical (the queue counters are reset by the
    kernels themselves), and the bf16 forward is unaffected."""
    import torch
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bf16, to_device_bounds, to_device_u8
    w = M.custom(M.sliding_window_bounds(1024, 300), B=1, H=4, Sq=1024, D=128, seed=63)
    say("[fp8] repeated and interleaved calls")
    tensors = w.draw()
    q8, k8, v8, ds = M.fp8_inputs(tensors)
    att = MaskedAttention.for_workload(w)
    tb = to_device_bounds(w.bounds)
    t8 = [to_device_u8(c) for c in (q8, k8, v8)]
    tq, tk, tv = (to_device_bf16(x) for x in tensors[:3])
    att.tile_bounds(tb)
    o1, l1 = att.forward_fp8(*t8, ds, tb)
    ob, lb = att.forward(tq, tk, tv, tb)
    o2, l2 = att.forward_fp8(*t8, ds, tb)
    ob2, lb2 = att.forward(tq, tk, tv, tb)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(ob, ob2) and torch.equal(lb, lb2)
    assert att.read_tileinfo()["counters"][2:6].tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fp8_full_size(cfg):
    """The head-dim-128 evaluation workloads at full size (8K sliding window,
    32K share-question, 128K documents, the context-parallel share), in the
    benchmark's launch configuration; sampled rows (random, block edges and
    the mask's boundary rows) of two heads."""
    w = M.config(cfg)
    say(f"[fp8] full size config {cfg} ({M.CONFIG_NAMES[cfg]}): drawing inputs")
    q8, k8, v8, ds = M.fp8_inputs(w.draw())
    go, gl, att = run_gpu_fp8(w, (q8, k8, v8), ds)
    check_tileinfo(w, att.read_tileinfo())
    rng = np.random.default_rng(200 + cfg)
    lts = np.unique(np.clip(w.bounds[0, 0, :, 0].astype(np.int64), 1, w.Sq - 1))
    edges = lts[np.linspace(0, lts.size - 1, min(8, lts.size)).astype(int)]
    rows = np.unique(np.concatenate([rng.integers(0, w.Sq, 40), [0, 1, 127, 128, w.Sq - 1], edges - 1, edges]))
    rows = rows[(rows >= 0) & (rows < w.Sq)]
    check_fp8(w, go, gl, (q8, k8, v8), ds, heads=[(0, 0), (w.B - 1, w.H - 1)], rows_of=lambda b, h: rows,
              label=f"config {cfg} (sampled rows)")
