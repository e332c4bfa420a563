"""GPU fuzz of the tile pass: a few hundred random small problems in one
process, each compared bit for bit with the oracle's key-block summaries and
tile classes, and checked for exact lists, counts, queues, tile slots and
counters (stops at the first mismatch).

FlashMask-3 paper summary, abstract: the four boundary vectors compress the
mask to O(n), which is what lets whole tiles be classified from per-block
minima and maxima."""
import numpy as np
import pytest

from column_sparse_masked_amd import masks as M
from _parity import check_tileinfo, say

pytestmark = pytest.mark.gpu


def _random_problem(rng):
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 5))
    Hm = H if rng.random() < 0.3 else 1
    small = rng.random() < 0.6
    Sq = int(rng.integers(0, 400 if small else 1500))
    Sk = int(rng.integers(0, 400 if small else 1500))
    kind = rng.integers(0, 5)
    if kind == 0:      # arbitrary intervals, also far outside [0, Sq)
        b = rng.integers(-100, Sq + 100, size=(B, Hm, Sk, 4))
    elif kind == 1:    # int32 extremes mixed in
        b = rng.integers(-2 ** 31, 2 ** 31 - 1, size=(B, Hm, Sk, 4), dtype=np.int64)
        b = np.where(rng.random(b.shape) < 0.5, rng.integers(0, max(Sq, 1), size=b.shape), b)
    elif kind == 2:    # causal documents (Sq = Sk)
        Sk = Sq
        cuts = M.composition(rng, Sq, int(rng.integers(1, 6))) if Sq > 6 else [Sq] if Sq else []
        b = np.broadcast_to(M.causal_document_bounds(list(cuts)) if Sq else np.zeros((0, 4)), (B, Hm, Sk, 4))
    elif kind == 3:    # sliding windows
        Sk = Sq
        b = np.broadcast_to(M.sliding_window_bounds(Sq, int(rng.integers(1, 300))) if Sq else np.zeros((0, 4)),
                            (B, Hm, Sk, 4))
    else:              # block-aligned intervals (full and skipped tiles)
        lo = rng.integers(0, 12, size=(B, Hm, Sk, 2)) * 128
        b = np.concatenate([lo, lo + rng.integers(0, 4, size=(B, Hm, Sk, 2)) * 128], axis=-1)[..., [0, 2, 1, 3]]
    b = np.ascontiguousarray(b, dtype=np.int64).astype(np.int32)
    return M.custom(None, B=B, H=H, Sq=Sq, D=64, seed=0, per_head_bounds=b)


def test_tile_pass_fuzz():
    """Also in pair mode (head_dim 128 with fwd_rows 256: union lists of the
    query-block pairs and a queue of pairs), on a third of the problems."""
    import torch
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bounds
    rng = np.random.default_rng(2024)
    rng_mode = np.random.default_rng(77)
    n = 300
    for i in range(n):
        w = _random_problem(rng)
        fwd_rows = 256 if rng_mode.random() < 1 / 3 else 0
        if fwd_rows:
            w.D = 128
        att = MaskedAttention.for_workload(w, fwd_rows=fwd_rows)
        att.buf.tileinfo.fill_(0xA5)          # garbage from a previous user
        att.tile_bounds(to_device_bounds(w.bounds))
        torch.cuda.synchronize()
        try:
            check_tileinfo(w, att.read_tileinfo(), fwd_rows)
        except AssertionError as e:
            raise AssertionError(f"problem {i}: B={w.B} H={w.H} Hm={w.Hm} Sq={w.Sq} Sk={w.Sk} "
                                 f"fwd_rows={fwd_rows}: {e}") from e
        if i % 50 == 0:
            say(f"[fuzz] {i} problems bit-exact (last: B={w.B} H={w.H} Hm={w.Hm} Sq={w.Sq} Sk={w.Sk})")
    say(f"[fuzz] {n} problems bit-exact")


@pytest.mark.parametrize("B,H,Hm,Sq,Sk,fwd_rows", [(2, 24, 24, 13000, 9000, 0),    # 4896 forward entries
                                                   (48, 2, 1, 9000, 13000, 0),     # 4896 backward entries
                                                   (1, 40, 40, 16384, 16384, 0),   # 5120 of each
                                                   (2, 40, 40, 26000, 9000, 256)])  # 8160 pair entries
def test_tile_pass_many_entries(B, H, Hm, Sq, Sk, fwd_rows):
    """More (batch, mask head, block) entries than the sort keeps in LDS: the
    last workgroup reads the counts from global memory instead."""
    import torch
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bounds
    rng = np.random.default_rng(B * 1000 + H)
    b = rng.integers(-50, Sq + 50, size=(B, Hm, Sk, 4))
    w = M.custom(None, B=B, H=H, Sq=Sq, D=128 if fwd_rows else 64, seed=0,
                 per_head_bounds=np.ascontiguousarray(b, dtype=np.int64).astype(np.int32))
    assert w.Sk == Sk
    say(f"[many entries] B={B} H={H} Hm={Hm} Sq={Sq} Sk={Sk} fwd_rows={fwd_rows}")
    att = MaskedAttention.for_workload(w, fwd_rows=fwd_rows)
    att.buf.tileinfo.fill_(0xA5)
    att.tile_bounds(to_device_bounds(w.bounds))
    torch.cuda.synchronize()
    check_tileinfo(w, att.read_tileinfo(), fwd_rows)
