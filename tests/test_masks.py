"""Bounds builders against the patterns' own definitions (CPU only).

Three independent pins: hand-drawn masks (tests/golden/masks_small.txt), brute
force from each pattern's definition on tiny lengths, and the closed-form
unmasked count against the dense count.
"""
import os

import numpy as np
import pytest

from column_sparse_masked_amd import masks as M
from oracle import dense_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "masks_small.txt")


def _read_golden():
    blocks, cur = [], None
    for line in open(GOLDEN):
        line = line.rstrip("\n")
        if line.startswith("#"):
            continue
        if line.startswith("@"):
            parts = line[1:].split()
            cur = {"name": parts[0], "args": dict(p.split("=") for p in parts[1:]), "rows": []}
            blocks.append(cur)
        elif line.strip() and cur is not None:
            cur["rows"].append([c == "x" for c in line.strip()])
    return [(b["name"], b["args"], np.array(b["rows"], dtype=bool)) for b in blocks]


def _ints(s):
    return [int(x) for x in s.split(",")]


def _bounds_for(name, args):
    if name == "causal_document":
        b = M.causal_document_bounds(_ints(args["docs"]))
        return b, np.arange(b.shape[0])
    if name == "sliding_window":
        b = M.sliding_window_bounds(int(args["S"]), int(args["window"]))
        return b, np.arange(b.shape[0])
    if name == "share_question":
        b = M.share_question_bounds(int(args["question"]), _ints(args["answers"]))
        return b, np.arange(b.shape[0])
    if name == "prefix_document":
        b = M.prefix_document_bounds(_ints(args["docs"]), float(args["prefix_frac"]))
        return b, np.arange(b.shape[0])
    if name == "block_causal":
        b = M.blockwise_causal_bounds(int(args["S"]), int(args["block"]))
        return b, np.arange(b.shape[0])
    if name == "document":
        b = M.document_bounds(_ints(args["docs"]))
        return b, np.arange(b.shape[0])
    if name == "global_sliding":
        b = M.global_sliding_bounds(int(args["S"]), int(args["global"]), int(args["window"]))
        return b, np.arange(b.shape[0])
    if name == "eviction":
        b = M.eviction_bounds(_ints(args["ends"]))
        return b, np.arange(b.shape[0])
    if name == "cp_local":
        docs = _ints(args["docs"])
        S, world, rank = sum(docs), int(args["world"]), int(args["rank"])
        C = S // (2 * world)
        starts = [rank * C, (2 * world - 1 - rank) * C]
        lb = M.localize_bounds(M.causal_document_bounds(docs), starts, C)
        return lb, np.arange(2 * C)
    raise KeyError(name)


@pytest.mark.parametrize("idx", range(len(_read_golden())))
def test_hand_drawn_masks(idx):
    name, args, expected = _read_golden()[idx]
    bounds, rows = _bounds_for(name, args)
    got = dense_mask(bounds, rows)
    assert got.shape == expected.shape, name
    assert np.array_equal(got, expected), f"{name} {args}\n{got.astype(int)}"


# --------------------------------------------------------------------------- #
# brute force from the definitions                                            #
# --------------------------------------------------------------------------- #
SIZES = [1, 2, 3, 7, 16, 64, 130]


def _doc_ids(lens):
    return np.repeat(np.arange(len(lens)), lens)


def _visible_causal_doc(lens):
    d = _doc_ids(lens)
    i, j = np.meshgrid(np.arange(len(d)), np.arange(len(d)), indexing="ij")
    return (d[i] == d[j]) & (j <= i)


@pytest.mark.parametrize("S", SIZES)
def test_causal_document_definition(S):
    rng = np.random.default_rng(S)
    for _ in range(5):
        k = int(rng.integers(1, min(S, 6) + 1))
        lens = M.composition(rng, S, k)
        assert sum(lens) == S and min(lens) >= 1
        got = ~dense_mask(M.causal_document_bounds(lens), np.arange(S))
        assert np.array_equal(got, _visible_causal_doc(lens))


@pytest.mark.parametrize("S", SIZES)
@pytest.mark.parametrize("w", [1, 2, 5, 1000])
def test_sliding_window_definition(S, w):
    i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    want = (i - j >= 0) & (i - j < w)
    got = ~dense_mask(M.sliding_window_bounds(S, w), np.arange(S))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("S", [s for s in SIZES if s >= 3])
def test_share_question_definition(S):
    rng = np.random.default_rng(100 + S)
    for _ in range(5):
        Q = int(rng.integers(1, S - 1))
        n = int(rng.integers(1, min(S - Q, 5) + 1))
        ans = M.composition(rng, S - Q, n)
        aid = np.concatenate([np.full(Q, -1), np.repeat(np.arange(n), ans)])
        i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
        want = (j <= i) & ((j < Q) | (aid[i] == aid[j]))
        got = ~dense_mask(M.share_question_bounds(Q, ans), np.arange(S))
        assert np.array_equal(got, want)


@pytest.mark.parametrize("S", SIZES)
@pytest.mark.parametrize("frac", [0.1, 0.25, 0.5])
def test_prefix_document_definition(S, frac):
    rng = np.random.default_rng(200 + S)
    for _ in range(5):
        k = int(rng.integers(1, min(S, 5) + 1))
        lens = M.composition(rng, S, k)
        d = _doc_ids(lens)
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
        plen = np.floor(np.asarray(lens) * frac).astype(int)
        i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
        want = (d[i] == d[j]) & ((j <= i) | (j < starts[d[j]] + plen[d[j]]))
        got = ~dense_mask(M.prefix_document_bounds(lens, frac), np.arange(S))
        assert np.array_equal(got, want)


@pytest.mark.parametrize("S", SIZES)
@pytest.mark.parametrize("blk", [1, 4, 32])
def test_block_causal_definition(S, blk):
    i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    want = (j // blk) <= (i // blk)
    got = ~dense_mask(M.blockwise_causal_bounds(S, blk), np.arange(S))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("S", SIZES)
def test_document_definition(S):
    rng = np.random.default_rng(300 + S)
    for _ in range(5):
        lens = M.composition(rng, S, int(rng.integers(1, min(S, 6) + 1)))
        d = _doc_ids(lens)
        i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
        got = ~dense_mask(M.document_bounds(lens), np.arange(S))
        assert np.array_equal(got, d[i] == d[j])


@pytest.mark.parametrize("S", SIZES)
@pytest.mark.parametrize("g,w", [(0, 1), (0, 3), (1, 2), (3, 1), (5, 4), (200, 2), (2, 1000)])
def test_global_sliding_definition(S, g, w):
    i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    want = (np.abs(i - j) < w) | (i < g) | (j < g)
    got = ~dense_mask(M.global_sliding_bounds(S, g, w), np.arange(S))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("S", SIZES)
def test_eviction_definition(S):
    rng = np.random.default_rng(400 + S)
    for _ in range(5):
        e = M.random_eviction_rows(rng, S)
        assert (e >= np.arange(S) + 1).all() and (e <= S).all()
        i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
        want = (j <= i) & (i < e[j])
        got = ~dense_mask(M.eviction_bounds(e), np.arange(S))
        assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        M.eviction_bounds(np.arange(S))   # key j evicted at its own row


@pytest.mark.parametrize("S,world", [(16, 2), (64, 4), (128, 8), (96, 4)])
def test_cp_localisation_is_gather_of_global_rows(S, world):
    """Local bounds reproduce exactly the global mask's rows of the rank's chunks
    (the per-rank localisation needs no data from other ranks)."""
    rng = np.random.default_rng(S)
    lens = M.composition(rng, S, 4)
    gb = M.causal_document_bounds(lens)
    C = S // (2 * world)
    for rank in range(world):
        starts = [rank * C, (2 * world - 1 - rank) * C]
        lb = M.localize_bounds(gb, starts, C)
        rows = np.concatenate([np.arange(s, s + C) for s in starts])
        assert np.array_equal(dense_mask(lb, np.arange(2 * C)), dense_mask(gb, rows))
        # arbitrary (also out-of-range) bound values; local rows stacked in
        # increasing global order, as the localisation requires
        rb = rng.integers(-3, S + 3, size=(S, 4)).astype(np.int32)
        assert np.array_equal(dense_mask(M.localize_bounds(rb, starts, C), np.arange(2 * C)),
                              dense_mask(rb, rows))


@pytest.mark.parametrize("seed", range(6))
def test_nnz_closed_form(seed):
    rng = np.random.default_rng(seed)
    Sq, Sk = int(rng.integers(1, 70)), int(rng.integers(1, 70))
    b = rng.integers(-5, Sq + 5, size=(1, 2, Sk, 4)).astype(np.int32)
    w = M.custom(None, B=1, H=4, Sq=Sq, D=8, seed=seed, per_head_bounds=b)
    for hm in range(2):
        dense = int((~dense_mask(b[0, hm], np.arange(Sq))).sum())
        assert w.nnz_per_head()[0, hm] == dense
    assert w.nnz_total() == 2 * sum(int((~dense_mask(b[0, hm], np.arange(Sq))).sum()) for hm in range(2))


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -7 + 2 ** -9], dtype=np.float32)
    bits = M.bf16_bits(x)
    back = M.bf16_to_f32(bits)
    # 1+2^-8 is a tie between 1 and 1+2^-7: rounds to the even mantissa (1.0);
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6: rounds to 1+2^-6.
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0 + 2 ** -7]
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(t, bits)


def test_config_structures_and_counts():
    """The five evaluation workloads: lengths add up, bounds are in range and
    the structure matches the workload descriptions."""
    w1 = M.config(1)
    assert (w1.B, w1.H, w1.Sq, w1.D) == (1, 2, 1024, 64) and len(w1.structure["docs"]) == 4
    w2 = M.config(2)
    assert (w2.B, w2.H, w2.Sq, w2.D, w2.structure["window"]) == (2, 16, 8192, 128, 1024)
    w3 = M.config(3)
    assert w3.structure["question"] == 4096 and sum(w3.structure["answers"]) == 28672
    w4 = M.config(4)
    assert sum(w4.structure["docs"]) == 131072
    assert min(w4.structure["docs"]) >= 512 and max(w4.structure["docs"]) <= 65536
    w5 = M.config(5)
    assert (w5.Sq, w5.Sk, w5.H) == (8192, 65536, 16)
    assert w5.structure["chunks"] == [3, 12]
    for w in (w1, w2, w3, w4, w5):
        assert w.bounds.shape == (w.B, w.Hm, w.Sk, 4) and w.bounds.dtype == np.int32
        assert w.bounds.min() >= 0 and w.bounds.max() <= w.Sq
