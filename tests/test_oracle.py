"""Pins of the fp64 oracle against things other than itself (CPU only).

* torch's float64 scaled-dot-product attention on the CPU (a library routine)
  with autograd, for the unmasked case, the causal case and general masks;
* central finite differences of L = <dO, O> for the gradients;
* the fully-masked-row convention (O = 0, LSE = +inf, zero gradients);
* invariants of exact arithmetic (sum_j dK_j = 0, shift of V, unseen columns);
* brute-force tile classes from the dense mask;
* context-parallel consistency: a rank's share equals the matching rows of
  the global problem, and the ranks' dK/dV add up to the global ones.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle as O
from column_sparse_masked_amd import masks as M


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _torch_sdpa(q, k, v, do, visible, scale):
    """float64 CPU reference through torch SDPA + autograd; ``visible`` is
    bool [Sq][Sk] (True = may attend)."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None],
        attn_mask=torch.tensor(visible)[None, None], scale=scale)[0, 0]
    out.backward(torch.tensor(do))
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _oracle_head(q, k, v, do, bounds, scale):
    o, lse = O.head_forward(q, k, v, bounds, scale)
    dq, dk, dv = O.head_backward(q, k, v, do, bounds, scale, lse=lse)
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("Sq,Sk,D", [(37, 37, 16), (64, 200, 8), (300, 260, 32)])
def test_unmasked_equals_plain_attention(Sq, Sk, D):
    rng = np.random.default_rng(Sq + Sk)
    q, k, v, do = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D), _rand(rng, Sq, D)
    scale = 1 / math.sqrt(D)
    b = M.empty_bounds(Sk, Sq)
    o, lse, dq, dk, dv = _oracle_head(q, k, v, do, b, scale)
    ro, rdq, rdk, rdv = _torch_sdpa(q, k, v, do, np.ones((Sq, Sk), bool), scale)
    for a, r in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, r, rtol=1e-10, atol=1e-11)
    # LSE against its definition through scipy's logsumexp
    from scipy.special import logsumexp
    np.testing.assert_allclose(lse, logsumexp(scale * q @ k.T, axis=1), rtol=1e-12)


def test_causal_equals_sdpa_is_causal():
    rng = np.random.default_rng(7)
    S, D = 290, 16
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    scale = 1 / math.sqrt(D)
    b = M.causal_document_bounds([S])
    o, _, dq, dk, dv = _oracle_head(q, k, v, do, b, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], is_causal=True, scale=scale)[0, 0]
    out.backward(torch.tensor(do))
    for a, r in ((o, out.detach()), (dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(a, r.numpy(), rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("family", ["causal_document", "sliding", "share_question", "prefix", "block",
                                    "document", "global_sliding", "eviction"])
def test_masked_equals_sdpa_with_dense_mask(family):
    rng = np.random.default_rng(11)
    S, D = 333, 16
    if family == "causal_document":
        b = M.causal_document_bounds(M.composition(rng, S, 5))
    elif family == "sliding":
        b = M.sliding_window_bounds(S, 40)
    elif family == "share_question":
        b = M.share_question_bounds(60, M.composition(rng, S - 60, 4))
    elif family == "prefix":
        b = M.prefix_document_bounds(M.composition(rng, S, 3), 0.3)
    elif family == "block":
        b = M.blockwise_causal_bounds(S, 64)
    elif family == "document":
        b = M.document_bounds(M.composition(rng, S, 4))
    elif family == "global_sliding":
        b = M.global_sliding_bounds(S, 17, 30)
    else:
        b = M.eviction_bounds(M.random_eviction_rows(rng, S))
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    scale = 1 / math.sqrt(D)
    o, _, dq, dk, dv = _oracle_head(q, k, v, do, b, scale)
    # visibility written from the pattern definition here, not from the oracle
    i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    vis = ~(((b[None, :, 0] <= i) & (i < b[None, :, 1])) | ((b[None, :, 2] <= i) & (i < b[None, :, 3])))
    assert vis.any(axis=1).all()
    ro, rdq, rdk, rdv = _torch_sdpa(q, k, v, do, vis, scale)
    for a, r in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, r, rtol=1e-9, atol=1e-11)


def _loss(q, k, v, do, b, scale):
    o, _ = O.head_forward(q, k, v, b, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gradients_match_finite_differences(seed):
    """Central differences of L = <dO, O>, h = 1e-6, fp64.  Masks are piecewise
    constant in the inputs, so the difference quotient is valid everywhere."""
    rng = np.random.default_rng(seed)
    Sq, Sk, D = 23, 29, 6
    b = rng.integers(-2, Sq + 2, size=(Sk, 4)).astype(np.int32)
    b[3] = (5, 6, 0, 0)   # a column masked only on one row
    q, k, v = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D)
    do = _rand(rng, Sq, D)
    scale = 1 / math.sqrt(D)
    _, _, dq, dk, dv = _oracle_head(q, k, v, do, b, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            orig = x[idx]
            x[idx] = orig + h
            lp = _loss(q, k, v, do, b, scale)
            x[idx] = orig - h
            lm = _loss(q, k, v, do, b, scale)
            x[idx] = orig
            num[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(g), 1e-300)
        assert err <= 1e-6, (name, err)


def test_fully_masked_everything():
    rng = np.random.default_rng(3)
    Sq, Sk, D = 40, 50, 8
    b = np.zeros((Sk, 4), np.int32)
    b[:, 0], b[:, 1] = 0, Sq          # lower interval covers every row
    q, k, v, do = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D), _rand(rng, Sq, D)
    o, lse, dq, dk, dv = _oracle_head(q, k, v, do, b, 0.3)
    assert (o == 0).all() and np.isposinf(lse).all()
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()


def test_single_fully_masked_row():
    """Row 5 masked in every column: O_5 = 0, LSE_5 = +inf; the other rows and
    all gradients equal the unmasked problem with dO_5 set to zero."""
    rng = np.random.default_rng(4)
    Sq, Sk, D = 30, 33, 8
    b = np.tile(np.array([5, 6, 0, 0], np.int32), (Sk, 1))
    q, k, v, do = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D), _rand(rng, Sq, D)
    o, lse, dq, dk, dv = _oracle_head(q, k, v, do, b, 0.4)
    assert (o[5] == 0).all() and np.isposinf(lse[5]) and (dq[5] == 0).all()
    do0 = do.copy()
    do0[5] = 0
    ro, rdq, rdk, rdv = _torch_sdpa(q, k, v, do0, np.ones((Sq, Sk), bool), 0.4)
    keep = np.arange(Sq) != 5
    np.testing.assert_allclose(o[keep], ro[keep], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dq[keep], rdq[keep], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, rdk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, rdv, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_invariants(seed):
    rng = np.random.default_rng(seed)
    S, D = 270, 16
    b = M.prefix_document_bounds(M.composition(rng, S, 3), 0.2)
    b[40:44] = (0, S, 0, 0)                   # four columns nobody sees
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    o, lse, dq, dk, dv = _oracle_head(q, k, v, do, b, 0.25)
    # sum_j dS_ij = 0 for every row, hence sum_j dK_j = 0
    np.testing.assert_allclose(dk.sum(axis=0), 0, atol=1e-10)
    # unseen columns get no gradient
    assert (dk[40:44] == 0).all() and (dv[40:44] == 0).all()
    # softmax rows sum to one: shifting V by a constant vector shifts O by it
    c = rng.standard_normal(D)
    o2, _ = O.head_forward(q, k, v + c, b, 0.25)
    np.testing.assert_allclose(o2, o + c, atol=1e-12)
    # total dV equals the column sums of dO for rows that see anything
    live = np.isfinite(lse)
    np.testing.assert_allclose(dv.sum(axis=0), do[live].sum(axis=0), atol=1e-10)


def test_row_subset_gradients_complete_for_their_columns():
    """head_backward on the rows that see a column set gives those columns'
    complete dK/dV; row-subset forward equals the full forward's rows."""
    rng = np.random.default_rng(9)
    S, D = 400, 8
    b = M.causal_document_bounds(M.composition(rng, S, 6))
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    full = _oracle_head(q, k, v, do, b, 0.3)
    cols = np.arange(100, 140)
    rows = O.rows_seeing(b, S, cols)
    dq, dk, dv = O.head_backward(q, k, v, do, b, 0.3, rows=rows)
    np.testing.assert_allclose(dk[cols], full[3][cols], atol=1e-12)
    np.testing.assert_allclose(dv[cols], full[4][cols], atol=1e-12)
    np.testing.assert_allclose(dq, full[2][rows], atol=1e-12)
    o, lse = O.head_forward(q, k, v, b, 0.3, rows=rows[::7])
    np.testing.assert_allclose(o, full[0][rows[::7]], atol=1e-14)


@pytest.mark.parametrize("family", ["documents", "share_question", "fully_masked_band"])
def test_column_gradients_match_sdpa(family):
    """column_gradients (dK, dV of a few key columns from the rows that see
    them, with Delta from dO.O) against torch's float64 SDPA autograd on the
    dense mask, and against head_backward's columns."""
    rng = np.random.default_rng(21)
    S, D, scale = 300, 16, 0.27
    if family == "documents":
        b = M.causal_document_bounds(M.composition(rng, S, 5))
    elif family == "share_question":
        b = M.share_question_bounds(60, M.composition(rng, S - 60, 4))
    else:   # rows 40..70 see nothing
        b = np.stack([np.full(S, 40), np.full(S, 70), np.zeros(S), np.arange(S)], 1)
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    vis = ~O.dense_mask(b, np.arange(S))
    live = vis.any(axis=1)
    # torch's SDPA gives NaN rows where nothing is visible: zero those rows' dO
    do_t = do * live[:, None]
    _, _, rdk, rdv = _torch_sdpa(q, k, v, do_t, vis | ~live[:, None], scale)
    cols = np.array([0, 3, 59, 60, 61, 150, 299])
    rows = O.rows_seeing(b, S, cols)
    o, lse = O.head_forward(q, k, v, b, scale, rows)
    dk, dv = O.column_gradients(q, k, v, do, b, scale, cols, rows, o, lse)
    np.testing.assert_allclose(dk, rdk[cols], atol=1e-11)
    np.testing.assert_allclose(dv, rdv[cols], atol=1e-11)
    full = _oracle_head(q, k, v, do, b, scale)
    np.testing.assert_allclose(dk, full[3][cols], atol=1e-12)
    np.testing.assert_allclose(dv, full[4][cols], atol=1e-12)


def _random_chunks(rng, S, n):
    """n disjoint chunks of [0, S) in increasing order (lengths may be 0)."""
    cuts = np.sort(rng.integers(0, S + 1, size=2 * n))
    return cuts[0::2].tolist(), (cuts[1::2] - cuts[0::2]).tolist()


@pytest.mark.parametrize("seed", range(6))
def test_localize_bounds_is_gather_of_global_rows(seed):
    """Brute force: with the localised bounds, the dense mask of the rank's
    local rows equals the global dense mask gathered at the rank's global
    rows, for random bounds (including values far outside [0, S)) and random
    chunk sets."""
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 300))
    gb = rng.integers(-40, S + 40, size=(S + 7, 4))
    gb[::13] = [-2 ** 31, 2 ** 31 - 1, 0, 0]
    for n in (1, 2, 3, 5):
        starts, lens = _random_chunks(rng, S, n)
        rows = np.concatenate([np.arange(s, s + l) for s, l in zip(starts, lens)] + [np.zeros(0, int)])
        lb = O.localize_bounds(gb, starts, lens)
        assert lb.shape == gb.shape
        assert np.array_equal(O.dense_mask(lb, np.arange(rows.size)), O.dense_mask(gb, rows))
        assert lb.min() >= 0 and lb.max() <= rows.size


def test_localize_bounds_by_hand():
    """Rows 0..15 in 4 chunks of 4; the rank holds chunks 1 and 2 (global
    rows 4..11, local rows 0..7).  Bound 0 -> 0, 5 -> 1 (row 4 is below 5),
    8 -> 4, 10 -> 6, 12 and 100 -> 8, -3 -> 0."""
    lb = O.localize_bounds(np.array([[0, 5, 8, 10], [12, 100, -3, 4]]), [4, 8], [4, 4])
    assert lb.tolist() == [[0, 1, 4, 6], [8, 8, 0, 0]]


def test_localize_bounds_matches_clip_shift_max():
    """The paper summary's clip-shift-max on the boundary vectors (the
    maximum over chunks starting at or before g of the chunk's local offset
    plus g clipped into the chunk) equals the oracle's count, written out
    here as a closed form over all int32-range values."""
    rng = np.random.default_rng(3)
    starts, lens = [100, 350, 900], [200, 0, 64]
    g = np.concatenate([rng.integers(-2 ** 31, 2 ** 31 - 1, size=500), np.arange(-5, 1200)])
    offs = np.cumsum([0] + lens[:-1])
    csm = np.zeros(g.shape, np.int64)
    for s, l, o in zip(starts, lens, offs):
        csm = np.where(g >= s, np.maximum(csm, o + np.clip(g - s, 0, l)), csm)
    assert np.array_equal(O.localize_bounds(g, starts, lens), csm)


# --------------------------------------------------------------------------- #
# tile classification                                                         #
# --------------------------------------------------------------------------- #
def test_classification_hand_example():
    """One key block of 4 columns against a query block of 4 rows (BQ=BK=4):
    column 0 has its upper interval covering rows [0, 2) and its lower
    interval rows [2, 4): every element is masked, yet neither single interval
    covers the tile, so the min/max rule says partial (it is conservative)."""
    b = np.array([[2, 4, 0, 2], [0, 4, 0, 0], [0, 4, 0, 0], [0, 4, 0, 0]], np.int32)
    assert O.exact_tile_classes(b, 4, 4, 4)[0, 0] == O.SKIP
    _, cls, cq, ck = O.classify(b[None, None], 4, 4, 4)
    assert cls[0, 0, 0, 0] == O.PARTIAL and cq[0, 0, 0] == 1 and ck[0, 0, 0] == 1
    # all four columns fully covered by the lower interval: skip
    b2 = np.tile(np.array([0, 4, 0, 0], np.int32), (4, 1))
    assert O.classify(b2[None, None], 4, 4, 4)[1][0, 0, 0, 0] == O.SKIP
    # rows 0..3 of 8, all columns' intervals in rows >= 4: full for block 0,
    # skip for block 1
    b3 = np.tile(np.array([4, 8, 4, 6], np.int32), (4, 1))
    c3 = O.classify(b3[None, None], 8, 4, 4)[1][0, 0, :, 0]
    assert c3.tolist() == [O.FULL, O.SKIP]


def test_key_block_summary_by_hand():
    b = np.array([[5, 9, -3, 2], [7, 100, 0, 0], [1, 1, 4, 8]], np.int32)
    ks = O.key_block_summary(b, 10, 2)
    # block 0 = columns 0,1 clamped to [0,10]: LTS {5,7}, LTE {9,10}, UTS {0,0}, UTE {2,0}
    assert ks[0].tolist() == [5, 7, 9, 10, 0, 0, 0, 2]
    assert ks[1].tolist() == [1, 1, 1, 1, 4, 4, 8, 8]


@settings(max_examples=150, deadline=None)
@given(Sq=st.integers(1, 40), Sk=st.integers(1, 40), BQ=st.sampled_from([1, 2, 4, 8, 16]),
       BK=st.sampled_from([1, 3, 4, 8, 16]), seed=st.integers(0, 2 ** 31))
def test_classification_is_sound(Sq, Sk, BQ, BK, seed):
    """skip => every element masked; full => no element masked (brute force)."""
    rng = np.random.default_rng(seed)
    mode = seed % 3
    if mode == 0:
        b = rng.integers(-3, Sq + 3, size=(Sk, 4))
    elif mode == 1:      # structured: mostly document-like columns
        b = np.stack([rng.integers(0, Sq + 1, Sk), np.full(Sk, Sq),
                      np.zeros(Sk), rng.integers(0, Sq + 1, Sk)], axis=1)
    else:                # many empty intervals
        s = rng.integers(0, Sq + 1, size=(Sk, 2))
        b = np.stack([s[:, 0], s[:, 0], np.zeros(Sk), s[:, 1]], axis=1)
    b = b.astype(np.int32)
    _, cls, cq, ck = O.classify(b[None, None], Sq, BQ, BK)
    ex = O.exact_tile_classes(b, Sq, BQ, BK)
    c = cls[0, 0]
    assert np.all(ex[c == O.SKIP] == O.SKIP)
    assert np.all(ex[c == O.FULL] == O.FULL)
    assert np.all((c == O.SKIP) | (c == O.FULL) | (c == O.PARTIAL))
    assert np.array_equal(cq[0, 0], (c != O.SKIP).sum(axis=1))
    assert np.array_equal(ck[0, 0], (c != O.SKIP).sum(axis=0))


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_rule_is_tight_on_workload_masks(k):
    """On the evaluation masks the min/max rule equals the brute-force classes
    (the bit-exact class map is then the same under either reading)."""
    w = M.config(k)
    Sq = w.Sq
    if Sq > 8192:          # share-question at 32K: test the first 8K rows and keys
        b = w.bounds[0, 0][:8192].copy()
        b = np.clip(b, 0, 8192)
        Sq = 8192
    else:
        b = w.bounds[0, 0]
    for BQ, BK in ((128, 128), (64, 128)):
        cls = O.classify(b[None, None], Sq, BQ, BK)[1][0, 0]
        assert np.array_equal(cls, O.exact_tile_classes(b, Sq, BQ, BK))


# --------------------------------------------------------------------------- #
# context-parallel consistency                                                #
# --------------------------------------------------------------------------- #
def test_cp_shares_reassemble_global_problem():
    rng = np.random.default_rng(5)
    S, D, world = 256, 8, 4
    docs = M.composition(rng, S, 5)
    gb = M.causal_document_bounds(docs)
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    go, glse, gdq, gdk, gdv = _oracle_head(q, k, v, do, gb, 0.3)
    C = S // (2 * world)
    sdk, sdv = np.zeros_like(k), np.zeros_like(v)
    for r in range(world):
        starts = [r * C, (2 * world - 1 - r) * C]
        rows = np.concatenate([np.arange(s, s + C) for s in starts])
        lb = M.localize_bounds(gb, starts, C)
        lo, llse, ldq, ldk, ldv = _oracle_head(q[rows], k, v, do[rows], lb, 0.3)
        np.testing.assert_allclose(lo, go[rows], atol=1e-14)
        np.testing.assert_allclose(llse, glse[rows], atol=1e-13)
        np.testing.assert_allclose(ldq, gdq[rows], atol=1e-13)
        sdk += ldk
        sdv += ldv
    np.testing.assert_allclose(sdk, gdk, atol=1e-12)
    np.testing.assert_allclose(sdv, gdv, atol=1e-12)


def test_batched_entry_points_match_heads():
    """forward/backward over [B][H] with per-head masks equal per-head calls."""
    rng = np.random.default_rng(12)
    B, H, Sq, Sk, D = 2, 3, 40, 50, 8
    bounds = rng.integers(0, Sq + 1, size=(B, H, Sk, 4)).astype(np.int32)
    q, do = _rand(rng, B, H, Sq, D), _rand(rng, B, H, Sq, D)
    k, v = _rand(rng, B, H, Sk, D), _rand(rng, B, H, Sk, D)
    o, lse, dq, dk, dv = O.attention(q, k, v, do, bounds, 0.35)
    for b in range(B):
        for h in range(H):
            ref = _oracle_head(q[b, h], k[b, h], v[b, h], do[b, h], bounds[b, h], 0.35)
            for a, r in zip((o, lse, dq, dk, dv), ref):
                np.testing.assert_array_equal(a[b, h], r)
    # one shared mask head
    o1, *_ = O.attention(q, k, v, do, bounds[:, :1], 0.35)
    for h in range(H):
        r = O.head_forward(q[1, h], k[1, h], v[1, h], bounds[1, 0], 0.35)[0]
        np.testing.assert_array_equal(o1[1, h], r)


# --------------------------------------------------------------------------- #
# inputs                                                                       #
# --------------------------------------------------------------------------- #
def test_upcast_bf16_matches_torch_on_every_pattern():
    """Every oracle operand goes through upcast_bf16: checked against torch's
    own bfloat16 -> float64 conversion on all 65536 bit patterns (signed
    zeros, subnormals, infinities and NaN positions included)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.upcast_bf16(bits)
    assert got.dtype == np.float64 and got.shape == bits.shape
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2 * 127
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # a few values by hand: 1.0, -2.0, the smallest subnormal, +inf
    hand = O.upcast_bf16(np.array([0x3F80, 0xC000, 0x0001, 0x7F80], np.uint16))
    assert hand.tolist() == [1.0, -2.0, 2.0 ** -133, np.inf]
    # shape and order are kept (a transposed or reshaped view maps element-wise)
    grid = bits[:12].reshape(3, 4).T
    assert np.array_equal(O.upcast_bf16(grid), ref[:12].reshape(3, 4).T)


# --------------------------------------------------------------------------- #
# fp8 forward                                                                  #
# --------------------------------------------------------------------------- #
def test_e4m3_decode_table():
    """Code points of the OCP OFP8 E4M3 encoding (the specification's table of
    special values: zero, smallest subnormal and normal, one, the largest
    finite value, NaN)."""
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
            0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    got = O.decode_e4m3(np.array(list(want), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(want.values())))
    assert np.signbit(O.decode_e4m3(np.array([0x80], np.uint8)))[0]
    assert np.isnan(O.decode_e4m3(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # positive finite codes are strictly increasing
    assert np.all(np.diff(got[:0x7F]) > 0)


def test_e4m3_inputs_round_trip():
    """Encoding in the input module: every value within half an E4M3 step of
    x / descale (relative 2^-4 for normals, 2^-10 absolute for subnormals)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(4096).astype(np.float32) * 3
    codes, ds = M.e4m3_codes(x)
    assert ds == np.float32(np.abs(x).max() / 448)
    y = x / np.float64(ds)
    err = np.abs(O.decode_e4m3(codes) - y)
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


@pytest.mark.parametrize("family", ["causal", "sliding"])
def test_fp8_forward_equals_sdpa_on_decoded_inputs(family):
    """The fp8 forward is masked attention of decode(codes) * descale: checked
    against torch's float64 SDPA with the dense mask."""
    rng = np.random.default_rng(11)
    Sq = Sk = 200
    D = 32
    q, k, v = (rng.standard_normal((1, 1, Sq, D)).astype(np.float32) for _ in range(3))
    (q8, dq), (k8, dk), (v8, dv) = (M.e4m3_codes(x) for x in (q, k, v))
    bounds = (M.causal_document_bounds([120, 80]) if family == "causal"
              else M.sliding_window_bounds(Sq, 37))[None, None].astype(np.int32)
    scale = 0.3
    o, lse = O.forward_fp8(q8, k8, v8, (dq, dk, dv), bounds, scale)
    vis = ~O.dense_mask(bounds[0, 0], np.arange(Sq))
    qd, kd, vd = (O.decode_e4m3(c)[0, 0] * float(d) for c, d in ((q8, dq), (k8, dk), (v8, dv)))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(qd)[None], torch.tensor(kd)[None], torch.tensor(vd)[None],
        attn_mask=torch.tensor(vis)[None], scale=scale)[0].numpy()
    live = vis.any(axis=1)
    assert np.allclose(o[0, 0][live], ref[live], atol=1e-12, rtol=1e-10)
    s = (qd @ kd.T) * scale
    s[~vis] = -np.inf
    m = s.max(axis=1)
    lse_ref = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    assert np.allclose(lse[0, 0][live], lse_ref[live], atol=1e-12)
