"""GPU parity at the five evaluation workloads' full sizes (causal documents
S=1K D=64; sliding window S=8K; share-question S=32K; documents with prefix-LM
S=128K; one context-parallel rank's share Sq=8K Sk=64K), run in the launch
configuration the benchmark times.

The oracle cannot run these sizes whole, so:
  * tile classification, key-block summaries, counts and lists are compared
    bit for bit over the whole problem (the oracle's classification is cheap);
  * O, LSE and dQ are compared on sampled query rows (random rows plus rows at
    the mask's boundaries), which the oracle computes row set by row set;
  * dK and dV are compared on sampled key columns, using every query row that
    sees them (so those columns' gradients are complete);
  * properties that hold at any size are checked over whole tensors:
    sum_j dK_j = 0 per (batch, head) (rows of dS sum to zero), |O| <= max |V|,
    and LSE = +inf exactly on the rows no key is visible to.
Tolerances are those of the small-problem tests, applied to the samples.
"""
import numpy as np
import pytest

import oracle
from column_sparse_masked_amd import masks as M
from _parity import GRAD_TOL, LSE_TOL, O_TOL, check_tileinfo, rel_l2, say

pytestmark = pytest.mark.gpu


def _fully_masked_rows(bounds_h, Sq):
    """bool[Sq]: rows that no key column leaves visible.  Per row, the number
    of columns masking it is the number of columns whose first interval holds
    it, plus those whose second interval does, minus those whose intervals
    overlap there: three difference arrays, one prefix sum."""
    b = np.clip(bounds_h.astype(np.int64), 0, Sq)
    diff = np.zeros(Sq + 1, dtype=np.int64)
    ivals = [(b[:, 0], b[:, 1], 1), (b[:, 2], b[:, 3], 1),
             (np.maximum(b[:, 0], b[:, 2]), np.minimum(b[:, 1], b[:, 3]), -1)]
    for lo, hi, sign in ivals:
        ok = hi > lo
        np.add.at(diff, lo[ok], sign)
        np.add.at(diff, hi[ok], -sign)
    return np.cumsum(diff)[:Sq] == bounds_h.shape[0]


def _sample_rows(w, rng, n_random=24, n_boundaries=8):
    rows = set(rng.integers(0, w.Sq, size=n_random).tolist())
    rows.update([0, w.Sq - 1])
    lts = np.unique(np.clip(w.bounds[0, 0, :, 0].astype(np.int64), 0, w.Sq))
    lts = lts[(lts > 0) & (lts < w.Sq)]
    if lts.size:
        pick = lts[np.linspace(0, lts.size - 1, min(n_boundaries, lts.size)).astype(int)]
        for r in pick:
            rows.update([int(r) - 1, int(r)])
    return np.array(sorted(r for r in rows if 0 <= r < w.Sq))


def _sample_cols(w, bounds_h, rng, max_rows=2048, n_cols=12):
    """Key columns whose complete set of seeing rows stays small enough for
    the oracle: the last columns of the mask's structural segments, where
    few rows look back, plus random columns that pass the same bound."""
    Sq, Sk = w.Sq, w.Sk
    b = bounds_h.astype(np.int64)
    lo1, hi1 = np.clip(b[:, 0], 0, Sq), np.clip(b[:, 1], 0, Sq)
    lo2, hi2 = np.clip(b[:, 2], 0, Sq), np.clip(b[:, 3], 0, Sq)
    l1 = np.maximum(hi1 - lo1, 0)
    l2 = np.maximum(hi2 - lo2, 0)
    ov = np.maximum(np.minimum(hi1, hi2) - np.maximum(lo1, lo2), 0)
    seen_by = Sq - (l1 + l2 - np.where((l1 > 0) & (l2 > 0), ov, 0))
    ok = np.nonzero((seen_by > 0) & (seen_by <= max_rows))[0]
    if ok.size == 0:
        return np.zeros(0, dtype=np.int64)
    cols = set(rng.choice(ok, size=min(n_cols // 2, ok.size), replace=False).tolist())
    # columns just before a change of the lower bound (ends of segments)
    ends = ok[np.isin(ok + 1, np.nonzero(np.diff(b[:, 0]) != 0)[0] + 1)]
    if ends.size:
        cols.update(ends[np.linspace(0, ends.size - 1, min(n_cols - len(cols), ends.size)).astype(int)].tolist())
    cols = np.array(sorted(cols))
    # keep the union of seeing rows bounded
    keep = []
    for c in cols:
        trial = keep + [c]
        if oracle.rows_seeing(bounds_h, Sq, trial).size <= 2 * max_rows:
            keep = trial
    return np.array(keep, dtype=np.int64)


def _run(w, tensors):
    import torch
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bf16, to_device_bounds
    q, k, v, do = tensors
    tq, tk, tv, tdo = (to_device_bf16(x) for x in (q, k, v, do))
    tb = to_device_bounds(w.bounds)
    att = MaskedAttention.for_workload(w)
    att.tile_bounds(tb)
    att.reserve_tile_cache()      # the benchmark's configuration: dQ from the tile cache
    o, lse = att.forward(tq, tk, tv, tb)
    dq, dk, dv = att.backward(tq, tk, tv, o, tdo, lse, tb)
    torch.cuda.synchronize()
    return att, dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, v=tv)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size_parity(cfg):
    import torch
    w = M.config(cfg)
    say(f"[full] config {cfg} ({M.CONFIG_NAMES[cfg]}), seed {w.seed}: drawing inputs")
    tensors = w.draw()
    att, g = _run(w, tensors)
    say(f"[full] config {cfg}: GPU done; checking the tile pass")
    check_tileinfo(w, att.read_tileinfo())

    # ---- properties over whole tensors ----
    vmax = g["v"].float().abs().amax(dim=(2, 3))                # [B][H]
    omax = g["o"].float().abs().amax(dim=(2, 3))
    assert bool((omax <= vmax * (1 + 1e-2) + 1e-2).all()), "an O row leaves the convex hull of V"
    dk = g["dk"].float()
    colsum = dk.sum(dim=2).abs().amax(dim=-1)                     # [B][H]
    scale_ref = dk.abs().sum(dim=2).amax(dim=-1).clamp_min(1e-30)
    assert bool((colsum <= 2e-2 * scale_ref).all()), f"sum_j dK_j != 0: {(colsum / scale_ref).max().item()}"
    lse = g["lse"].cpu().numpy()
    for b in range(w.B):
        for hm in range(w.Hm):
            dead = _fully_masked_rows(w.bounds[b, hm], w.Sq)
            for h in (range(w.H) if w.Hm == 1 else [hm]):
                assert np.array_equal(np.isposinf(lse[b, h]), dead), f"LSE +inf rows differ (b={b}, h={h})"

    # ---- sampled comparisons against the oracle ----
    rng = np.random.default_rng(100 + cfg)
    q, k, v, do = tensors
    up = oracle.upcast_bf16
    heads = sorted({(0, 0), (0, w.H // 2), (w.B - 1, w.H - 1)})
    errs = {"o": 0.0, "lse": 0.0}
    num = {n: 0.0 for n in ("dq", "dk", "dv")}
    den = {n: 0.0 for n in ("dq", "dk", "dv")}
    for (b, h) in heads:
        bh = w.bounds[b, oracle.mask_head(w.bounds, h)]
        qh, kh, vh, doh = up(q[b, h]), up(k[b, h]), up(v[b, h]), up(do[b, h])
        rows = _sample_rows(w, rng)
        ro, rl = oracle.head_forward(qh, kh, vh, bh, w.scale, rows)
        go = g["o"][b, h, torch.as_tensor(rows, device=g["o"].device)].float().cpu().numpy()
        gl = g["lse"][b, h].cpu().numpy()[rows]
        errs["o"] = max(errs["o"], float(np.abs(go - ro).max()))
        fin = np.isfinite(rl)
        assert np.array_equal(np.isposinf(gl), ~fin), "LSE +inf positions differ on the sample"
        if fin.any():
            errs["lse"] = max(errs["lse"], float(np.abs(gl[fin] - rl[fin]).max()))
        rdq, _, _ = oracle.head_backward(qh, kh, vh, doh, bh, w.scale, rows, rl)
        gdq = g["dq"][b, h, torch.as_tensor(rows, device=g["dq"].device)].float().cpu().numpy()
        num["dq"] += float(np.sum((gdq - rdq) ** 2))
        den["dq"] += float(np.sum(rdq ** 2))
        cols = _sample_cols(w, bh, rng)
        if cols.size:
            seeing = oracle.rows_seeing(bh, w.Sq, cols)
            _, lse_s = oracle.head_forward(qh, kh, vh, bh, w.scale, seeing)
            _, rdk, rdv = oracle.head_backward(qh, kh, vh, doh, bh, w.scale, seeing, lse_s)
            ci = torch.as_tensor(cols, device=g["dk"].device)
            for n, ref in (("dk", rdk[cols]), ("dv", rdv[cols])):
                got = g[n][b, h, ci].float().cpu().numpy()
                num[n] += float(np.sum((got - ref) ** 2))
                den[n] += float(np.sum(ref ** 2))
        say(f"[full] config {cfg} head ({b},{h}): {rows.size} rows, {cols.size} key columns compared")
    assert errs["o"] <= O_TOL, f"O max-abs {errs['o']}"
    assert errs["lse"] <= LSE_TOL, f"LSE max-abs {errs['lse']}"
    rel = {n: (np.sqrt(num[n] / den[n]) if den[n] > 0 else np.sqrt(num[n])) for n in num}
    for n, e in rel.items():
        assert e <= GRAD_TOL, f"{n} rel-L2 {e} on the sample"
    say(f"[full] config {cfg}: O max-abs {errs['o']:.2e}, LSE {errs['lse']:.2e}, "
        + ", ".join(f"{n} rel-L2 {e:.2e}" for n, e in rel.items()))


def _heaviest_key_block(bounds_h, Sq, BK=128):
    """The key block whose columns are seen by the most query rows (the
    longest key-stationary item of the backward): per column, Sq minus the
    rows its two intervals hide, then the block maximum."""
    b = np.clip(bounds_h.astype(np.int64), 0, Sq)
    l1 = np.maximum(b[:, 1] - b[:, 0], 0)
    l2 = np.maximum(b[:, 3] - b[:, 2], 0)
    ov = np.maximum(np.minimum(b[:, 1], b[:, 3]) - np.maximum(b[:, 0], b[:, 2]), 0)
    seen = Sq - (l1 + l2 - np.where((l1 > 0) & (l2 > 0), ov, 0))
    return int(np.argmax(seen)) // BK


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_heavy_key_columns(cfg):
    """dK and dV of the whole key block that the most query rows see, compared
    element by element with the oracle over every row that sees it (the
    backward's longest key-stationary item: the shared question's first
    block, seen by all 32768 rows, at the share-question workload; the first
    block of the longest document, seen by its 43257 rows, at the 128K
    documents workload; the densest block of the context-parallel share).
    The oracle runs the forward over those rows for their LSE and O, then
    the gradients of the block's columns alone."""
    import torch
    w = M.config(cfg)
    b, h = 0, 0
    bh = w.bounds[b, oracle.mask_head(w.bounds, h)]
    kb = _heaviest_key_block(bh, w.Sq)
    cols = np.arange(kb * 128, min(w.Sk, kb * 128 + 128))
    rows = oracle.rows_seeing(bh, w.Sq, cols)
    say(f"[heavy] config {cfg}: key block {kb} seen by {rows.size} rows; drawing inputs")
    tensors = w.draw()
    _, g = _run(w, tensors)
    ci = torch.as_tensor(cols, device=g["dk"].device)
    got = {n: g[n][b, h, ci].float().cpu().numpy() for n in ("dk", "dv")}
    del g
    say(f"[heavy] config {cfg}: GPU done; oracle over {rows.size} rows")
    q, k, v, do = tensors
    up = oracle.upcast_bf16
    qh, kh, vh, doh = up(q[b, h]), up(k[b, h]), up(v[b, h]), up(do[b, h])
    o_r, lse_r = oracle.head_forward(qh, kh, vh, bh, w.scale, rows)
    rdk, rdv = oracle.column_gradients(qh, kh, vh, doh, bh, w.scale, cols, rows, o_r, lse_r)
    for n, ref in (("dk", rdk), ("dv", rdv)):
        e = rel_l2(got[n], ref)
        say(f"[heavy] config {cfg}: {n} of key block {kb} rel-L2 {e:.2e}")
        assert e <= GRAD_TOL, f"{n} rel-L2 {e} on key block {kb}"


def test_context_parallel_shares_add_up():
    """The eight ranks' shares of the context-parallel workload (each: its two
    query chunks, all keys, its own clipped-and-shifted bounds) reproduce one
    global call: each rank's O and LSE equal the global rows, and the ranks'
    dK, dV add up to the global dK, dV (FlashMask-3 paper summary, abstract:
    the per-rank localisation needs no communication and feeds the same
    single-GPU kernel).  Each rank's bounds come from fm_localize_bounds on
    the device."""
    import torch
    from column_sparse_masked_amd.api import MaskedAttention, localize_bounds, to_device_bf16, to_device_bounds
    H, S, D, world = 16, 65536, 128, 8
    base = M.cp_rank_share(H=H, S=S, D=D, world=world, rank=0, seed=5)
    gb = base.structure["global_bounds"]
    say("[cp] drawing global inputs")
    sq, sk, sv, sdo = np.random.SeedSequence(55).spawn(4)
    q, k, v, do = (M.draw_bf16_normal(ss, (1, H, S, D)) for ss in (sq, sk, sv, sdo))
    tq, tk, tv, tdo = (to_device_bf16(x) for x in (q, k, v, do))
    glob = M.custom(gb, B=1, H=H, Sq=S, D=D, seed=0, name="cp_global")
    gatt = MaskedAttention.for_workload(glob)
    tgb = to_device_bounds(glob.bounds)
    gatt.tile_bounds(tgb)
    gatt.reserve_tile_cache()
    go, glse = gatt.forward(tq, tk, tv, tgb)
    gdq, gdk, gdv = gatt.backward(tq, tk, tv, go, tdo, glse, tgb)
    sum_dk = torch.zeros_like(gdk, dtype=torch.float32)
    sum_dv = torch.zeros_like(gdv, dtype=torch.float32)
    C = S // (2 * world)
    for r in range(world):
        share = M.cp_rank_share(H=H, S=S, D=D, world=world, rank=r, seed=5)
        idx = torch.as_tensor(share.structure["global_rows"], device=tq.device)
        lq, ldo = tq[:, :, idx].contiguous(), tdo[:, :, idx].contiguous()
        att = MaskedAttention.for_workload(share)
        # the rank's bounds localised on the device from the global ones
        tb = localize_bounds(tgb, [r * C, (2 * world - 1 - r) * C], [C, C])
        assert np.array_equal(tb.cpu().numpy(), share.bounds), f"rank {r}: localised bounds differ"
        att.tile_bounds(tb)
        att.reserve_tile_cache()
        lo, llse = att.forward(lq, tk, tv, tb)
        ldq, ldk, ldv = att.backward(lq, tk, tv, lo, ldo, llse, tb)
        torch.cuda.synchronize()
        err_o = (lo.float() - go[:, :, idx].float()).abs().max().item()
        assert err_o <= O_TOL, f"rank {r}: O differs from the global rows by {err_o}"
        gl, ll = glse[:, :, idx], llse
        assert torch.equal(torch.isinf(gl), torch.isinf(ll)), f"rank {r}: LSE +inf rows differ"
        fin = torch.isfinite(gl)
        if fin.any():
            assert (gl[fin] - ll[fin]).abs().max().item() <= LSE_TOL, f"rank {r}: LSE differs"
        dq_rel = ((ldq.float() - gdq[:, :, idx].float()).norm() / gdq[:, :, idx].float().norm().clamp_min(1e-30)).item()
        assert dq_rel <= GRAD_TOL, f"rank {r}: dQ rel-L2 {dq_rel}"
        sum_dk += ldk.float()
        sum_dv += ldv.float()
        say(f"[cp] rank {r}: rows {r * C}.. and {(2 * world - 1 - r) * C}.., O err {err_o:.2e}, dQ rel {dq_rel:.2e}")
    for n, s_, gref in (("dk", sum_dk, gdk), ("dv", sum_dv, gdv)):
        rel = ((s_ - gref.float()).norm() / gref.float().norm().clamp_min(1e-30)).item()
        assert rel <= GRAD_TOL, f"sum over ranks of {n} differs from the global {n}: rel-L2 {rel}"
        say(f"[cp] sum over ranks of {n}: rel-L2 {rel:.2e}")
