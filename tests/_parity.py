"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare with the fp64 oracle.

Tolerances (fixed by the evaluation contract for this library):
  O      max-abs <= 2e-2 over the tensor,
  dQ/dK/dV  relative L2 = ||x - ref|| / ||ref|| <= 1e-2 per tensor,
  LSE    max-abs <= 1e-3 on finite entries, +inf at the same positions,
  tile classes, key-block summaries, counts, lists: bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

O_TOL = 2e-2
GRAD_TOL = 1e-2
LSE_TOL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(w, tensors=None, device="cuda", want_bwd=True, both_paths=False, fwd_rows=0):
    """Upload a workload, run tile pass + forward (+ backward) on the GPU and
    return numpy results (float64) and the tileinfo dictionary.  The backward
    runs with the tile cache (dQ from the cached dS / scale, as the benchmark
    runs it); with both_paths it runs again without the cache (dQ recomputed)
    into dq_rc, dk_rc, dv_rc.  fwd_rows: query rows per forward item (0: the
    library's choice; 256: pairs of query blocks)."""
    import torch
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bf16, to_device_bounds
    q, k, v, do = tensors if tensors is not None else w.draw()
    tq, tk, tv, tdo = (to_device_bf16(x, device) for x in (q, k, v, do))
    tb = to_device_bounds(w.bounds, device)
    att = MaskedAttention.for_workload(w, device, fwd_rows)
    att.tile_bounds(tb)
    o, lse = att.forward(tq, tk, tv, tb)
    res = {"o": o, "lse": lse}
    if want_bwd:
        att.reserve_tile_cache()
        dq, dk, dv = att.backward(tq, tk, tv, o, tdo, lse, tb)
        res.update(dq=dq, dk=dk, dv=dv)
        if both_paths:
            att.drop_tile_cache()
            dq2, dk2, dv2 = att.backward(tq, tk, tv, o, tdo, lse, tb)
            res.update(dq_rc=dq2, dk_rc=dk2, dv_rc=dv2)
    torch.cuda.synchronize()
    out = {n: t.float().cpu().numpy().astype(np.float64) for n, t in res.items()}
    out["tileinfo"] = att.read_tileinfo()
    return out, (q, k, v, do)


def rel_l2(x, ref):
    nr = np.linalg.norm(ref)
    if nr == 0:
        return float(np.linalg.norm(x))
    return float(np.linalg.norm(x - ref) / nr)


def check_lse(got, ref):
    ref_inf = np.isposinf(ref)
    assert np.array_equal(np.isposinf(got), ref_inf), "LSE +inf positions differ"
    fin = ~ref_inf
    if fin.any():
        err = float(np.abs(got[fin] - ref[fin]).max())
        assert err <= LSE_TOL, f"LSE max-abs {err}"


def check_full(w, got, tensors, label=""):
    """Complete oracle comparison (small problems)."""
    up = oracle.upcast_bf16
    q, k, v, do = tensors
    ro, rl, rdq, rdk, rdv = oracle.attention(up(q), up(k), up(v), up(do), w.bounds, w.scale)
    err_o = float(np.abs(got["o"] - ro).max()) if ro.size else 0.0
    assert err_o <= O_TOL, f"{label} O max-abs {err_o}"
    check_lse(got["lse"], rl)
    errs = {}
    for n, r in (("dq", rdq), ("dk", rdk), ("dv", rdv), ("dq_rc", rdq), ("dk_rc", rdk), ("dv_rc", rdv)):
        if n in got:
            errs[n] = rel_l2(got[n], r)
            assert errs[n] <= GRAD_TOL, f"{label} {n} rel-L2 {errs[n]}"
    # the two backward paths run the same dK / dV kernel: identical dK, dV
    for n in ("dk", "dv"):
        if n + "_rc" in got:
            assert np.array_equal(got[n], got[n + "_rc"]), f"{label} {n} differs between the dQ paths"
    say(f"{label}: O max-abs {err_o:.3e} " + " ".join(f"{n} {e:.3e}" for n, e in errs.items()))
    return err_o, errs


def expected_pairs(w, fwd_rows=0):
    """Whether the library runs the forward on pairs of query blocks: asked
    for (fwd_rows 256), or with head_dim 128 and at least two pairs per
    compute unit (the pair kernel's grid), unless fwd_rows is 128."""
    from column_sparse_masked_amd import _lib
    if w.D != 128 or fwd_rows == 128:
        return False
    if fwd_rows == 256:
        return True
    nQ = -(-w.Sq // 128)
    return w.B * w.H * ((nQ + 1) // 2) >= 2 * _lib.device_cu_count()


def pair_lists(cls):
    """Per pair of query blocks (2qp, 2qp+1 < nQ): the key blocks either one
    sees, in increasing order, each with the flags: bit 16 block 2qp sees it,
    bit 17 that tile is partial, bits 18, 19 the same for block 2qp+1."""
    B, Hm, nQ, nK = cls.shape
    nP = (nQ + 1) // 2
    lists = {}
    cnt = np.zeros((B, Hm, nP), np.int64)
    for b in range(B):
        for hm in range(Hm):
            for qp in range(nP):
                c0 = cls[b, hm, 2 * qp].astype(np.int64)
                c1 = cls[b, hm, 2 * qp + 1].astype(np.int64) if 2 * qp + 1 < nQ else np.zeros(nK, np.int64)
                kbs = np.nonzero((c0 != 0) | (c1 != 0))[0]
                lists[b, hm, qp] = (kbs | ((c0[kbs] != 0) << 16) | ((c0[kbs] == 2) << 17)
                                    | ((c1[kbs] != 0) << 18) | ((c1[kbs] == 2) << 19))
                cnt[b, hm, qp] = kbs.size
    return lists, cnt


def check_tileinfo(w, ti, fwd_rows=0):
    """Bit-exact tile pass against the oracle's classification."""
    kbsum, cls, cq, ck = oracle.classify(w.bounds, w.Sq, 128, 128)
    assert np.array_equal(ti["kbsum"], kbsum), "kbsum differs"
    assert np.array_equal(ti["cls"], cls), "tile classes differ"
    assert np.array_equal(ti["cnt_q"], cq), "cnt_q differs"
    assert np.array_equal(ti["cnt_k"], ck), "cnt_k differs"
    B, Hm, nQ, nK = cls.shape
    for b in range(B):
        for hm in range(Hm):
            for qb in range(nQ):
                row = cls[b, hm, qb]
                kbs = np.nonzero(row)[0]
                want = kbs | np.where(row[kbs] == 2, 0x8000, 0)
                assert np.array_equal(ti["list_q"][b, hm, qb, :kbs.size], want), (b, hm, qb)
            for kb in range(nK):
                col = cls[b, hm, :, kb]
                qbs = np.nonzero(col)[0]
                want = qbs | np.where(col[qbs] == 2, 0x8000, 0)
                assert np.array_equal(ti["list_k"][b, hm, kb, :qbs.size], want), (b, hm, kb)
    # pair mode: the union lists of the query-block pairs and their counts
    pairs = expected_pairs(w, fwd_rows)
    c = ti["counters"]
    assert c[11] == (1 if pairs else 0), "pair mode differs"
    nP = (nQ + 1) // 2
    if pairs:
        plists, cp = pair_lists(cls)
        assert np.array_equal(ti["cnt_p"], cp), "cnt_p differs"
        for key, want in plists.items():
            assert np.array_equal(ti["list_p"][key][:want.size].astype(np.int64), want), ("list_p", key)
    # queues: a permutation of every item, tile counts non-increasing
    H = w.H
    fwd = ("fwd_queue", cp, nP) if pairs else ("fwd_queue", cq, nQ)
    for name, cnt, nb in (fwd, ("bwd_queue", ck, nK)):
        qu = ti[name][:B * H * nb].astype(np.int64)
        assert np.array_equal(np.sort(qu), np.arange(B * H * nb)), name
        bh, blk = qu // nb, qu % nb
        b_, h_ = bh // H, bh % H
        cost = cnt[b_, 0 if Hm == 1 else h_, blk]
        assert np.all(np.diff(np.minimum(cost, 4095)) <= 0), f"{name} not sorted by tile count"
    assert c[0] == B * H * (nP if pairs else nQ) and c[1] == B * H * nK and c[2] == 0 and c[3] == 0
    assert c[8] == (0 if pairs else expected_split_count(cq, H, Hm)), "number of split forward items differs"
    # the backward's tile slots: each listed tile's position in its key
    # block's list, and each backward item's first slot.  Slots go to the
    # (b, mask head, key block) entries in order, and within an entry to the
    # heads sharing it one after the other: item h of entry e starts at
    # reps * (tiles of the entries before e) + h * cnt[e], reps = H / Hm.
    for b in range(B):
        for hm in range(Hm):
            for kb in range(nK):
                qbs = np.nonzero(cls[b, hm, :, kb])[0]
                assert np.array_equal(ti["cpos"][b, hm, kb, qbs], np.arange(qbs.size)), ("cpos", b, hm, kb)
    reps = H // Hm
    ent = ck.reshape(-1).astype(np.int64)                             # entries (b, hm, kb)
    before = np.concatenate([[0], np.cumsum(ent)[:-1]]) if ent.size else ent
    want = np.zeros((B, H, nK), np.int64)
    for h in range(H):
        r, hm = (h, 0) if Hm == 1 else (0, h)
        want[:, h, :] = (reps * before + r * ent).reshape(B, Hm, nK)[:, hm, :]
    want = np.minimum(want, 2 ** 32 - 1)
    # each item's slots are its own: the ranges [start, start + count) tile
    # 0 .. total - 1 without gaps or overlaps
    per_item = np.repeat(ck, reps, axis=1) if Hm == 1 else ck        # [B][H][nK]
    counts = per_item.reshape(-1).astype(np.int64)
    order = np.lexsort((counts, want.reshape(-1)))      # by start, empty items first
    starts, counts = want.reshape(-1)[order], counts[order]
    assert np.array_equal(starts[1:], (starts + counts)[:-1]) and (starts.size == 0 or starts[0] == 0)
    assert np.array_equal(ti["colbase"].astype(np.int64), want.reshape(-1)), "colbase differs"
    assert c[9] == int(per_item.sum()), "tile count differs"
    assert c[10] == 0


def expected_split_count(cq, H, Hm):
    """Forward items the tile pass splits in two: none when there are at
    least 4 W items; else those with more than
    max(16, ceil(total / (2 W))) non-skipped tiles, W the forward's persistent
    grid (two workgroups per compute unit), at most min(items, 512) of them,
    none when the threshold or any item reaches the top bucket of the sort
    (4095 tiles)."""
    from column_sparse_masked_amd import _lib
    B, Hm_, nQ = cq.shape
    per_item = np.repeat(cq, H // Hm, axis=1) if Hm == 1 else cq      # [B][H][nQ]
    total = int(per_item.sum())
    W = 2 * _lib.device_cu_count()
    if B * per_item.shape[1] * nQ >= 4 * W:      # enough items per workgroup: never split
        return 0
    thr = max(16, -(-total // (2 * W)))
    if thr >= 4095 or (per_item >= 4095).any():
        return 0
    return min(int((per_item > thr).sum()), min(B * H * nQ, 512))


# --------------------------------------------------------------------------- #
# fp8 forward                                                                  #
# --------------------------------------------------------------------------- #
# Tolerance contract of the fp8 forward, derived from what its kernel rounds.
# Its scores are exact products of E4M3 values accumulated in fp32, so LSE
# keeps the bf16 forward's bound.  Its probabilities p (relative to a running
# reference m' with m' <= the row maximum m) are rounded to E4M3 before the
# P.V product: |round(p) - p| <= 2^-4 p for normal values and <= 2^-10 for
# subnormal ones.  With l' = sum_j p_j >= l = sum_j exp(s_j - m), the error of
# O_id = sum_j p_j v_jd / l' is at most
#     2^-4 sum_j P_ij |v_jd|  +  2^-10 sum_{j visible} |v_jd| / l_i
# (P the exact softmax), plus bf16 rounding of O (2^-8 |O| covers it) and a
# small fp32 allowance.  Over a tensor, the errors are a weighted mean of
# independent relative roundings, so ||O - O_ref|| / ||O_ref|| <= 2^-4.
FP8_O_REL_L2 = 2.0 ** -4


def fp8_decoded(codes, descale):
    q8, k8, v8 = codes
    return tuple(oracle.decode_e4m3(c) * float(d) for c, d in zip((q8, k8, v8), descale))


def fp8_head_check(qd, kd, vd, bounds_h, scale, rows, go, gl):
    """Compare GPU O (rows x D, float64) and LSE (rows) of one head with the
    exact attention of the decoded inputs, within the per-element bound
    above.  Returns (sum of squared errors, sum of squared references, max
    LSE error, max error / bound)."""
    num = den = lse_err = worst = 0.0
    for s0 in range(0, rows.size, 256):
        r = rows[s0:s0 + 256]
        vis = ~oracle.dense_mask(bounds_h, r)
        s = scale * (qd[r] @ kd.T)
        s[~vis] = -np.inf
        m = s.max(axis=1) if s.shape[1] else np.full(r.size, -np.inf)
        live = np.isfinite(m)
        e = np.zeros_like(s)
        e[live] = np.exp(s[live] - m[live, None])
        l = e.sum(axis=1)
        P = np.zeros_like(s)
        P[live] = e[live] / l[live, None]
        ref = P @ vd
        absv = np.abs(vd)
        bound = np.zeros_like(ref)
        bound[live] = (2.0 ** -4 * (P[live] @ absv) + 2.0 ** -10 * (vis[live] @ absv) / l[live, None]
                       + 2.0 ** -8 * np.abs(ref[live]) + 1e-5 * (absv.max() if absv.size else 0.0))
        o = go[s0:s0 + 256]
        lse = gl[s0:s0 + 256]
        assert (o[~live] == 0).all(), "a row with no visible key has O != 0"
        assert np.isposinf(lse[~live]).all() and np.isfinite(lse[live]).all(), "LSE +inf positions differ"
        err = np.abs(o - ref)
        if live.any():
            worst = max(worst, float((err[live] / bound[live]).max()))
            lse_err = max(lse_err, float(np.abs(lse[live] - (m[live] + np.log(l[live]))).max()))
        num += float(np.sum(err ** 2))
        den += float(np.sum(ref ** 2))
    return num, den, lse_err, worst


def run_gpu_fp8(w, codes, descale, device="cuda", fwd_rows=0):
    import torch
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bounds, to_device_u8
    tq, tk, tv = (to_device_u8(c, device) for c in codes)
    tb = to_device_bounds(w.bounds, device)
    att = MaskedAttention.for_workload(w, device, fwd_rows)
    att.tile_bounds(tb)
    o, lse = att.forward_fp8(tq, tk, tv, descale, tb)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), att


def check_fp8(w, go, gl, codes, descale, heads=None, rows_of=None, label=""):
    qd, kd, vd = fp8_decoded(codes, descale)
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    num = den = lse_err = worst = 0.0
    for (b, h) in heads:
        bh = w.bounds[b, oracle.mask_head(w.bounds, h)]
        rows = np.arange(w.Sq) if rows_of is None else rows_of(b, h)
        n_, d_, le, wo = fp8_head_check(qd[b, h], kd[b, h], vd[b, h], bh, w.scale, rows,
                                        go[b, h][rows], gl[b, h][rows])
        num, den = num + n_, den + d_
        lse_err, worst = max(lse_err, le), max(worst, wo)
    rel = float(np.sqrt(num / den)) if den > 0 else float(np.sqrt(num))
    say(f"{label}: fp8 O rel-L2 {rel:.3e}, max error/bound {worst:.3f}, LSE max-abs {lse_err:.2e}")
    assert worst <= 1.0, f"{label} O error above its bound ({worst})"
    assert rel <= FP8_O_REL_L2, f"{label} O rel-L2 {rel}"
    assert lse_err <= LSE_TOL, f"{label} LSE max-abs {lse_err}"
    return rel, worst, lse_err
