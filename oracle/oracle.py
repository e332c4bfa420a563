"""Plain, slow, float64 CPU oracle for column-sparse masked attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  It shares no code with the HIP
library or its Python binding, and it never imports either.

What it computes (FlashMask-3 paper summary, abstract: a structured mask is
stored per key column as the row ranges that column hides):

* mask:  element (i, j) is masked iff LTS[j] <= i < LTE[j] or
  UTS[j] <= i < UTE[j]  (half-open intervals, empty when start >= end);
* forward: scaled dot-product attention with masked scores at -inf;
  a row with every score masked outputs O = 0 and LSE = +inf;
* backward: the exact gradients of that forward with respect to Q, K, V;
* tile classification: per key block the min/max of the clamped bounds, and
  each (query block, key block) tile classed skip (0) / full (1) / partial (2).

Everything is written as its definition: the dense mask is materialised for a
strip of rows, scores are an fp64 matrix product, softmax is taken row by row.
Restricting a strip to the column range its own dense mask leaves visible is
exact, because masked terms are exactly zero.

Parity pins (in tests/test_oracle.py) tie every function to something other than
itself: hand-drawn masks, torch's float64 SDPA, central finite differences,
closed forms and invariants, and brute-force tile classes.
"""
from __future__ import annotations

import numpy as np

STRIP = 256


# --------------------------------------------------------------------------- #
# inputs                                                                      #
# --------------------------------------------------------------------------- #
def upcast_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- #
# the mask                                                                    #
# --------------------------------------------------------------------------- #
def dense_mask(bounds: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """bool[len(rows)][Sk], True where (i, j) is masked.

    ``bounds`` is int[Sk][4] = (LTS, LTE, UTS, UTE) for one mask head; the
    predicate is the two half-open row intervals per key column."""
    b = np.asarray(bounds, dtype=np.int64)
    i = np.asarray(rows, dtype=np.int64)[:, None]
    lower = (b[None, :, 0] <= i) & (i < b[None, :, 1])
    upper = (b[None, :, 2] <= i) & (i < b[None, :, 3])
    return lower | upper


def mask_head(bounds_all: np.ndarray, h: int) -> int:
    """Mask head used by attention head h (one mask for all heads, or one per head)."""
    return 0 if bounds_all.shape[1] == 1 else h


# --------------------------------------------------------------------------- #
# forward                                                                     #
# --------------------------------------------------------------------------- #
def _strip_scores(qh, kh, bounds_h, scale, rows):
    """Masked scores of one strip of rows, restricted to the visible column range."""
    M = dense_mask(bounds_h, rows)
    vis_cols = np.nonzero(~M.all(axis=0))[0]
    if vis_cols.size == 0:
        return None, None, None
    c0, c1 = int(vis_cols[0]), int(vis_cols[-1]) + 1
    S = scale * (qh[rows] @ kh[c0:c1].T)
    S[M[:, c0:c1]] = -np.inf
    return S, c0, c1


def head_forward(qh, kh, vh, bounds_h, scale, rows=None):
    """O[rows] and LSE[rows] for one (batch, head); inputs float64 2-D."""
    Sq, D = qh.shape
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    O = np.zeros((rows.size, vh.shape[1]))
    L = np.full(rows.size, np.inf)
    for s0 in range(0, rows.size, STRIP):
        r = rows[s0:s0 + STRIP]
        S, c0, c1 = _strip_scores(qh, kh, bounds_h, scale, r)
        if S is None:
            continue
        m = S.max(axis=1)
        live = np.isfinite(m)
        e = np.zeros_like(S)
        e[live] = np.exp(S[live] - m[live, None])
        l = e.sum(axis=1)
        P = np.zeros_like(S)
        P[live] = e[live] / l[live, None]
        O[s0:s0 + r.size] = P @ vh[c0:c1]
        L[s0:s0 + r.size][live] = m[live] + np.log(l[live])
    return O, L


def forward(q, k, v, bounds, scale):
    """O [B][H][Sq][Dv], LSE [B][H][Sq] (float64) for float64 q, k, v."""
    B, H, Sq, D = q.shape
    O = np.zeros((B, H, Sq, v.shape[-1]))
    L = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = head_forward(q[b, h], k[b, h], v[b, h],
                                            bounds[b, mask_head(bounds, h)], scale)
    return O, L


# --------------------------------------------------------------------------- #
# the fp8 forward                                                             #
# --------------------------------------------------------------------------- #
def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point, E4M3 format (OCP OFP8 specification, the
    E4M3 encoding table) -> float64, exactly.  Bit 7 is the sign, bits 6..3 the
    exponent (bias 7), bits 2..0 the mantissa.  Exponent field 0 encodes
    subnormals m/8 * 2^-6; the code with every exponent and mantissa bit set
    is NaN; there are no infinities, so the largest finite value is
    1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def forward_fp8(q8, k8, v8, descale, bounds, scale):
    """O [B][H][Sq][D], LSE [B][H][Sq] (float64) of the fp8 forward.

    The pages name FP8 mixed precision as part of FlashMask V3 (PaddlePaddle
    3.2.0 release note, FlashMask V3 highlights) and give nothing more.  The
    reading taken: Q, K and V arrive as E4M3 codes with one fp32 descale
    factor per tensor (value = decode(code) * descale), and the result is the
    same masked attention of those values.  This is that definition: decode,
    scale, and the float64 forward above.  Rounding the kernel does on the
    way (P to E4M3 before the P V product) is not modelled here; its effect is
    bounded in the tests."""
    dq, dk, dv = (float(x) for x in descale)
    return forward(decode_e4m3(q8) * dq, decode_e4m3(k8) * dk, decode_e4m3(v8) * dv, bounds, scale)


# --------------------------------------------------------------------------- #
# backward                                                                    #
# --------------------------------------------------------------------------- #
def head_backward(qh, kh, vh, doh, bounds_h, scale, rows=None, lse=None):
    """Gradients for one (batch, head).

    Returns dQ[rows] and the contributions of ``rows`` to dK, dV over all key
    columns.  With ``rows`` = every row, dK and dV are complete; with ``rows`` =
    every row that sees a set of columns C, dK[C] and dV[C] are complete.

    P = exp(S - LSE) (zero where masked and on fully masked rows),
    dP = dO V^T, Delta_i = sum_j P_ij dP_ij, dS = P * (dP - Delta),
    dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO."""
    Sq, D = qh.shape
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    if lse is None:
        _, lse = head_forward(qh, kh, vh, bounds_h, scale, rows)
    dQ = np.zeros((rows.size, D))
    dK = np.zeros_like(kh)
    dV = np.zeros_like(vh)
    for s0 in range(0, rows.size, STRIP):
        r = rows[s0:s0 + STRIP]
        S, c0, c1 = _strip_scores(qh, kh, bounds_h, scale, r)
        if S is None:
            continue
        P = np.exp(S - lse[s0:s0 + r.size, None])
        dP = doh[r] @ vh[c0:c1].T
        delta = (P * dP).sum(axis=1)
        dS = P * (dP - delta[:, None])
        dQ[s0:s0 + r.size] = scale * (dS @ kh[c0:c1])
        dK[c0:c1] += scale * (dS.T @ qh[r])
        dV[c0:c1] += P.T @ doh[r]
    return dQ, dK, dV


def column_gradients(qh, kh, vh, doh, bounds_h, scale, cols, rows, o_rows, lse_rows):
    """dK[cols] and dV[cols] for one (batch, head), complete when ``rows``
    holds every query row that sees one of ``cols``; ``o_rows`` and
    ``lse_rows`` are the forward's O and LSE of those rows.

    The same gradients as head_backward, restricted to a few key columns so
    that heavily seen columns of long sequences stay affordable: for
    j in cols, P_ij = exp(scale q_i.k_j - LSE_i) (0 where masked),
    dP_ij = dO_i.v_j, Delta_i = dO_i.O_i (equal to sum_j P_ij dP_ij, because
    O_i = sum_j P_ij v_j), dS_ij = P_ij (dP_ij - Delta_i),
    dK_j = scale sum_i dS_ij q_i, dV_j = sum_i P_ij dO_i."""
    cols = np.asarray(cols)
    rows = np.asarray(rows)
    dK = np.zeros((cols.size, kh.shape[1]))
    dV = np.zeros((cols.size, vh.shape[1]))
    for s0 in range(0, rows.size, STRIP):
        r = rows[s0:s0 + STRIP]
        lse = lse_rows[s0:s0 + r.size]
        live = np.isfinite(lse)
        if not live.any():
            continue
        r, lse, o = r[live], lse[live], o_rows[s0:s0 + STRIP][live]
        M = dense_mask(bounds_h[cols], r)
        S = scale * (qh[r] @ kh[cols].T)
        P = np.exp(S - lse[:, None])
        P[M] = 0.0
        dP = doh[r] @ vh[cols].T
        delta = (doh[r] * o).sum(axis=1)
        dS = P * (dP - delta[:, None])
        dK += scale * (dS.T @ qh[r])
        dV += P.T @ doh[r]
    return dK, dV


def backward(q, k, v, do, bounds, scale, lse=None):
    """dQ, dK, dV (float64) for float64 inputs."""
    B, H, Sq, D = q.shape
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = head_backward(
                q[b, h], k[b, h], v[b, h], do[b, h], bounds[b, mask_head(bounds, h)],
                scale, None, None if lse is None else lse[b, h])
    return dQ, dK, dV


def attention(q, k, v, do, bounds, scale):
    """Forward and backward together: (O, LSE, dQ, dK, dV)."""
    O, L = forward(q, k, v, bounds, scale)
    dQ, dK, dV = backward(q, k, v, do, bounds, scale, lse=L)
    return O, L, dQ, dK, dV


def rows_seeing(bounds_h, Sq, cols) -> np.ndarray:
    """Every query row that sees at least one of the key columns ``cols``."""
    cols = np.asarray(cols)
    out = []
    for s0 in range(0, Sq, 4096):
        r = np.arange(s0, min(Sq, s0 + 4096))
        M = dense_mask(bounds_h[cols], r)
        out.append(r[~M.all(axis=1)])
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


# --------------------------------------------------------------------------- #
# context-parallel localisation                                               #
# --------------------------------------------------------------------------- #
def localize_bounds(global_bounds, chunk_start, chunk_len):
    """One context-parallel rank's bounds (FlashMask-3 paper summary,
    abstract: a rank's mask comes from the global boundary vectors without
    communication).  The rank's local rows are its chunks' global rows
    stacked in the given (increasing) order; a global bound g becomes the
    number of local rows whose global index is below g, counted directly:
    the plain definition, which makes a local row masked exactly when its
    global row is.  Returns int64 values of the same shape."""
    rows = np.concatenate([np.arange(int(s), int(s) + int(n), dtype=np.int64)
                           for s, n in zip(chunk_start, chunk_len)] + [np.zeros(0, np.int64)])
    g = np.asarray(global_bounds, dtype=np.int64)
    # count of rows < g for every bound: searchsorted on the sorted rows
    return np.searchsorted(np.sort(rows), g, side="left").astype(np.int64)


# --------------------------------------------------------------------------- #
# tile classification                                                         #
# --------------------------------------------------------------------------- #
SKIP, FULL, PARTIAL = 0, 1, 2


def key_block_summary(bounds_h, Sq, BK):
    """int64[nK][8]: per key block, over its columns j < Sk, the min and max of
    each bound after clamping to [0, Sq]:
    (LTS min, LTS max, LTE min, LTE max, UTS min, UTS max, UTE min, UTE max)."""
    Sk = bounds_h.shape[0]
    nK = -(-Sk // BK)
    out = np.zeros((nK, 8), dtype=np.int64)
    for kb in range(nK):
        blk = np.clip(np.asarray(bounds_h[kb * BK:min(Sk, (kb + 1) * BK)], dtype=np.int64), 0, Sq)
        for c in range(4):
            out[kb, 2 * c] = blk[:, c].min()
            out[kb, 2 * c + 1] = blk[:, c].max()
    return out


def classify_tile(ks, q0, q1):
    """Class of rows [q0, q1) against one key block summary ``ks``.

    skip: one of the two intervals covers every row of the tile in every column
    (its latest start <= q0 and its earliest end >= q1);
    full: neither interval meets the tile in any column (each interval starts
    at or after q1 in every column, or ends at or before q0 in every column);
    partial: otherwise."""
    lts_min, lts_max, lte_min, lte_max, uts_min, uts_max, ute_min, ute_max = ks
    if (lts_max <= q0 and lte_min >= q1) or (uts_max <= q0 and ute_min >= q1):
        return SKIP
    lower_clear = lts_min >= q1 or lte_max <= q0
    upper_clear = uts_min >= q1 or ute_max <= q0
    return FULL if (lower_clear and upper_clear) else PARTIAL


def classify(bounds, Sq, BQ, BK):
    """For bounds [B][Hm][Sk][4]: kbsum [B][Hm][nK][8], cls [B][Hm][nQ][nK]
    (0 skip, 1 full, 2 partial), non-skipped counts per query block
    cnt_q [B][Hm][nQ] and per key block cnt_k [B][Hm][nK]."""
    B, Hm, Sk, _ = bounds.shape
    nQ, nK = -(-Sq // BQ), -(-Sk // BK)
    kbsum = np.zeros((B, Hm, nK, 8), dtype=np.int64)
    cls = np.zeros((B, Hm, nQ, nK), dtype=np.uint8)
    for b in range(B):
        for hm in range(Hm):
            kbsum[b, hm] = key_block_summary(bounds[b, hm], Sq, BK)
            for qb in range(nQ):
                q0, q1 = qb * BQ, min(Sq, (qb + 1) * BQ)
                for kb in range(nK):
                    cls[b, hm, qb, kb] = classify_tile(kbsum[b, hm, kb], q0, q1)
    nonskip = cls != SKIP
    return kbsum, cls, nonskip.sum(axis=3).astype(np.int64), nonskip.sum(axis=2).astype(np.int64)


def exact_tile_classes(bounds_h, Sq, BQ, BK):
    """Brute force from the dense mask: 0 if every element of the tile is
    masked, 1 if none is, 2 otherwise (columns >= Sk and rows >= Sq excluded)."""
    Sk = bounds_h.shape[0]
    nQ, nK = -(-Sq // BQ), -(-Sk // BK)
    out = np.zeros((nQ, nK), dtype=np.uint8)
    for qb in range(nQ):
        M = dense_mask(bounds_h, np.arange(qb * BQ, min(Sq, (qb + 1) * BQ)))
        for kb in range(nK):
            t = M[:, kb * BK:min(Sk, (kb + 1) * BK)]
            out[qb, kb] = SKIP if t.all() else (FULL if not t.any() else PARTIAL)
    return out
