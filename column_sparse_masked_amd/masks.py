"""Seeded synthetic workloads for column-sparse masked attention.

This module only *describes inputs*: the four boundary vectors of a structured
mask and the bf16 tensors Q, K, V, dO.  It holds none of the attention
arithmetic and none of the tile classification; both the oracle and the HIP
path consume what it produces.

Column-sparse mask (FlashMask-3 paper summary, abstract): a structured mask is
stored as four vectors over key positions j that hold query-row interval
boundaries.  Following the predicate used throughout this library, element
(i, j) is masked iff ``LTS[j] <= i < LTE[j]`` or ``UTS[j] <= i < UTE[j]``
(half-open intervals; an interval with start >= end is empty).  Bounds are
stored interleaved, ``int32 bounds[B][Hm][Sk][4] = (LTS, LTE, UTS, UTE)``.

Mask families named by the paper summary's abstract (document, prefix-LM,
share-question, sliding-window, block-sparse) are built here; every builder is
checked against a direct definition of its pattern by the tests.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

LTS, LTE, UTS, UTE = 0, 1, 2, 3


# --------------------------------------------------------------------------- #
# bf16 encoding of seeded fp32 draws (round to nearest even)                   #
# --------------------------------------------------------------------------- #
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


_CHUNK = 1 << 22          # elements per independently seeded block of a tensor


def _pool_size() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def draw_bf16_normal(seed_seq: np.random.SeedSequence, shape) -> np.ndarray:
    """bf16 bits of N(0, 1) fp32 draws of the given shape.  The flat tensor is
    cut into blocks of 2^22 elements; block i is drawn by
    default_rng(seed_seq.spawn(n_blocks)[i]) and rounded to bf16 (nearest
    even).  Blocks are independent, so they are filled by a thread pool, and
    the values do not depend on the number of threads."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    n_blocks = max(1, -(-n // _CHUNK))
    children = seed_seq.spawn(n_blocks)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = np.random.default_rng(children[i]).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = bf16_bits(x)

    if n_blocks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=_pool_size()) as ex:
            list(ex.map(fill, range(n_blocks)))
    return out.reshape(shape)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


E4M3_MAX = 448.0


def e4m3_codes(x: np.ndarray):
    """Per-tensor E4M3 encoding of fp32 values for the fp8 forward's inputs:
    descale = max|x| / 448 (1 for an all-zero tensor) and codes = x / descale
    rounded to E4M3 (nearest, ties to even; torch's float8_e4m3fn cast).
    Returns (uint8 codes of x's shape, float32 descale)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    descale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    t = torch.from_numpy(x) / float(descale)
    codes = t.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, descale


def fp8_inputs(tensors):
    """E4M3 Q, K, V (uint8 codes) and their descale factors (float32[3]) from
    the bf16 draws (q, k, v, ...) of a workload."""
    out, ds = [], []
    for x in tensors[:3]:
        c, d = e4m3_codes(bf16_to_f32(x))
        out.append(c)
        ds.append(d)
    return out[0], out[1], out[2], np.array(ds, dtype=np.float32)


# --------------------------------------------------------------------------- #
# seeded structure draws                                                       #
# --------------------------------------------------------------------------- #
def composition(rng: np.random.Generator, total: int, k: int) -> list[int]:
    """k positive lengths summing to ``total`` (uniform random cut points)."""
    if k <= 1:
        return [int(total)]
    cuts = np.sort(rng.choice(np.arange(1, total), size=k - 1, replace=False))
    return [int(x) for x in np.diff(np.concatenate([[0], cuts, [total]]))]


def lognormal_docs(rng: np.random.Generator, total: int, median: float,
                   sigma: float = 1.0, lo: int = 512, hi: int = 65536) -> list[int]:
    """Document lengths drawn log-normally (median ``median``, log-space sigma),
    clipped to [lo, hi], until they cover ``total``; the last one is cut to the
    remainder and merged into its predecessor if that leaves it below ``lo``."""
    lens: list[int] = []
    while sum(lens) < total:
        x = rng.lognormal(math.log(median), sigma)
        lens.append(int(round(float(np.clip(x, lo, hi)))))
    lens[-1] -= sum(lens) - total
    if lens[-1] < lo and len(lens) > 1:
        lens[-2] += lens.pop()
    return lens


def _starts_ends(lens):
    ends = np.cumsum(np.asarray(lens, dtype=np.int64))
    starts = ends - np.asarray(lens, dtype=np.int64)
    return starts, ends


# --------------------------------------------------------------------------- #
# bound builders, one per mask family; each returns int32 [S][4]               #
# --------------------------------------------------------------------------- #
def causal_document_bounds(doc_lens) -> np.ndarray:
    """Causal attention inside each document: row i sees column j iff both are
    in the same document and j <= i.  Rows from the end of j's document on are
    the lower interval, rows above the diagonal the upper interval."""
    S = int(sum(doc_lens))
    starts, ends = _starts_ends(doc_lens)
    j = np.arange(S, dtype=np.int64)
    doc_end = np.repeat(ends, doc_lens)
    b = np.empty((S, 4), dtype=np.int64)
    b[:, LTS], b[:, LTE] = doc_end, S
    b[:, UTS], b[:, UTE] = 0, j
    return b.astype(np.int32)


def sliding_window_bounds(S: int, window: int) -> np.ndarray:
    """Causal sliding window of ``window`` keys including the diagonal: row i
    sees column j iff 0 <= i - j < window."""
    j = np.arange(S, dtype=np.int64)
    b = np.empty((S, 4), dtype=np.int64)
    b[:, LTS], b[:, LTE] = np.minimum(j + window, S), S
    b[:, UTS], b[:, UTE] = 0, j
    return b.astype(np.int32)


def share_question_bounds(question_len: int, answer_lens) -> np.ndarray:
    """A causal question shared by several answers: question rows attend the
    question causally; rows of an answer attend the whole question prefix up to
    themselves (causally) and their own answer causally, never other answers."""
    S = int(question_len + sum(answer_lens))
    j = np.arange(S, dtype=np.int64)
    b = np.empty((S, 4), dtype=np.int64)
    b[:, UTS], b[:, UTE] = 0, j
    b[:question_len, LTS] = S
    b[:question_len, LTE] = S
    starts, ends = _starts_ends(answer_lens)
    b[question_len:, LTS] = np.repeat(ends + question_len, answer_lens)
    b[question_len:, LTE] = S
    return b.astype(np.int32)


def prefix_document_bounds(doc_lens, prefix_frac: float = 0.1) -> np.ndarray:
    """Documents with a bidirectional prefix of floor(frac * length) tokens and
    causal attention after it.  Prefix columns are visible to every row of the
    document; later columns only to rows at or below the diagonal."""
    S = int(sum(doc_lens))
    starts, ends = _starts_ends(doc_lens)
    j = np.arange(S, dtype=np.int64)
    doc_start = np.repeat(starts, doc_lens)
    doc_end = np.repeat(ends, doc_lens)
    plen = np.repeat(np.floor(np.asarray(doc_lens) * prefix_frac).astype(np.int64), doc_lens)
    in_prefix = j < doc_start + plen
    b = np.empty((S, 4), dtype=np.int64)
    b[:, LTS], b[:, LTE] = doc_end, S
    b[:, UTS] = 0
    b[:, UTE] = np.where(in_prefix, doc_start, j)
    return b.astype(np.int32)


def blockwise_causal_bounds(S: int, block: int) -> np.ndarray:
    """Block-sparse (block-causal) pattern: row i sees column j iff
    block(j) <= block(i); rows of earlier blocks form the upper interval."""
    j = np.arange(S, dtype=np.int64)
    b = np.empty((S, 4), dtype=np.int64)
    b[:, LTS], b[:, LTE] = S, S
    b[:, UTS], b[:, UTE] = 0, (j // block) * block
    return b.astype(np.int32)


def document_bounds(doc_lens) -> np.ndarray:
    """Bidirectional attention inside each document: row i sees column j iff
    both are in the same document.  Rows of earlier documents form the upper
    interval, rows of later documents the lower one."""
    S = int(sum(doc_lens))
    starts, ends = _starts_ends(doc_lens)
    b = np.empty((S, 4), dtype=np.int64)
    b[:, LTS], b[:, LTE] = np.repeat(ends, doc_lens), S
    b[:, UTS], b[:, UTE] = 0, np.repeat(starts, doc_lens)
    return b.astype(np.int32)


def global_sliding_bounds(S: int, n_global: int, window: int) -> np.ndarray:
    """Bidirectional sliding window with global tokens: row i sees column j iff
    |i - j| < window, or i < n_global, or j < n_global.  A global column is
    never masked; any other column j is masked on the non-global rows above
    the window, [n_global, j - window + 1), and on the rows below it,
    [j + window, S).  The upper interval starts past row 0 here, unlike the
    other families."""
    j = np.arange(S, dtype=np.int64)
    g = min(max(int(n_global), 0), S)
    glob = j < g
    b = np.empty((S, 4), dtype=np.int64)
    b[:, LTS] = np.where(glob, S, np.minimum(j + window, S))
    b[:, LTE] = S
    b[:, UTS] = np.where(glob, 0, g)
    b[:, UTE] = np.where(glob, 0, np.maximum(j - window + 1, g))
    return b.astype(np.int32)


def eviction_bounds(evict_row) -> np.ndarray:
    """Causal attention in which key j is evicted from row evict_row[j] on:
    row i sees column j iff j <= i < evict_row[j] (evict_row[j] >= j + 1 keeps
    the diagonal; evict_row[j] = S never evicts)."""
    e = np.asarray(evict_row, dtype=np.int64)
    S = e.shape[0]
    j = np.arange(S, dtype=np.int64)
    if S and (e < j + 1).any():
        raise ValueError("eviction row must come after the key's own row")
    b = np.empty((S, 4), dtype=np.int64)
    b[:, LTS], b[:, LTE] = np.minimum(e, S), S
    b[:, UTS], b[:, UTE] = 0, j
    return b.astype(np.int32)


def random_eviction_rows(rng: np.random.Generator, S: int) -> np.ndarray:
    """Eviction row of each key drawn uniformly from [j + 1, S]."""
    j = np.arange(S, dtype=np.int64)
    return j + 1 + np.floor(rng.random(S) * (S - j)).astype(np.int64)


def empty_bounds(Sk: int, Sq: int) -> np.ndarray:
    """No element masked (both intervals empty)."""
    b = np.empty((Sk, 4), dtype=np.int32)
    b[:, LTS], b[:, LTE], b[:, UTS], b[:, UTE] = Sq, Sq, 0, 0
    return b


def localize_bounds(global_bounds: np.ndarray, chunk_starts, chunk_len: int) -> np.ndarray:
    """Context-parallel localisation (FlashMask-3 paper summary, abstract:
    each rank clips, shifts and takes the maximum of the bounds without
    any communication).  A rank holds query chunks
    ``[c0, c0+chunk_len)`` (in the given order, stacked as its local rows).
    A global bound g becomes the number of local rows whose global index is
    below g: for every chunk that starts at or before g take the chunk's local
    offset plus g clipped into the chunk, and keep the maximum (0 if none).
    The chunks must be listed in increasing global order, so that local row
    order follows global row order; then a local row i is masked exactly when
    its global row is."""
    g = global_bounds.astype(np.int64)
    out = np.zeros_like(g)
    for ci, c0 in enumerate(chunk_starts):
        shifted = ci * chunk_len + np.clip(g - c0, 0, chunk_len)
        out = np.where(g >= c0, np.maximum(out, shifted), out)
    return out.astype(np.int32)


# --------------------------------------------------------------------------- #
# workloads                                                                    #
# --------------------------------------------------------------------------- #
@dataclass
class Workload:
    name: str
    B: int
    H: int
    Hm: int
    Sq: int
    Sk: int
    D: int
    bounds: np.ndarray            # int32 [B][Hm][Sk][4]
    seed: int
    structure: dict = field(default_factory=dict)
    # how the tensors are drawn: (rows of Q drawn, slice of drawn Q rows used)
    q_rows_drawn: int | None = None
    q_row_index: np.ndarray | None = None
    tensor_seed: int = 0          # entropy of the tensors' SeedSequence

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def draw(self):
        """Return bf16 bit arrays (uint16) q[B][H][Sq][D], k, v [B][H][Sk][D],
        do[B][H][Sq][D].  The four tensors are drawn from four children of one
        SeedSequence whose entropy is the next draw of the workload's own
        generator after the structure (see draw_bf16_normal)."""
        B, H, D = self.B, self.H, self.D
        qr = self.q_rows_drawn or self.Sq
        sq, sk, sv, sdo = np.random.SeedSequence(self.tensor_seed).spawn(4)
        q = draw_bf16_normal(sq, (B, H, qr, D))
        if self.q_row_index is not None:
            q = np.ascontiguousarray(q[:, :, self.q_row_index, :])
        k = draw_bf16_normal(sk, (B, H, self.Sk, D))
        v = draw_bf16_normal(sv, (B, H, self.Sk, D))
        do = draw_bf16_normal(sdo, (B, H, self.Sq, D))
        return q, k, v, do

    def nnz_per_head(self) -> np.ndarray:
        """Unmasked (i, j) count per (b, hm), from the interval lengths (the
        union of two half-open intervals clipped to [0, Sq))."""
        b = self.bounds.astype(np.int64)
        lo1, hi1 = np.clip(b[..., LTS], 0, self.Sq), np.clip(b[..., LTE], 0, self.Sq)
        lo2, hi2 = np.clip(b[..., UTS], 0, self.Sq), np.clip(b[..., UTE], 0, self.Sq)
        l1 = np.maximum(hi1 - lo1, 0)
        l2 = np.maximum(hi2 - lo2, 0)
        ov = np.maximum(np.minimum(hi1, hi2) - np.maximum(lo1, lo2), 0)
        ov = np.where((l1 > 0) & (l2 > 0), ov, 0)
        masked = l1 + l2 - ov
        return (self.Sq - masked).sum(axis=-1)

    def nnz_total(self) -> int:
        per = self.nnz_per_head()                 # [B][Hm]
        mult = self.H // self.Hm
        return int(per.sum()) * mult

    def flops(self) -> tuple[float, float]:
        """Mask-effective flops (forward 4*D*nnz, backward 10*D*nnz)."""
        nnz = self.nnz_total()
        return 4.0 * self.D * nnz, 10.0 * self.D * nnz


def _finish(name, rng, B, H, Sq, Sk, D, bounds_2d, seed, structure, **kw) -> Workload:
    bounds = np.ascontiguousarray(
        np.broadcast_to(bounds_2d[None, None], (B, 1, Sk, 4))).astype(np.int32)
    return Workload(name=name, B=B, H=H, Hm=1, Sq=Sq, Sk=Sk, D=D, bounds=bounds,
                    seed=seed, structure=structure,
                    tensor_seed=int(rng.integers(0, 2**63)), **kw)


def causal_document(B=1, H=2, S=1024, D=64, n_docs=4, seed=1) -> Workload:
    rng = np.random.default_rng(seed)
    docs = composition(rng, S, n_docs)
    return _finish("causal_document", rng, B, H, S, S, D,
                   causal_document_bounds(docs), seed, {"docs": docs})


def sliding_window(B=2, H=16, S=8192, D=128, window=1024, seed=2) -> Workload:
    rng = np.random.default_rng(seed)
    return _finish("sliding_window", rng, B, H, S, S, D,
                   sliding_window_bounds(S, window), seed, {"window": window})


def share_question(B=1, H=16, S=32768, D=128, question=4096, n_answers=8, seed=3) -> Workload:
    rng = np.random.default_rng(seed)
    answers = composition(rng, S - question, n_answers)
    return _finish("share_question", rng, B, H, S, S, D,
                   share_question_bounds(question, answers), seed,
                   {"question": question, "answers": answers})


def prefix_document(B=1, H=8, S=131072, D=128, median=8192, seed=4,
                    lo=512, hi=65536, prefix_frac=0.1) -> Workload:
    rng = np.random.default_rng(seed)
    docs = lognormal_docs(rng, S, median, 1.0, lo, hi)
    return _finish("prefix_document", rng, B, H, S, S, D,
                   prefix_document_bounds(docs, prefix_frac), seed,
                   {"docs": docs, "prefix_frac": prefix_frac})


def cp_rank_share(H=16, S=65536, D=128, median=4096, world=8, rank=3, seed=5,
                  lo=512, hi=65536) -> Workload:
    """One context-parallel rank's share under the two-chunks-per-rank layout:
    the sequence is cut into 2*world chunks, rank r holds chunks r and
    2*world-1-r as its local query rows and attends all S keys through the
    localised bounds."""
    rng = np.random.default_rng(seed)
    docs = lognormal_docs(rng, S, median, 1.0, lo, hi)
    gb = causal_document_bounds(docs)
    n_chunks = 2 * world
    C = S // n_chunks
    chunks = [rank, n_chunks - 1 - rank]
    starts = [c * C for c in chunks]
    lb = localize_bounds(gb, starts, C)
    rows = np.concatenate([np.arange(s, s + C) for s in starts])
    w = _finish("cp_rank_share", rng, 1, H, 2 * C, S, D, lb, seed,
                {"docs": docs, "world": world, "rank": rank, "chunks": chunks,
                 "chunk_len": C, "global_rows": rows},
                q_rows_drawn=S, q_row_index=rows)
    w.structure["global_bounds"] = gb
    return w


def block_causal(B=1, H=4, S=4096, D=128, block=512, seed=6) -> Workload:
    rng = np.random.default_rng(seed)
    return _finish("block_causal", rng, B, H, S, S, D,
                   blockwise_causal_bounds(S, block), seed, {"block": block})


def document(B=1, H=4, S=4096, D=128, n_docs=6, seed=7) -> Workload:
    rng = np.random.default_rng(seed)
    lens = composition(rng, S, n_docs)
    return _finish("document", rng, B, H, S, S, D, document_bounds(lens), seed,
                   {"doc_lens": lens})


def global_sliding(B=1, H=4, S=4096, D=128, n_global=64, window=512, seed=8) -> Workload:
    rng = np.random.default_rng(seed)
    return _finish("global_sliding", rng, B, H, S, S, D,
                   global_sliding_bounds(S, n_global, window), seed,
                   {"n_global": n_global, "window": window})


def random_eviction(B=1, H=4, S=4096, D=128, seed=10) -> Workload:
    rng = np.random.default_rng(seed)
    rows = random_eviction_rows(rng, S)
    return _finish("random_eviction", rng, B, H, S, S, D, eviction_bounds(rows), seed,
                   {"evict_row": rows})


CONFIGS = {
    1: causal_document,
    2: sliding_window,
    3: share_question,
    4: prefix_document,
    5: cp_rank_share,
}

CONFIG_NAMES = {
    1: "causal_document B1 H2 S1024 D64",
    2: "sliding_window w1024 B2 H16 S8192 D128",
    3: "share_question q4096 a8 B1 H16 S32768 D128",
    4: "prefix_document lognormal(8192) B1 H8 S131072 D128",
    5: "cp_rank_share r3/8 Sq8192 Sk65536 H16 D128",
}


def config(k: int, seed: int | None = None) -> Workload:
    """The five evaluation workloads at full size; default seed = k."""
    return CONFIGS[k](seed=k if seed is None else seed)


def custom(bounds_2d: np.ndarray, B: int, H: int, Sq: int, D: int, seed: int,
           name: str = "custom", Hm: int = 1, per_head_bounds: np.ndarray | None = None) -> Workload:
    """Workload from explicit bounds ([Sk][4], or [B][Hm][Sk][4] via
    ``per_head_bounds``); tensors drawn from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    if per_head_bounds is not None:
        bounds = np.ascontiguousarray(per_head_bounds, dtype=np.int32)
        Sk = bounds.shape[2]
        Hm = bounds.shape[1]
    else:
        Sk = bounds_2d.shape[0]
        bounds = np.ascontiguousarray(
            np.broadcast_to(bounds_2d[None, None], (B, Hm, Sk, 4))).astype(np.int32)
    return Workload(name=name, B=B, H=H, Hm=Hm, Sq=Sq, Sk=Sk, D=D, bounds=bounds,
                    seed=seed, tensor_seed=int(rng.integers(0, 2**63)))
