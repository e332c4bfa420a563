"""torch-facing helpers over the C ABI: allocate outputs, pass pointers, read
back the tile pass's buffers.  No arithmetic of the method happens here; all
of it runs in libfm's kernels."""
from __future__ import annotations

import math

import numpy as np
import torch

from . import _lib


def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 tensor on ``device`` (bit-exact)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_device_u8(codes: np.ndarray, device="cuda") -> torch.Tensor:
    """uint8 codes (E4M3) -> uint8 tensor on ``device``."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(device)


def to_device_bounds(bounds: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bounds, dtype=np.int32)).to(device)


def localize_bounds(global_bounds: torch.Tensor, chunk_start, chunk_len, stream=None) -> torch.Tensor:
    """One context-parallel rank's bounds, computed on the device from the
    global ones (fm_localize_bounds): the rank's query chunks are
    [chunk_start[c], chunk_start[c] + chunk_len[c]), in increasing order."""
    if global_bounds.dtype != torch.int32 or global_bounds.dim() != 4 or global_bounds.shape[-1] != 4 \
            or not global_bounds.is_contiguous():
        raise ValueError("global_bounds: expected a contiguous int32 tensor [B][Hm][Sk][4]")
    if len(chunk_start) != len(chunk_len):
        raise ValueError("chunk_start and chunk_len differ in length")
    out = torch.empty_like(global_bounds)
    _lib.fm_localize_bounds(global_bounds, chunk_start, chunk_len, out, stream)
    return out


class MaskedAttention:
    """One problem shape: owns the tileinfo and backward workspace buffers.

    Every tensor handed to an entry point is checked before the library is
    called: dtype, shape of this problem, contiguity and device.  A tensor
    that is too small, of the wrong type or strided would make the kernels
    read or write outside it, so a mismatch raises ValueError instead."""

    def __init__(self, batch, heads, mask_heads, seqlen_q, seqlen_k, head_dim,
                 softmax_scale=None, device="cuda", fwd_rows=0):
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(head_dim)
        self.p = _lib.problem(batch, heads, mask_heads, seqlen_q, seqlen_k, head_dim, softmax_scale, fwd_rows)
        self.device = torch.device(device)
        self.buf = _lib.alloc_buffers(self.p, self.device)
        self.block_q, self.block_k = _lib.tile_shape(self.p)

    @classmethod
    def for_workload(cls, w, device="cuda", fwd_rows=0):
        return cls(w.B, w.H, w.Hm, w.Sq, w.Sk, w.D, w.scale, device, fwd_rows)

    # ---- argument checks ----
    def _shape(self, kind):
        p = self.p
        return {"q": (p.batch, p.heads, p.seqlen_q, p.head_dim),
                "k": (p.batch, p.heads, p.seqlen_k, p.head_dim),
                "rows": (p.batch, p.heads, p.seqlen_q),
                "bounds": (p.batch, p.mask_heads, p.seqlen_k, 4)}[kind]

    def _check(self, name, t, dtype, kind):
        shape = self._shape(kind)
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
        if t.dtype != dtype or tuple(t.shape) != shape:
            raise ValueError(f"{name}: expected {dtype} of shape {shape}, got {t.dtype} {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous tensor (the kernels ignore strides)")
        same_device = t.device.type == self.device.type and (
            self.device.index is None or t.device.index == self.device.index)
        if not same_device:
            raise ValueError(f"{name}: on {t.device}, expected {self.device}")

    def _check_all(self, specs):
        for name, t, dtype, kind in specs:
            self._check(name, t, dtype, kind)

    # ---- the three entry points ----
    def tile_bounds(self, bounds, stream=None):
        self._check("bounds", bounds, torch.int32, "bounds")
        _lib.fm_tile_bounds(self.p, bounds, self.buf.tileinfo, stream)

    def forward(self, q, k, v, bounds, o=None, lse=None, stream=None):
        p = self.p
        if o is None:
            o = torch.empty(self._shape("q"), dtype=torch.bfloat16, device=self.device)
        if lse is None:
            lse = torch.empty(self._shape("rows"), dtype=torch.float32, device=self.device)
        bf = torch.bfloat16
        self._check_all([("q", q, bf, "q"), ("k", k, bf, "k"), ("v", v, bf, "k"),
                         ("bounds", bounds, torch.int32, "bounds"), ("o", o, bf, "q"),
                         ("lse", lse, torch.float32, "rows")])
        _lib.fm_attn_fwd(p, q, k, v, bounds, self.buf.tileinfo, o, lse, stream)
        return o, lse

    def forward_fp8(self, q8, k8, v8, descale, bounds, o=None, lse=None, stream=None):
        """The forward with E4M3 inputs: q8, k8, v8 uint8 code tensors in the
        bf16 tensors' layouts, descale three floats (q, k, v)."""
        p = self.p
        self._check_all([("q8", q8, torch.uint8, "q"), ("k8", k8, torch.uint8, "k"),
                         ("v8", v8, torch.uint8, "k")])
        if o is None:
            o = torch.empty(self._shape("q"), dtype=torch.bfloat16, device=self.device)
        if lse is None:
            lse = torch.empty(self._shape("rows"), dtype=torch.float32, device=self.device)
        self._check_all([("bounds", bounds, torch.int32, "bounds"), ("o", o, torch.bfloat16, "q"),
                         ("lse", lse, torch.float32, "rows")])
        _lib.fm_attn_fwd_fp8(p, q8, k8, v8, descale, bounds, self.buf.tileinfo, o, lse, stream)
        return o, lse

    def backward(self, q, k, v, o, dout, lse, bounds, dq=None, dk=None, dv=None, stream=None):
        bf = torch.bfloat16
        self._check_all([("q", q, bf, "q"), ("k", k, bf, "k"), ("v", v, bf, "k"), ("o", o, bf, "q"),
                         ("dout", dout, bf, "q"), ("lse", lse, torch.float32, "rows"),
                         ("bounds", bounds, torch.int32, "bounds")])
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        self._check_all([("dq", dq, bf, "q"), ("dk", dk, bf, "k"), ("dv", dv, bf, "k")])
        _lib.fm_attn_bwd(self.p, q, k, v, o, dout, lse, bounds, self.buf.tileinfo, dq, dk, dv,
                         self.buf.workspace, stream)
        return dq, dk, dv

    def tile_count(self) -> int:
        """Non-skipped tiles over every (batch, head) pair, as counted by the
        last tile pass on this object's tileinfo (synchronises the device)."""
        return int(self.buf.tileinfo[:64].cpu().numpy().view(np.uint32)[9])

    def reserve_tile_cache(self, n_tiles=None):
        """Grow the backward workspace to hold the tile cache for n_tiles
        tiles (default: the last tile pass's count), so that the backward
        computes dQ from cached dS / scale instead of recomputing S and dP.
        Returns the workspace size in bytes."""
        n = self.tile_count() if n_tiles is None else int(n_tiles)
        need = _lib.bwd_cache_bytes(self.p, n)
        if self.buf.workspace.numel() < need:
            self.buf.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.buf.workspace.numel()

    def drop_tile_cache(self):
        """Back to the smallest workspace (Delta only): dQ is recomputed."""
        self.buf.workspace = torch.empty(max(_lib.bwd_workspace_bytes(self.p), 256), dtype=torch.uint8,
                                         device=self.device)

    # ---- inspection of the tile pass (tests) ----
    def read_tileinfo(self) -> dict:
        p, L = self.p, self.buf.layout
        raw = self.buf.tileinfo.cpu().numpy()
        bhm, bh = p.batch * p.mask_heads, p.batch * p.heads
        nQ, nK = L.n_qblocks, L.n_kblocks
        # the pair lists exist where pair mode can be chosen (head_dim 128)
        nP = (nQ + 1) // 2 if p.head_dim == 128 and p.fwd_rows != 128 else 0

        def view(off, dtype, shape):
            n = int(np.prod(shape))
            return raw[off:off + n * np.dtype(dtype).itemsize].view(dtype).reshape(shape)

        return {
            "counters": view(L.counters, np.uint32, (16,)),
            "kbsum": view(L.kbsum, np.int32, (p.batch, p.mask_heads, nK, 8)),
            "cls": view(L.cls, np.uint8, (p.batch, p.mask_heads, nQ, nK)),
            "cnt_q": view(L.cnt_q, np.int32, (p.batch, p.mask_heads, nQ)),
            "cnt_k": view(L.cnt_k, np.int32, (p.batch, p.mask_heads, nK)),
            "list_q": view(L.list_q, np.uint16, (bhm, nQ, nK)).reshape(p.batch, p.mask_heads, nQ, nK),
            "list_k": view(L.list_k, np.uint16, (bhm, nK, nQ)).reshape(p.batch, p.mask_heads, nK, nQ),
            "fwd_queue": view(L.fwd_queue, np.uint32, (bh * nQ,)),
            "bwd_queue": view(L.bwd_queue, np.uint32, (bh * nK,)),
            "cpos": view(L.cpos, np.uint16, (bhm, nK, nQ)).reshape(p.batch, p.mask_heads, nK, nQ),
            "colbase": view(L.colbase, np.uint32, (bh * nK,)),
            "cnt_p": view(L.cnt_p, np.int32, (p.batch, p.mask_heads, nP)),
            "list_p": view(L.list_p, np.uint32, (bhm, nP, nK)).reshape(p.batch, p.mask_heads, nP, nK),
            "nQ": nQ, "nK": nK,
        }
