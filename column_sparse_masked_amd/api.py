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


class MaskedAttention:
    """One problem shape: owns the tileinfo and backward workspace buffers."""

    def __init__(self, batch, heads, mask_heads, seqlen_q, seqlen_k, head_dim,
                 softmax_scale=None, device="cuda"):
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(head_dim)
        self.p = _lib.problem(batch, heads, mask_heads, seqlen_q, seqlen_k, head_dim, softmax_scale)
        self.device = torch.device(device)
        self.buf = _lib.alloc_buffers(self.p, self.device)
        self.block_q, self.block_k = _lib.tile_shape(self.p)

    @classmethod
    def for_workload(cls, w, device="cuda"):
        return cls(w.B, w.H, w.Hm, w.Sq, w.Sk, w.D, w.scale, device)

    # ---- the three entry points ----
    def tile_bounds(self, bounds, stream=None):
        _lib.fm_tile_bounds(self.p, bounds, self.buf.tileinfo, stream)

    def forward(self, q, k, v, bounds, o=None, lse=None, stream=None):
        p = self.p
        if o is None:
            o = torch.empty((p.batch, p.heads, p.seqlen_q, p.head_dim), dtype=torch.bfloat16,
                            device=self.device)
        if lse is None:
            lse = torch.empty((p.batch, p.heads, p.seqlen_q), dtype=torch.float32, device=self.device)
        _lib.fm_attn_fwd(p, q, k, v, bounds, self.buf.tileinfo, o, lse, stream)
        return o, lse

    def forward_fp8(self, q8, k8, v8, descale, bounds, o=None, lse=None, stream=None):
        """The forward with E4M3 inputs: q8, k8, v8 uint8 code tensors in the
        bf16 tensors' layouts, descale three floats (q, k, v)."""
        p = self.p
        for name, t, rows in (("q8", q8, p.seqlen_q), ("k8", k8, p.seqlen_k), ("v8", v8, p.seqlen_k)):
            if t.dtype != torch.uint8 or not t.is_contiguous() or \
                    tuple(t.shape) != (p.batch, p.heads, rows, p.head_dim):
                raise ValueError(f"{name}: expected contiguous uint8 E4M3 codes of shape "
                                 f"{(p.batch, p.heads, rows, p.head_dim)}, got {t.dtype} {tuple(t.shape)}")
        if o is None:
            o = torch.empty((p.batch, p.heads, p.seqlen_q, p.head_dim), dtype=torch.bfloat16,
                            device=self.device)
        if lse is None:
            lse = torch.empty((p.batch, p.heads, p.seqlen_q), dtype=torch.float32, device=self.device)
        _lib.fm_attn_fwd_fp8(p, q8, k8, v8, descale, bounds, self.buf.tileinfo, o, lse, stream)
        return o, lse

    def backward(self, q, k, v, o, dout, lse, bounds, dq=None, dk=None, dv=None, stream=None):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        _lib.fm_attn_bwd(self.p, q, k, v, o, dout, lse, bounds, self.buf.tileinfo, dq, dk, dv,
                         self.buf.workspace, stream)
        return dq, dk, dv

    # ---- inspection of the tile pass (tests) ----
    def read_tileinfo(self) -> dict:
        p, L = self.p, self.buf.layout
        raw = self.buf.tileinfo.cpu().numpy()
        bhm, bh = p.batch * p.mask_heads, p.batch * p.heads
        nQ, nK = L.n_qblocks, L.n_kblocks

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
            "nQ": nQ, "nK": nK,
        }
