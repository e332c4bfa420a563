"""ctypes binding of libfm (include/fm.h): argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
only turns torch tensors and streams into the pointers and sizes the C ABI
takes, and raises on a non-zero status.  If libfm.so has not been built the
import fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfm.so")

FM_OK, FM_ERR_NULL, FM_ERR_SHAPE, FM_ERR_UNSUPPORTED, FM_ERR_ALIGN, FM_ERR_HIP, FM_ERR_SCRATCH = range(7)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m column_sparse_masked_amd.build`")

# torch ships its own copy of the HIP runtime.  libfm must bind to that same
# copy, or the process holds two runtimes and the streams torch hands over are
# foreign handles to libfm (every launch is then rejected).  Loading torch
# first makes the dynamic loader resolve libfm's runtime dependency to it.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped() -> list[str]:
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process (libfm would not share "
                      f"torch's streams): {_hip_runtimes_mapped()}")


class Problem(ctypes.Structure):
    """fm_problem: sizes of one masked-attention call."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("mask_heads", ctypes.c_int32), ("seqlen_q", ctypes.c_int32),
                ("seqlen_k", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("fwd_rows", ctypes.c_int32)]


class TileinfoLayout(ctypes.Structure):
    """fm_tileinfo_layout: byte offsets of the tile pass's outputs."""
    _fields_ = [("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("n_qblocks", ctypes.c_int32), ("n_kblocks", ctypes.c_int32),
                ("counters", ctypes.c_size_t), ("kbsum", ctypes.c_size_t),
                ("cls", ctypes.c_size_t), ("cnt_q", ctypes.c_size_t),
                ("cnt_k", ctypes.c_size_t), ("list_q", ctypes.c_size_t),
                ("list_k", ctypes.c_size_t), ("fwd_queue", ctypes.c_size_t),
                ("bwd_queue", ctypes.c_size_t), ("fwd_partials", ctypes.c_size_t),
                ("cpos", ctypes.c_size_t), ("colbase", ctypes.c_size_t),
                ("cnt_p", ctypes.c_size_t), ("list_p", ctypes.c_size_t),
                ("total", ctypes.c_size_t)]


_P = ctypes.POINTER(Problem)
_vp = ctypes.c_void_p
lib.fm_status_str.restype = ctypes.c_char_p
lib.fm_status_str.argtypes = [ctypes.c_int]
lib.fm_tile_shape.argtypes = [_P, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
lib.fm_tileinfo_layout_query.argtypes = [_P, ctypes.POINTER(TileinfoLayout)]
lib.fm_bwd_workspace_bytes.argtypes = [_P, ctypes.POINTER(ctypes.c_size_t)]
lib.fm_device_cu_count.argtypes = [ctypes.POINTER(ctypes.c_int32)]
lib.fm_tile_bounds.argtypes = [_P, _vp, _vp, _vp]
lib.fm_attn_fwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
lib.fm_attn_fwd_fp8.argtypes = [_P, _vp, _vp, _vp, ctypes.POINTER(ctypes.c_float), _vp, _vp, _vp, _vp, _vp]
lib.fm_attn_bwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.fm_bwd_cache_bytes.argtypes = [_P, ctypes.c_uint64, ctypes.POINTER(ctypes.c_size_t)]
_i32p = ctypes.POINTER(ctypes.c_int32)
lib.fm_localize_bounds.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int32,
                                   _i32p, _i32p, _vp, _vp]
lib.fm_attn_bwd_noalloc.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
for _f in ("fm_tile_shape", "fm_tileinfo_layout_query", "fm_bwd_workspace_bytes", "fm_bwd_cache_bytes",
           "fm_device_cu_count", "fm_tile_bounds", "fm_attn_fwd", "fm_attn_fwd_fp8", "fm_attn_bwd",
           "fm_attn_bwd_noalloc", "fm_localize_bounds"):
    getattr(lib, _f).restype = ctypes.c_int


class FmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.fm_status_str(status).decode()}")


def _check(status: int, where: str):
    if status != FM_OK:
        raise FmError(status, where)


def status_str(status: int) -> str:
    return lib.fm_status_str(status).decode()


def problem(batch, heads, mask_heads, seqlen_q, seqlen_k, head_dim, softmax_scale, fwd_rows=0) -> Problem:
    return Problem(batch, heads, mask_heads, seqlen_q, seqlen_k, head_dim, softmax_scale, fwd_rows)


def tile_shape(p: Problem) -> tuple[int, int]:
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.fm_tile_shape(ctypes.byref(p), ctypes.byref(bq), ctypes.byref(bk)), "fm_tile_shape")
    return bq.value, bk.value


def tileinfo_layout(p: Problem) -> TileinfoLayout:
    out = TileinfoLayout()
    _check(lib.fm_tileinfo_layout_query(ctypes.byref(p), ctypes.byref(out)), "fm_tileinfo_layout_query")
    return out


def bwd_workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t()
    _check(lib.fm_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)), "fm_bwd_workspace_bytes")
    return n.value


def bwd_cache_bytes(p: Problem, n_tiles: int) -> int:
    n = ctypes.c_size_t()
    _check(lib.fm_bwd_cache_bytes(ctypes.byref(p), ctypes.c_uint64(n_tiles), ctypes.byref(n)),
           "fm_bwd_cache_bytes")
    return n.value


def device_cu_count() -> int:
    n = ctypes.c_int32()
    _check(lib.fm_device_cu_count(ctypes.byref(n)), "fm_device_cu_count")
    return n.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def fm_tile_bounds(p: Problem, bounds, tileinfo, stream=None):
    """bounds: int32 [B][Hm][Sk][4] device tensor; tileinfo: uint8 device tensor
    of tileinfo_layout(p).total bytes (256-byte aligned)."""
    _check(lib.fm_tile_bounds(ctypes.byref(p), _ptr(bounds), _ptr(tileinfo), _stream(stream)),
           "fm_tile_bounds")


def fm_attn_fwd(p: Problem, q, k, v, bounds, tileinfo, o, lse, stream=None):
    _check(lib.fm_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(bounds), _ptr(tileinfo),
                           _ptr(o), _ptr(lse), _stream(stream)), "fm_attn_fwd")


def fm_attn_fwd_fp8(p: Problem, q8, k8, v8, descale, bounds, tileinfo, o, lse, stream=None):
    """q8, k8, v8: uint8 device tensors of E4M3 codes; descale: three host
    floats (q, k, v)."""
    ds = (ctypes.c_float * 3)(*[float(x) for x in descale])
    _check(lib.fm_attn_fwd_fp8(ctypes.byref(p), _ptr(q8), _ptr(k8), _ptr(v8), ds, _ptr(bounds),
                               _ptr(tileinfo), _ptr(o), _ptr(lse), _stream(stream)), "fm_attn_fwd_fp8")


def fm_attn_bwd(p: Problem, q, k, v, o, dout, lse, bounds, tileinfo, dq, dk, dv, workspace,
                stream=None):
    """workspace: a uint8 device tensor of at least bwd_workspace_bytes(p)
    bytes; its whole size is passed (room beyond Delta is the tile cache)."""
    _check(lib.fm_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                           _ptr(bounds), _ptr(tileinfo), _ptr(dq), _ptr(dk), _ptr(dv),
                           _ptr(workspace), ctypes.c_size_t(0 if workspace is None else workspace.numel()),
                           _stream(stream)), "fm_attn_bwd")


def fm_attn_bwd_noalloc(p: Problem, q, k, v, o, dout, lse, bounds, tileinfo, dq, dk, dv, stream=None):
    """fm_attn_bwd with the library's static scratch array in place of a
    workspace (for callers that cannot allocate)."""
    _check(lib.fm_attn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                   _ptr(lse), _ptr(bounds), _ptr(tileinfo), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _stream(stream)), "fm_attn_bwd_noalloc")


def fm_localize_bounds(global_bounds, chunk_start, chunk_len, local_bounds, stream=None):
    """global_bounds, local_bounds: int32 [B][Hm][Sk][4] device tensors;
    chunk_start, chunk_len: the rank's query chunks (host sequences)."""
    B, Hm, Sk, _ = global_bounds.shape
    n = len(chunk_start)
    starts = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in chunk_start])
    lens = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in chunk_len])
    _check(lib.fm_localize_bounds(B, Hm, Sk, _ptr(global_bounds), n, starts, lens, _ptr(local_bounds),
                                  _stream(stream)), "fm_localize_bounds")


@dataclass
class Buffers:
    """Device buffers the library needs besides the tensors themselves."""
    tileinfo: object
    workspace: object
    layout: TileinfoLayout


def alloc_buffers(p: Problem, device) -> Buffers:
    """tileinfo and backward workspace, allocated with torch (the library
    allocates nothing).  torch's caching allocator returns 512-byte aligned
    blocks, which satisfies the 256-byte alignment of tileinfo."""
    import torch
    L = tileinfo_layout(p)
    ti = torch.empty(max(int(L.total), 256), dtype=torch.uint8, device=device)
    ws = torch.empty(max(bwd_workspace_bytes(p), 256), dtype=torch.uint8, device=device)
    assert ti.data_ptr() % 256 == 0 and ws.data_ptr() % 16 == 0
    return Buffers(ti, ws, L)


lib.fm_set_kernel_events.argtypes = [_vp, _vp, _vp, _vp]
lib.fm_set_kernel_events.restype = ctypes.c_int


def set_kernel_events(begin, end, begin2=None, end2=None):
    """Record the torch.cuda.Event pair ``begin``/``end`` around the main
    attention kernel of the following fm_attn_fwd / fm_attn_bwd calls on this
    thread (the forward kernel; the backward's dK/dV kernel) and
    ``begin2``/``end2`` around the backward's dQ kernel; all ``None`` turns it
    off.  The events must already exist on the device (torch creates them at
    their first record)."""
    def ptr(e):
        return None if e is None else ctypes.c_void_p(e.cuda_event)
    _check(lib.fm_set_kernel_events(ptr(begin), ptr(end), ptr(begin2), ptr(end2)),
           "fm_set_kernel_events")
