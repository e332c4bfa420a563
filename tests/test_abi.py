"""The C ABI on the host (no GPU): exported symbols, argument checks, layout.

Only calls that fail validation (which returns before any HIP call) or that
are host-only queries are made here."""
import ctypes
import os
import re

import pytest

from column_sparse_masked_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = _declared_functions()
    assert {"fm_tile_bounds", "fm_attn_fwd", "fm_attn_bwd"} <= set(names)
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_sizes_match_header():
    assert ctypes.sizeof(L.Problem) == 32
    assert ctypes.sizeof(L.TileinfoLayout) == 16 + 15 * 8


def _p(**kw):
    base = dict(batch=1, heads=2, mask_heads=1, seqlen_q=300, seqlen_k=500, head_dim=128, softmax_scale=0.1)
    base.update(kw)
    return L.problem(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), L.FM_ERR_SHAPE),
    (dict(heads=0), L.FM_ERR_SHAPE),
    (dict(seqlen_q=-5), L.FM_ERR_SHAPE),
    (dict(seqlen_k=-1), L.FM_ERR_SHAPE),
    (dict(seqlen_q=32768 * 128 + 1), L.FM_ERR_SHAPE),
    (dict(head_dim=96), L.FM_ERR_UNSUPPORTED),
    (dict(head_dim=256), L.FM_ERR_UNSUPPORTED),
    (dict(mask_heads=3, heads=4), L.FM_ERR_UNSUPPORTED),
    (dict(softmax_scale=0.0), L.FM_ERR_UNSUPPORTED),
    (dict(softmax_scale=-1.0), L.FM_ERR_UNSUPPORTED),
    (dict(softmax_scale=float("nan")), L.FM_ERR_UNSUPPORTED),
    (dict(softmax_scale=float("inf")), L.FM_ERR_UNSUPPORTED),
    (dict(batch=65536, heads=1024, seqlen_q=4096), L.FM_ERR_SHAPE),
    (dict(fwd_rows=64), L.FM_ERR_UNSUPPORTED),
    (dict(fwd_rows=-1), L.FM_ERR_UNSUPPORTED),
    (dict(fwd_rows=256, head_dim=64), L.FM_ERR_UNSUPPORTED),
])
def test_bad_problems_rejected_everywhere(kw, code):
    p = _p(**kw)
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    assert L.lib.fm_tile_shape(ctypes.byref(p), ctypes.byref(bq), ctypes.byref(bk)) == code
    lay = L.TileinfoLayout()
    assert L.lib.fm_tileinfo_layout_query(ctypes.byref(p), ctypes.byref(lay)) == code
    n = ctypes.c_size_t()
    assert L.lib.fm_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == code
    fake = ctypes.c_void_p(1 << 20)
    assert L.lib.fm_tile_bounds(ctypes.byref(p), fake, fake, None) == code
    assert L.lib.fm_attn_fwd(ctypes.byref(p), *([fake] * 7), None) == code
    assert L.lib.fm_attn_bwd(ctypes.byref(p), *([fake] * 12), 1 << 20, None) == code


def test_null_problem_and_outputs():
    assert L.lib.fm_tile_shape(None, None, None) == L.FM_ERR_NULL
    p = _p()
    assert L.lib.fm_tile_shape(ctypes.byref(p), None, None) == L.FM_ERR_NULL
    assert L.lib.fm_tileinfo_layout_query(ctypes.byref(p), None) == L.FM_ERR_NULL
    assert L.lib.fm_bwd_workspace_bytes(ctypes.byref(p), None) == L.FM_ERR_NULL
    assert L.lib.fm_device_cu_count(None) == L.FM_ERR_NULL


def test_null_tensors_rejected_before_launch():
    p = _p()
    ok = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced: validation fails first
    assert L.lib.fm_tile_bounds(ctypes.byref(p), ok, None, None) == L.FM_ERR_NULL
    assert L.lib.fm_tile_bounds(ctypes.byref(p), None, ok, None) == L.FM_ERR_NULL
    args = [ok] * 7
    for i in range(7):
        a = list(args)
        a[i] = None
        assert L.lib.fm_attn_fwd(ctypes.byref(p), *a, None) == L.FM_ERR_NULL, i
    args = [ok] * 12
    for i in range(12):
        a = list(args)
        a[i] = None
        assert L.lib.fm_attn_bwd(ctypes.byref(p), *a, 1 << 20, None) == L.FM_ERR_NULL, i


def test_misaligned_tensors_rejected_before_launch():
    p = _p()
    ok = ctypes.c_void_p(1 << 20)
    bad = ctypes.c_void_p((1 << 20) + 8)
    assert L.lib.fm_tile_bounds(ctypes.byref(p), ok, bad, None) == L.FM_ERR_ALIGN   # tileinfo needs 256
    assert L.lib.fm_tile_bounds(ctypes.byref(p), bad, ok, None) == L.FM_ERR_ALIGN   # bounds need 16
    for i in range(7):
        a = [ok] * 7
        a[i] = bad
        want = L.FM_OK if i == 6 else L.FM_ERR_ALIGN   # lse only needs 4-byte alignment
        if want == L.FM_OK:
            continue
        assert L.lib.fm_attn_fwd(ctypes.byref(p), *a, None) == want, i
    for i in range(12):
        a = [ok] * 12
        a[i] = bad
        if i == 5:     # lse
            continue
        assert L.lib.fm_attn_bwd(ctypes.byref(p), *a, 1 << 20, None) == L.FM_ERR_ALIGN, i


def test_backward_workspace_smaller_than_delta_rejected():
    """fm_attn_bwd's workspace must hold Delta (B*H*Sq fp32 values); a
    smaller one is refused before any HIP call instead of being overrun."""
    p = _p()                              # 1 x 2 x 300 rows: 2400 bytes of Delta
    ok = ctypes.c_void_p(1 << 20)
    for nbytes in (0, 16, 2396):
        assert L.lib.fm_attn_bwd(ctypes.byref(p), *([ok] * 12), nbytes, None) == L.FM_ERR_SHAPE, nbytes


def test_status_strings():
    for c in range(7):
        s = L.status_str(c)
        assert s.startswith("FM_")
    assert L.status_str(99) == "unknown fm_status"


@pytest.mark.parametrize("B,H,Hm,Sq,Sk", [(1, 2, 1, 1024, 1024), (2, 3, 3, 300, 517),
                                          (1, 16, 1, 8192, 65536), (1, 1, 1, 1, 1), (0, 1, 1, 5, 5),
                                          (1, 4, 1, 0, 100), (1, 4, 4, 100, 0)])
def test_tileinfo_layout(B, H, Hm, Sq, Sk):
    p = _p(batch=B, heads=H, mask_heads=Hm, seqlen_q=Sq, seqlen_k=Sk)
    lay = L.tileinfo_layout(p)
    nQ, nK = -(-Sq // 128), -(-Sk // 128)
    assert (lay.block_q, lay.block_k, lay.n_qblocks, lay.n_kblocks) == (128, 128, nQ, nK)
    parts = [("counters", 64), ("kbsum", B * Hm * nK * 32), ("cls", B * Hm * nQ * nK),
             ("cnt_q", B * Hm * nQ * 4), ("cnt_k", B * Hm * nK * 4),
             ("list_q", B * Hm * nQ * nK * 2), ("list_k", B * Hm * nK * nQ * 2),
             ("fwd_queue", B * H * nQ * 4), ("bwd_queue", B * H * nK * 4),
             # two partial-result slots (bf16 O, fp32 LSE of 128 rows) per forward
             # item that may be split, at most 512 of them
             ("fwd_partials", 2 * min(B * H * nQ, 512) * 128 * (128 * 2 + 4)),
             ("cpos", B * Hm * nK * nQ * 2), ("colbase", B * H * nK * 4)]
    end = 0
    for name, size in parts:
        off = getattr(lay, name)
        assert off % 256 == 0 and off >= end, name
        end = off + size
    assert lay.total >= end
    ws = L.bwd_workspace_bytes(p)
    assert ws >= B * H * Sq * 4   # Delta of every row
    # the tile cache follows Delta at a 256-byte boundary, 32 KiB per tile
    assert L.bwd_cache_bytes(p, 0) == ws
    assert L.bwd_cache_bytes(p, 37) == ws + 37 * 128 * 128 * 2


def test_fp8_forward_validation():
    """fm_attn_fwd_fp8 rejects head_dim 64, a missing or bad descale, null and
    misaligned tensors before any launch."""
    fake = ctypes.c_void_p(1 << 20)
    ds = (ctypes.c_float * 3)(0.01, 0.02, 0.03)
    p64 = _p(head_dim=64)
    assert L.lib.fm_attn_fwd_fp8(ctypes.byref(p64), fake, fake, fake, ds, fake, fake, fake, fake, None) \
        == L.FM_ERR_UNSUPPORTED
    p = _p()
    assert L.lib.fm_attn_fwd_fp8(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake, None) \
        == L.FM_ERR_NULL
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        for i in range(3):
            d = (ctypes.c_float * 3)(0.01, 0.02, 0.03)
            d[i] = bad
            assert L.lib.fm_attn_fwd_fp8(ctypes.byref(p), fake, fake, fake, d, fake, fake, fake, fake,
                                         None) == L.FM_ERR_UNSUPPORTED, (bad, i)
    tensors = [fake] * 3 + [None] + [fake] * 4   # q k v | descale slot | bounds tileinfo o lse
    for i in (0, 1, 2, 4, 5, 6, 7):
        a = list(tensors)
        a[i] = None
        a[3] = ds
        assert L.lib.fm_attn_fwd_fp8(ctypes.byref(p), *a, None) == L.FM_ERR_NULL, i
    bad = ctypes.c_void_p((1 << 20) + 8)
    for i in (0, 1, 2, 4, 5, 6):
        a = list(tensors)
        a[i] = bad
        a[3] = ds
        assert L.lib.fm_attn_fwd_fp8(ctypes.byref(p), *a, None) == L.FM_ERR_ALIGN, i
    for kw in (dict(batch=-1), dict(heads=0), dict(softmax_scale=0.0)):
        q = _p(**kw)
        assert L.lib.fm_attn_fwd_fp8(ctypes.byref(q), fake, fake, fake, ds, fake, fake, fake, fake, None) \
            != L.FM_OK


def test_fp8_binding_rejects_wrong_tensors():
    """The Python wrapper checks dtype and shape of the code tensors before
    calling the library (CPU tensors: nothing reaches a kernel)."""
    import torch
    from column_sparse_masked_amd.api import MaskedAttention
    att = MaskedAttention.__new__(MaskedAttention)
    att.p = _p(seqlen_q=5, seqlen_k=7)
    att.device = torch.device("cpu")
    ok_q = torch.zeros((1, 2, 5, 128), dtype=torch.uint8)
    ok_k = torch.zeros((1, 2, 7, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        att.forward_fp8(ok_q.to(torch.bfloat16), ok_k, ok_k, (1.0, 1.0, 1.0), None)
    with pytest.raises(ValueError):
        att.forward_fp8(ok_q, ok_k[:, :, :6], ok_k, (1.0, 1.0, 1.0), None)


def _cpu_wrapper(**kw):
    """A MaskedAttention whose buffers are never allocated (CPU tensors:
    whatever the checks let through would fail in the library, not a kernel)."""
    import torch
    from column_sparse_masked_amd.api import MaskedAttention
    att = MaskedAttention.__new__(MaskedAttention)
    att.p = _p(**kw)
    att.device = torch.device("cpu")
    return att


def test_binding_rejects_wrong_bf16_tensors():
    """forward / backward / tile_bounds check dtype, shape, contiguity and
    device of every tensor before the library sees a pointer."""
    import torch
    att = _cpu_wrapper(batch=1, heads=2, mask_heads=1, seqlen_q=5, seqlen_k=7, head_dim=64)
    bf = torch.bfloat16
    q = torch.zeros((1, 2, 5, 64), dtype=bf)
    k = torch.zeros((1, 2, 7, 64), dtype=bf)
    o = torch.zeros_like(q)
    lse = torch.zeros((1, 2, 5), dtype=torch.float32)
    bounds = torch.zeros((1, 1, 7, 4), dtype=torch.int32)
    fwd_ok = dict(q=q, k=k, v=k, bounds=bounds, o=o, lse=lse)
    bad = {
        "q": [q.float(), q[:, :, :4], torch.zeros((1, 2, 64, 5), dtype=bf).transpose(2, 3)],
        "k": [k.to(torch.float16), k[:, :1]],
        "v": [k[:, :, :6], torch.zeros((1, 2, 7, 128), dtype=bf)],
        "bounds": [bounds.to(torch.int64), bounds[:, :, :6], torch.zeros((1, 1, 4, 7), dtype=torch.int32).transpose(2, 3)],
        "o": [o.float(), o[..., :32]],
        "lse": [lse.double(), lse[:, :, :4]],
    }
    for name, variants in bad.items():
        for t in variants:
            args = dict(fwd_ok)
            args[name] = t
            with pytest.raises(ValueError, match=name):
                att.forward(**args)
    bwd_ok = dict(q=q, k=k, v=k, o=o, dout=q, lse=lse, bounds=bounds, dq=torch.zeros_like(q),
                  dk=torch.zeros_like(k), dv=torch.zeros_like(k))
    bad_bwd = {"dout": q[:, :, :3], "dq": q.float(), "dk": k[..., :32], "dv": torch.zeros((1, 2, 8, 64), dtype=bf),
               "lse": lse.half(), "o": o[:, :1]}
    for name, t in bad_bwd.items():
        args = dict(bwd_ok)
        args[name] = t
        with pytest.raises(ValueError, match=name):
            att.backward(**args)
    with pytest.raises(ValueError, match="bounds"):
        att.tile_bounds(bounds[:, :, :5])
    with pytest.raises(ValueError, match="bounds"):
        att.tile_bounds(bounds.numpy())


def test_binding_rejects_tensors_on_another_device():
    import torch
    att = _cpu_wrapper(seqlen_q=5, seqlen_k=7, head_dim=64)
    att.device = torch.device("cuda", 0)   # tensors below live on the CPU
    bounds = torch.zeros((1, 1, 7, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="expected cuda"):
        att.tile_bounds(bounds)


def test_noalloc_backward_validation():
    """fm_attn_bwd_noalloc: problems beyond its static scratch array (more
    than 4194304 query rows over batch and heads) are rejected with
    FM_ERR_SCRATCH, bad problems, null and misaligned tensors as in
    fm_attn_bwd, all before any HIP call."""
    fake = ctypes.c_void_p(1 << 20)
    big = _p(batch=2, heads=16, seqlen_q=131073, seqlen_k=128)
    assert L.lib.fm_attn_bwd_noalloc(ctypes.byref(big), *([fake] * 11), None) == L.FM_ERR_SCRATCH
    assert "static scratch" in L.status_str(L.FM_ERR_SCRATCH)
    for kw, code in ((dict(batch=-1), L.FM_ERR_SHAPE), (dict(head_dim=96), L.FM_ERR_UNSUPPORTED)):
        q = _p(**kw)
        assert L.lib.fm_attn_bwd_noalloc(ctypes.byref(q), *([fake] * 11), None) == code
    p = _p()
    for i in range(11):
        a = [fake] * 11
        a[i] = None
        assert L.lib.fm_attn_bwd_noalloc(ctypes.byref(p), *a, None) == L.FM_ERR_NULL, i
    bad = ctypes.c_void_p((1 << 20) + 8)
    for i in range(11):
        if i == 5:   # lse only needs 4-byte alignment
            continue
        a = [fake] * 11
        a[i] = bad
        assert L.lib.fm_attn_bwd_noalloc(ctypes.byref(p), *a, None) == L.FM_ERR_ALIGN, i


def test_cache_bytes_validation():
    p = _p()
    n = ctypes.c_size_t()
    assert L.lib.fm_bwd_cache_bytes(ctypes.byref(p), ctypes.c_uint64(1), None) == L.FM_ERR_NULL
    assert L.lib.fm_bwd_cache_bytes(ctypes.byref(p), ctypes.c_uint64(1 << 32), ctypes.byref(n)) == L.FM_ERR_SHAPE
    bad = _p(head_dim=96)
    assert L.lib.fm_bwd_cache_bytes(ctypes.byref(bad), ctypes.c_uint64(1), ctypes.byref(n)) == L.FM_ERR_UNSUPPORTED


def test_localize_validation():
    """fm_localize_bounds rejects bad sizes and chunk lists (decreasing,
    overlapping, negative, none, more than 64) before any HIP call."""
    fake = ctypes.c_void_p(1 << 20)
    I = ctypes.c_int32

    def call(B, Hm, Sk, starts, lens, gb=fake, lb=fake):
        n = len(starts)
        s = (I * max(n, 1))(*starts)
        l_ = (I * max(n, 1))(*lens)
        return L.lib.fm_localize_bounds(B, Hm, Sk, gb, n, s, l_, lb, None)

    assert call(1, 1, 8, [5, 0], [2, 2]) == L.FM_ERR_SHAPE      # decreasing
    assert call(1, 1, 8, [0, 3], [5, 1]) == L.FM_ERR_SHAPE      # overlapping
    assert call(1, 1, 8, [-1], [3]) == L.FM_ERR_SHAPE
    assert call(1, 1, 8, [0], [-2]) == L.FM_ERR_SHAPE
    assert call(1, 1, 8, [], []) == L.FM_ERR_SHAPE
    assert call(1, 1, 8, list(range(0, 130, 2)), [1] * 65) == L.FM_ERR_SHAPE
    assert call(-1, 1, 8, [0], [3]) == L.FM_ERR_SHAPE
    assert call(1, 0, 8, [0], [3]) == L.FM_ERR_SHAPE
    assert call(1, 1, 8, [0], [3], gb=None) == L.FM_ERR_NULL
    assert call(1, 1, 8, [0], [3], lb=ctypes.c_void_p((1 << 20) + 4)) == L.FM_ERR_ALIGN
    assert L.lib.fm_localize_bounds(1, 1, 8, fake, 1, None, None, fake, None) == L.FM_ERR_NULL
