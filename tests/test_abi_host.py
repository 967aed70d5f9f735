"""The C-ABI library on the host: it loads, exports every declared entry
point, and rejects malformed arguments before touching any GPU state (so these
run without a GPU)."""
import ctypes
import math
import os
import re
import subprocess

import pytest
import torch

from block_sparse_backward_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lazyflash.h")
# The library under test: the in-tree build, or (LF_ABI_TEST_LIB) a build of
# the same sources whose host code runs under AddressSanitizer and UBSan
# (tests/test_abi_sanitized.py).
LIB = os.environ.get("LF_ABI_TEST_LIB", bd.LIB_PATH)


@pytest.fixture(autouse=True)
def _library_under_test():
    bd.load(LIB)  # the first load fixes the library every later call uses


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lf_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = bd.load(LIB)
    names = declared_functions()
    assert set(names) == set(bd.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lf_[a-z_0-9]+)$", out, flags=re.M))
    assert set(names) <= exported


def test_abi_version_and_status_names():
    lib = bd.load(LIB)
    assert lib.lf_abi_version() == bd.ABI_VERSION
    assert lib.lf_status_str(0) == b"LF_OK"
    assert lib.lf_status_str(1) == b"LF_EINVAL"
    assert lib.lf_status_str(2) == b"LF_EUNSUPPORTED"
    assert lib.lf_status_str(3) == b"LF_EHIP"
    assert lib.lf_status_str(99) == b"unknown lf_status"


def _shape(**kw):
    base = dict(batch=1, heads_q=4, heads_kv=2, seqlen=256, head_dim=128, block=128, causal=1,
                scale=128 ** -0.5, dtype=bd.LF_BF16)
    base.update(kw)
    return bd.LfShape(**base)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
NULL = ctypes.c_void_p(0)


def _fwd(lib, shp, ptr=FAKE):
    return lib.lf_attn_fwd(ctypes.byref(shp) if shp is not None else None, ptr, ptr, ptr, ptr,
                           ptr, NULL)


def _sel(lib, shp, delta, ptr=FAKE):
    return lib.lf_block_select(ctypes.byref(shp), ptr, ptr, delta, 0, ptr, ptr, ptr, ptr, ptr,
                               ptr, NULL)


BIG = 1 << 40  # workspace bytes larger than any requirement


def _bwd(lib, shp, ptr=FAKE, ws=FAKE, ws_bytes=BIG):
    return lib.lf_attn_bwd(ctypes.byref(shp), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                           ptr, ptr, ws, ws_bytes, NULL)


def _ws_size(lib, shp):
    n = ctypes.c_size_t(12345)
    st = lib.lf_bwd_workspace_size(ctypes.byref(shp), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3, heads_kv=2), bd.LF_EINVAL),
    (dict(heads_kv=0), bd.LF_EINVAL),
    (dict(batch=-1), bd.LF_EINVAL),
    (dict(dtype=7), bd.LF_EINVAL),
    (dict(scale=math.inf), bd.LF_EINVAL),
    (dict(scale=math.nan), bd.LF_EINVAL),
    (dict(head_dim=96), bd.LF_EUNSUPPORTED),
    (dict(block=32), bd.LF_EUNSUPPORTED),
    (dict(seqlen=128 * 4096 + 1), bd.LF_EUNSUPPORTED),   # 4097 blocks, the last partial
    (dict(seqlen=128 * 4097), bd.LF_EUNSUPPORTED),
    (dict(seqlen=2**31 - 1), bd.LF_EUNSUPPORTED),        # block count in 64 bits
])
def test_bad_shapes_rejected_by_every_entry_point(kw, status):
    lib = bd.load(LIB)
    shp = _shape(**kw)
    assert _fwd(lib, shp) == status
    assert lib.lf_last_error() != b""
    assert _sel(lib, shp, 0.1) == status
    assert _bwd(lib, shp) == status
    assert _ws_size(lib, shp)[0] == status


def test_null_shape_and_null_pointers():
    lib = bd.load(LIB)
    assert lib.lf_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == bd.LF_EINVAL
    assert _fwd(lib, _shape(), ptr=NULL) == bd.LF_EINVAL
    assert b"NULL" in lib.lf_last_error()
    assert _sel(lib, _shape(), 0.1, ptr=NULL) == bd.LF_EINVAL
    assert _bwd(lib, _shape(), ptr=NULL) == bd.LF_EINVAL


@pytest.mark.parametrize("delta", [-0.01, 1.0, 2.0, math.nan, math.inf])
def test_select_rejects_bad_delta(delta):
    lib = bd.load(LIB)
    assert _sel(lib, _shape(), delta) == bd.LF_EINVAL
    assert b"delta" in lib.lf_last_error()


def test_empty_problems_are_noops():
    lib = bd.load(LIB)
    for kw in (dict(batch=0), dict(seqlen=0)):
        shp = _shape(**kw)
        assert _fwd(lib, shp, ptr=NULL) == bd.LF_OK
        assert _sel(lib, shp, 0.1, ptr=NULL) == bd.LF_OK
        assert _bwd(lib, shp, ptr=NULL) == bd.LF_OK
    # delta is still checked on an empty problem
    assert _sel(lib, _shape(batch=0), 1.5, ptr=NULL) == bd.LF_EINVAL


def test_binding_rejects_unsupported_dtype():
    import torch
    with pytest.raises(bd.LazyFlashError):
        bd.make_shape(1, 1, 1, 64, 64, 64, True, 0.1, torch.float16)


def test_bwd_phase_mask_checked():
    lib = bd.load(LIB)
    shp = _shape()

    def call(mask, dq=FAKE, dk=FAKE, dv=FAKE):
        return lib.lf_attn_bwd_phases(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, dq, dk, dv, FAKE, BIG, mask, NULL)
    assert call(0) == bd.LF_EINVAL
    assert call(4) == bd.LF_EINVAL
    assert b"phase" in lib.lf_last_error()
    # each half checks only its own outputs
    assert call(bd.BWD_DKDV, dk=NULL) == bd.LF_EINVAL
    assert call(bd.BWD_DQ, dq=NULL) == bd.LF_EINVAL
    assert b"NULL" in lib.lf_last_error()


def test_workspace_size_and_checks():
    lib = bd.load(LIB)
    # bf16: fp32 partial tiles of 1536 blocks plus the item and block tables
    shp = _shape(batch=2, heads_q=4, heads_kv=2, seqlen=1024, head_dim=128, block=128)
    st, n = _ws_size(lib, shp)
    nblocks = 2 * 4 * 1024 // 128
    assert st == bd.LF_OK
    assert 1536 * 128 * 128 * 4 <= n <= 1536 * 128 * 128 * 4 + 30 * nblocks + 29 * 1024
    # grows with the number of blocks once they exceed the partial slots
    st2, n2 = _ws_size(lib, _shape(batch=64, heads_q=32, heads_kv=8, seqlen=8192,
                                   head_dim=128, block=128))
    assert st2 == bd.LF_OK and n2 > n
    assert _ws_size(lib, _shape(dtype=bd.LF_F32)) == (bd.LF_OK, 0)
    assert _ws_size(lib, _shape(batch=0)) == (bd.LF_OK, 0)
    assert lib.lf_bwd_workspace_size(ctypes.byref(shp), None) == bd.LF_EINVAL
    # the backward refuses a missing or short workspace before launching anything
    assert _bwd(lib, shp, ws=NULL) == bd.LF_EINVAL
    assert b"workspace" in lib.lf_last_error()
    assert _bwd(lib, shp, ws_bytes=n - 1) == bd.LF_EINVAL
    assert b"workspace" in lib.lf_last_error()


def test_draw_seed_is_distinct_and_bounded():
    from block_sparse_backward_amd.autograd import draw_seed
    seeds = {draw_seed(s, l, b) for b in (0, 5) for s in (0, 1, 2**32 - 1) for l in (0, 1, 2**16 - 1)}
    assert len(seeds) == 18 and all(0 <= s < 2**64 for s in seeds)
    for bad in ((-1, 0, 0), (2**32, 0, 0), (0, 2**16, 0), (0, 0, 2**16)):
        with pytest.raises(ValueError):
            draw_seed(*bad)


def test_wrapper_and_binding_reject_host_tensors():
    # Host pointers never reach the library: the binding checks the device
    # before any call.
    from block_sparse_backward_amd.autograd import lazyflash_attention
    q = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        lazyflash_attention(q, q, q, 0.1, 0, block=64)
    with pytest.raises(ValueError, match="delta"):
        lazyflash_attention(q, q, q, 1.0, 0, block=64)
    with pytest.raises(ValueError, match="delta"):
        lazyflash_attention(q, q, q, float("nan"), 0, block=64)


def test_ragged_seqlen_passes_validation():
    # N not a multiple of the block: the last query block is partial; the shape
    # is valid, so only the NULL tensor pointers are reported
    lib = bd.load(LIB)
    shp = _shape(seqlen=200)
    assert _fwd(lib, shp, ptr=NULL) == bd.LF_EINVAL
    assert b"NULL" in lib.lf_last_error()
    st, n = _ws_size(lib, shp)
    assert st == bd.LF_OK and n > 0


def _varlen(lib, shp, cu, ptr=FAKE):
    arr = (ctypes.c_int32 * len(cu))(*cu) if cu is not None else None
    f = lib.lf_attn_fwd_varlen(ctypes.byref(shp), arr, ptr, ptr, ptr, ptr, ptr, NULL)
    s = lib.lf_block_select_varlen(ctypes.byref(shp), arr, ptr, ptr, 0, 0.1, 0, ptr, ptr, ptr,
                                   ptr, ptr, ptr, NULL)
    b = lib.lf_attn_bwd_varlen(ctypes.byref(shp), arr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                               ptr, ptr, ptr, ptr, ptr, BIG, NULL)
    n = ctypes.c_size_t(7)
    w = lib.lf_bwd_workspace_size_varlen(ctypes.byref(shp), arr, ctypes.byref(n))
    return f, s, b, w, n.value


@pytest.mark.parametrize("cu,status", [
    ([1, 5, 9], bd.LF_EINVAL),                 # must start at 0
    ([0, 300, 200], bd.LF_EINVAL),             # decreasing
    ([0, 300, 300 + 128 * 4096 + 1], bd.LF_EUNSUPPORTED),  # one sequence too long
    ([0, 100, 50, 200], bd.LF_EINVAL),         # decreasing in the middle
    ([0, -5], bd.LF_EINVAL),                   # a negative length
    ([0, 2**31 - 1], bd.LF_EUNSUPPORTED),      # the longest int32 length
    ([0, 64, 2**31 - 1, 2**31 - 1], bd.LF_EUNSUPPORTED),
])
def test_varlen_bad_offsets_rejected_before_any_launch(cu, status):
    lib = bd.load(LIB)
    shp = _shape(batch=len(cu) - 1, seqlen=0)
    f, s, b, w, _ = _varlen(lib, shp, cu)
    assert f == s == b == w == status


def test_varlen_null_offsets_and_pointers():
    lib = bd.load(LIB)
    shp = _shape(batch=2, seqlen=0)
    assert _varlen(lib, shp, None)[:4] == (bd.LF_EINVAL,) * 4
    f, s, b, w, n = _varlen(lib, shp, [0, 100, 356], ptr=NULL)
    assert (f, s, b) == (bd.LF_EINVAL,) * 3
    assert w == bd.LF_OK
    # the workspace of the longest sequence serves every sequence
    one = _shape(batch=1, seqlen=256)
    assert n == _ws_size(lib, one)[1] > 0


def test_varlen_bad_rule_parameter():
    lib = bd.load(LIB)
    shp = _shape(batch=1, seqlen=0)
    arr = (ctypes.c_int32 * 2)(0, 256)
    for rule, param in ((0, 1.0), (1, 0.0), (2, 1.5), (9, 0.5)):
        assert lib.lf_block_select_varlen(ctypes.byref(shp), arr, FAKE, FAKE, rule, param, 0,
                                          FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == bd.LF_EINVAL


def test_varlen_binding_checks_packed_sizes_before_any_call():
    # The C ABI cannot see how long the packed buffers are, so the binding
    # checks every buffer against cu_seqlens first: a cu_seqlens whose total
    # exceeds the tensors is a ValueError (host tensors here: the size check
    # comes before the device check, and nothing reaches the library).
    Hq, Hkv, d, blk = 4, 2, 64, 64
    cu = [0, 100, 356]
    T = cu[-1]
    nb = sum(-(-(b - a) // blk) for a, b in zip(cu, cu[1:]))
    q = torch.zeros(Hq * T * d, dtype=torch.bfloat16)
    kv = torch.zeros(Hkv * T * d, dtype=torch.bfloat16)
    long_cu = [0, 100, 357]
    with pytest.raises(ValueError, match="cu_seqlens"):
        bd.attn_fwd_varlen(q, kv, kv, long_cu, Hq, Hkv, d, block=blk)
    with pytest.raises(ValueError, match="cu_seqlens"):
        bd.block_select_varlen(q, q, long_cu, Hq, d, 0.1, 0, block=blk, heads_kv=Hkv)
    sel = dict(D=torch.zeros(Hq * T), block_w=torch.zeros(Hq * nb),
               kept_idx=torch.zeros(Hq * nb, dtype=torch.int32),
               kept_count=torch.zeros(Hq * 2, dtype=torch.int32))
    lse = torch.zeros(Hq * T)
    with pytest.raises(ValueError, match="cu_seqlens"):
        bd.attn_bwd_varlen(q, kv, kv, lse, q, sel, long_cu, Hq, Hkv, d, block=blk)
    # every per-head and per-block array is checked too
    for key, n in (("D", Hq * T - 1), ("block_w", Hq * nb + 1), ("kept_idx", 3),
                   ("kept_count", Hq * 3)):
        bad = dict(sel)
        bad[key] = torch.zeros(n, dtype=sel[key].dtype)
        with pytest.raises(ValueError, match=key):
            bd.attn_bwd_varlen(q, kv, kv, lse, q, bad, cu, Hq, Hkv, d, block=blk)
    with pytest.raises(ValueError, match="lse"):
        bd.attn_bwd_varlen(q, kv, kv, lse[:-1], q, sel, cu, Hq, Hkv, d, block=blk)
    with pytest.raises(ValueError, match="k holds"):
        bd.attn_bwd_varlen(q, q, kv, lse, q, sel, cu, Hq, Hkv, d, block=blk)
    with pytest.raises(ValueError, match="nondecreasing"):
        bd.attn_fwd_varlen(q, kv, kv, [0, 300, 200], Hq, Hkv, d, block=blk)
    # right sizes: only then does the device check refuse the host tensors
    with pytest.raises(ValueError, match="GPU tensor"):
        bd.attn_bwd_varlen(q, kv, kv, lse, q, sel, cu, Hq, Hkv, d, block=blk)


def test_noalloc_backward_checks_before_any_launch():
    lib = bd.load(LIB)

    def call(shp, ptr=FAKE):
        return lib.lf_attn_bwd_noalloc(ctypes.byref(shp), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                                       ptr, ptr, ptr, ptr, NULL)
    assert call(_shape(heads_q=3)) == bd.LF_EINVAL
    assert call(_shape(head_dim=96)) == bd.LF_EUNSUPPORTED
    assert call(_shape(), ptr=NULL) == bd.LF_EINVAL
    assert call(_shape(batch=0), ptr=NULL) == bd.LF_OK
    # a problem whose workspace exceeds the static scratch (128 MiB): 2**27
    # blocks need 30 bytes each in the dQ tables alone
    big = _shape(batch=512, heads_q=64, heads_kv=8, seqlen=4096 * 128)
    st, need = _ws_size(lib, big)
    assert st == bd.LF_OK and need > 128 << 20
    assert call(big) == bd.LF_EUNSUPPORTED
    assert b"static scratch" in lib.lf_last_error()
    # the headline shape fits
    st, need = _ws_size(lib, _shape(batch=1, heads_q=32, heads_kv=8, seqlen=32768))
    assert st == bd.LF_OK and need <= 128 << 20


@pytest.mark.parametrize("addr", [0x1008, 0x1002])
def test_misaligned_pointers_rejected_before_any_launch(addr):
    # element tensors and the workspace move in 16-byte pieces: a pointer off a
    # 16-byte boundary is refused on the host, whatever else is right
    lib = bd.load(LIB)
    mis = ctypes.c_void_p(addr)
    shp = _shape()
    assert _fwd(lib, shp, ptr=mis) == bd.LF_EINVAL
    assert b"misaligned" in lib.lf_last_error()
    assert _sel(lib, shp, 0.1, ptr=mis) == bd.LF_EINVAL
    assert _bwd(lib, shp, ptr=mis) == bd.LF_EINVAL
    assert _bwd(lib, shp, ws=mis) == bd.LF_EINVAL     # only the workspace is off
    assert b"misaligned" in lib.lf_last_error()
    assert lib.lf_attn_bwd_noalloc(ctypes.byref(shp), mis, mis, mis, mis, mis, mis, mis, mis, mis,
                                   mis, mis, mis, NULL) == bd.LF_EINVAL
    f, s, b, _, _ = _varlen(lib, _shape(batch=2, seqlen=0), [0, 100, 356], ptr=mis)
    assert (f, s, b) == (bd.LF_EINVAL,) * 3
