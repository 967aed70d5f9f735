"""ctypes binding of liblazyflash.so (C ABI in include/lazyflash.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch provides device memory (outputs are allocated here as torch
tensors) and the current HIP stream.  The library is
loaded from this package directory; if it is missing the import of any entry
point raises, there is no fallback.
"""
import ctypes
import os

import torch

__all__ = ["LazyFlashError", "LfShape", "load", "make_shape", "attn_fwd", "block_select",
           "select_outputs", "attn_bwd", "bwd_workspace_bytes", "bwd_workspace",
           "EXPORTED_SYMBOLS", "LIB_PATH", "attn_fwd_varlen", "block_select_varlen",
           "attn_bwd_varlen", "varlen_block_offsets", "attn_bwd_noalloc"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblazyflash.so")
ABI_VERSION = 8
LF_OK, LF_EINVAL, LF_EUNSUPPORTED, LF_EHIP = 0, 1, 2, 3
LF_BF16, LF_F32 = 0, 1
EXPORTED_SYMBOLS = ("lf_attn_fwd", "lf_block_select", "lf_block_select_rule", "lf_attn_bwd",
                    "lf_bwd_workspace_size", "lf_attn_fwd_varlen", "lf_block_select_varlen",
                    "lf_bwd_workspace_size_varlen", "lf_attn_bwd_varlen",
                    "lf_attn_bwd_phases", "lf_attn_bwd_noalloc", "lf_status_str",
                    "lf_last_error", "lf_abi_version")
BWD_DKDV, BWD_DQ, BWD_ALL = 1, 2, 3
SELECT_BUDGET, SELECT_FRACTION, SELECT_TOPK = 0, 1, 2


class LazyFlashError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


class LfShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


_lib = None


def load(path=LIB_PATH):
    """Load the shared library once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LazyFlashError(-1, f"{path} is missing: build it with "
                                 "`python -m block_sparse_backward_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, I32, U64, D, Z = (ctypes.c_void_p, ctypes.POINTER(LfShape), ctypes.c_int32,
                            ctypes.c_uint64, ctypes.c_double, ctypes.c_size_t)
    lib.lf_attn_fwd.argtypes = [S, P, P, P, P, P, P]
    lib.lf_attn_fwd.restype = I32
    lib.lf_block_select.argtypes = [S, P, P, D, U64, P, P, P, P, P, P, P]
    lib.lf_block_select.restype = I32
    lib.lf_block_select_rule.argtypes = [S, P, P, I32, D, U64, P, P, P, P, P, P, P]
    lib.lf_block_select_rule.restype = I32
    lib.lf_attn_bwd.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.lf_attn_bwd.restype = I32
    lib.lf_bwd_workspace_size.argtypes = [S, ctypes.POINTER(ctypes.c_size_t)]
    lib.lf_bwd_workspace_size.restype = I32
    lib.lf_attn_bwd_phases.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, Z,
                                       ctypes.c_uint32, P]
    lib.lf_attn_bwd_phases.restype = I32
    lib.lf_attn_bwd_noalloc.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.lf_attn_bwd_noalloc.restype = I32
    CU = ctypes.POINTER(ctypes.c_int32)
    lib.lf_attn_fwd_varlen.argtypes = [S, CU, P, P, P, P, P, P]
    lib.lf_attn_fwd_varlen.restype = I32
    lib.lf_block_select_varlen.argtypes = [S, CU, P, P, I32, D, U64, P, P, P, P, P, P, P]
    lib.lf_block_select_varlen.restype = I32
    lib.lf_bwd_workspace_size_varlen.argtypes = [S, CU, ctypes.POINTER(ctypes.c_size_t)]
    lib.lf_bwd_workspace_size_varlen.restype = I32
    lib.lf_attn_bwd_varlen.argtypes = [S, CU, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.lf_attn_bwd_varlen.restype = I32
    lib.lf_status_str.argtypes = [I32]
    lib.lf_status_str.restype = ctypes.c_char_p
    lib.lf_last_error.argtypes = []
    lib.lf_last_error.restype = ctypes.c_char_p
    lib.lf_abi_version.argtypes = []
    lib.lf_abi_version.restype = I32
    if lib.lf_abi_version() != ABI_VERSION:
        raise LazyFlashError(-1, "liblazyflash.so ABI version mismatch; rebuild it")
    _lib = lib
    return lib


def _check(lib, status):
    if status != LF_OK:
        raise LazyFlashError(status, "%s: %s" % (lib.lf_status_str(status).decode(),
                                                 lib.lf_last_error().decode()))


def make_shape(B, Hq, Hkv, N, d, block, causal, scale, dtype):
    code = {torch.bfloat16: LF_BF16, torch.float32: LF_F32}.get(dtype)
    if code is None:
        raise LazyFlashError(LF_EUNSUPPORTED, f"dtype {dtype} is not supported")
    return LfShape(int(B), int(Hq), int(Hkv), int(N), int(d), int(block), int(bool(causal)),
                   float(scale), code)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (the library takes device pointers), "
                         f"got one on {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape_from(q, k, block, causal, scale):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = d ** -0.5
    return make_shape(B, Hq, Hkv, N, d, block, causal, scale, q.dtype), scale


def attn_fwd(q, k, v, causal=True, scale=None, block=128, out=None):
    """Dense forward: returns (o [B,Hq,N,d] like q, lse [B,Hq,N] float32).
    `out` optionally gives preallocated (o, lse)."""
    lib = load()
    shp, _ = _shape_from(q, k, block, causal, scale)
    dev = q.device
    _need(q, "q", q.shape, q.dtype, dev)
    _need(k, "k", (shp.batch, shp.heads_kv, shp.seqlen, shp.head_dim), q.dtype, dev)
    _need(v, "v", k.shape, q.dtype, dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=dev))
    o, lse = out
    _need(o, "o", q.shape, q.dtype, dev)
    _need(lse, "lse", q.shape[:3], torch.float32, dev)
    _check(lib, lib.lf_attn_fwd(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                _stream(dev)))
    return o, lse


def select_outputs(B, Hq, N, block, device):
    """Preallocated output tensors of block_select."""
    nqb = -(-N // block) if block else 0  # the last block may be partial
    return dict(
        D=torch.empty((B, Hq, N), dtype=torch.float32, device=device),
        mass=torch.empty((B, Hq, nqb), dtype=torch.float64, device=device),
        tau=torch.empty((B, Hq), dtype=torch.float64, device=device),
        block_w=torch.empty((B, Hq, nqb), dtype=torch.float32, device=device),
        kept_idx=torch.empty((B, Hq, nqb), dtype=torch.int32, device=device),
        kept_count=torch.empty((B, Hq), dtype=torch.int32, device=device),
    )


def block_select(o, dout, delta, seed, block=128, causal=True, scale=None, heads_kv=None,
                 out=None, rule=SELECT_BUDGET):
    """Masses, tau, draw and compaction.  Returns a dict of device tensors:
    D [B,Hq,N] f32, mass [B,Hq,nqb] f64, tau [B,Hq] f64, block_w [B,Hq,nqb] f32,
    kept_idx [B,Hq,nqb] i32, kept_count [B,Hq] i32 (`out`: preallocated dict
    from select_outputs).  `rule` picks the selection rule (SELECT_BUDGET:
    `delta` is the budget; SELECT_FRACTION or SELECT_TOPK: `delta` is the
    kept fraction f in (0, 1])."""
    lib = load()
    B, Hq, N, d = o.shape
    shp = make_shape(B, Hq, heads_kv or Hq, N, d, block, causal,
                     d ** -0.5 if scale is None else scale, o.dtype)
    dev = o.device
    _need(o, "o", o.shape, o.dtype, dev)
    _need(dout, "dout", o.shape, o.dtype, dev)
    nqb = -(-N // block) if block else 0  # the last block may be partial
    if out is None:
        out = select_outputs(B, Hq, N, block, dev)
    _need(out["D"], "D", (B, Hq, N), torch.float32, dev)
    _need(out["mass"], "mass", (B, Hq, nqb), torch.float64, dev)
    _need(out["tau"], "tau", (B, Hq), torch.float64, dev)
    _need(out["block_w"], "block_w", (B, Hq, nqb), torch.float32, dev)
    _need(out["kept_idx"], "kept_idx", (B, Hq, nqb), torch.int32, dev)
    _need(out["kept_count"], "kept_count", (B, Hq), torch.int32, dev)
    _check(lib, lib.lf_block_select_rule(ctypes.byref(shp), _ptr(o), _ptr(dout), int(rule),
                                         float(delta), ctypes.c_uint64(int(seed) & (2**64 - 1)),
                                         _ptr(out["D"]), _ptr(out["mass"]), _ptr(out["tau"]),
                                         _ptr(out["block_w"]), _ptr(out["kept_idx"]),
                                         _ptr(out["kept_count"]), _stream(dev)))
    return out


def bwd_workspace_bytes(B, Hq, Hkv, N, d, block, causal, dtype):
    """Device workspace bytes the backward needs for this shape."""
    lib = load()
    shp = make_shape(B, Hq, Hkv, N, d, block, causal, d ** -0.5, dtype)
    n = ctypes.c_size_t(0)
    _check(lib, lib.lf_bwd_workspace_size(ctypes.byref(shp), ctypes.byref(n)))
    return n.value


def bwd_workspace(q, k, block=128, causal=True):
    """A workspace tensor (uint8, on q's device) sized for the backward of q, k."""
    B, Hq, N, d = q.shape
    n = bwd_workspace_bytes(B, Hq, k.shape[1], N, d, block, causal, q.dtype)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def attn_bwd(q, k, v, lse, dout, sel, block=128, causal=True, scale=None, out=None,
             phases=BWD_ALL, workspace=None):
    """Sparse backward over the kept blocks of `sel` (the dict of block_select).
    Returns (dq, dk, dv).  `out` optionally gives preallocated (dq, dk, dv);
    `phases` selects the dK/dV walk, the dQ walk, or both; `workspace`
    optionally gives a preallocated uint8 device tensor (bwd_workspace)."""
    lib = load()
    shp, _ = _shape_from(q, k, block, causal, scale)
    dev = q.device
    B, Hq, N, d = q.shape
    nqb = -(-N // block)
    _need(k, "k", (B, shp.heads_kv, N, d), q.dtype, dev)
    _need(v, "v", k.shape, q.dtype, dev)
    _need(dout, "dout", q.shape, q.dtype, dev)
    _need(lse, "lse", (B, Hq, N), torch.float32, dev)
    _need(sel["D"], "D", (B, Hq, N), torch.float32, dev)
    _need(sel["kept_idx"], "kept_idx", (B, Hq, nqb), torch.int32, dev)
    _need(sel["kept_count"], "kept_count", (B, Hq), torch.int32, dev)
    _need(sel["block_w"], "block_w", (B, Hq, nqb), torch.float32, dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    _need(dq, "dq", q.shape, q.dtype, dev)
    _need(dk, "dk", k.shape, q.dtype, dev)
    _need(dv, "dv", k.shape, q.dtype, dev)
    if workspace is None:
        workspace = bwd_workspace(q, k, block, causal)
    if (not isinstance(workspace, torch.Tensor) or workspace.device != dev
            or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on " + str(dev))
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(sel["D"]),
            _ptr(sel["kept_idx"]), _ptr(sel["kept_count"]), _ptr(sel["block_w"]), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(workspace), ctypes.c_size_t(ws_bytes))
    if phases == BWD_ALL:
        _check(lib, lib.lf_attn_bwd(*args, _stream(dev)))
    else:
        _check(lib, lib.lf_attn_bwd_phases(*args, ctypes.c_uint32(phases), _stream(dev)))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, lse, dout, sel, block=128, causal=True, scale=None, out=None):
    """attn_bwd without a workspace: the library's static device scratch of
    this GPU serves the dQ phase (lf_attn_bwd_noalloc; calls that overlap on
    one GPU race).  Returns (dq, dk, dv); `out` optionally gives them
    preallocated, and then nothing is allocated at all."""
    lib = load()
    shp, _ = _shape_from(q, k, block, causal, scale)
    dev = q.device
    B, Hq, N, d = q.shape
    nqb = -(-N // block)
    _need(k, "k", (B, shp.heads_kv, N, d), q.dtype, dev)
    _need(v, "v", k.shape, q.dtype, dev)
    _need(dout, "dout", q.shape, q.dtype, dev)
    _need(lse, "lse", (B, Hq, N), torch.float32, dev)
    _need(sel["D"], "D", (B, Hq, N), torch.float32, dev)
    _need(sel["kept_idx"], "kept_idx", (B, Hq, nqb), torch.int32, dev)
    _need(sel["kept_count"], "kept_count", (B, Hq), torch.int32, dev)
    _need(sel["block_w"], "block_w", (B, Hq, nqb), torch.float32, dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    _need(dq, "dq", q.shape, q.dtype, dev)
    _need(dk, "dk", k.shape, q.dtype, dev)
    _need(dv, "dv", k.shape, q.dtype, dev)
    _check(lib, lib.lf_attn_bwd_noalloc(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(lse),
                                        _ptr(dout), _ptr(sel["D"]), _ptr(sel["kept_idx"]),
                                        _ptr(sel["kept_count"]), _ptr(sel["block_w"]), _ptr(dq),
                                        _ptr(dk), _ptr(dv), _stream(dev)))
    return dq, dk, dv


# ---------------------------------------------------------------------------
# variable-length batches (layouts in include/lazyflash.h)
# ---------------------------------------------------------------------------
def _cu(cu_seqlens):
    cu = [int(x) for x in cu_seqlens]
    arr = (ctypes.c_int32 * len(cu))(*cu)
    return cu, arr


def varlen_block_offsets(cu_seqlens, block):
    """cb[b] = blocks of the sequences before b (the packed block arrays)."""
    cu = [int(x) for x in cu_seqlens]
    cb = [0]
    for b in range(len(cu) - 1):
        cb.append(cb[-1] + -(-(cu[b + 1] - cu[b]) // block))
    return cb


def _need_packed(items, device):
    """Flat packed buffers of a variable-length batch, as (tensor, name,
    numel, dtype) items: each must hold exactly `numel` elements of `dtype`,
    contiguous, on `device`.  The library cannot see the packed lengths, so a
    short buffer would be read or written past its end: every size is checked
    before anything else."""
    for t, name, numel, _ in items:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.numel() != numel:
            raise ValueError(f"{name} holds {t.numel()} elements; cu_seqlens and the head "
                             f"counts give {numel}")
    for t, name, _, dtype in items:
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != device or t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor on {device}, got one on {t.device}")


def _check_cu(cu, block):
    if len(cu) < 1 or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and be nondecreasing")
    if int(block) < 1:
        raise ValueError("block must be >= 1")


def _varlen_shape(cu, Hq, Hkv, d, block, causal, scale, dtype):
    return make_shape(len(cu) - 1, Hq, Hkv, 0, d, block, causal,
                      d ** -0.5 if scale is None else scale, dtype)


def attn_fwd_varlen(q, k, v, cu_seqlens, heads_q, heads_kv, head_dim, causal=True, scale=None,
                    block=128):
    """Forward over a variable-length batch; q, k, v are flat packed device
    tensors.  Returns (o like q, lse float32 [Hq * total])."""
    lib = load()
    cu, arr = _cu(cu_seqlens)
    shp = _varlen_shape(cu, heads_q, heads_kv, head_dim, block, causal, scale, q.dtype)
    dev = q.device
    _check_cu(cu, block)
    T = cu[-1]
    _need_packed([(q, "q", heads_q * T * head_dim, q.dtype),
                  (k, "k", heads_kv * T * head_dim, q.dtype),
                  (v, "v", heads_kv * T * head_dim, q.dtype)], dev)
    o = torch.empty_like(q)
    lse = torch.empty(heads_q * T, dtype=torch.float32, device=dev)
    _check(lib, lib.lf_attn_fwd_varlen(ctypes.byref(shp), arr, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                       _ptr(lse), _stream(dev)))
    return o, lse


def block_select_varlen(o, dout, cu_seqlens, heads_q, head_dim, delta, seed, block=128,
                        causal=True, scale=None, heads_kv=None, rule=SELECT_BUDGET):
    """Selection over a variable-length batch.  Returns a dict of flat device
    tensors: D [Hq * total], mass / block_w / kept_idx [Hq * total_blocks],
    tau / kept_count [Hq * B]."""
    lib = load()
    cu, arr = _cu(cu_seqlens)
    _check_cu(cu, block)
    cb = varlen_block_offsets(cu, block)
    shp = _varlen_shape(cu, heads_q, heads_kv or heads_q, head_dim, block, causal, scale, o.dtype)
    dev = o.device
    B, nb = len(cu) - 1, cb[-1]
    _need_packed([(o, "o", heads_q * cu[-1] * head_dim, o.dtype),
                  (dout, "dout", heads_q * cu[-1] * head_dim, o.dtype)], dev)
    out = dict(
        D=torch.empty(heads_q * cu[-1], dtype=torch.float32, device=dev),
        mass=torch.empty(heads_q * nb, dtype=torch.float64, device=dev),
        tau=torch.empty(heads_q * B, dtype=torch.float64, device=dev),
        block_w=torch.empty(heads_q * nb, dtype=torch.float32, device=dev),
        kept_idx=torch.empty(heads_q * nb, dtype=torch.int32, device=dev),
        kept_count=torch.empty(heads_q * B, dtype=torch.int32, device=dev),
    )
    _check(lib, lib.lf_block_select_varlen(
        ctypes.byref(shp), arr, _ptr(o), _ptr(dout), int(rule), float(delta),
        ctypes.c_uint64(int(seed) & (2**64 - 1)), _ptr(out["D"]), _ptr(out["mass"]),
        _ptr(out["tau"]), _ptr(out["block_w"]), _ptr(out["kept_idx"]), _ptr(out["kept_count"]),
        _stream(dev)))
    return out


def attn_bwd_varlen(q, k, v, lse, dout, sel, cu_seqlens, heads_q, heads_kv, head_dim, block=128,
                    causal=True, scale=None):
    """Sparse backward over a variable-length batch (`sel` from
    block_select_varlen).  Returns (dq, dk, dv) like q, k, v."""
    lib = load()
    cu, arr = _cu(cu_seqlens)
    shp = _varlen_shape(cu, heads_q, heads_kv, head_dim, block, causal, scale, q.dtype)
    dev = q.device
    _check_cu(cu, block)
    T, B = cu[-1], len(cu) - 1
    nb = varlen_block_offsets(cu, block)[-1]
    _need_packed([(q, "q", heads_q * T * head_dim, q.dtype),
                  (k, "k", heads_kv * T * head_dim, q.dtype),
                  (v, "v", heads_kv * T * head_dim, q.dtype),
                  (dout, "dout", heads_q * T * head_dim, q.dtype),
                  (lse, "lse", heads_q * T, torch.float32),
                  (sel["D"], "D", heads_q * T, torch.float32),
                  (sel["block_w"], "block_w", heads_q * nb, torch.float32),
                  (sel["kept_idx"], "kept_idx", heads_q * nb, torch.int32),
                  (sel["kept_count"], "kept_count", heads_q * B, torch.int32)], dev)
    n = ctypes.c_size_t(0)
    _check(lib, lib.lf_bwd_workspace_size_varlen(ctypes.byref(shp), arr, ctypes.byref(n)))
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib, lib.lf_attn_bwd_varlen(
        ctypes.byref(shp), arr, _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(sel["D"]),
        _ptr(sel["kept_idx"]), _ptr(sel["kept_count"]), _ptr(sel["block_w"]), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev)))
    return dq, dk, dv
