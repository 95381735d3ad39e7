"""Block-diffusion attention over a cached prefix on AMD MI355X (gfx950).

Thin Python binding of libblkattn.so (C ABI in include/blkattn.h). Every
function here only marshals arguments: torch tensors supply device memory and
the current HIP stream; all arithmetic runs in the library's HIP kernels. There
is no CPU fallback: the functions raise if the library is missing or a tensor
is not on the GPU.

Tensors are [B, H, T, d] with a unit stride along d (head_dim):
  q [B, Hq, Bq, d]; k_pre/v_pre [B, Hkv, P, d]; k_blk/v_blk [B, Hkv, Bq, d];
  idx int32 [B, Hkv, n_keep] (contiguous); o [B, Hq, Bq, d] (dtype of q);
  lse fp32 [B, Hq, Bq]; a partial is (o fp32 [B, Hq, Bq, d], m, l fp32 [B, Hq, Bq]).
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import NamedTuple, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libblkattn.so")

F32 = 0
BF16 = 1
OP_FULL = 0
OP_PREFIX_PARTIAL = 1
OP_SELECT = 2
OP_SEQUENCE = 3

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_MISALIGNED = -3
ERR_WORKSPACE = -4
ERR_HIP = -5


class Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_heads", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_len", ctypes.c_int32),
        ("n_keep", ctypes.c_int32),
        ("prefix_len", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("splits", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class Tensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_t", ctypes.c_int64),
    ]


class PartialDesc(ctypes.Structure):
    _fields_ = [("o", ctypes.c_void_p), ("m", ctypes.c_void_p), ("l", ctypes.c_void_p)]


class Partial(NamedTuple):
    """A partial online-softmax state: o (normalised), m (max score), l (sum)."""
    o: "object"
    m: "object"
    l: "object"


class BlkAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"blkattn status {status}: {message}")
        self.status = status


_lib = None

_P = ctypes.POINTER


def library() -> ctypes.CDLL:
    """Load libblkattn.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c "
                          "'import __graft_entry__; __graft_entry__.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pd, pt, pp = _P(Dims), _P(Tensor), _P(PartialDesc)
    sig = {
        "blkattn_full": (ctypes.c_int, [pd, pt, pt, pt, vp, pt, pt, pt, vp, vp, sz, vp]),
        "blkattn_full_noalloc": (ctypes.c_int, [pd, pt, pt, pt, vp, pt, pt, pt, vp, vp]),
        "blkattn_prefix_partial": (ctypes.c_int, [pd, pt, pt, pt, vp, pp, vp, sz, vp]),
        "blkattn_block_partial": (ctypes.c_int, [pd, pt, pt, pt, pp, vp]),
        "blkattn_block_step": (ctypes.c_int, [pd, pt, pt, pt, pp, pt, vp, vp]),
        "blkattn_merge": (ctypes.c_int, [pd, pp, pp, pt, vp, pp, vp]),
        "blkattn_gather_prefix": (ctypes.c_int, [pd, pt, pt, vp, pt, pt, vp]),
        "blkattn_prefix_mass": (ctypes.c_int, [pd, pt, pt, vp, vp, vp]),
        "blkattn_sequence_step": (ctypes.c_int, [pd, ctypes.c_int64, ctypes.c_int, pt, pt, pt, pp, pt, vp, vp, sz,
                                                 vp]),
        "blkattn_select_retained": (ctypes.c_int, [pd, vp, vp, vp, sz, vp]),
        "blkattn_workspace_bytes": (ctypes.c_size_t, [pd, ctypes.c_int]),
        "blkattn_plan_splits": (ctypes.c_int, [pd, ctypes.c_int]),
        "blkattn_set_kernel_events": (None, [vp, vp]),
        "blkattn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "blkattn_last_error": (ctypes.c_char_p, []),
        "blkattn_abi_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _check_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("blkattn runs on the GPU only: every tensor must be a CUDA/HIP tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")


def _expect(t, name: str, shape, dtype=None, contiguous: bool = False, optional: bool = False):
    """Raise ValueError unless `t` has exactly `shape` (and `dtype`, and is
    contiguous when asked). The C ABI takes pointers and one set of sizes, so a
    tensor that disagrees with those sizes would be read or written out of
    bounds by the kernels: every argument is checked here first."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dim() != len(shape) or tuple(int(x) for x in t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_partial_shape(p, name: str, B: int, Hq: int, rows: int, d: int, optional: bool = False):
    torch = _torch()
    if p is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    _expect(p.o, f"{name}.o", (B, Hq, rows, d), torch.float32, contiguous=True)
    _expect(p.m, f"{name}.m", (B, Hq, rows), torch.float32, contiguous=True)
    _expect(p.l, f"{name}.l", (B, Hq, rows), torch.float32, contiguous=True)


def _check_qkv(q, k, v, k_name: str, v_name: str, rows=None):
    """q [B, Hq, T, d]; k, v [B, Hkv, rows, d] of q's dtype with Hq % Hkv == 0."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, T, d], got shape {tuple(q.shape)}")
    _dtype_code(q)
    B, Hq, _, d = q.shape
    if k.dim() != 4:
        raise ValueError(f"{k_name} must be [B, H, T, d], got shape {tuple(k.shape)}")
    Hkv = k.shape[1]
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError(f"q has {Hq} heads, not a multiple of the {Hkv} heads of {k_name}")
    n = k.shape[2] if rows is None else rows
    _expect(k, k_name, (B, Hkv, n, d), q.dtype)
    _expect(v, v_name, (B, Hkv, n, d), q.dtype)
    return B, Hq, Hkv, d


def _check_idx(idx, B: int, Hkv: int):
    torch = _torch()
    if idx is None:
        return 0
    if idx.dim() != 3:
        raise ValueError(f"idx must be [B, Hkv, n_keep], got shape {tuple(idx.shape)}")
    _expect(idx, "idx", (B, Hkv, idx.shape[2]), torch.int32, contiguous=True)
    return int(idx.shape[2])


def _tensor(t) -> Optional[Tensor]:
    if t is None:
        return None
    if t.dim() != 4:
        raise ValueError(f"expected a [B, H, T, d] tensor, got shape {tuple(t.shape)}")
    if t.numel() == 0:
        return Tensor(None, 0, 0, 0)
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("the head_dim axis must have unit stride")
    return Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _partial(p: Optional[Partial]) -> Optional[PartialDesc]:
    if p is None:
        return None
    for x in p:
        if not x.is_contiguous():
            raise ValueError("partial tensors must be contiguous")
    return PartialDesc(p.o.data_ptr(), p.m.data_ptr(), p.l.data_ptr())


def _ref(x):
    return ctypes.byref(x) if x is not None else None


def _ptr(t) -> Optional[int]:
    return t.data_ptr() if t is not None else None


def _retained(idx, n_keep: int, prefix_len: int):
    """(prefix_len, idx) as the C ABI takes them. An empty retained set is an
    empty prefix: a zero-element tensor has no device address, and a NULL index
    array would mean the dense prefix."""
    if idx is not None and n_keep == 0:
        return 0, None
    return prefix_len, idx


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _raise(status: int):
    if status != OK:
        lib = library()
        raise BlkAttnError(status, lib.blkattn_last_error().decode() or lib.blkattn_strerror(status).decode())


def make_dims(q, kv_heads: int, prefix_len: int, n_keep: int = 0, scale: Optional[float] = None,
              splits: int = 0) -> Dims:
    B, Hq, Bq, d = q.shape
    return Dims(B, Hq, kv_heads, d, Bq, n_keep, prefix_len, _dtype_code(q),
                float(1.0 / math.sqrt(d) if scale is None else scale), splits, 0)


def workspace_bytes(dims: Dims, op: int) -> int:
    return int(library().blkattn_workspace_bytes(ctypes.byref(dims), op))


def plan_splits(dims: Dims, op: int) -> int:
    s = library().blkattn_plan_splits(ctypes.byref(dims), op)
    if s < 0:
        _raise(s)
    return s


def _workspace(dims: Dims, op: int, device, workspace):
    torch = _torch()
    need = workspace_bytes(dims, op)
    if need == 0:
        return None, 0
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def empty_partial(B: int, Hq: int, Bq: int, d: int, device) -> Partial:
    torch = _torch()
    return Partial(torch.empty(B, Hq, Bq, d, dtype=torch.float32, device=device),
                   torch.empty(B, Hq, Bq, dtype=torch.float32, device=device),
                   torch.empty(B, Hq, Bq, dtype=torch.float32, device=device))


def set_kernel_events(start, stop):
    """Record torch.cuda.Event `start`/`stop` around the next attention kernel."""
    handles = []
    for ev in (start, stop):
        if ev is None:
            handles.append(None)
            continue
        if not ev.cuda_event:          # torch creates the HIP event on first record
            ev.record()
        handles.append(ev.cuda_event)
    library().blkattn_set_kernel_events(*handles)


# ---------------------------------------------------------------------------
# the five entry points
# ---------------------------------------------------------------------------

def blkattn_full(q, k_pre, v_pre, k_blk, v_blk, o, lse=None, idx=None, scale=None, splits=0,
                 workspace=None, stream=None):
    """O (and LSE) of the block queries over [prefix (or its idx rows); block]."""
    torch = _torch()
    B, Hq, Hkv, d = _check_qkv(q, k_pre, v_pre, "k_pre", "v_pre")
    Bq = q.shape[2]
    _expect(k_blk, "k_blk", (B, Hkv, Bq, d), q.dtype)
    _expect(v_blk, "v_blk", (B, Hkv, Bq, d), q.dtype)
    _expect(o, "o", (B, Hq, Bq, d), q.dtype)
    _expect(lse, "lse", (B, Hq, Bq), torch.float32, contiguous=True, optional=True)
    n_keep = _check_idx(idx, B, Hkv)
    _check_gpu(q, k_pre, v_pre, k_blk, v_blk, o, lse, idx)
    P, idx = _retained(idx, n_keep, k_pre.shape[2])
    dims = make_dims(q, k_pre.shape[1], P, n_keep, scale, splits)
    ws, nbytes = _workspace(dims, OP_FULL, q.device, workspace)
    st = library().blkattn_full(ctypes.byref(dims), _ref(_tensor(q)), _ref(_tensor(k_pre)),
                                _ref(_tensor(v_pre)), _ptr(idx), _ref(_tensor(k_blk)),
                                _ref(_tensor(v_blk)), _ref(_tensor(o)), _ptr(lse), _ptr(ws),
                                nbytes, _stream(stream))
    _raise(st)
    return o, lse


def blkattn_full_noalloc(q, k_pre, v_pre, k_blk, v_blk, o, lse=None, idx=None, scale=None, splits=0,
                         stream=None):
    """blkattn_full with the key-split scratch in the library's static device
    array (no allocation, no workspace argument; see include/blkattn.h)."""
    torch = _torch()
    B, Hq, Hkv, d = _check_qkv(q, k_pre, v_pre, "k_pre", "v_pre")
    Bq = q.shape[2]
    _expect(k_blk, "k_blk", (B, Hkv, Bq, d), q.dtype)
    _expect(v_blk, "v_blk", (B, Hkv, Bq, d), q.dtype)
    _expect(o, "o", (B, Hq, Bq, d), q.dtype)
    _expect(lse, "lse", (B, Hq, Bq), torch.float32, contiguous=True, optional=True)
    n_keep = _check_idx(idx, B, Hkv)
    _check_gpu(q, k_pre, v_pre, k_blk, v_blk, o, lse, idx)
    P, idx = _retained(idx, n_keep, k_pre.shape[2])
    dims = make_dims(q, k_pre.shape[1], P, n_keep, scale, splits)
    st = library().blkattn_full_noalloc(ctypes.byref(dims), _ref(_tensor(q)), _ref(_tensor(k_pre)),
                                        _ref(_tensor(v_pre)), _ptr(idx), _ref(_tensor(k_blk)),
                                        _ref(_tensor(v_blk)), _ref(_tensor(o)), _ptr(lse), _stream(stream))
    _raise(st)
    return o, lse


def blkattn_prefix_partial(q, k_pre, v_pre, out: Partial, idx=None, scale=None, splits=0,
                           workspace=None, stream=None):
    """Partial state of the block queries over the prefix (the FACache state)."""
    B, Hq, Hkv, d = _check_qkv(q, k_pre, v_pre, "k_pre", "v_pre")
    _check_partial_shape(out, "out", B, Hq, q.shape[2], d)
    n_keep = _check_idx(idx, B, Hkv)
    _check_gpu(q, k_pre, v_pre, idx, *out)
    P, idx = _retained(idx, n_keep, k_pre.shape[2])
    dims = make_dims(q, k_pre.shape[1], P, n_keep, scale, splits)
    ws, nbytes = _workspace(dims, OP_PREFIX_PARTIAL, q.device, workspace)
    st = library().blkattn_prefix_partial(ctypes.byref(dims), _ref(_tensor(q)), _ref(_tensor(k_pre)),
                                          _ref(_tensor(v_pre)), _ptr(idx), _ref(_partial(out)),
                                          _ptr(ws), nbytes, _stream(stream))
    _raise(st)
    return out


def blkattn_block_partial(q, k_blk, v_blk, out: Partial, scale=None, stream=None):
    """Partial state of the block queries over the block's own keys (no mask)."""
    B, Hq, _, d = _check_qkv(q, k_blk, v_blk, "k_blk", "v_blk", rows=q.shape[2] if q.dim() == 4 else None)
    _check_partial_shape(out, "out", B, Hq, q.shape[2], d)
    _check_gpu(q, k_blk, v_blk, *out)
    dims = make_dims(q, k_blk.shape[1], 0, 0, scale, 0)
    st = library().blkattn_block_partial(ctypes.byref(dims), _ref(_tensor(q)), _ref(_tensor(k_blk)),
                                         _ref(_tensor(v_blk)), _ref(_partial(out)), _stream(stream))
    _raise(st)
    return out


def blkattn_block_step(q, k_blk, v_blk, cached: Partial, o, lse=None, scale=None, stream=None):
    """One reuse step in one launch: the block queries' state starts from the cached
    prefix partial and continues over the block's own keys; writes O and LSE."""
    torch = _torch()
    B, Hq, _, d = _check_qkv(q, k_blk, v_blk, "k_blk", "v_blk", rows=q.shape[2] if q.dim() == 4 else None)
    Bq = q.shape[2]
    _check_partial_shape(cached, "cached", B, Hq, Bq, d)
    _expect(o, "o", (B, Hq, Bq, d), q.dtype)
    _expect(lse, "lse", (B, Hq, Bq), torch.float32, contiguous=True, optional=True)
    _check_gpu(q, k_blk, v_blk, *cached, o, lse)
    dims = make_dims(q, k_blk.shape[1], 0, 0, scale, 0)
    st = library().blkattn_block_step(ctypes.byref(dims), _ref(_tensor(q)), _ref(_tensor(k_blk)),
                                      _ref(_tensor(v_blk)), _ref(_partial(cached)), _ref(_tensor(o)),
                                      _ptr(lse), _stream(stream))
    _raise(st)
    return o, lse


def blkattn_sequence_step(q, k, v, block_start: int, block_len: int, cache: Partial, gen_step: bool, o,
                          lse=None, scale=None, splits=0, workspace=None, stream=None):
    """First-layer attention of the whole sequence (q [B, Hq, N, d], k/v
    [B, Hkv, N, d]) at one step of the block at rows [block_start, +block_len),
    with the FACache of the other rows' queries over the other rows' keys:
    built when gen_step is true, reused otherwise. Writes o and lse [B, Hq, N]."""
    torch = _torch()
    B, Hq, _, d = _check_qkv(q, k, v, "k", "v", rows=q.shape[2] if q.dim() == 4 else None)
    N = q.shape[2]
    _check_partial_shape(cache, "cache", B, Hq, N, d)
    _expect(o, "o", (B, Hq, N, d), q.dtype)
    _expect(lse, "lse", (B, Hq, N), torch.float32, contiguous=True, optional=True)
    _check_gpu(q, k, v, *cache, o, lse)
    dims = Dims(B, Hq, k.shape[1], d, int(block_len), 0, N, _dtype_code(q),
                float(1.0 / math.sqrt(d) if scale is None else scale), splits, 0)
    ws, nbytes = _workspace(dims, OP_SEQUENCE, q.device, workspace)
    st = library().blkattn_sequence_step(ctypes.byref(dims), int(block_start), 1 if gen_step else 0,
                                         _ref(_tensor(q)), _ref(_tensor(k)), _ref(_tensor(v)),
                                         _ref(_partial(cache)), _ref(_tensor(o)), _ptr(lse), _ptr(ws), nbytes,
                                         _stream(stream))
    _raise(st)
    return o, lse


def blkattn_merge(a: Partial, b: Partial, o=None, lse=None, ab: Optional[Partial] = None,
                  dtype=None, stream=None):
    """Log-sum-exp merge of two partials; writes O (dtype of `o`), LSE and/or `ab`."""
    torch = _torch()
    if a.o.dim() != 4:
        raise ValueError(f"a.o must be [B, Hq, Bq, d], got shape {tuple(a.o.shape)}")
    B, Hq, Bq, d = a.o.shape
    _check_partial_shape(a, "a", B, Hq, Bq, d)
    _check_partial_shape(b, "b", B, Hq, Bq, d)
    _check_partial_shape(ab, "ab", B, Hq, Bq, d, optional=True)
    if o is not None:
        _dtype_code(o)
        _expect(o, "o", (B, Hq, Bq, d))
    _expect(lse, "lse", (B, Hq, Bq), torch.float32, contiguous=True, optional=True)
    _check_gpu(*a, *b, o, lse, *(ab or ()))
    code = _dtype_code(o) if o is not None else (BF16 if dtype == torch.bfloat16 else F32)
    dims = Dims(B, Hq, 1, d, Bq, 0, 0, code, 1.0, 0, 0)
    st = library().blkattn_merge(ctypes.byref(dims), _ref(_partial(a)), _ref(_partial(b)),
                                 _ref(_tensor(o)), _ptr(lse), _ref(_partial(ab)), _stream(stream))
    _raise(st)
    return o, lse, ab


def blkattn_gather_prefix(k_full, v_full, idx, k_out, v_out, stream=None):
    """Bit copy of the retained prefix rows named by idx."""
    if k_full.dim() != 4:
        raise ValueError(f"k_full must be [B, Hkv, P, d], got shape {tuple(k_full.shape)}")
    _dtype_code(k_full)
    B, Hkv, P, d = k_full.shape
    _expect(v_full, "v_full", (B, Hkv, P, d), k_full.dtype)
    n = _check_idx(idx, B, Hkv) if idx is not None else None
    if n is None:
        raise ValueError("idx is required")
    _expect(k_out, "k_out", (B, Hkv, n, d), k_full.dtype)
    _expect(v_out, "v_out", (B, Hkv, n, d), k_full.dtype)
    _check_gpu(k_full, v_full, idx, k_out, v_out)
    if n == 0:  # no rows to copy (an empty tensor has no device address to pass)
        return k_out, v_out
    dims = Dims(B, Hkv, Hkv, d, 1, int(idx.shape[-1]), P, _dtype_code(k_full), 1.0, 0, 0)
    st = library().blkattn_gather_prefix(ctypes.byref(dims), _ref(_tensor(k_full)), _ref(_tensor(v_full)),
                                         _ptr(idx), _ref(_tensor(k_out)), _ref(_tensor(v_out)),
                                         _stream(stream))
    _raise(st)
    return k_out, v_out


def blkattn_prefix_mass(q, k_pre, lse, mass, scale=None, stream=None):
    """Attention mass of every prefix row (summed probabilities over the block
    queries of the kv group), given each row's LSE over all keys."""
    torch = _torch()
    if k_pre.dim() != 4:
        raise ValueError(f"k_pre must be [B, Hkv, P, d], got shape {tuple(k_pre.shape)}")
    B, Hq, Hkv, d = _check_qkv(q, k_pre, k_pre, "k_pre", "k_pre")
    _expect(lse, "lse", (B, Hq, q.shape[2]), torch.float32, contiguous=True)
    _expect(mass, "mass", (B, Hkv, k_pre.shape[2]), torch.float32, contiguous=True)
    _check_gpu(q, k_pre, lse, mass)
    dims = make_dims(q, k_pre.shape[1], k_pre.shape[2], 0, scale, 0)
    st = library().blkattn_prefix_mass(ctypes.byref(dims), _ref(_tensor(q)), _ref(_tensor(k_pre)),
                                       _ptr(lse), _ptr(mass), _stream(stream))
    _raise(st)
    return mass


def blkattn_select_retained(mass, idx, workspace=None, stream=None):
    """The idx.shape[-1] rows of largest mass per (batch, kv head), ascending."""
    torch = _torch()
    if mass.dim() != 3:
        raise ValueError(f"mass must be [B, Hkv, P], got shape {tuple(mass.shape)}")
    B, Hkv, P = mass.shape
    _expect(mass, "mass", (B, Hkv, P), torch.float32, contiguous=True)
    n = _check_idx(idx, B, Hkv) if idx is not None else None
    if n is None:
        raise ValueError("idx is required")
    if n > P:
        raise ValueError(f"idx asks for {n} rows of {P}")
    _check_gpu(mass, idx)
    if n == 0:  # nothing to select (an empty tensor has no device address to pass)
        return idx
    dims = Dims(B, Hkv, Hkv, 64, 1, int(idx.shape[-1]), P, F32, 1.0, 0, 0)
    ws, nbytes = _workspace(dims, OP_SELECT, mass.device, workspace)
    st = library().blkattn_select_retained(ctypes.byref(dims), _ptr(mass), _ptr(idx), _ptr(ws), nbytes,
                                           _stream(stream))
    _raise(st)
    return idx


# ---------------------------------------------------------------------------
# allocating conveniences (device memory from torch, compute in the library)
# ---------------------------------------------------------------------------

def attention(q, k_pre, v_pre, k_blk, v_blk, idx=None, scale=None, splits=0, stream=None):
    """Allocate O and LSE and run blkattn_full."""
    torch = _torch()
    B, Hq, Bq, d = q.shape
    o = torch.empty(B, Hq, Bq, d, dtype=q.dtype, device=q.device)
    lse = torch.empty(B, Hq, Bq, dtype=torch.float32, device=q.device)
    return blkattn_full(q, k_pre, v_pre, k_blk, v_blk, o, lse, idx=idx, scale=scale, splits=splits,
                        stream=stream)


def prefix_partial(q, k_pre, v_pre, idx=None, scale=None, splits=0, stream=None) -> Partial:
    B, Hq, Bq, d = q.shape
    out = empty_partial(B, Hq, Bq, d, q.device)
    return blkattn_prefix_partial(q, k_pre, v_pre, out, idx=idx, scale=scale, splits=splits, stream=stream)


def block_partial(q, k_blk, v_blk, scale=None, stream=None) -> Partial:
    B, Hq, Bq, d = q.shape
    out = empty_partial(B, Hq, Bq, d, q.device)
    return blkattn_block_partial(q, k_blk, v_blk, out, scale=scale, stream=stream)


def block_step(q, k_blk, v_blk, cached: Partial, scale=None, stream=None):
    """Allocate O and LSE and run blkattn_block_step."""
    torch = _torch()
    B, Hq, Bq, d = q.shape
    o = torch.empty(B, Hq, Bq, d, dtype=q.dtype, device=q.device)
    lse = torch.empty(B, Hq, Bq, dtype=torch.float32, device=q.device)
    return blkattn_block_step(q, k_blk, v_blk, cached, o, lse, scale=scale, stream=stream)


def merge(a: Partial, b: Partial, dtype=None, stream=None):
    """Return (O in `dtype`, LSE) of two merged partials."""
    torch = _torch()
    dtype = dtype or torch.float32
    B, Hq, Bq, d = a.o.shape
    o = torch.empty(B, Hq, Bq, d, dtype=dtype, device=a.o.device)
    lse = torch.empty(B, Hq, Bq, dtype=torch.float32, device=a.o.device)
    blkattn_merge(a, b, o=o, lse=lse, stream=stream)
    return o, lse


def prefix_mass(q, k_pre, lse, scale=None, stream=None):
    torch = _torch()
    B, Hkv, P, _ = k_pre.shape
    mass = torch.empty(B, Hkv, P, dtype=torch.float32, device=q.device)
    return blkattn_prefix_mass(q, k_pre, lse, mass, scale=scale, stream=stream)


def select_retained(mass, n_keep: int, workspace=None, stream=None):
    torch = _torch()
    B, Hkv, _ = mass.shape
    idx = torch.empty(B, Hkv, n_keep, dtype=torch.int32, device=mass.device)
    return blkattn_select_retained(mass, idx, workspace=workspace, stream=stream)


def sequence_step(q, k, v, block_start: int, block_len: int, cache: Optional[Partial] = None,
                  gen_step: Optional[bool] = None, scale=None, stream=None):
    """Allocate O, LSE (and the cache when none is given, which implies a first
    step) and run blkattn_sequence_step; returns (o, lse, cache)."""
    torch = _torch()
    B, Hq, N, d = q.shape
    if cache is None:
        cache = empty_partial(B, Hq, N, d, q.device)
        gen_step = True if gen_step is None else gen_step
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, dtype=torch.float32, device=q.device)
    blkattn_sequence_step(q, k, v, block_start, block_len, cache, bool(gen_step), o, lse, scale=scale,
                          stream=stream)
    return o, lse, cache


def gather_prefix(k_full, v_full, idx, stream=None):
    torch = _torch()
    B, Hkv, P, d = k_full.shape
    n = int(idx.shape[-1])
    k_out = torch.empty(B, Hkv, n, d, dtype=k_full.dtype, device=k_full.device)
    v_out = torch.empty(B, Hkv, n, d, dtype=v_full.dtype, device=v_full.device)
    return blkattn_gather_prefix(k_full, v_full, idx, k_out, v_out, stream=stream)
