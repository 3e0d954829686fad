"""Thin ctypes binding of libttbag (the C ABI in include/tt_bag.h).

Argument marshalling only: every function checks device/dtype/contiguity of the
torch tensors it is handed, passes their device pointers and the current HIP
stream to the C entry point of the same name, and raises ``TTError`` on a
negative return code.  No arithmetic of the method happens here.  Loading fails
loudly (``RuntimeError``) when the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttbag.so")

TT_OK = 0
TT_DEV_BAD_INDEX = 1
TT_DEV_BAD_OFFSETS = 2
TT_DEV_BAD_SLOT = 4
TT_DEV_HASH_FULL = 8
TT_DEV_STALE_PLAN = 16
TT_DEV_SYNC_TIMEOUT = 32
TT_POOL_SUM = 0
TT_POOL_MEAN = 1
TT_CACHE_TOPK = 0
TT_CACHE_LFU32 = 1
TT_INIT_UNIFORM = 0
TT_INIT_NORMAL = 1
TT_INIT_APPROX_UNIFORM = 2
TT_INIT_APPROX_NORMAL = 3


class TTError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__("%s failed: %d (%s)" % (fn, code, status_string(code)))
        self.code = code


class TTDesc(ctypes.Structure):
    _fields_ = [("num_tables", ctypes.c_int32), ("num_embeddings", ctypes.c_int64),
                ("p", ctypes.c_int32 * 3), ("q", ctypes.c_int32 * 3),
                ("ranks", ctypes.c_int32 * 2), ("pooling", ctypes.c_int32)]


TT_MAX_CORES = 8


class TTDescD(ctypes.Structure):
    _fields_ = [("num_tables", ctypes.c_int32), ("d", ctypes.c_int32),
                ("num_embeddings", ctypes.c_int64), ("p", ctypes.c_int32 * TT_MAX_CORES),
                ("q", ctypes.c_int32 * TT_MAX_CORES),
                ("ranks", ctypes.c_int32 * (TT_MAX_CORES - 1)), ("pooling", ctypes.c_int32)]


class TTCacheView(ctypes.Structure):
    _fields_ = [("slots", ctypes.c_void_p), ("rows", ctypes.c_void_p),
                ("cache_size", ctypes.c_int64)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIG = {
    "tt_bag_workspace_size": (ctypes.c_size_t, [_P, _I64, _I64, _I64]),
    "tt_bag_forward": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P, ctypes.c_size_t,
                                      _P, _P]),
    "tt_bag_backward_sgd": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, ctypes.c_float,
                                           _P, ctypes.c_size_t, _P, _P]),
    "tt_bag_forward_static": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P, _P]),
    "tt_bag_plan": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "tt_bag_forward_planned": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P,
                                              ctypes.c_size_t, _P, _P]),
    "tt_bag_backward_sgd_planned": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P,
                                                   ctypes.c_float, _P, ctypes.c_size_t, _P, _P]),
    "tt_bag_backward_adagrad": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P,
                                               ctypes.c_float, ctypes.c_float, _P, _P, _P,
                                               ctypes.c_size_t, _P, _P]),
    "tt_bag_backward_adagrad_planned": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P,
                                                       ctypes.c_float, ctypes.c_float, _P, _P,
                                                       _P, ctypes.c_size_t, _P, _P]),
    "tt_bag_backward_grad": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _P,
                                            ctypes.c_size_t, _P, _P]),
    "tt_bag_backward_grad_planned": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P,
                                                    _P, _P, ctypes.c_size_t, _P, _P]),
    "tt_bag_weight_grad": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P, _P]),
    "tt_bag_weight_grad_planned": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P,
                                                  _P, ctypes.c_size_t, _P, _P]),
    "tt_bag_route": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _P, _I64, _P, _P, _P, ctypes.c_size_t,
                                    _P, _P]),
    "tt_init_cores": (ctypes.c_int, [_P, _P, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, _P]),
    "tt_factorize": (ctypes.c_int, [_I64, ctypes.c_int, _P]),
    "tt_full_weight": (ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _I64, _P, _P]),
    "tt_bag_workspace_size_dedup": (ctypes.c_size_t, [_P, _I64, _I64]),
    "tt_bag_plan_dedup": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _P, _P, ctypes.c_size_t, _P, _P,
                                         _P]),
    "tt_bag_backward_sgd_dedup": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P,
                                                 ctypes.c_float, _P, _P, ctypes.c_size_t, _P,
                                                 _P]),
    "tt_bag_backward_grad_dedup": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P, _P,
                                                  ctypes.c_size_t, _P, _P]),
    "tt_bag_dedup_counts": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_size_t, _P, _P]),
    "tt_bag_workspace_size_d": (ctypes.c_size_t, [_P, _I64, _I64]),
    "tt_bag_groups_d": (ctypes.c_int, [_P, _P]),
    "tt_bag_forward_d": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, ctypes.c_size_t,
                                        _P, _P]),
    "tt_bag_backward_sgd_d": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, ctypes.c_float,
                                             _P, ctypes.c_size_t, _P, _P]),
    "tt_bag_backward_grad_d": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P,
                                              ctypes.c_size_t, _P, _P]),
    "tt_bag_plan_d": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _P, _P, ctypes.c_size_t, _P, _P]),
    "tt_bag_forward_d_planned": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P,
                                                ctypes.c_size_t, _P, _P]),
    "tt_bag_backward_sgd_d_planned": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P,
                                                     ctypes.c_float, _P, ctypes.c_size_t, _P,
                                                     _P]),
    "tt_bag_backward_grad_d_planned": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I64, _P, _P, _P,
                                                      _P, ctypes.c_size_t, _P, _P]),
    "tt_cache_create": (ctypes.c_int, [_P, _P, _I64, _I64]),
    "tt_cache_create_policy": (ctypes.c_int, [_P, _P, _I64, _I64, ctypes.c_int]),
    "tt_cache_export": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "tt_cache_import": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "tt_cache_lookup": (ctypes.c_int, [_P, _P, _I64, _P, ctypes.c_int, _P, _P]),
    "tt_cache_populate": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "tt_cache_cached_indices": (ctypes.c_int, [_P, _P, _P]),
    "tt_cache_destroy": (ctypes.c_int, [_P]),
    "tt_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "tt_profile_num_kernels": (ctypes.c_int, []),
    "tt_profile_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
    "tt_profile_read": (ctypes.c_int, [ctypes.c_int, _P, _P]),
    "tt_debug_sync_poll_limit": (ctypes.c_int, [_I64]),
    "tt_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}
EXPORTS = tuple(_SIG)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libttbag; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libttbag.so is not built (%s); run __graft_entry__.build() or "
                               "python -m tensor_train_compressed_ttembeddingbag_amd.build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().tt_status_string(int(code)).decode()


def make_desc(p, q, ranks, num_embeddings: Optional[int] = None, num_tables: int = 1,
              pooling: int = 0) -> TTDesc:
    d = TTDesc()
    d.pooling = int(pooling)
    d.num_tables = int(num_tables)
    d.num_embeddings = int(num_embeddings if num_embeddings is not None else p[0] * p[1] * p[2])
    for k in range(3):
        d.p[k] = int(p[k])
        d.q[k] = int(q[k])
    d.ranks[0], d.ranks[1] = int(ranks[0]), int(ranks[1])
    return d


# Marshalling is kept cheap: a training step makes a few of these calls, and their host
# cost adds to every step's latency when the kernels are short.
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()  # argtypes convert the int to void*


def _need(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _numel(t: torch.Tensor, n: int, name: str):
    """The kernels index every buffer by the sizes the call states, so a buffer of any
    other size would be read or written out of bounds: reject it here."""
    if t.numel() != n:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), n))


def _dim(desc) -> int:
    return desc.q[0] * desc.q[1] * desc.q[2]


def _core_numels(desc):
    """Elements of core k of all tables: T * p_k * R_{k-1} * q_k * R_k."""
    T, r = desc.num_tables, (1, desc.ranks[0], desc.ranks[1], 1)
    return tuple(T * desc.p[k] * r[k] * desc.q[k] * r[k + 1] for k in range(3))


def _batch_sizes(desc, indices, offsets, num_bags: int, per_sample_weights=None):
    """offsets must hold T*num_bags + 1 entries (the terminal one included) and the
    per-sample weights one per index."""
    _numel(offsets, desc.num_tables * int(num_bags) + 1, "offsets")
    if per_sample_weights is not None:
        _numel(per_sample_weights, indices.numel(), "per_sample_weights")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, like: Optional[torch.Tensor] = None):
    """The HIP stream handle: the given torch stream, else the current stream of the
    device that holds `like` (of the current device without it)."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(like.get_device() if like is not None else torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int):
    if rc != TT_OK:
        raise TTError(fn, rc)


def tt_bag_workspace_size(desc: TTDesc, nnz: int, num_bags: int, cache_size: int = 0) -> int:
    n = lib().tt_bag_workspace_size(ctypes.byref(desc), int(nnz), int(num_bags), int(cache_size))
    if n == 0:
        raise TTError("tt_bag_workspace_size", -2)
    return int(n)


def workspace(desc: TTDesc, nnz: int, num_bags: int, cache_size: int = 0, device=None) -> torch.Tensor:
    """A workspace tensor of the required size (torch's allocations are 256-B aligned)."""
    n = tt_bag_workspace_size(desc, nnz, num_bags, cache_size)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


_core_arrays = {}


def _cores(cores: Sequence[torch.Tensor], desc=None, name: str = "cores"):
    if len(cores) != 3:
        raise ValueError("three cores expected")
    for c in cores:
        _need(c, torch.float32, name)
    if desc is not None:
        for k, n in enumerate(_core_numels(desc)):
            _numel(cores[k], n, "%s[%d]" % (name, k))
    key = (cores[0].data_ptr(), cores[1].data_ptr(), cores[2].data_ptr())
    arr = _core_arrays.get(key)
    if arr is None:  # pointer triples are reused across calls: keep their ctypes arrays
        if len(_core_arrays) >= 64:
            _core_arrays.clear()
        arr = _core_arrays[key] = (ctypes.c_void_p * 3)(*key)
    return arr


def _cache_view(cache, desc=None, nnz: Optional[int] = None):
    if cache is None:
        return None, None
    slots, rows = cache
    _need(slots, torch.int32, "cache slots")
    _need(rows, torch.float32, "cache rows")
    if rows.dim() != 2 or (desc is not None and rows.shape[1] != _dim(desc)):
        raise ValueError("cache rows must be [cache_size, D], got %s" % (tuple(rows.shape),))
    if nnz is not None:
        _numel(slots, nnz, "cache slots")
    v = TTCacheView()
    v.slots = slots.data_ptr()
    v.rows = rows.data_ptr()
    v.cache_size = rows.shape[0]
    return v, rows.shape[0]


def tt_bag_plan(desc: TTDesc, indices, offsets, num_bags: int, per_sample_weights=None,
                cache=None, ws=None, dev_status=None, stream=None) -> torch.Tensor:
    """Run the grouping step into ws (allocated if None) and return ws."""
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    view, csize = _cache_view(cache, desc, indices.numel())
    if ws is None:
        ws = workspace(desc, indices.numel(), num_bags, csize or 0, indices.device)
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    rc = lib().tt_bag_plan(ctypes.byref(desc), _ptr(indices), indices.numel(), _ptr(offsets),
                           int(num_bags), _ptr(per_sample_weights),
                           None if view is None else ctypes.byref(view), _ptr(ws),
                           ws.numel(), _ptr(dev_status), _stream(stream, indices))
    _check("tt_bag_plan", rc)
    return ws


def tt_bag_forward(desc: TTDesc, cores, indices, offsets, num_bags: int,
                   per_sample_weights=None, cache=None, out=None, ws=None,
                   dev_status=None, stream=None, planned: bool = False) -> torch.Tensor:
    """out[T*num_bags, D] = pooled rows (see tt_bag.h).  cache = (slots, rows) or None.
    planned=True reuses the grouping that tt_bag_plan left in ws."""
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    D = _dim(desc)
    if out is None:
        out = torch.empty(desc.num_tables * num_bags, D, dtype=torch.float32, device=indices.device)
    _need(out, torch.float32, "out")
    _numel(out, desc.num_tables * int(num_bags) * D, "out")
    view, csize = _cache_view(cache, desc, indices.numel())
    if ws is None:
        ws = workspace(desc, indices.numel(), num_bags, csize or 0, indices.device)
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    core_ptrs = _cores(cores, desc)
    fn = lib().tt_bag_forward_planned if planned else lib().tt_bag_forward
    rc = fn(ctypes.byref(desc), core_ptrs, _ptr(indices), indices.numel(),
                              _ptr(offsets), int(num_bags), _ptr(per_sample_weights),
                              None if view is None else ctypes.byref(view), _ptr(out), _ptr(ws),
                              ws.numel(), _ptr(dev_status), _stream(stream, indices))
    _check("tt_bag_forward_planned" if planned else "tt_bag_forward", rc)
    return out


TT_STATIC_SCRATCH_BYTES = 8388608


def tt_bag_forward_static(desc: TTDesc, cores, indices, offsets, num_bags: int,
                          per_sample_weights=None, cache=None, out=None, dev_status=None,
                          stream=None) -> torch.Tensor:
    """tt_bag_forward in the library's static scratch: no workspace, no allocation in the
    library (out is allocated here only when not given)."""
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    D = _dim(desc)
    if out is None:
        out = torch.empty(desc.num_tables * num_bags, D, dtype=torch.float32, device=indices.device)
    _need(out, torch.float32, "out")
    _numel(out, desc.num_tables * int(num_bags) * D, "out")
    view, _ = _cache_view(cache, desc, indices.numel())
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    core_ptrs = _cores(cores, desc)
    rc = lib().tt_bag_forward_static(ctypes.byref(desc), core_ptrs, _ptr(indices),
                                     indices.numel(), _ptr(offsets), int(num_bags),
                                     _ptr(per_sample_weights),
                                     None if view is None else ctypes.byref(view), _ptr(out),
                                     _ptr(dev_status), _stream(stream, indices))
    _check("tt_bag_forward_static", rc)
    return out


def tt_bag_backward_sgd(desc: TTDesc, cores, indices, offsets, num_bags: int, grad_out,
                        lr: float, per_sample_weights=None, cache=None, ws=None,
                        dev_status=None, stream=None, planned: bool = False) -> None:
    """In-place fused SGD on the cores (and cache rows) touched by this batch.
    planned=True reuses the grouping that tt_bag_plan left in ws."""
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    _need(grad_out, torch.float32, "grad_out")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    _numel(grad_out, desc.num_tables * int(num_bags) * _dim(desc), "grad_out")
    view, csize = _cache_view(cache, desc, indices.numel())
    if ws is None:
        ws = workspace(desc, indices.numel(), num_bags, csize or 0, indices.device)
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    core_ptrs = _cores(cores, desc)
    fn = lib().tt_bag_backward_sgd_planned if planned else lib().tt_bag_backward_sgd
    rc = fn(ctypes.byref(desc), core_ptrs, _ptr(indices), indices.numel(),
                                   _ptr(offsets), int(num_bags), _ptr(per_sample_weights),
                                   None if view is None else ctypes.byref(view), _ptr(grad_out),
                                   float(lr), _ptr(ws), ws.numel(), _ptr(dev_status),
                                   _stream(stream, indices))
    _check("tt_bag_backward_sgd_planned" if planned else "tt_bag_backward_sgd", rc)


def _batch_args(desc, indices, offsets, num_bags, grad_out, per_sample_weights, cache, ws,
                dev_status):
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    _need(grad_out, torch.float32, "grad_out")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    _numel(grad_out, desc.num_tables * int(num_bags) * _dim(desc), "grad_out")
    view, csize = _cache_view(cache, desc, indices.numel())
    if ws is None:
        ws = workspace(desc, indices.numel(), num_bags, csize or 0, indices.device)
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    return view, csize, ws


def _rows_arg(t, csize, name, D):
    if not csize:
        return None
    if t is None:
        raise ValueError("%s is required with a cache" % name)
    _need(t, torch.float32, name)
    _numel(t, int(csize) * D, name)
    return t


def tt_bag_backward_adagrad(desc: TTDesc, cores, indices, offsets, num_bags: int, grad_out,
                            lr: float, eps: float, state, state_rows=None,
                            per_sample_weights=None, cache=None, ws=None, dev_status=None,
                            stream=None, planned: bool = False) -> None:
    """In-place fused Adagrad on the touched cores / cache rows; state = three running-sum
    tensors shaped like the cores (and state_rows for the cache rows), updated in place."""
    view, csize, ws = _batch_args(desc, indices, offsets, num_bags, grad_out, per_sample_weights,
                                  cache, ws, dev_status)
    st = _cores(state, desc, "state")
    sr = _rows_arg(state_rows, csize, "state_rows", _dim(desc))
    name = "tt_bag_backward_adagrad_planned" if planned else "tt_bag_backward_adagrad"
    core_ptrs = _cores(cores, desc)
    rc = getattr(lib(), name)(ctypes.byref(desc), core_ptrs, _ptr(indices),
                              indices.numel(), _ptr(offsets), int(num_bags),
                              _ptr(per_sample_weights),
                              None if view is None else ctypes.byref(view), _ptr(grad_out),
                              float(lr), float(eps), st, _ptr(sr), _ptr(ws), ws.numel(),
                              _ptr(dev_status), _stream(stream, indices))
    _check(name, rc)


def tt_bag_backward_grad(desc: TTDesc, cores, indices, offsets, num_bags: int, grad_out,
                         grad_cores=None, grad_rows=None, per_sample_weights=None, cache=None,
                         ws=None, dev_status=None, stream=None, planned: bool = False):
    """Gradients with respect to the cores (and cache rows), fully overwritten; the
    cores are not changed.  Returns (grad_cores, grad_rows)."""
    view, csize, ws = _batch_args(desc, indices, offsets, num_bags, grad_out, per_sample_weights,
                                  cache, ws, dev_status)
    if grad_cores is None:
        grad_cores = [torch.empty_like(c) for c in cores]
    if csize and grad_rows is None:
        grad_rows = torch.empty_like(cache[1])
    gr = _rows_arg(grad_rows, csize, "grad_rows", _dim(desc))
    name = "tt_bag_backward_grad_planned" if planned else "tt_bag_backward_grad"
    core_ptrs = _cores(cores, desc)
    grad_ptrs = _cores(grad_cores, desc, "grad_cores")
    rc = getattr(lib(), name)(ctypes.byref(desc), core_ptrs, _ptr(indices),
                              indices.numel(), _ptr(offsets), int(num_bags),
                              _ptr(per_sample_weights),
                              None if view is None else ctypes.byref(view), _ptr(grad_out),
                              grad_ptrs, _ptr(gr), _ptr(ws), ws.numel(),
                              _ptr(dev_status), _stream(stream, indices))
    _check(name, rc)
    return grad_cores, gr


def tt_bag_weight_grad(desc: TTDesc, cores, indices, offsets, num_bags: int, grad_out,
                       per_sample_weights=None, cache=None, out=None, ws=None, dev_status=None,
                       stream=None, planned: bool = False) -> torch.Tensor:
    """dL/dw per element (see tt_bag.h); returns out [nnz] fp32."""
    view, csize, ws = _batch_args(desc, indices, offsets, num_bags, grad_out, per_sample_weights,
                                  cache, ws, dev_status)
    if out is None:
        out = torch.empty(indices.numel(), dtype=torch.float32, device=indices.device)
    _need(out, torch.float32, "out")
    _numel(out, indices.numel(), "out")
    name = "tt_bag_weight_grad_planned" if planned else "tt_bag_weight_grad"
    core_ptrs = _cores(cores, desc)
    rc = getattr(lib(), name)(ctypes.byref(desc), core_ptrs, _ptr(indices), indices.numel(),
                              _ptr(offsets), int(num_bags), _ptr(per_sample_weights),
                              None if view is None else ctypes.byref(view), _ptr(grad_out),
                              _ptr(out), _ptr(ws), ws.numel(), _ptr(dev_status), _stream(stream, indices))
    _check(name, rc)
    return out


def tt_init_cores(desc: TTDesc, cores, dist: int, scale: float, seed: int, stream=None) -> None:
    """Fill the three core tensors (slice-major, all tables) on the device (see tt_bag.h)."""
    core_ptrs = _cores(cores, desc)
    _check("tt_init_cores", lib().tt_init_cores(ctypes.byref(desc), core_ptrs, int(dist),
                                                float(scale), int(seed) & ((1 << 64) - 1),
                                                _stream(stream)))


def tt_full_weight(desc: TTDesc, cores, first: int, count: int, table: int = 0, out=None,
                   stream=None) -> torch.Tensor:
    """Rows [first, first + count) of one table as a dense [count, D] tensor."""
    D = _dim(desc)
    if out is None:
        out = torch.empty(int(count), D, dtype=torch.float32, device=cores[0].device)
    _need(out, torch.float32, "out")
    _numel(out, max(int(count), 0) * D, "out")
    core_ptrs = _cores(cores, desc)
    _check("tt_full_weight", lib().tt_full_weight(ctypes.byref(desc), core_ptrs, int(table),
                                                  int(first), int(count), _ptr(out),
                                                  _stream(stream)))
    return out


def tt_factorize(n: int, exact: bool):
    """Automatic factorisation of a table size (exact: product == n, else >= n)."""
    out = (ctypes.c_int32 * 3)()
    _check("tt_factorize", lib().tt_factorize(int(n), 1 if exact else 0, out))
    return tuple(int(x) for x in out)


def tt_bag_route(desc: TTDesc, indices, offsets, num_bags: int, slots=None, cache_size: int = 0,
                 ws=None, dev_status=None, stream=None):
    """(order[nnz] int32, group_off[T*p2+2] int32) -- the grouping order (tt_bag.h)."""
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    if slots is not None:
        _need(slots, torch.int32, "slots")
        _numel(slots, indices.numel(), "slots")
    _batch_sizes(desc, indices, offsets, num_bags)
    dev = indices.device
    order = torch.empty(indices.numel(), dtype=torch.int32, device=dev)
    goff = torch.empty(desc.num_tables * desc.p[1] + 2, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(desc, indices.numel(), num_bags, cache_size if slots is not None else 0, dev)
    rc = lib().tt_bag_route(ctypes.byref(desc), _ptr(indices), indices.numel(), _ptr(offsets),
                            int(num_bags), _ptr(slots), int(cache_size), _ptr(order), _ptr(goff),
                            _ptr(ws), ws.numel(), _ptr(dev_status), _stream(stream, indices))
    _check("tt_bag_route", rc)
    return order, goff


def tt_debug_sync_poll_limit(polls: int) -> None:
    """Bound the device-side waits of later calls (polls < 0: the default); see tt_bag.h."""
    _check("tt_debug_sync_poll_limit", lib().tt_debug_sync_poll_limit(int(polls)))


def tt_profile_enable(on: bool = True) -> None:
    """Start (clearing totals) or stop per-kernel event timing inside the library."""
    _check("tt_profile_enable", lib().tt_profile_enable(1 if on else 0))


def tt_profile_read() -> dict:
    """{kernel name: (total_ms, launches)} for every kernel timed since enabling."""
    L = lib()
    out = {}
    for k in range(L.tt_profile_num_kernels()):
        ms = ctypes.c_double(0.0)
        n = ctypes.c_int64(0)
        _check("tt_profile_read", L.tt_profile_read(k, ctypes.byref(ms), ctypes.byref(n)))
        out[L.tt_profile_kernel_name(k).decode()] = (ms.value, n.value)
    return out


class Cache:
    """Owner of a tt_cache handle (frequency table + index->slot map)."""

    def __init__(self, desc: TTDesc, cache_size: int, hashtbl_size: int,
                 policy: int = TT_CACHE_TOPK):
        self.desc = desc
        self.cache_size = int(cache_size)
        self.hashtbl_size = int(hashtbl_size)
        self._h = ctypes.c_void_p()
        _check("tt_cache_create_policy",
               lib().tt_cache_create_policy(ctypes.byref(self._h), ctypes.byref(desc),
                                            int(cache_size), int(hashtbl_size), int(policy)))

    def lookup(self, indices, slot_out=None, count_freq: bool = True, dev_status=None,
               stream=None) -> torch.Tensor:
        _need(indices, torch.int64, "indices")
        if slot_out is None:
            slot_out = torch.empty(indices.numel(), dtype=torch.int32, device=indices.device)
        _need(slot_out, torch.int32, "slot_out")
        _numel(slot_out, indices.numel(), "slot_out")
        _check("tt_cache_lookup", lib().tt_cache_lookup(self._h, _ptr(indices), indices.numel(),
                                                        _ptr(slot_out), 1 if count_freq else 0,
                                                        _ptr(dev_status), _stream(stream, indices)))
        return slot_out

    def populate(self, cores, rows, stream=None) -> int:
        _need(rows, torch.float32, "rows")
        _numel(rows, self.cache_size * _dim(self.desc), "rows")
        n = ctypes.c_int64(0)
        core_ptrs = _cores(cores, self.desc)
        _check("tt_cache_populate", lib().tt_cache_populate(self._h, core_ptrs, _ptr(rows),
                                                            ctypes.byref(n), _stream(stream)))
        return int(n.value)

    def cached_indices(self, stream=None) -> torch.Tensor:
        out = torch.empty(self.cache_size, dtype=torch.int64, device="cuda")
        _check("tt_cache_cached_indices",
               lib().tt_cache_cached_indices(self._h, _ptr(out), _stream(stream)))
        return out

    def export_state(self, stream=None):
        """(cached [cache_size] int64, keys [hashtbl_size] int64, counts [hashtbl_size] int32)."""
        cached = torch.empty(self.cache_size, dtype=torch.int64, device="cuda")
        keys = torch.empty(self.hashtbl_size, dtype=torch.int64, device="cuda")
        counts = torch.empty(self.hashtbl_size, dtype=torch.int32, device="cuda")
        _check("tt_cache_export", lib().tt_cache_export(self._h, _ptr(cached), _ptr(keys),
                                                        _ptr(counts), _stream(stream)))
        return cached, keys, counts

    def import_state(self, cached, keys, counts, stream=None) -> None:
        _need(cached, torch.int64, "cached")
        _need(keys, torch.int64, "keys")
        _need(counts, torch.int32, "counts")
        if (cached.numel() != self.cache_size or keys.numel() != self.hashtbl_size
                or counts.numel() != self.hashtbl_size):
            raise ValueError("state sizes do not match this cache")
        _check("tt_cache_import", lib().tt_cache_import(self._h, _ptr(cached), _ptr(keys),
                                                        _ptr(counts), _stream(stream)))

    def close(self):
        if self._h:
            lib().tt_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------ backward over distinct indices

def workspace_dedup(desc: TTDesc, nnz: int, num_bags: int, device=None) -> torch.Tensor:
    n = lib().tt_bag_workspace_size_dedup(ctypes.byref(desc), int(nnz), int(num_bags))
    if n == 0:
        raise TTError("tt_bag_workspace_size_dedup", -2)
    return torch.empty(int(n), dtype=torch.uint8, device=device or "cuda")


def tt_bag_plan_dedup(desc: TTDesc, indices, offsets, num_bags: int, per_sample_weights=None,
                      ws=None, dev_status=None, stream=None):
    """Group the batch and its distinct indices (asynchronous: the number of distinct
    indices stays on the device).  Returns (ws, info), info = the virtual batch's bounds
    (nnz, nnz): pass both to tt_bag_forward(planned=True) / tt_bag_backward_*_dedup."""
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    if ws is None:
        ws = workspace_dedup(desc, indices.numel(), num_bags, indices.device)
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    info = (ctypes.c_int64 * 2)()
    rc = lib().tt_bag_plan_dedup(ctypes.byref(desc), _ptr(indices), indices.numel(),
                                 _ptr(offsets), int(num_bags), _ptr(per_sample_weights), _ptr(ws),
                                 ws.numel(), _ptr(dev_status), info, _stream(stream, indices))
    _check("tt_bag_plan_dedup", rc)
    return ws, (int(info[0]), int(info[1]))


def tt_bag_dedup_counts(desc: TTDesc, nnz: int, num_bags: int, ws, stream=None):
    """Distinct-index counts of the batch last planned in ws by tt_bag_plan_dedup (waits for
    the stream): [before table 0, ..., before table T-1, all]."""
    _need(ws, torch.uint8, "ws")
    out = (ctypes.c_int64 * (desc.num_tables + 1))()
    rc = lib().tt_bag_dedup_counts(ctypes.byref(desc), int(nnz), int(num_bags), _ptr(ws),
                                   ws.numel(), out, _stream(stream, ws))
    _check("tt_bag_dedup_counts", rc)
    return [int(x) for x in out]


def _dedup_args(desc, indices, offsets, num_bags, grad_out, per_sample_weights, ws, dev_status):
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    _need(grad_out, torch.float32, "grad_out")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    _numel(grad_out, desc.num_tables * int(num_bags) * _dim(desc), "grad_out")
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")


def _info(info):
    return (ctypes.c_int64 * 2)(int(info[0]), int(info[1]))


def tt_bag_backward_sgd_dedup(desc: TTDesc, cores, indices, offsets, num_bags: int, grad_out,
                              lr: float, info, per_sample_weights=None, ws=None, dev_status=None,
                              stream=None) -> None:
    """In-place SGD through the backward over distinct indices (plan: tt_bag_plan_dedup)."""
    _dedup_args(desc, indices, offsets, num_bags, grad_out, per_sample_weights, ws, dev_status)
    core_ptrs = _cores(cores, desc)
    rc = lib().tt_bag_backward_sgd_dedup(ctypes.byref(desc), core_ptrs, _ptr(indices),
                                         indices.numel(), _ptr(offsets), int(num_bags),
                                         _ptr(per_sample_weights), _ptr(grad_out), float(lr),
                                         _info(info), _ptr(ws), ws.numel(), _ptr(dev_status),
                                         _stream(stream, indices))
    _check("tt_bag_backward_sgd_dedup", rc)


def tt_bag_backward_grad_dedup(desc: TTDesc, cores, indices, offsets, num_bags: int, grad_out,
                               info, grad_cores=None, per_sample_weights=None, ws=None,
                               dev_status=None, stream=None):
    """Dense core gradients through the backward over distinct indices; returns them."""
    _dedup_args(desc, indices, offsets, num_bags, grad_out, per_sample_weights, ws, dev_status)
    if grad_cores is None:
        grad_cores = [torch.empty_like(c) for c in cores]
    core_ptrs = _cores(cores, desc)
    grad_ptrs = _cores(grad_cores, desc, "grad_cores")
    rc = lib().tt_bag_backward_grad_dedup(ctypes.byref(desc), core_ptrs, _ptr(indices),
                                          indices.numel(), _ptr(offsets), int(num_bags),
                                          _ptr(per_sample_weights), _ptr(grad_out),
                                          grad_ptrs, _info(info), _ptr(ws), ws.numel(),
                                          _ptr(dev_status), _stream(stream, indices))
    _check("tt_bag_backward_grad_dedup", rc)
    return grad_cores


# ------------------------------------------------------------------ d-core tables

def make_desc_d(p, q, ranks, num_embeddings: Optional[int] = None, num_tables: int = 1,
                pooling: int = 0) -> TTDescD:
    """Descriptor of d-core tables, d = len(p) = len(q) = len(ranks) + 1."""
    d = len(p)
    if not (3 <= d <= TT_MAX_CORES and len(q) == d and len(ranks) == d - 1):
        raise ValueError("d-core shape: 3 <= len(p) == len(q) == len(ranks) + 1 <= %d"
                         % TT_MAX_CORES)
    x = TTDescD()
    x.num_tables, x.d, x.pooling = int(num_tables), d, int(pooling)
    x.num_embeddings = int(num_embeddings if num_embeddings is not None else math.prod(p))
    for k in range(d):
        x.p[k], x.q[k] = int(p[k]), int(q[k])
    for k in range(d - 1):
        x.ranks[k] = int(ranks[k])
    return x


def _core_numels_d(desc: TTDescD):
    d, r = desc.d, [1] + [desc.ranks[k] for k in range(desc.d - 1)] + [1]
    return tuple(desc.num_tables * desc.p[k] * r[k] * desc.q[k] * r[k + 1] for k in range(d))


def _cores_d(desc: TTDescD, cores, name: str = "cores"):
    if len(cores) != desc.d:
        raise ValueError("%d cores expected" % desc.d)
    for k, (c, n) in enumerate(zip(cores, _core_numels_d(desc))):
        _need(c, torch.float32, name)
        _numel(c, n, "%s[%d]" % (name, k))
    return (ctypes.c_void_p * desc.d)(*[c.data_ptr() for c in cores])


def tt_bag_workspace_size_d(desc: TTDescD, nnz: int, num_bags: int) -> int:
    n = lib().tt_bag_workspace_size_d(ctypes.byref(desc), int(nnz), int(num_bags))
    if n == 0:
        raise TTError("tt_bag_workspace_size_d", -2)
    return int(n)


def workspace_d(desc: TTDescD, nnz: int, num_bags: int, device=None) -> torch.Tensor:
    return torch.empty(tt_bag_workspace_size_d(desc, nnz, num_bags), dtype=torch.uint8,
                       device=device or "cuda")


def tt_bag_groups_d(desc: TTDescD):
    """The cut of the d cores into three groups: (a, b) for [0, a), [a, b), [b, d)."""
    cut = (ctypes.c_int32 * 2)()
    _check("tt_bag_groups_d", lib().tt_bag_groups_d(ctypes.byref(desc), cut))
    return int(cut[0]), int(cut[1])


def _args_d(desc, indices, offsets, num_bags, per_sample_weights, ws, dev_status):
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    if ws is None:
        ws = workspace_d(desc, indices.numel(), num_bags, indices.device)
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    return ws


def tt_bag_plan_d(desc: TTDescD, indices, offsets, num_bags: int, per_sample_weights=None,
                  ws=None, dev_status=None, stream=None) -> torch.Tensor:
    """Group the batch into ws (allocated if None) for the _planned d-core calls."""
    ws = _args_d(desc, indices, offsets, num_bags, per_sample_weights, ws, dev_status)
    rc = lib().tt_bag_plan_d(ctypes.byref(desc), _ptr(indices), indices.numel(), _ptr(offsets),
                             int(num_bags), _ptr(per_sample_weights), _ptr(ws), ws.numel(),
                             _ptr(dev_status), _stream(stream, indices))
    _check("tt_bag_plan_d", rc)
    return ws


def tt_bag_forward_d(desc: TTDescD, cores, indices, offsets, num_bags: int,
                     per_sample_weights=None, out=None, ws=None, dev_status=None,
                     stream=None, planned: bool = False) -> torch.Tensor:
    """out[T*num_bags, D] = pooled rows of d-core tables (see tt_bag.h)."""
    ws = _args_d(desc, indices, offsets, num_bags, per_sample_weights, ws, dev_status)
    D = math.prod(desc.q[k] for k in range(desc.d))
    if out is None:
        out = torch.empty(desc.num_tables * num_bags, D, dtype=torch.float32,
                          device=indices.device)
    _need(out, torch.float32, "out")
    _numel(out, desc.num_tables * int(num_bags) * D, "out")
    core_ptrs = _cores_d(desc, cores)
    fn = lib().tt_bag_forward_d_planned if planned else lib().tt_bag_forward_d
    rc = fn(ctypes.byref(desc), core_ptrs, _ptr(indices),
                                indices.numel(), _ptr(offsets), int(num_bags),
                                _ptr(per_sample_weights), _ptr(out), _ptr(ws), ws.numel(),
                                _ptr(dev_status), _stream(stream, indices))
    _check("tt_bag_forward_d", rc)
    return out


def tt_bag_backward_sgd_d(desc: TTDescD, cores, indices, offsets, num_bags: int, grad_out,
                          lr: float, per_sample_weights=None, ws=None, dev_status=None,
                          stream=None, planned: bool = False) -> None:
    """In-place SGD on the d cores."""
    ws = _args_d(desc, indices, offsets, num_bags, per_sample_weights, ws, dev_status)
    _need(grad_out, torch.float32, "grad_out")
    _numel(grad_out, desc.num_tables * int(num_bags) * math.prod(desc.q[k] for k in range(desc.d)),
           "grad_out")
    core_ptrs = _cores_d(desc, cores)
    fn = lib().tt_bag_backward_sgd_d_planned if planned else lib().tt_bag_backward_sgd_d
    rc = fn(ctypes.byref(desc), core_ptrs, _ptr(indices),
                                     indices.numel(), _ptr(offsets), int(num_bags),
                                     _ptr(per_sample_weights), _ptr(grad_out), float(lr),
                                     _ptr(ws), ws.numel(), _ptr(dev_status),
                                     _stream(stream, indices))
    _check("tt_bag_backward_sgd_d", rc)


def tt_bag_backward_grad_d(desc: TTDescD, cores, indices, offsets, num_bags: int, grad_out,
                           grad_cores=None, per_sample_weights=None, ws=None, dev_status=None,
                           stream=None, planned: bool = False):
    """Dense gradients with respect to the d cores (fully overwritten); returns them."""
    ws = _args_d(desc, indices, offsets, num_bags, per_sample_weights, ws, dev_status)
    _need(grad_out, torch.float32, "grad_out")
    _numel(grad_out, desc.num_tables * int(num_bags) * math.prod(desc.q[k] for k in range(desc.d)),
           "grad_out")
    if grad_cores is None:
        grad_cores = [torch.empty_like(c) for c in cores]
    core_ptrs = _cores_d(desc, cores)
    grad_ptrs = _cores_d(desc, grad_cores, "grad_cores")
    fn = lib().tt_bag_backward_grad_d_planned if planned else lib().tt_bag_backward_grad_d
    rc = fn(ctypes.byref(desc), core_ptrs, _ptr(indices),
                                      indices.numel(), _ptr(offsets), int(num_bags),
                                      _ptr(per_sample_weights), _ptr(grad_out),
                                      grad_ptrs, _ptr(ws), ws.numel(),
                                      _ptr(dev_status), _stream(stream, indices))
    _check("tt_bag_backward_grad_d", rc)
    return grad_cores


# ------------------------------------------------------------------ prepared calls
# A training loop repeats the same calls with the same buffers: the checks and the
# marshalling of a call can be done once, and the call then replayed with its ctypes
# arguments as they are.  prepare_* validates exactly as the function of the same name
# (without the "prepare_") and returns a zero-argument callable that enqueues the C call
# again (on the same stream, with the same pointers: the buffers' contents may change
# between replays, not their addresses or sizes) and raises TTError on a negative return.

class Prepared:
    __slots__ = ("fn", "args", "name", "keep")

    def __init__(self, name, args, keep):
        self.fn = getattr(lib(), name)
        self.args, self.name, self.keep = args, name, keep

    def __call__(self):
        rc = self.fn(*self.args)
        if rc:
            raise TTError(self.name, rc)


def _stream_handle(stream, like):
    return _stream(stream, like)


def prepare_plan(desc: TTDesc, indices, offsets, num_bags: int, per_sample_weights=None,
                 cache=None, ws=None, dev_status=None, stream=None) -> Prepared:
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    view, _ = _cache_view(cache, desc, indices.numel())
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    args = (ctypes.byref(desc), _ptr(indices), indices.numel(), _ptr(offsets), int(num_bags),
            _ptr(per_sample_weights), None if view is None else ctypes.byref(view), _ptr(ws),
            ws.numel(), _ptr(dev_status), _stream_handle(stream, indices))
    return Prepared("tt_bag_plan", args, (desc, indices, offsets, per_sample_weights, cache, ws,
                                          dev_status, view))


def prepare_forward(desc: TTDesc, cores, indices, offsets, num_bags: int, per_sample_weights=None,
                    cache=None, out=None, ws=None, dev_status=None, stream=None) -> Prepared:
    """The planned forward (tt_bag_forward_planned) as a prepared call."""
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    _need(out, torch.float32, "out")
    _numel(out, desc.num_tables * int(num_bags) * _dim(desc), "out")
    view, _ = _cache_view(cache, desc, indices.numel())
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    core_ptrs = _cores(cores, desc)
    args = (ctypes.byref(desc), core_ptrs, _ptr(indices), indices.numel(), _ptr(offsets),
            int(num_bags), _ptr(per_sample_weights), None if view is None else ctypes.byref(view),
            _ptr(out), _ptr(ws), ws.numel(), _ptr(dev_status), _stream_handle(stream, indices))
    return Prepared("tt_bag_forward_planned", args, (desc, core_ptrs, cores, indices, offsets,
                                                     per_sample_weights, cache, out, ws,
                                                     dev_status, view))


def prepare_plan_dedup(desc: TTDesc, indices, offsets, num_bags: int, per_sample_weights=None,
                       ws=None, dev_status=None, stream=None):
    """tt_bag_plan_dedup as a prepared call.  Returns (call, info): info = the virtual
    batch's bounds (nnz, nnz) that every replay writes, for prepare_backward_dedup."""
    _need(indices, torch.int64, "indices")
    _need(offsets, torch.int64, "offsets")
    if per_sample_weights is not None:
        _need(per_sample_weights, torch.float32, "per_sample_weights")
    _batch_sizes(desc, indices, offsets, num_bags, per_sample_weights)
    _need(ws, torch.uint8, "ws")
    if dev_status is not None:
        _need(dev_status, torch.int32, "dev_status")
    out = (ctypes.c_int64 * 2)()
    args = (ctypes.byref(desc), _ptr(indices), indices.numel(), _ptr(offsets), int(num_bags),
            _ptr(per_sample_weights), _ptr(ws), ws.numel(), _ptr(dev_status), out,
            _stream_handle(stream, indices))
    n = int(indices.numel())
    return (Prepared("tt_bag_plan_dedup", args, (desc, indices, offsets, per_sample_weights, ws,
                                                 dev_status, out)), (n, n))


def prepare_backward_dedup(desc: TTDesc, cores, indices, offsets, num_bags: int, grad_out, info,
                           update: str = "sgd", lr: float = 0.0, aux=None,
                           per_sample_weights=None, ws=None, dev_status=None,
                           stream=None) -> Prepared:
    """The backward over distinct indices as a prepared call: update "sgd"
    (tt_bag_backward_sgd_dedup) or "grad" (aux = the gradient outputs,
    tt_bag_backward_grad_dedup)."""
    _dedup_args(desc, indices, offsets, num_bags, grad_out, per_sample_weights, ws, dev_status)
    core_ptrs = _cores(cores, desc)
    head = (ctypes.byref(desc), core_ptrs, _ptr(indices), indices.numel(), _ptr(offsets),
            int(num_bags), _ptr(per_sample_weights), _ptr(grad_out))
    inf = _info(info)
    tail = (inf, _ptr(ws), ws.numel(), _ptr(dev_status), _stream_handle(stream, indices))
    keep = [desc, core_ptrs, cores, indices, offsets, per_sample_weights, grad_out, ws,
            dev_status, inf]
    if update == "sgd":
        return Prepared("tt_bag_backward_sgd_dedup", head + (float(lr),) + tail, keep)
    if update == "grad":
        gp = _cores(aux, desc, "grad_cores")
        return Prepared("tt_bag_backward_grad_dedup", head + (gp,) + tail, keep + [gp, aux])
    raise ValueError("the backward over distinct indices updates by sgd or grad")


def prepare_backward(desc: TTDesc, cores, indices, offsets, num_bags: int, grad_out,
                     update: str = "sgd", lr: float = 0.0, eps: float = 0.0, aux=None,
                     aux_rows=None, per_sample_weights=None, cache=None, ws=None,
                     dev_status=None, stream=None) -> Prepared:
    """The planned backward as a prepared call: update "sgd" (tt_bag_backward_sgd_planned),
    "adagrad" (aux / aux_rows = running sums) or "grad" (aux / aux_rows = gradient outputs)."""
    view, csize, ws = _batch_args(desc, indices, offsets, num_bags, grad_out, per_sample_weights,
                                  cache, ws, dev_status)
    core_ptrs = _cores(cores, desc)
    head = (ctypes.byref(desc), core_ptrs, _ptr(indices), indices.numel(), _ptr(offsets),
            int(num_bags), _ptr(per_sample_weights), None if view is None else ctypes.byref(view),
            _ptr(grad_out))
    tail = (_ptr(ws), ws.numel(), _ptr(dev_status), _stream_handle(stream, indices))
    keep = [desc, core_ptrs, cores, indices, offsets, per_sample_weights, cache, grad_out, ws,
            dev_status, view]
    if update == "sgd":
        name, mid = "tt_bag_backward_sgd_planned", (float(lr),)
    elif update == "adagrad":
        st = _cores(aux, desc, "state")
        sr = _rows_arg(aux_rows, csize, "state_rows", _dim(desc))
        name, mid = "tt_bag_backward_adagrad_planned", (float(lr), float(eps), st, _ptr(sr))
        keep += [st, aux, sr]
    elif update == "grad":
        gp = _cores(aux, desc, "grad_cores")
        gr = _rows_arg(aux_rows, csize, "grad_rows", _dim(desc))
        name, mid = "tt_bag_backward_grad_planned", (gp, _ptr(gr))
        keep += [gp, aux, gr]
    else:
        raise ValueError("update must be sgd, adagrad or grad")
    return Prepared(name, head + mid + tail, keep)
