"""Drop-in PyTorch modules over the C ABI: ``TTEmbeddingBag`` and
``TableBatchedTTEmbeddingBag``.

"FBTT-Embedding" README, "Parameters" / "Initialization" / "Fused Kernel" / "Software
Cache" / "TableBatchedTTEmbeddingBag": an EmbeddingBag whose table is held as three TT
cores, built like PyTorch's EmbeddingBag (``module(input, offsets)``), with
``sparse=True`` updating the cores inside the backward pass (SGD or Adagrad) instead of
returning gradients, ``sparse=False`` returning the gradient with respect to the cores
(and the cache rows) to an external optimizer, an optional cache of decompressed rows
refreshed by ``cache_populate()``, and several tables of one shape in one module.

Argument marshalling only: the cores live in the library's layout (core k of all tables
as one flat fp32 parameter, each table slice-major [p_k][R_{k-1}][q_k][R_k]); offsets
given in PyTorch's form (one start per bag) get their terminal entry appended; every
step of the computation runs in libttbag.
"""
from __future__ import annotations

import enum
import math
from typing import Optional, Sequence

import torch

from . import abi


class OptimType(enum.Enum):
    """Optimizer of the fused backward ("Parameters": `optimizer`)."""
    SGD = "sgd"
    ADAGRAD = "adagrad"


_DIST = {"uniform": abi.TT_INIT_UNIFORM, "naive-uniform": abi.TT_INIT_UNIFORM,
         "normal": abi.TT_INIT_NORMAL, "approx-uniform": abi.TT_INIT_APPROX_UNIFORM,
         "approx-normal": abi.TT_INIT_APPROX_NORMAL}


class _TTBagFunction(torch.autograd.Function):
    """Forward: grouping (tt_bag_plan) + planned forward.  Backward: the planned backward
    on the same grouping -- fused update (no gradient returned) or core gradients."""

    @staticmethod
    def forward(ctx, mod, indices, offsets, psw, *params):
        ws, cache = mod._plan(indices, offsets, psw)
        out = abi.tt_bag_forward(mod.desc, mod._cores(), indices, offsets, mod.num_bags, psw,
                                 cache=cache, ws=ws, dev_status=mod.dev_status, planned=True)
        ctx.mod, ctx.ws, ctx.cache = mod, ws, cache
        ctx.inputs = (indices, offsets, psw)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        mod, ws, cache = ctx.mod, ctx.ws, ctx.cache
        indices, offsets, psw = ctx.inputs
        g = grad_out.contiguous()
        cores = mod._cores()
        # dL/dw of the per-sample weights, at the cores of the forward (before any update)
        gw = None
        if psw is not None and ctx.needs_input_grad[3]:
            gw = abi.tt_bag_weight_grad(mod.desc, cores, indices, offsets, mod.num_bags, g,
                                        per_sample_weights=psw, cache=cache, ws=ws,
                                        dev_status=mod.dev_status, planned=True)
        none = (None, None, None, gw)
        if mod.sparse:
            if mod.optimizer == OptimType.ADAGRAD:
                abi.tt_bag_backward_adagrad(mod.desc, cores, indices, offsets, mod.num_bags, g,
                                            mod.learning_rate, mod.eps, mod._state,
                                            state_rows=mod._state_rows, per_sample_weights=psw,
                                            cache=cache, ws=ws, dev_status=mod.dev_status,
                                            planned=True)
            else:
                abi.tt_bag_backward_sgd(mod.desc, cores, indices, offsets, mod.num_bags, g,
                                        mod.learning_rate, per_sample_weights=psw, cache=cache,
                                        ws=ws, dev_status=mod.dev_status, planned=True)
            return none + (None,) * len(mod._param_list())
        grads, grad_rows = abi.tt_bag_backward_grad(mod.desc, cores, indices, offsets,
                                                    mod.num_bags, g, per_sample_weights=psw,
                                                    cache=cache, ws=ws,
                                                    dev_status=mod.dev_status, planned=True)
        extra = (grad_rows,) if mod.use_cache else ()
        return none + tuple(grads) + extra


class TableBatchedTTEmbeddingBag(torch.nn.Module):
    """num_tables TT tables of one shape in one module ("TableBatchedTTEmbeddingBag").

    forward(input, offsets, per_sample_weights=None): input holds the indices of table 0's
    bags, then table 1's, ...; offsets the starts of all num_tables * B bags (table-major;
    with or without the terminal entry, see include_last_offset).  Returns
    [num_tables * B, embedding_dim].  mode: "sum" or "mean"."""

    def __init__(self, num_tables: int, num_embeddings: int, embedding_dim: int,
                 tt_p_shapes: Optional[Sequence[int]] = None,
                 tt_q_shapes: Optional[Sequence[int]] = None,
                 tt_ranks: Sequence[int] = (8, 8), sparse: bool = False,
                 optimizer: OptimType = OptimType.SGD, learning_rate: float = 0.1,
                 eps: float = 1.0e-10, use_cache: bool = False, cache_size: int = 0,
                 hashtbl_size: int = 0, weight_dist: str = "approx-normal",
                 init_scale: Optional[float] = None, mode: str = "sum",
                 include_last_offset: bool = False, seed: int = 0, device=None):
        super().__init__()
        if mode not in ("sum", "mean"):
            raise ValueError("mode must be 'sum' or 'mean'")
        if weight_dist not in _DIST:
            raise ValueError("weight_dist must be one of %s" % sorted(_DIST))
        if use_cache and num_tables != 1:
            raise ValueError("the cache serves a single table")
        if len(tt_ranks) != 2:
            raise ValueError("three cores: tt_ranks has two entries")
        p = tuple(tt_p_shapes) if tt_p_shapes is not None else abi.tt_factorize(num_embeddings,
                                                                                False)
        q = tuple(tt_q_shapes) if tt_q_shapes is not None else abi.tt_factorize(embedding_dim,
                                                                                True)
        if math.prod(q) != embedding_dim or math.prod(p) < num_embeddings:
            raise ValueError("prod(tt_q_shapes) must equal embedding_dim and prod(tt_p_shapes) "
                             "must be >= num_embeddings")
        self.num_tables, self.num_embeddings, self.embedding_dim = num_tables, num_embeddings, \
            embedding_dim
        self.tt_p_shapes, self.tt_q_shapes, self.tt_ranks = p, q, tuple(tt_ranks)
        self.sparse, self.optimizer = sparse, optimizer
        self.learning_rate, self.eps = float(learning_rate), float(eps)
        self.use_cache, self.mode, self.include_last_offset = use_cache, mode, include_last_offset
        self.desc = abi.make_desc(p, q, tt_ranks, num_embeddings, num_tables=num_tables,
                                  pooling=abi.TT_POOL_MEAN if mode == "mean" else abi.TT_POOL_SUM)
        dev = torch.device(device) if device is not None else torch.device("cuda")
        n = abi._core_numels(self.desc)
        self.cores = torch.nn.ParameterList(
            [torch.nn.Parameter(torch.empty(n[k], dtype=torch.float32, device=dev))
             for k in range(3)])
        # "Initialization": i.i.d. cores, or cores whose full table follows weight_dist;
        # the default scale puts the table's entries at standard deviation 1/sqrt(D)
        scale = init_scale if init_scale is not None else 1.0 / math.sqrt(embedding_dim)
        with torch.no_grad():
            abi.tt_init_cores(self.desc, [c.data for c in self.cores], _DIST[weight_dist], scale,
                              seed)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=dev)
        self._state = self._state_rows = None
        if sparse and optimizer == OptimType.ADAGRAD:
            self._state = [torch.zeros_like(c.data) for c in self.cores]
        self.cache = self.cache_rows = None
        if use_cache:
            if cache_size < 1 or hashtbl_size < 1:
                raise ValueError("use_cache needs cache_size >= 1 and hashtbl_size >= 1")
            self.cache = abi.Cache(self.desc, cache_size, hashtbl_size)
            self.cache_rows = torch.nn.Parameter(torch.zeros(cache_size, embedding_dim,
                                                             dtype=torch.float32, device=dev))
            self._slots = None
            if self._state is not None:
                self._state_rows = torch.zeros_like(self.cache_rows.data)
        self._ws = None
        self.num_bags = 0

    # ---------------------------------------------------------------- marshalling
    def _cores(self):
        return [c.data for c in self.cores]

    def _param_list(self):
        return list(self.cores) + ([self.cache_rows] if self.use_cache else [])

    def _workspace(self, nnz: int, num_bags: int):
        csize = self.cache.cache_size if self.use_cache else 0
        need = abi.tt_bag_workspace_size(self.desc, nnz, num_bags, csize)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.dev_status.device)
        return self._ws

    def _plan(self, indices, offsets, psw):
        ws = self._workspace(indices.numel(), self.num_bags)
        cache = None
        if self.use_cache:
            if self._slots is None or self._slots.numel() != indices.numel():
                self._slots = torch.empty(indices.numel(), dtype=torch.int32,
                                          device=indices.device)
            # "Software Cache": every lookup counts the frequencies; before the first
            # cache_populate() no row is cached and every index is a miss
            self.cache.lookup(indices, slot_out=self._slots, count_freq=True,
                              dev_status=self.dev_status)
            cache = (self._slots, self.cache_rows.data)
        abi.tt_bag_plan(self.desc, indices, offsets, self.num_bags, psw, cache=cache, ws=ws,
                        dev_status=self.dev_status)
        return ws, cache

    def forward(self, input: torch.Tensor, offsets: torch.Tensor,
                per_sample_weights: Optional[torch.Tensor] = None) -> torch.Tensor:
        indices = input.to(torch.int64).contiguous()
        offsets = offsets.to(torch.int64).contiguous()
        if not self.include_last_offset:  # PyTorch form: one start per bag
            offsets = torch.cat([offsets, offsets.new_full((1,), indices.numel())])
        nb = offsets.numel() - 1
        if nb % self.num_tables:
            raise ValueError("the number of bags must be a multiple of num_tables")
        self.num_bags = nb // self.num_tables
        psw = None if per_sample_weights is None else \
            per_sample_weights.to(torch.float32).contiguous()
        return _TTBagFunction.apply(self, indices, offsets, psw, *self._param_list())

    def check_status(self) -> None:
        """Raise if a device-side content error (bad index, bad offsets, ...) was reported
        since the module was built (synchronises the device)."""
        st = int(self.dev_status.item())
        if st:
            raise RuntimeError("libttbag reported device status 0x%x (see tt_bag.h)" % st)

    # ---------------------------------------------------------------- cache and weights
    def cache_populate(self) -> int:
        """Refill the cache from the counted frequencies, rows from the current cores
        ("Software Cache"); returns the number of rows filled."""
        if not self.use_cache:
            raise RuntimeError("this module has no cache")
        with torch.no_grad():
            return self.cache.populate(self._cores(), self.cache_rows.data)

    def full_weight(self, table: int = 0, first: int = 0,
                    count: Optional[int] = None) -> torch.Tensor:
        """Rows [first, first + count) of one table, decompressed from the cores."""
        count = self.num_embeddings - first if count is None else count
        with torch.no_grad():
            return abi.tt_full_weight(self.desc, self._cores(), first, count, table=table)


class TTEmbeddingBag(TableBatchedTTEmbeddingBag):
    """One TT table ("Parameters", "Initialization"): TTEmbeddingBag(num_embeddings,
    embedding_dim, tt_p_shapes, tt_q_shapes, tt_ranks, sparse, optimizer, learning_rate,
    eps, use_cache, cache_size, hashtbl_size, weight_dist, ...)."""

    def __init__(self, num_embeddings: int, embedding_dim: int,
                 tt_p_shapes: Optional[Sequence[int]] = None,
                 tt_q_shapes: Optional[Sequence[int]] = None,
                 tt_ranks: Sequence[int] = (8, 8), sparse: bool = False,
                 optimizer: OptimType = OptimType.SGD, learning_rate: float = 0.1,
                 eps: float = 1.0e-10, use_cache: bool = False, cache_size: int = 0,
                 hashtbl_size: int = 0, weight_dist: str = "approx-normal", **kw):
        super().__init__(1, num_embeddings, embedding_dim, tt_p_shapes, tt_q_shapes, tt_ranks,
                         sparse, optimizer, learning_rate, eps, use_cache, cache_size,
                         hashtbl_size, weight_dist, **kw)
