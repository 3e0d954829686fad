"""Seeded synthetic workloads for TT-EmbeddingBag (numpy only).

This module draws random inputs and nothing else: it holds none of the method's
arithmetic, so the tests can feed the very same bytes to the HIP path and to the
CPU oracle.  The shapes follow the five workloads the TT-EmbeddingBag pages
describe or imply:

* ``tiny``      p=(4,5,6), q=(2,2,2), ranks=(4,4), 8 bags of 1..4 indices.
* ``readme``    p=(200,220,250), q=(4,4,4), ranks=(32,32), 512 bags of 20
                uniform indices: the shape of the benchmark line in the
                "FBTT-Embedding" README ("Installing FBTT-Embedding").
* ``skewed``    q=(4,8,4), ranks=(64,64), 2048 bags, Poisson(20) lengths
                clipped to >= 1, Zipf(1.1) indices through a random permutation,
                per-sample weights U(0,1).
* ``multitable`` 8 tables of the ``readme`` shape ("TableBatchedTTEmbeddingBag"),
                4096 one-index bags per table, Zipf(1.2) per table.
* ``cached``    the ``readme`` shape, 4096 bags of 20 Zipf(1.2) indices, with an
                HBM cache of 110,000 rows filled from a 10-batch warm-up
                ("Software Cache" section).
* ``readme4``   the ``readme`` table size and batch as four cores p=(10,20,220,250),
                q=(2,2,4,4), ranks=(32,32,32) (the shape lists may have any length).

Seeds: cores come from PCG64(seed); batch k from PCG64(seed*1000 + k); the Zipf
permutation of table t from PCG64(seed*100 + 50 + t).  ``seed`` defaults to the
workload's number (tiny=1 ... cached=5, readme4=6).

Cores are returned in the pages' logical layout ``[R_{k-1}][p_k][q_k][R_k]``
("Initialization" section).  ``slice_major`` reorders one to the
``[p_k][R_{k-1}][q_k][R_k]`` layout the library takes (a pure transpose).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    number: int
    p: tuple
    q: tuple
    ranks: tuple
    num_tables: int
    bags_per_table: int
    lengths: tuple          # ("uniform", lo, hi) | ("fixed", n) | ("poisson", mean)
    dist: tuple             # ("uniform",) | ("zipf", alpha)
    init_std: float
    lr: float
    weighted: bool = False
    cache_size: int = 0
    warmup_batches: int = 0
    hashtbl_size: int = 0
    num_embeddings: Optional[int] = None

    @property
    def E(self) -> int:
        return self.num_embeddings if self.num_embeddings is not None else int(np.prod(self.p))

    @property
    def D(self) -> int:
        return int(np.prod(self.q))


WORKLOADS = {
    "tiny": Workload("tiny", 1, (4, 5, 6), (2, 2, 2), (4, 4), 1, 8,
                     ("uniform", 1, 4), ("uniform",), 0.5, 0.1),
    "readme": Workload("readme", 2, (200, 220, 250), (4, 4, 4), (32, 32), 1, 512,
                       ("fixed", 20), ("uniform",), 1.0 / math.sqrt(32), 0.01),
    "skewed": Workload("skewed", 3, (200, 220, 250), (4, 8, 4), (64, 64), 1, 2048,
                       ("poisson", 20), ("zipf", 1.1), 1.0 / math.sqrt(64), 0.01,
                       weighted=True),
    "multitable": Workload("multitable", 4, (200, 220, 250), (4, 4, 4), (32, 32), 8, 4096,
                           ("fixed", 1), ("zipf", 1.2), 1.0 / math.sqrt(32), 0.01),
    "cached": Workload("cached", 5, (200, 220, 250), (4, 4, 4), (32, 32), 1, 4096,
                       ("fixed", 20), ("zipf", 1.2), 1.0 / math.sqrt(32), 0.01,
                       cache_size=110_000, warmup_batches=10, hashtbl_size=1 << 21),
    # the readme table and batch with E = 11,000,000 split over four cores
    "readme4": Workload("readme4", 6, (10, 20, 220, 250), (2, 2, 4, 4), (32, 32, 32), 1, 512,
                        ("fixed", 20), ("uniform",), 1.0 / math.sqrt(32), 0.01),
}


def custom(name="custom", p=(4, 5, 6), q=(2, 2, 2), ranks=(4, 4), num_tables=1,
           bags_per_table=8, lengths=("uniform", 1, 4), dist=("uniform",),
           init_std=0.5, lr=0.1, weighted=False, num_embeddings=None, number=9,
           cache_size=0, hashtbl_size=0) -> Workload:
    """A workload of any shape (small parity cases, edge cases)."""
    return Workload(name, number, tuple(p), tuple(q), tuple(ranks), num_tables,
                    bags_per_table, tuple(lengths), tuple(dist), init_std, lr,
                    weighted, cache_size, 0, hashtbl_size, num_embeddings)


def core_shapes(wl: Workload):
    """Logical core shapes [R_{k-1}, p_k, q_k, R_k] with ranks [1]+ranks+[1]."""
    full = (1,) + tuple(wl.ranks) + (1,)
    return [(full[k], wl.p[k], wl.q[k], full[k + 1]) for k in range(len(wl.p))]


def make_cores(wl: Workload, seed: Optional[int] = None):
    """T lists of three fp32 cores, i.i.d. N(0, init_std), logical layout."""
    seed = wl.number if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(wl.num_tables):
        out.append([(rng.standard_normal(s, dtype=np.float64) * wl.init_std).astype(np.float32)
                    for s in core_shapes(wl)])
    return out


def slice_major(core: np.ndarray) -> np.ndarray:
    """[R_{k-1}][p_k][q_k][R_k] -> contiguous [p_k][R_{k-1}][q_k][R_k]."""
    return np.ascontiguousarray(core.transpose(1, 0, 2, 3))


def logical(core_sm: np.ndarray, shape) -> np.ndarray:
    """Inverse of slice_major: [p_k][R_{k-1}][q_k][R_k] -> logical layout."""
    ra, pk, qk, rb = shape
    return np.ascontiguousarray(core_sm.reshape(pk, ra, qk, rb).transpose(1, 0, 2, 3))


_ZIPF_CACHE: dict = {}


def _zipf_cdf(E: int, alpha: float) -> np.ndarray:
    key = (E, alpha)
    if key not in _ZIPF_CACHE:
        k = np.arange(1, E + 1, dtype=np.float64)
        w = np.power(k, -alpha)
        c = np.cumsum(w)
        _ZIPF_CACHE[key] = c / c[-1]
    return _ZIPF_CACHE[key]


_PERM_CACHE: dict = {}


def _zipf_perm(wl: Workload, seed: int, t: int) -> np.ndarray:
    key = (wl.E, seed, t)
    if key not in _PERM_CACHE:
        rng = np.random.Generator(np.random.PCG64(seed * 100 + 50 + t))
        _PERM_CACHE[key] = rng.permutation(wl.E).astype(np.int64)
    return _PERM_CACHE[key]


def _lengths(wl: Workload, rng, nbags: int) -> np.ndarray:
    kind = wl.lengths[0]
    if kind == "fixed":
        return np.full(nbags, wl.lengths[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(wl.lengths[1], wl.lengths[2] + 1, size=nbags).astype(np.int64)
    if kind == "poisson":
        return np.maximum(1, rng.poisson(wl.lengths[1], size=nbags)).astype(np.int64)
    if kind == "list":
        return np.asarray(wl.lengths[1], dtype=np.int64)
    raise ValueError(kind)


def _draw_indices(wl: Workload, rng, n: int, seed: int, t: int) -> np.ndarray:
    if wl.dist[0] == "uniform":
        return rng.integers(0, wl.E, size=n).astype(np.int64)
    if wl.dist[0] == "zipf":
        cdf = _zipf_cdf(wl.E, float(wl.dist[1]))
        u = rng.random(n)
        rank = np.minimum(np.searchsorted(cdf, u, side="right"), wl.E - 1)
        return _zipf_perm(wl, seed, t)[rank]
    raise ValueError(wl.dist)


def make_batch(wl: Workload, k: int = 0, seed: Optional[int] = None, bags_per_table=None):
    """One batch: indices (int64), offsets (int64, T*B+1 entries, CSR with the
    terminal entry), per-sample weights (fp32 or None) and the upstream gradient
    dY (fp32 [T*B][D]).  Bags are table-major."""
    seed = wl.number if seed is None else seed
    B = wl.bags_per_table if bags_per_table is None else bags_per_table
    rng = np.random.Generator(np.random.PCG64(seed * 1000 + k))
    idx_parts, len_parts = [], []
    for t in range(wl.num_tables):
        lens = _lengths(wl, rng, B)
        len_parts.append(lens)
        idx_parts.append(_draw_indices(wl, rng, int(lens.sum()), seed, t))
    lens = np.concatenate(len_parts)
    offsets = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=offsets[1:])
    indices = np.concatenate(idx_parts).astype(np.int64)
    psw = rng.random(len(indices)).astype(np.float32) if wl.weighted else None
    dY = rng.standard_normal((wl.num_tables * B, wl.D)).astype(np.float32)
    return dict(indices=indices, offsets=offsets, per_sample_weights=psw, grad_out=dY,
                num_bags=B)
