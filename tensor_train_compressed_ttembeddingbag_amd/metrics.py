"""Work counts used by the benchmark (host logic, no GPU).

Per looked-up row the TT chain is two small GEMMs ("FBTT-Embedding" README,
"Software Cache" section): stage 1 multiplies the q1 x R1 slice of core 1 by the
R1 x (q2 R2) slice of core 2, stage 2 multiplies the resulting (q1 q2) x R2 matrix
by the R2 x q3 slice of core 3.  The backward pass is the same chain in reverse:
two GEMMs of each size.  Hence per element

    F1 = 2 q1 R1 q2 R2,   F2 = 2 q1 q2 R2 q3,   fwd = F1 + F2,   fwd+bwd = 3 (F1 + F2).

The README's benchmark line reports GFLOPS and time per nnz whose product is
30 (F1 + F2) per nnz, i.e. the fwd+bwd count times 10; this module counts one
fwd+bwd pass (3 (F1 + F2)) per element and says so.
"""
from __future__ import annotations

import numpy as np


def stage_flops(q, ranks):
    q1, q2, q3 = (int(x) for x in q)
    r1, r2 = (int(x) for x in ranks)
    return 2 * q1 * r1 * q2 * r2, 2 * q1 * q2 * r2 * q3


def fwd_flops_per_nnz(q, ranks) -> int:
    f1, f2 = stage_flops(q, ranks)
    return f1 + f2


def step_flops_per_nnz(q, ranks) -> int:
    """fwd + bwd flops per element, no reuse of shared stage-1 products."""
    return 3 * fwd_flops_per_nnz(q, ranks)


def unique_pairs(p, num_tables, num_bags, indices, offsets, slots=None, E=None) -> int:
    """Number of distinct (table, i1, i2) among the elements that take the TT
    path (cache misses): the count of stage-1 products a reuse-aware kernel forms."""
    idx = np.asarray(indices, dtype=np.int64)
    off = np.asarray(offsets, dtype=np.int64)
    bag = np.searchsorted(off, np.arange(len(idx)), side="right") - 1
    t = bag // num_bags
    keep = np.ones(len(idx), dtype=bool)
    if slots is not None:
        keep &= np.asarray(slots) < 0
    if E is not None:
        keep &= (idx >= 0) & (idx < E)
    pair = (t[keep] * p[1] + (idx[keep] // p[2]) % p[1]) * p[0] + idx[keep] // (p[1] * p[2])
    return int(np.unique(pair).size)


def bwd_kernel_flops(q, ranks, n_miss: int, n_pairs: int) -> int:
    """Algorithmic flops of the backward contraction: 2 F1 per distinct stage-1
    product (gradients of the core-1 and core-2 slices) + 2 F2 per element
    (gradient of the stage-1 product and of the core-3 slice)."""
    f1, f2 = stage_flops(q, ranks)
    return 2 * f1 * n_pairs + 2 * f2 * n_miss


def fwd_kernel_flops(q, ranks, n_miss: int, n_pairs: int) -> int:
    """Algorithmic flops of the forward contraction: F1 per distinct stage-1
    product + F2 per element."""
    f1, f2 = stage_flops(q, ranks)
    return f1 * n_pairs + f2 * n_miss


def route_bytes(nnz: float, num_bags: int, weighted: bool, has_cache: bool) -> float:
    """Algorithmic bytes of one grouping call: every input read once (int64 index,
    int64 offset per bag, fp32 weight, int32 cache slot) and the grouped order written
    once (32 bytes per position: element, three digits, bag, two segment positions,
    weight)."""
    per = 8 + (4 if weighted else 0) + (4 if has_cache else 0) + 32
    return nnz * per + 8.0 * (num_bags + 1)
