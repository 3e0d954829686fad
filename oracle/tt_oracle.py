"""CPU oracle for TT-EmbeddingBag -- TEST INFRASTRUCTURE ONLY.

Floating-point side: ``tt_oracle.c`` (plain double loops over the definition of
the TT table, EmbeddingBag pooling, the product-rule backward, plain SGD and
Adagrad),
loaded here through ctypes.  Integer side (index split, bag ids, the grouping
order, cache frequency counts, top-K selection, the set-associative LFU populate,
slot lookup): plain numpy / dict code in this file.

Pages followed ("FBTT-Embedding" README unless stated):
  * "Initialization": core shapes R_{k-1} x p_k x q_k x R_k, ranks [1]+tt_ranks+[1].
  * "Parameters": prod(p) >= num_embeddings, prod(q) == embedding_dim; `sparse`
    fuses the weight update into the backward pass.
  * README intro + "EmbeddingBag and Product-Key Memory Layers" (tensorflow/addons
    #2201): EmbeddingBag = gather + (weighted) sum per bag.
  * "Software Cache": hits read decompressed rows; the frequency of every lookup
    is counted and the cache is (re)filled from the most frequent rows on
    `cache_populate()`, each row initialised from the TT cores.
  * "TableBatchedTTEmbeddingBag": T tables of one shape in one call.
  * "Parameters": the shape lists have one length d (any number of cores); the
    d-core functions (``*_d``) take the row as the product of the d slice matrices.

Readings where the pages are silent: row-major mixed radix for the index split;
offsets carry a terminal entry; duplicates sum; the cache is filled with the K
most frequent indices, ties broken by the smaller index, slot = rank in that
order; one count per occurrence.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tt_oracle.c")
_SO = os.path.join(_HERE, "libtt_oracle.so")

__all__ = ["build", "forward", "backward", "sgd", "adagrad", "tt_row", "split_index", "bag_ids",
           "route_order", "group_counts", "count_frequencies", "select_cache",
           "lookup_slots", "populate_rows", "splitmix64", "lfu_set", "lfu_populate", "LFU_WAYS",
           "philox4x32_10", "init_param", "init_core", "factorize", "tt_row_d", "forward_d",
           "backward_d", "sgd_d", "MAX_D"]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Shape(ctypes.Structure):
    _fields_ = [("num_tables", ctypes.c_int32), ("num_embeddings", ctypes.c_int64),
                ("p", ctypes.c_int32 * 3), ("q", ctypes.c_int32 * 3),
                ("r", ctypes.c_int32 * 2), ("pooling", ctypes.c_int32)]


_lib = None


def _L():
    global _lib
    if _lib is None:
        # TT_ORACLE_LIB: a build of the same source to load instead (the sanitizer test
        # runs the pins against an -fsanitize=address,undefined build this way)
        lib = ctypes.CDLL(os.environ.get("TT_ORACLE_LIB") or build())
        P = ctypes.c_void_p
        lib.oracle_forward.argtypes = [P, P, P, ctypes.c_int64, P, ctypes.c_int64, P, P, P,
                                       ctypes.c_int64, P]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_backward.argtypes = [P, P, P, ctypes.c_int64, P, ctypes.c_int64, P, P,
                                        ctypes.c_int64, P, P, P, P, P, P, P]
        lib.oracle_backward.restype = ctypes.c_int
        lib.oracle_sgd_core.argtypes = [P, ctypes.c_int, P, P, P, ctypes.c_double]
        lib.oracle_sgd_rows.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_double]
        lib.oracle_adagrad_core.argtypes = [P, ctypes.c_int, P, P, P, P, ctypes.c_double,
                                            ctypes.c_double]
        lib.oracle_adagrad_rows.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_double, ctypes.c_double]
        lib.oracle_tt_row.argtypes = [P, P, P, P, ctypes.c_int64, P]
        lib.oracle_forward_d.argtypes = [P, P, P, ctypes.c_int64, P, ctypes.c_int64, P, P]
        lib.oracle_forward_d.restype = ctypes.c_int
        lib.oracle_backward_d.argtypes = [P, P, P, ctypes.c_int64, P, ctypes.c_int64, P, P, P,
                                          P]
        lib.oracle_backward_d.restype = ctypes.c_int
        lib.oracle_tt_row_d.argtypes = [P, P, ctypes.c_int64, P]
        _lib = lib
    return _lib


MAX_D = 8


class _ShapeD(ctypes.Structure):
    _fields_ = [("num_tables", ctypes.c_int32), ("d", ctypes.c_int32),
                ("num_embeddings", ctypes.c_int64), ("p", ctypes.c_int32 * MAX_D),
                ("q", ctypes.c_int32 * MAX_D), ("r", ctypes.c_int32 * (MAX_D - 1)),
                ("pooling", ctypes.c_int32)]


def _shape_d(p, q, ranks, E, T, pooling=0):
    d = len(p)
    if not (1 <= d <= MAX_D and len(q) == d and len(ranks) == d - 1):
        raise ValueError("d-core shape: len(p) == len(q) == len(ranks) + 1 <= %d" % MAX_D)
    s = _ShapeD()
    s.num_tables, s.d, s.num_embeddings, s.pooling = int(T), d, int(E), int(pooling)
    for k in range(d):
        s.p[k], s.q[k] = int(p[k]), int(q[k])
    for k in range(d - 1):
        s.r[k] = int(ranks[k])
    return s


def tt_row_d(p, q, ranks, cores, i: int) -> np.ndarray:
    """One row W[i, :] (float64) of a single d-core table (cores in the logical layout)."""
    c = [_f32(x) for x in cores]
    s = _shape_d(p, q, ranks, int(np.prod(p)), 1)
    out = np.zeros(int(np.prod(q)), dtype=np.float64)
    _L().oracle_tt_row_d(ctypes.byref(s), _ptr_array(c), int(i), _ptr(out))
    return out


def forward_d(p, q, ranks, E, cores, indices, offsets, num_bags, per_sample_weights=None,
              pooling=0):
    """EmbeddingBag forward over d-core TT tables (d = len(p)); cores: T lists of d
    arrays in the logical layout [R_{k-1}][p_k][q_k][R_k].  Returns Y float64."""
    T = len(cores)
    flat = [_f32(c) for tbl in cores for c in tbl]
    s = _shape_d(p, q, ranks, E, T, pooling)
    idx = np.ascontiguousarray(indices, dtype=np.int64)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    psw = None if per_sample_weights is None else _f32(per_sample_weights)
    Y = np.zeros((T * num_bags, int(np.prod(q))), dtype=np.float64)
    rc = _L().oracle_forward_d(ctypes.byref(s), _ptr_array(flat), _ptr(idx), len(idx),
                               _ptr(off), int(num_bags), _ptr(psw), _ptr(Y))
    if rc != 0:
        raise ValueError("oracle_forward_d: invalid input")
    return Y


def backward_d(p, q, ranks, E, cores, indices, offsets, num_bags, grad_out,
               per_sample_weights=None, pooling=0):
    """Core gradients of L = sum_b <dY[b], Y[b]> for d-core tables: (grads, touched),
    T lists of d float64 arrays (logical layout) and of d uint8 slice masks."""
    T, d = len(cores), len(p)
    flat = [_f32(c) for tbl in cores for c in tbl]
    s = _shape_d(p, q, ranks, E, T, pooling)
    idx = np.ascontiguousarray(indices, dtype=np.int64)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    psw = None if per_sample_weights is None else _f32(per_sample_weights)
    dY = _f32(grad_out)
    grads = [[np.zeros(c.shape, dtype=np.float64) for c in tbl] for tbl in cores]
    touched = [[np.zeros(p[k], dtype=np.uint8) for k in range(d)] for _ in cores]
    rc = _L().oracle_backward_d(ctypes.byref(s), _ptr_array(flat), _ptr(idx), len(idx),
                                _ptr(off), int(num_bags), _ptr(psw), _ptr(dY),
                                _ptr_array([g for tbl in grads for g in tbl]),
                                _ptr_array([m for tbl in touched for m in tbl]))
    if rc != 0:
        raise ValueError("oracle_backward_d: invalid input")
    return grads, touched


def sgd_d(cores, grads, touched, lr):
    """Plain SGD on the touched slices of d-core tables, in fp64, rounded to fp32:
    G <- fp32(double(G) - lr * dG); untouched slices keep their bits."""
    out = []
    for tbl, gt, mt in zip(cores, grads, touched):
        row = []
        for c, g, m in zip(tbl, gt, mt):
            new = np.array(c, dtype=np.float32, copy=True)
            upd = (c.astype(np.float64) - float(lr) * g).astype(np.float32)
            sel = m.astype(bool)
            new[:, sel] = upd[:, sel]
            row.append(new)
        out.append(row)
    return out


def _shape(p, q, ranks, E, T, pooling=0):
    s = _Shape()
    s.pooling = int(pooling)
    s.num_tables = int(T)
    s.num_embeddings = int(E)
    for k in range(3):
        s.p[k] = int(p[k])
        s.q[k] = int(q[k])
    s.r[0], s.r[1] = int(ranks[0]), int(ranks[1])
    return s


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr_array(arrs):
    arr = (ctypes.c_void_p * len(arrs))()
    for i, a in enumerate(arrs):
        arr[i] = a.ctypes.data
    return arr


def tt_row(p, q, ranks, cores3, i: int) -> np.ndarray:
    """One row W[i, :] (float64) of a single table, straight from the definition."""
    c = [_f32(x) for x in cores3]
    s = _shape(p, q, ranks, int(np.prod(p)), 1)
    out = np.zeros(int(np.prod(q)), dtype=np.float64)
    _L().oracle_tt_row(ctypes.byref(s), _ptr(c[0]), _ptr(c[1]), _ptr(c[2]), int(i), _ptr(out))
    return out


def forward(p, q, ranks, E, cores, indices, offsets, num_bags, per_sample_weights=None,
            slots=None, cache_rows=None, pooling=0):
    """EmbeddingBag forward over the implicit TT table(s).

    cores: list of T lists [G1, G2, G3] in the logical layout; pooling 0 = sum,
    1 = mean.  Returns Y as float64 [T*num_bags, D]."""
    T = len(cores)
    flat = [_f32(c) for tbl in cores for c in tbl]
    s = _shape(p, q, ranks, E, T, pooling)
    idx = np.ascontiguousarray(indices, dtype=np.int64)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    psw = None if per_sample_weights is None else _f32(per_sample_weights)
    sl = None if slots is None else np.ascontiguousarray(slots, dtype=np.int32)
    cr = None if cache_rows is None else _f32(cache_rows)
    csize = 0 if cr is None else cr.shape[0]
    D = int(np.prod(q))
    Y = np.zeros((T * num_bags, D), dtype=np.float64)
    rc = _L().oracle_forward(ctypes.byref(s), _ptr_array(flat), _ptr(idx), len(idx), _ptr(off),
                             int(num_bags), _ptr(psw), _ptr(sl), _ptr(cr), csize, _ptr(Y))
    if rc != 0:
        raise ValueError("oracle_forward: invalid input")
    return Y


def backward(p, q, ranks, E, cores, indices, offsets, num_bags, grad_out,
             per_sample_weights=None, slots=None, cache_size=0, pooling=0, cache_rows=None,
             weight_grad=False):
    """Gradients of L = sum_b <dY[b], Y[b]>.

    Returns (grads, touched, grad_cache, touched_cache): grads is a list of T lists
    of float64 arrays in the logical core layout, touched a list of T lists of
    uint8 masks over the slices p_k.  weight_grad=True appends dL/dw per element."""
    T = len(cores)
    flat = [_f32(c) for tbl in cores for c in tbl]
    s = _shape(p, q, ranks, E, T, pooling)
    idx = np.ascontiguousarray(indices, dtype=np.int64)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    psw = None if per_sample_weights is None else _f32(per_sample_weights)
    sl = None if slots is None else np.ascontiguousarray(slots, dtype=np.int32)
    dY = _f32(grad_out)
    grads = [[np.zeros(c.shape, dtype=np.float64) for c in tbl] for tbl in cores]
    touched = [[np.zeros(p[k], dtype=np.uint8) for k in range(3)] for _ in cores]
    D = int(np.prod(q))
    gc = np.zeros((cache_size, D), dtype=np.float64) if sl is not None else None
    tc = np.zeros(cache_size, dtype=np.uint8) if sl is not None else None
    gw = np.zeros(len(idx), dtype=np.float64) if weight_grad else None
    cr = None if cache_rows is None else _f32(cache_rows)
    if weight_grad and sl is not None and cr is None:
        raise ValueError("the weight gradient of cache hits needs the cache rows")
    rc = _L().oracle_backward(ctypes.byref(s), _ptr_array(flat), _ptr(idx), len(idx), _ptr(off),
                              int(num_bags), _ptr(psw), _ptr(sl), int(cache_size), _ptr(dY),
                              _ptr_array([g for tbl in grads for g in tbl]),
                              _ptr_array([m for tbl in touched for m in tbl]),
                              _ptr(gc), _ptr(tc), _ptr(gw), _ptr(cr))
    if rc != 0:
        raise ValueError("oracle_backward: invalid input")
    if weight_grad:
        return grads, touched, gc, tc, gw
    return grads, touched, gc, tc


def sgd(p, q, ranks, E, cores, grads, touched, lr, cache_rows=None, grad_cache=None,
        touched_cache=None):
    """Plain SGD on touched slices (copies): returns (new_cores, new_cache_rows)."""
    T = len(cores)
    s = _shape(p, q, ranks, E, T)
    new = [[_f32(c).copy() for c in tbl] for tbl in cores]
    for t in range(T):
        for k in range(3):
            _L().oracle_sgd_core(ctypes.byref(s), k, _ptr(new[t][k]),
                                 _ptr(np.ascontiguousarray(grads[t][k])),
                                 _ptr(np.ascontiguousarray(touched[t][k])), float(lr))
    rows = None
    if cache_rows is not None:
        rows = _f32(cache_rows).copy()
        _L().oracle_sgd_rows(_ptr(rows), _ptr(np.ascontiguousarray(grad_cache)),
                             _ptr(np.ascontiguousarray(touched_cache)), rows.shape[0],
                             rows.shape[1], float(lr))
    return new, rows


def adagrad(p, q, ranks, E, cores, states, grads, touched, lr, eps, cache_rows=None,
            cache_state=None, grad_cache=None, touched_cache=None):
    """Diagonal Adagrad on touched slices (copies): per parameter, S += g^2 and
    x -= lr * g / (sqrt(S) + eps).  states: T lists of fp32 arrays shaped like the
    cores.  Returns (new_cores, new_states, new_cache_rows, new_cache_state)."""
    T = len(cores)
    s = _shape(p, q, ranks, E, T)
    new = [[_f32(c).copy() for c in tbl] for tbl in cores]
    st = [[_f32(c).copy() for c in tbl] for tbl in states]
    for t in range(T):
        for k in range(3):
            _L().oracle_adagrad_core(ctypes.byref(s), k, _ptr(new[t][k]), _ptr(st[t][k]),
                                     _ptr(np.ascontiguousarray(grads[t][k])),
                                     _ptr(np.ascontiguousarray(touched[t][k])), float(lr),
                                     float(eps))
    rows = rst = None
    if cache_rows is not None:
        rows = _f32(cache_rows).copy()
        rst = _f32(cache_state).copy()
        _L().oracle_adagrad_rows(_ptr(rows), _ptr(rst), _ptr(np.ascontiguousarray(grad_cache)),
                                 _ptr(np.ascontiguousarray(touched_cache)), rows.shape[0],
                                 rows.shape[1], float(lr), float(eps))
    return new, st, rows, rst


# ---------------------------------------------------------------- integer side

def split_index(p, indices):
    """Row-major mixed-radix split i -> (i1, i2, i3) by div/mod."""
    i = np.asarray(indices, dtype=np.int64)
    return i // (p[1] * p[2]), (i // p[2]) % p[1], i % p[2]


def bag_ids(offsets, nnz):
    """bag(n) = upper_bound(offsets, n) - 1 over the CSR offsets."""
    return np.searchsorted(np.asarray(offsets, dtype=np.int64), np.arange(nnz), side="right") - 1


def route_order(p, E, num_tables, num_bags, indices, offsets, slots=None):
    """The grouping order of the elements, as a plain stable sort.

    Misses (no cache slot) first, ordered by (table, i2, i1) and, for equal
    keys, by position n; then cache hits ordered by (slot, n).  Elements with an index
    outside [0, E) are left out.  Returns (order, group_counts) where
    group_counts[t*p2 + i2] counts the misses of each (table, i2) group."""
    idx = np.asarray(indices, dtype=np.int64)
    nnz = len(idx)
    b = bag_ids(offsets, nnz)
    t = b // num_bags
    i1, i2, i3 = split_index(p, idx)
    keys_miss, keys_hit = [], []
    for n in range(nnz):
        hit = slots is not None and slots[n] >= 0
        if hit:
            keys_hit.append((int(slots[n]), n))
        elif 0 <= idx[n] < E:
            keys_miss.append((int(t[n]), int(i2[n]), int(i1[n]), n))
    keys_miss.sort()
    keys_hit.sort()
    order = [k[-1] for k in keys_miss] + [k[-1] for k in keys_hit]
    counts = np.zeros(num_tables * p[1], dtype=np.int64)
    for k in keys_miss:
        counts[k[0] * p[1] + k[1]] += 1
    return np.asarray(order, dtype=np.int64), counts


def group_counts(p, num_tables, num_bags, indices, offsets):
    """Number of elements per (table, i2) group (misses only, no cache)."""
    _, c = route_order(p, np.iinfo(np.int64).max, num_tables, num_bags, indices, offsets)
    return c


def count_frequencies(batches, counts=None):
    """One count per occurrence of each index over the given index arrays."""
    counts = {} if counts is None else counts
    for arr in batches:
        for v in np.asarray(arr, dtype=np.int64).tolist():
            counts[v] = counts.get(v, 0) + 1
    return counts


def select_cache(counts: dict, cache_size: int):
    """The cached indices in slot order: the cache_size most frequent ones,
    ordered by count descending then index ascending; slot = position."""
    items = sorted(counts.items(), key=lambda kv: (-kv[1], kv[0]))
    return np.asarray([k for k, _ in items[:cache_size]], dtype=np.int64)


def lookup_slots(cached, indices):
    """slot of each index in the cached list, -1 for a miss."""
    pos = {int(v): s for s, v in enumerate(np.asarray(cached).tolist())}
    return np.asarray([pos.get(int(v), -1) for v in np.asarray(indices).tolist()], dtype=np.int32)


def populate_rows(p, q, ranks, cores3, cached):
    """Decompressed rows for the cached indices (float64 [K, D])."""
    D = int(np.prod(q))
    out = np.zeros((len(cached), D), dtype=np.float64)
    for s, i in enumerate(np.asarray(cached).tolist()):
        out[s] = tt_row(p, q, ranks, cores3, i)
    return out


# ---------------------------------------------------------------- set-associative LFU
# "Software Cache" names a 32-way set-associative least-frequently-used cache whose
# frequencies are counted in an open-addressing hash table, refreshed on populate.  The
# pages fix no hash, no replacement detail and no row handling; the reading taken:
#   * slot = set * 32 + way; set of index i = (splitmix64(i) >> 32) mod (cache_size / 32),
#     with the splitmix64 finalizer of Steele, Lea and Flood (2014);
#   * on populate each set holds the (at most) 32 counted indices of that set with the
#     highest counts, ties to the smaller index;
#   * an index that stays keeps its way (and its row, with whatever updates it received);
#     the newcomers, in (count desc, index asc) order, take the freed ways in ascending
#     order; ways left over are empty (-1); only the newcomers' rows are rebuilt from the
#     TT cores.

LFU_WAYS = 32
_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """The splitmix64 output finalizer (Steele, Lea, Flood 2014) on a 64-bit word."""
    x &= _M64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _M64
    return x ^ (x >> 31)


def lfu_set(index: int, nsets: int) -> int:
    return (splitmix64(index) >> 32) % nsets


def lfu_populate(counts: dict, cached, cache_size: int):
    """One populate of the set-associative LFU cache.  cached: current index per slot
    (-1 = empty).  Returns (new cached array, fresh mask: slots whose row is rebuilt)."""
    assert cache_size % LFU_WAYS == 0
    nsets = cache_size // LFU_WAYS
    old = [int(v) for v in np.asarray(cached, dtype=np.int64).tolist()]
    assert len(old) == cache_size
    by_set = {}
    for k, c in counts.items():
        by_set.setdefault(lfu_set(k, nsets), []).append((-c, k))
    new = [-1] * cache_size
    fresh = np.zeros(cache_size, dtype=bool)
    for s in range(nsets):
        members = [k for _, k in sorted(by_set.get(s, []))[:LFU_WAYS]]
        ways = old[s * LFU_WAYS:(s + 1) * LFU_WAYS]
        kept = [w for w in range(LFU_WAYS) if ways[w] >= 0 and ways[w] in members]
        free = [w for w in range(LFU_WAYS) if w not in kept]
        newcomers = [k for k in members if k not in ways]
        for w in kept:
            new[s * LFU_WAYS + w] = ways[w]
        for w, k in zip(free, newcomers):
            new[s * LFU_WAYS + w] = k
            fresh[s * LFU_WAYS + w] = True
    return np.asarray(new, dtype=np.int64), fresh


# ---------------------------------------------------------------- initialisation
# "Parameters" (`weight_dist`) and the TT-Rec abstract: i.i.d. cores, or cores drawn so
# that the full table's entries follow the target; readings in the C ABI's header.

_PHILOX_M = (0xD2511F53, 0xCD9E8D57)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) on uint32 numpy arrays (or
    ints): ten rounds of two 32x32->64 multiplications, the Weyl-sequence key bumps."""
    u = np.uint64
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) for x in (c0, c1, c2, c3))
    k0, k1 = np.asarray(k0, dtype=np.uint64), np.asarray(k1, dtype=np.uint64)
    m32 = u(0xFFFFFFFF)
    for _ in range(10):
        p0 = u(_PHILOX_M[0]) * c0
        p1 = u(_PHILOX_M[1]) * c2
        c0, c1, c2, c3 = ((p1 >> u(32)) ^ c1 ^ k0) & m32, p1 & m32, \
            ((p0 >> u(32)) ^ c3 ^ k1) & m32, p0 & m32
        k0 = (k0 + u(_PHILOX_W[0])) & m32
        k1 = (k1 + u(_PHILOX_W[1])) & m32
    return c0, c1, c2, c3


def init_param(dist: int, scale: float, R1: int, R2: int) -> float:
    """Parameter of the core distribution: 0 uniform U(-s,s), 1 normal N(0,s^2),
    2 approx-uniform, 3 approx-normal (table entries with the target's variance)."""
    rr = float(R1) * float(R2)
    if dist == 3:
        return (scale * scale / rr) ** (1.0 / 6.0)
    if dist == 2:
        return (3.0 * (scale * scale / (3.0 * rr)) ** (1.0 / 3.0)) ** 0.5
    return float(scale)


def init_core(n: int, k: int, dist: int, a: float, seed: int):
    """The n values (fp64) of core k's stored array for the given seed."""
    i = np.arange(n, dtype=np.uint64)
    x0, x1, _, _ = philox4x32_10(i & np.uint64(0xFFFFFFFF), i >> np.uint64(32),
                                 np.full(n, k, dtype=np.uint64), np.zeros(n, dtype=np.uint64),
                                 seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    u0 = ((x0 >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23
    if dist in (1, 3):
        u1 = ((x1 >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23
        return a * np.sqrt(-2.0 * np.log(u0)) * np.cos(2.0 * np.pi * u1)
    return a * (2.0 * u0 - 1.0)


def factorize(n: int, exact: bool):
    """Brute force of the automatic-shape rule: exact (q1 q2 q3 == n, q1 in {1,2,4},
    q3 <= 16): the smallest largest factor, then the largest smallest, then the
    smallest q1, then the largest q2; not exact (p1 <= p2 <= p3, product >= n): the
    smallest largest factor, then the smallest product, then the smallest p1."""
    best = None
    if exact:
        for a in (1, 2, 4):
            for b in range(1, n + 1):
                for c in range(1, 17):
                    if a * b * c != n:
                        continue
                    key = (max(a, b, c), -min(a, b, c), a, -b)
                    if best is None or key < best[0]:
                        best = (key, (a, b, c))
        return None if best is None else best[1]
    for p3 in range(1, n + 1):
        for p2 in range(1, p3 + 1):
            for p1 in range(1, p2 + 1):
                if p1 * p2 * p3 < n:
                    continue
                key = (p3, p1 * p2 * p3, p1)
                if best is None or key < best[0]:
                    best = (key, (p1, p2, p3))
        if best is not None and best[0][0] <= p3:
            break
    return best[1]
