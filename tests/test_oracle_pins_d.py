"""Pins of the oracle's d-core functions (any number of cores) to facts that do not
come from the oracle itself: the Kronecker closed form at unit ranks, torch's
EmbeddingBag and autograd over a dense rebuild of the table (torch.einsum, one core
at a time), exact secants of the affine loss, and the three-core oracle at d = 3.
test_d_pins_catch_planted_mistakes plants mistakes into a copy of the oracle's C
source (on the CPU) and checks that these pins notice them.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_cores_d(rng, p, q, ranks, std=0.7):
    full = (1,) + tuple(ranks) + (1,)
    return [(rng.standard_normal((full[k], p[k], q[k], full[k + 1])) * std).astype(np.float32)
            for k in range(len(p))]


def _dense_torch(cores):
    """W (prod p x prod q) from torch tensors G_k [R][p][q][R'], contracting one core at a
    time: X[P, Q, r] * G[r, p, q, s] -> X'[P*p + p, Q*q + q, s] (row-major)."""
    X = cores[0][0]  # [p1][q1][R1]
    for G in cores[1:]:
        P, Q, _ = X.shape
        X = torch.einsum("abr,rpqs->apbqs", X, G).reshape(P * G.shape[1], Q * G.shape[2],
                                                          G.shape[3])
    return X[:, :, 0]


def _bags(rng, E, lens):
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    idx = rng.integers(0, E, off[-1]).astype(np.int64)
    return idx, off


# --------------------------------------------------------------- the table W

@pytest.mark.parametrize("p,q", [((3, 2, 4, 2), (2, 3, 1, 2)), ((2, 3, 2, 2, 3), (2, 1, 2, 3, 1))])
def test_d_rank_one_table_is_kronecker_product(p, q):
    """Closed form: with unit ranks, W = kron(M1, ..., Md) where M_k is core k reshaped
    p_k x q_k (numpy.kron orders rows and columns row-major)."""
    rng = _rng(31)
    d = len(p)
    cores = _rand_cores_d(rng, p, q, (1,) * (d - 1))
    M = [c.reshape(p[k], q[k]).astype(np.float64) for k, c in enumerate(cores)]
    Wk = M[0]
    for m in M[1:]:
        Wk = np.kron(Wk, m)
    Wo = np.stack([oracle.tt_row_d(p, q, (1,) * (d - 1), cores, i) for i in range(int(np.prod(p)))])
    np.testing.assert_allclose(Wo, Wk, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("pooling", [0, 1])
def test_d_forward_matches_torch_embedding_bag(pooling):
    """Library routine: torch's EmbeddingBag (float64, sum or mean, per-sample weights)
    over a dense rebuild of each table; two tables, an empty bag, E < prod(p)."""
    rng = _rng(32)
    p, q, ranks, E, B, T = (3, 2, 2, 3), (2, 1, 3, 2), (2, 3, 2), 31, 4, 2
    cores = [_rand_cores_d(rng, p, q, ranks) for _ in range(T)]
    idx, off = _bags(rng, E, [3, 0, 5, 2, 1, 4, 2, 6])
    w = rng.random(len(idx)).astype(np.float32)
    Y = oracle.forward_d(p, q, ranks, E, cores, idx, off, B, per_sample_weights=w,
                         pooling=pooling)
    for t in range(T):
        Wt = _dense_torch([torch.from_numpy(c.astype(np.float64)) for c in cores[t]])[:E]
        lo, hi = off[t * B], off[(t + 1) * B]
        if pooling == 0:
            Yt = torch.nn.functional.embedding_bag(
                torch.from_numpy(idx[lo:hi]), Wt, torch.from_numpy(off[t * B:(t + 1) * B] - lo),
                mode="sum", per_sample_weights=torch.from_numpy(w[lo:hi].astype(np.float64)))
        else:  # torch's mean mode takes no weights: weight the rows, then average
            rows = Wt[torch.from_numpy(idx[lo:hi])] * torch.from_numpy(
                w[lo:hi].astype(np.float64))[:, None]
            Yt = torch.stack([rows[off[b] - lo:off[b + 1] - lo].mean(0) if off[b + 1] > off[b]
                              else torch.zeros(Wt.shape[1], dtype=torch.float64)
                              for b in range(t * B, (t + 1) * B)])
        np.testing.assert_allclose(Y[t * B:(t + 1) * B], Yt.numpy(), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------- backward

@pytest.mark.parametrize("p,q,ranks", [((3, 2, 2, 3), (2, 1, 3, 2), (2, 3, 2)),
                                       ((2, 2, 3, 2, 2), (1, 2, 2, 1, 3), (2, 2, 3, 2))])
def test_d_backward_matches_torch_autograd(p, q, ranks):
    """Library routine: torch.autograd (float64) through the dense rebuild and torch's
    EmbeddingBag; every core gradient, two tables, weights, and the touched masks."""
    rng = _rng(33)
    E, B, T = int(np.prod(p)) - 2, 3, 2
    D = int(np.prod(q))
    cores = [_rand_cores_d(rng, p, q, ranks) for _ in range(T)]
    idx, off = _bags(rng, E, [2, 4, 0, 3, 5, 1])
    w = rng.random(len(idx)).astype(np.float32)
    dY = rng.standard_normal((T * B, D)).astype(np.float32)
    grads, touched = oracle.backward_d(p, q, ranks, E, cores, idx, off, B, dY,
                                       per_sample_weights=w)
    for t in range(T):
        G = [torch.tensor(c.astype(np.float64), requires_grad=True) for c in cores[t]]
        Wt = _dense_torch(G)[:E]
        lo, hi = off[t * B], off[(t + 1) * B]
        Y = torch.nn.functional.embedding_bag(
            torch.from_numpy(idx[lo:hi]), Wt, torch.from_numpy(off[t * B:(t + 1) * B] - lo),
            mode="sum", per_sample_weights=torch.from_numpy(w[lo:hi].astype(np.float64)))
        (Y * torch.from_numpy(dY[t * B:(t + 1) * B].astype(np.float64))).sum().backward()
        ii = np.stack(np.unravel_index(idx[lo:hi], p))
        for k in range(len(p)):
            np.testing.assert_allclose(grads[t][k], G[k].grad.numpy(), rtol=1e-11, atol=1e-12)
            assert set(np.flatnonzero(touched[t][k])) == set(ii[k].tolist())


def _loss_d(p, q, ranks, E, cores, idx, off, B, dY, w, pooling):
    Y = oracle.forward_d(p, q, ranks, E, cores, idx, off, B, per_sample_weights=w,
                         pooling=pooling)
    return float(np.sum(Y * dY.astype(np.float64)))


@pytest.mark.parametrize("pooling", [0, 1])
def test_d_backward_equals_exact_finite_differences(pooling):
    """Invariant: L = sum <dY, Y> is affine in any single core entry, so a secant through
    two fp32 values of that entry is the partial derivative up to rounding; duplicates
    of an index add up; mean pooling carries 1/len."""
    rng = _rng(34)
    p, q, ranks, B = (2, 3, 2, 2, 2), (2, 1, 2, 1, 2), (2, 3, 2, 2), 4
    E = int(np.prod(p))
    D = int(np.prod(q))
    cores = [_rand_cores_d(rng, p, q, ranks)]
    idx, off = _bags(rng, E, [4, 1, 0, 6])
    idx[:3] = idx[3]
    w = rng.random(len(idx)).astype(np.float32)
    dY = rng.standard_normal((B, D)).astype(np.float32)
    grads, _ = oracle.backward_d(p, q, ranks, E, cores, idx, off, B, dY, per_sample_weights=w,
                                 pooling=pooling)
    for k in range(len(p)):
        G = cores[0][k]
        for flat in rng.choice(G.size, size=min(G.size, 8), replace=False):
            pert = [c.copy() for c in cores[0]]
            a0 = float(G.flat[flat])
            a1 = float(np.float32(a0 + 0.5))
            pert[k].flat[flat] = np.float32(a1)
            l0 = _loss_d(p, q, ranks, E, cores, idx, off, B, dY, w, pooling)
            l1 = _loss_d(p, q, ranks, E, [pert], idx, off, B, dY, w, pooling)
            fd = (l1 - l0) / (a1 - a0)
            assert abs(fd - grads[0][k].flat[flat]) <= 1e-10 * (1 + abs(fd)), (k, flat)


def test_d_three_cores_equal_three_core_oracle():
    """Special case: at d = 3 the d-core functions agree with the three-core ones
    (whose own pins cover the three-core definition)."""
    rng = _rng(35)
    p, q, ranks, E, B = (4, 3, 5), (2, 3, 2), (3, 4), 55, 5
    cores = [_rand_cores_d(rng, p, q, ranks)]
    idx, off = _bags(rng, E, [3, 0, 4, 2, 6])
    w = rng.random(len(idx)).astype(np.float32)
    dY = rng.standard_normal((B, 12)).astype(np.float32)
    Yd = oracle.forward_d(p, q, ranks, E, cores, idx, off, B, per_sample_weights=w)
    Y3 = oracle.forward(p, q, ranks, E, cores, idx, off, B, per_sample_weights=w)
    np.testing.assert_allclose(Yd, Y3, rtol=1e-13, atol=1e-14)
    gd, td = oracle.backward_d(p, q, ranks, E, cores, idx, off, B, dY, per_sample_weights=w)
    g3, t3, _, _ = oracle.backward(p, q, ranks, E, cores, idx, off, B, dY, per_sample_weights=w)
    for k in range(3):
        np.testing.assert_allclose(gd[0][k], g3[0][k], rtol=1e-12, atol=1e-13)
        np.testing.assert_array_equal(td[0][k], t3[0][k])


def test_d_sgd_step_invariants():
    """Invariant: the SGD delta is -lr * gradient (rounded once to fp32) on touched
    slices, and untouched slices keep their bits."""
    rng = _rng(36)
    p, q, ranks, E, B = (3, 2, 4, 2), (2, 2, 1, 2), (2, 3, 2), 40, 3
    cores = [_rand_cores_d(rng, p, q, ranks)]
    idx, off = _bags(rng, E, [2, 1, 2])
    dY = rng.standard_normal((B, 8)).astype(np.float32)
    grads, touched = oracle.backward_d(p, q, ranks, E, cores, idx, off, B, dY)
    new = oracle.sgd_d(cores, grads, touched, 0.05)
    for k in range(len(p)):
        m = touched[0][k].astype(bool)
        assert np.array_equal(new[0][k][:, ~m].view(np.uint32), cores[0][k][:, ~m].view(np.uint32))
        want = (cores[0][k].astype(np.float64) - 0.05 * grads[0][k]).astype(np.float32)
        assert np.array_equal(new[0][k][:, m], want[:, m])
        assert m.any()


# --------------------------------------------------------------- planted mistakes

_MUTANTS_D = [
    # column split of j in the wrong order
    ("static void split_d(const int32_t *e, int d, int64_t v, int64_t *out)\n{\n    for (int k = d - 1; k >= 0; --k) {",
     "static void split_d(const int32_t *e, int d, int64_t v, int64_t *out)\n{\n    for (int k = 0; k < d; ++k) {"),
    # a core slice read transposed in the prefix product
    ("acc += L[k * M + a] * (double)G[k][core_index_d(s, k, a, ii[k], jj[k], b)];",
     "acc += L[k * M + a] * (double)G[k][core_index_d(s, k, b % ra, ii[k], jj[k], a % rb)];"),
    # gradient without the suffix factor
    ("g * L[k * M + a] * S[(k + 1) * M + c];", "g * L[k * M + a];"),
    # gradient with the wrong suffix (the one that includes core k itself)
    ("g * L[k * M + a] * S[(k + 1) * M + c];", "g * L[k * M + a] * S[k * M + c % ra];"),
    # per-sample weight dropped in the d-core backward
    ("const double w = (psw ? (double)psw[n] : 1.0) * inv;\n            split_d(",
     "const double w = inv;\n            split_d("),
    # mean pooling forgotten in the d-core forward
    ("        if (s->pooling == 1 && off[b + 1] > off[b])\n            for (int64_t j = 0; j < D; ++j) Y[b * D + j] /= (double)(off[b + 1] - off[b]);\n    }\n    free(row);\n    return 0;\n}\n\n/* Backward over d-core",
     "    }\n    free(row);\n    return 0;\n}\n\n/* Backward over d-core"),
]


@pytest.mark.parametrize("mi", range(len(_MUTANTS_D)))
def test_d_pins_catch_planted_mistakes(mi, tmp_path, monkeypatch):
    """Plant one mistake into a copy of the oracle's d-core code (CPU only) and check
    that the d-core pins above fail on it."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "tt_oracle.c")).read()
    old, new = _MUTANTS_D[mi]
    assert src.count(old) >= 1, old
    at = src.index("General number of cores d")
    mutated = src[:at] + src[at:].replace(old, new, 1)
    assert mutated != src
    c = tmp_path / ("d%d.c" % mi)
    so = tmp_path / ("d%d.so" % mi)
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(c), "-o", str(so),
                           "-lm"])
    import oracle.tt_oracle as O
    saved = O._lib
    O._lib = None
    monkeypatch.setattr(O, "build", lambda force=False: str(so))
    pins = [lambda: test_d_rank_one_table_is_kronecker_product((3, 2, 4, 2), (2, 3, 1, 2)),
            lambda: test_d_forward_matches_torch_embedding_bag(0),
            lambda: test_d_forward_matches_torch_embedding_bag(1),
            lambda: test_d_backward_matches_torch_autograd((3, 2, 2, 3), (2, 1, 3, 2), (2, 3, 2)),
            lambda: test_d_backward_equals_exact_finite_differences(1)]
    failures = 0
    try:
        for f in pins:
            try:
                f()
            except (AssertionError, ValueError):
                failures += 1
    finally:
        O._lib = saved
    assert failures > 0, "planted mistake %d went unnoticed" % mi
