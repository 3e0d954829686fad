"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol declared in include/tt_bag.h, and rejects bad arguments before enqueuing
anything (these calls return from the host validation and touch no device)."""
import ctypes
import os
import re

import pytest
import torch

from tensor_train_compressed_ttembeddingbag_amd import abi, workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tt_bag.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tt_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = abi.lib()
    names = _declared()
    assert "tt_bag_forward" in names and "tt_cache_lookup" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(abi.EXPORTS)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert abi.status_string(code)
    assert abi.status_string(-99) == "unknown status"


def test_workspace_size_and_shape_envelope():
    wl = W.WORKLOADS["readme"]
    d = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    n = abi.tt_bag_workspace_size(d, 10240, 512)
    assert n > 10240 * 16
    assert abi.tt_bag_workspace_size(d, 20480, 512) > n
    L = abi.lib()
    bad = [abi.make_desc(wl.p, (3, 4, 4), wl.ranks, wl.E),        # q1 = 3
           abi.make_desc(wl.p, wl.q, (65, 32), wl.E),             # rank above 64
           abi.make_desc(wl.p, wl.q, (0, 32), wl.E),              # rank 0
           abi.make_desc((10, 10, 10), wl.q, wl.ranks, 1001),     # E > prod(p)
           abi.make_desc((9000, 2, 2), wl.q, wl.ranks, 100),      # too many bins
           abi.make_desc(wl.p, (4, 4, 17), wl.ranks, wl.E)]       # q3 > 16
    for b in bad:
        assert L.tt_bag_workspace_size(ctypes.byref(b), 100, 10, 0) == 0
    # a cache needs a single table
    d8 = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, num_tables=8)
    assert L.tt_bag_workspace_size(ctypes.byref(d8), 100, 10, 1000) == 0
    assert L.tt_bag_workspace_size(ctypes.byref(d8), 100, 10, 0) > 0


def test_entry_points_reject_bad_arguments_without_device_work():
    wl = W.WORKLOADS["tiny"]
    L = abi.lib()
    d = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    cores = (ctypes.c_void_p * 3)(0x1000, 0x2000, 0x3000)
    null_cores = (ctypes.c_void_p * 3)(0x1000, 0, 0x3000)
    # negative nnz / zero bags
    assert L.tt_bag_forward(ctypes.byref(d), cores, fake, -1, fake, 8, None, None, fake, fake,
                            1 << 20, None, None) == -1
    assert L.tt_bag_forward(ctypes.byref(d), cores, fake, 10, fake, 0, None, None, fake, fake,
                            1 << 20, None, None) == -1
    # a null core pointer
    assert L.tt_bag_forward(ctypes.byref(d), null_cores, fake, 10, fake, 8, None, None, fake, fake,
                            1 << 20, None, None) == -1
    # workspace too small or misaligned
    assert L.tt_bag_forward(ctypes.byref(d), cores, fake, 10, fake, 8, None, None, fake, fake,
                            16, None, None) == -3
    assert L.tt_bag_forward(ctypes.byref(d), cores, fake, 10, fake, 8, None, None, fake,
                            P(0x1004), 1 << 20, None, None) == -3
    # shape outside the envelope
    d3 = abi.make_desc(wl.p, (3, 2, 2), wl.ranks, wl.E)
    assert L.tt_bag_backward_sgd(ctypes.byref(d3), cores, fake, 10, fake, 8, None, None, fake,
                                 ctypes.c_float(0.1), fake, 1 << 20, None, None) == -2
    # non-finite learning rate
    assert L.tt_bag_backward_sgd(ctypes.byref(d), cores, fake, 10, fake, 8, None, None, fake,
                                 ctypes.c_float(float("nan")), fake, 1 << 20, None, None) == -1
    # cache handle checks
    assert L.tt_cache_lookup(None, fake, 10, fake, 1, None, None) == -1
    assert L.tt_cache_destroy(None) == -1
    h = ctypes.c_void_p()
    d8 = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, num_tables=2)
    assert L.tt_cache_create(ctypes.byref(h), ctypes.byref(d8), 10, 100) == -2
    assert L.tt_cache_create(ctypes.byref(h), ctypes.byref(d), 0, 100) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(abi, "_lib", None)
    monkeypatch.setattr(abi, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        abi.lib()


def test_multiply_high_division_is_exact_on_its_range():
    """The kernels divide small indices (k < 2^16) by runtime extents (q3, D) with one
    high multiply by ceil(2^32 / d); check floor(k * m / 2^32) == k // d exhaustively
    in k for every divisor the shape envelope allows (d <= 1024)."""
    import numpy as np
    k = np.arange(1 << 16, dtype=np.uint64)
    for d in range(2, 1025):
        m = np.uint64(((1 << 32) + d - 1) // d)
        assert np.array_equal((k * m) >> np.uint64(32), k // np.uint64(d)), d


def test_row_split_through_double_reciprocals():
    """The routing kernels split a row index with double reciprocals and one correction
    step; emulate that arithmetic (IEEE double, as on the GPU) on edge rows -- multiples
    of p3 and p2*p3, their neighbours, the last row -- and random rows for a range of
    shapes up to p_k = 8191 and E < 2^40."""
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(11))
    shapes = [(200, 220, 250), (8191, 8191, 8191), (1, 1, 1), (3, 8191, 1), (8191, 1, 7),
              (97, 89, 83)] + [tuple(int(x) for x in rng.integers(1, 8192, 3)) for _ in range(40)]
    for p1, p2, p3 in shapes:
        p23 = p2 * p3
        E = p1 * p23
        rows = [0, E - 1] + [k * p23 + d for k in rng.integers(0, p1, 50) for d in (-1, 0, 1)]
        rows += [k * p3 + d for k in rng.integers(0, p1 * p2, 50) for d in (-1, 0, 1)]
        rows += list(rng.integers(0, E, 500))
        i = np.array([r for r in rows if 0 <= r < E], dtype=np.int64)
        rp23, rp3 = np.float64(1.0) / np.float64(p23), np.float64(1.0) / np.float64(p3)
        q1 = (i.astype(np.float64) * rp23).astype(np.int64)  # truncation toward zero
        r = i - q1 * p23
        q1 = np.where(r >= p23, q1 + 1, np.where(r < 0, q1 - 1, q1))
        r = np.where(r >= p23, r - p23, np.where(r < 0, r + p23, r))
        q2 = (r.astype(np.float64) * rp3).astype(np.int64)
        r3 = r - q2 * p3
        q2 = np.where(r3 >= p3, q2 + 1, np.where(r3 < 0, q2 - 1, q2))
        r3 = np.where(r3 >= p3, r3 - p3, np.where(r3 < 0, r3 + p3, r3))
        assert np.array_equal(q1, i // p23) and np.array_equal(q2, (i % p23) // p3)
        assert np.array_equal(r3, i % p3)


def test_factorize_host_function_matches_the_oracle_rule():
    """tt_factorize (host code of the library, no GPU) against the oracle's brute force."""
    import oracle.tt_oracle as O
    for n in range(1, 160):
        assert abi.tt_factorize(n, False) == O.factorize(n, False), n
        want = O.factorize(n, True)
        if want is None:
            with pytest.raises(abi.TTError):
                abi.tt_factorize(n, True)
        else:
            assert abi.tt_factorize(n, True) == want, n
    assert abi.tt_factorize(11000000, False) == (222, 223, 223)


def test_train_loop_rejects_invalid_options():
    """The benchmark's training loop refuses, before any device work, an unknown update
    and the backward over distinct indices combined with a cache or with Adagrad."""
    from tensor_train_compressed_ttembeddingbag_amd.loop import TrainLoop
    batch = [{"indices": torch.zeros(1, dtype=torch.int64)}]
    with pytest.raises(ValueError):
        TrainLoop(None, [], batch, 1, 0.1, None, None, update="adam")
    with pytest.raises(ValueError):
        TrainLoop(None, [], batch, 1, 0.1, None, None, cache=object(), dedup=True)
    with pytest.raises(ValueError):
        TrainLoop(None, [], batch, 1, 0.1, None, None, update="adagrad", dedup=True)
    # with a cache, one batch would let a lookup rewrite the slots a forward still reads
    with pytest.raises(ValueError):
        TrainLoop(None, [], batch, 1, 0.1, None, None, cache=object())


def _host_only_binding(monkeypatch):
    """The binding with its device check relaxed to dtype/contiguity (CPU tensors stand in
    for device ones) and a library that must never be called: a size mismatch has to be
    rejected before any call into libttbag."""
    def need(t, dtype, name):
        if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_contiguous():
            raise TypeError(name)

    def no_lib():
        raise AssertionError("the library was called with mis-sized buffers")

    monkeypatch.setattr(abi, "_need", need)
    monkeypatch.setattr(abi, "lib", no_lib)


def test_binding_rejects_mis_sized_buffers_before_any_device_work(monkeypatch):
    """Every size the kernels index by is checked by the binding: offsets without the
    terminal entry (the README example's [0, 4] form), a wrong out / grad_out shape, a
    wrong core size, per-sample weights or slots of the wrong length, and cache rows of
    the wrong width each raise ValueError before the C entry point is reached."""
    _host_only_binding(monkeypatch)
    wl = W.WORKLOADS["tiny"]
    d = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    D, B, nnz = 8, 2, 8
    sizes = abi._core_numels(d)
    assert sizes == (4 * 2 * 4, 5 * 4 * 2 * 4, 6 * 4 * 2)
    cores = [torch.zeros(n) for n in sizes]
    idx = torch.tensor([1, 2, 4, 5, 4, 3, 2, 9], dtype=torch.int64)
    off = torch.tensor([0, 4, 8], dtype=torch.int64)
    ws = torch.zeros(16, dtype=torch.uint8)
    out = torch.zeros(B, D)
    gout = torch.zeros(B, D)

    def fwd(**kw):
        args = dict(cores=cores, indices=idx, offsets=off, num_bags=B, out=out, ws=ws)
        args.update(kw)
        return abi.tt_bag_forward(d, args.pop("cores"), args.pop("indices"), args.pop("offsets"),
                                  args.pop("num_bags"), **args)

    def bwd(**kw):
        args = dict(cores=cores, offsets=off, grad_out=gout, ws=ws)
        args.update(kw)
        return abi.tt_bag_backward_sgd(d, args.pop("cores"), idx, args.pop("offsets"), B,
                                       args.pop("grad_out"), 0.1, **args)

    cases = [
        lambda: fwd(offsets=torch.tensor([0, 4], dtype=torch.int64)),  # no terminal entry
        lambda: fwd(out=torch.zeros(B, D + 1)),
        lambda: fwd(out=torch.zeros(B + 1, D)),
        lambda: fwd(cores=[cores[0], torch.zeros(sizes[1] - 1), cores[2]]),
        lambda: fwd(per_sample_weights=torch.ones(nnz - 1)),
        lambda: fwd(cache=(torch.zeros(nnz, dtype=torch.int32), torch.zeros(10, D + 1))),
        lambda: fwd(cache=(torch.zeros(nnz - 1, dtype=torch.int32), torch.zeros(10, D))),
        lambda: bwd(offsets=torch.tensor([0, 4], dtype=torch.int64)),
        lambda: bwd(grad_out=torch.zeros(B, D - 1)),
        lambda: bwd(cores=[torch.zeros(sizes[0] + 4), cores[1], cores[2]]),
        lambda: abi.tt_bag_plan(d, idx, torch.tensor([0, 8], dtype=torch.int64), B, ws=ws),
        lambda: abi.tt_bag_backward_grad(d, cores, idx, off, B, gout, ws=ws,
                                         grad_cores=[c.clone() for c in cores[:2]]
                                         + [torch.zeros(3)]),
        lambda: abi.tt_bag_backward_adagrad(d, cores, idx, off, B, gout, 0.1, 1e-8,
                                            [torch.zeros(1), cores[1], cores[2]], ws=ws),
        lambda: abi.tt_bag_weight_grad(d, cores, idx, off, B, gout, ws=ws,
                                       out=torch.zeros(nnz + 1)),
        lambda: abi.tt_full_weight(d, cores, 0, 4, out=torch.zeros(4, D - 1)),
        lambda: abi.tt_init_cores(d, [cores[0], cores[1], torch.zeros(1)], 0, 1.0, 0),
        lambda: abi.tt_bag_route(d, idx, off, B, slots=torch.zeros(3, dtype=torch.int32),
                                 cache_size=10, ws=ws),
    ]
    for k, case in enumerate(cases):
        with pytest.raises(ValueError):
            case()
            pytest.fail("case %d was accepted" % k)
    # the d-core binding checks its cores the same way
    dd = abi.make_desc_d((2, 2, 5, 6), (1, 2, 2, 2), (2, 4, 4), 120)
    nd = abi._core_numels_d(dd)
    assert nd == (2 * 1 * 1 * 2, 2 * 2 * 2 * 4, 5 * 4 * 2 * 4, 6 * 4 * 2 * 1)
    with pytest.raises(ValueError):
        abi.tt_bag_forward_d(dd, [torch.zeros(n) for n in nd[:3]] + [torch.zeros(nd[3] + 1)],
                             idx, off, B, ws=ws)


@pytest.mark.parametrize("ahead,every", [(1, 1), (1, 4), (2, 1), (2, 4), (2, 3)])
def test_train_loop_grouping_waits_cover_workspace_reuse(ahead, every):
    """The pipelined loop's reuse rule, brute force: the grouping of batch j (enqueued
    during step j - ahead, into workspace j % (ahead + every)) waits for a step whose done
    event has already been recorded by then (k <= j - ahead - 1, k one of the steps that
    record one) and that is at or after the last step that used the same workspace."""
    from tensor_train_compressed_ttembeddingbag_amd.loop import TrainLoop
    L = object.__new__(TrainLoop)
    L.ahead, L.every = ahead, every
    W = ahead + every
    for j in range(300):
        k = L.done_step(j)
        # the first `ahead` groupings are enqueued before step 0, behind the loop's first
        # event (-1); every later one behind a recorded step
        assert k == -1 or (k <= j - ahead - 1 and k % every == every - 1)
        last_user = j - W  # the previous batch in workspace j % W
        assert k >= last_user or last_user < 0


def test_package_star_import_names_only_existing_modules():
    """Every name the package exports imports on a host without a GPU (the HIP library
    itself loads only at the first call)."""
    import subprocess
    import sys
    code = ("from tensor_train_compressed_ttembeddingbag_amd import *\n"
            "import tensor_train_compressed_ttembeddingbag_amd as p\n"
            "assert all(hasattr(p, n) for n in p.__all__)\n"
            "from tensor_train_compressed_ttembeddingbag_amd.module import TTEmbeddingBag, "
            "TableBatchedTTEmbeddingBag, OptimType\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
