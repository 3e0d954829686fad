"""Backward over distinct indices (tt_bag_plan_dedup + tt_bag_backward_*_dedup): the
gradients and the SGD step against the oracle on small Zipf-skewed batches (two tables,
weights, sum and mean pooling, empty bags), the distinct-index counts (kept on the device,
read by the diagnostic query) bit-exact against numpy, and, at the skewed and
table-batched workloads' full sizes, against the three-core backward over every element.
The plan does not synchronise the host: a captured plan + backward replays like the
eager calls."""
import numpy as np
import pytest
import torch

import oracle
from tensor_train_compressed_ttembeddingbag_amd import abi, workloads as W
from helpers import TOL, rel_err

pytestmark = pytest.mark.gpu


def _dev(cores, k):
    return torch.from_numpy(np.concatenate([W.slice_major(tbl[k]).ravel() for tbl in cores])).cuda()


def _host(t, cores, k):
    x = t.cpu().numpy()
    out, at = [], 0
    for tbl in cores:
        shp = tbl[k].shape
        n = tbl[k].size
        out.append(W.logical(x[at:at + n], shp))
        at += n
    return out


def _check_counts(desc, nnz, B, ws, idx, off, T):
    """The device's distinct-index counts (the diagnostic query) bit-exact against numpy."""
    got = abi.tt_bag_dedup_counts(desc, nnz, B, ws)
    bag = np.searchsorted(off, np.arange(len(idx)), side="right") - 1
    t = bag // B
    per = [len(np.unique(idx[t == x])) for x in range(T)]
    assert got == list(np.concatenate([[0], np.cumsum(per)])), (got, per)


@pytest.mark.parametrize("pooling", [0, 1])
def test_dedup_matches_oracle_small(pooling):
    print("case dedup small pooling", pooling, flush=True)
    rng = np.random.Generator(np.random.PCG64(800 + pooling))
    p, q, ranks, T, B = (6, 5, 7), (2, 4, 2), (8, 6), 2, 40
    E = 200
    D = 16
    cores = [[(rng.standard_normal(s) * 0.5).astype(np.float32)
              for s in W.core_shapes(W.custom(p=p, q=q, ranks=ranks))] for _ in range(T)]
    lens = rng.integers(0, 9, T * B)
    lens[3] = 0
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    z = rng.zipf(1.3, off[-1])
    idx = ((z - 1) * 37 % E).astype(np.int64)  # heavy repeats
    w = rng.random(off[-1]).astype(np.float32)
    dY = rng.standard_normal((T * B, D)).astype(np.float32)
    desc = abi.make_desc(p, q, ranks, E, T, pooling)
    g = [_dev(cores, k) for k in range(3)]
    d_idx, d_off = torch.from_numpy(idx).cuda(), torch.from_numpy(off).cuda()
    d_w, d_dY = torch.from_numpy(w).cuda(), torch.from_numpy(dY).cuda()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws, info = abi.tt_bag_plan_dedup(desc, d_idx, d_off, B, d_w, dev_status=st)
    assert info == (len(idx), len(idx))
    _check_counts(desc, len(idx), B, ws, idx, off, T)
    assert abi.tt_bag_dedup_counts(desc, len(idx), B, ws)[T] < len(idx) // 2
    Y = abi.tt_bag_forward(desc, g, d_idx, d_off, B, d_w, ws=ws, dev_status=st, planned=True)
    Yref = oracle.forward(p, q, ranks, E, cores, idx, off, B, per_sample_weights=w,
                          pooling=pooling)
    assert rel_err(Y.cpu().numpy(), Yref) <= TOL
    grads, touched, _, _ = oracle.backward(p, q, ranks, E, cores, idx, off, B, dY,
                                           per_sample_weights=w, pooling=pooling)
    gg = abi.tt_bag_backward_grad_dedup(desc, g, d_idx, d_off, B, d_dY, info,
                                        per_sample_weights=d_w, ws=ws, dev_status=st)
    for k in range(3):
        got = _host(gg[k], cores, k)
        for t in range(T):
            assert rel_err(got[t], grads[t][k]) <= TOL, (k, t)
            assert np.all(got[t][:, ~touched[t][k].astype(bool)] == 0.0), (k, t)
    lr = 0.05
    new = [x.clone() for x in g]
    abi.tt_bag_backward_sgd_dedup(desc, new, d_idx, d_off, B, d_dY, lr, info,
                                  per_sample_weights=d_w, ws=ws, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for k in range(3):
        got = _host(new[k], cores, k)
        for t in range(T):
            delta = got[t].astype(np.float64) - cores[t][k].astype(np.float64)
            assert rel_err(delta, -lr * grads[t][k]) <= TOL, (k, t)
            m = ~touched[t][k].astype(bool)
            assert np.array_equal(got[t][:, m], cores[t][k][:, m]), (k, t)


@pytest.mark.parametrize("name", ["skewed", "multitable"])
def test_dedup_full_size_matches_every_element_backward(name):
    """Full-size workloads: the distinct counts bit-exact, and the core gradients of the
    virtual batch equal those over every element (the three-core backward, itself
    parity-tested against the oracle) within the bound."""
    print("case dedup full", name, flush=True)
    wl = W.WORKLOADS[name]
    cores = W.make_cores(wl)
    b = W.make_batch(wl, 0)
    B = wl.bags_per_table
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, wl.num_tables)
    g = [_dev(cores, k) for k in range(3)]
    d_idx = torch.from_numpy(b["indices"]).cuda()
    d_off = torch.from_numpy(b["offsets"]).cuda()
    d_dY = torch.from_numpy(b["grad_out"]).cuda()
    d_w = None if b["per_sample_weights"] is None else torch.from_numpy(b["per_sample_weights"]).cuda()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws, info = abi.tt_bag_plan_dedup(desc, d_idx, d_off, B, d_w, dev_status=st)
    nnz = len(b["indices"])
    assert info == (nnz, nnz)  # the bounds: the counts stay on the device
    _check_counts(desc, nnz, B, ws, b["indices"], b["offsets"], wl.num_tables)
    gd = abi.tt_bag_backward_grad_dedup(desc, g, d_idx, d_off, B, d_dY, info,
                                        per_sample_weights=d_w, ws=ws, dev_status=st)
    ge, _ = abi.tt_bag_backward_grad(desc, g, d_idx, d_off, B, d_dY, per_sample_weights=d_w)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for k in range(3):
        a, e = gd[k].cpu().numpy().astype(np.float64), ge[k].cpu().numpy().astype(np.float64)
        assert rel_err(a, e) <= TOL, k
        assert np.array_equal(a == 0, e == 0), k  # the same slices touched


def test_dedup_empty_batch():
    print("case dedup empty", flush=True)
    p, q, ranks, E, T, B = (4, 5, 6), (2, 2, 2), (4, 4), 120, 1, 3
    rng = np.random.Generator(np.random.PCG64(803))
    cores = [[(rng.standard_normal(s) * 0.5).astype(np.float32)
              for s in W.core_shapes(W.custom(p=p, q=q, ranks=ranks))]]
    desc = abi.make_desc(p, q, ranks, E, T)
    g = [_dev(cores, k) for k in range(3)]
    idx = torch.zeros(0, dtype=torch.int64, device="cuda")
    off = torch.zeros(B + 1, dtype=torch.int64, device="cuda")
    dY = torch.randn(B, 8, device="cuda")
    ws, info = abi.tt_bag_plan_dedup(desc, idx, off, B)
    assert info == (0, 0)
    gg = abi.tt_bag_backward_grad_dedup(desc, g, idx, off, B, dY, info, ws=ws)
    assert all(torch.all(x == 0) for x in gg)
    new = [x.clone() for x in g]
    abi.tt_bag_backward_sgd_dedup(desc, new, idx, off, B, dY, 0.1, info, ws=ws)
    assert all(torch.equal(a, b) for a, b in zip(new, g))


def test_dedup_backward_refuses_another_batchs_plan():
    """A distinct-index backward for batch B on a workspace planned for batch A (same nnz,
    so every size agrees) finds another batch's plan: it reports TT_DEV_STALE_PLAN and
    leaves the cores bit-identical."""
    print("case dedup stale plan", flush=True)
    wl = W.custom(p=(6, 5, 7), q=(2, 4, 2), ranks=(8, 6), bags_per_table=30,
                  lengths=("fixed", 6), dist=("zipf", 1.2), lr=0.05)
    cores = W.make_cores(wl)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    ba, bb = W.make_batch(wl, 0), W.make_batch(wl, 1)
    assert len(ba["indices"]) == len(bb["indices"])
    # both batches stay allocated: a freed buffer's address may be handed to the next one,
    # and a plan cannot tell new contents at an old address (the documented contract)
    ia, oa = torch.from_numpy(ba["indices"]).cuda(), torch.from_numpy(ba["offsets"]).cuda()
    ib, ob = torch.from_numpy(bb["indices"]).cuda(), torch.from_numpy(bb["offsets"]).cuda()
    gb = torch.from_numpy(bb["grad_out"]).cuda()
    g = [_dev(cores, k) for k in range(3)]
    before = [x.clone() for x in g]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws, info = abi.tt_bag_plan_dedup(desc, ia, oa, 30, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and info[0] > 0
    abi.tt_bag_backward_sgd_dedup(desc, g, ib, ob, 30, gb, wl.lr, info, ws=ws, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & abi.TT_DEV_STALE_PLAN
    for k in range(3):
        assert torch.equal(before[k], g[k]), k
    # the workspace still serves its own batch once it is planned again
    st.zero_()
    ws, info = abi.tt_bag_plan_dedup(desc, ib, ob, 30, ws=ws, dev_status=st)
    abi.tt_bag_backward_sgd_dedup(desc, g, ib, ob, 30, gb, wl.lr, info, ws=ws, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    grads, touched, _, _ = oracle.backward(wl.p, wl.q, wl.ranks, wl.E, cores, bb["indices"],
                                           bb["offsets"], 30, bb["grad_out"])
    for k in range(3):
        got = _host(g[k], cores, k)[0].astype(np.float64)
        assert rel_err(got - cores[0][k], -wl.lr * grads[0][k]) <= TOL, k


def test_dedup_plan_and_backward_replay_from_a_graph():
    """The distinct-index plan does not wait on the host, so the plan and the SGD backward
    can be captured into one HIP graph: three replays (with eager work and a
    synchronisation between them) leave the cores bit for bit equal to the same calls made
    eagerly, and the counts on the device equal numpy's."""
    print("case dedup graph replay", flush=True)
    wl = W.custom(p=(6, 5, 7), q=(2, 4, 2), ranks=(8, 6), bags_per_table=30,
                  lengths=("fixed", 6), dist=("zipf", 1.2), lr=0.05)
    cores = W.make_cores(wl)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    b = W.make_batch(wl, 3)
    idx, off = torch.from_numpy(b["indices"]).cuda(), torch.from_numpy(b["offsets"]).cuda()
    dY = torch.from_numpy(b["grad_out"]).cuda()
    nnz = len(b["indices"])
    g_e = [_dev(cores, k) for k in range(3)]
    g_c = [x.clone() for x in g_e]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws_e = abi.workspace_dedup(desc, nnz, 30, idx.device)
    ws_c = abi.workspace_dedup(desc, nnz, 30, idx.device)
    info = (nnz, nnz)
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=cap):
        _, ic = abi.tt_bag_plan_dedup(desc, idx, off, 30, ws=ws_c, dev_status=st, stream=cap)
        abi.tt_bag_backward_sgd_dedup(desc, g_c, idx, off, 30, dY, wl.lr, info, ws=ws_c,
                                      dev_status=st, stream=cap)
    assert ic == info
    for rep in range(3):
        _, ie = abi.tt_bag_plan_dedup(desc, idx, off, 30, ws=ws_e, dev_status=st)
        abi.tt_bag_backward_sgd_dedup(desc, g_e, idx, off, 30, dY, wl.lr, ie, ws=ws_e,
                                      dev_status=st)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0, rep
        for k in range(3):
            assert torch.equal(g_c[k], g_e[k]), (rep, k)
        _check_counts(desc, nnz, 30, ws_c, b["indices"], b["offsets"], 1)
        # eager work between replays
        (g_e[0] * 2.0).sum().item()
