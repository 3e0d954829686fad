"""The training loop the benchmark times (loop.TrainLoop: the grouping of batch i+1 on a
second stream during the backward of batch i, two alternating workspaces, event ordering),
at the full readme and table-batched sizes: every step's pooled forward and core update
against the oracle evaluated at the cores that step started from."""
import numpy as np
import pytest
import torch

import oracle
from tensor_train_compressed_ttembeddingbag_amd import abi, workloads as W
from tensor_train_compressed_ttembeddingbag_amd.loop import TrainLoop
from helpers import TOL, gpu_cores, host_cores, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name, steps", [("readme", 3), ("multitable", 2)])
def test_pipelined_loop_matches_oracle(name, steps):
    print("case train loop", name, steps, flush=True)
    wl = W.WORKLOADS[name]
    T, B = wl.num_tables, wl.bags_per_table
    cores = W.make_cores(wl)
    g = gpu_cores(wl, cores)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, T)
    host_batches = [W.make_batch(wl, k) for k in range(2)]  # cycled, as the benchmark does
    out = torch.empty(T * B, wl.D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    loop = TrainLoop(desc, g, [to_dev(b) for b in host_batches], B, wl.lr, out, status)
    snaps, ys = [[x.clone() for x in g]], []
    for _ in range(steps):
        loop.step()
        # both copies run on the main stream: after forward i / backward i, before step i+1
        ys.append(out.clone())
        snaps.append([x.clone() for x in g])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in range(steps):
        b = host_batches[i % 2]
        start, end = host_cores(wl, snaps[i]), host_cores(wl, snaps[i + 1])
        yref = oracle.forward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"], b["offsets"], B,
                              per_sample_weights=b["per_sample_weights"])
        assert rel_err(ys[i].cpu().numpy(), yref) <= TOL, i
        grads, touched, _, _ = oracle.backward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"],
                                               b["offsets"], B, b["grad_out"],
                                               per_sample_weights=b["per_sample_weights"])
        for t in range(T):
            for k in range(3):
                delta = end[t][k].astype(np.float64) - start[t][k].astype(np.float64)
                assert rel_err(delta, -wl.lr * grads[t][k]) <= TOL, (i, t, k)
                m = ~touched[t][k].astype(bool)
                assert np.array_equal(end[t][k][:, m], start[t][k][:, m]), (i, t, k)


@pytest.mark.parametrize("nb, steps", [(2, 3), (3, 5)])
def test_pipelined_loop_with_cache_matches_oracle(nb, steps):
    """The loop with a cache (each batch's lookup and grouping on the second stream,
    started right after a forward: one batch ahead with two batches, two ahead with three,
    where the lookup of batch i + 2 reuses the slot buffer of step i - 1): every step's
    forward, core update and cache-row update against the oracle, whose slots come from
    its own top-K selection."""
    print("case train loop cache", nb, steps, flush=True)
    wl = W.custom("cache", p=(20, 22, 25), q=(4, 4, 4), ranks=(32, 32), bags_per_table=256,
                  lengths=("fixed", 20), dist=("zipf", 1.2), init_std=1 / 32 ** 0.5, lr=0.01,
                  weighted=True)
    K, B = 900, 256
    cores = W.make_cores(wl)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    cache = abi.Cache(desc, K, 1 << 14)
    warm = [W.make_batch(wl, 100 + i) for i in range(4)]
    for bt in warm:
        cache.lookup(torch.from_numpy(bt["indices"]).cuda(), count_freq=True)
    g = gpu_cores(wl, cores)
    rows = torch.zeros(K, wl.D, device="cuda")
    nf = cache.populate(g, rows)
    sel = oracle.select_cache(oracle.count_frequencies([bt["indices"] for bt in warm]), K)
    assert nf == len(sel)
    host_batches = [W.make_batch(wl, k) for k in range(nb)]
    batches = [to_dev(b) for b in host_batches]
    slots = [torch.empty(b["indices"].numel(), dtype=torch.int32, device="cuda")
             for b in batches]
    out = torch.empty(B, wl.D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    loop = TrainLoop(desc, g, batches, B, wl.lr, out, status, cache=cache, rows=rows,
                     slots=slots)
    assert loop.ahead == (2 if nb >= 3 else 1)
    snaps, rsnaps, ys = [[x.clone() for x in g]], [rows.clone()], []
    for _ in range(steps):
        loop.step()
        ys.append(out.clone())
        snaps.append([x.clone() for x in g])
        rsnaps.append(rows.clone())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in range(steps):
        b = host_batches[i % nb]
        ref_slots = oracle.lookup_slots(sel, b["indices"])
        assert (ref_slots >= 0).any() and (ref_slots < 0).any()
        start, end = host_cores(wl, snaps[i]), host_cores(wl, snaps[i + 1])
        r0 = rsnaps[i].cpu().numpy()
        r1 = rsnaps[i + 1].cpu().numpy()
        yref = oracle.forward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"], b["offsets"], B,
                              per_sample_weights=b["per_sample_weights"], slots=ref_slots,
                              cache_rows=r0)
        assert rel_err(ys[i].cpu().numpy(), yref) <= TOL, i
        grads, touched, gc, tc = oracle.backward(wl.p, wl.q, wl.ranks, wl.E, start,
                                                 b["indices"], b["offsets"], B, b["grad_out"],
                                                 per_sample_weights=b["per_sample_weights"],
                                                 slots=ref_slots, cache_size=K)
        for k in range(3):
            delta = end[0][k].astype(np.float64) - start[0][k].astype(np.float64)
            assert rel_err(delta, -wl.lr * grads[0][k]) <= TOL, (i, k)
            m = ~touched[0][k].astype(bool)
            assert np.array_equal(end[0][k][:, m], start[0][k][:, m]), (i, k)
        drows = r1.astype(np.float64) - r0.astype(np.float64)
        assert rel_err(drows, -wl.lr * gc) <= TOL, i
        untouched = np.flatnonzero(tc == 0)
        assert np.array_equal(r1[untouched].view(np.uint32), r0[untouched].view(np.uint32)), i


def test_pipelined_loop_with_distinct_index_backward_matches_oracle():
    """The loop with the backward over distinct indices (its grouping waits on the host
    and is enqueued after each backward): two tables, heavy repeats, per-sample weights,
    empty bags; every step's forward and core update against the oracle."""
    print("case train loop dedup", flush=True)
    wl = W.custom("dedup loop", p=(6, 5, 7), q=(2, 4, 2), ranks=(8, 6), num_tables=2,
                  bags_per_table=40, lengths=("uniform", 0, 8), dist=("zipf", 1.3),
                  init_std=0.5, lr=0.05, weighted=True, num_embeddings=200)
    T, B, steps = wl.num_tables, wl.bags_per_table, 3
    cores = W.make_cores(wl)
    g = gpu_cores(wl, cores)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, T)
    host_batches = [W.make_batch(wl, k) for k in range(2)]
    assert len(np.unique(host_batches[0]["indices"])) < len(host_batches[0]["indices"]) // 2
    out = torch.empty(T * B, wl.D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    loop = TrainLoop(desc, g, [to_dev(b) for b in host_batches], B, wl.lr, out, status,
                     dedup=True)
    snaps, ys = [[x.clone() for x in g]], []
    for _ in range(steps):
        loop.step()
        ys.append(out.clone())
        snaps.append([x.clone() for x in g])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in range(steps):
        b = host_batches[i % 2]
        start, end = host_cores(wl, snaps[i]), host_cores(wl, snaps[i + 1])
        yref = oracle.forward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"], b["offsets"], B,
                              per_sample_weights=b["per_sample_weights"])
        assert rel_err(ys[i].cpu().numpy(), yref) <= TOL, i
        grads, touched, _, _ = oracle.backward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"],
                                               b["offsets"], B, b["grad_out"],
                                               per_sample_weights=b["per_sample_weights"])
        for t in range(T):
            for k in range(3):
                delta = end[t][k].astype(np.float64) - start[t][k].astype(np.float64)
                assert rel_err(delta, -wl.lr * grads[t][k]) <= TOL, (i, t, k)
                m = ~touched[t][k].astype(bool)
                assert np.array_equal(end[t][k][:, m], start[t][k][:, m]), (i, t, k)


def _host_d(wl, gcores):
    """d device tensors (core k of every table, slice-major) -> T lists of d logical cores."""
    shapes = W.core_shapes(wl)
    T, d = wl.num_tables, len(wl.p)
    res = [[None] * d for _ in range(T)]
    for k in range(d):
        arr = gcores[k].detach().cpu().numpy().reshape(T, -1)
        for t in range(T):
            res[t][k] = W.logical(arr[t], shapes[k])
    return res


def test_pipelined_loop_four_cores_matches_oracle():
    """The same loop on the four-core readme-sized table (d-core calls; the grouping is
    the three-core one of the multiplied-out cut): two steps against the d-core oracle."""
    print("case train loop readme4", flush=True)
    wl = W.WORKLOADS["readme4"]
    T, B, d, steps = wl.num_tables, wl.bags_per_table, len(wl.p), 2
    cores = W.make_cores(wl)
    g = [torch.from_numpy(np.concatenate([W.slice_major(cores[t][k]).ravel() for t in range(T)]))
         .cuda() for k in range(d)]
    desc = abi.make_desc_d(wl.p, wl.q, wl.ranks, wl.E, T)
    host_batches = [W.make_batch(wl, k) for k in range(2)]
    out = torch.empty(T * B, wl.D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    loop = TrainLoop(desc, g, [to_dev(b) for b in host_batches], B, wl.lr, out, status)
    snaps, ys = [[x.clone() for x in g]], []
    for _ in range(steps):
        loop.step()
        ys.append(out.clone())
        snaps.append([x.clone() for x in g])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in range(steps):
        b = host_batches[i % 2]
        start, end = _host_d(wl, snaps[i]), _host_d(wl, snaps[i + 1])
        yref = oracle.forward_d(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"], b["offsets"],
                                B, b["per_sample_weights"])
        assert rel_err(ys[i].cpu().numpy(), yref) <= TOL, i
        grads, touched = oracle.backward_d(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"],
                                           b["offsets"], B, b["grad_out"],
                                           b["per_sample_weights"])
        for t in range(T):
            for k in range(d):
                delta = end[t][k].astype(np.float64) - start[t][k].astype(np.float64)
                assert rel_err(delta, -wl.lr * grads[t][k]) <= TOL, (i, t, k)
                m = ~touched[t][k].astype(bool)
                assert np.array_equal(end[t][k][:, m], start[t][k][:, m]), (i, t, k)


@pytest.mark.parametrize("update, pipeline", [("adagrad", True), ("grad", True), ("sgd", False)],
                         ids=["adagrad", "grad", "sgd-unpipelined"])
def test_loop_update_modes_match_oracle(update, pipeline):
    """The loop's other update modes and its unpipelined form, on two tables with
    ranks 32, weights, empty bags and repeats (E short of p1 p2 p3, so ten core-1 slices
    stay untouched): fused Adagrad (parameter and running-sum
    deltas against the oracle's Adagrad of the oracle's gradients), gradients returned
    (against the oracle's gradients; cores unchanged) and SGD without the second stream,
    two steps each, every step's forward against the oracle."""
    print("case train loop mode", update, pipeline, flush=True)
    wl = W.custom("loop modes", p=(40, 44, 50), q=(4, 4, 4), ranks=(32, 32), num_tables=2,
                  bags_per_table=96, lengths=("uniform", 0, 24), dist=("zipf", 1.1),
                  init_std=1 / 32 ** 0.5, lr=0.02, weighted=True, num_embeddings=30 * 44 * 50)
    T, B, steps, eps = wl.num_tables, wl.bags_per_table, 2, 1e-10
    cores = W.make_cores(wl)
    g = gpu_cores(wl, cores)
    aux = None
    if update == "adagrad":
        rng = np.random.Generator(np.random.PCG64(3))
        aux = gpu_cores(wl, [[rng.uniform(0.2, 2.0, c.shape).astype(np.float32) for c in tbl]
                             for tbl in cores])
    elif update == "grad":
        aux = [torch.full_like(x, float("nan")) for x in g]
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, T)
    host_batches = [W.make_batch(wl, k) for k in range(2)]
    out = torch.empty(T * B, wl.D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    loop = TrainLoop(desc, g, [to_dev(b) for b in host_batches], B, wl.lr, out, status,
                     update=update, aux=aux, pipeline=pipeline)
    snaps, asnaps, ys = [[x.clone() for x in g]], [], []
    if aux is not None:
        asnaps.append([x.clone() for x in aux])
    for _ in range(steps):
        loop.step()
        ys.append(out.clone())
        snaps.append([x.clone() for x in g])
        if aux is not None:
            asnaps.append([x.clone() for x in aux])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in range(steps):
        b = host_batches[i % 2]
        start, end = host_cores(wl, snaps[i]), host_cores(wl, snaps[i + 1])
        yref = oracle.forward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"], b["offsets"], B,
                              per_sample_weights=b["per_sample_weights"])
        assert rel_err(ys[i].cpu().numpy(), yref) <= TOL, i
        grads, touched, _, _ = oracle.backward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"],
                                               b["offsets"], B, b["grad_out"],
                                               per_sample_weights=b["per_sample_weights"])
        if update == "adagrad":
            s0, s1 = host_cores(wl, asnaps[i]), host_cores(wl, asnaps[i + 1])
            ref_c, ref_s, _, _ = oracle.adagrad(wl.p, wl.q, wl.ranks, wl.E, start, s0, grads,
                                                touched, wl.lr, eps)
        if update == "grad":
            gk = host_cores(wl, asnaps[i + 1])
        for t in range(T):
            for k in range(3):
                m = ~touched[t][k].astype(bool)
                old = start[t][k].astype(np.float64)
                if update == "grad":
                    got = gk[t][k]
                    assert rel_err(got, grads[t][k]) <= TOL, (i, t, k)
                    assert np.all(got[:, m] == 0.0), (i, t, k)
                    assert np.array_equal(end[t][k], start[t][k]), (i, t, k)
                    continue
                if update == "adagrad":
                    ds = s1[t][k].astype(np.float64) - s0[t][k]
                    assert rel_err(ds, ref_s[t][k] - s0[t][k]) <= TOL, (i, t, k)
                    assert np.array_equal(s1[t][k][:, m], s0[t][k][:, m]), (i, t, k)
                    ref = ref_c[t][k] - old
                else:
                    ref = -wl.lr * grads[t][k]
                assert rel_err(end[t][k].astype(np.float64) - old, ref) <= TOL, (i, t, k)
                assert np.array_equal(end[t][k][:, m], start[t][k][:, m]), (i, t, k)


@pytest.mark.parametrize("dedup", [False, True], ids=["plain", "dedup"])
def test_loop_reuses_its_workspaces_over_many_steps(dedup):
    """Fourteen pipelined steps over three batches of different sizes, so that every one
    of the loop's workspaces is reused (its done events follow only every few steps):
    every step's forward and core update against the oracle."""
    from tensor_train_compressed_ttembeddingbag_amd import loop as L
    print("case train loop reuse", dedup, flush=True)
    wl = W.custom("loop reuse", p=(12, 10, 14), q=(4, 4, 4), ranks=(16, 32), num_tables=2,
                  bags_per_table=48, lengths=("uniform", 0, 30), dist=("zipf", 1.2),
                  init_std=1 / 32 ** 0.5, lr=0.002, weighted=True)  # stays bounded 14 steps
    T, B, steps = wl.num_tables, wl.bags_per_table, 14
    cores = W.make_cores(wl)
    g = gpu_cores(wl, cores)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, T)
    host_batches = [W.make_batch(wl, k) for k in range(3)]
    assert len({len(b["indices"]) for b in host_batches}) == 3
    out = torch.empty(T * B, wl.D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    loop = TrainLoop(desc, g, [to_dev(b) for b in host_batches], B, wl.lr, out, status,
                     dedup=dedup)
    assert len(loop.wss) == loop.ahead + L.DONE_EVERY
    assert loop.ahead == 2  # the distinct-index grouping does not wait on the host either
    assert steps > 2 * len(loop.wss)
    snaps, ys = [[x.clone() for x in g]], []
    for _ in range(steps):
        loop.step()
        ys.append(out.clone())
        snaps.append([x.clone() for x in g])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in range(steps):
        b = host_batches[i % 3]
        start, end = host_cores(wl, snaps[i]), host_cores(wl, snaps[i + 1])
        yref = oracle.forward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"], b["offsets"], B,
                              per_sample_weights=b["per_sample_weights"])
        assert rel_err(ys[i].cpu().numpy(), yref) <= TOL, i
        grads, touched, _, _ = oracle.backward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"],
                                               b["offsets"], B, b["grad_out"],
                                               per_sample_weights=b["per_sample_weights"])
        for t in range(T):
            for k in range(3):
                delta = end[t][k].astype(np.float64) - start[t][k].astype(np.float64)
                assert rel_err(delta, -wl.lr * grads[t][k]) <= TOL, (i, t, k)


def test_captured_loop_replays_match_the_eager_loop():
    """The loop captured into HIP graphs (graph=True: one graph per (batch, workspace)
    pair, the grouping of batch i + 2 forked onto the second stream inside the capture):
    13 steps replayed, each one checked right after it against the same step enqueued
    eagerly by a second loop on its own copy of the cores (the host synchronises between
    them).  The backward is deterministic, so the cores must agree bit for bit after
    every step; the forward pools with atomics, so its output agrees to rounding.  The
    first and the last replayed forwards are also checked against the oracle at the cores
    they started from.  Replays reuse each graph (6 graphs for 13 steps), so the kernels'
    flag tags must move on without the host."""
    print("case captured train loop readme 13", flush=True)
    wl = W.WORKLOADS["readme"]
    B, steps = wl.bags_per_table, 13
    cores = W.make_cores(wl)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    host_batches = [W.make_batch(wl, k) for k in range(2)]
    batches = [to_dev(b) for b in host_batches]
    g_e, g_c = gpu_cores(wl, cores), gpu_cores(wl, cores)
    out_e, out_c = (torch.empty(B, wl.D, device="cuda") for _ in range(2))
    st_e, st_c = (torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2))
    eager = TrainLoop(desc, g_e, batches, B, wl.lr, out_e, st_e)
    cap = TrainLoop(desc, g_c, batches, B, wl.lr, out_c, st_c, graph=True)
    assert len(cap.graphs) == 6  # lcm(2 batches, 6 workspaces)
    checks = {}
    for i in range(steps):
        start = [x.clone() for x in g_c] if i in (0, steps - 1) else None
        eager.step()
        torch.cuda.synchronize()
        cap.step()
        torch.cuda.synchronize()
        assert rel_err(out_c.cpu().numpy(), out_e.cpu().numpy()) <= 1e-6, i
        for k in range(3):
            assert torch.equal(g_c[k], g_e[k]), (i, k)
        if start is not None:
            checks[i] = (host_cores(wl, start), out_c.cpu().numpy())
    assert int(st_e.item()) == 0 and int(st_c.item()) == 0
    for i, (start, y) in checks.items():
        b = host_batches[i % 2]
        yref = oracle.forward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"], b["offsets"], B)
        assert rel_err(y, yref) <= TOL, i


def test_captured_loop_takes_the_plain_path_only():
    """Graph capture is for the plain pipelined path; the others are rejected up front."""
    wl = W.custom(p=(8, 9, 10), q=(4, 4, 4), ranks=(16, 16), bags_per_table=8,
                  lengths=("uniform", 1, 4))
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    g = gpu_cores(wl, W.make_cores(wl))
    b = [to_dev(W.make_batch(wl, 0))]
    out = torch.empty(8, wl.D, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        TrainLoop(desc, g, b, 8, 0.1, out, st, pipeline=False, graph=True)
    with pytest.raises(ValueError):
        TrainLoop(desc, g, b, 8, 0.1, out, st, dedup=True, graph=True)
