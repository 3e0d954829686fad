"""Full-size parity of the configurations the benchmark runs besides the readme shape:
the cached workload (110,000-row cache over E = 11M, 4,096 x 20 Zipf(1.2) indices, a
10-batch warm-up that under-fills the cache), the skewed workload (D = 128, ranks 64,
Zipf(1.1), weights, ragged bags) on every bag and every slice, and the backward over
distinct indices at the skewed and table-batched sizes.  The oracle runs over chunks of
bags in threads (tests/helpers.py: par_forward / par_backward / par_rows), which gives
its own results up to the fp64 rounding of the final sums."""
import sys

import numpy as np
import pytest
import torch

import oracle
from tensor_train_compressed_ttembeddingbag_amd import abi, workloads as W
from helpers import (TOL, gpu_cores, host_cores, par_backward, par_forward, par_rows, rel_err,
                     to_dev)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_all_slices(wl, cores, new, grads, touched, lr):
    """Every core delta against -lr * gradient (per tensor, every element); untouched
    slices keep their bits."""
    for t in range(wl.num_tables):
        for k in range(3):
            old = cores[t][k].astype(np.float64)
            delta = new[t][k].astype(np.float64) - old
            exp = -lr * grads[t][k]
            assert rel_err(delta, exp) <= TOL, (t, k)
            o_sl, n_sl = np.moveaxis(cores[t][k], 1, 0), np.moveaxis(new[t][k], 1, 0)
            for ik in np.flatnonzero(touched[t][k] == 0):
                assert np.array_equal(o_sl[ik].view(np.uint32), n_sl[ik].view(np.uint32))


def test_cached_workload_full_size():
    """The cached configuration end to end at its real size: 10 warm-up lookups counting
    frequencies, populate with K = 110,000 (the warm-up sees fewer distinct indices, so the
    cache under-fills), then lookup + forward + backward with SGD on a fresh batch.  Cache
    selection and slots bit-exact; rows, pooled output, core deltas and cache-row deltas
    element by element against the oracle."""
    wl = W.WORKLOADS["cached"]
    K = wl.cache_size
    _say("case cached full: K", K)
    cores = W.make_cores(wl)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    cache = abi.Cache(desc, K, wl.hashtbl_size)
    warm = [W.make_batch(wl, 500 + k)["indices"] for k in range(wl.warmup_batches)]
    for idx in warm:
        cache.lookup(torch.from_numpy(idx).cuda(), count_freq=True)
    g = gpu_cores(wl, cores)
    rows = torch.zeros(K, wl.D, device="cuda")
    nf = cache.populate(g, rows)
    sel = oracle.select_cache(oracle.count_frequencies(warm), K)
    _say("populated", nf, "of", K)
    assert nf == len(sel) and nf < K  # under-fill: fewer distinct warm-up indices than K
    got = cache.cached_indices().cpu().numpy()
    assert np.array_equal(got[:nf], sel) and np.all(got[nf:] == -1)
    rows_np = rows.cpu().numpy()
    assert rel_err(rows_np[:nf], par_rows(wl, cores[0], sel)) <= TOL
    assert not rows_np[nf:].any()
    b = W.make_batch(wl, 0)
    B = b["num_bags"]
    d = to_dev(b)
    slots = cache.lookup(d["indices"], count_freq=False)
    ref_slots = oracle.lookup_slots(sel, b["indices"])
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    _say("hit rate", float(np.mean(ref_slots >= 0)))
    rows_old = rows_np.copy()
    ws = abi.workspace(desc, d["indices"].numel(), B, K)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    Y = abi.tt_bag_forward(desc, g, d["indices"], d["offsets"], B, cache=(slots, rows), ws=ws,
                           dev_status=st).cpu().numpy()
    abi.tt_bag_backward_sgd(desc, g, d["indices"], d["offsets"], B, d["grad_out"], wl.lr,
                            cache=(slots, rows), ws=ws, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    Yo = par_forward(wl, cores, b, slots=ref_slots, cache_rows=rows_old)
    assert rel_err(Y, Yo) <= TOL
    grads, touched, gc, tc = par_backward(wl, cores, b, slots=ref_slots, cache_size=K)
    _check_all_slices(wl, cores, host_cores(wl, g), grads, touched, wl.lr)
    rows_new = rows.cpu().numpy()
    drows = rows_new.astype(np.float64) - rows_old
    assert rel_err(drows, -wl.lr * gc) <= TOL
    hit = np.flatnonzero(tc)
    assert rel_err(drows[hit], -wl.lr * gc[hit]) <= TOL
    untouched = np.flatnonzero(tc == 0)
    assert np.array_equal(rows_new[untouched].view(np.uint32), rows_old[untouched].view(np.uint32))
    cache.close()


def test_skewed_workload_full_size_every_bag_and_slice():
    """Skewed configuration (D = 128, ranks 64, Poisson lengths, Zipf(1.1), weights):
    every pooled bag and every slice of the three cores against the oracle."""
    wl = W.WORKLOADS["skewed"]
    _say("case skewed full, every bag and slice")
    cores = W.make_cores(wl)
    b = W.make_batch(wl, 0)
    B = b["num_bags"]
    g = gpu_cores(wl, cores)
    d = to_dev(b)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    ws = abi.workspace(desc, d["indices"].numel(), B)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    Y = abi.tt_bag_forward(desc, g, d["indices"], d["offsets"], B, d["per_sample_weights"],
                           ws=ws, dev_status=st).cpu().numpy()
    abi.tt_bag_backward_sgd(desc, g, d["indices"], d["offsets"], B, d["grad_out"], wl.lr,
                            d["per_sample_weights"], ws=ws, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert rel_err(Y, par_forward(wl, cores, b)) <= TOL
    grads, touched, _, _ = par_backward(wl, cores, b)
    _check_all_slices(wl, cores, host_cores(wl, g), grads, touched, wl.lr)


@pytest.mark.parametrize("name", ["skewed", "multitable"])
def test_distinct_index_backward_full_size_against_the_oracle(name):
    """The backward over distinct indices (plan_dedup + backward_sgd_dedup) at full size,
    against the oracle's backward of the real batch (not against the every-element HIP
    backward)."""
    wl = W.WORKLOADS[name]
    _say("case dedup full", name)
    cores = W.make_cores(wl)
    b = W.make_batch(wl, 0)
    B = b["num_bags"]
    g = gpu_cores(wl, cores)
    d = to_dev(b)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, wl.num_tables)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws, info = abi.tt_bag_plan_dedup(desc, d["indices"], d["offsets"], B,
                                     d["per_sample_weights"], dev_status=st)
    Y = abi.tt_bag_forward(desc, g, d["indices"], d["offsets"], B, d["per_sample_weights"],
                           ws=ws, dev_status=st, planned=True).cpu().numpy()
    abi.tt_bag_backward_sgd_dedup(desc, g, d["indices"], d["offsets"], B, d["grad_out"],
                                  wl.lr, info, d["per_sample_weights"], ws=ws, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    distinct = sum(len(np.unique(b["indices"][b["offsets"][t * B]:b["offsets"][(t + 1) * B]]))
                   for t in range(wl.num_tables))
    nnz = d["indices"].numel()
    assert info == (nnz, nnz)  # the bounds; the count itself stays on the device
    assert abi.tt_bag_dedup_counts(desc, nnz, B, ws)[-1] == distinct
    assert rel_err(Y, par_forward(wl, cores, b)) <= TOL
    grads, touched, _, _ = par_backward(wl, cores, b)
    _check_all_slices(wl, cores, host_cores(wl, g), grads, touched, wl.lr)
